"""The entry points captured into one HIP graph: every replay must equal the
eager result of the same inputs (the library records no memset nodes;
replays are interleaved with eager work and synchronisations).  Two step
forms: the separate calls, and the fused append + select writing the
log-gate bias with the gated decode; and the whole step as one
bsa_append_select_decode call (selection inside the decode launch)."""
import math

import numpy as np
import pytest

import block_sparse_attention_build_amd as bsa
from harness import prefill, random_page_table, to_dev
from test_gpu_parity import make_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("form", ["separate", "fused_gated", "one_call"])
def test_graph_replays_match_eager(form):
    import torch
    d, blk, f = 128, 64, 32
    lengths = [3000, 1777]
    L = bsa.Layout(2, 8, 2, d, blk, 80, bsa.DTYPE_BF16, bsa.DESC_MINMAX)
    P = bsa.SelectParams(sparsity_bp=8000, n_local=2, n_min=4)
    P.n_max = bsa.block_count(P, 80, blk)
    q, Ks, Vs, _ = make_inputs(5, 2, 8, 2, d, lengths, bsa.DTYPE_BF16, bsa.DESC_MINMAX)
    rng = np.random.Generator(np.random.PCG64(6))
    dev = "cuda"
    qd = to_dev(q, L)
    kn = torch.from_numpy(rng.standard_normal((2, 2, 1, d), dtype=np.float32)).to(dev, torch.bfloat16)
    vn = torch.from_numpy(rng.standard_normal((2, 2, 1, d), dtype=np.float32)).to(dev, torch.bfloat16)
    qr = torch.from_numpy(rng.standard_normal((2, 8, f, d), dtype=np.float32)).to(dev, torch.bfloat16)
    kr = torch.from_numpy(rng.standard_normal((2, 2, f, d), dtype=np.float32)).to(dev, torch.bfloat16)
    vr = torch.from_numpy(rng.standard_normal((2, 2, f, d), dtype=np.float32)).to(dev, torch.bfloat16)
    ws_bytes = max(bsa.workspace_size(L, op, n) for op, n in
                   [(bsa.OP_SELECT, P.n_max), (bsa.OP_DECODE, P.n_max), (bsa.OP_RECTIFY, f),
                    (bsa.OP_STEP, P.n_max)])

    def fresh():
        cache = bsa.allocate_cache(L, page_table=random_page_table(L, 8))
        for t in (cache.k_pool, cache.v_pool, cache.desc):
            t.zero_()  # unwritten regions compare equal at the end
        prefill(L, cache, Ks, Vs, lengths)
        bufs = dict(idx=torch.full((2, 2, P.n_max), -7, dtype=torch.int32, device=dev),
                    cnt=torch.zeros(2, 2, dtype=torch.int32, device=dev),
                    o=torch.zeros(2, 8, d, dtype=torch.bfloat16, device=dev),
                    lse=torch.zeros(2, 8, dtype=torch.float32, device=dev),
                    o_r=torch.zeros(2, 8, f, d, dtype=torch.bfloat16, device=dev),
                    lse_r=torch.zeros(2, 8, f, dtype=torch.float32, device=dev),
                    bias=torch.zeros(2, 2, P.n_max, dtype=torch.float32, device=dev),
                    ws=torch.zeros(ws_bytes, dtype=torch.uint8, device=dev))
        return cache, bufs

    def step(cache, b):
        cache.seq_lens.add_(1)
        if form == "separate":
            bsa.build_block_desc(L, cache, kn, vn, 1)
            bsa.select_blocks(L, cache, qd, P, b["idx"], b["cnt"], b["ws"])
            bsa.sparse_decode(L, cache, qd, b["idx"], b["cnt"], P.n_max, 1 / math.sqrt(d), b["o"],
                              b["lse"], b["ws"])
        elif form == "one_call":
            bsa.append_select_decode(L, cache, kn, vn, qd, P, b["idx"], b["cnt"], 1 / math.sqrt(d),
                                     b["o"], b["lse"], b["ws"])
        else:
            Pg = bsa.SelectParams(sparsity_bp=8000, n_local=2, n_min=4, n_max=P.n_max,
                                  gate_tau=0.02, gate_bias=b["bias"])
            bsa.append_select(L, cache, kn, vn, qd, Pg, b["idx"], b["cnt"], b["ws"])
            bsa.sparse_decode_gated(L, cache, qd, b["idx"], b["cnt"], b["bias"], P.n_max,
                                    1 / math.sqrt(d), b["o"], b["lse"], b["ws"])
        bsa.rectify_chunk(L, cache, qr, kr, vr, f, 1 / math.sqrt(d), b["o_r"], b["lse_r"], b["ws"])

    # eager reference: three consecutive steps from the same start
    cache_e, be = fresh()
    ref = []
    for _ in range(3):
        step(cache_e, be)
        torch.cuda.synchronize()
        ref.append({k: v.clone() for k, v in be.items() if k != "ws"})
    # graph: one step captured, replayed three times
    cache_g, bg = fresh()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(cache_g, bg)
    for r in range(3):
        _ = torch.randn(1000, device=dev).sum()  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in ref[r].items():
            assert torch.equal(bg[k], v), f"replay {r}: {k} differs from eager"
    assert torch.equal(cache_g.seq_lens, cache_e.seq_lens)
    assert torch.equal(cache_g.k_pool, cache_e.k_pool) and torch.equal(cache_g.desc, cache_e.desc)

"""bsa_sparse_decode_static, the decode entry point that takes no workspace
(its split partials live in the library's per-GPU scratch array), against
bsa_sparse_decode with a caller workspace: two calls in a row on one GPU,
the second on a smaller input, each bit-identical to the workspace call and
within the decode bars of the oracle.  Named to be collected last, so that a
failure here hides no other test of a `pytest -x` run."""
import math

import numpy as np
import pytest

import block_sparse_attention_build_amd as bsa
import workloads as W
from harness import compare_step, oracle_decode, prefill, random_page_table

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, blk, lengths, budget, seed):
    import torch
    d = 128
    max_blocks = (max(lengths) + blk - 1) // blk + 2
    L = bsa.Layout(B, Hq, Hkv, d, blk, max_blocks, bsa.DTYPE_BF16, bsa.DESC_MINMAX)
    rng = np.random.Generator(np.random.PCG64(seed))
    Ks = [W.round_bf16(rng.standard_normal((Hkv, T, d), dtype=np.float32)) for T in lengths]
    Vs = [W.round_bf16(rng.standard_normal((Hkv, T, d), dtype=np.float32)) for T in lengths]
    q = W.round_bf16(rng.standard_normal((B, Hq, d), dtype=np.float32))
    cache = bsa.allocate_cache(L, page_table=random_page_table(L, seed + 1))
    prefill(L, cache, Ks, Vs, lengths)
    cache.seq_lens.copy_(torch.tensor(lengths, dtype=torch.int32))
    P = bsa.SelectParams(budget_tokens=budget, n_local=1)
    P.n_max = bsa.block_count(P, max_blocks, blk)
    dev = "cuda"
    idx = torch.empty(B, Hkv, P.n_max, dtype=torch.int32, device=dev)
    cnt = torch.empty(B, Hkv, dtype=torch.int32, device=dev)
    ws = torch.empty(max(bsa.workspace_size(L, bsa.OP_SELECT, P.n_max),
                         bsa.workspace_size(L, bsa.OP_DECODE, P.n_max)),
                     dtype=torch.uint8, device=dev)
    qt = torch.from_numpy(q).to(dev, torch.bfloat16)
    bsa.select_blocks(L, cache, qt, P, idx, cnt, ws)
    return L, cache, P, qt, idx, cnt, ws, (q, Ks, Vs, lengths)


def test_static_scratch_decode_matches_workspace_decode():
    import torch
    # the second call is smaller (fewer sequences, fewer groups and splits)
    # and follows the first on the same scratch array
    cases = [dict(B=3, Hq=32, Hkv=8, blk=64, lengths=[9000, 5000, 777], budget=2048, seed=11),
             dict(B=1, Hq=16, Hkv=4, blk=64, lengths=[3000], budget=512, seed=12)]
    for cs in cases:
        L, cache, P, qt, idx, cnt, ws, host = _case(**cs)
        assert bsa.workspace_size(L, bsa.OP_DECODE, P.n_max) <= bsa.STATIC_SCRATCH_BYTES
        scale = 1.0 / math.sqrt(L.d)
        o_ws = torch.full((L.B, L.Hq, L.d), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse_ws = torch.full((L.B, L.Hq), float("nan"), dtype=torch.float32, device="cuda")
        bsa.sparse_decode(L, cache, qt, idx, cnt, P.n_max, scale, o_ws, lse_ws, ws)
        o_st = torch.full_like(o_ws, float("nan"))
        lse_st = torch.full_like(lse_ws, float("nan"))
        bsa.sparse_decode_static(L, cache, qt, idx, cnt, P.n_max, scale, o_st, lse_st)
        torch.cuda.synchronize()
        assert torch.equal(o_st.view(torch.int16), o_ws.view(torch.int16)), cs
        assert torch.equal(lse_st.view(torch.int32), lse_ws.view(torch.int32)), cs
        q, Ks, Vs, lengths = host
        ref = oracle_decode(P, q, Ks, Vs, lengths, L, scale=scale)
        compare_step(L, idx, cnt, o_st, lse_st, ref)


def test_static_scratch_refuses_oversized_calls():
    # more split partials than the scratch array holds: refused before any
    # work is enqueued, outputs untouched
    import torch
    B, Hq, Hkv, d, blk = 256, 128, 8, 128, 64
    L = bsa.Layout(B, Hq, Hkv, d, blk, 64, bsa.DTYPE_BF16, bsa.DESC_MINMAX)
    P = bsa.SelectParams(budget_tokens=1024, n_local=1)
    P.n_max = bsa.block_count(P, L.max_blocks, blk)
    assert bsa.workspace_size(L, bsa.OP_DECODE, P.n_max) > bsa.STATIC_SCRATCH_BYTES
    cache = bsa.allocate_cache(L, num_pages=1)
    q = torch.zeros(B, Hq, d, dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros(B, Hkv, P.n_max, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(B, Hkv, dtype=torch.int32, device="cuda")
    o = torch.full((B, Hq, d), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, Hq), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(bsa.BsaError) as e:
        bsa.sparse_decode_static(L, cache, q, idx, cnt, P.n_max, 0.1, o, lse)
    assert e.value.status == bsa.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())

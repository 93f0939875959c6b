"""The Python binding's tensor checks on the GPU: a tensor of the wrong dtype,
a non-contiguous view or a buffer smaller than the documented shape is
refused with ValueError before the library is called, so nothing is
enqueued and the outputs keep their contents."""
import math

import numpy as np
import pytest

import block_sparse_attention_build_amd as bsa
import workloads as W
from harness import prefill, to_dev

pytestmark = pytest.mark.gpu

B, HQ, HKV, D, BLK, MAXB = 2, 8, 2, 64, 64, 16


def _state():
    import torch
    L = bsa.Layout(B, HQ, HKV, D, BLK, MAXB, bsa.DTYPE_BF16, bsa.DESC_MINMAX)
    rng = np.random.Generator(np.random.PCG64(61))
    lengths = [500, 300]
    Ks = [W.quantize(rng.standard_normal((HKV, T, D), dtype=np.float32), "bf16") for T in lengths]
    Vs = [W.quantize(rng.standard_normal((HKV, T, D), dtype=np.float32), "bf16") for T in lengths]
    cache = bsa.allocate_cache(L)
    prefill(L, cache, Ks, Vs, lengths)
    q = to_dev(W.quantize(rng.standard_normal((B, HQ, D), dtype=np.float32), "bf16"), L)
    P = bsa.SelectParams(budget_tokens=192, n_local=1)
    P.n_max = bsa.block_count(P, MAXB, BLK)
    idx = torch.full((B, HKV, P.n_max), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, HKV), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(bsa.workspace_size(L, bsa.OP_SELECT, P.n_max),
                         bsa.workspace_size(L, bsa.OP_DECODE, P.n_max),
                         bsa.workspace_size(L, bsa.OP_RECTIFY, 8)),
                     dtype=torch.uint8, device="cuda")
    o = torch.full((B, HQ, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, HQ), float("nan"), dtype=torch.float32, device="cuda")
    return L, cache, q, P, idx, cnt, ws, o, lse


def test_select_refuses_bad_tensors():
    import torch
    L, cache, q, P, idx, cnt, ws, o, lse = _state()
    bad = [
        ("dtype", dict(q=q.float())),
        ("contiguous", dict(q=q.transpose(1, 2).contiguous().transpose(1, 2))),
        ("at least", dict(idx=idx[:, :, :1].contiguous())),
        ("dtype", dict(cnt=cnt.long())),
    ]
    for what, kw in bad:
        args = dict(q=q, idx=idx, cnt=cnt)
        args.update(kw)
        with pytest.raises(ValueError, match=what):
            bsa.select_blocks(L, cache, args["q"], P, args["idx"], args["cnt"], ws)
    torch.cuda.synchronize()
    assert bool((idx == -7).all()) and bool((cnt == -7).all())


def test_decode_and_rectify_refuse_bad_tensors():
    import torch
    L, cache, q, P, idx, cnt, ws, o, lse = _state()
    bsa.select_blocks(L, cache, q, P, idx, cnt, ws)
    torch.cuda.synchronize()
    scale = 1 / math.sqrt(D)
    with pytest.raises(ValueError, match="dtype"):
        bsa.sparse_decode(L, cache, q, idx, cnt, P.n_max, scale, o.float(), lse, ws)
    with pytest.raises(ValueError, match="at least"):
        bsa.sparse_decode(L, cache, q, idx, cnt, P.n_max, scale, o, lse[:1], ws)
    with pytest.raises(ValueError, match="at least"):
        bias = torch.zeros(B, HKV, 1, dtype=torch.float32, device="cuda")
        bsa.sparse_decode_gated(L, cache, q, idx, cnt, bias, P.n_max, scale, o, lse, ws)
    bad_cache = bsa.Cache(cache.k_pool, cache.v_pool, cache.page_table.long(), cache.seq_lens,
                          cache.desc)
    with pytest.raises(ValueError, match="page_table"):
        bsa.sparse_decode(L, bad_cache, q, idx, cnt, P.n_max, scale, o, lse, ws)
    f = 8
    qr = torch.zeros(B, HQ, f, D, dtype=torch.bfloat16, device="cuda")
    kr = torch.zeros(B, HKV, f - 1, D, dtype=torch.bfloat16, device="cuda")  # one row short
    o_r = torch.full((B, HQ, f, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse_r = torch.full((B, HQ, f), float("nan"), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="k_new"):
        bsa.rectify_chunk(L, cache, qr, kr, kr, f, scale, o_r, lse_r, ws)
    torch.cuda.synchronize()
    assert bool(torch.isnan(o.float()).all()) and bool(torch.isnan(lse).all())
    assert bool(torch.isnan(o_r.float()).all())
    # the same call with proper tensors runs
    bsa.sparse_decode(L, cache, q, idx, cnt, P.n_max, scale, o, lse, ws)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(lse).any())

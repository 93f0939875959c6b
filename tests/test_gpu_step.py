"""bsa_append_select_decode, the whole decode step in one call: on every
shape it gives the cache, descriptors, idx, cnt, o and lse of
bsa_append_select followed by bsa_sparse_decode (bit for bit: the decode's
split ranges and units are the same), step after step, and the oracle's
selection, o and lse.  Rows of at most 8192 candidate blocks (bf16, no
log-gate bias) select inside the decode launch: those cases cover two, four,
eight and sixteen rows per thread up to the last thread's last row, rows
shorter than the capacity, single-block sequences, a budget covering the
whole context, long runs of tied scores and both descriptor kinds; the
others check the four-launch form.  Seeded random shapes add combinations no
hand-written case names."""
import math

import numpy as np
import pytest

import block_sparse_attention_build_amd as bsa
import workloads as W
from harness import compare_step, enforce_gap, oracle_decode, prefill, random_page_table, to_dev
from test_gpu_parity import make_inputs

pytestmark = pytest.mark.gpu

BF16, F32 = bsa.DTYPE_BF16, bsa.DTYPE_F32
MINMAX, MEAN = bsa.DESC_MINMAX, bsa.DESC_MEANPOOL

STEP_CASES = [
    # dtype, d, blk, kind, Hq, Hkv, lengths, budget, bp, n_local, n_min, steps, gated
    (BF16, 128, 64, MINMAX, 32, 8, [3000, 1700], 0, 9000, 2, 16, 3, False),
    (BF16, 128, 128, MEAN, 8, 2, [3000, 2049], 0, 9000, 2, 0, 3, False),
    (BF16, 128, 64, MINMAX, 8, 2, [1000, 1537], 256, 0, 1, 0, 2, False),
    # 1024 blocks of capacity (b = 32): thread 511 holds blocks 1022 and 1023
    (BF16, 64, 32, MINMAX, 4, 1, [32765], 0, 9000, 2, 4, 3, False),
    # rows far shorter than the capacity, single-block and block-edge sequences
    (BF16, 128, 64, MINMAX, 8, 2, [1, 64, 65, 2000], 0, 8000, 1, 3, 2, False),
    # budget >= context: every candidate kept
    (BF16, 64, 64, MINMAX, 4, 2, [700, 1283], 64 * 40, 0, 1, 0, 2, False),
    # three local blocks against sequences of 1-2 blocks (every block local,
    # no candidate) beside a longer one
    (BF16, 128, 64, MINMAX, 8, 2, [1, 100, 1500], 0, 9000, 3, 6, 2, False),
    # G = 1 and G = 16 groups
    (BF16, 64, 64, MINMAX, 2, 2, [1900], 0, 9000, 3, 0, 2, False),
    (BF16, 128, 64, MINMAX, 16, 1, [4000], 0, 9500, 2, 2, 2, False),
    # four blocks per thread (1251 blocks), and a ragged batch at eight per
    # thread (3126 blocks of capacity, the short rows in one or two waves)
    (BF16, 64, 32, MINMAX, 4, 1, [40000], 0, 9000, 2, 4, 2, False),
    (BF16, 128, 32, MINMAX, 8, 2, [100000, 16384, 3000, 40000], 0, 9000, 2, 16, 2, False),
    # 4096 blocks of capacity (eight rows per thread)
    (BF16, 64, 32, MEAN, 4, 1, [131069], 0, 9500, 2, 0, 3, False),
    # sixteen rows per thread: 4374 candidates, and 8192 (the last thread's
    # last row is a candidate; the two local blocks lie past the rows)
    (BF16, 64, 32, MINMAX, 4, 1, [140000], 0, 9000, 2, 4, 2, False),
    (BF16, 64, 32, MINMAX, 4, 1, [262176], 0, 9000, 2, 16, 3, False),
    # the four-launch form: more than 8192 candidates, a log-gate bias, fp32
    (BF16, 64, 32, MINMAX, 4, 1, [300000], 0, 9500, 2, 4, 2, False),
    (BF16, 128, 64, MINMAX, 8, 2, [3000, 1700], 0, 9000, 2, 4, 2, True),
    (F32, 64, 64, MINMAX, 4, 1, [2049], 512, 0, 1, 2, 2, False),
]


def _step_pair(L, P, caches, q_dev, kn, vn, scale, ws, gated):
    """One step on each cache: [0] through the one call, [1] through
    append_select + sparse_decode(_gated).  Returns both results."""
    import torch
    dev = q_dev.device
    out = []
    for which, c in enumerate(caches):
        c.seq_lens += 1
        idx = torch.full((L.B, L.Hkv, P.n_max), -7, dtype=torch.int32, device=dev)
        cnt = torch.full((L.B, L.Hkv), -7, dtype=torch.int32, device=dev)
        o = torch.full((L.B, L.Hq, L.d), float("nan"), dtype=q_dev.dtype, device=dev)
        lse = torch.full((L.B, L.Hq), float("nan"), dtype=torch.float32, device=dev)
        bias = None
        Pc = P
        if gated:
            bias = torch.full((L.B, L.Hkv, P.n_max), float("nan"), dtype=torch.float32, device=dev)
            Pc = bsa.SelectParams(P.budget_tokens, P.sparsity_bp, P.n_local, P.n_min, P.n_max,
                                  P.gate_w, 0.05, bias)
        ws.view(torch.float32)[: ws.numel() // 4].fill_(float("nan"))  # poison
        if which == 0:
            bsa.append_select_decode(L, c, kn, vn, q_dev, Pc, idx, cnt, scale, o, lse, ws)
        else:
            bsa.append_select(L, c, kn, vn, q_dev, Pc, idx, cnt, ws)
            if gated:
                bsa.sparse_decode_gated(L, c, q_dev, idx, cnt, bias, P.n_max, scale, o, lse, ws)
            else:
                bsa.sparse_decode(L, c, q_dev, idx, cnt, P.n_max, scale, o, lse, ws)
        torch.cuda.synchronize()
        out.append((idx, cnt, o, lse, bias))
    return out


@pytest.mark.parametrize("case", STEP_CASES, ids=[f"s{i}" for i in range(len(STEP_CASES))])
def test_step_equals_the_calls_and_the_oracle(case):
    _run_step_case(case, 41)


def _draw(seed):
    """A seeded random step case: mostly short rows of any block size, a
    quarter long rows at b = 32 (up to about 4700 blocks, every in-launch
    tier), some fp32 and some with the log-gate bias (the four-launch form)."""
    rng = np.random.Generator(np.random.PCG64(7700 + seed))
    gated = rng.random() < 0.2
    dtype = F32 if rng.random() < 0.15 else BF16
    kind = MINMAX if rng.random() < 0.7 else MEAN
    if rng.random() < 0.25:
        d, blk, Hkv = 64, 32, 1
        G = int(rng.choice([1, 2, 4]))
        B = int(rng.integers(1, 3))
        lengths = [int(x) for x in rng.integers(1, 150000, size=B)]
    else:
        d = int(rng.choice([64, 128]))
        blk = int(rng.choice([32, 64, 128, 256]))
        Hkv = int(rng.integers(1, 5))
        G = int(rng.choice([1, 2, 3, 4, 5, 8]))
        B = int(rng.integers(1, 5))
        lengths = [int(x) for x in rng.integers(1, 40 * blk, size=B)]
    if rng.random() < 0.4:
        budget, bp = int(rng.integers(1, 24)) * blk, 0
    else:
        budget, bp = 0, int(rng.choice([5000, 8000, 9000, 9500]))
    n_local = int(rng.integers(1, 4))
    n_min = int(rng.integers(0, 6))
    return (dtype, d, blk, kind, G * Hkv, Hkv, lengths, budget, bp, n_local, n_min, 2, gated)


@pytest.mark.parametrize("seed", range(24))
def test_random_shape_step(seed):
    case = _draw(seed)
    print(f"seed {seed}: {case}", flush=True)
    _run_step_case(case, 800 + seed)


def _run_step_case(case, seed):
    import torch
    dtype, d, blk, kind, Hq, Hkv, lengths, budget, bp, nl, nm, steps, gated = case
    B = len(lengths)
    max_blocks = (max(lengths) + steps + blk - 1) // blk
    L = bsa.Layout(B, Hq, Hkv, d, blk, max_blocks, dtype, kind)
    P = bsa.SelectParams(budget_tokens=budget, sparsity_bp=bp, n_local=nl, n_min=nm)
    P.n_max = bsa.block_count(P, max_blocks, blk)
    total = [T + steps for T in lengths]
    q, Ks, Vs, Wg = make_inputs(seed + B, B, Hq, Hkv, d, total, dtype, kind)
    if not gated:
        enforce_gap(L, P, q, Ks, [[T + i + 1 for i in range(steps)] for T in lengths], W_gate=Wg)
    if Wg is not None:
        P.gate_w = to_dev(Wg, bsa.Layout(1, 1, 1, d, blk, 1, BF16))
    caches = []
    for _ in range(2):
        c = bsa.allocate_cache(L, page_table=random_page_table(L, 4))
        for t in (c.k_pool, c.v_pool, c.desc):
            t.zero_()  # unwritten regions compare equal
        prefill(L, c, Ks, Vs, lengths)
        caches.append(c)
    ws = torch.empty(bsa.workspace_size(L, bsa.OP_STEP, P.n_max), dtype=torch.uint8,
                     device="cuda")
    q_dev = to_dev(q, L)
    scale = 1.0 / math.sqrt(d)
    for step in range(steps):
        kn = to_dev(np.stack([Ks[s][:, lengths[s] + step] for s in range(B)])[:, :, None], L)
        vn = to_dev(np.stack([Vs[s][:, lengths[s] + step] for s in range(B)])[:, :, None], L)
        one, two = _step_pair(L, P, caches, q_dev, kn, vn, scale, ws, gated)
        for name, a, b in zip(("idx", "cnt", "o", "lse", "bias"), one, two):
            if a is not None:
                assert torch.equal(a, b), f"step {step}: {name} differs from the two calls"
        assert torch.equal(caches[0].k_pool, caches[1].k_pool)
        assert torch.equal(caches[0].v_pool, caches[1].v_pool)
        assert torch.equal(caches[0].desc, caches[1].desc)
        if not gated:
            now = [T + step + 1 for T in lengths]
            ref = oracle_decode(P, q, [K[:, :T] for K, T in zip(Ks, now)],
                                [V[:, :T] for V, T in zip(Vs, now)], now, L, W_gate=Wg)
            compare_step(L, one[0], one[1], one[2], one[3], ref)


def test_step_long_run_of_ties():
    """About 1000 candidates with nearly all scores equal (a tiled key
    template): the threshold select takes the tied keys by ascending index,
    in the one call as in the top-n kernel and the oracle."""
    import torch
    d, blk, Hq, Hkv = 64, 32, 4, 1
    T0 = 1000 * blk + 5
    max_blocks = (T0 + 2 + blk - 1) // blk
    L = bsa.Layout(1, Hq, Hkv, d, blk, max_blocks, BF16, MINMAX)
    P = bsa.SelectParams(budget_tokens=0, sparsity_bp=9000, n_local=1, n_min=0)
    P.n_max = bsa.block_count(P, max_blocks, blk)
    rng = np.random.Generator(np.random.PCG64(321))
    q = W.quantize(rng.standard_normal((1, Hq, d), dtype=np.float32), "bf16")
    u = W.group_direction(q[0])
    T = T0 + 2
    tmpl = rng.standard_normal((blk, d), dtype=np.float32)
    K = np.tile(tmpl, ((T + blk - 1) // blk, 1))[:T].copy()
    K[-7:] = rng.standard_normal((7, d), dtype=np.float32)
    for j in (3, 200, 555, 998):   # clearly above the tied mass
        K[j * blk:(j + 1) * blk] += 3.0 * u
    for j in (1, 600):             # clearly below it
        K[j * blk:(j + 1) * blk] -= 3.0 * u
    K = W.quantize(K, "bf16")[None]
    V = W.quantize(rng.standard_normal((1, T, d), dtype=np.float32), "bf16")
    caches = []
    for _ in range(2):
        c = bsa.allocate_cache(L, page_table=random_page_table(L, 9))
        prefill(L, c, [K], [V], [T0])
        caches.append(c)
    ws = torch.empty(bsa.workspace_size(L, bsa.OP_STEP, P.n_max), dtype=torch.uint8,
                     device="cuda")
    q_dev = to_dev(q, L)
    for step in range(2):
        kn = to_dev(K[:, T0 + step][None, :, None], L)
        vn = to_dev(V[:, T0 + step][None, :, None], L)
        one, two = _step_pair(L, P, caches, q_dev, kn, vn, 1 / math.sqrt(d), ws, False)
        for a, b in zip(one[:4], two[:4]):
            assert torch.equal(a, b)
        now = T0 + step + 1
        ref = oracle_decode(P, q, [K[:, :now]], [V[:, :now]], [now], L)
        compare_step(L, one[0], one[1], one[2], one[3], ref)
        assert {3, 200, 555, 998} <= set(ref[(0, 0)][0].tolist())


def test_step_checked_build_matches_default():
    """The checked build (host-side contract checks, then the same kernels)
    gives the default build's results for the one-call step, bit for bit, on
    the in-launch form and on the four-launch form (log-gate bias)."""
    import torch
    d, blk, Hq, Hkv = 128, 64, 8, 2
    lengths = [3000, 1700]
    L = bsa.Layout(2, Hq, Hkv, d, blk, 60, BF16, MINMAX)
    q, Ks, Vs, _ = make_inputs(61, 2, Hq, Hkv, d, [T + 2 for T in lengths], BF16, MINMAX)
    q_dev = to_dev(q, L)
    outs = []
    for path in (bsa.LIB_DEFAULT, bsa.LIB_CHECKED):
        before = bsa.use_library(path)
        try:
            c = bsa.allocate_cache(L, page_table=random_page_table(L, 12))
            for t in (c.k_pool, c.v_pool, c.desc):
                t.zero_()
            prefill(L, c, Ks, Vs, lengths)
            res = []
            for gated in (False, True):
                P = bsa.SelectParams(sparsity_bp=9000, n_local=2, n_min=4)
                P.n_max = bsa.block_count(P, L.max_blocks, blk)
                ws = torch.empty(bsa.workspace_size(L, bsa.OP_STEP, P.n_max), dtype=torch.uint8,
                                 device="cuda")
                idx = torch.full((2, Hkv, P.n_max), -7, dtype=torch.int32, device="cuda")
                cnt = torch.full((2, Hkv), -7, dtype=torch.int32, device="cuda")
                o = torch.full((2, Hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
                lse = torch.full((2, Hq), float("nan"), dtype=torch.float32, device="cuda")
                if gated:
                    P.gate_tau = 0.05
                    P.gate_bias = torch.zeros(2, Hkv, P.n_max, dtype=torch.float32, device="cuda")
                step = 1 if gated else 0
                kn = to_dev(np.stack([Ks[s][:, lengths[s] + step] for s in range(2)])[:, :, None], L)
                vn = to_dev(np.stack([Vs[s][:, lengths[s] + step] for s in range(2)])[:, :, None], L)
                c.seq_lens += 1
                bsa.append_select_decode(L, c, kn, vn, q_dev, P, idx, cnt, 1 / math.sqrt(d), o,
                                         lse, ws)
                torch.cuda.synchronize()
                res += [idx, cnt, o, lse] + ([P.gate_bias] if gated else [])
            res += [c.k_pool, c.v_pool, c.desc]
            outs.append(res)
        finally:
            bsa.use_library(before)
    for a, b in zip(*outs):
        assert torch.equal(a, b)

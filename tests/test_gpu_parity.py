"""GPU parity of every C-ABI entry point against the fp64 oracle, at sizes
the oracle finishes in seconds that still span many 32-token tiles, several
splits and ragged tails.  Selection is compared bit-exactly (inputs carry a
score gap at the top-n boundary), o within 2e-2 absolute (bf16 I/O, fp32
accumulation), lse within 1e-4 relative."""
import math

import numpy as np
import pytest

import block_sparse_attention_build_amd as bsa
import oracle as O
import workloads as W
from harness import (compare_step, enforce_gap, oracle_decode, page_index_maps, prefill,
                     random_page_table, read_cache, to_dev)

pytestmark = pytest.mark.gpu

BF16, F32 = bsa.DTYPE_BF16, bsa.DTYPE_F32
MINMAX, MEAN = bsa.DESC_MINMAX, bsa.DESC_MEANPOOL


def _torch():
    import torch
    return torch


def make_inputs(seed, B, Hq, Hkv, d, lengths, dtype, desc_kind, planted=0.05):
    """Seeded q [B,Hq,d], per-sequence K,V [Hkv,T,d] with channel scales and
    planted blocks (the workload recipe), W for mean-pool."""
    rng = np.random.Generator(np.random.PCG64(seed))
    st = "bf16" if dtype == BF16 else "f32"
    ks = rng.lognormal(0, 0.5, size=(Hkv, d)).astype(np.float32)
    vs = rng.lognormal(0, 0.5, size=(Hkv, d)).astype(np.float32)
    q = W.quantize(rng.standard_normal((B, Hq, d), dtype=np.float32), st)
    Ks, Vs = [], []
    G = Hq // Hkv
    for T in lengths:
        K = rng.standard_normal((Hkv, T, d), dtype=np.float32) * ks[:, None]
        V = rng.standard_normal((Hkv, T, d), dtype=np.float32) * vs[:, None]
        Ks.append(K)
        Vs.append(V)
    for s, T in enumerate(lengths):
        nb = T // 64
        npl = int(planted * nb)
        if npl:
            for h in range(Hkv):
                u = W.group_direction(q[s, h * G:(h + 1) * G])
                for j in rng.choice(nb, size=npl, replace=False):
                    Ks[s][h, j * 64:(j + 1) * 64] += 2.0 * u
        Ks[s] = W.quantize(Ks[s], st)
        Vs[s] = W.quantize(Vs[s], st)
    Wg = None
    if desc_kind == MEAN:
        Wg = W.quantize(rng.standard_normal((d, d), dtype=np.float32) / np.sqrt(d), "bf16")
    return q, Ks, Vs, Wg


def run_select_decode(L, cache, q_dev, P, scale=None):
    torch = _torch()
    dev = q_dev.device
    idx = torch.full((L.B, L.Hkv, P.n_max), -7, dtype=torch.int32, device=dev)
    cnt = torch.full((L.B, L.Hkv), -7, dtype=torch.int32, device=dev)
    ws = torch.empty(max(bsa.workspace_size(L, bsa.OP_SELECT, P.n_max),
                         bsa.workspace_size(L, bsa.OP_DECODE, P.n_max)),
                     dtype=torch.uint8, device=dev)
    ws.view(torch.float32)[: ws.numel() // 4].fill_(float("nan"))  # poison
    bsa.select_blocks(L, cache, q_dev, P, idx, cnt, ws)
    o = torch.full((L.B, L.Hq, L.d), float("nan"), dtype=q_dev.dtype, device=dev)
    lse = torch.full((L.B, L.Hq), float("nan"), dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(L.d) if scale is None else scale
    bsa.sparse_decode(L, cache, q_dev, idx, cnt, P.n_max, scale, o, lse, ws)
    torch.cuda.synchronize()
    return idx, cnt, o, lse


# --------------------------------------------------------------------------
# Cache writes and descriptors
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,d,blk,kind", [(BF16, 128, 64, MINMAX), (BF16, 64, 128, MEAN),
                                              (F32, 64, 64, MINMAX), (BF16, 128, 32, MINMAX),
                                              (F32, 128, 256, MEAN)])
def test_append_writes_layout_and_descriptors(dtype, d, blk, kind):
    """Bulk prefill + one-token appends land in the documented page layout
    (read back exactly); descriptors equal the oracle's (min/max bit-exact,
    mean within fp32 rounding); a from-scratch rebuild gives bit-identical
    descriptors."""
    torch = _torch()
    lengths0 = [150, 333]
    extra = 70
    Hkv, Hq = 2, 4
    total = [t + extra for t in lengths0]
    max_blocks = (max(total) + blk - 1) // blk + 1
    L = bsa.Layout(2, Hq, Hkv, d, blk, max_blocks, dtype, kind)
    q, Ks, Vs, _ = make_inputs(7, 2, Hq, Hkv, d, total, dtype, kind)
    cache = bsa.allocate_cache(L, page_table=random_page_table(L, 3))
    cache.k_pool.fill_(float("nan"))
    cache.v_pool.fill_(float("nan"))
    prefill(L, cache, Ks, Vs, lengths0)
    for step in range(extra):
        cache.seq_lens += 1
        kn = np.stack([Ks[s][:, lengths0[s] + step] for s in range(2)])[:, :, None]
        vn = np.stack([Vs[s][:, lengths0[s] + step] for s in range(2)])[:, :, None]
        bsa.build_block_desc(L, cache, to_dev(kn, L), to_dev(vn, L), 1)
    torch.cuda.synchronize()
    desc_append = cache.desc.clone()
    for s in range(2):
        K, V = read_cache(L, cache, s, total[s])
        assert np.array_equal(K, Ks[s]) and np.array_equal(V, Vs[s])
        NB = (total[s] + blk - 1) // blk
        for h in range(Hkv):
            if kind == MINMAX:
                mn, mx = O.desc_minmax(Ks[s][h], blk)
                got = cache.desc[s, h, :NB].float().cpu().numpy()
                assert np.array_equal(got[:, 0], mn) and np.array_equal(got[:, 1], mx)
            else:
                mean = O.desc_mean(Ks[s][h], blk)
                cnts = np.minimum(blk, total[s] - np.arange(NB) * blk)[:, None]
                got = cache.desc[s, h, :NB].cpu().numpy() / cnts
                np.testing.assert_allclose(got, mean, rtol=2e-6, atol=2e-6)
    # rebuild everything from the cache contents
    cache.desc.zero_()
    bsa.build_block_desc(L, cache, None, None, 0, None)
    torch.cuda.synchronize()
    for s in range(2):
        NB = (total[s] + blk - 1) // blk
        assert torch.equal(cache.desc[s, :, :NB], desc_append[s, :, :NB])
    # rebuild only a suffix range
    rb = torch.tensor([total[0] - 5, 0], dtype=torch.int32, device="cuda")
    cache.desc[0].zero_()
    bsa.build_block_desc(L, cache, None, None, 0, rb)
    torch.cuda.synchronize()
    NB0 = (total[0] + blk - 1) // blk
    j0 = (total[0] - 5) // blk
    assert torch.equal(cache.desc[0, :, j0:NB0], desc_append[0, :, j0:NB0])
    assert torch.all(cache.desc[0, :, :j0] == 0)


# --------------------------------------------------------------------------
# Select + decode, one step, many shapes
# --------------------------------------------------------------------------

CASES = [
    # dtype, d, blk, kind, Hq, Hkv, lengths, budget, bp, n_local, n_min
    (BF16, 128, 64, MINMAX, 8, 2, [1000, 1537], 256, 0, 1, 0),
    (BF16, 128, 64, MINMAX, 32, 8, [4099], 0, 9000, 2, 16),
    (BF16, 128, 128, MEAN, 8, 2, [3000, 2049], 0, 9000, 2, 0),
    (BF16, 64, 64, MINMAX, 16, 1, [2500], 512, 0, 1, 2),
    (BF16, 128, 32, MINMAX, 4, 4, [777, 1025, 64, 65], 0, 8000, 1, 3),
    (BF16, 128, 256, MINMAX, 8, 4, [5000, 1], 0, 9500, 1, 4),
    (BF16, 64, 64, MEAN, 2, 2, [1900], 0, 9000, 3, 0),
    (F32, 64, 64, MINMAX, 4, 1, [2049], 512, 0, 1, 2),
    (F32, 128, 128, MEAN, 8, 2, [1500, 700], 0, 9000, 2, 0),
    # mid-size rows (about 1900 and 3100 candidates)
    (BF16, 64, 32, MINMAX, 4, 1, [60000], 0, 9000, 1, 2),
    (BF16, 64, 32, MINMAX, 8, 2, [98000, 40000], 0, 9500, 2, 4),
    # groups of 3, 5 and 7 query heads (operand columns past G stay empty)
    (BF16, 128, 64, MINMAX, 6, 2, [3100, 777], 0, 9000, 2, 3),
    (BF16, 64, 32, MEAN, 10, 2, [1200, 2500], 256, 0, 1, 0),
    (F32, 64, 64, MINMAX, 7, 1, [1500], 0, 8500, 1, 2),
    # 33 x 8 = 264 groups: one split per group, so the merge kernel sees S = 1
    (BF16, 64, 64, MINMAX, 16, 8, [100 + 97 * i for i in range(33)], 512, 0, 1, 2),
    # fp32 min/max scoring launches of 316 and 280 workgroups (at least 256:
    # each lane forms its own query weights)
    (F32, 128, 32, MINMAX, 8, 2, [80000, 3000], 0, 9000, 2, 4),
    (F32, 64, 32, MINMAX, 16, 4, [70000, 5000], 1024, 0, 1, 2),
]


@pytest.mark.parametrize("case", CASES, ids=[f"c{i}" for i in range(len(CASES))])
def test_select_decode_parity(case):
    torch = _torch()
    dtype, d, blk, kind, Hq, Hkv, lengths, budget, bp, nl, nm = case
    B = len(lengths)
    max_blocks = (max(lengths) + blk - 1) // blk + 2
    L = bsa.Layout(B, Hq, Hkv, d, blk, max_blocks, dtype, kind)
    P = bsa.SelectParams(budget_tokens=budget, sparsity_bp=bp, n_local=nl, n_min=nm)
    P.n_max = bsa.block_count(P, max_blocks, blk)
    q, Ks, Vs, Wg = make_inputs(11 + len(lengths), B, Hq, Hkv, d, lengths, dtype, kind)
    enforce_gap(L, P, q, Ks, [[T] for T in lengths], W_gate=Wg)
    cache = bsa.allocate_cache(L, page_table=random_page_table(L, 5))
    cache.k_pool.fill_(float("nan"))
    cache.v_pool.fill_(float("nan"))
    prefill(L, cache, Ks, Vs, lengths)
    if Wg is not None:
        P.gate_w = to_dev(Wg, bsa.Layout(1, 1, 1, d, blk, 1, BF16))
    idx, cnt, o, lse = run_select_decode(L, cache, to_dev(q, L), P)
    ref = oracle_decode(P, q, Ks, Vs, lengths, L, W_gate=Wg)
    eo, el = compare_step(L, idx, cnt, o, lse, ref)
    if dtype == F32:
        assert eo <= 1e-4, eo  # fp32 I/O diagnostic bar


def test_select_decode_at_the_longest_row():
    """The longest row the top-n accepts: max_blocks = 32768 (32 keys per
    thread), one sequence of about 1M tokens at b = 32 with a partial last
    block, p = 0.9 (3277 kept blocks, 256 splits)."""
    d, blk, Hq, Hkv = 64, 32, 4, 1
    max_blocks = 32768
    T = max_blocks * blk - 40
    L = bsa.Layout(1, Hq, Hkv, d, blk, max_blocks, BF16, MINMAX)
    P = bsa.SelectParams(sparsity_bp=9000, n_local=2, n_min=16)
    P.n_max = bsa.block_count(P, max_blocks, blk)
    q, Ks, Vs, _ = make_inputs(202, 1, Hq, Hkv, d, [T], BF16, MINMAX)
    enforce_gap(L, P, q, Ks, [[T]])
    cache = bsa.allocate_cache(L, page_table=random_page_table(L, 6))
    prefill(L, cache, Ks, Vs, [T])
    idx, cnt, o, lse = run_select_decode(L, cache, to_dev(q, L), P)
    ref = oracle_decode(P, q, Ks, Vs, [T], L)
    compare_step(L, idx, cnt, o, lse, ref)
    assert int(cnt[0, 0]) == P.n_max


@pytest.mark.parametrize("dtype,d,blk,kind", [(BF16, 128, 64, MINMAX), (BF16, 64, 128, MEAN),
                                              (F32, 64, 32, MINMAX)])
def test_append_select_equals_the_two_calls(dtype, d, blk, kind):
    """bsa_append_select gives the cache, descriptors, idx and cnt of
    bsa_build_block_desc (one token) followed by bsa_select_blocks, over
    several steps that open and fill blocks."""
    torch = _torch()
    lengths = [blk * 9 - 2, blk * 5 + 3]
    Hq, Hkv = 8, 2
    B = len(lengths)
    max_blocks = (max(lengths) + 8 + blk - 1) // blk + 1
    L = bsa.Layout(B, Hq, Hkv, d, blk, max_blocks, dtype, kind)
    P = bsa.SelectParams(budget_tokens=0, sparsity_bp=8000, n_local=1, n_min=2)
    P.n_max = bsa.block_count(P, max_blocks, blk)
    q, Ks, Vs, Wg = make_inputs(77, B, Hq, Hkv, d, [T + 8 for T in lengths], dtype, kind)
    if Wg is not None:
        P.gate_w = to_dev(Wg, bsa.Layout(1, 1, 1, d, blk, 1, BF16))
    caches = []
    for _ in range(2):
        c = bsa.allocate_cache(L, page_table=random_page_table(L, 3))
        c.k_pool.zero_()
        c.v_pool.zero_()
        c.desc.zero_()
        prefill(L, c, Ks, Vs, lengths)
        caches.append(c)
    ws = torch.empty(bsa.workspace_size(L, bsa.OP_SELECT, P.n_max), dtype=torch.uint8, device="cuda")
    q_dev = to_dev(q, L)
    for step in range(8):
        kn = to_dev(np.stack([Ks[s][:, lengths[s] + step] for s in range(B)])[:, :, None], L)
        vn = to_dev(np.stack([Vs[s][:, lengths[s] + step] for s in range(B)])[:, :, None], L)
        out = []
        for which, c in enumerate(caches):
            c.seq_lens += 1
            idx = torch.full((B, Hkv, P.n_max), -7, dtype=torch.int32, device="cuda")
            cnt = torch.full((B, Hkv), -7, dtype=torch.int32, device="cuda")
            if which == 0:
                bsa.build_block_desc(L, c, kn, vn, 1)
                bsa.select_blocks(L, c, q_dev, P, idx, cnt, ws)
            else:
                bsa.append_select(L, c, kn, vn, q_dev, P, idx, cnt, ws)
            torch.cuda.synchronize()
            out.append((idx.clone(), cnt.clone()))
        assert torch.equal(out[0][0], out[1][0]) and torch.equal(out[0][1], out[1][1]), step
        assert torch.equal(caches[0].k_pool, caches[1].k_pool)
        assert torch.equal(caches[0].v_pool, caches[1].v_pool)
        assert torch.equal(caches[0].desc, caches[1].desc)


def test_topn_long_row_of_ties():
    """About 8000 candidates whose scores are almost all equal: the threshold
    digit then holds thousands of keys after the first radix pass, which
    exercises the whole-workgroup passes (the gathered-list path covers the
    other cases).  Ties go to the lower block index on both sides."""
    torch = _torch()
    d, blk, Hq, Hkv = 64, 32, 4, 1
    T = 8000 * blk + 17
    L = bsa.Layout(1, Hq, Hkv, d, blk, (T + blk - 1) // blk + 1, BF16, MINMAX)
    P = bsa.SelectParams(budget_tokens=0, sparsity_bp=9000, n_local=1, n_min=0)
    P.n_max = bsa.block_count(P, L.max_blocks, blk)
    rng = np.random.Generator(np.random.PCG64(123))
    q = W.quantize(rng.standard_normal((1, Hq, d), dtype=np.float32), "bf16")
    u = W.group_direction(q[0])
    tmpl = rng.standard_normal((blk, d), dtype=np.float32)
    K = np.tile(tmpl, ((T + blk - 1) // blk, 1))[:T].copy()
    K[-17:] = rng.standard_normal((17, d), dtype=np.float32)
    for j in (7, 1000, 4321, 7777, 7990):   # clearly above the tied mass
        K[j * blk:(j + 1) * blk] += 3.0 * u
    for j in (3, 2500, 6000):               # clearly below it
        K[j * blk:(j + 1) * blk] -= 3.0 * u
    K = W.quantize(K, "bf16")[None]
    V = W.quantize(rng.standard_normal((1, T, d), dtype=np.float32), "bf16")
    cache = bsa.allocate_cache(L, page_table=random_page_table(L, 8))
    prefill(L, cache, [K], [V], [T])
    idx, cnt, o, lse = run_select_decode(L, cache, to_dev(q, L), P)
    ref = oracle_decode(P, q, [K], [V], [T], L)
    compare_step(L, idx, cnt, o, lse, ref)
    ridx = ref[(0, 0)][0]
    assert {7, 1000, 4321, 7777, 7990} <= set(ridx.tolist())


def test_dense_when_budget_covers_context():
    """Budget >= context: every block kept, equal to dense attention."""
    dtype, d, blk = BF16, 128, 64
    lengths = [700, 1283]
    L = bsa.Layout(2, 8, 2, d, blk, 25, dtype, MINMAX)
    P = bsa.SelectParams(budget_tokens=25 * 64, n_local=1)
    P.n_max = 25
    q, Ks, Vs, _ = make_inputs(21, 2, 8, 2, d, lengths, dtype, MINMAX)
    cache = bsa.allocate_cache(L, page_table=random_page_table(L, 9))
    prefill(L, cache, Ks, Vs, lengths)
    idx, cnt, o, lse = run_select_decode(L, cache, to_dev(q, L), P)
    G = 4
    for s, T in enumerate(lengths):
        NB = (T + blk - 1) // blk
        for h in range(2):
            assert cnt[s, h].item() == NB
            assert idx[s, h, :NB].cpu().numpy().tolist() == list(range(NB))
            for g in range(G):
                ro, rl = O.dense_attend(q[s, h * G + g], Ks[s][h], Vs[s][h], T, 1 / math.sqrt(d))
                assert np.abs(o[s, h * G + g].float().cpu().numpy() - ro).max() <= 2e-2
                assert abs(lse[s, h * G + g].item() - rl) <= 1e-4 * max(1, abs(rl))


def test_decode_deterministic_and_split_invariant():
    """Two identical runs are bit-identical; a different n_max (hence a
    different split count) agrees within the tolerance."""
    torch = _torch()
    d, blk = 128, 64
    lengths = [6000, 4100]
    L = bsa.Layout(2, 32, 8, d, blk, 100, BF16, MINMAX)
    P = bsa.SelectParams(sparsity_bp=9000, n_local=2, n_min=16)
    P.n_max = bsa.block_count(P, 100, blk)
    q, Ks, Vs, _ = make_inputs(31, 2, 32, 8, d, lengths, BF16, MINMAX)
    enforce_gap(L, P, q, Ks, [[T] for T in lengths])
    cache = bsa.allocate_cache(L, page_table=random_page_table(L, 2))
    prefill(L, cache, Ks, Vs, lengths)
    qd = to_dev(q, L)
    a = run_select_decode(L, cache, qd, P)
    b = run_select_decode(L, cache, qd, P)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    P2 = bsa.SelectParams(sparsity_bp=9000, n_local=2, n_min=16, n_max=100)
    c = run_select_decode(L, cache, qd, P2)
    assert torch.equal(a[1], c[1])
    assert torch.equal(a[0], c[0][:, :, :P.n_max])
    assert (a[2].float() - c[2].float()).abs().max().item() <= 2e-2
    assert ((a[3] - c[3]).abs() / a[3].abs().clamp_min(1)).max().item() <= 1e-4


# --------------------------------------------------------------------------
# A short decode loop: append, select, decode, every step
# --------------------------------------------------------------------------

def test_tiny_fp32_decode_loop():
    """The tiny fp32 workload: 1 KV head, 4 query heads, d = 64, 2048-token
    context, blocks of 64, 512-token budget (8 blocks incl. the local one),
    minimum 2, three planted blocks, 16 decode steps appending one token."""
    torch = _torch()
    w = W.get("tiny")
    hi = W.make_host(w)
    L = bsa.Layout(w.B, w.Hq, w.Hkv, w.d, w.block, w.max_blocks() + 1, F32, MINMAX)
    P = bsa.SelectParams(budget_tokens=w.budget_tokens, n_local=w.n_local, n_min=w.n_min)
    P.n_max = bsa.block_count(P, L.max_blocks, w.block)
    steps = [[w.T0[0] + k + 1 for k in range(w.steps)]]
    enforce_gap(L, P, hi.q, hi.K, steps)
    cache = bsa.allocate_cache(L, page_table=random_page_table(L, 1))
    prefill(L, cache, hi.K, hi.V, [w.T0[0]])
    qd = to_dev(hi.q, L)
    for k in range(w.steps):
        T = w.T0[0] + k + 1
        cache.seq_lens += 1
        bsa.build_block_desc(L, cache, to_dev(hi.K[0][:, T - 1:T][None], L),
                             to_dev(hi.V[0][:, T - 1:T][None], L), 1)
        idx, cnt, o, lse = run_select_decode(L, cache, qd, P)
        ref = oracle_decode(P, hi.q, hi.K, hi.V, [T], L)
        eo, _ = compare_step(L, idx, cnt, o, lse, ref)
        assert eo <= 1e-4
        # the planted blocks are the ones kept
        assert set(hi.planted[0].tolist()) <= set(idx[0, 0, :cnt[0, 0]].cpu().numpy().tolist())


# --------------------------------------------------------------------------
# Rectification
# --------------------------------------------------------------------------

@pytest.mark.parametrize("dtype,d,blk,f,lengths,Hq,Hkv", [
    (BF16, 128, 64, 32, [300, 517], 8, 2),
    (BF16, 128, 64, 16, [2100], 8, 2),
    (BF16, 128, 128, 64, [4500, 200, 64], 8, 2),
    (BF16, 64, 64, 1, [129], 8, 2),
    (F32, 64, 64, 32, [300, 97], 8, 2),
    (BF16, 128, 32, 33, [1000], 8, 2),
    (BF16, 128, 64, 128, [3000, 700], 8, 2),   # 512 rows per KV head: two row groups
    (BF16, 64, 64, 20, [1500], 16, 1),         # G = 16: 320 rows, a partial second group
    (BF16, 128, 64, 16, [900, 1300], 2, 2),    # G = 1: 16 rows (the 4-wave shape)
])
def test_rectify_parity(dtype, d, blk, f, lengths, Hq, Hkv):
    """Overwrite + descriptor refresh + causal dense attention of the f
    queries, against the oracle (all rows)."""
    torch = _torch()
    B = len(lengths)
    G = Hq // Hkv
    max_blocks = (max(lengths) + blk - 1) // blk + 1
    L = bsa.Layout(B, Hq, Hkv, d, blk, max_blocks, dtype, MINMAX)
    q0, Ks, Vs, _ = make_inputs(41 + f, B, Hq, Hkv, d, lengths, dtype, MINMAX)
    st = "bf16" if dtype == BF16 else "f32"
    rng = np.random.Generator(np.random.PCG64(99))
    qr = W.quantize(rng.standard_normal((B, Hq, f, d), dtype=np.float32), st)
    kn = [W.quantize(Ks[s][:, T - f:T] + 0.1 * rng.standard_normal((Hkv, f, d), dtype=np.float32), st)
          for s, T in enumerate(lengths)]
    vn = [W.quantize(Vs[s][:, T - f:T] + 0.1 * rng.standard_normal((Hkv, f, d), dtype=np.float32), st)
          for s, T in enumerate(lengths)]
    cache = bsa.allocate_cache(L, page_table=random_page_table(L, 4))
    prefill(L, cache, Ks, Vs, lengths)
    # pad the per-sequence k_new to [B, Hkv, f, d]
    kn_d = to_dev(np.stack(kn), L)
    vn_d = to_dev(np.stack(vn), L)
    ws = torch.empty(bsa.workspace_size(L, bsa.OP_RECTIFY, f), dtype=torch.uint8, device="cuda")
    o = torch.full((B, Hq, f, d), float("nan"), dtype=torch_dtype_of(L), device="cuda")
    lse = torch.full((B, Hq, f), float("nan"), dtype=torch.float32, device="cuda")
    scale = 1 / math.sqrt(d)
    bsa.rectify_chunk(L, cache, to_dev(qr, L), kn_d, vn_d, f, scale, o, lse, ws)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    worst = 0.0
    for s, T in enumerate(lengths):
        for h in range(Hkv):
            K = np.ascontiguousarray(Ks[s][h].copy())
            V = np.ascontiguousarray(Vs[s][h].copy())
            ro, rl = O.rectify(qr[s, h * G:(h + 1) * G], K, V, kn[s][h], vn[s][h], scale)
            err = np.abs(o[s, h * G:(h + 1) * G] - ro).max()
            worst = max(worst, err)
            assert err <= (2e-2 if dtype == BF16 else 1e-4), (s, h, err)
            rel = np.abs(lse[s, h * G:(h + 1) * G] - rl) / np.maximum(1, np.abs(rl))
            assert rel.max() <= 1e-4
            # cache rewritten and descriptors refreshed
            Kc, Vc = read_cache(L, cache, s, T)
            assert np.array_equal(Kc[h], K) and np.array_equal(Vc[h], V)
            mn, mx = O.desc_minmax(K, blk)
            NB = (T + blk - 1) // blk
            got = cache.desc[s, h, :NB].float().cpu().numpy()
            assert np.array_equal(got[:, 0], mn) and np.array_equal(got[:, 1], mx)


def torch_dtype_of(L):
    torch = _torch()
    return torch.bfloat16 if L.kv_dtype == BF16 else torch.float32


@pytest.mark.parametrize("dtype,gated", [(BF16, False), (BF16, True), (F32, False)])
def test_empty_sequences_in_a_ragged_batch(dtype, gated):
    """Sequences with seq_lens = 0 next to non-empty ones: the empty groups
    keep no block (cnt 0, idx all -1, bias 0) and attend to nothing (o = 0,
    lse = -inf, as documented); the others equal the oracle."""
    torch = _torch()
    d, blk, Hq, Hkv = 64, 64, 8, 2
    lengths = [0, 700, 0, 65]
    B = len(lengths)
    max_blocks = 14
    L = bsa.Layout(B, Hq, Hkv, d, blk, max_blocks, dtype, MINMAX)
    P = bsa.SelectParams(sparsity_bp=8000, n_local=1, n_min=2)
    P.n_max = bsa.block_count(P, max_blocks, blk)
    q, Ks, Vs, _ = make_inputs(303, B, Hq, Hkv, d, lengths, dtype, MINMAX)
    enforce_gap(L, P, q, Ks, [[T] for T in lengths])
    cache = bsa.allocate_cache(L, page_table=random_page_table(L, 7))
    prefill(L, cache, Ks, Vs, lengths)
    cache.seq_lens.copy_(torch.tensor(lengths, dtype=torch.int32, device="cuda"))
    q_dev = to_dev(q, L)
    idx = torch.full((B, Hkv, P.n_max), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, Hkv), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(bsa.workspace_size(L, bsa.OP_SELECT, P.n_max),
                         bsa.workspace_size(L, bsa.OP_DECODE, P.n_max)),
                     dtype=torch.uint8, device="cuda")
    ws.view(torch.float32)[: ws.numel() // 4].fill_(float("nan"))
    if gated:
        P.gate_tau = 0.01
        P.gate_bias = torch.full((B, Hkv, P.n_max), float("nan"), dtype=torch.float32,
                                 device="cuda")
    bsa.select_blocks(L, cache, q_dev, P, idx, cnt, ws)
    o = torch.full((B, Hq, d), float("nan"), dtype=q_dev.dtype, device="cuda")
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    if gated:
        bsa.sparse_decode_gated(L, cache, q_dev, idx, cnt, P.gate_bias, P.n_max,
                                1 / math.sqrt(d), o, lse, ws)
    else:
        bsa.sparse_decode(L, cache, q_dev, idx, cnt, P.n_max, 1 / math.sqrt(d), o, lse, ws)
    torch.cuda.synchronize()
    G = Hq // Hkv
    for s in (0, 2):
        assert cnt[s].tolist() == [0, 0]
        assert torch.all(idx[s] == -1)
        assert torch.all(o[s] == 0)
        assert torch.all(torch.isneginf(lse[s]))
        if gated:
            assert torch.all(P.gate_bias[s] == 0)
    live = [1, 3]
    if gated:
        ref = {}
        for s in live:
            for h in range(Hkv):
                r_idx, r_o, r_lse, _ = O.decode_group_gated(
                    q[s, h * G:(h + 1) * G], Ks[s][h, :lengths[s]], Vs[s][h, :lengths[s]], blk,
                    0, 0.01, sparsity_bp=8000, n_local=1, n_min=2, scale=1 / math.sqrt(d))
                ref[(s, h)] = (r_idx, r_o, r_lse)
    else:
        ref = oracle_decode(P, q[live], [Ks[s] for s in live], [Vs[s] for s in live],
                            [lengths[s] for s in live], L)
        ref = {(live[s], h): v for (s, h), v in ref.items()}
    compare_step(L, idx, cnt, o, lse, ref)


# --------------------------------------------------------------------------
# A ReSA decode loop in bf16: fused append + select, decode, rectify every f
# --------------------------------------------------------------------------

@pytest.mark.parametrize("gated", [False, True])
def test_resa_decode_loop(gated):
    """24 decode steps on a ragged batch (blocks of 32, so appends open new
    blocks), a rectification every f = 8 steps, all through the C ABI, each
    step checked against the oracle on a host copy that follows the rectify
    rewrites.  No score gap is enforced here (rewrites change blocks that
    later become candidates), so where the selections differ the GPU's set
    must be a valid top-n within the gap tolerance and o / lse are checked
    against the oracle's attention over that same set; exact agreement must
    still be the large majority."""
    torch = _torch()
    d, blk, Hq, Hkv, f, steps = 64, 32, 8, 2, 8, 24
    T0 = [700, 333]
    B, G = len(T0), Hq // Hkv
    tau, scale = 0.02, 1 / math.sqrt(d)
    total = [t + steps for t in T0]
    max_blocks = (max(total) + blk - 1) // blk + 1
    L = bsa.Layout(B, Hq, Hkv, d, blk, max_blocks, BF16, MINMAX)
    P = bsa.SelectParams(sparsity_bp=8000, n_local=2, n_min=2)
    P.n_max = bsa.block_count(P, max_blocks, blk)
    q, Ks, Vs, _ = make_inputs(404 + gated, B, Hq, Hkv, d, total, BF16, MINMAX)
    rng = np.random.Generator(np.random.PCG64(405))
    cache = bsa.allocate_cache(L, page_table=random_page_table(L, 11))
    prefill(L, cache, Ks, Vs, T0)
    q_dev = to_dev(q, L)
    dev = "cuda"
    idx = torch.empty((B, Hkv, P.n_max), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, Hkv), dtype=torch.int32, device=dev)
    ws = torch.empty(max(bsa.workspace_size(L, bsa.OP_SELECT, P.n_max),
                         bsa.workspace_size(L, bsa.OP_DECODE, P.n_max),
                         bsa.workspace_size(L, bsa.OP_RECTIFY, f)), dtype=torch.uint8, device=dev)
    o = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    bias = torch.empty((B, Hkv, P.n_max), dtype=torch.float32, device=dev)
    if gated:
        P.gate_tau, P.gate_bias = tau, bias
    exact = near = 0
    for k in range(steps):
        T = [t + k + 1 for t in T0]
        cache.seq_lens += 1
        kn = to_dev(np.stack([Ks[s][:, T[s] - 1] for s in range(B)])[:, :, None], L)
        vn = to_dev(np.stack([Vs[s][:, T[s] - 1] for s in range(B)])[:, :, None], L)
        bsa.append_select(L, cache, kn, vn, q_dev, P, idx, cnt, ws)
        if gated:
            bsa.sparse_decode_gated(L, cache, q_dev, idx, cnt, bias, P.n_max, scale, o, lse, ws)
        else:
            bsa.sparse_decode(L, cache, q_dev, idx, cnt, P.n_max, scale, o, lse, ws)
        torch.cuda.synchronize()
        gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
        go, gl, gb = o.float().cpu().numpy(), lse.cpu().numpy(), bias.cpu().numpy()
        for s in range(B):
            NB = (T[s] + blk - 1) // blk
            NC = NB - 2
            for h in range(Hkv):
                K, V = Ks[s][h, :T[s]], Vs[s][h, :T[s]]
                qg = q[s, h * G:(h + 1) * G]
                ridx, _, _, sc = O.decode_group(qg, K, V, blk, 0, sparsity_bp=8000, n_local=2,
                                                n_min=2, scale=scale, want_scores=True)
                c = int(gc[s, h])
                sel = gi[s, h, :c]
                assert c == len(ridx) and np.all(gi[s, h, c:] == -1)
                if np.array_equal(sel, ridx):
                    exact += 1
                else:
                    near += 1
                    mn, mx = O.desc_minmax(K, blk)
                    mag = (np.abs(qg.astype(np.float64)).sum(0)[None, :] *
                           np.maximum(np.abs(mn), np.abs(mx))).sum(1)
                    kept = [j for j in sel if j < NC]
                    dropped = [j for j in range(NC) if j not in set(kept)]
                    assert list(sel[len(kept):]) == list(range(NC, NB))
                    if kept and dropped:
                        lo_k = min(sc[j] for j in kept)
                        hi_d = max(sc[j] for j in dropped)
                        tol = 1e-3 * max(1.0, abs(lo_k), mag[kept].max(), mag[dropped].max())
                        assert lo_k >= hi_d - tol, (k, s, h, lo_k, hi_d)
                if gated:
                    # the page's partition: only the last block is current, so
                    # the older local block is historical (scored and gated)
                    mn, mx = O.desc_minmax(K, blk)
                    sh = O.score_quest(qg, mn, mx)[:NB - 1]
                    rb = O.gate_bias(sh, NB, 1, tau, sel)
                    smax = float(np.abs(sh).max()) if NB > 1 else 0.0
                    assert np.abs(gb[s, h, :c] - rb).max() <= tau * 2e-5 * smax + 1e-4 + NB * 1.2e-7
                for g in range(G):
                    if gated:
                        ro, rl = O.attend_biased(qg[g], K, V, blk, sel, rb, scale)
                    else:
                        ro, rl = O.attend(qg[g], K, V, blk, sel, scale)
                    assert np.abs(go[s, h * G + g] - ro).max() <= 2e-2, (k, s, h, g)
                    assert abs(gl[s, h * G + g] - rl) <= 1e-4 * max(1.0, abs(rl)), (k, s, h, g)
        if (k + 1) % f == 0:
            qr = W.quantize(rng.standard_normal((B, Hq, f, d), dtype=np.float32), "bf16")
            kr = [W.quantize(Ks[s][:, T[s] - f:T[s]] +
                             0.1 * rng.standard_normal((Hkv, f, d), dtype=np.float32), "bf16")
                  for s in range(B)]
            vr = [W.quantize(Vs[s][:, T[s] - f:T[s]] +
                             0.1 * rng.standard_normal((Hkv, f, d), dtype=np.float32), "bf16")
                  for s in range(B)]
            o_r = torch.empty((B, Hq, f, d), dtype=torch.bfloat16, device=dev)
            lse_r = torch.empty((B, Hq, f), dtype=torch.float32, device=dev)
            bsa.rectify_chunk(L, cache, to_dev(qr, L), to_dev(np.stack(kr), L),
                              to_dev(np.stack(vr), L), f, scale, o_r, lse_r, ws)
            torch.cuda.synchronize()
            o_r, lse_r = o_r.float().cpu().numpy(), lse_r.cpu().numpy()
            for s in range(B):
                for h in range(Hkv):
                    # the host copy follows the rewrite (the oracle writes in place)
                    ro, rl = O.rectify(qr[s, h * G:(h + 1) * G], Ks[s][h, :T[s]], Vs[s][h, :T[s]],
                                       kr[s][h], vr[s][h], scale)
                    assert np.abs(o_r[s, h * G:(h + 1) * G] - ro).max() <= 2e-2
                    assert (np.abs(lse_r[s, h * G:(h + 1) * G] - rl) /
                            np.maximum(1, np.abs(rl))).max() <= 1e-4
    print(f"selection: {exact} exact, {near} near-tie", flush=True)
    assert exact >= 0.75 * (exact + near), (exact, near)
    # the cache and its descriptors end equal to the host copy
    for s in range(B):
        Kc, Vc = read_cache(L, cache, s, total[s])
        assert np.array_equal(Kc, Ks[s]) and np.array_equal(Vc, Vs[s])
        NB = (total[s] + blk - 1) // blk
        for h in range(Hkv):
            mn, mx = O.desc_minmax(Ks[s][h], blk)
            got = cache.desc[s, h, :NB].float().cpu().numpy()
            assert np.array_equal(got[:, 0], mn) and np.array_equal(got[:, 1], mx)

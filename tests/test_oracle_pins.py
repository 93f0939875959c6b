"""Pins of the fp64 oracle against facts that do not come from the oracle
itself: brute force on tiny inputs, closed forms, invariants, and library
routines (torch's scaled-dot-product attention, scipy's logsumexp, Python's
sort).  CPU only.

Each test names the plausible oracle mistakes it would catch."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


# --------------------------------------------------------------------------
# Descriptors
# --------------------------------------------------------------------------

@pytest.mark.parametrize("T,b,d", [(1, 4, 3), (7, 4, 5), (64, 16, 8), (130, 64, 6)])
def test_minmax_desc_is_tight_box(T, b, d):
    """Every key of block j lies inside [mn_j, mx_j] and both bounds are
    attained by some key of the block.  Catches: off-by-one block ranges,
    partial-last-block overrun, swapped min/max, wrong channel index."""
    K = rng(T * 7 + d).standard_normal((T, d)).astype(np.float32)
    mn, mx = O.desc_minmax(K, b)
    NB = (T + b - 1) // b
    assert mn.shape == (NB, d)
    for j in range(NB):
        blk = K[j * b:min((j + 1) * b, T)].astype(np.float64)
        assert np.all(blk >= mn[j]) and np.all(blk <= mx[j])
        assert np.all(np.any(blk == mn[j], axis=0))
        assert np.all(np.any(blk == mx[j], axis=0))


@pytest.mark.parametrize("T,b,d", [(5, 2, 3), (64, 16, 8), (129, 64, 4)])
def test_mean_desc_matches_numpy_mean(T, b, d):
    """Mean-pooled key = numpy's mean over the block's present tokens.
    Catches: dividing by b instead of the partial count, range errors."""
    K = rng(T + b).standard_normal((T, d)).astype(np.float32)
    mean = O.desc_mean(K, b)
    for j in range((T + b - 1) // b):
        ref = K[j * b:min((j + 1) * b, T)].astype(np.float64).mean(axis=0)
        np.testing.assert_allclose(mean[j], ref, rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------
# Quest score
# --------------------------------------------------------------------------

@pytest.mark.parametrize("d,G", [(3, 1), (6, 2), (10, 4)])
def test_quest_score_equals_box_corner_enumeration(d, G):
    """The per-head Quest score is the maximum of q.c over all 2^d corners c
    of the block's channel-wise box (brute force); the group score sums the
    heads.  Catches: min instead of max, a dropped head, transposed indexing
    of q or of the descriptor, a sign error."""
    r = rng(100 + d * G)
    T, b = 5 * 8, 8
    K = r.standard_normal((T, d)).astype(np.float32)
    q = r.standard_normal((G, d)).astype(np.float32)
    mn, mx = O.desc_minmax(K, b)
    s = O.score_quest(q, mn, mx)
    for j in range(T // b):
        total = 0.0
        for h in range(G):
            best = -math.inf
            for corner in itertools.product((0, 1), repeat=d):
                c = np.where(np.array(corner) == 1, mx[j], mn[j])
                best = max(best, float(np.dot(q[h].astype(np.float64), c)))
            total += best
        assert abs(s[j] - total) <= 1e-12 * max(1.0, abs(total))


def test_quest_score_bounds_every_key():
    """For every head, the score is >= q.k for each key in the block (it is
    an upper bound).  Summed over the group likewise."""
    r = rng(7)
    T, b, d, G = 256, 32, 16, 4
    K = r.standard_normal((T, d)).astype(np.float32)
    q = r.standard_normal((G, d)).astype(np.float32)
    mn, mx = O.desc_minmax(K, b)
    for h in range(G):
        s = O.score_quest(q[h:h + 1], mn, mx)
        dots = (K.astype(np.float64) @ q[h].astype(np.float64)).reshape(T // b, b)
        assert np.all(s >= dots.max(axis=1) - 1e-12)


def test_quest_score_block_size_one_is_dot_product():
    """With b = 1 the box degenerates to the key, so the score is the exact
    sum over heads of q_h.k.  Catches a missing term in the max."""
    r = rng(11)
    T, d, G = 40, 12, 3
    K = r.standard_normal((T, d)).astype(np.float32)
    q = r.standard_normal((G, d)).astype(np.float32)
    mn, mx = O.desc_minmax(K, 1)
    s = O.score_quest(q, mn, mx)
    ref = K.astype(np.float64) @ q.astype(np.float64).sum(axis=0)
    np.testing.assert_allclose(s, ref, rtol=1e-12, atol=1e-12)


def test_quest_selection_invariant_under_head_permutation():
    r = rng(12)
    T, b, d, G = 512, 32, 16, 4
    K = r.standard_normal((T, d)).astype(np.float32)
    q = r.standard_normal((G, d)).astype(np.float32)
    mn, mx = O.desc_minmax(K, b)
    s1 = O.score_quest(q, mn, mx)
    s2 = O.score_quest(q[::-1].copy(), mn, mx)
    np.testing.assert_allclose(s1, s2, rtol=1e-12)


# --------------------------------------------------------------------------
# Gate score
# --------------------------------------------------------------------------

def test_gate_identity_is_mean_pooled_dot():
    """W = I: s_j = (sum_h q_h) . mean_j, computed with numpy's mean."""
    r = rng(21)
    T, b, d, G = 320, 64, 16, 4
    K = r.standard_normal((T, d)).astype(np.float32)
    q = r.standard_normal((G, d)).astype(np.float32)
    mean = O.desc_mean(K, b)
    s = O.score_gate(q, np.eye(d, dtype=np.float32), mean)
    ref = K.astype(np.float64).reshape(T // b, b, d).mean(axis=1) @ q.astype(np.float64).sum(0)
    np.testing.assert_allclose(s, ref, rtol=1e-12, atol=1e-12)


def test_gate_rank_one_closed_form():
    """W = a b^T (row r = a_r * b): W u = a (b.u), so s_j = (b.u)(a.mean_j).
    A transposed W would give (a.u)(b.mean_j) instead."""
    r = rng(22)
    T, b, d, G = 256, 32, 8, 2
    K = r.standard_normal((T, d)).astype(np.float32)
    q = r.standard_normal((G, d)).astype(np.float32)
    # small integers keep W = a b^T exact in float32
    a = r.integers(-4, 5, size=d).astype(np.float32)
    bb = r.integers(-4, 5, size=d).astype(np.float32)
    W = np.outer(a, bb).astype(np.float32)
    mean = O.desc_mean(K, b)
    s = O.score_gate(q, W, mean)
    u = q.astype(np.float64).sum(0)
    ref = (np.dot(bb.astype(np.float64), u)) * (mean @ a.astype(np.float64))
    np.testing.assert_allclose(s, ref, rtol=1e-10, atol=1e-10)


# --------------------------------------------------------------------------
# Block count
# --------------------------------------------------------------------------

def test_block_counts_golden():
    """Counts implied by the workloads' own statements (fixture cites them)."""
    with open(os.path.join(HERE, "golden", "block_counts.json")) as fh:
        cases = json.load(fh)["cases"]
    for c in cases:
        got = O.block_count(c["NB"], c["b"], c.get("budget_tokens", 0),
                            c.get("sparsity_bp", 0), c["n_local"], c["n_min"])
        assert got == c["n"], c


@pytest.mark.parametrize("bp", [9000, 9500, 9800, 8750])
def test_kept_fraction_tends_to_one_minus_p(bp):
    """The kept fraction n/NB is within 1/NB of 1 - p: the page's per-step
    cost model counts a (1 - p) share of the cache."""
    p = bp / 10000
    for NB in [10, 100, 1000, 8193, 100000]:
        n = O.block_count(NB, 64, 0, bp, 1, 0)
        assert abs(n / NB - (1 - p)) <= 1.0 / NB + 1e-12


def test_block_count_edges():
    assert O.block_count(1, 64, 512, 0, 2, 16) == 1          # everything is local
    assert O.block_count(5, 64, 0, 9000, 2, 0) == 2          # local dominates
    assert O.block_count(5, 64, 0, 0, 1, 0) == 5             # p = 0 keeps all
    assert O.block_count(100, 64, 32, 0, 1, 0) == 1          # budget < b
    assert O.block_count(100, 64, 0, 9999, 1, 3) == 3        # minimum binds
    assert O.block_count(100, 64, 64 * 1000, 0, 1, 0) == 100  # budget > context


# --------------------------------------------------------------------------
# Selection
# --------------------------------------------------------------------------

def _sorted_reference(scores, NB, n, n_local):
    nl = min(n_local, NB)
    cand = list(range(NB - nl))
    order = sorted(cand, key=lambda j: (-scores[j], j))
    return sorted(order[:max(0, n - nl)] + list(range(NB - nl, NB)))


@pytest.mark.parametrize("seed", range(6))
def test_select_equals_full_sort_with_ties(seed):
    """Repeated arg-max equals a full sort by (score desc, index asc);
    integer-valued scores force many ties.  The local blocks are kept and
    the size is n."""
    r = rng(300 + seed)
    for NB in [1, 2, 3, 17, 64, 257]:
        s = r.integers(-4, 5, size=NB).astype(np.float64)
        for n_local in [1, 2, 4]:
            for n in sorted({min(NB, max(min(n_local, NB), k)) for k in [0, 1, 3, NB // 3, NB]}):
                got = O.select(s, NB, n, n_local)
                ref = _sorted_reference(s, NB, n, n_local)
                assert list(got) == ref
                assert len(got) == n
                assert set(range(NB - min(n_local, NB), NB)) <= set(got.tolist())
                assert np.all(np.diff(got) > 0)


@pytest.mark.parametrize("seed", range(4))
def test_select_is_max_sum_subset_brute_force(seed):
    """On tiny inputs, the selection is the subset of size n containing the
    local blocks that maximises the summed score; among equal sums the
    lexicographically smallest index list wins."""
    r = rng(400 + seed)
    for NB in range(1, 11):
        s = r.integers(-3, 4, size=NB).astype(np.float64)
        for n_local in [1, 2]:
            nl = min(n_local, NB)
            for n in range(nl, NB + 1):
                local = set(range(NB - nl, NB))
                best = None
                for sub in itertools.combinations(range(NB - nl), n - nl):
                    full = sorted(set(sub) | local)
                    key = (-sum(s[j] for j in sub), full)
                    if best is None or key < best:
                        best = key
                assert list(O.select(s, NB, n, n_local)) == best[1]


def test_select_ignores_local_block_scores_and_pads():
    s = np.array([5.0, 1.0, 3.0, 100.0, -100.0])
    idx = O.select(s, 5, 3, 2, idx_cap=6)
    assert idx.tolist() == [0, 3, 4, -1, -1, -1]


def test_selection_invariant_under_affine_score_maps():
    r = rng(31)
    s = r.standard_normal(200)
    a = O.select(s, 200, 30, 2)
    b = O.select(3.5 * s + 7.0, 200, 30, 2)
    c = O.select(np.exp(s), 200, 30, 2)
    assert a.tolist() == b.tolist() == c.tolist()


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------

def _sdpa(q, K, V, mask, scale):
    """torch's scaled-dot-product attention in fp64 on the CPU, and the
    matching log-sum-exp from scipy."""
    qt = torch.from_numpy(q.astype(np.float64))[None, None, None, :]
    Kt = torch.from_numpy(K.astype(np.float64))[None, None]
    Vt = torch.from_numpy(V.astype(np.float64))[None, None]
    mt = torch.from_numpy(mask)[None, None, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mt,
                                                         scale=scale)
    z = scale * (K.astype(np.float64) @ q.astype(np.float64))
    lse = logsumexp(z[mask])
    return o[0, 0, 0].numpy(), lse


@pytest.mark.parametrize("T,b,d", [(1, 64, 8), (100, 16, 8), (257, 64, 32), (2048, 64, 64)])
def test_sparse_attend_equals_masked_sdpa(T, b, d):
    """Attention over the kept blocks equals torch SDPA with the block
    selection expanded to a token mask.  Catches: wrong token range of a
    block, partial last block handling, dropped normalisation, lse base."""
    r = rng(T + d)
    K = r.standard_normal((T, d)).astype(np.float32)
    V = r.standard_normal((T, d)).astype(np.float32)
    q = r.standard_normal(d).astype(np.float32)
    NB = (T + b - 1) // b
    idx = np.sort(r.choice(NB, size=max(1, NB // 3), replace=False)).astype(np.int32)
    if NB - 1 not in idx:
        idx = np.append(idx, NB - 1).astype(np.int32)
    mask = np.zeros(T, bool)
    for j in idx:
        mask[j * b:min((j + 1) * b, T)] = True
    scale = 1.0 / math.sqrt(d)
    o, lse = O.attend(q, K, V, b, idx, scale)
    o_ref, lse_ref = _sdpa(q, K, V, mask, scale)
    np.testing.assert_allclose(o, o_ref, rtol=1e-10, atol=1e-12)
    assert abs(lse - lse_ref) <= 1e-10 * max(1, abs(lse_ref))


def test_attend_all_blocks_equals_dense():
    r = rng(5)
    T, b, d = 1000, 64, 16
    K = r.standard_normal((T, d)).astype(np.float32)
    V = r.standard_normal((T, d)).astype(np.float32)
    q = r.standard_normal(d).astype(np.float32)
    idx = np.arange((T + b - 1) // b, dtype=np.int32)
    o1, l1 = O.attend(q, K, V, b, idx, 0.3)
    o2, l2 = O.dense_attend(q, K, V, T, 0.3)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    assert abs(l1 - l2) <= 1e-12


def test_attend_closed_forms():
    """Equal keys: uniform weights, o = mean V, lse = scale*q.k + ln N.
    One token: o = v, lse = scale*q.k."""
    r = rng(6)
    T, d = 50, 8
    k = r.standard_normal(d).astype(np.float32)
    K = np.tile(k, (T, 1))
    V = r.standard_normal((T, d)).astype(np.float32)
    q = r.standard_normal(d).astype(np.float32)
    o, lse = O.dense_attend(q, K, V, T, 0.5)
    np.testing.assert_allclose(o, V.astype(np.float64).mean(0), rtol=1e-12, atol=1e-14)
    z = 0.5 * float(np.dot(q.astype(np.float64), k.astype(np.float64)))
    assert abs(lse - (z + math.log(T))) < 1e-12
    o1, l1 = O.dense_attend(q, K, V, 1, 0.5)
    np.testing.assert_allclose(o1, V[0].astype(np.float64), rtol=0, atol=1e-15)
    assert abs(l1 - z) < 1e-13


def test_dense_attend_equals_sdpa():
    r = rng(8)
    T, d = 777, 24
    K = (3 * r.standard_normal((T, d))).astype(np.float32)
    V = r.standard_normal((T, d)).astype(np.float32)
    q = r.standard_normal(d).astype(np.float32)
    o, lse = O.dense_attend(q, K, V, T, 1 / math.sqrt(d))
    o_ref, lse_ref = _sdpa(q, K, V, np.ones(T, bool), 1 / math.sqrt(d))
    np.testing.assert_allclose(o, o_ref, rtol=1e-10, atol=1e-12)
    assert abs(lse - lse_ref) < 1e-10


# --------------------------------------------------------------------------
# Rectification
# --------------------------------------------------------------------------

def test_rectify_causal_mask_brute_force():
    """Each query i of the chunk attends exactly to tokens 0..T-f+i of the
    overwritten cache: compared with torch softmax over an explicit -inf
    mask matrix built independently."""
    r = rng(9)
    T, d, G, f = 300, 16, 2, 8
    K = r.standard_normal((T, d)).astype(np.float32)
    V = r.standard_normal((T, d)).astype(np.float32)
    kn = r.standard_normal((f, d)).astype(np.float32)
    vn = r.standard_normal((f, d)).astype(np.float32)
    q = r.standard_normal((G, f, d)).astype(np.float32)
    K2, V2 = K.copy(), V.copy()
    K2[T - f:] = kn
    V2[T - f:] = vn
    scale = 1 / math.sqrt(d)
    o, lse = O.rectify(q, K, V, kn, vn, scale)
    assert np.array_equal(K, K2) and np.array_equal(V, V2)
    pos = np.arange(T - f, T)
    mask = np.where(np.arange(T)[None, :] <= pos[:, None], 0.0, -np.inf)   # [f, T]
    for h in range(G):
        logits = scale * (q[h].astype(np.float64) @ K2.astype(np.float64).T) + mask
        w = torch.softmax(torch.from_numpy(logits), dim=-1).numpy()
        np.testing.assert_allclose(o[h], w @ V2.astype(np.float64), rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(lse[h], logsumexp(logits, axis=-1), rtol=1e-12)


def test_rectify_f1_identity_is_dense_decode():
    """f = 1 with k_new = k_old reproduces a dense decode at position T-1."""
    r = rng(10)
    T, d, G = 129, 8, 4
    K = r.standard_normal((T, d)).astype(np.float32)
    V = r.standard_normal((T, d)).astype(np.float32)
    q = r.standard_normal((G, 1, d)).astype(np.float32)
    o, lse = O.rectify(q, K.copy(), V.copy(), K[-1:].copy(), V[-1:].copy(), 0.25)
    for h in range(G):
        o2, l2 = O.dense_attend(q[h, 0], K, V, T, 0.25)
        np.testing.assert_allclose(o[h, 0], o2, rtol=0, atol=1e-14)
        assert abs(lse[h, 0] - l2) < 1e-14


# --------------------------------------------------------------------------
# Whole decode step
# --------------------------------------------------------------------------

@pytest.mark.parametrize("kind", [0, 1])
def test_decode_group_budget_ge_context_is_dense(kind):
    """With a budget at least the context every block is kept and the step
    equals dense softmax attention (torch SDPA)."""
    r = rng(40 + kind)
    T, b, d, G = 700, 64, 16, 4
    K = r.standard_normal((T, d)).astype(np.float32)
    V = r.standard_normal((T, d)).astype(np.float32)
    q = r.standard_normal((G, d)).astype(np.float32)
    W = r.standard_normal((d, d)).astype(np.float32) if kind else None
    idx, o, lse = O.decode_group(q, K, V, b, kind, W=W, budget_tokens=64 * 100, n_local=1)
    assert idx.tolist() == list(range((T + b - 1) // b))
    for h in range(G):
        o_ref, l_ref = _sdpa(q[h], K, V, np.ones(T, bool), 1 / math.sqrt(d))
        np.testing.assert_allclose(o[h], o_ref, rtol=1e-10, atol=1e-12)
        assert abs(lse[h] - l_ref) < 1e-10


def test_decode_group_planted_blocks_are_selected():
    """Blocks whose keys are pushed along the group's query direction are
    the ones selected (plus the local block)."""
    r = rng(50)
    T, b, d, G = 2048 + 1, 64, 64, 4
    K = r.standard_normal((T, d)).astype(np.float32)
    V = r.standard_normal((T, d)).astype(np.float32)
    q = r.standard_normal((G, d)).astype(np.float32)
    u = q.astype(np.float64).sum(0)
    u /= np.linalg.norm(u)
    planted = [3, 11, 20]
    for j in planted:
        K[j * b:(j + 1) * b] += (6.0 * u).astype(np.float32)
    idx, _, _ = O.decode_group(q, K, V, b, 0, budget_tokens=4 * 64, n_local=1, n_min=2)
    assert idx.tolist() == planted + [32]


# --------------------------------------------------------------------------
# Log-gate bias (SAS)
# --------------------------------------------------------------------------

def _bias_mask(T, b, idx, bias):
    """Per-token additive mask: the block's bias on its tokens, -inf on
    every token of a block that is not kept."""
    m = np.full(T, -np.inf)
    for j, g in zip(idx, bias):
        m[j * b:min((j + 1) * b, T)] = g
    return m


def test_gate_bias_equals_scipy_log_softmax():
    """The bias of a kept candidate is scipy's log_softmax of tau*s over ALL
    candidates (not only the kept ones); local blocks get 0.  Catches: a
    normaliser over the kept set only, a missing tau, a local block taken as a
    candidate, a sign error."""
    from scipy.special import log_softmax
    r = rng(60)
    NB, nl, tau = 40, 3, 0.37
    s = 20 * r.standard_normal(NB - nl)
    idx = np.array([1, 5, 17, 30, 37, 38, 39], np.int32)
    g = O.gate_bias(s, NB, nl, tau, idx)
    ref = log_softmax(tau * s)
    np.testing.assert_allclose(g[:4], ref[[1, 5, 17, 30]], rtol=0, atol=1e-13)
    assert g[4:].tolist() == [0.0, 0.0, 0.0]


def test_gate_bias_uniform_scores_is_minus_log_c():
    """Equal scores (or tau = 0): every candidate's gate is 1/C."""
    NB, nl = 25, 2
    idx = np.arange(NB, dtype=np.int32)
    for s, tau in [(np.full(NB - nl, 3.5), 1.0), (np.arange(NB - nl, dtype=float), 0.0)]:
        g = O.gate_bias(s, NB, nl, tau, idx)
        np.testing.assert_allclose(g[:NB - nl], -math.log(NB - nl), rtol=0, atol=1e-14)
        assert g[NB - nl:].tolist() == [0.0] * nl


def test_gate_bias_shift_invariant_and_normalised():
    """softmax is unchanged by a common shift of the scores, and the gates of
    all candidates sum to one, also with scores far beyond exp's range (the
    largest term must be factored out)."""
    r = rng(61)
    NB, nl, tau = 64, 1, 2.0
    s = 400 * r.standard_normal(NB - nl)
    idx = np.arange(NB, dtype=np.int32)
    g1 = O.gate_bias(s, NB, nl, tau, idx)
    g2 = O.gate_bias(s + 1234.5, NB, nl, tau, idx)
    np.testing.assert_allclose(g1, g2, rtol=0, atol=1e-9)
    assert np.all(np.isfinite(g1[:NB - nl]) | (g1[:NB - nl] == -np.inf))
    assert abs(np.exp(g1[:NB - nl]).sum() - 1.0) < 1e-12


def test_attend_biased_equals_sdpa_with_float_mask():
    """Attention with a per-block logit bias equals torch SDPA given the bias
    expanded to a float token mask.  Catches: the bias multiplied by the
    softmax scale, added to the wrong block, or left out of the lse."""
    r = rng(62)
    T, b, d = 517, 32, 16
    K = r.standard_normal((T, d)).astype(np.float32)
    V = r.standard_normal((T, d)).astype(np.float32)
    q = r.standard_normal(d).astype(np.float32)
    NB = (T + b - 1) // b
    idx = np.array([0, 3, 4, 9, 15, NB - 1], np.int32)
    bias = r.uniform(-4, 0, idx.shape[0])
    scale = 1 / math.sqrt(d)
    o, lse = O.attend_biased(q, K, V, b, idx, bias, scale)
    m = _bias_mask(T, b, idx, bias)
    qt = torch.from_numpy(q.astype(np.float64))[None, None, None, :]
    Kt = torch.from_numpy(K.astype(np.float64))[None, None]
    Vt = torch.from_numpy(V.astype(np.float64))[None, None]
    mt = torch.from_numpy(m)[None, None, None, :]
    o_ref = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, attn_mask=mt,
                                                             scale=scale)[0, 0, 0].numpy()
    z = scale * (K.astype(np.float64) @ q.astype(np.float64)) + m
    np.testing.assert_allclose(o, o_ref, rtol=1e-10, atol=1e-12)
    assert abs(lse - logsumexp(z)) < 1e-10


def test_attend_biased_equal_keys_weighted_mean():
    """With one shared key the weights are exp(bias) per token: o is the mean
    of V weighted by exp(bias_k) over every token of block k, and
    lse = scale*q.k + ln sum_k n_k exp(bias_k)."""
    r = rng(63)
    T, b, d = 200, 16, 8
    k = r.standard_normal(d).astype(np.float32)
    K = np.tile(k, (T, 1))
    V = r.standard_normal((T, d)).astype(np.float32)
    q = r.standard_normal(d).astype(np.float32)
    idx = np.array([2, 7, 12], np.int32)          # block 12 is the partial one
    bias = np.array([-1.0, 0.0, -2.5])
    o, lse = O.attend_biased(q, K, V, b, idx, bias, 0.25)
    num = np.zeros(d)
    den = 0.0
    for j, g in zip(idx, bias):
        rows = V[j * b:min((j + 1) * b, T)].astype(np.float64)
        num += math.exp(g) * rows.sum(0)
        den += math.exp(g) * rows.shape[0]
    np.testing.assert_allclose(o, num / den, rtol=1e-12, atol=1e-14)
    z = 0.25 * float(np.dot(q.astype(np.float64), k.astype(np.float64)))
    assert abs(lse - (z + math.log(den))) < 1e-12


def test_attend_biased_zero_bias_is_attend():
    r = rng(64)
    T, b, d = 300, 64, 8
    K = r.standard_normal((T, d)).astype(np.float32)
    V = r.standard_normal((T, d)).astype(np.float32)
    q = r.standard_normal(d).astype(np.float32)
    idx = np.array([0, 2, 4], np.int32)
    o1, l1 = O.attend_biased(q, K, V, b, idx, np.zeros(3), 0.4)
    o2, l2 = O.attend(q, K, V, b, idx, 0.4)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-15)
    assert abs(l1 - l2) < 1e-15


def test_gate_bias_current_block_only():
    """The page's partition: only the last block keeps the unit gate; an
    older local block is historical -- its gate is its own log_softmax entry
    and its score enters every other gate's normaliser.  Catches the reading
    that treats every local block as current (bias 0 there, a normaliser
    without its score)."""
    from scipy.special import log_softmax
    r = rng(67)
    NB, tau = 30, 0.8
    s = 3 * r.standard_normal(NB - 1)            # every block but the current one
    s[NB - 2] = s.max() + 1.0                    # a dominant older local block
    idx = np.array([3, 11, 20, NB - 2, NB - 1], np.int32)
    g = O.gate_bias(s, NB, 1, tau, idx)
    ref = log_softmax(tau * s)
    np.testing.assert_allclose(g[:4], ref[[3, 11, 20, NB - 2]], rtol=0, atol=1e-13)
    assert g[4] == 0.0
    # every local block current: block NB-2 unbiased and out of the normaliser
    g2 = O.gate_bias(s, NB, 2, tau, idx)
    ref2 = log_softmax(tau * s[:NB - 2])
    np.testing.assert_allclose(g2[:3], ref2[[3, 11, 20]], rtol=0, atol=1e-13)
    assert g2[3:].tolist() == [0.0, 0.0]
    assert np.all(g[:3] < g2[:3] - 0.1)          # the dominant block takes gate mass


@pytest.mark.parametrize("kind,n_current", [(0, 1), (1, 1), (0, 2)])
def test_decode_group_gated_matches_selection_and_sdpa(kind, n_current):
    """The gated step keeps the ungated step's selection, and its outputs are
    torch SDPA with log_softmax(tau*s) over the historical blocks' scores as
    the float mask: every block but the n_current trailing ones is historical
    (0 on the current ones).  The scores of the kept local blocks that are
    historical come from the pinned descriptor and score functions."""
    from scipy.special import log_softmax
    r = rng(65 + kind)
    T, b, d, G, nl = 1500, 64, 16, 4, 2
    K = r.standard_normal((T, d)).astype(np.float32)
    V = r.standard_normal((T, d)).astype(np.float32)
    q = r.standard_normal((G, d)).astype(np.float32)
    W = r.standard_normal((d, d)).astype(np.float32) if kind else None
    tau = 0.05
    idx0, _, _, s = O.decode_group(q, K, V, b, kind, W=W, budget_tokens=6 * 64,
                                   n_local=nl, n_min=2, want_scores=True)
    idx, o, lse, bias = O.decode_group_gated(q, K, V, b, kind, tau, W=W,
                                             budget_tokens=6 * 64, n_local=nl, n_min=2,
                                             n_current=n_current)
    assert idx.tolist() == idx0.tolist()
    NB = (T + b - 1) // b
    nh = NB - n_current                           # historical blocks
    if kind == 0:
        mn, mx = O.desc_minmax(K, b)
        s_all = O.score_quest(q, mn, mx)
    else:
        s_all = O.score_gate(q, W, O.desc_mean(K, b))
    np.testing.assert_array_equal(s_all[:NB - nl], s[:NB - nl])
    ls = log_softmax(tau * s_all[:nh])
    ref_bias = np.array([ls[j] if j < nh else 0.0 for j in idx])
    if n_current < nl:
        assert ref_bias[-2] != 0.0                # the older local block is gated
    np.testing.assert_allclose(bias, ref_bias, rtol=0, atol=1e-12)
    m = _bias_mask(T, b, idx, ref_bias)
    scale = 1 / math.sqrt(d)
    for h in range(G):
        qt = torch.from_numpy(q[h].astype(np.float64))[None, None, None, :]
        Kt = torch.from_numpy(K.astype(np.float64))[None, None]
        Vt = torch.from_numpy(V.astype(np.float64))[None, None]
        mt = torch.from_numpy(m)[None, None, None, :]
        o_ref = torch.nn.functional.scaled_dot_product_attention(
            qt, Kt, Vt, attn_mask=mt, scale=scale)[0, 0, 0].numpy()
        z = scale * (K.astype(np.float64) @ q[h].astype(np.float64)) + m
        np.testing.assert_allclose(o[h], o_ref, rtol=1e-10, atol=1e-12)
        assert abs(lse[h] - logsumexp(z)) < 1e-10


def test_attend_biased_constant_bias_is_a_shift():
    """One bias c on every kept block leaves o unchanged and moves lse by c
    (so uniform gates reduce the gated step to the plain one, up to a
    constant)."""
    r = rng(66)
    T, b, d = 450, 32, 8
    K = r.standard_normal((T, d)).astype(np.float32)
    V = r.standard_normal((T, d)).astype(np.float32)
    q = r.standard_normal(d).astype(np.float32)
    idx = np.array([1, 4, 6, 13, 14], np.int32)
    o1, l1 = O.attend_biased(q, K, V, b, idx, np.full(5, -2.75), 0.3)
    o2, l2 = O.attend(q, K, V, b, idx, 0.3)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    assert abs(l1 - (l2 - 2.75)) < 1e-12

"""GPU parity of the log-gate bias ("Simple Attention Sparsification",
Method: one current block with the unit gate, softmax gates over the
historical blocks, log g added to a kept block's logits) against the fp64
oracle: the bias the selecting call writes next to each kept block id, and
the gated decode that consumes it.  By default only the last block is
current, so with two local blocks the older one is historical: scored,
gated and part of the normaliser; the option gate_current = n_local treats
every local block as current.

Selection bit-exact (inputs carry a score gap at the top-n boundary).
Bias: the kernel works from fp32 scores; a score error ds moves a bias by at
most tau * 2 ds plus the fp32 rounding of the normaliser's sum (relative
n_candidates * 2^-24), so the bar is tau * 2e-5 * max|s| + 1e-4 + C * 1.2e-7
absolute.  o within 2e-2 absolute, lse within 1e-4 relative, as ungated."""
import math

import numpy as np
import pytest

import block_sparse_attention_build_amd as bsa
import oracle as O
from harness import compare_step, enforce_gap, prefill, random_page_table, to_dev
from test_gpu_parity import BF16, F32, MEAN, MINMAX, make_inputs

pytestmark = pytest.mark.gpu

GATE_CASES = [
    # dtype, d, blk, kind, Hq, Hkv, lengths, budget, bp, n_local, n_min[, gate_current]
    (BF16, 128, 64, MINMAX, 8, 2, [1000, 1537], 256, 0, 1, 0),
    (BF16, 128, 128, MEAN, 8, 2, [3000, 2049], 0, 9000, 2, 0),
    (BF16, 128, 256, MINMAX, 8, 4, [5000, 1], 0, 9500, 1, 4),   # a group with no candidate
    (BF16, 64, 32, MINMAX, 4, 4, [777, 1025, 64, 65], 0, 8000, 1, 3),
    (F32, 64, 64, MINMAX, 4, 1, [2049], 512, 0, 1, 2),
    (F32, 128, 128, MEAN, 8, 2, [1500, 700], 0, 9000, 2, 0),
    # mid-size rows (about 1900 and 3100 candidates)
    (BF16, 64, 32, MINMAX, 4, 1, [60000], 0, 9000, 1, 2),
    (BF16, 64, 32, MINMAX, 8, 2, [98000, 40000], 0, 9500, 2, 4),
    # three local blocks, two of them historical; and the option that keeps
    # every local block current
    (BF16, 128, 64, MINMAX, 8, 2, [4000, 2500], 0, 9000, 3, 2),
    (BF16, 128, 64, MINMAX, 8, 2, [4000, 2500], 0, 9000, 2, 2, 2),
    (BF16, 128, 128, MEAN, 8, 2, [3000, 2049], 0, 9000, 3, 0, 3),
    # every kept block local (nothing picked), the older ones historical
    (BF16, 64, 64, MINMAX, 4, 2, [300, 250], 0, 9900, 3, 0),
]


def _oracle_gated(L, P, q, Ks, Vs, lengths, tau, Wg, n_current):
    """Oracle selection, outputs and biases per group, and the largest
    |score| over the historical blocks (for the bias bar)."""
    G = L.Hq // L.Hkv
    kind = 0 if L.desc_kind == MINMAX else 1
    scale = 1.0 / math.sqrt(L.d)
    ref, bias, smax = {}, {}, 0.0
    for s, T in enumerate(lengths):
        for h in range(L.Hkv):
            qg, K, V = q[s, h * G:(h + 1) * G], Ks[s][h, :T], Vs[s][h, :T]
            idx, o, lse, b = O.decode_group_gated(qg, K, V, L.block, kind, tau, W=Wg,
                                                  budget_tokens=P.budget_tokens,
                                                  sparsity_bp=P.sparsity_bp,
                                                  n_local=P.n_local, n_min=P.n_min, scale=scale,
                                                  n_current=n_current)
            NB = -(-T // L.block)
            if kind == 0:
                mn, mx = O.desc_minmax(K, L.block)
                sh = O.score_quest(qg, mn, mx)
            else:
                sh = O.score_gate(qg, Wg, O.desc_mean(K, L.block))
            sh = sh[:max(0, NB - n_current)]
            if sh.size:
                smax = max(smax, float(np.abs(sh).max()))
            ref[(s, h)] = (idx, o, lse)
            bias[(s, h)] = b
    return ref, bias, smax


def _tau_for(L, P, q, Ks, lengths, Wg):
    """A tau that spreads the gates of group (0, 0) over a few units."""
    G = L.Hq // L.Hkv
    kind = 0 if L.desc_kind == MINMAX else 1
    _, _, _, sc = O.decode_group(q[0, :G], Ks[0][0, :lengths[0]], Ks[0][0, :lengths[0]],
                                 L.block, kind, W=Wg, budget_tokens=P.budget_tokens,
                                 sparsity_bp=P.sparsity_bp, n_local=P.n_local, n_min=P.n_min,
                                 want_scores=True)
    fin = sc[np.isfinite(sc)]
    sd = float(fin.std()) if fin.size > 1 else 1.0
    return 3.0 / max(sd, 1e-3)


@pytest.mark.parametrize("case", GATE_CASES, ids=[f"g{i}" for i in range(len(GATE_CASES))])
def test_gated_select_decode_parity(case):
    import torch
    dtype, d, blk, kind, Hq, Hkv, lengths, budget, bp, nl, nm = case[:11]
    n_current = case[11] if len(case) > 11 else 1
    B = len(lengths)
    max_blocks = (max(lengths) + blk - 1) // blk + 2
    L = bsa.Layout(B, Hq, Hkv, d, blk, max_blocks, dtype, kind)
    P = bsa.SelectParams(budget_tokens=budget, sparsity_bp=bp, n_local=nl, n_min=nm,
                         gate_current=n_current)
    P.n_max = bsa.block_count(P, max_blocks, blk)
    q, Ks, Vs, Wg = make_inputs(31 + len(lengths), B, Hq, Hkv, d, lengths, dtype, kind)
    enforce_gap(L, P, q, Ks, [[T] for T in lengths], W_gate=Wg)
    tau = _tau_for(L, P, q, Ks, lengths, Wg)
    print(f"case {case} tau {tau:.4g}", flush=True)
    cache = bsa.allocate_cache(L, page_table=random_page_table(L, 9))
    cache.k_pool.fill_(float("nan"))
    cache.v_pool.fill_(float("nan"))
    prefill(L, cache, Ks, Vs, lengths)
    if Wg is not None:
        P.gate_w = to_dev(Wg, bsa.Layout(1, 1, 1, d, blk, 1, BF16))
    dev = "cuda"
    idx = torch.full((B, Hkv, P.n_max), -7, dtype=torch.int32, device=dev)
    cnt = torch.full((B, Hkv), -7, dtype=torch.int32, device=dev)
    P.gate_tau = tau
    P.gate_bias = torch.full((B, Hkv, P.n_max), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(max(bsa.workspace_size(L, bsa.OP_SELECT, P.n_max),
                         bsa.workspace_size(L, bsa.OP_DECODE, P.n_max)),
                     dtype=torch.uint8, device=dev)
    ws.view(torch.float32)[: ws.numel() // 4].fill_(float("nan"))
    q_dev = to_dev(q, L)
    bsa.select_blocks(L, cache, q_dev, P, idx, cnt, ws)
    o = torch.full((B, Hq, d), float("nan"), dtype=q_dev.dtype, device=dev)
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=dev)
    bsa.sparse_decode_gated(L, cache, q_dev, idx, cnt, P.gate_bias, P.n_max, 1.0 / math.sqrt(d),
                            o, lse, ws)
    torch.cuda.synchronize()
    ref, rbias, smax = _oracle_gated(L, P, q, Ks, Vs, lengths, tau, Wg, n_current)
    compare_step(L, idx, cnt, o, lse, ref)
    gb = P.gate_bias.cpu().numpy()
    cn = cnt.cpu().numpy()
    worst = 0.0
    for (s, h), rb in rbias.items():
        c = int(cn[s, h])
        NH = max(0, -(-lengths[s] // blk) - n_current)  # historical blocks
        tol = tau * 2e-5 * smax + 1e-4 + NH * 1.2e-7
        err = np.abs(gb[s, h, :c] - rb).max() if c else 0.0
        assert err <= tol, f"group {(s, h)}: bias err {err} > {tol}"
        assert np.all(gb[s, h, c:] == 0.0)
        worst = max(worst, err)
    print(f"worst bias err {worst:.3g}", flush=True)


@pytest.mark.parametrize("dtype,d,blk", [(BF16, 128, 64), (BF16, 64, 128), (F32, 64, 32)])
def test_gated_decode_with_arbitrary_bias(dtype, d, blk):
    """The gated decode with a bias that no selection wrote (random values in
    [-4, 1], random kept lists) equals the oracle's biased attention."""
    import torch
    lengths = [blk * 40 + 5, blk * 13]
    Hq, Hkv = 8, 2
    B = len(lengths)
    max_blocks = (max(lengths) + blk - 1) // blk + 1
    L = bsa.Layout(B, Hq, Hkv, d, blk, max_blocks, dtype, MINMAX)
    q, Ks, Vs, _ = make_inputs(91, B, Hq, Hkv, d, lengths, dtype, MINMAX)
    cache = bsa.allocate_cache(L, page_table=random_page_table(L, 4))
    prefill(L, cache, Ks, Vs, lengths)
    rng = np.random.Generator(np.random.PCG64(5))
    n_max = max_blocks
    idx = np.full((B, Hkv, n_max), -1, np.int32)
    cnt = np.zeros((B, Hkv), np.int32)
    bias = np.zeros((B, Hkv, n_max), np.float32)
    for s, T in enumerate(lengths):
        NB = -(-T // blk)
        for h in range(Hkv):
            k = int(rng.integers(1, NB + 1))
            sel = np.sort(rng.choice(NB, size=k, replace=False)).astype(np.int32)
            idx[s, h, :k] = sel
            cnt[s, h] = k
            bias[s, h, :k] = rng.uniform(-4, 1, k).astype(np.float32)
    ws = torch.empty(bsa.workspace_size(L, bsa.OP_DECODE, n_max), dtype=torch.uint8,
                     device="cuda")
    q_dev = to_dev(q, L)
    o = torch.full((B, Hq, d), float("nan"), dtype=q_dev.dtype, device="cuda")
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    bsa.sparse_decode_gated(L, cache, q_dev, torch.from_numpy(idx).cuda(),
                            torch.from_numpy(cnt).cuda(), torch.from_numpy(bias).cuda(), n_max,
                            0.1, o, lse, ws)
    torch.cuda.synchronize()
    G = Hq // Hkv
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    worst_o = worst_l = 0.0
    for s, T in enumerate(lengths):
        for h in range(Hkv):
            k = cnt[s, h]
            for g in range(G):
                ro, rl = O.attend_biased(q[s, h * G + g], Ks[s][h, :T], Vs[s][h, :T], blk,
                                         idx[s, h, :k], bias[s, h, :k].astype(np.float64), 0.1)
                worst_o = max(worst_o, float(np.abs(o[s, h * G + g] - ro).max()))
                worst_l = max(worst_l, abs(lse[s, h * G + g] - rl) / max(1.0, abs(rl)))
    assert worst_o <= 2e-2, worst_o
    assert worst_l <= 1e-4, worst_l


def test_gated_decode_constant_bias_is_shifted_plain_decode():
    """A constant bias c on every kept block: o equals the ungated decode's
    and lse moves by c (same kernels, same split)."""
    import torch
    d, blk, Hq, Hkv = 128, 64, 8, 2
    lengths = [3000, 1234]
    B = len(lengths)
    max_blocks = (max(lengths) + blk - 1) // blk + 1
    L = bsa.Layout(B, Hq, Hkv, d, blk, max_blocks, BF16, MINMAX)
    P = bsa.SelectParams(sparsity_bp=8000, n_local=2, n_min=2)
    P.n_max = bsa.block_count(P, max_blocks, blk)
    q, Ks, Vs, _ = make_inputs(17, B, Hq, Hkv, d, lengths, BF16, MINMAX)
    cache = bsa.allocate_cache(L, page_table=random_page_table(L, 2))
    prefill(L, cache, Ks, Vs, lengths)
    idx = torch.empty((B, Hkv, P.n_max), dtype=torch.int32, device="cuda")
    cnt = torch.empty((B, Hkv), dtype=torch.int32, device="cuda")
    ws = torch.empty(max(bsa.workspace_size(L, bsa.OP_SELECT, P.n_max),
                         bsa.workspace_size(L, bsa.OP_DECODE, P.n_max)),
                     dtype=torch.uint8, device="cuda")
    q_dev = to_dev(q, L)
    bsa.select_blocks(L, cache, q_dev, P, idx, cnt, ws)
    outs = []
    for c in (None, -1.5):
        o = torch.empty((B, Hq, d), dtype=q_dev.dtype, device="cuda")
        lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        if c is None:
            bsa.sparse_decode(L, cache, q_dev, idx, cnt, P.n_max, 0.09, o, lse, ws)
        else:
            bias = torch.full((B, Hkv, P.n_max), c, dtype=torch.float32, device="cuda")
            bsa.sparse_decode_gated(L, cache, q_dev, idx, cnt, bias, P.n_max, 0.09, o, lse, ws)
        torch.cuda.synchronize()
        outs.append((o.float().cpu(), lse.cpu()))
    assert (outs[0][0] - outs[1][0]).abs().max().item() <= 1e-2
    assert ((outs[1][1] - (outs[0][1] - 1.5)).abs() / outs[0][1].abs().clamp(min=1)).max() <= 1e-5


def test_gated_topn_long_row_of_ties():
    """The gated selection on about 8000 almost-tied candidates: the
    threshold digit holds more keys than the gathered list takes, so the
    whole-workgroup radix passes run and the normaliser's parts are formed
    after them rather than beside the wave-0 passes.  Selection, biases and
    the gated decode against the oracle."""
    import torch
    import workloads as W
    d, blk, Hq, Hkv = 64, 32, 4, 1
    T = 8000 * blk + 17
    L = bsa.Layout(1, Hq, Hkv, d, blk, (T + blk - 1) // blk + 1, BF16, MINMAX)
    P = bsa.SelectParams(budget_tokens=0, sparsity_bp=9000, n_local=1, n_min=0)
    P.n_max = bsa.block_count(P, L.max_blocks, blk)
    rng = np.random.Generator(np.random.PCG64(124))
    q = W.quantize(rng.standard_normal((1, Hq, d), dtype=np.float32), "bf16")
    u = W.group_direction(q[0])
    tmpl = rng.standard_normal((blk, d), dtype=np.float32)
    K = np.tile(tmpl, ((T + blk - 1) // blk, 1))[:T].copy()
    K[-17:] = rng.standard_normal((17, d), dtype=np.float32)
    for j in (7, 1000, 4321, 7777, 7990):   # clearly above the tied mass
        K[j * blk:(j + 1) * blk] += 3.0 * u
    for j in (3, 2500, 6000):               # clearly below it
        K[j * blk:(j + 1) * blk] -= 3.0 * u
    Ks = [W.quantize(K, "bf16")[None]]
    Vs = [W.quantize(rng.standard_normal((1, T, d), dtype=np.float32), "bf16")]
    tau = 0.05
    cache = bsa.allocate_cache(L, page_table=random_page_table(L, 10))
    prefill(L, cache, Ks, Vs, [T])
    dev = "cuda"
    idx = torch.full((1, Hkv, P.n_max), -7, dtype=torch.int32, device=dev)
    cnt = torch.full((1, Hkv), -7, dtype=torch.int32, device=dev)
    P.gate_tau = tau
    P.gate_bias = torch.full((1, Hkv, P.n_max), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(max(bsa.workspace_size(L, bsa.OP_SELECT, P.n_max),
                         bsa.workspace_size(L, bsa.OP_DECODE, P.n_max)),
                     dtype=torch.uint8, device=dev)
    q_dev = to_dev(q, L)
    bsa.select_blocks(L, cache, q_dev, P, idx, cnt, ws)
    o = torch.full((1, Hq, d), float("nan"), dtype=q_dev.dtype, device=dev)
    lse = torch.full((1, Hq), float("nan"), dtype=torch.float32, device=dev)
    bsa.sparse_decode_gated(L, cache, q_dev, idx, cnt, P.gate_bias, P.n_max, 1.0 / math.sqrt(d),
                            o, lse, ws)
    torch.cuda.synchronize()
    ref, rbias, smax = _oracle_gated(L, P, q, Ks, Vs, [T], tau, None, 1)
    compare_step(L, idx, cnt, o, lse, ref)
    assert {7, 1000, 4321, 7777, 7990} <= set(ref[(0, 0)][0].tolist())
    c = int(cnt[0, 0])
    NC = -(-T // blk) - 1
    tol = tau * 2e-5 * smax + 1e-4 + NC * 1.2e-7
    gb = P.gate_bias.cpu().numpy()
    err = np.abs(gb[0, 0, :c] - rbias[(0, 0)]).max()
    assert err <= tol, (err, tol)
    assert np.all(gb[0, 0, c:] == 0.0)

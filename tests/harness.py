"""Test-side helpers shared by the GPU parity tests: moving seeded host
inputs into a paged cache through the library's own entry points, reading
pages back through the documented page layout, the oracle side of a decode
step, and the score-gap enforcement that makes bit-exact selection
well-defined.  Test infrastructure; may use the oracle."""
import math

import numpy as np

import block_sparse_attention_build_amd as bsa
import oracle as O
import workloads as W


def torch_dtype(L):
    import torch
    return torch.bfloat16 if L.kv_dtype == bsa.DTYPE_BF16 else torch.float32


def to_dev(x, L, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(device, torch_dtype(L))


def seq_view(L, cache, s):
    """Layout and cache views of sequence s alone (B = 1)."""
    L1 = bsa.Layout(1, L.Hq, L.Hkv, L.d, L.block, L.max_blocks, L.kv_dtype, L.desc_kind)
    c1 = bsa.Cache(cache.k_pool, cache.v_pool, cache.page_table[s:s + 1],
                   cache.seq_lens[s:s + 1], cache.desc[s:s + 1])
    return L1, c1


def random_page_table(L, seed):
    """Each sequence gets max_blocks distinct pages, scattered over the pool."""
    import torch
    rng = np.random.Generator(np.random.PCG64(seed))
    perm = rng.permutation(L.B * L.max_blocks).astype(np.int32)
    return torch.from_numpy(perm.reshape(L.B, L.max_blocks))


def prefill(L, cache, Ks, Vs, lengths, device="cuda"):
    """Write tokens [0, lengths[s]) of every sequence with one bulk append
    each (seq_lens is set to the lengths)."""
    import torch
    for s, T in enumerate(lengths):
        if T == 0:
            continue
        L1, c1 = seq_view(L, cache, s)
        c1.seq_lens.fill_(T)
        kt = to_dev(Ks[s][:, :T], L, device)[None]
        vt = to_dev(Vs[s][:, :T], L, device)[None]
        bsa.build_block_desc(L1, c1, kt, vt, T)
    torch.cuda.synchronize()


# --------------------------------------------------------------------------
# Reading pages back (numpy restatement of the layout documented in bsa.h)
# --------------------------------------------------------------------------

def _k_off_bf16(t, i, d):
    return (((t // 16) * (d // 32) + i // 32) * 512 + ((t % 16) + 16 * ((i % 32) // 8)) * 8
            + i % 8)


def _v_off_bf16(t, i, d):
    u = t % 32
    g = (u % 16) // 4
    e = (u % 4) + 4 * (u // 16)
    return ((t // 32) * (d // 16) + i // 16) * 512 + ((i % 16) + 16 * g) * 8 + e


def page_index_maps(L):
    """[b, d] arrays of element offsets inside a page for K and for V."""
    t = np.arange(L.block)[:, None]
    i = np.arange(L.d)[None, :]
    if L.kv_dtype == bsa.DTYPE_BF16:
        return _k_off_bf16(t, i, L.d), _v_off_bf16(t, i, L.d)
    off = t * L.d + i
    return off, off


def read_cache(L, cache, s, T):
    """K, V [Hkv, T, d] float32 of sequence s, gathered through the page
    table and the documented in-page layout."""
    kp = cache.k_pool.float().cpu().numpy()
    vp = cache.v_pool.float().cpu().numpy()
    pt = cache.page_table.cpu().numpy()
    km, vm = page_index_maps(L)
    NB = (T + L.block - 1) // L.block
    K = np.empty((L.Hkv, NB * L.block, L.d), np.float32)
    V = np.empty_like(K)
    for j in range(NB):
        pg = pt[s, j]
        K[:, j * L.block:(j + 1) * L.block] = kp[pg][:, km]
        V[:, j * L.block:(j + 1) * L.block] = vp[pg][:, vm]
    return K[:, :T], V[:, :T]


# --------------------------------------------------------------------------
# Oracle side
# --------------------------------------------------------------------------

def oracle_decode(w_or_params, q, Ks, Vs, lengths, L, W_gate=None, scale=None):
    """Per (sequence, kv head): (idx list, o [G, d], lse [G]) from the oracle
    over tokens [0, lengths[s])."""
    p = w_or_params
    G = L.Hq // L.Hkv
    kind = 0 if L.desc_kind == bsa.DESC_MINMAX else 1
    scale = 1.0 / math.sqrt(L.d) if scale is None else scale
    out = {}
    for s, T in enumerate(lengths):
        for h in range(L.Hkv):
            out[(s, h)] = O.decode_group(q[s, h * G:(h + 1) * G], Ks[s][h, :T], Vs[s][h, :T],
                                         L.block, kind, W=W_gate,
                                         budget_tokens=p.budget_tokens,
                                         sparsity_bp=p.sparsity_bp, n_local=p.n_local,
                                         n_min=p.n_min, scale=scale)
    return out


def compare_step(L, idx, cnt, o, lse, ref, groups=None, o_tol=2e-2, lse_rtol=1e-4):
    """Selection bit-exact; o within o_tol absolute; lse within lse_rtol
    relative (denominator max(1, |lse|)).  Returns the worst errors."""
    G = L.Hq // L.Hkv
    idx = idx.cpu().numpy()
    cnt = cnt.cpu().numpy()
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    worst_o, worst_l = 0.0, 0.0
    for (s, h), (ridx, ro, rl) in ref.items():
        if groups is not None and (s, h) not in groups:
            continue
        c = int(cnt[s, h])
        assert c == len(ridx), f"group {(s, h)}: cnt {c} vs oracle {len(ridx)}"
        assert np.array_equal(idx[s, h, :c], ridx), \
            f"group {(s, h)}: selection differs\n gpu {idx[s, h, :c]}\n ref {ridx}"
        assert np.all(idx[s, h, c:] == -1)
        eo = np.abs(o[s, h * G:(h + 1) * G] - ro).max()
        el = (np.abs(lse[s, h * G:(h + 1) * G] - rl) / np.maximum(1.0, np.abs(rl))).max()
        worst_o, worst_l = max(worst_o, eo), max(worst_l, el)
    assert worst_o <= o_tol, f"max |o - o_ref| = {worst_o}"
    assert worst_l <= lse_rtol, f"max lse rel err = {worst_l}"
    return worst_o, worst_l


# --------------------------------------------------------------------------
# Score gap at the top-n boundary
# --------------------------------------------------------------------------

def _scores_and_mag(L, qg, K, T_full, W_gate):
    """Oracle candidate scores of every full block of K[:T_full] and a bound
    on the magnitude of the terms each score sums (for the gap rule)."""
    b = L.block
    if L.desc_kind == bsa.DESC_MINMAX:
        mn, mx = O.desc_minmax(K[:T_full], b)
        s = O.score_quest(qg, mn, mx)
        qd = qg.astype(np.float64)
        mag = (np.abs(qd).sum(0)[None, :] * np.maximum(np.abs(mn), np.abs(mx))).sum(1)
    else:
        mean = O.desc_mean(K[:T_full], b)
        s = O.score_gate(qg, W_gate, mean)
        wv = W_gate.astype(np.float64) @ qg.astype(np.float64).sum(0)
        mag = (np.abs(wv)[None, :] * np.abs(mean)).sum(1)
    return s, mag


def gap_direction(L, qg, W_gate):
    if L.desc_kind == bsa.DESC_MINMAX:
        v = qg.astype(np.float64).sum(0)
    else:
        v = W_gate.astype(np.float64) @ qg.astype(np.float64).sum(0)
    return (v / np.linalg.norm(v)).astype(np.float32)


def enforce_gap(L, params, q, Ks, lengths_per_step, W_gate=None, rel=1e-3, max_iter=30,
                on_shift=None, groups=None):
    """Make the top-n boundary clear-cut at every checked step.

    Ks[s]: [Hkv, T_total, d] float32 (exact stored values; modified in place),
    or a dict {kv head: [T_total, d]} holding only the checked heads.
    lengths_per_step[s]: the cache lengths T at which selection is checked.
    groups: optional set of (s, kv head) to enforce; default all.
    The candidates at length T are the full blocks 0..NB-n_local'-1, which no
    later append changes, so one score array at the final length serves all
    steps.  A violated boundary (gap < rel * max(1, |s|, term magnitude))
    raises the keys of the blocks above it by delta * u (u = the score's
    gradient direction for a uniform key shift), which raises their scores
    uniformly; values are re-rounded to the storage type and everything is
    re-checked.  on_shift(s, kvh, t0, t1, vec) is called for every shift so
    that callers can mirror it into other copies of those tokens."""
    G = L.Hq // L.Hkv
    b = L.block
    for it in range(max_iter):
        changed = False
        for s, steps in enumerate(lengths_per_step):
            Tmax = max(steps)
            for h in range(L.Hkv):
                if groups is not None and (s, h) not in groups:
                    continue
                qg = q[s, h * G:(h + 1) * G]
                NBf = Tmax // b
                sc, mag = _scores_and_mag(L, qg, Ks[s][h], NBf * b, W_gate)
                u = gap_direction(L, qg, W_gate)
                for T in steps:
                    NB = (T + b - 1) // b
                    nl = min(params.n_local, NB)
                    NC = NB - nl
                    n = O.block_count(NB, b, params.budget_tokens, params.sparsity_bp,
                                      params.n_local, params.n_min)
                    k = n - nl
                    if k <= 0 or k >= NC:
                        continue
                    order = sorted(range(NC), key=lambda j: (-sc[j], j))
                    s_in, s_out = sc[order[k - 1]], sc[order[k]]
                    need = rel * max(1.0, abs(s_in), mag[order[k - 1]], mag[order[k]])
                    if s_in - s_out >= need:
                        continue
                    # raise every block above the boundary by ~3x what is missing
                    grad = float(np.dot(
                        u.astype(np.float64),
                        (qg.astype(np.float64).sum(0) if L.desc_kind == bsa.DESC_MINMAX
                         else W_gate.astype(np.float64) @ qg.astype(np.float64).sum(0))))
                    # at least a few storage ulps per channel: the min/max entries
                    # are the largest-magnitude keys, and smaller shifts of them
                    # round away in bf16
                    delta = max(4.0 * (need - (s_in - s_out)) / grad, 0.25 * (1 + it))
                    for j in order[:k]:
                        t0, t1 = j * b, (j + 1) * b
                        Ks[s][h][t0:t1] = W.quantize(Ks[s][h][t0:t1] + delta * u,
                                                     "bf16" if L.kv_dtype == bsa.DTYPE_BF16
                                                     else "f32")
                        if on_shift:
                            on_shift(s, h, t0, t1, delta * u)
                    changed = True
                    break  # scores changed: recompute for this group
        if not changed:
            return it
    raise AssertionError("score gap enforcement did not converge")

"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (its cache layout, selection parameters, workspace and hence
its split counts), on sampled (sequence, KV head) groups.

Every group of the cache is filled (sampled groups from host arrays, the
others from the device generator) and the kernels run over all of them; the
oracle then recomputes the sampled groups one by one from scratch: block
selection bit-exactly (the sampled groups' inputs carry the score gap at
the top-n boundary), o within 2e-2 absolute, lse within 1e-4 relative.
Every other group is read back from the device cache and checked by what
holds whatever the inputs: the kept count, the id layout, a top-n that no
left-out candidate beats by more than the rounding of an fp32 score, and o
and lse against the oracle's attention over the kept blocks."""
import math

import numpy as np
import pytest

import block_sparse_attention_build_amd as bsa
import oracle as O
import workloads as W
from bench import bench_layout
from harness import enforce_gap, page_index_maps, seq_view

pytestmark = pytest.mark.gpu

O_TOL, LSE_RTOL = 2e-2, 1e-4


def _torch():
    import torch
    return torch


class Filled:
    """A cache of workload w at lengths T (per sequence): host float32 K, V
    [T_s + extra, d] for the sampled (s, kvh) groups, device bf16 for all."""

    def __init__(self, w, T, sampled, seed, extra=1, sparsities=None, gate=None):
        self.w, self.T, self.sampled = w, list(T), set(sampled)
        self.L, self.params = bench_layout(w, sparsities, gate)
        # the benchmark's capacity is sized from the workload's contexts; a
        # test that prefills beyond them must still fit
        assert max(self.T) + extra <= self.L.max_blocks * w.block
        self.rng = np.random.Generator(np.random.PCG64(seed))
        self.seed = seed
        self.gen = None
        d, G = w.d, w.G
        self.q = W.quantize(self.rng.standard_normal((w.B, w.Hq, d), dtype=np.float32), w.dtype)
        self.Wg = None
        if w.desc_kind == W.DESC_MEANPOOL:
            self.Wg = W.quantize(self.rng.standard_normal((d, d), dtype=np.float32) / np.sqrt(d),
                                 "bf16")
        self.readback = {}  # (s, h, T) -> K, V, candidate scores, score magnitudes
        self.K = [dict() for _ in range(w.B)]
        self.V = [dict() for _ in range(w.B)]
        self.kscale = {}
        for (s, h) in sorted(self.sampled):
            n = self.T[s] + extra
            ks = self.rng.lognormal(0.0, 0.5, size=d).astype(np.float32)
            vs = self.rng.lognormal(0.0, 0.5, size=d).astype(np.float32)
            K = self.rng.standard_normal((n, d), dtype=np.float32) * ks
            V = self.rng.standard_normal((n, d), dtype=np.float32) * vs
            nb0 = self.T[s] // w.block
            cand = max(nb0 - w.n_local, 0)
            npl = int(round(0.05 * nb0))
            u = W.group_direction(self.q[s, h * G:(h + 1) * G])
            for j in self.rng.choice(cand, size=min(npl, cand), replace=False):
                K[j * w.block:(j + 1) * w.block] += 2.0 * u
            self.K[s][h] = W.quantize(K, w.dtype)
            self.V[s][h] = W.quantize(V, w.dtype)
            self.kscale[(s, h)] = (ks, vs)

    def enforce(self, plist, lengths):
        """Score gap at the boundary of every params in plist at lengths."""
        for _ in range(10):
            moved = 0
            for P in plist:
                moved += enforce_gap(self.L, P, self.q, self.K, [[T] for T in lengths],
                                     W_gate=self.Wg, groups=self.sampled)
            if moved == 0:
                return
        raise AssertionError("score gaps of several sparsities did not settle")

    def device_tokens(self, s, t0, t1):
        """[1, Hkv, t1 - t0, d] device tensor of tokens [t0, t1) of sequence s:
        host rows for sampled heads, device draws for the others."""
        torch = _torch()
        w = self.w
        if self.gen is None:
            self.gen = torch.Generator(device="cuda")
            self.gen.manual_seed(self.seed)
        tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        K = torch.empty(1, w.Hkv, t1 - t0, w.d, dtype=tdt, device="cuda")
        V = torch.empty_like(K)
        for h in range(w.Hkv):
            if (s, h) in self.sampled:
                K[0, h] = torch.from_numpy(self.K[s][h][t0:t1]).to("cuda", tdt)
                V[0, h] = torch.from_numpy(self.V[s][h][t0:t1]).to("cuda", tdt)
            else:
                K[0, h] = torch.randn(t1 - t0, w.d, device="cuda", generator=self.gen).to(tdt)
                V[0, h] = torch.randn(t1 - t0, w.d, device="cuda", generator=self.gen).to(tdt)
        return K, V

    def allocate_and_prefill(self):
        torch = _torch()
        self.cache = bsa.allocate_cache(self.L)
        for s, T in enumerate(self.T):
            L1, c1 = seq_view(self.L, self.cache, s)
            c1.seq_lens.fill_(T)
            K, V = self.device_tokens(s, 0, T)
            bsa.build_block_desc(L1, c1, K, V, T)
            del K, V
        torch.cuda.synchronize()

    def next_tokens(self):
        """Token T_s of every sequence, [B, Hkv, 1, d] K and V on the device."""
        torch = _torch()
        toks = [self.device_tokens(s, T, T + 1) for s, T in enumerate(self.T)]
        return torch.cat([k for k, _ in toks]), torch.cat([v for _, v in toks])

    def append_one(self):
        """Append token T_s of every sequence (one decode step's append)."""
        torch = _torch()
        kn, vn = self.next_tokens()
        self.cache.seq_lens += 1
        bsa.build_block_desc(self.L, self.cache, kn, vn, 1)
        self.T = [T + 1 for T in self.T]
        torch.cuda.synchronize()

    def workspace(self, f=0):
        torch = _torch()
        n = max([bsa.workspace_size(self.L, bsa.OP_STEP, P.n_max) for P in self.params.values()]
                + [bsa.workspace_size(self.L, bsa.OP_DECODE, P.n_max) for P in self.params.values()]
                + ([bsa.workspace_size(self.L, bsa.OP_RECTIFY, f)] if f else []))
        return torch.empty(n, dtype=torch.uint8, device="cuda")


# bound on |gpu score - exact score| relative to the magnitude of the terms
# a score sums: a few hundred fp32 roundings of 2^-24 each at most
SCORE_RTOL = 1e-4


def read_tokens(F, s, h, t0, t1):
    """K, V [t1 - t0, d] float32 of tokens [t0, t1) of group (s, h) as the
    device cache holds them, gathered through the page table."""
    L, b, d = F.L, F.w.block, F.w.d
    j0, j1 = t0 // b, -(-t1 // b)
    pages = F.cache.page_table[s, j0:j1].long()
    km, vm = page_index_maps(L)
    kp = F.cache.k_pool[pages, h].float().cpu().numpy()
    vp = F.cache.v_pool[pages, h].float().cpu().numpy()
    n = (j1 - j0) * b
    K = np.ascontiguousarray(kp[:, km].reshape(n, d)[t0 - j0 * b:t1 - j0 * b])
    V = np.ascontiguousarray(vp[:, vm].reshape(n, d)[t0 - j0 * b:t1 - j0 * b])
    return K, V


def group_from_cache(F, s, h):
    """K, V [T_s, d] float32 of group (s, h) as the device cache holds them
    (gathered through the page table), the oracle scores of its full blocks
    and, per block, the magnitude of the terms its score sums."""
    T = F.T[s]
    hit = F.readback.get((s, h, T))
    if hit is not None:
        return hit
    b, d, G = F.w.block, F.w.d, F.w.G
    K, V = read_tokens(F, s, h, 0, T)
    qg = F.q[s, h * G:(h + 1) * G]
    qa = np.abs(qg.astype(np.float64)).sum(0)
    nfull = T // b
    Kb = K[:nfull * b].reshape(nfull, b, d).astype(np.float64)
    if F.w.desc_kind == W.DESC_MINMAX:
        mn, mx = O.desc_minmax(K[:nfull * b], b)
        S = O.score_quest(qg, mn, mx)
        mag = (qa[None, :] * np.maximum(np.abs(mn), np.abs(mx))).sum(1)
    else:
        S = O.score_gate(qg, F.Wg, O.desc_mean(K[:nfull * b], b))
        wa = np.abs(F.Wg.astype(np.float64)) @ qa
        mag = (wa[None, :] * np.abs(Kb).mean(1)).sum(1)
    del Kb
    F.readback[(s, h, T)] = (K, V, S, mag)
    return K, V, S, mag


def check_every_group(F, P, idx, cnt, o, lse, scale):
    """Every group of the batch (numpy idx, cnt, o, lse from the device):
    the kept count is the closed form at the group's length; the ids are the
    picked candidates in ascending order, then the local blocks, then -1; no
    left-out candidate outscores a kept one by more than SCORE_RTOL of the
    scores' term magnitude; o and lse match the oracle's attention over the
    kept blocks of the cache's own K and V."""
    w, b, G = F.w, F.w.block, F.w.G
    worst = 0.0
    n_exact = 0
    for s in range(w.B):
        T = F.T[s]
        NB = -(-T // b)
        nl = min(P.n_local, NB)
        NC = NB - nl
        n = O.block_count(NB, b, P.budget_tokens, P.sparsity_bp, P.n_local, P.n_min)
        for h in range(w.Hkv):
            K, V, S, mag = group_from_cache(F, s, h)
            c = int(cnt[s, h])
            assert c == n, (s, h, c, n)
            ids = idx[s, h, :c]
            assert np.all(idx[s, h, c:] == -1), (s, h)
            assert np.all(np.diff(ids) > 0), (s, h)
            assert np.array_equal(ids[c - nl:], np.arange(NC, NB)), (s, h)
            picked = ids[:c - nl]
            assert picked.size == 0 or (picked[0] >= 0 and picked[-1] < NC), (s, h)
            assert NC <= S.shape[0]
            kept = np.zeros(NC, bool)
            kept[picked] = True
            if kept.any() and not kept.all():
                inv = S[:NC][~kept].max() - S[:NC][kept].min()
                rel = inv / mag[:NC].max()
                assert rel <= SCORE_RTOL, (s, h, rel)
                worst = max(worst, rel)
            # the oracle's own pick from its exact scores, counted (near-ties
            # at the boundary may legitimately go either way)
            n_exact += int(np.array_equal(ids, O.select(S[:NC], NB, n, P.n_local)))
            for g in range(G):
                ro, rl = O.attend(F.q[s, h * G + g], K, V, b, ids, scale)
                eo = np.abs(o[s, h * G + g] - ro).max()
                el = abs(lse[s, h * G + g] - rl) / max(1.0, abs(rl))
                assert eo <= O_TOL, (s, h, g, eo)
                assert el <= LSE_RTOL, (s, h, g, el)
    print(f"{w.name}: all {w.B * w.Hkv} groups valid, {n_exact} with the oracle's exact pick; "
          f"worst score inversion {worst:.2e} of the term magnitude", flush=True)


def select_decode_and_check(F, P, ws, every_group=False, one_call=False):
    """Select and decode at the current lengths (one_call=False: the cache
    already holds the step's token; bsa_select_blocks + bsa_sparse_decode),
    or append token T_s of every sequence and do the whole step in one
    bsa_append_select_decode call, the call the benchmark times
    (one_call=True); then check against the oracle."""
    torch = _torch()
    w, L = F.w, F.L
    G = w.G
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q_dev = torch.from_numpy(F.q).to("cuda", tdt)
    idx = torch.full((w.B, w.Hkv, P.n_max), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((w.B, w.Hkv), -7, dtype=torch.int32, device="cuda")
    o = torch.full((w.B, w.Hq, w.d), float("nan"), dtype=tdt, device="cuda")
    lse = torch.full((w.B, w.Hq), float("nan"), dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(w.d)
    if one_call:
        kn, vn = F.next_tokens()
        F.cache.seq_lens += 1
        F.T = [T + 1 for T in F.T]
        bsa.append_select_decode(L, F.cache, kn, vn, q_dev, P, idx, cnt, scale, o, lse, ws)
    else:
        bsa.select_blocks(L, F.cache, q_dev, P, idx, cnt, ws)
        bsa.sparse_decode(L, F.cache, q_dev, idx, cnt, P.n_max, scale, o, lse, ws)
    torch.cuda.synchronize()
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    kind = 0 if w.desc_kind == W.DESC_MINMAX else 1
    for (s, h) in sorted(F.sampled):
        T = F.T[s]
        ridx, ro, rl = O.decode_group(F.q[s, h * G:(h + 1) * G], F.K[s][h][:T], F.V[s][h][:T],
                                      w.block, kind, W=F.Wg, budget_tokens=P.budget_tokens,
                                      sparsity_bp=P.sparsity_bp, n_local=P.n_local,
                                      n_min=P.n_min, scale=scale)
        c = int(cnt[s, h])
        assert c == len(ridx), (s, h, c, len(ridx))
        assert np.array_equal(idx[s, h, :c], ridx), (s, h)
        assert np.all(idx[s, h, c:] == -1)
        eo = np.abs(o[s, h * G:(h + 1) * G] - ro).max()
        el = (np.abs(lse[s, h * G:(h + 1) * G] - rl) / np.maximum(1.0, np.abs(rl))).max()
        assert eo <= O_TOL, (s, h, eo)
        assert el <= LSE_RTOL, (s, h, el)
    if every_group:
        check_every_group(F, P, idx, cnt, o, lse, scale)


@pytest.mark.parametrize("form", ["one_call", "separate"])
@pytest.mark.parametrize("name,sampled", [
    ("qwen3_4b_32k", [(0, h) for h in range(8)]),
    ("batched_64k_gate", [(0, 0), (3, 5), (7, 7)]),
])
def test_fullsize_decode_step(name, sampled, form):
    torch = _torch()
    w = W.get(name)
    gate = None
    F0_seed = 1000 + w.cfg_id
    F = Filled(w, w.T0, sampled, F0_seed)
    if F.Wg is not None:
        gate = torch.from_numpy(F.Wg).to("cuda", torch.bfloat16)
        for P in F.params.values():
            P.gate_w = gate
    P = F.params[w.sparsity_bp]
    F.enforce([P], [T + 1 for T in F.T])
    F.allocate_and_prefill()
    if form == "one_call":  # in-launch selection (rows of 575 and 542 candidates)
        select_decode_and_check(F, P, F.workspace(), every_group=True, one_call=True)
    else:
        F.append_one()
        select_decode_and_check(F, P, F.workspace(), every_group=True)


def test_split_cap_decides_the_split_count():
    """256 groups (32 sequences x 8 KV heads) leave one split per group by the
    workgroup target, but a split covers at most 4096 kept blocks (its block
    and page ids are staged in LDS): 4400 kept blocks per group therefore run
    as two splits.  Ragged contexts of 150K-181K tokens, b = 32, d = 64,
    G = 8, token budget 140800 (4400 blocks)."""
    w = W.Workload("split_cap", 90, B=32, Hq=64, Hkv=8, d=64, dtype="bf16",
                   T0=tuple(150000 + 1000 * i for i in range(32)), block=32,
                   budget_tokens=4400 * 32, n_local=2, n_min=0)
    F = Filled(w, w.T0, [(0, 3), (17, 0), (31, 7)], 1090)
    P = F.params[w.sparsity_bp]
    assert P.n_max == 4400
    F.enforce([P], [T + 1 for T in F.T])
    F.allocate_and_prefill()
    F.append_one()
    select_decode_and_check(F, P, F.workspace())


def test_fullsize_512k_sparsity_sweep():
    w = W.get("long_512k")
    sweep = [w.sparsity_bp] + [b for b in w.sparsity_sweep if b != w.sparsity_bp]
    F = Filled(w, w.T0, [(0, 2), (0, 7)], 1004, sparsities=sweep)
    F.enforce(list(F.params.values()), [T + 1 for T in F.T])
    F.allocate_and_prefill()
    F.append_one()
    ws = F.workspace()
    for bp in sweep:
        select_decode_and_check(F, F.params[bp], ws, every_group=True)


@pytest.mark.parametrize("f", [32, 64, 128])
def test_fullsize_resa_rectify_then_decode(f):
    """The ragged ReSA workload at the rectify intervals the ReSA page
    recommends (Key points: f = 32 or 64, and 128): caches at T0 + f tokens,
    one rectify of the last f tokens (checked on the sampled groups' rows and
    cache contents), then one decode step over the rectified cache.  At G = 4,
    f = 64 is one 256-row group per KV head and f = 128 two, run as two
    co-scheduled sets of workgroups over the same tile list."""
    torch = _torch()
    w = W.get("resa_ragged", rectify_f=f)
    G = w.G
    sampled = [(0, 1), (3, 6)]
    T = [t + f for t in w.T0]
    F = Filled(w, T, sampled, 1005)
    P = F.params[w.sparsity_bp]
    # the rectified tokens lie in the local blocks of the next step, so the
    # candidates' gap can be set before the rectification
    F.enforce([P], [t + 1 for t in T])
    F.allocate_and_prefill()
    rng = np.random.Generator(np.random.PCG64(77))
    qr = W.quantize(rng.standard_normal((w.B, w.Hq, f, w.d), dtype=np.float32), w.dtype)
    kr = torch.empty(w.B, w.Hkv, f, w.d, dtype=torch.bfloat16, device="cuda")
    vr = torch.empty_like(kr)
    kr_h, vr_h = {}, {}
    for s in range(w.B):
        for h in range(w.Hkv):
            if (s, h) in F.sampled:
                ks, vs = F.kscale[(s, h)]
                Ts = T[s]
                kn = W.quantize(F.K[s][h][Ts - f:Ts] + 0.1 * ks * rng.standard_normal((f, w.d), dtype=np.float32), "bf16")
                vn = W.quantize(F.V[s][h][Ts - f:Ts] + 0.1 * vs * rng.standard_normal((f, w.d), dtype=np.float32), "bf16")
                kr_h[(s, h)], vr_h[(s, h)] = kn, vn
                kr[s, h] = torch.from_numpy(kn).to("cuda", torch.bfloat16)
                vr[s, h] = torch.from_numpy(vn).to("cuda", torch.bfloat16)
            else:
                kr[s, h] = torch.randn(f, w.d, device="cuda").to(torch.bfloat16)
                vr[s, h] = torch.randn(f, w.d, device="cuda").to(torch.bfloat16)
    ws = F.workspace(f)
    o = torch.full((w.B, w.Hq, f, w.d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((w.B, w.Hq, f), float("nan"), dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(w.d)
    bsa.rectify_chunk(F.L, F.cache, torch.from_numpy(qr).to("cuda", torch.bfloat16), kr, vr, f,
                      scale, o, lse, ws)
    torch.cuda.synchronize()
    o, lse = o.float().cpu().numpy(), lse.cpu().numpy()
    for (s, h) in sorted(F.sampled):
        Ts = T[s]
        Kh = F.K[s][h][:Ts]  # views: the oracle overwrites [Ts - f, Ts) in place
        Vh = F.V[s][h][:Ts]
        ro, rl = O.rectify(qr[s, h * G:(h + 1) * G], Kh, Vh, kr_h[(s, h)], vr_h[(s, h)], scale)
        assert np.array_equal(F.K[s][h][Ts - f:Ts], kr_h[(s, h)])
        eo = np.abs(o[s, h * G:(h + 1) * G] - ro).max()
        el = (np.abs(lse[s, h * G:(h + 1) * G] - rl) / np.maximum(1.0, np.abs(rl))).max()
        assert eo <= O_TOL, (s, h, eo)
        assert el <= LSE_RTOL, (s, h, el)
    # every group's cache now holds its re-encoded tokens, bit for bit
    kr_all, vr_all = kr.float().cpu().numpy(), vr.float().cpu().numpy()
    for s in range(w.B):
        for h in range(w.Hkv):
            Kc, Vc = read_tokens(F, s, h, T[s] - f, T[s])
            assert np.array_equal(Kc, kr_all[s, h]) and np.array_equal(Vc, vr_all[s, h]), (s, h)
    F.append_one()
    select_decode_and_check(F, P, ws, every_group=True)


def test_fullsize_resa_loop_two_rectifies():
    """The ragged ReSA loop at full size for 2f steps: every step appends a
    token, selects and decodes in one bsa_append_select_decode call (the
    call the benchmark times; 2110 candidates select in-launch); after steps
    f and 2f the last f tokens are rectified.  On two
    sampled groups (the 16K and the 128K sequence) the oracle follows on host
    copies that take the same rewrites: the rectify rows at each rectify, and
    the selection (bit-exact), o and lse at sampled steps before, between and
    after the rectifies.  The candidates' score gap holds at every checked
    length: over 2f = 64 steps no block changes from local to candidate
    (contexts start block-aligned), and the rewritten tokens lie in the
    current block."""
    torch = _torch()
    w = W.get("resa_ragged")
    f = w.rectify_f
    G = w.G
    steps = 2 * f
    sampled = [(0, 1), (3, 6)]
    F = Filled(w, w.T0, sampled, 1006, extra=steps)
    P = F.params[w.sparsity_bp]
    assert all(t % w.block == 0 for t in w.T0) and steps <= w.block
    F.enforce([P], [t + steps for t in w.T0])
    F.allocate_and_prefill()
    ws = F.workspace(f)
    scale = 1.0 / math.sqrt(w.d)
    tdt = torch.bfloat16
    rng = np.random.Generator(np.random.PCG64(78))
    idx = torch.empty(w.B, w.Hkv, P.n_max, dtype=torch.int32, device="cuda")
    cnt = torch.empty(w.B, w.Hkv, dtype=torch.int32, device="cuda")
    o = torch.empty(w.B, w.Hq, w.d, dtype=tdt, device="cuda")
    lse = torch.empty(w.B, w.Hq, dtype=torch.float32, device="cuda")
    check_at = {1, 2, f - 1, f, f + 1, f + 17, steps}
    n_checked = 0
    for k in range(1, steps + 1):
        # one decode step: the step's query is fresh, the sampled groups' from host
        qh = W.quantize(rng.standard_normal((w.B, w.Hq, w.d), dtype=np.float32), w.dtype)
        for (s, h) in sampled:
            qh[s, h * G:(h + 1) * G] = F.q[s, h * G:(h + 1) * G]
        toks = [F.device_tokens(s, T, T + 1) for s, T in enumerate(F.T)]
        kn = torch.cat([a for a, _ in toks])
        vn = torch.cat([b for _, b in toks])
        F.cache.seq_lens += 1
        F.T = [T + 1 for T in F.T]
        q_dev = torch.from_numpy(qh).to("cuda", tdt)
        # the step as the benchmark times it: one call, selecting in-launch
        bsa.append_select_decode(F.L, F.cache, kn, vn, q_dev, P, idx, cnt, scale, o, lse, ws)
        if k in check_at:
            torch.cuda.synchronize()
            gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
            go, gl = o.float().cpu().numpy(), lse.cpu().numpy()
            for (s, h) in sampled:
                T = F.T[s]
                ridx, ro, rl = O.decode_group(F.q[s, h * G:(h + 1) * G], F.K[s][h][:T],
                                              F.V[s][h][:T], w.block, 0,
                                              sparsity_bp=P.sparsity_bp, n_local=P.n_local,
                                              n_min=P.n_min, scale=scale)
                c = int(gc[s, h])
                assert c == len(ridx) and np.array_equal(gi[s, h, :c], ridx), (k, s, h)
                assert np.abs(go[s, h * G:(h + 1) * G] - ro).max() <= O_TOL, (k, s, h)
                el = np.abs(gl[s, h * G:(h + 1) * G] - rl) / np.maximum(1.0, np.abs(rl))
                assert el.max() <= LSE_RTOL, (k, s, h)
                n_checked += 1
        if k % f == 0:
            # rectify the last f tokens of every sequence
            qr = W.quantize(rng.standard_normal((w.B, w.Hq, f, w.d), dtype=np.float32), w.dtype)
            kr = torch.empty(w.B, w.Hkv, f, w.d, dtype=tdt, device="cuda")
            vr = torch.empty_like(kr)
            new = {}
            for s in range(w.B):
                for h in range(w.Hkv):
                    if (s, h) in F.sampled:
                        ks, vs = F.kscale[(s, h)]
                        Ts = F.T[s]
                        kh = W.quantize(F.K[s][h][Ts - f:Ts] + 0.1 * ks *
                                        rng.standard_normal((f, w.d), dtype=np.float32), "bf16")
                        vh = W.quantize(F.V[s][h][Ts - f:Ts] + 0.1 * vs *
                                        rng.standard_normal((f, w.d), dtype=np.float32), "bf16")
                        new[(s, h)] = (kh, vh)
                        kr[s, h] = torch.from_numpy(kh).to("cuda", tdt)
                        vr[s, h] = torch.from_numpy(vh).to("cuda", tdt)
                    else:
                        kr[s, h] = torch.randn(f, w.d, device="cuda").to(tdt)
                        vr[s, h] = torch.randn(f, w.d, device="cuda").to(tdt)
            orr = torch.empty(w.B, w.Hq, f, w.d, dtype=tdt, device="cuda")
            lr = torch.empty(w.B, w.Hq, f, dtype=torch.float32, device="cuda")
            bsa.rectify_chunk(F.L, F.cache, torch.from_numpy(qr).to("cuda", tdt), kr, vr, f,
                              scale, orr, lr, ws)
            torch.cuda.synchronize()
            orr, lr = orr.float().cpu().numpy(), lr.cpu().numpy()
            for (s, h) in sampled:
                Ts = F.T[s]
                kh, vh = new[(s, h)]
                # the oracle rewrites the host copies in place, which the
                # following steps' checks then see
                ro, rl = O.rectify(qr[s, h * G:(h + 1) * G], F.K[s][h][:Ts], F.V[s][h][:Ts],
                                   kh, vh, scale)
                assert np.array_equal(F.K[s][h][Ts - f:Ts], kh)
                assert np.abs(orr[s, h * G:(h + 1) * G] - ro).max() <= O_TOL, (k, s, h)
                el = np.abs(lr[s, h * G:(h + 1) * G] - rl) / np.maximum(1.0, np.abs(rl))
                assert el.max() <= LSE_RTOL, (k, s, h)
                n_checked += 1
    assert n_checked == 2 * (len(check_at) + 2)

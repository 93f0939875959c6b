"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times (its cache layout, selection parameters, workspace and hence
its split counts), on sampled (sequence, KV head) groups.

Every group of the cache is filled (sampled groups from host arrays, the
others from the device generator) and the kernels run over all of them; the
oracle then recomputes the sampled groups one by one from scratch: block
selection bit-exactly (the sampled groups' inputs carry the score gap at
the top-n boundary), o within 2e-2 absolute, lse within 1e-4 relative."""
import math

import numpy as np
import pytest

import block_sparse_attention_build_amd as bsa
import oracle as O
import workloads as W
from bench import bench_layout
from harness import enforce_gap, seq_view

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

    def append_one(self):
        """Append token T_s of every sequence (one decode step's append)."""
        torch = _torch()
        w = self.w
        toks = [self.device_tokens(s, T, T + 1) for s, T in enumerate(self.T)]
        kn = torch.cat([k for k, _ in toks])
        vn = torch.cat([v for _, v in toks])
        self.cache.seq_lens += 1
        bsa.build_block_desc(self.L, self.cache, kn, vn, 1)
        self.T = [T + 1 for T in self.T]
        torch.cuda.synchronize()

    def workspace(self, f=0):
        torch = _torch()
        n = max([bsa.workspace_size(self.L, bsa.OP_SELECT, P.n_max) for P in self.params.values()]
                + [bsa.workspace_size(self.L, bsa.OP_DECODE, P.n_max) for P in self.params.values()]
                + ([bsa.workspace_size(self.L, bsa.OP_RECTIFY, f)] if f else []))
        return torch.empty(n, dtype=torch.uint8, device="cuda")


def select_decode_and_check(F, P, ws):
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


@pytest.mark.parametrize("name,sampled", [
    ("qwen3_4b_32k", [(0, h) for h in range(8)]),
    ("batched_64k_gate", [(0, 0), (3, 5), (7, 7)]),
])
def test_fullsize_decode_step(name, sampled):
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
    F.append_one()
    select_decode_and_check(F, P, F.workspace())


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
        select_decode_and_check(F, F.params[bp], ws)


def test_fullsize_resa_rectify_then_decode():
    """The ragged ReSA workload: caches at T0 + f tokens, one rectify of the
    last f tokens (checked on the sampled groups' rows and cache contents),
    then one decode step over the rectified cache."""
    torch = _torch()
    w = W.get("resa_ragged")
    f = w.rectify_f
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
    F.append_one()
    select_decode_and_check(F, P, ws)

"""Seeded synthetic workloads for block-sparse attention decoding.

This module is shared by the tests and the benchmark.  It produces inputs
only -- queries, key/value caches, appended tokens, gate weights, re-encoded
keys/values -- and holds none of the method's arithmetic (no descriptors, no
scores, no selection, no attention).

Shapes come from the five workloads the method is measured on (a tiny fp32
case, a Qwen3-4B-like single layer at 32K, a batch of eight 64K sequences
with a plug-in gate, a 512K single sequence with a sparsity sweep and a
ragged ReSA-style rectified decode loop).  Value recipe:
  * q, K, V ~ N(0, 1) drawn as float32 from numpy's PCG64 (host) or from a
    seeded torch generator (device), K and V multiplied by a per
    (KV head, channel) scale ~ LogNormal(0, 0.5) drawn separately for K and V;
  * bf16 workloads are rounded to bf16 with round-to-nearest-even;
  * "planted" salient blocks: the keys of a chosen set of non-local blocks get
    +2 * u added, u = (sum of the group's query heads) / |that sum|;
  * gate weight W ~ N(0, 1/d), rounded to bf16;
  * re-encoded keys/values for rectification: old + 0.1 * scale * N(0, 1).
Seed of workload c, layer l: 0x5EED0000 + 16 * c + l.
"""
from dataclasses import dataclass, field, replace
from typing import List, Optional

import numpy as np

SEED_BASE = 0x5EED0000

DESC_MINMAX = 0
DESC_MEANPOOL = 1


@dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    B: int
    Hq: int
    Hkv: int
    d: int
    dtype: str                 # "bf16" or "f32"
    T0: tuple                  # context length of each sequence before decoding
    block: int
    budget_tokens: int = 0     # > 0: size the kept set by a token budget
    sparsity_bp: int = 0       # otherwise: sparsity p in basis points (9000 = 0.9)
    n_local: int = 1
    n_min: int = 0
    desc_kind: int = DESC_MINMAX
    steps: int = 16
    rectify_f: int = 0         # 0: no rectification
    planted_frac: float = 0.0  # fraction of non-local blocks planted
    planted_count: int = 0     # or an explicit count
    sparsity_sweep: tuple = ()

    @property
    def G(self):
        return self.Hq // self.Hkv

    def max_T(self):
        return max(self.T0) + self.steps

    def max_blocks(self):
        return (self.max_T() + self.block - 1) // self.block

    def seed(self, layer=0):
        return SEED_BASE + 16 * self.cfg_id + layer


WORKLOADS = {
    "tiny": Workload("tiny", 1, B=1, Hq=4, Hkv=1, d=64, dtype="f32", T0=(2048,),
                     block=64, budget_tokens=512, n_local=1, n_min=2, steps=16,
                     planted_count=3),
    "qwen3_4b_32k": Workload("qwen3_4b_32k", 2, B=1, Hq=32, Hkv=8, d=128, dtype="bf16",
                             T0=(32768,), block=64, budget_tokens=4096, n_local=1,
                             n_min=0, steps=128, planted_frac=0.05),
    "batched_64k_gate": Workload("batched_64k_gate", 3, B=8, Hq=32, Hkv=8, d=128,
                                 dtype="bf16", T0=(65536,) * 8, block=128,
                                 sparsity_bp=9000, n_local=2, n_min=0,
                                 desc_kind=DESC_MEANPOOL, steps=128, planted_frac=0.05),
    "long_512k": Workload("long_512k", 4, B=1, Hq=32, Hkv=8, d=128, dtype="bf16",
                          T0=(524288,), block=64, sparsity_bp=9000, n_local=2, n_min=16,
                          steps=128, planted_frac=0.05, sparsity_sweep=(9000, 9500, 9800)),
    "resa_ragged": Workload("resa_ragged", 5, B=4, Hq=32, Hkv=8, d=128, dtype="bf16",
                            T0=(16384, 49152, 98304, 131072), block=64, sparsity_bp=9500,
                            n_local=2, n_min=16, steps=512, rectify_f=32,
                            planted_frac=0.05),
}


def get(name, **overrides) -> Workload:
    w = WORKLOADS[name]
    return replace(w, **overrides) if overrides else w


# ---------------------------------------------------------------------------
# bf16 rounding (round-to-nearest-even), host side
# ---------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round-to-nearest-even.
    Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rnd = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rnd) >> 16).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits).astype(np.uint32) << 16).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bf16 value (kept as float32)."""
    return bf16_to_f32(bf16_bits(x))


def quantize(x: np.ndarray, dtype: str) -> np.ndarray:
    x = np.asarray(x, np.float32)
    return round_bf16(x) if dtype == "bf16" else x


# ---------------------------------------------------------------------------
# Host-side generation (numpy PCG64)
# ---------------------------------------------------------------------------

@dataclass
class HostInputs:
    """Everything one decode run needs, as float32 arrays holding the exact
    stored values (bf16-representable for bf16 workloads)."""
    w: Workload
    q: np.ndarray                    # [B, Hq, d]   (fixed over the steps)
    K: List[np.ndarray]              # per sequence [Hkv, T0+steps, d]
    V: List[np.ndarray]              # (tokens T0.. are the appended ones)
    W: Optional[np.ndarray] = None   # [d, d] gate weight (mean-pool workloads)
    k_scale: Optional[np.ndarray] = None  # [Hkv, d]
    v_scale: Optional[np.ndarray] = None
    planted: List[np.ndarray] = field(default_factory=list)  # per seq: block ids


def _channel_scales(rng, Hkv, d):
    return rng.lognormal(0.0, 0.5, size=(Hkv, d)).astype(np.float32)


def group_direction(q_group: np.ndarray) -> np.ndarray:
    """Unit vector along the sum of a GQA group's query heads ([G, d])."""
    s = q_group.astype(np.float64).sum(axis=0)
    return (s / np.linalg.norm(s)).astype(np.float32)


def make_host(w: Workload, layer: int = 0, steps: Optional[int] = None,
              T0: Optional[tuple] = None) -> HostInputs:
    """Generate a full decode run on the host.  The cache of sequence b holds
    T0[b] prefilled tokens followed by `steps` appended tokens; q is fixed
    over the steps (parity runs keep the planted blocks clear-cut)."""
    steps = w.steps if steps is None else steps
    T0 = w.T0 if T0 is None else T0
    rng = np.random.Generator(np.random.PCG64(w.seed(layer)))
    d, Hkv, G = w.d, w.Hkv, w.G
    k_scale = _channel_scales(rng, Hkv, d)
    v_scale = _channel_scales(rng, Hkv, d)
    q = quantize(rng.standard_normal((w.B, w.Hq, d), dtype=np.float32), w.dtype)
    W = None
    if w.desc_kind == DESC_MEANPOOL:
        W = quantize(rng.standard_normal((d, d), dtype=np.float32) / np.sqrt(d), "bf16")
    Ks, Vs, planted = [], [], []
    for b in range(w.B):
        T = T0[b] + steps
        K = rng.standard_normal((Hkv, T, d), dtype=np.float32) * k_scale[:, None, :]
        V = rng.standard_normal((Hkv, T, d), dtype=np.float32) * v_scale[:, None, :]
        nb0 = T0[b] // w.block                     # complete prefilled blocks
        n_plant = w.planted_count or int(round(w.planted_frac * nb0))
        cand = max(nb0 - w.n_local, 0)
        pb = np.sort(rng.choice(cand, size=min(n_plant, cand), replace=False)) \
            if cand > 0 and n_plant > 0 else np.zeros(0, np.int64)
        for kvh in range(Hkv):
            u = group_direction(q[b, kvh * G:(kvh + 1) * G])
            for j in pb:
                K[kvh, j * w.block:(j + 1) * w.block] += 2.0 * u
        Ks.append(quantize(K, w.dtype))
        Vs.append(quantize(V, w.dtype))
        planted.append(pb)
    return HostInputs(w=w, q=q, K=Ks, V=Vs, W=W, k_scale=k_scale, v_scale=v_scale,
                      planted=planted)


def make_rectify_kv(w: Workload, K_old: np.ndarray, V_old: np.ndarray,
                    k_scale: np.ndarray, v_scale: np.ndarray, seed: int):
    """Re-encoded keys/values for a rectification of the last f tokens:
    old + 0.1 * scale * N(0, 1).  K_old, V_old: [Hkv, f, d]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    kn = K_old + 0.1 * k_scale[:, None, :] * rng.standard_normal(K_old.shape, dtype=np.float32)
    vn = V_old + 0.1 * v_scale[:, None, :] * rng.standard_normal(V_old.shape, dtype=np.float32)
    return quantize(kn, w.dtype), quantize(vn, w.dtype)


def make_queries(w: Workload, seed: int, shape_tail=()):
    """Fresh seeded queries [B, Hq, *shape_tail, d] (host)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return quantize(rng.standard_normal((w.B, w.Hq) + tuple(shape_tail) + (w.d,),
                                        dtype=np.float32), w.dtype)


# ---------------------------------------------------------------------------
# Device-side generation (torch; benchmark-sized caches)
# ---------------------------------------------------------------------------

def make_device_kv(w: Workload, layer: int, seq: int, T: int, device, gen=None):
    """Seeded K, V for one sequence on the device: [Hkv, T, d] in the
    workload's dtype, same recipe as the host generator (scales, planting
    along the direction of a seeded query group sum).  Returns (K, V, q)
    with q [Hq, d] the query used for the planting direction."""
    import torch
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    g = torch.Generator(device=device)
    g.manual_seed(w.seed(layer) * 1000 + seq)
    d, Hkv, G = w.d, w.Hkv, w.G
    k_scale = torch.empty(Hkv, d, device=device).log_normal_(0.0, 0.5, generator=g)
    v_scale = torch.empty(Hkv, d, device=device).log_normal_(0.0, 0.5, generator=g)
    q = torch.randn(w.Hq, d, device=device, generator=g)
    K = torch.empty(Hkv, T, d, device=device, dtype=tdt)
    V = torch.empty(Hkv, T, d, device=device, dtype=tdt)
    chunk = 1 << 16
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        K[:, t0:t1] = (torch.randn(Hkv, t1 - t0, d, device=device, generator=g)
                       * k_scale[:, None, :]).to(tdt)
        V[:, t0:t1] = (torch.randn(Hkv, t1 - t0, d, device=device, generator=g)
                       * v_scale[:, None, :]).to(tdt)
    nb0 = T // w.block
    n_plant = w.planted_count or int(round(w.planted_frac * nb0))
    cand = max(nb0 - w.n_local, 0)
    if cand > 0 and n_plant > 0:
        pb = torch.randperm(cand, device=device, generator=g)[:n_plant]
        u = q.view(Hkv, G, d).sum(1)
        u = u / u.norm(dim=-1, keepdim=True)
        tok = (pb[:, None] * w.block + torch.arange(w.block, device=device)[None, :]).reshape(-1)
        K[:, tok] = (K[:, tok].float() + 2.0 * u[:, None, :]).to(tdt)
    return K, V, q.to(tdt)

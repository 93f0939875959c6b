"""Benchmark: block-sparse attention decode on one MI355X.

One step = the whole decode hot path for one generated token of every
sequence, run for L distinct layer caches (default 8, so that the kept-block
working set cannot stay resident in the 256 MB last-level cache):
  seq_lens += 1                          (shared by the layers)
  per layer: bsa_build_block_desc (append the new k, v; update descriptors)
             bsa_select_blocks     (score every non-local block, top-n)
             bsa_sparse_decode     (split-K attention over the kept blocks,
                                    log-sum-exp merge)
Queries and appended tokens are fresh per step and seeded; caches are
generated on the device from the workload recipe.  Timing: W untimed warm-up
steps, then K steps between two HIP events on the stream the library runs on
(torch's current stream), after a device synchronize.  Each decode call is
also bracketed by its own events to give the decode kernel's average launch
duration for the roofline.

Output: one JSON line.  value = effective HBM GB/s of the whole step:
  effective bytes / step / layer = descriptor bytes of every block
  + K and V bytes of every kept token (the method's algorithmic bytes);
ms_per_step covers all L layers; us_per_step_layer = ms_per_step*1000/L.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=32)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="long_512k")
    ap.add_argument("--sparsity-bp", type=int, default=None,
                    help="override the workload's sparsity (basis points)")
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-steps", type=int, default=2)
    ap.add_argument("--extra", action="store_true",
                    help="also measure the other workloads (sparsity sweep, batched, 32K, ReSA loop)")
    return ap.parse_args()


def effective_bytes(w, lengths, n_kept, d, esize):
    """Descriptor bytes of every block + K/V bytes of every kept token, for
    one layer.  n_kept[s] blocks kept per (sequence, kv head); the last block
    (always kept) holds T - (NB-1)*b tokens."""
    b = w.block
    desc_per_block = 2 * d * esize if w.desc_kind == 0 else d * 4
    tot_desc = tot_kv = 0
    for T, n in zip(lengths, n_kept):
        NB = (T + b - 1) // b
        tokens = n * b - (NB * b - T)
        tot_desc += w.Hkv * NB * desc_per_block
        tot_kv += w.Hkv * tokens * 2 * d * esize
    return tot_desc, tot_kv


class Run:
    """L layer caches of one workload, ready for decode steps."""

    def __init__(self, w, layers, sparsity_bp, dev, keep_host_layer0=False):
        import torch
        import block_sparse_attention_build_amd as bsa
        import workloads as W
        self.w, self.layers, self.dev = w, layers, dev
        self.bsa = bsa
        self.steps_done = 0
        T0 = list(w.T0)
        self.T0 = T0
        cap_tokens = max(T0) + 4096
        max_blocks = (cap_tokens + w.block - 1) // w.block
        kv = bsa.DTYPE_BF16 if w.dtype == "bf16" else bsa.DTYPE_F32
        self.L = bsa.Layout(w.B, w.Hq, w.Hkv, w.d, w.block, max_blocks, kv, w.desc_kind)
        self.P = bsa.SelectParams(budget_tokens=w.budget_tokens, sparsity_bp=sparsity_bp,
                                  n_local=w.n_local, n_min=w.n_min)
        self.P.n_max = bsa.block_count(self.P, max_blocks, w.block)
        self.tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        self.seq_lens = torch.zeros(w.B, dtype=torch.int32, device=dev)
        self.caches = []
        self.host = None
        for l in range(layers):
            c = bsa.allocate_cache(self.L, device=dev)
            c.seq_lens = self.seq_lens
            for s in range(w.B):
                K, V, qdir = W.make_device_kv(w, l, s, T0[s], dev)
                L1 = bsa.Layout(1, w.Hq, w.Hkv, w.d, w.block, max_blocks, kv, w.desc_kind)
                c1 = bsa.Cache(c.k_pool, c.v_pool, c.page_table[s:s + 1],
                               self.seq_lens[s:s + 1], c.desc[s:s + 1])
                self.seq_lens[s] = T0[s]
                bsa.build_block_desc(L1, c1, K[None], V[None], T0[s])
                if keep_host_layer0 and l == 0 and s == 0:
                    self.host = (K.float().cpu().numpy(), V.float().cpu().numpy())
                del K, V
            self.caches.append(c)
        torch.cuda.synchronize()
        if w.desc_kind == W.DESC_MEANPOOL:
            g = torch.Generator(device=dev)
            g.manual_seed(w.seed(0) + 7)
            self.P.gate_w = (torch.randn(w.d, w.d, device=dev, generator=g) /
                             math.sqrt(w.d)).to(torch.bfloat16)
        ws_bytes = max(bsa.workspace_size(self.L, bsa.OP_SELECT, self.P.n_max),
                       bsa.workspace_size(self.L, bsa.OP_DECODE, self.P.n_max))
        self.ws = [torch.empty(ws_bytes, dtype=torch.uint8, device=dev) for _ in range(layers)]
        self.idx = [torch.empty(w.B, w.Hkv, self.P.n_max, dtype=torch.int32, device=dev)
                    for _ in range(layers)]
        self.cnt = [torch.empty(w.B, w.Hkv, dtype=torch.int32, device=dev) for _ in range(layers)]
        self.o = [torch.empty(w.B, w.Hq, w.d, dtype=self.tdt, device=dev) for _ in range(layers)]
        self.lse = [torch.empty(w.B, w.Hq, dtype=torch.float32, device=dev) for _ in range(layers)]
        self.scale = 1.0 / math.sqrt(w.d)

    def make_inputs(self, nsteps, seed):
        """Fresh queries and appended tokens for nsteps steps x L layers."""
        import torch
        w = self.w
        g = torch.Generator(device=self.dev)
        g.manual_seed(seed)
        q = torch.randn(nsteps, self.layers, w.B, w.Hq, w.d, device=self.dev,
                        generator=g).to(self.tdt)
        kn = torch.randn(nsteps, self.layers, w.B, w.Hkv, 1, w.d, device=self.dev,
                         generator=g).to(self.tdt)
        vn = torch.randn(nsteps, self.layers, w.B, w.Hkv, 1, w.d, device=self.dev,
                         generator=g).to(self.tdt)
        return q, kn, vn

    def step(self, q, kn, vn, i, ev=None):
        bsa = self.bsa
        self.seq_lens.add_(1)
        for l in range(self.layers):
            c = self.caches[l]
            bsa.build_block_desc(self.L, c, kn[i, l], vn[i, l], 1)
            bsa.select_blocks(self.L, c, q[i, l], self.P, self.idx[l], self.cnt[l], self.ws[l])
            if ev is not None:
                ev[l][0].record()
            bsa.sparse_decode(self.L, c, q[i, l], self.idx[l], self.cnt[l], self.P.n_max,
                              self.scale, self.o[l], self.lse[l], self.ws[l])
            if ev is not None:
                ev[l][1].record()
        self.steps_done += 1

    def lengths(self):
        return [t + self.steps_done for t in self.T0]

    def kept_counts(self):
        """Per-sequence kept blocks at the current lengths (host formula)."""
        return [self.bsa.block_count(self.P, (T + self.w.block - 1) // self.w.block,
                                     self.w.block) for T in self.lengths()]


def measure(run, steps, warmup, seed=1):
    import torch
    qi, ki, vi = run.make_inputs(warmup + steps, seed)
    for i in range(warmup):
        run.step(qi, ki, vi, i)
    torch.cuda.synchronize()
    eb_desc = eb_kv = 0
    # bytes of the steps about to be timed (lengths advance by one per step)
    for k in range(steps):
        lens = [t + 1 + k for t in run.lengths()]
        ns = [run.bsa.block_count(run.P, (T + run.w.block - 1) // run.w.block, run.w.block)
              for T in lens]
        a, b = effective_bytes(run.w, lens, ns, run.w.d, 2 if run.w.dtype == "bf16" else 4)
        eb_desc += a
        eb_kv += b
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(run.layers)] for _ in range(steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        run.step(qi, ki, vi, warmup + i, ev=ev[i])
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    dec_ms = [e0.elapsed_time(e1) for row in ev for (e0, e1) in row]
    nl = steps * run.layers
    # eb_* are summed over the timed steps for ONE layer (every layer has the
    # same shape), so per step-layer they are divided by `steps` only
    return {
        "ms_per_step": total_ms / steps,
        "us_per_step_layer": total_ms * 1000.0 / nl,
        "eff_bytes_per_step_layer": (eb_desc + eb_kv) / steps,
        "desc_bytes_per_step_layer": eb_desc / steps,
        "kv_bytes_per_step_layer": eb_kv / steps,
        "decode_us_avg": 1000.0 * sum(dec_ms) / len(dec_ms),
    }


def cpu_baseline(run, steps):
    """The oracle, as it stands, on a bounded sample: the first `steps`
    decode steps of layer 0, sequence 0, every KV-head group, one thread
    per group (ctypes releases the GIL)."""
    import concurrent.futures as cf

    import numpy as np
    import torch

    import oracle as O
    w = run.w
    K, V = run.host  # [Hkv, T0, d]
    G = w.G
    T0 = run.T0[0]
    rng = np.random.Generator(np.random.PCG64(77))
    qs = rng.standard_normal((steps, w.Hq, w.d)).astype(np.float32)
    kn = rng.standard_normal((steps, w.Hkv, w.d)).astype(np.float32)
    vn = rng.standard_normal((steps, w.Hkv, w.d)).astype(np.float32)
    Kx = np.concatenate([K, kn.transpose(1, 0, 2)], axis=1)
    Vx = np.concatenate([V, vn.transpose(1, 0, 2)], axis=1)
    Wg = run.P.gate_w.float().cpu().numpy() if run.P.gate_w is not None else None
    kind = w.desc_kind
    cores = min(w.Hkv, os.cpu_count() or 1, 16)

    def one(step, h):
        T = T0 + step + 1
        O.decode_group(qs[step, h * G:(h + 1) * G], Kx[h, :T], Vx[h, :T], w.block, kind, W=Wg,
                       budget_tokens=w.budget_tokens, sparsity_bp=run.P.sparsity_bp,
                       n_local=w.n_local, n_min=w.n_min)

    O.lib()
    t = time.time()
    with cf.ThreadPoolExecutor(max_workers=cores) as ex:
        for step in range(steps):
            list(ex.map(lambda h: one(step, h), range(w.Hkv)))
    el = time.time() - t
    # one layer-step of sequence 0; scale to the batch
    us_per_layer_step = el * 1e6 / steps * w.B
    lens = [t + 1 for t in run.T0]
    ns = [run.bsa.block_count(run.P, (T + w.block - 1) // w.block, w.block) for T in lens]
    a, b = effective_bytes(w, lens, ns, w.d, 2 if w.dtype == "bf16" else 4)
    return {"value": round((a + b) / (us_per_layer_step * 1e-6) / 1e9, 4), "unit": "GB/s",
            "us_per_step_layer": round(us_per_layer_step, 1), "cores": cores, "kind": "oracle",
            "sample": f"{steps} decode steps of layer 0, sequence 0, all {w.Hkv} KV-head groups "
                      f"at {T0}+ tokens (fp64 scalar C, {cores} threads, one group each); "
                      f"scaled by the batch size {w.B}",
            "seconds": round(el, 2)}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; multi-GPU sharding is a "
                                   "design note, not an implementation", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import workloads as W
    dev = torch.device("cuda:0")
    w = W.get(args.workload)
    bp = args.sparsity_bp if args.sparsity_bp is not None else w.sparsity_bp
    t0 = time.time()
    run = Run(w, args.layers, bp, dev, keep_host_layer0=not args.no_cpu_baseline)
    print(f"# setup {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    m = measure(run, args.steps, args.warmup)
    print(f"# timed: {m}", file=sys.stderr, flush=True)
    value = m["eff_bytes_per_step_layer"] / (m["us_per_step_layer"] * 1e-6) / 1e9
    dec_achieved = m["kv_bytes_per_step_layer"] / (m["decode_us_avg"] * 1e-6) / 1e9
    out = {
        "metric": "sparse decode us/step/layer + effective HBM GB/s (% of peak) at 64K-512K ctx",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["ms_per_step"], 4),
        "us_per_step_layer": round(m["us_per_step_layer"], 2),
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; caches generated on the device)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d,
                   "context": list(w.T0), "block": w.block, "sparsity_bp": bp,
                   "budget_tokens": w.budget_tokens, "n_local": w.n_local, "n_min": w.n_min,
                   "descriptor": "minmax" if w.desc_kind == 0 else "meanpool+gate",
                   "layers": args.layers, "parallelism": "none (1 GPU)"},
        "bytes": {"effective_per_step_layer": int(m["eff_bytes_per_step_layer"]),
                  "descriptor_per_step_layer": int(m["desc_bytes_per_step_layer"]),
                  "kept_kv_per_step_layer": int(m["kv_bytes_per_step_layer"])},
        "roofline": {"kernel": "sparse_decode (split-K decode + log-sum-exp merge)",
                     "bound": "hbm", "achieved": round(dec_achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dec_achieved / HBM_PEAK_GBS, 4),
                     "avg_launch_us": round(m["decode_us_avg"], 3), "traffic": None},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(run, args.cpu_steps)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark: block-sparse attention decode on one MI355X.

One step = the decode hot path for one generated token of every sequence,
run for L distinct layer caches (default 8, so that the kept-block working
set cannot stay resident in the 256 MB last-level cache):
  seq_lens += 1                          (shared by the layers)
  per layer: bsa_append_select_decode, which is
             bsa_append_select     (append the new k, v and update the
                                   descriptors = bsa_build_block_desc, then
                                   score every non-local block and keep the
                                   top-n = bsa_select_blocks; the append rides
                                   in the scoring launch)
             + bsa_sparse_decode   (split-K attention over the kept blocks,
                                    log-sum-exp merge) in one call; for rows
                                    of at most 8192 candidate blocks the top-n
                                    runs in the decode launch
             bsa_rectify_chunk     (every f steps, workloads with rectification)
  (--step-form separate times the two calls instead).
Queries, appended tokens and re-encoded keys/values are fresh per step and
seeded; caches are generated on the device from the workload recipe.

Timing, per workload: W untimed warm-up steps, then
  (1) K steps launched eagerly, every decode (and rectify) call bracketed by
      its own HIP events on the stream the library runs on (torch's current
      stream) -> the decode kernel's average launch duration for the roofline;
  (2) the same K steps captured once into a HIP graph, replayed once untimed,
      then replayed between two events after a device synchronize -> the
      headline step time (serving engines replay decode steps as graphs).
value = effective HBM GB/s of the graph-timed step:
  effective bytes / step / layer = descriptor bytes of every block
  + K and V bytes of every kept token (+ the rectify pass's full-cache read,
  amortised, where the workload rectifies).
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix, published
METRIC = "sparse decode us/step/layer + effective HBM GB/s (% of peak) at 64K-512K ctx"


# HBM traffic of one bsa_sparse_decode call, from the committed rocprofv3
# counter runs (FETCH_SIZE, WRITE_SIZE, calibrated on a plain copy); reported
# only while the decode sources are the ones the counters were taken on.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sparse_decode_long_512k_p90_traffic.md")
TRAFFIC_SOURCES = ("block_sparse_attention_build_amd/csrc/decode.hip",
                   "block_sparse_attention_build_amd/csrc/bsa_device.h")


def code_only(src):
    """Source text without // comments and blank lines (comment edits do not
    change the kernel the counters were taken on)."""
    lines = (re.sub(r"//.*$", "", ln).rstrip() for ln in src.splitlines())
    return "\n".join(ln for ln in lines if ln).encode()


def measured_traffic(workload, bp):
    if workload != "long_512k" or bp != 9000:
        return None
    try:
        txt = open(TRAFFIC_FILE).read()
        h = hashlib.sha256()
        for f in TRAFFIC_SOURCES:
            h.update(code_only(open(os.path.join(ROOT, f)).read()))
    except OSError:
        return None
    t = re.search(r"traffic_bytes_per_launch:\s*(\d+)", txt)
    src = re.search(r"sources sha256[^:]*:\s*([0-9a-f]{64})", txt)
    if not t or not src or src.group(1) != h.hexdigest():
        return None
    return int(t.group(1))


def read_ceiling(dev):
    """The device's streaming-read rate: the best over a few grid sizes and
    three access modes (grid-stride plain loads, grid-stride nontemporal
    loads, one contiguous share per workgroup with nontemporal loads) of a
    16-byte streaming read over 4 GiB (libbsa_probe.so), timed with HIP
    events on the current stream.  A fourth mode, the decode's pattern
    (scattered 16 KiB chunks, two per wave in flight), is reported beside it
    in by_mode_GBps but does not set the ceiling."""
    import ctypes

    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "block_sparse_attention_build_amd", "libbsa_probe.so"))
    lib.bsa_probe_read_mode.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_void_p]
    lib.bsa_probe_read_mode.restype = ctypes.c_int
    nbytes = 4 << 30
    cases = [(0, g) for g in (8192, 16384, 32768, 65536)] + \
            [(1, g) for g in (8192, 32768)] + [(2, g) for g in (256, 512, 1024, 2048)] + \
            [(3, g) for g in (256, 512, 1024)]
    names = {0: "grid-stride plain loads", 1: "grid-stride nontemporal loads",
             2: "contiguous share per workgroup, nontemporal loads",
             3: "scattered 16 KiB chunks, nontemporal loads (the decode's pattern)"}
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.empty(65536 * 256 * 16, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best, best_case, by_mode = 0.0, None, {}
    for mode, g in cases:
        for _ in range(3):
            e0.record()
            rc = lib.bsa_probe_read_mode(buf.data_ptr(), nbytes, sink.data_ptr(), g, mode, stream.cuda_stream)
            e1.record()
            torch.cuda.synchronize()
            if rc != 0:
                raise RuntimeError(f"bsa_probe_read_mode failed ({rc})")
            gbps = nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
            by_mode[names[mode]] = max(by_mode.get(names[mode], 0.0), round(gbps, 1))
            if mode != 3 and gbps > best:
                best, best_case = gbps, (mode, g)
    del buf, sink
    torch.cuda.empty_cache()
    return {"GBps": round(best, 1), "workgroups": best_case[1], "mode": names[best_case[0]],
            "by_mode_GBps": by_mode,
            "probe": "streaming read of 4 GiB, 16-byte loads, best of three access modes and "
                     "several grid sizes x 3 (libbsa_probe.so)"}


def pattern_read(dev, nbytes, copies=8, reps=4):
    """The read rate of the decode's access pattern at the decode's size:
    `copies` distinct buffers of nbytes (rounded up to 16 KiB; more than the
    last-level cache together) each read once as scattered 16 KiB chunks
    (libbsa_probe.so mode 3, 512 workgroups of 256 threads), captured into a
    HIP graph and replayed back to back like the decode calls of the
    benchmark's layers, so ramp-up and tail costs are included."""
    import ctypes

    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "block_sparse_attention_build_amd", "libbsa_probe.so"))
    lib.bsa_probe_read_mode.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_void_p]
    lib.bsa_probe_read_mode.restype = ctypes.c_int
    chunk = 16 << 10
    nb = (int(nbytes) + chunk - 1) // chunk * chunk
    wgs = 512
    bufs = [torch.empty(nb, dtype=torch.uint8, device=dev) for _ in range(copies)]
    sink = torch.empty(wgs * 256 * 16, dtype=torch.uint8, device=dev)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        s = torch.cuda.current_stream().cuda_stream
        for _ in range(reps):
            for b in bufs:
                if lib.bsa_probe_read_mode(b.data_ptr(), nb, sink.data_ptr(), wgs, 3, s) != 0:
                    raise RuntimeError("bsa_probe_read_mode failed")
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = float("inf")
    for _ in range(3):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1000 / (reps * copies))
    g.reset()
    del bufs, sink
    torch.cuda.empty_cache()
    return {"bytes_per_read": nb, "us_per_read": round(best, 3), "GBps": round(nb / best / 1e3, 1),
            "probe": f"scattered 16 KiB chunks, 2 per wave in flight, {wgs} workgroups of 256 threads; "
                     f"{copies} buffers read in turn, {reps} rounds, graph replay, best of 3"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=32)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="long_512k")
    ap.add_argument("--sparsity-bp", type=int, default=None)
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-steps", type=int, default=120)
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the other workloads (sparsity sweep, 32K, batched, ReSA loop)")
    ap.add_argument("--gate-tau", type=float, default=None,
                    help="also time the headline workload with the log-gate bias "
                         "(select writes it, bsa_sparse_decode_gated adds it) at this tau")
    ap.add_argument("--no-resa-sweep", action="store_true",
                    help="skip the ragged ReSA loop over f in {16,32,64,128} x p in "
                         "{0.9,0.95,0.98} (bytes against 1/b + (1-p) + 1/f)")
    ap.add_argument("--sweep-steps", type=int, default=0,
                    help="timed steps per sweep point (0: 2f, two rectifies)")
    ap.add_argument("--step-form", choices=["one_call", "separate"], default="one_call",
                    help="the timed step as one bsa_append_select_decode call per layer, or as "
                         "bsa_append_select + bsa_sparse_decode")
    ap.add_argument("--rectify-f", type=int, default=None,
                    help="rectify interval of a rectifying --workload (default: the workload's)")
    return ap.parse_args()


def kv_bytes(w, T, n):
    """Descriptor and kept-K/V bytes of one (sequence, all KV heads) at
    length T with n kept blocks (the last, always kept, holds T-(NB-1)*b)."""
    b, d = w.block, w.d
    es = 2 if w.dtype == "bf16" else 4
    NB = (T + b - 1) // b
    desc_per_block = 2 * d * es if w.desc_kind == 0 else d * 4
    tokens = n * b - (NB * b - T)
    return w.Hkv * NB * desc_per_block, w.Hkv * tokens * 2 * d * es


def bench_layout(w, sparsities=None, gate=None):
    """The cache layout and selection parameters the benchmark launches with
    (capacity = the longest context + 4096 tokens of decode headroom; idx
    rows sized for the largest kept count the capacity allows).  Returns
    (layout, {sparsity_bp: params})."""
    import block_sparse_attention_build_amd as bsa
    cap_tokens = max(w.T0) + 4096
    max_blocks = (cap_tokens + w.block - 1) // w.block
    kv = bsa.DTYPE_BF16 if w.dtype == "bf16" else bsa.DTYPE_F32
    L = bsa.Layout(w.B, w.Hq, w.Hkv, w.d, w.block, max_blocks, kv, w.desc_kind)
    params = {}
    for bp in (sparsities or [w.sparsity_bp]):
        P = bsa.SelectParams(budget_tokens=w.budget_tokens, sparsity_bp=bp, n_local=w.n_local,
                             n_min=w.n_min, gate_w=gate)
        P.n_max = bsa.block_count(P, max_blocks, w.block)
        params[bp] = P
    return L, params


class Run:
    """L layer caches of one workload, ready for decode steps."""

    def __init__(self, w, layers, dev, keep_host_layer0=False, sparsities=None):
        import torch
        import block_sparse_attention_build_amd as bsa
        import workloads as W
        self.w, self.layers, self.dev, self.bsa = w, layers, dev, bsa
        self.T0 = list(w.T0)
        self.steps_done = 0
        self.tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        gate = None
        if w.desc_kind == W.DESC_MEANPOOL:
            g = torch.Generator(device=dev)
            g.manual_seed(w.seed(0) + 7)
            gate = (torch.randn(w.d, w.d, device=dev, generator=g) / math.sqrt(w.d)).to(torch.bfloat16)
        sps = sparsities or [w.sparsity_bp]
        self.L, self.params = bench_layout(w, sps, gate)
        max_blocks = self.L.max_blocks
        kv = self.L.kv_dtype
        self.P = self.params[sps[0]]
        n_max_all = max(P.n_max for P in self.params.values())
        self.seq_lens = torch.zeros(w.B, dtype=torch.int32, device=dev)
        self.caches, self.host = [], None
        for l in range(layers):
            c = bsa.allocate_cache(self.L, device=dev)
            c.seq_lens = self.seq_lens
            for s in range(w.B):
                K, V, _ = W.make_device_kv(w, l, s, self.T0[s], dev)
                L1 = bsa.Layout(1, w.Hq, w.Hkv, w.d, w.block, max_blocks, kv, w.desc_kind)
                c1 = bsa.Cache(c.k_pool, c.v_pool, c.page_table[s:s + 1],
                               self.seq_lens[s:s + 1], c.desc[s:s + 1])
                self.seq_lens[s] = self.T0[s]
                bsa.build_block_desc(L1, c1, K[None], V[None], self.T0[s])
                if keep_host_layer0 and l == 0 and s == 0:
                    self.host = (K.float().cpu().numpy(), V.float().cpu().numpy())
                del K, V
            self.caches.append(c)
        torch.cuda.synchronize()
        ws_bytes = max([bsa.workspace_size(self.L, bsa.OP_STEP, P.n_max) for P in self.params.values()] +
                       [bsa.workspace_size(self.L, bsa.OP_DECODE, P.n_max) for P in self.params.values()])
        self.f = w.rectify_f
        if self.f:
            ws_bytes = max(ws_bytes, bsa.workspace_size(self.L, bsa.OP_RECTIFY, self.f))
        self.ws = [torch.empty(ws_bytes, dtype=torch.uint8, device=dev) for _ in range(layers)]
        self.idx = [torch.empty(w.B, w.Hkv, n_max_all, dtype=torch.int32, device=dev)
                    for _ in range(layers)]
        self.cnt = [torch.empty(w.B, w.Hkv, dtype=torch.int32, device=dev) for _ in range(layers)]
        self.o = [torch.empty(w.B, w.Hq, w.d, dtype=self.tdt, device=dev) for _ in range(layers)]
        self.lse = [torch.empty(w.B, w.Hq, dtype=torch.float32, device=dev) for _ in range(layers)]
        self.gate_tau = None  # set to a float to run the gated step
        self.one_call = True  # timed steps: bsa_append_select_decode (False: the two calls)
        self.gbias = [torch.zeros(w.B, w.Hkv, n_max_all, dtype=torch.float32, device=dev)
                      for _ in range(layers)]
        if self.f:
            self.o_r = [torch.empty(w.B, w.Hq, self.f, w.d, dtype=self.tdt, device=dev)
                        for _ in range(layers)]
            self.lse_r = [torch.empty(w.B, w.Hq, self.f, dtype=torch.float32, device=dev)
                          for _ in range(layers)]
        self.scale = 1.0 / math.sqrt(w.d)

    def make_inputs(self, nsteps, seed):
        """Fresh queries, appended tokens and (for rectifying workloads) the
        re-encoded chunk, for nsteps steps x L layers."""
        import torch
        w, L = self.w, self.layers
        g = torch.Generator(device=self.dev)
        g.manual_seed(seed)
        inp = {"q": torch.randn(nsteps, L, w.B, w.Hq, w.d, device=self.dev, generator=g).to(self.tdt),
               "kn": torch.randn(nsteps, L, w.B, w.Hkv, 1, w.d, device=self.dev, generator=g).to(self.tdt),
               "vn": torch.randn(nsteps, L, w.B, w.Hkv, 1, w.d, device=self.dev, generator=g).to(self.tdt)}
        if self.f:
            nr = nsteps // self.f + 1
            inp["qr"] = torch.randn(nr, L, w.B, w.Hq, self.f, w.d, device=self.dev, generator=g).to(self.tdt)
            inp["kr"] = torch.randn(nr, L, w.B, w.Hkv, self.f, w.d, device=self.dev, generator=g).to(self.tdt)
            inp["vr"] = torch.randn(nr, L, w.B, w.Hkv, self.f, w.d, device=self.dev, generator=g).to(self.tdt)
        return inp

    def step(self, inp, i, ev=None, ev_r=None):
        """Launch one decode step (all layers).  Returns True if it also
        rectified."""
        bsa, P = self.bsa, self.P
        self.seq_lens.add_(1)
        self.steps_done += 1
        rect = bool(self.f) and self.steps_done % self.f == 0
        for l in range(self.layers):
            c = self.caches[l]
            # append + select (the append shares the scoring launch); idx rows
            # are n_max long (the buffer fits the largest n_max of the sweep)
            gated = self.gate_tau is not None
            P.gate_tau = self.gate_tau if gated else 0.0
            P.gate_bias = self.gbias[l] if gated else None
            if self.one_call and ev is None:
                # the whole step in one call (the eager pass below keeps the
                # two calls, so that events can bracket the decode call)
                bsa.append_select_decode(self.L, c, inp["kn"][i, l], inp["vn"][i, l],
                                         inp["q"][i, l], P, self.idx[l], self.cnt[l], self.scale,
                                         self.o[l], self.lse[l], self.ws[l])
            else:
                bsa.append_select(self.L, c, inp["kn"][i, l], inp["vn"][i, l], inp["q"][i, l], P,
                                  self.idx[l], self.cnt[l], self.ws[l])
                if ev is not None:
                    ev[l][0].record()
                self.decode_call(l, inp["q"][i, l])
                if ev is not None:
                    ev[l][1].record()
            if rect:
                r = i // self.f
                if ev_r is not None:
                    ev_r[l][0].record()
                bsa.rectify_chunk(self.L, c, inp["qr"][r, l], inp["kr"][r, l], inp["vr"][r, l],
                                  self.f, self.scale, self.o_r[l], self.lse_r[l], self.ws[l])
                if ev_r is not None:
                    ev_r[l][1].record()
        return rect

    def decode_call(self, l, q):
        """bsa_sparse_decode (gated when the run has a gate tau) of layer l on
        its current selection."""
        bsa, P = self.bsa, self.P
        if self.gate_tau is not None:
            bsa.sparse_decode_gated(self.L, self.caches[l], q, self.idx[l], self.cnt[l],
                                    self.gbias[l], P.n_max, self.scale, self.o[l], self.lse[l],
                                    self.ws[l])
        else:
            bsa.sparse_decode(self.L, self.caches[l], q, self.idx[l], self.cnt[l], P.n_max,
                              self.scale, self.o[l], self.lse[l], self.ws[l])

    def lengths(self):
        return [t + self.steps_done for t in self.T0]


def step_bytes(run, lens):
    """Effective bytes of one decode step of one layer at lengths `lens`."""
    w, P = run.w, run.P
    desc = kv = 0
    for T in lens:
        n = run.bsa.block_count(P, (T + w.block - 1) // w.block, w.block)
        a, b = kv_bytes(w, T, n)
        desc += a
        kv += b
    return desc, kv


def expected_counts(run, lens):
    """Kept blocks of every sequence at lengths lens by the closed form
    (bsa_block_count): the count the byte accounting assumes, which every KV
    head's selection must report."""
    b = run.w.block
    return [run.bsa.block_count(run.P, (T + b - 1) // b, b) for T in lens]


def check_counts(cnts, expected):
    """cnts: per layer, the [B, Hkv] kept counts copied back from the device
    after the timed steps; raises unless every group reports its sequence's
    expected count.  Returns the number of groups checked."""
    import numpy as np
    n = 0
    for layer, c in enumerate(cnts):
        c = np.asarray(c)
        for s, e in enumerate(expected):
            if not np.all(c[s] == e):
                raise RuntimeError(f"layer {layer}, sequence {s}: kept counts {c[s].tolist()}, "
                                   f"the closed form gives {e}")
            n += c.shape[1]
    return n


def rectify_cost(run, lens):
    """Bytes (full-cache K and V read) and flops of one rectify call, one layer."""
    w = run.w
    es = 2 if w.dtype == "bf16" else 4
    f = run.f
    byts = sum(T * w.Hkv * 2 * w.d * es for T in lens)
    # QK and PV: 4*d flops per (query row, attended token); row i of a head
    # attends to T-f+i+1 tokens
    flops = sum(4 * w.d * w.Hq * (f * (T - f) + f * (f + 1) // 2) for T in lens)
    return byts, flops


def measure(run, steps, warmup, seed=1):
    """Eager pass with per-call events, then the graph-replayed headline pass."""
    import torch
    inp = run.make_inputs(warmup + 3 * steps, seed)
    for i in range(warmup):
        run.step(inp, i)
    torch.cuda.synchronize()

    def account(first):
        d = k = rb = rf = 0
        n_rect = 0
        for s in range(steps):
            lens = [t + first + s + 1 for t in run.T0]
            a, b = step_bytes(run, lens)
            d, k = d + a, k + b
            if run.f and (run.steps_done + s + 1) % run.f == 0:
                x, y = rectify_cost(run, lens)
                rb, rf, n_rect = rb + x, rf + y, n_rect + 1
        return d, k, rb, rf, n_rect

    # (1) eager, per-call events
    d1, k1, rb1, rf1, nr1 = account(run.steps_done)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(run.layers)] for _ in range(steps)]
    ev_r = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(run.layers)] for _ in range(steps)]
    rect_steps = []
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for s in range(steps):
        if run.step(inp, warmup + s, ev=ev[s], ev_r=ev_r[s]):
            rect_steps.append(s)
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1)
    dec_us = [1000 * a.elapsed_time(b) for row in ev for (a, b) in row]
    rect_us = [1000 * a.elapsed_time(b) for s in rect_steps for (a, b) in ev_r[s]]

    # (2) graph: capture K steps, replay once untimed, once timed
    base = warmup + steps
    g = torch.cuda.CUDAGraph()
    saved = run.steps_done
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for s in range(steps):
            run.step(inp, base + s)
    run.steps_done = saved          # capture launched nothing
    g.replay()
    run.steps_done += steps
    torch.cuda.synchronize()
    d2, k2, rb2, rf2, nr2 = account(run.steps_done)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    run.steps_done += steps
    graph_ms = e0.elapsed_time(e1)
    # the selection the timed steps left behind: every layer's counts equal
    # the closed form the byte accounting uses
    counts_checked = check_counts([run.cnt[l].cpu().numpy() for l in range(run.layers)],
                                  expected_counts(run, run.lengths()))
    # (3) the decode call alone: every layer's call on its current selection,
    # captured into a graph and replayed between two events, so the per-call
    # time is the GPU's own (the eager pass above is host-bound for the short
    # workloads, and its per-call events then include launch gaps).  The
    # decode only reads the cache, so replays change nothing.
    gd = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(gd):
        for s in range(steps):
            for l in range(run.layers):
                run.decode_call(l, inp["q"][base + s, l])
    gd.replay()
    torch.cuda.synchronize()
    e0.record()
    gd.replay()
    e1.record()
    torch.cuda.synchronize()
    dec_graph_us = e0.elapsed_time(e1) * 1000 / (steps * run.layers)
    gd.reset()
    L = run.layers
    out = {
        "graph": {"ms_per_step": graph_ms / steps, "us_per_step_layer": graph_ms * 1000 / (steps * L),
                  "eff_bytes_per_step_layer": (d2 + k2 + rb2) / steps,
                  "desc_bytes": d2 / steps, "kv_bytes": k2 / steps,
                  "rectify_bytes": rb2 / steps},
        "eager": {"ms_per_step": eager_ms / steps, "us_per_step_layer": eager_ms * 1000 / (steps * L),
                  "eff_bytes_per_step_layer": (d1 + k1 + rb1) / steps},
        "decode_us_avg": dec_graph_us,
        "decode_us_eager_events": sum(dec_us) / len(dec_us),
        "decode_kv_bytes_per_call": k1 / steps,
        "counts_checked": counts_checked,
    }
    if rect_us:
        # The eager per-call events above include the host's launch gaps
        # (the eager loop is host-bound); the rectify call time is taken from
        # back-to-back calls instead, after the step measurements (the calls
        # rewrite the last f tokens of each cache).
        L = run.layers
        r = (warmup + steps) // run.f
        torch.cuda.synchronize()
        e0.record()
        for k in range(2 * L):
            l = k % L
            run.bsa.rectify_chunk(run.L, run.caches[l], inp["qr"][r, l], inp["kr"][r, l],
                                  inp["vr"][r, l], run.f, run.scale, run.o_r[l], run.lse_r[l],
                                  run.ws[l])
        e1.record()
        torch.cuda.synchronize()
        rect_us = [1000 * e0.elapsed_time(e1) / (2 * L)] * (2 * L)
        out["rectify"] = {"us_avg": sum(rect_us) / len(rect_us), "calls": len(rect_us),
                          "bytes_per_call": rb1 / max(nr1, 1), "flops_per_call": rf1 / max(nr1, 1)}
    g.reset()
    return out


def summarize(w, bp, layers, m):
    gm = m["graph"]
    value = gm["eff_bytes_per_step_layer"] / (gm["us_per_step_layer"] * 1e-6) / 1e9
    s = {"workload": w.name, "sparsity_bp": bp, "budget_tokens": w.budget_tokens,
         "us_per_step_layer": round(gm["us_per_step_layer"], 2),
         "effective_GBps": round(value, 1), "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
         "eager_us_per_step_layer": round(m["eager"]["us_per_step_layer"], 2),
         "decode_kernel_us": round(m["decode_us_avg"], 2),
         "decode_GBps": round(m["decode_kv_bytes_per_call"] / (m["decode_us_avg"] * 1e-6) / 1e9, 1),
         "bytes_per_step_layer": int(gm["eff_bytes_per_step_layer"]),
         "kept_counts_checked": m["counts_checked"]}
    if not w.rectify_f:
        # the step's time beyond the decode call alone: append, scoring and
        # top-n (in the one-call step, whatever the in-launch selection adds)
        sel = gm["us_per_step_layer"] - m["decode_us_avg"]
        s["select_us"] = round(sel, 2)
        s["select_share"] = round(sel / gm["us_per_step_layer"], 3)
    if "rectify" in m:
        r = m["rectify"]
        s["rectify"] = {"us_per_call": round(r["us_avg"], 1),
                        "GBps": round(r["bytes_per_call"] / (r["us_avg"] * 1e-6) / 1e9, 1),
                        "TFLOPs": round(r["flops_per_call"] / (r["us_avg"] * 1e-6) / 1e12, 1),
                        "mfma_util_pct_of_bf16_peak": round(
                            100 * r["flops_per_call"] / (r["us_avg"] * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 2),
                        "every_f_steps": w.rectify_f}
    return value, s


def cpu_baseline(run, steps):
    """The oracle, as it stands, on a bounded sample: `steps` decode steps of
    layer 0, sequence 0, every KV-head group, one thread per group (ctypes
    releases the GIL), scaled to one layer-step of the batch."""
    import concurrent.futures as cf

    import numpy as np

    import oracle as O
    w = run.w
    K, V = run.host  # [Hkv, T0, d]
    G, T0 = w.G, run.T0[0]
    rng = np.random.Generator(np.random.PCG64(77))
    qs = rng.standard_normal((steps, w.Hq, w.d)).astype(np.float32)
    kn = rng.standard_normal((steps, w.Hkv, w.d)).astype(np.float32)
    vn = rng.standard_normal((steps, w.Hkv, w.d)).astype(np.float32)
    Kx = np.concatenate([K, kn.transpose(1, 0, 2)], axis=1)
    Vx = np.concatenate([V, vn.transpose(1, 0, 2)], axis=1)
    Wg = run.P.gate_w.float().cpu().numpy() if run.P.gate_w is not None else None
    cores = min(w.Hkv, os.cpu_count() or 1, 16)

    def one(step, h):
        T = T0 + step + 1
        O.decode_group(qs[step, h * G:(h + 1) * G], Kx[h, :T], Vx[h, :T], w.block, w.desc_kind,
                       W=Wg, budget_tokens=w.budget_tokens, sparsity_bp=run.P.sparsity_bp,
                       n_local=w.n_local, n_min=w.n_min)

    O.lib()
    t = time.time()
    with cf.ThreadPoolExecutor(max_workers=cores) as ex:
        for step in range(steps):
            list(ex.map(lambda h: one(step, h), range(w.Hkv)))
    el = time.time() - t
    us = el * 1e6 / steps * w.B
    # the same work on one core, over an eighth of the steps
    steps1 = max(1, steps // 8)
    t = time.time()
    for step in range(steps1):
        for h in range(w.Hkv):
            one(step, h)
    el1 = time.time() - t
    us1 = el1 * 1e6 / steps1 * w.B
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    a, b = step_bytes(run, [t + 1 for t in run.T0])
    return {"value": round((a + b) / (us * 1e-6) / 1e9, 4), "unit": "GB/s",
            "us_per_step_layer": round(us, 1), "cores": cores, "kind": "oracle",
            "sample": f"{steps} decode steps of layer 0, sequence 0, all {w.Hkv} KV-head groups at "
                      f"{T0}+ tokens (fp64 scalar C oracle, one thread per group); "
                      f"scaled by the batch size {w.B}",
            "seconds": round(el, 2),
            "one_core": {"us_per_step_layer": round(us1, 1), "steps": steps1,
                         "seconds": round(el1, 2)},
            "cpu_model": model, "host_cpus": os.cpu_count()}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; sharding across GPUs is a "
                                   "design note, not an implementation", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import workloads as W
    dev = torch.device("cuda:0")
    w = W.get(args.workload) if args.rectify_f is None else \
        W.get(args.workload, rectify_f=args.rectify_f)
    sweep = [args.sparsity_bp] if args.sparsity_bp is not None else \
        ([w.sparsity_bp] + [b for b in w.sparsity_sweep if b != w.sparsity_bp])
    t0 = time.time()
    run = Run(w, args.layers, dev, keep_host_layer0=not args.no_cpu_baseline, sparsities=sweep)
    run.one_call = args.step_form == "one_call"
    print(f"# {w.name}: setup {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    results = []
    for bp in sweep:
        run.P = run.params[bp]
        m = measure(run, args.steps, args.warmup)
        results.append((bp, m))
        print(f"# {w.name} bp={bp}: {json.dumps(m)}", file=sys.stderr, flush=True)
    bp0, m0 = results[0]
    run.P = run.params[bp0]
    value, head = summarize(w, bp0, args.layers, m0)
    dec_gbps = m0["decode_kv_bytes_per_call"] / (m0["decode_us_avg"] * 1e-6) / 1e9
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m0["graph"]["ms_per_step"], 4),
        "us_per_step_layer": head["us_per_step_layer"],
        "pct_of_hbm_peak": head["pct_of_hbm_peak"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; caches generated on the device)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d,
                   "context": list(w.T0), "block": w.block, "sparsity_bp": bp0,
                   "budget_tokens": w.budget_tokens, "n_local": w.n_local, "n_min": w.n_min,
                   "descriptor": "minmax" if w.desc_kind == 0 else "meanpool+gate",
                   "layers": args.layers, "timing": "HIP graph replay of K steps",
                   "step_form": args.step_form,
                   "parallelism": "none (1 GPU)"},
        "bytes": {"effective_per_step_layer": head["bytes_per_step_layer"],
                  "descriptor_per_step_layer": int(m0["graph"]["desc_bytes"]),
                  "kept_kv_per_step_layer": int(m0["graph"]["kv_bytes"])},
        "roofline": {"kernel": "bsa_sparse_decode (decode_bf16_kernel + combine_kernel)",
                     "bound": "hbm", "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(dec_gbps / HBM_PEAK_GBS, 4),
                     "avg_launch_us": round(m0["decode_us_avg"], 3),
                     "launch_timing": "HIP events around a graph replay of the call alone "
                                      "(every layer, K steps) on the launch stream",
                     "eager_event_us": round(m0["decode_us_eager_events"], 3),
                     "algorithmic_bytes_per_launch": int(m0["decode_kv_bytes_per_call"]),
                     "traffic": measured_traffic(w.name, bp0),
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE x 2.0 + WRITE_SIZE)"},
        "eager_us_per_step_layer": head["eager_us_per_step_layer"],
        "workloads": [head] + [summarize(w, bp, args.layers, m)[1] for bp, m in results[1:]],
    }
    if args.gate_tau is not None:
        run.gate_tau = args.gate_tau
        mg = measure(run, args.steps, args.warmup, seed=2)
        run.gate_tau = None
        gh = summarize(w, bp0, args.layers, mg)[1]
        gh["gate_tau"] = args.gate_tau
        gh["decode_us_avg"] = round(mg["decode_us_avg"], 3)
        gh["note"] = "same step with the log-gate bias written by select and added by the decode"
        out["gated"] = gh
        print(f"# gated tau={args.gate_tau}: {json.dumps(mg)}", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(run, args.cpu_steps)
    del run
    torch.cuda.empty_cache()
    ceil = read_ceiling(dev)
    out["read_ceiling"] = ceil
    out["pct_of_read_ceiling"] = round(100.0 * out["value"] / ceil["GBps"], 2)
    out["roofline"]["frac_of_read_ceiling"] = round(out["roofline"]["achieved"] / ceil["GBps"], 4)
    # the same bytes read in the decode's pattern, at its size, back to back
    pat = pattern_read(dev, out["roofline"]["algorithmic_bytes_per_launch"])
    out["read_ceiling"]["decode_pattern_at_size"] = pat
    out["roofline"]["frac_of_pattern_read"] = round(out["roofline"]["achieved"] / pat["GBps"], 4)
    if not args.headline_only:
        for name in ["qwen3_4b_32k", "batched_64k_gate", "resa_ragged"]:
            wx = W.get(name)
            t0 = time.time()
            rx = Run(wx, args.layers, dev)
            rx.one_call = args.step_form == "one_call"
            mx = measure(rx, args.steps if not wx.rectify_f else max(args.steps, 2 * wx.rectify_f),
                         args.warmup)
            out["workloads"].append(summarize(wx, rx.P.sparsity_bp, args.layers, mx)[1])
            print(f"# {name}: {time.time() - t0:.1f}s {json.dumps(mx)}", file=sys.stderr, flush=True)
            del rx
            torch.cuda.empty_cache()
    if not args.no_resa_sweep and not args.headline_only:
        out["resa_sweep"] = resa_sweep(args, dev)
    print(json.dumps(out), flush=True)


def resa_sweep(args, dev):
    """The ragged ReSA loop over the rectify interval f and the sparsity p:
    amortised step time and bytes per step against the dense read of the
    whole cache, next to the cost model 1/b + (1 - p) + 1/f."""
    import torch

    import workloads as W
    rows = []
    for f in (16, 32, 64, 128):
        for bp in (9000, 9500, 9800):
            w = W.get("resa_ragged", rectify_f=f, sparsity_bp=bp)
            run = Run(w, args.layers, dev)
            m = measure(run, args.sweep_steps or 2 * f, args.warmup)
            gm = m["graph"]
            dense = sum(T * w.Hkv * 2 * w.d * 2 for T in w.T0)
            rows.append({"f": f, "sparsity_bp": bp,
                         "us_per_step_layer": round(gm["us_per_step_layer"], 2),
                         "bytes_per_step_layer": int(gm["eff_bytes_per_step_layer"]),
                         "bytes_over_dense": round(gm["eff_bytes_per_step_layer"] / dense, 4),
                         "model_1/b+(1-p)+1/f": round(1 / w.block + (10000 - bp) / 10000 + 1 / f, 4),
                         "effective_GBps": round(gm["eff_bytes_per_step_layer"] /
                                                 (gm["us_per_step_layer"] * 1e-6) / 1e9, 1),
                         "rectify_us_per_call": round(m["rectify"]["us_avg"], 1) if "rectify" in m else None})
            print(f"# resa sweep {rows[-1]}", file=sys.stderr, flush=True)
            del run
            torch.cuda.empty_cache()
    return rows


if __name__ == "__main__":
    main()

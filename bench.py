"""Throughput of Fibonacci-offset sparse attention, forward + backward, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one pass of the whole path over one batch: for each of the 16 layers of the paper's
model shape (B = 32, L = 1024, 8 query / 2 key-value heads, head dim 64, bfloat16 storage, W = 12,
Fibonacci base, linear stagger alpha_l = 0.5 + l/15), the forward call (RoPE'd keys, attention,
lse) and the backward call (dq, dk, dv). Both use one workspace: the backward reads the rotated
keys and the values the forward staged there and skips its own prep wherever the library reports
that this prep would write the same arrays. Each layer has its own input set in HBM (16 sets, more
than the 256 MB Infinity Cache holds), resident before timing starts. The same protocol is then
run once more at the 4x extrapolation shape (B = 8, L = 4096, coprime stagger) and reported under
"l4096".

Prints one JSON line on stdout. Progress goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import multiprocessing as mp
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, 8 TB/s
# HBM bytes per launch measured with FETCH_SIZE / WRITE_SIZE (calibrated on a plain copy), with the
# hash of the sources each kernel was built from: a figure is used only while the sources match
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_bytes_l1024_linear.json")
TRAFFIC_WORKLOAD = "l1024_linear_bf16"
FP16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix-core peak (the forward's products run there)
FWD_TARGET_FRAC = 0.60          # the forward attention's target: 60 % of peak HBM bandwidth
STREAM_BYTES = 1 << 30
LDS_PROBE_BYTES = 16 << 20          # streaming probe buffers (four times the Infinity Cache)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------------------------------------
# CPU baseline: the float64 oracle as it stands, on the host's cores, on a bounded sample.
# ------------------------------------------------------------------------------------------------

def _one_thread():
    # one thread per worker process: the pool's size is the core count
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)
    torch.set_num_threads(1)


def _oracle_unit(args):
    name, layer, b = args
    import numpy as np  # noqa: F401
    from oracle import fibattn_oracle as O
    w = workloads.WORKLOADS[name]
    q, k, v, do = workloads.draw(w, layer, B=b + 1, with_grad=True)
    q, k, v, do = [x[b:b + 1].double().numpy() for x in (q, k, v, do)]
    fn = {"fixed": O.alpha_fixed, "linear": O.alpha_linear, "coprime": O.alpha_coprime}[w.schedule]
    alpha = fn(layer, w.n_layers)
    base = O.FIB_BASE if w.base == "fib" else {1024: O.POW2_BASE_1024, 2048: O.POW2_BASE_2048}[workloads.pow2_max(w)]
    O.forward(q, k, v, alpha, w.W, base)
    O.backward(q, k, v, do, alpha, w.W, base)
    return 1


def cpu_share() -> int:
    """Host cores this job may use: the affinity mask, capped by OMP_NUM_THREADS where the host sets
    it (a GPU machine gives each GPU's jobs a fixed share of its cores and says so there)."""
    n = len(os.sched_getaffinity(0))
    try:
        return max(1, min(n, int(os.environ.get("OMP_NUM_THREADS", n))))
    except ValueError:
        return n


def cpu_baseline(name: str, budget_s: float = 15.0):
    w = workloads.WORKLOADS[name]
    workers = cpu_share()
    # (layer, repeat) units, each on batch element 0 of that layer's inputs: the oracle's cost does
    # not depend on the values, and a B = 1 draw keeps input generation out of the way; more units
    # than the budget lets finish, so that the budget sets the sample
    units = [(name, layer, 0) for _ in range(8 * w.B) for layer in range(w.n_layers)]
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    done = 0
    with ctx.Pool(workers, initializer=_one_thread) as pool:
        it = pool.imap_unordered(_oracle_unit, units)
        for _ in it:
            done += 1
            if time.perf_counter() - t0 > budget_s and done % workers == 0:
                break
        wall = time.perf_counter() - t0
        pool.terminate()
    qh = done * w.L * w.Hq
    # the rate of one single-threaded worker, on a few of the same units
    t1 = time.perf_counter()
    with ctx.Pool(1, initializer=_one_thread) as pool:
        n1 = len(pool.map(_oracle_unit, units[:4]))
    wall1 = time.perf_counter() - t1
    cpu = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                cpu = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": qh / wall, "unit": "queries*heads/s (fwd+bwd)", "cores": workers, "kind": "oracle",
        "value_1worker": n1 * w.L * w.Hq / wall1,
        "sample": f"{done} (layer, batch element 0) units of {name}, each a float64 forward + backward at "
                  f"B=1, L={w.L}, {wall:.1f} s wall on {workers} single-threaded worker processes ({cpu}, "
                  f"{platform.machine()}; {len(os.sched_getaffinity(0))} cores in the affinity mask, "
                  f"OMP_NUM_THREADS={os.environ.get('OMP_NUM_THREADS', 'unset')})",
    }


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None when it was taken
    on another workload or the kernel's sources have changed since."""
    if workload != TRAFFIC_WORKLOAD or not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        entry = json.load(f)["kernels"].get(kernel)
    if entry is None:
        return None
    paths = [os.path.join(ROOT, "fibonacci_offset_sparse_amd", "csrc", fn) for fn in entry["sources"]]
    return entry["bytes_per_launch"] if code_hash(paths) == entry["sources_sha256"] else None


def measured_limiter(kernel: str, workload: str):
    """What the committed counter summary names as the kernel's limiter (with its evidence), or
    "unknown" when it was taken on another workload or the kernel's sources have changed since."""
    path = os.path.join(ROOT, "profiles", "limiters_l1024_linear.json")
    if workload != TRAFFIC_WORKLOAD or not os.path.exists(path):
        return "unknown"
    with open(path) as f:
        entry = json.load(f)["kernels"].get(kernel)
    if entry is None:
        return "unknown"
    paths = [os.path.join(ROOT, "fibonacci_offset_sparse_amd", "csrc", fn) for fn in entry["sources"]]
    if code_hash(paths) != entry["sources_sha256"]:
        return "unknown"
    return {"limiter": entry["limiter"], "evidence": entry["evidence"]}


def code_hash(paths) -> str:
    """sha256 of the sources with // comments and blank lines left out, so that a comment edit
    does not retire a measurement of unchanged code."""
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(p) as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()


# ------------------------------------------------------------------------------------------------
# Streaming probe: what plain coalesced reads, writes and copies reach on this GPU's HBM
# ------------------------------------------------------------------------------------------------

def stream_probe(dev, reps: int = 10):
    """TB/s of the probe's patterns over 1 GiB buffers (libstreamprobe.so), timed with events on the
    current stream (the probe launches there)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "fibonacci_offset_sparse_amd", "libstreamprobe.so"))
    lib.streamprobe_launch.restype = ctypes.c_int
    lib.streamprobe_launch.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_int64, ctypes.c_void_p]
    lib.streamprobe_read_blocks.restype = ctypes.c_int64
    lib.streamprobe_read_blocks.argtypes = [ctypes.c_int64]
    a = torch.ones(STREAM_BYTES, dtype=torch.uint8, device=dev)
    b = torch.empty(STREAM_BYTES, dtype=torch.uint8, device=dev)
    sink = torch.empty(int(lib.streamprobe_read_blocks(STREAM_BYTES)), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    out = {}
    for name, pat, moved in (("read", 0, 1), ("write", 1, 1), ("write_nt", 2, 1), ("copy", 3, 2)):
        def launch():
            rc = lib.streamprobe_launch(pat, a.data_ptr(), b.data_ptr(), sink.data_ptr(), STREAM_BYTES,
                                        stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"stream probe launch failed ({rc})")
        for _ in range(3):
            launch()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            launch()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[f"{name}_TBps"] = moved * STREAM_BYTES / (ms * 1e-3) / 1e12
    # LDS staging from a buffer that stays on chip (the attention kernels' staging instruction and
    # grain), 16 MiB read 16 times per launch
    lib.streamprobe_lds_bytes.restype = ctypes.c_int64
    lib.streamprobe_lds_bytes.argtypes = [ctypes.c_int64]
    small = LDS_PROBE_BYTES
    moved = int(lib.streamprobe_lds_bytes(small))

    def launch_lds():
        rc = lib.streamprobe_launch(4, a.data_ptr(), b.data_ptr(), sink.data_ptr(), small, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"stream probe launch failed ({rc})")
    for _ in range(3):
        launch_lds()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        launch_lds()
    e1.record()
    torch.cuda.synchronize()
    out["lds_stage_TBps"] = moved / (e0.elapsed_time(e1) / reps * 1e-3) / 1e12
    out["what"] = ("1 GiB buffers, 16-byte coalesced accesses, one pass per launch (libstreamprobe.so); copy "
                   "counts bytes read plus bytes written; lds_stage: 1 KB buffer-to-LDS transfers (the "
                   "attention kernels' staging) from a 16 MiB buffer that stays on chip, read 16 times")
    del a, b, sink
    torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------------------------------------------
# GPU timing
# ------------------------------------------------------------------------------------------------

class Layers:
    """Per-layer inputs, outputs and shared workspaces for one workload, resident on the GPU."""

    def __init__(self, fa, w, dev, n_sets=None):
        self.fa, self.w, self.dev = fa, w, dev
        self.n_sets = w.n_layers if n_sets is None else n_sets
        if w.base == "fib":
            base = fa.fibattn_base_offsets(fa.BASE_FIB)
        else:
            base = fa.fibattn_base_offsets(fa.BASE_POW2, workloads.pow2_max(w))
        self.base = base
        code = {"fixed": fa.SCHEDULE_FIXED, "linear": fa.SCHEDULE_LINEAR, "coprime": fa.SCHEDULE_COPRIME}
        self.alphas, self.dadt = [], []
        thetas = workloads.draw_theta(w.n_layers).tolist() if w.schedule == "learned" else None
        for layer in range(w.n_layers):
            if thetas is not None:
                a, d = fa.fibattn_alpha_from_theta(thetas[layer])
            else:
                a, d = fa.fibattn_alpha_schedule(code[w.schedule], layer, w.n_layers), 0.0
            self.alphas.append(a)
            self.dadt.append(d)
        # d(alpha) only where every rung is interpolated (the learned schedule); static schedules
        # need no alpha gradient
        self.want_dalpha = []
        for a in self.alphas:
            kind = fa.fibattn_plan(a, w.W, base)[0]
            self.want_dalpha.append(w.schedule == "learned" and bool((kind == fa.INTERP).all()))
        self.inputs = []
        for layer in range(self.n_sets):
            q, k, v, do = workloads.draw(w, layer, with_grad=True)
            self.inputs.append(tuple(x.to(dev) for x in (q, k, v, do)))
            log(f"  inputs of layer {layer} resident")
        B, L, Hq, Hkv, D = w.B, w.L, w.Hq, w.Hkv, w.D
        self.o = [torch.empty(B, Hq, L, D, dtype=w.torch_dtype, device=dev) for _ in range(self.n_sets)]
        self.lse = [torch.empty(B, Hq, L, dtype=torch.float32, device=dev) for _ in range(self.n_sets)]
        self.dq = [torch.empty(B, Hq, L, D, dtype=w.torch_dtype, device=dev) for _ in range(self.n_sets)]
        self.dk = [torch.empty(B, Hkv, L, D, dtype=w.torch_dtype, device=dev) for _ in range(self.n_sets)]
        self.dv = [torch.empty(B, Hkv, L, D, dtype=w.torch_dtype, device=dev) for _ in range(self.n_sets)]
        self.dalpha = torch.empty(1, dtype=torch.float32, device=dev)
        self.dtheta = torch.empty(1, dtype=torch.float32, device=dev)
        # one workspace for the forward and the backward: the forward's prep (rotated keys, fp16
        # keys and values, the cos/sin table) is a prefix of it, and where the backward's own prep
        # would write the same arrays the backward runs its query and key stages only
        nbytes = max(fa.fibattn_fwd_workspace_bytes(B, L, Hkv), fa.fibattn_bwd_workspace_bytes(B, L, Hq, Hkv, D, w.W, len(base)))
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.reuse = [fa.fibattn_bwd_reuses_fwd_prep(a, w.W, base, B, L, Hq, Hkv, D) for a in self.alphas]
        # the rounded-integer variant of the same schedule (integer offsets, read at alpha = 1)
        self.rounded = [fa.fibattn_round_offsets(a, base) for a in self.alphas]
        self.reuse_rounded = [fa.fibattn_bwd_reuses_fwd_prep(1.0, w.W, r, B, L, Hq, Hkv, D) for r in self.rounded]

    def fwd(self, layer):
        q, k, v, _ = self.inputs[layer]
        self.fa.fibattn_fwd(q, k, v, self.alphas[layer], self.w.W, self.base, o=self.o[layer],
                            lse=self.lse[layer], workspace=self.ws)

    def fwd_rounded(self, layer):
        q, k, v, _ = self.inputs[layer]
        self.fa.fibattn_fwd(q, k, v, 1.0, self.w.W, self.rounded[layer], o=self.o[layer], lse=self.lse[layer],
                            workspace=self.ws)

    def bwd_rounded(self, layer):
        q, k, v, do = self.inputs[layer]
        fa = self.fa
        st = fa.STAGE_QUERY | fa.STAGE_KEY if self.reuse_rounded[layer] else fa.STAGE_ALL
        fa.fibattn_bwd_stages(st, q, k, v, do, 1.0, self.w.W, self.rounded[layer], self.dq[layer], self.dk[layer],
                              self.dv[layer], self.ws)

    def decode_setup(self):
        """Each sequence's last row as its new token; the layer's k and v as the cache."""
        if getattr(self, "dq_last", None) is None:
            L = self.w.L
            self.dq_last = [inp[0][:, :, L - 1].contiguous() for inp in self.inputs]
            self.dpos = torch.full((self.w.B,), L - 1, dtype=torch.int32, device=self.dev)
            self.do_last = [torch.empty_like(x) for x in self.dq_last]

    def decode(self, layer):
        _, k, v, _ = self.inputs[layer]
        self.fa.fibattn_decode(self.dq_last[layer], k, v, self.dpos, self.alphas[layer], self.w.W, self.base,
                               o=self.do_last[layer], need_lse=False)

    def decode_rounded(self, layer):
        _, k, v, _ = self.inputs[layer]
        self.fa.fibattn_decode(self.dq_last[layer], k, v, self.dpos, 1.0, self.w.W, self.rounded[layer],
                               o=self.do_last[layer], need_lse=False)

    def prep(self, layer):
        self.fa.fibattn_fwd_prep(self.inputs[layer][1], self.inputs[layer][2], self.ws)

    def attend(self, layer):
        q, k, v, _ = self.inputs[layer]
        self.fa.fibattn_fwd_attend(q, k, v, self.alphas[layer], self.w.W, self.base, self.ws, self.o[layer],
                                   self.lse[layer])

    def bwd_stages(self, layer, stages):
        q, k, v, do = self.inputs[layer]
        wd = self.want_dalpha[layer]
        self.fa.fibattn_bwd_stages(stages, q, k, v, do, self.alphas[layer], self.w.W, self.base, self.dq[layer],
                                   self.dk[layer], self.dv[layer], self.ws, dalpha_dtheta=self.dadt[layer],
                                   dalpha=self.dalpha if wd else None, dtheta=self.dtheta if wd else None)

    def bwd(self, layer):
        """The backward as a training step runs it, after this layer's forward on the same workspace."""
        fa = self.fa
        self.bwd_stages(layer, fa.STAGE_QUERY | fa.STAGE_KEY if self.reuse[layer] else fa.STAGE_ALL)

    def bwd_prep(self, layer):
        self.bwd_stages(layer, self.fa.STAGE_PREP)

    def bwd_query(self, layer):
        self.bwd_stages(layer, self.fa.STAGE_QUERY)

    def bwd_key(self, layer):
        self.bwd_stages(layer, self.fa.STAGE_KEY)

    def step(self):
        for layer in range(self.n_sets):
            self.fwd(layer)
            self.bwd(layer)


def profile_pass(fa, name: str, dev):
    """A short program for hardware-counter runs: two layers of the workload, two forward + backward
    passes over them, then a plain 256 MiB device-to-device copy (torch's copy kernel) whose byte
    counters calibrate the kernels' (it reads and writes exactly 2^28 bytes)."""
    w = workloads.WORKLOADS[name]
    net = Layers(fa, w, dev, n_sets=2)
    for _ in range(2):
        net.step()
    src = torch.ones(1 << 28, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[{name}] profile pass done")


PHASES = ("q and key near block", "key pass", "value near block", "value pass", "stores")
RTC_MHZ = 100.0   # the GPU's real-time counter (s_memrealtime), a constant 100 MHz


def phase_trace(name: str, dev, reps: int = 3):
    """Per-workgroup phase timeline of the forward attention kernel (bf16 storage), every layer of
    the workload, from the trace build (libfibattn_trace.so, which records stamps at the phase
    boundaries of each workgroup): per phase the median and 90th percentile over workgroups (µs), the
    spread of workgroup start and end times, the span from the first start to the last end (to be
    read beside the kernel's duration in a kernel trace, a check of the clock), and when workgroups
    end by their number of far steps."""
    import fibonacci_offset_sparse_amd as fa
    fa.lib = fa._load_from(fa.TRACE_LIB_PATH)
    w = workloads.WORKLOADS[name]
    code = {"fixed": fa.SCHEDULE_FIXED, "linear": fa.SCHEDULE_LINEAR, "coprime": fa.SCHEDULE_COPRIME}
    thetas = workloads.draw_theta(w.n_layers).tolist() if w.schedule == "learned" else None
    base = fa.fibattn_base_offsets(fa.BASE_FIB) if w.base == "fib" else \
        fa.fibattn_base_offsets(fa.BASE_POW2, workloads.pow2_max(w))
    n_wg = w.B * w.Hkv * (w.Hq // w.Hkv // 4) * ((w.L + 63) // 64)
    q_ = lambda a, f: float(np.quantile(a, f))
    layers = []
    for layer in range(w.n_layers):
        alpha = fa.fibattn_alpha_from_theta(thetas[layer])[0] if thetas else \
            fa.fibattn_alpha_schedule(code[w.schedule], layer, w.n_layers)
        q, k, v = (x.to(dev) for x in workloads.draw(w, layer, with_grad=False))
        for _ in range(reps):
            fa.fibattn_fwd(q, k, v, alpha, w.W, base)
        torch.cuda.synchronize()
        # the traced call: only the attention kernel records, and its last launch is this one
        fa.fibattn_fwd(q, k, v, alpha, w.W, base)
        torch.cuda.synchronize()
        rec = fa.fibattn_phase_trace_read(n_wg).astype(np.float64)
        us = 1.0 / RTC_MHZ
        t = rec[:, :6]
        t0 = t[:, 0].min()
        dur = np.diff(t, axis=1) * us
        starts, ends = (t[:, 0] - t0) * us, (t[:, 5] - t0) * us
        info = rec[:, 6].astype(np.uint64)
        far = ((info >> np.uint64(16)) & np.uint64(0xff)).astype(int) - ((info >> np.uint64(24)) & np.uint64(0xff)).astype(int)
        by_far = {int(f): {"workgroups": int((far == f).sum()), "end_median_us": q_(ends[far == f], 0.5)}
                  for f in sorted(set(far.tolist()))}
        layers.append({
            "layer": layer, "alpha": alpha, "span_us": float(ends.max()),
            "phases_us": {PHASES[j]: {"median": q_(dur[:, j], 0.5), "p90": q_(dur[:, j], 0.9)} for j in range(5)},
            "start_us": {"p50": q_(starts, 0.5), "p90": q_(starts, 0.9), "max": float(starts.max())},
            "end_us": {"p10": q_(ends, 0.1), "p50": q_(ends, 0.5), "p90": q_(ends, 0.9), "max": float(ends.max())},
            "end_by_far_steps": by_far,
        })
        log(f"[{name}] layer {layer} alpha={alpha:.4f}: span {ends.max():.2f} us, "
            + ", ".join(f"{PHASES[j]} {np.median(dur[:, j]):.2f}" for j in range(5)))
        del q, k, v
    summary = {PHASES[j]: {"median_over_layers_of_median": float(np.median([l["phases_us"][PHASES[j]]["median"] for l in layers])),
                           "median_over_layers_of_p90": float(np.median([l["phases_us"][PHASES[j]]["p90"] for l in layers]))}
               for j in range(5)}
    return {"workload": name, "workgroups": n_wg, "clock_MHz": RTC_MHZ, "layers": layers, "summary": summary,
            "span_us_mean": float(np.mean([l["span_us"] for l in layers]))}


def time_steps(net: Layers, steps: int, warmup: int):
    for _ in range(warmup):
        net.step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        net.step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


def time_stages(net: Layers, sweeps: int, stages=None):
    """Average duration of each stage, from HIP events on the stream the kernels run on.

    Each stage is launched for all layers back to back behind a short GPU spin, so the launches
    are queued before the GPU reaches them and the events see kernel time, not host gaps. A later
    stage reads what the earlier one left in the shared workspace, from the last layer it ran on
    (the same work: the workspace holds values only, its layout does not depend on the layer)."""
    n = net.w.n_layers
    if stages is None:
        stages = {"fwd_prep": net.prep, "fwd_attend": net.attend, "bwd": net.bwd, "bwd_prep": net.bwd_prep,
                  "bwd_query": net.bwd_query, "bwd_key": net.bwd_key}
    tot = {k: 0.0 for k in stages}
    for _ in range(sweeps):
        for name, fn in stages.items():
            torch.cuda.synchronize()
            torch.cuda._sleep(20_000_000)               # keeps the GPU busy while the launches queue
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for layer in range(n):
                fn(layer)
            e1.record()
            torch.cuda.synchronize()
            tot[name] += e0.elapsed_time(e1) / n
    return {k: v / sweeps for k, v in tot.items()}


def time_layers(net: Layers, sweeps: int, stages):
    """Per-layer call durations: median, 10th and 90th percentile over the sweeps.

    Each stage runs over all layers back to back behind a short GPU spin, with an event between
    consecutive calls, so each call's duration is the gap between the events around it."""
    import numpy as np
    n = net.w.n_layers
    out = {}
    for name, fn in stages.items():
        samples = np.zeros((sweeps, n))
        for s in range(sweeps):
            torch.cuda.synchronize()
            torch.cuda._sleep(20_000_000)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
            ev[0].record()
            for layer in range(n):
                fn(layer)
                ev[layer + 1].record()
            torch.cuda.synchronize()
            samples[s] = [ev[i].elapsed_time(ev[i + 1]) for i in range(n)]
        med, p10, p90 = (np.percentile(samples, q, axis=0) for q in (50, 10, 90))
        out[name] = {"median": [round(x, 5) for x in med.tolist()], "p10": [round(x, 5) for x in p10.tolist()],
                     "p90": [round(x, 5) for x in p90.tolist()], "total_median": float(med.sum())}
    return out


def fwd_slot_counts(fa, w, alpha: float, base):
    """(valid (query-head, slot) pairs, (key row, interpolated rung) pairs) of one forward call,
    from the library's offset plan: window distance d is valid at query i >= d, a kept rung at
    i >= its reach."""
    kind, _, _, reach = fa.fibattn_plan(alpha, w.W, base)
    win = sum(min(w.W, i) + 1 for i in range(w.L))
    kept = sum(max(0, w.L - int(r)) for kd, r in zip(kind, reach) if kd != fa.DUP)
    interp = sum(max(0, w.L - int(r)) for kd, r in zip(kind, reach) if kd == fa.INTERP)
    return w.B * w.Hq * (win + kept), w.B * w.Hkv * interp


def fwd_staged_bytes(fa, w, alpha: float, base) -> int:
    """Bytes the matrix-core forward stages from the staged key and value rows into LDS in one call
    (rows inside [0, L) only: the rest arrive as zeros without a memory access). Per workgroup
    (64 queries, 4 heads of one key-value head): for keys and for values, the near block (rows
    i0 - 64 .. i0 + 63) and each rung step from the first far pair on (two blocks of 72 rows,
    i0 - a - 1 and i0 - a' - 3 on, a block only where its rung is reached)."""
    kind, a_all, _, reach = fa.fibattn_plan(alpha, w.W, base)
    kept = [(int(a), int(r) - int(a)) for kd, a, r in zip(kind, a_all, reach) if kd != fa.DUP]
    L = w.L

    def rows(j0, n):
        return max(0, min(j0 + n, L) - max(j0, 0))
    per_unit = 0
    for i0 in range(0, L, 64):
        n_reach = 0
        for n, (a, it) in enumerate(kept):
            if i0 + 63 >= a + it:
                n_reach = n + 1
        n_steps = (n_reach + 1) >> 1
        n_near = 0
        for n in range(n_reach):
            if kept[n][0] <= 63:
                n_near = n + 1
        kn = (n_near >> 1) & ~1
        r = rows(i0 - 64, 128)
        for k in range(kn, n_steps):
            if 2 * k < n_reach:
                r += rows(i0 - kept[2 * k][0] - 1, 72)
            if 2 * k + 1 < n_reach:
                r += rows(i0 - kept[2 * k + 1][0] - 3, 72)
        per_unit += 2 * r * w.D * 2                      # keys and values, fp16 rows
    return per_unit * w.B * w.Hkv * (w.Hq // w.Hkv // 4)


def measure(fa, name: str, steps: int, warmup: int, dev):
    w = workloads.WORKLOADS[name]
    log(f"[{name}] allocating inputs")
    net = Layers(fa, w, dev)
    log(f"[{name}] warmup {warmup} + timed {steps} steps")
    ms_step, wall = time_steps(net, steps, warmup)
    log(f"[{name}] {ms_step:.3f} ms per step; timing stages")
    st = time_stages(net, 3)
    log(f"[{name}] timing each layer's calls")
    per_layer = time_layers(net, 10, {"fwd_ms": net.fwd, "bwd_ms": net.bwd})
    per_layer["alpha"] = [round(a, 6) for a in net.alphas]
    per_layer["what"] = ("each layer's forward and backward call (ms): median, p10, p90 over 10 sweeps; the "
                         "event between calls drains the queue, so these read 1-4 us per call above kernels_ms")
    integer_path = None
    if w.schedule in ("linear", "coprime"):
        # the same schedule with rounded offsets on the integer path, against the interpolated
        # gather, per layer call on the same inputs
        log(f"[{name}] timing the rounded-integer variant")
        it = time_stages(net, 3, {"fwd_interp": net.fwd, "fwd_int": net.fwd_rounded, "bwd_interp": net.bwd,
                                  "bwd_int": net.bwd_rounded})
        net.decode_setup()
        dt = time_stages(net, 3, {"decode_interp": net.decode, "decode_int": net.decode_rounded})
        integer_path = {
            "what": "rounded-integer stagger (offsets round-half-even(alpha_l f_k), read at alpha = 1) against "
                    "the interpolated stagger, same inputs, ms per layer call",
            "decode_us_interp": dt["decode_interp"] * 1e3, "decode_us_int": dt["decode_int"] * 1e3,
            "decode_ratio": dt["decode_interp"] / dt["decode_int"],
            "decode_what": f"single-token decode, {w.B} sequences each at position {w.L - 1} of a {w.L}-row cache",
            "fwd_ms_interp": it["fwd_interp"], "fwd_ms_int": it["fwd_int"], "fwd_ratio": it["fwd_interp"] / it["fwd_int"],
            "bwd_ms_interp": it["bwd_interp"], "bwd_ms_int": it["bwd_int"], "bwd_ratio": it["bwd_interp"] / it["bwd_int"],
            "paper": "about 5x inference latency for the learned (interpolated, unfused gather) variant against the "
                     "fused boolean-mask path of the integer variants (other hardware; context only)",
        }
    qh = w.B * w.L * w.Hq
    eb = 2 if w.dtype == "bf16" else 4
    rows = w.B * w.L * w.D * eb                                                # one head's rows
    fwd_bytes = (2 * w.Hq + 2 * w.Hkv) * rows + qh * 4                          # q, k, v, o, lse
    bwd_bytes = (3 * w.Hq + 2 * w.Hkv) * rows + qh * 4 \
        + (w.Hq + 2 * w.Hkv) * rows                                            # + dq, dk, dv
    # per kernel: the caller's tensors each one reads or writes (workspace hand-offs excluded)
    kernel_bytes = {
        "fwd_attend": fwd_bytes,                                                # q, k, v (staged), o, lse
        "bwd_query": (3 * w.Hq + 2 * w.Hkv) * rows,                             # q, dout, k, v; dq
        "bwd_key": (2 * w.Hq + 2 * w.Hkv) * rows,                               # q, dout; dk, dv
    }
    fwd_ms = st["fwd_prep"] + st["fwd_attend"]
    # algorithmic arithmetic of the forward attention: 2 D FMA per valid (query-head, slot) for
    # QK and P.V, plus 2 D per (key row, interpolated rung) for blending the key and value rows
    # (shared by the group's heads); masked slots and dropped rungs are not counted
    fma, slots = [], []
    for a in net.alphas:
        n_valid, n_interp = fwd_slot_counts(fa, w, a, net.base)
        fma.append(2 * w.D * n_valid + 2 * w.D * n_interp)
        slots.append(n_valid / qh)
    fma_call = sum(fma) / len(fma)
    arith = {"fma_per_call": fma_call, "valid_slots_per_qh": sum(slots) / len(slots),
             "achieved_tflops": 2 * fma_call / (st["fwd_attend"] * 1e-3) / 1e12,
             "fp16_mfma_peak_tflops": FP16_MFMA_PEAK_TFLOPS,
             "frac_fp16_mfma_peak": 2 * fma_call / (st["fwd_attend"] * 1e-3) / 1e12 / FP16_MFMA_PEAK_TFLOPS,
             "what": "forward attention kernel, layer average: algorithmic flops (QK, P.V and the blend of "
                     "interpolated rows) over its time, against the dense fp16 matrix-core peak, where its "
                     "products run"}
    staged = sum(fwd_staged_bytes(fa, w, a, net.base) for a in net.alphas) / len(net.alphas)
    staging = {"bytes_per_call": staged, "TBps": staged / (st["fwd_attend"] * 1e-3) / 1e12,
               "what": "forward attention kernel, layer average: bytes it stages from the on-chip-resident "
                       "staged key and value rows into LDS, over its time"}
    res = {
        "ms_per_step": ms_step,
        "wall_s": wall,
        "qh_per_s": w.n_layers * qh / (ms_step * 1e-3),
        "fwd": {"ms_per_call": fwd_ms, "qh_per_s": qh / (fwd_ms * 1e-3),
                "GB_per_s": fwd_bytes / (fwd_ms * 1e-3) / 1e9,
                "frac_hbm_peak": fwd_bytes / (fwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "algorithmic_bytes": fwd_bytes},
        "bwd": {"ms_per_call": st["bwd"], "qh_per_s": qh / (st["bwd"] * 1e-3),
                "GB_per_s": bwd_bytes / (st["bwd"] * 1e-3) / 1e9,
                "frac_hbm_peak": bwd_bytes / (st["bwd"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "algorithmic_bytes": bwd_bytes},
        "kernels_ms": st,
        "arith_fwd_attend": arith,
        "staging_fwd_attend": staging,
        "per_layer": per_layer,
        "kernel_bytes": kernel_bytes,
        "integer_path": integer_path,
    }
    del net
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="l1024_linear_bf16")
    ap.add_argument("--long-workload", default="l4096_coprime_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-long", action="store_true")
    ap.add_argument("--profile-pass", action="store_true",
                    help="run the short counter-collection program instead of the timed bench")
    ap.add_argument("--stream-probe", action="store_true",
                    help="run only the streaming-bandwidth probe and print its JSON line")
    ap.add_argument("--phase-trace", action="store_true",
                    help="run the forward attention kernel's phase trace (libfibattn_trace.so) on every "
                         "layer of --workload and print its JSON line instead of the timed bench")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)

    if args.profile_pass:
        import fibonacci_offset_sparse_amd as fa
        profile_pass(fa, args.workload, torch.device("cuda:0"))
        return
    if args.stream_probe:
        print(json.dumps(stream_probe(torch.device("cuda:0"))), flush=True)
        return
    if args.phase_trace:
        print(json.dumps({"phase_trace": phase_trace(args.workload, torch.device("cuda:0"))}), flush=True)
        return

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: timing the float64 oracle on the host cores")
        cpu = cpu_baseline(args.workload)
        log(f"cpu baseline: {cpu['value']:.0f} q*h/s on {cpu['cores']} cores")

    import fibonacci_offset_sparse_amd as fa
    dev = torch.device("cuda:0")
    log("streaming probe")
    probe = stream_probe(dev)
    log(f"streaming probe: {probe}")
    main_res = measure(fa, args.workload, args.steps, args.warmup, dev)
    long_res = None if args.no_long else measure(fa, args.long_workload, max(3, args.steps // 4), 1, dev)

    w = workloads.WORKLOADS[args.workload]
    kms = main_res["kernels_ms"]

    def roofline(stage, kernel):
        ms, nbytes = kms[stage], main_res["kernel_bytes"][stage]
        achieved = nbytes / (ms * 1e-3) / 1e9
        return {"kernel": kernel, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(kernel, args.workload),
                "frac_of_measured_copy": achieved / (probe["copy_TBps"] * 1e3),
                "limiter": measured_limiter(kernel, args.workload),
                "traffic_unit": "bytes per launch", "avg_launch_ms": ms, "algorithmic_bytes_per_launch": nbytes}
    kernel_names = {"fwd_attend": "fwd_mfma_kernel", "bwd_query": "bwd_q_mfma_kernel",
                    "bwd_key": "bwd_k_dot_kernel"}
    dominant = max(kernel_names, key=lambda s: kms[s])
    line = {
        "metric": "fwd+bwd queries*heads/sec (and fwd HBM GB/s, % of peak)",
        "value": main_res["qh_per_s"],
        "unit": "queries*heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16/f32acc",
        "io_dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "B": w.B, "L": w.L, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D,
                   "W": w.W, "base": w.base, "schedule": w.schedule, "layers": w.n_layers,
                   "pass": "fwd+bwd", "parallelism": "none (1 GPU)"},
        "roofline": roofline(dominant, kernel_names[dominant]),
        "roofline_fwd_attend": roofline("fwd_attend", kernel_names["fwd_attend"]),
        "fwd": main_res["fwd"],
        "bwd": main_res["bwd"],
        "kernels_ms": main_res["kernels_ms"],
        "arith_fwd_attend": main_res["arith_fwd_attend"],
        "staging_fwd_attend": dict(main_res["staging_fwd_attend"],
                                   frac_of_lds_stage_probe=main_res["staging_fwd_attend"]["TBps"] / probe["lds_stage_TBps"]),
        "per_layer": main_res["per_layer"],
        "integer_path": main_res["integer_path"],
        "cpu_baseline": cpu,
        "stream_probe": probe,
    }
    # the forward's target: 60 % of peak HBM bandwidth at L = 1024 and L = 4096, for the attention
    # kernel on its own and for the whole forward call (prep included)
    target = {"target_frac": FWD_TARGET_FRAC}
    for key, res in (("l1024", main_res), ("l4096", long_res)):
        if res is None:
            continue
        att = res["kernel_bytes"]["fwd_attend"] / (res["kernels_ms"]["fwd_attend"] * 1e-3) / 1e9 / HBM_PEAK_GBS
        target[key] = {"attend_frac": att, "call_frac": res["fwd"]["frac_hbm_peak"],
                       "attend_met": att >= FWD_TARGET_FRAC, "call_met": res["fwd"]["frac_hbm_peak"] >= FWD_TARGET_FRAC}
    line["fwd_hbm_target"] = target
    if long_res is not None:
        lw = workloads.WORKLOADS[args.long_workload]
        line["l4096"] = {"workload": args.long_workload, "B": lw.B, "L": lw.L, "ms_per_step": long_res["ms_per_step"],
                         "qh_per_s": long_res["qh_per_s"], "fwd": long_res["fwd"], "bwd": long_res["bwd"],
                         "kernels_ms": long_res["kernels_ms"], "per_layer": long_res["per_layer"],
                         "arith_fwd_attend": long_res["arith_fwd_attend"],
                         "staging_fwd_attend": dict(long_res["staging_fwd_attend"],
                                                    frac_of_lds_stage_probe=long_res["staging_fwd_attend"]["TBps"]
                                                    / probe["lds_stage_TBps"]),
                         "integer_path": long_res["integer_path"]}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

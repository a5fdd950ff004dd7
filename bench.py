"""Benchmark: RMSNorm fwd+bwd achieved HBM GB/s on one MI355X.

One step = the whole path over one batch: forward (y, r), backward row pass
(dx written in place over dy, per-workgroup dgamma partials) and the dgamma
column reduction -- three launches through the C ABI.  Inputs are seeded
synthetic tensors already resident in HBM.  The default workload is bf16
M=16384 N=8192 with the Gemma (1+gamma) weight and an in-place dx: the
configuration the metric is quoted on.

Prints ONE JSON line.  ``value`` is algorithmic bytes of fwd+bwd per step
divided by the step time measured over exactly ``--steps`` timed steps
(after ``--warmup`` steps and a settle period), all three launches on
torch's current stream (``schedule``; the step with the column reduction on a
second stream, overlapping the next forward, is timed beside it).  ``roofline`` describes the dominant kernel
(the backward row pass) timed per launch with HIP events on its stream.
``configs`` holds the five RMSNorm workloads measured with the RMSNorm
tutorial's protocol (median of samples, each an event pair around 20
back-to-back calls): forward, backward (row pass + reduction) and the step,
hot (the same buffers every call) and flushed (operand sets rotated so that
no call finds its operands in the 256 MB Infinity Cache).
``cpu_baseline`` is the fp64 oracle timed on a bounded sample of the same
workload on this host, on one core (``value``) and sharded over up to 16
cores (``all_cores``).  ``layernorm`` holds the LayerNorm chapter's sweep
(M = 4096, fp16, N = 1024 .. 15872), ``rope`` and ``swiglu`` the two
elementwise ops of the Unsloth walkthrough on their workloads, each timed
with the same protocol.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import workloads as wl  # noqa: E402

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, published peak
DTYPE_CODE = {"f32": 0, "bf16": 1, "f16": 2}
METRIC = "RMSNorm fwd+bwd achieved HBM GB/s and % of peak, bf16 M=16384 N=8192"
# the sources every kernel and its launch plan are built from (their
# fingerprint ties the committed counter summary to the code it was taken on;
# comments excluded)
KERNEL_SRCS = tuple(os.path.join(ROOT, "row_normalization_amd", "csrc", f)
                    for f in ("rmsnorm_kernels.hip", "layernorm_kernels.hip", "elementwise_kernels.hip",
                              "device_common.h", "launch.h", "host_plan.h"))
PMC_SUMMARY = os.path.join(ROOT, "profiles", "hbm_traffic_and_lds_all_kernels.md")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1, help="GPUs (this benchmark runs on one)")
    ap.add_argument("--steps", type=int, default=200, help="timed fwd + bwd steps")
    ap.add_argument("--warmup", type=int, default=100, help="untimed steps before them")
    ap.add_argument("--workload", default="c3", choices=sorted(wl.RMS_WORKLOADS),
                    help="RMSNorm workload: " + "; ".join(f"{k} = {v.name}" for k, v in sorted(wl.RMS_WORKLOADS.items())))
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing (profiling runs)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--cpu-all-cores-seconds", type=float, default=8.0,
                    help="wall time of the oracle sample sharded over the host's cores (0: skip)")
    ap.add_argument("--schedule", default="one_stream", choices=("one_stream", "overlapped_reduce"),
                    help="the timed step's schedule: all three launches on one stream, or the dgamma reduction on "
                         "a second stream overlapping the next forward (the other is timed for context; measured "
                         "on MI355X the overlapped one was 3 %% slower: its two cross-stream waits per step cost "
                         "more than the 3.6 us reduction)")
    ap.add_argument("--samples", type=int, default=SAMPLES,
                    help=f"samples of {CALLS} back-to-back calls per per-launch or per-config figure (median)")
    ap.add_argument("--configs", nargs="*", default=sorted(wl.RMS_WORKLOADS), choices=sorted(wl.RMS_WORKLOADS),
                    help="RMSNorm workloads of the per-workload protocol block (default: all five)")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-workload protocol block")
    ap.add_argument("--no-layernorm", action="store_true", help="skip the LayerNorm sweep")
    ap.add_argument("--ln-samples", type=int, default=20, help="samples per LayerNorm sweep point and kernel")
    ap.add_argument("--ln-ns", type=int, nargs="*", default=None,
                    help="LayerNorm sweep points (N) to run; default: the chapter's 30 points")
    ap.add_argument("--no-elementwise", action="store_true", help="skip the RoPE and SwiGLU legs")
    ap.add_argument("--counter-pass", metavar="MANIFEST",
                    help="launch the fixed counter sequence (run under rocprofv3 --pmc) and write its manifest")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="print the counter summary of DIR/manifest.json and DIR/{fetch,write,lds} (no GPU)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the plain streaming kernels timed as the reference for the row kernels")
    return ap.parse_args()


def kernel_hash() -> str:
    """Fingerprint of the code the RMSNorm kernels are built from: the
    sources with comments and blank lines removed, so that an edit of a
    comment does not invalidate counters taken on the same code."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        lines = (re.sub(r"//.*", "", line).strip() for line in text.splitlines())
        h.update("\n".join(line for line in lines if line).encode())
    return h.hexdigest()[:16]


def traffic_table(h: str) -> dict:
    """Calibrated HBM bytes per launch, by counter-pass label ("rms c3
    bwd_rows", ...), from the committed counter summary, if it was taken on
    the current kernel sources; else {}."""
    if not os.path.exists(PMC_SUMMARY):
        return {}
    m = re.search(r"```json\n(.*?)\n```", open(PMC_SUMMARY).read(), flags=re.S)
    if not m:
        return {}
    data = json.loads(m.group(1))
    if data.get("kernel_sha") != h:
        return {}
    return {label: e["scaled_bytes"] for label, e in data["entries"].items()}


class Path:
    """Device buffers and pre-marshalled C-ABI calls for one workload.

    ``sets`` operand sets (x, dy, y, rstd, dx, workspace) share one gamma;
    call ``k`` uses set ``k % sets``, so rotating through enough sets keeps
    every call's operands out of the caches.  Every set is uploaded from the
    generated host tensors (no device-to-device copy: under rocprofv3's
    counter collection those crashed inside the runtime).  Every call's
    arguments are built once (a launch then costs one ctypes call on the
    host)."""

    def __init__(self, w: wl.Workload, sets: int = 1):
        import row_normalization_amd as rn

        self.w = w
        self.L = rn.lib()
        t = wl.make_inputs(w)
        dev = "cuda"
        self.gamma = t["gamma"].to(dev)
        self.sets = sets
        self.x = [t["x"].to(dev) for _ in range(sets)]
        self.dy = [t["dy"].to(dev) for _ in range(sets)]
        self.dy_host = t["dy"] if w.dx_in_place else None
        del t
        x0, dy0 = self.x[0], self.dy[0]
        self.y = [torch.empty_like(x0) for _ in range(sets)]
        self.rstd = [torch.empty(w.M, dtype=torch.float32, device=dev) for _ in range(sets)]
        self.dx = self.dy if w.dx_in_place else [torch.empty_like(dy0) for _ in range(sets)]
        self.dgamma = torch.empty(w.N, dtype=torch.float32, device=dev)
        self.ws_bytes = rn.rmsnorm_bwd_workspace_bytes(w.M, w.N, w.torch_dtype)
        # two workspaces per set: the overlapped schedule alternates between them
        self.ws = [torch.empty(max(self.ws_bytes // 4, 1), dtype=torch.float32, device=dev)
                   for _ in range(2 * sets)]
        self.dtype = DTYPE_CODE[w.dtype]
        self.rows = ctypes_int64()
        self.stream = torch.cuda.current_stream().cuda_stream
        M, N, flags = w.M, w.N, int(w.gemma)
        self._fwd = [(self.x[k].data_ptr(), self.gamma.data_ptr(), self.y[k].data_ptr(), self.rstd[k].data_ptr(), M,
                      N, N, w.eps, self.dtype, flags) for k in range(sets)]
        self._rows = [[(self.x[k].data_ptr(), self.gamma.data_ptr(), self.dy[k].data_ptr(), self.rstd[k].data_ptr(),
                        self.dx[k].data_ptr(), self.ws[2 * k + b].data_ptr(), self.ws_bytes, M, N, N, self.dtype,
                        flags, self.rows.ref) for b in range(2)] for k in range(sets)]
        self.bwd_rows()
        torch.cuda.synchronize()
        self.partial_rows = self.rows.value
        self._red = [[(self.ws[2 * k + b].data_ptr(), self.partial_rows, N, self.dgamma.data_ptr())
                      for b in range(2)] for k in range(sets)]

    def fwd(self, k: int = 0, stream=None):
        st = self.L.rmsnorm_fwd(*self._fwd[k % self.sets], stream or self.stream)
        assert st == 0, st

    def bwd_rows(self, k: int = 0, ws: int = 0, stream=None):
        st = self.L.rmsnorm_bwd_rows(*self._rows[k % self.sets][ws], stream or self.stream)
        assert st == 0, st

    def reduce(self, k: int = 0, ws: int = 0, stream=None):
        st = self.L.rmsnorm_dgamma_reduce(*self._red[k % self.sets][ws], stream or self.stream)
        assert st == 0, st

    def bwd(self, k: int = 0):
        self.bwd_rows(k)
        self.reduce(k)

    def step(self, k: int = 0):
        self.fwd(k)
        self.bwd_rows(k)
        self.reduce(k)

    def restore(self):
        """dy back to its generated values in every set (in place, dx overwrote
        it), then a read sweep so that the copies' dirty cache lines are
        written back before the timed calls."""
        if self.dy_host is not None:
            for d in self.dy:
                d.copy_(self.dy_host)
            flush_by_reading()


_FLUSH = None


def flush_by_reading() -> None:
    """Read a 1 GiB buffer: it takes the place of everything in L2 and the
    256 MB Infinity Cache, and any dirty line there is written back now."""
    global _FLUSH
    if _FLUSH is None:
        _FLUSH = torch.zeros(1 << 28, dtype=torch.float32, device="cuda")
    _FLUSH.sum()


class OverlappedSteps:
    """The step with the dgamma column reduction on a second stream: step k's
    reduction waits for its row pass (an event) and overlaps step k + 1's
    forward.  The row passes alternate between two workspaces; before the row
    pass of step k + 2 reuses a workspace, its stream waits for step k's
    reduction.  Nothing in a training step reads dgamma before the optimizer,
    so the reduction has only to be done by then.  Both streams have the
    default priority."""

    def __init__(self, path: Path):
        self.p = path
        self.side = torch.cuda.Stream()
        self.side_handle = self.side.cuda_stream
        self.rows_done = [torch.cuda.Event() for _ in range(2)]
        self.reduce_done = [torch.cuda.Event() for _ in range(2)]
        self.used = [False, False]
        self.k = 0

    def step(self, _=None):
        p, b = self.p, self.k % 2
        main = torch.cuda.current_stream()
        p.fwd()
        if self.used[b]:
            main.wait_event(self.reduce_done[b])  # step k - 2's reduction has read this workspace
        p.bwd_rows(0, b)
        self.rows_done[b].record(main)
        self.side.wait_event(self.rows_done[b])
        p.reduce(0, b, self.side_handle)
        self.reduce_done[b].record(self.side)
        self.used[b] = True
        self.k += 1

    def join(self):
        """Make the current stream wait for every reduction issued so far."""
        for b in range(2):
            if self.used[b]:
                torch.cuda.current_stream().wait_event(self.reduce_done[b])


class ctypes_int64:
    def __init__(self):
        import ctypes

        self._v = ctypes.c_int64(0)
        self.ref = ctypes.byref(self._v)

    @property
    def value(self):
        return self._v.value


class LnPath:
    """Device buffers and C-ABI calls of the LayerNorm path for one workload."""

    def __init__(self, w: wl.Workload):
        import row_normalization_amd as rn

        self.w = w
        self.L = rn.lib()
        t = wl.make_inputs(w)
        self.x, self.weight, self.bias, self.dy = (t[k].to("cuda") for k in ("x", "gamma", "beta", "dy"))
        self.y = torch.empty_like(self.x)
        self.dx = torch.empty_like(self.x)
        self.mean = torch.empty(w.M, dtype=torch.float32, device="cuda")
        self.rstd = torch.empty(w.M, dtype=torch.float32, device="cuda")
        self.dw = torch.empty(w.N, dtype=torch.float32, device="cuda")
        self.db = torch.empty(w.N, dtype=torch.float32, device="cuda")
        self.ws_bytes = rn.layernorm_bwd_workspace_bytes(w.M, w.N, w.torch_dtype)
        self.ws = torch.empty(self.ws_bytes // 4, dtype=torch.float32, device="cuda")
        self.dtype = DTYPE_CODE[w.dtype]
        self.stream = torch.cuda.current_stream().cuda_stream
        self.rows = ctypes_int64()
        self.partial_rows = None

    def fwd(self):
        st = self.L.layernorm_fwd(self.x.data_ptr(), self.weight.data_ptr(), self.bias.data_ptr(), self.y.data_ptr(),
                                  self.mean.data_ptr(), self.rstd.data_ptr(), self.w.M, self.w.N, self.w.N,
                                  self.w.eps, self.dtype, self.stream)
        assert st == 0, st

    def bwd_rows(self):
        st = self.L.layernorm_bwd_rows(self.x.data_ptr(), self.weight.data_ptr(), self.dy.data_ptr(),
                                       self.mean.data_ptr(), self.rstd.data_ptr(), self.dx.data_ptr(),
                                       self.ws.data_ptr(), self.ws_bytes, self.w.M, self.w.N, self.w.N, self.dtype,
                                       self.rows.ref, self.stream)
        assert st == 0, st
        self.partial_rows = self.rows.value

    def reduce(self):
        st = self.L.layernorm_dwdb_reduce(self.ws.data_ptr(), self.partial_rows, self.w.N, self.dw.data_ptr(),
                                          self.db.data_ptr(), self.stream)
        assert st == 0, st

    def bwd(self):
        self.bwd_rows()
        self.reduce()

    def step(self):
        self.fwd()
        self.bwd_rows()
        self.reduce()


# The RMSNorm tutorial's protocol ("Benchmark đo thời gian nào?"): warm up,
# then the median over samples, each an event pair around back-to-back calls.
SAMPLES = 50
CALLS = 20


def _ln_point(w, samples: int) -> dict:
    """Forward, row pass, column sum and the dependent backward pair of one
    LayerNorm workload, each the median over `samples` samples."""
    path = LnPath(w)
    path.step()
    t_f, t_r, t_d = (time_calls(fn, samples)["median_s"] for fn in (path.fwd, path.bwd_rows, path.reduce))
    t_b = time_calls(path.bwd, samples)["median_s"]
    b = wl.ln_algorithmic_bytes(w.M, w.N, w.elsize)
    numel_bytes = w.M * w.N * w.elsize
    point = {
        "N": w.N,
        "fwd_us": round(t_f * 1e6, 2), "bwd_rows_us": round(t_r * 1e6, 2), "reduce_us": round(t_d * 1e6, 2),
        "bwd_us": round(t_b * 1e6, 2),
        "fwd_gbps_page_formula": round(2 * numel_bytes / t_f / 1e9, 1),
        "bwd_gbps_page_formula": round(3 * numel_bytes / t_b / 1e9, 1),
        "fwd_frac": round(b["fwd"] / t_f / 1e9 / PEAK_HBM_GBPS, 4),
        "bwd_rows_frac": round(b["bwd_rows"] / t_r / 1e9 / PEAK_HBM_GBPS, 4),
        "bwd_frac": round(b["bwd"] / t_b / 1e9 / PEAK_HBM_GBPS, 4),
        # the backward's two launches timed apart and added (no dependent pair)
        "bwd_parts_frac": round(b["bwd"] / (t_r + t_d) / 1e9 / PEAK_HBM_GBPS, 4),
        "partial_rows": path.partial_rows,
    }
    del path
    torch.cuda.empty_cache()
    return point


def layernorm_sweep(samples: int, ns=None) -> dict:
    """The LayerNorm chapter's sweep: M = 4096 fp16, N = 512 * i, i = 2 .. 31;
    beside it, outside the medians, rows beyond 16384 elements up to the
    chapter's 64 KB (the wide kernels)."""
    points = []
    for N in (ns or wl.LN_SWEEP_NS):
        points.append(_ln_point(wl.ln_sweep(N), samples))
        print(f"[layernorm sweep] N={N}: fwd {points[-1]['fwd_us']} us, bwd {points[-1]['bwd_us']} us",
              file=sys.stderr, flush=True)
    wide = []
    for N in (() if ns else LN_WIDE_NS):
        wide.append(_ln_point(wl.ln_sweep(8192).scaled(N=N, name=f"ln_f16_4096x{N}"), samples))
        print(f"[layernorm wide] N={N}: fwd {wide[-1]['fwd_us']} us, bwd {wide[-1]['bwd_us']} us",
              file=sys.stderr, flush=True)
    med = lambda key: float(np.median([p[key] for p in points]))
    return {"workload": f"layernorm fp16 M={wl.LN_SWEEP_M}, N = 512*i for i = 2..31",
            "protocol": f"median of {samples} samples x {CALLS} back-to-back calls; bwd: row pass and column sum "
                        "as one dependent pair per call; bwd_parts: the two timed apart, added",
            "median_fwd_frac": round(med("fwd_frac"), 4), "median_bwd_frac": round(med("bwd_frac"), 4),
            "median_bwd_parts_frac": round(med("bwd_parts_frac"), 4),
            "median_bwd_gbps_page_formula": round(med("bwd_gbps_page_formula"), 1), "points": points,
            "wide": {"workload": f"layernorm fp16 M={wl.LN_SWEEP_M}, rows beyond 16384 elements (wide kernels), "
                                 "not in the medians", "points": wide}}


# Wide LayerNorm rows timed beside the sweep: 3 chunks with one vector in the
# last, 3 full chunks, 4 full chunks (the chapter's 64 KB rows).
LN_WIDE_NS = (16392, 24576, 32768)


# Untimed work before each measurement.  On MI355X a new stream of launches
# runs up to ~15 % slower for its first ~10 ms and then settles (seen in
# rocprofv3 traces of 150 back-to-back SwiGLU forwards: ~150 us, rising to
# ~176 us around 6-9 ms in, back to ~152 us from ~15 ms on).
WARM_SECONDS = 0.025
# Before the headline's timed steps, whatever --warmup asks for: its 20-200
# timed steps last only 4-45 ms.
SETTLE_SECONDS = 0.1


def settle(fn, seconds: float = SETTLE_SECONDS, batch: int = 10) -> int:
    """Call fn(k) in batches until `seconds` of synchronised wall time have
    passed; returns the number of calls."""
    t0, calls = time.perf_counter(), 0
    while True:
        for _ in range(batch):
            fn(calls)
            calls += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return calls


def _call(fn):
    """fn as a function of the call index (ignored when fn takes none)."""
    import inspect

    try:
        takes = len(inspect.signature(fn).parameters) > 0
    except (TypeError, ValueError):
        takes = False
    return fn if takes else (lambda k: fn())


def time_calls(fn, samples: int = SAMPLES, calls: int = CALLS, before_sample=None, join=None) -> dict:
    """Seconds per call: the median (min, max) over `samples` event pairs, each
    around `calls` back-to-back calls of fn(k) on the current stream, after a
    settle period.  before_sample() runs outside the events; join() (if
    given) makes the current stream wait for work fn queued elsewhere before
    the closing event."""
    f = _call(fn)
    settle(f, WARM_SECONDS, 3)
    if join:
        join()
    out, k = [], 0
    for _ in range(samples):
        if before_sample:
            before_sample()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(calls):
            f(k)
            k += 1
        if join:
            join()
        e.record()
        torch.cuda.synchronize()
        out.append(s.elapsed_time(e) * 1e-3 / calls)
    return {"median_s": float(np.median(out)), "min_s": float(np.min(out)), "max_s": float(np.max(out))}


def rope_leg(samples: int) -> dict:
    import row_normalization_amd as rn

    w = wl.ROPE1
    t = wl.make_rope_inputs(w)
    q, cos, sin, pos = t["q"].cuda(), t["cos"].cuda(), t["sin"].cuda(), t["positions"].cuda()
    L = rn.lib()
    stream = torch.cuda.current_stream().cuda_stream
    args = (q.data_ptr(), w.tokens, w.heads, w.head_dim, w.heads * w.head_dim, cos.data_ptr(), sin.data_ptr(),
            w.seq_len, pos.data_ptr(), w.seq_len, DTYPE_CODE[w.dtype], stream)

    def fwd():
        assert L.rope_fwd(*args) == 0

    def bwd():
        assert L.rope_bwd(*args) == 0

    t_f, t_b = (time_calls(fn, samples)["median_s"] for fn in (fwd, bwd))
    nbytes = wl.rope_algorithmic_bytes(w.tokens, w.heads, w.head_dim, w.elsize, w.seq_len)
    return {"workload": w.name, "fwd_us": round(t_f * 1e6, 2), "bwd_us": round(t_b * 1e6, 2),
            "algorithmic_bytes": nbytes, "fwd_gbps": round(nbytes / t_f / 1e9, 1),
            "bwd_gbps": round(nbytes / t_b / 1e9, 1), "fwd_frac": round(nbytes / t_f / 1e9 / PEAK_HBM_GBPS, 4),
            "bwd_frac": round(nbytes / t_b / 1e9 / PEAK_HBM_GBPS, 4)}


def swiglu_leg(samples: int) -> dict:
    import row_normalization_amd as rn

    w = wl.SWIGLU1
    t = wl.make_swiglu_inputs(w)
    e, g, dh = (t[k].cuda() for k in ("e", "g", "dh"))
    h, df, de = (torch.empty_like(e) for _ in range(3))
    L = rn.lib()
    stream = torch.cuda.current_stream().cuda_stream
    code = DTYPE_CODE[w.dtype]

    def fwd():
        assert L.swiglu_fwd(e.data_ptr(), g.data_ptr(), h.data_ptr(), w.M, w.N, w.N, code, stream) == 0

    def bwd():
        assert L.swiglu_bwd(dh.data_ptr(), e.data_ptr(), g.data_ptr(), h.data_ptr(), df.data_ptr(), de.data_ptr(),
                            w.M, w.N, w.N, code, stream) == 0

    t_f, t_b = (time_calls(fn, samples)["median_s"] for fn in (fwd, bwd))
    b = wl.swiglu_algorithmic_bytes(w.M, w.N, w.elsize)
    return {"workload": w.name, "fwd_us": round(t_f * 1e6, 2), "bwd_us": round(t_b * 1e6, 2),
            "fwd_gbps": round(b["fwd"] / t_f / 1e9, 1), "bwd_gbps": round(b["bwd"] / t_b / 1e9, 1),
            "fwd_frac": round(b["fwd"] / t_f / 1e9 / PEAK_HBM_GBPS, 4),
            "bwd_frac": round(b["bwd"] / t_b / 1e9 / PEAK_HBM_GBPS, 4), "algorithmic_bytes": b}


def time_steps(step, steps: int, join=None) -> float:
    """Seconds per step over exactly `steps` back-to-back steps, bracketed by
    HIP events on the current stream and device synchronisations."""
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for k in range(steps):
        step(k)
    if join:
        join()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) * 1e-3 / steps


# Bytes of operand sets rotated through for the "flushed" figures: more than
# four times the 256 MB Infinity Cache, so a call's operands have always been
# pushed out by the calls between two uses of the same set.
ROTATION_BYTES = 1 << 30


def config_protocol(w: wl.Workload, samples: int) -> dict:
    """Forward, backward (row pass + reduction) and the step of one workload,
    hot (one operand set) and flushed (sets rotated), medians per call."""
    b = wl.algorithmic_bytes(w.M, w.N, w.elsize)
    per_set = (2 if w.dx_in_place else 3) * w.M * w.N * w.elsize + w.M * w.N * w.elsize
    sets = max(2, -(-ROTATION_BYTES // per_set) + 1)
    path = Path(w, sets)
    path.step()
    torch.cuda.synchronize()
    out = {"workload": w.name, "M": w.M, "N": w.N, "dtype": w.dtype, "gemma": w.gemma,
           "dx_in_place": w.dx_in_place, "partial_rows": path.partial_rows, "rotated_sets": sets,
           "protocol": f"median of {samples} samples x {CALLS} back-to-back calls; in place: dy restored "
                       "before each sample, outside the events"}
    legs = {"fwd": (path.fwd, b["fwd"]), "bwd": (path.bwd, b["bwd"]), "step": (path.step, b["fwd_bwd"])}
    for mode in ("hot", "flushed"):
        res = {}
        for leg, (fn, nbytes) in legs.items():
            f = fn if mode == "flushed" else (lambda k, fn=fn: fn(0))
            t = time_calls(f, samples, before_sample=path.restore if w.dx_in_place else None)
            res[leg] = {"us": round(t["median_s"] * 1e6, 2), "min_us": round(t["min_s"] * 1e6, 2),
                        "gbps": round(nbytes / t["median_s"] / 1e9, 1),
                        "pct_of_peak": round(100 * nbytes / t["median_s"] / 1e9 / PEAK_HBM_GBPS, 2),
                        "rows_per_s": round(w.M / t["median_s"], 1)}
        out[mode] = res
    print(f"[config] {w.name}: hot step {out['hot']['step']['us']} us ({out['hot']['step']['pct_of_peak']} %), "
          f"flushed {out['flushed']['step']['us']} us", file=sys.stderr, flush=True)
    del path
    torch.cuda.empty_cache()
    return out


def copy_reference(nbytes: int, steps: int) -> float:
    """GB/s of a plain device-to-device copy (read + write counted) of nbytes."""
    a = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(steps):
        b.copy_(a)
    e.record()
    torch.cuda.synchronize()
    t = s.elapsed_time(e) * 1e-3 / steps
    return 2 * nbytes / t / 1e9


_ORACLE_SAMPLE = None


def _oracle_sample_init(w: wl.Workload, rows: int):
    """Pool initializer: the worker's own copy of the sample, upcast to fp64."""
    global _ORACLE_SAMPLE
    t = wl.make_inputs(w.scaled(M=rows))
    _ORACLE_SAMPLE = (w, *(wl.to_f64(t[k]) for k in ("x", "gamma", "dy")))


def _oracle_sample_pass(_=None) -> int:
    """One fwd + bwd of the oracle over the sample."""
    import oracle

    w, x, g, dy = _ORACLE_SAMPLE
    oracle.forward(x, g, w.eps, w.gemma)
    oracle.backward(x, g, dy, w.eps, w.gemma)
    return 1


def oracle_all_cores(w: wl.Workload, rows: int, seconds: float) -> dict:
    """The same oracle sample, row-sharded over the host's cores.

    One process per core (at most 16), each holding its own copy of the
    sample; the timed region covers whole batches of one pass per worker
    after every worker has done one untimed pass.  Workers are spawned (not
    forked), so they share no state with this process's HIP runtime.
    """
    import multiprocessing as mp

    k = max(1, min(len(os.sched_getaffinity(0)), 16))
    with mp.get_context("spawn").Pool(k, initializer=_oracle_sample_init, initargs=(w, rows)) as pool:
        pool.map(_oracle_sample_pass, range(k), chunksize=1)
        passes, t0 = 0, time.perf_counter()
        while True:
            passes += sum(pool.map(_oracle_sample_pass, range(k), chunksize=1))
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    nbytes = wl.algorithmic_bytes(rows, w.N, w.elsize)["fwd_bwd"] * passes
    return {"value": nbytes / el / 1e9, "unit": "GB/s", "cores": k, "kind": "oracle",
            "sample": f"{passes} passes of fwd+bwd over {rows} rows x N={w.N}, {k} worker processes, "
                      f"{el:.1f} s"}


def device_info() -> dict:
    """Name, compute units, and the clocks and memory bus width the HIP runtime reports."""
    import ctypes

    props = torch.cuda.get_device_properties(0)
    out = {"name": props.name, "arch": getattr(props, "gcnArchName", None), "cus": props.multi_processor_count}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        return out

    def attr(code: int):
        v = ctypes.c_int(0)
        return v.value if hip.hipDeviceGetAttribute(ctypes.byref(v), code, 0) == 0 else None

    # hipDeviceAttribute_t codes of ROCm 7's hip_runtime_api.h: ClockRate,
    # MemoryBusWidth, MemoryClockRate (clocks in kHz)
    sclk, bus, mclk = attr(5), attr(59), attr(60)
    out.update({"sclk_mhz": sclk and sclk / 1000, "mem_clock_mhz": mclk and mclk / 1000, "mem_bus_bits": bus})
    return out


def cpu_baseline(w: wl.Workload, seconds: float, all_cores_seconds: float) -> dict:
    """The fp64 oracle (as it stands) on a sample of rows of the same workload."""
    rows = min(w.M, 1024)
    _oracle_sample_init(w, rows)
    reps, t0 = 0, time.perf_counter()
    while True:
        reps += _oracle_sample_pass()
        el = time.perf_counter() - t0
        if el >= seconds and reps >= 2:
            break
    per = el / reps
    nbytes = wl.algorithmic_bytes(rows, w.N, w.elsize)["fwd_bwd"]
    out = {"value": nbytes / per / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"{rows} of {w.M} rows x N={w.N} ({w.dtype} inputs upcast to fp64), fwd+bwd repeated {reps}x "
                     f"in {el:.1f} s; numpy elementwise ops, single thread; {per * 1e3:.1f} ms per sample",
           "host_cpus_visible": len(os.sched_getaffinity(0))}
    out["all_cores"] = None
    if all_cores_seconds > 0:
        try:
            out["all_cores"] = oracle_all_cores(w, rows, all_cores_seconds)
        except Exception as e:  # a host without process spawning still gets the one-core figure
            out["all_cores"] = {"error": f"{type(e).__name__}: {e}"}
    return out


CEILING_PROBE = os.path.join(ROOT, "tests", "native", "bin", "stream_ceiling")
CEILING_MIXES = ("read", "read1_write1", "read2_write1", "read2_write1_in_place", "read3_write3")


def stream_ceiling():
    """GB/s of plain streaming kernels (16-byte nontemporal vectors, 256 MiB per
    operand) for the read/write mixes of the row kernels: read only, one read
    per write, two reads per write, and two reads per write in place (dx over
    dy), each the best over grid-stride and row-walk shapes, both cache
    policies, and three reads with three writes (the SwiGLU backward)
    (tests/native/stream_ceiling.hip).  Run as a
    child process before this process touches the GPU.  None if the probe has
    not been built."""
    import subprocess

    if not os.path.exists(CEILING_PROBE):
        print(f"[ceiling] {CEILING_PROBE} not built; skipped", file=sys.stderr, flush=True)
        return None
    r = subprocess.run([CEILING_PROBE], capture_output=True, text=True, timeout=180)
    if r.returncode != 0:
        print(f"[ceiling] probe failed ({r.returncode}): {r.stderr.strip()[-300:]}", file=sys.stderr, flush=True)
        return None
    res = json.loads(r.stdout.strip().splitlines()[-1])
    print(f"[ceiling] {res}", file=sys.stderr, flush=True)
    # the JSON line keeps the three fastest shapes of each mix; the probe itself lists all
    for mix in CEILING_MIXES:
        shapes = res[mix].pop("hot_gbps_by_shape", {})
        res[mix]["top_hot_shapes"] = dict(sorted(shapes.items(), key=lambda kv: -kv[1])[:3])
        res[mix]["shapes_timed"] = len(shapes)
    return res


# ---------------------------------------------------------------------------
# Counter collection.  `--counter-pass MANIFEST` launches a fixed sequence
# (COUNTER_CALLS launches of each kernel of each workload: the five RMSNorm
# workloads, every point of the LayerNorm sweep, its unit-test shape, a wide
# LayerNorm shape, RoPE and SwiGLU; then a plain copy
# of COPY_BYTES for calibration) under rocprofv3 --pmc, one counter set per
# run, and writes the sequence to MANIFEST; `--summarize-counters DIR` then
# attributes the dispatches of DIR/{fetch,write,lds}/*counter_collection.csv
# to it in launch order and prints the summary committed under profiles/.
# ---------------------------------------------------------------------------
COUNTER_CALLS = 3
COPY_BYTES = 256 << 20
COPY_KERNEL = "elementwise_kernel"  # torch.neg(a, out=b): reads a, writes b
LDS_COUNTERS = ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS", "SQ_INSTS_VALU", "SQ_INSTS_VMEM_RD",
                "SQ_INSTS_VMEM_WR", "SQ_WAVES", "GRBM_GUI_ACTIVE")


def counter_workloads() -> list:
    """(label prefix, kind, workload) of the counter pass, in launch order."""
    out = [(f"rms {k}", "rms", wl.RMS_WORKLOADS[k]) for k in ("c1", "c2", "c3", "c4", "c5")]
    out += [(f"ln {n}", "ln", wl.ln_sweep(n)) for n in wl.LN_SWEEP_NS]
    out.append(("ln unit-test", "ln", wl.LN1))
    out.append(("ln wide", "ln", wl.ln_sweep(8192).scaled(N=32768, name="ln_f16_4096x32768",
                                                             note="16-bit rows beyond 16384 (wide kernels)")))
    return out


def counter_pass(manifest: str) -> None:
    import row_normalization_amd as rn

    entries = []

    def launch(label, kernel, fn, nbytes, scratch=0, workload="", elements=0):
        for _ in range(COUNTER_CALLS):
            fn()
        torch.cuda.synchronize()
        entries.append({"label": label, "kernel": kernel, "calls": COUNTER_CALLS, "algorithmic_bytes": int(nbytes),
                        "scratch_bytes": int(scratch), "workload": workload, "elements": int(elements)})
        print(f"[counters] {label}", file=sys.stderr, flush=True)

    for prefix, kind, w in counter_workloads():
        if kind == "rms":
            path = Path(w)  # its set-up runs one backward row pass
            b = wl.algorithmic_bytes(w.M, w.N, w.elsize)
            part = path.partial_rows * w.N * 4
            launch(f"{prefix} fwd", "rmsnorm_fwd_kernel", path.fwd, b["fwd"], 0, w.name, w.M * w.N)
            launch(f"{prefix} bwd_rows", "rmsnorm_bwd_rows_kernel", path.bwd_rows, b["bwd_rows"], part, w.name,
                   w.M * w.N)
            launch(f"{prefix} reduce", "rmsnorm_dgamma_reduce_kernel", path.reduce, 4 * w.N, part, w.name)
        else:
            path = LnPath(w)
            b = wl.ln_algorithmic_bytes(w.M, w.N, w.elsize)
            wide = w.N > 16384  # 16-bit rows beyond the register plans
            launch(f"{prefix} fwd", "layernorm_fwd_wide_kernel" if wide else "layernorm_fwd_kernel", path.fwd,
                   b["fwd"], 0, w.name, w.M * w.N)
            path.bwd_rows()  # the partial-row count, before the counted launches
            torch.cuda.synchronize()
            part = 2 * path.partial_rows * w.N * 4
            # wide rows in 16-byte vectors (dense, N a multiple of 8) take the held-row kernel
            bwd_kernel = ("layernorm_bwd_wide_held_kernel" if w.N % 8 == 0 else "layernorm_bwd_wide_kernel") if wide \
                else "layernorm_bwd_rows_kernel"
            launch(f"{prefix} bwd_rows", bwd_kernel, path.bwd_rows, b["bwd_rows"], part, w.name, w.M * w.N)
            launch(f"{prefix} reduce", "rmsnorm_dgamma_reduce_kernel", path.reduce, 8 * w.N, part, w.name)
        del path
        torch.cuda.empty_cache()

    r = wl.ROPE1
    t = wl.make_rope_inputs(r)
    q, cos, sin, pos = t["q"].cuda(), t["cos"].cuda(), t["sin"].cuda(), t["positions"].cuda()
    L, stream = rn.lib(), torch.cuda.current_stream().cuda_stream
    args = (q.data_ptr(), r.tokens, r.heads, r.head_dim, r.heads * r.head_dim, cos.data_ptr(), sin.data_ptr(),
            r.seq_len, pos.data_ptr(), r.seq_len, DTYPE_CODE[r.dtype], stream)
    nb = wl.rope_algorithmic_bytes(r.tokens, r.heads, r.head_dim, r.elsize, r.seq_len)
    launch("rope fwd", "rope_kernel", lambda: L.rope_fwd(*args), nb, 0, r.name)
    launch("rope bwd", "rope_kernel", lambda: L.rope_bwd(*args), nb, 0, r.name)
    del q, cos, sin, pos, t

    g = wl.SWIGLU1
    t = wl.make_swiglu_inputs(g)
    e, gg, dh = (t[k].cuda() for k in ("e", "g", "dh"))
    h, df, de = (torch.empty_like(e) for _ in range(3))
    code = DTYPE_CODE[g.dtype]
    b = wl.swiglu_algorithmic_bytes(g.M, g.N, g.elsize)
    launch("swiglu fwd", "swiglu_fwd_kernel",
           lambda: L.swiglu_fwd(e.data_ptr(), gg.data_ptr(), h.data_ptr(), g.M, g.N, g.N, code, stream), b["fwd"], 0,
           g.name)
    launch("swiglu bwd", "swiglu_bwd_kernel",
           lambda: L.swiglu_bwd(dh.data_ptr(), e.data_ptr(), gg.data_ptr(), h.data_ptr(), df.data_ptr(),
                                de.data_ptr(), g.M, g.N, g.N, code, stream), b["bwd"], 0, g.name)
    del e, gg, dh, h, df, de, t
    torch.cuda.empty_cache()

    a = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    c = torch.empty_like(a)
    launch("copy", COPY_KERNEL, lambda: torch.neg(a, out=c), 2 * COPY_BYTES, 0, f"{COPY_BYTES >> 20} MiB bf16 negation")
    with open(manifest, "w") as f:
        json.dump({"kernel_sha": kernel_hash(), "entries": entries}, f, indent=1)


def _dispatches(csv_dir: str) -> list:
    """[(dispatch id, kernel name, grid, workgroup, {counter: value})] of the
    counter_collection.csv under csv_dir, in dispatch order."""
    import csv
    import glob

    files = glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True)
    if len(files) != 1:
        raise SystemExit(f"expected one counter_collection.csv under {csv_dir}, found {files}")
    rows = {}
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            d = rows.setdefault(int(r["Dispatch_Id"]), [r["Kernel_Name"], int(r["Grid_Size"]),
                                                        int(r["Workgroup_Size"]), {}])
            d[3][r["Counter_Name"]] = float(r["Counter_Value"])
    return [(k, *rows[k]) for k in sorted(rows)]


def _attribute(entries: list, dispatches: list) -> list:
    """For each manifest entry, its `calls` dispatches: the next ones in
    dispatch order whose kernel name matches (other launches are skipped)."""
    out, i = [], 0
    for e in entries:
        got = []
        while len(got) < e["calls"]:
            if i >= len(dispatches):
                raise SystemExit(f"ran out of dispatches looking for {e['label']} ({e['kernel']})")
            if e["kernel"] in dispatches[i][1]:
                got.append(dispatches[i])
            i += 1
        out.append(got)
    return out


def summarize_counters(d: str) -> None:
    """Print the markdown counter summary of the runs under d (see above)."""
    man = json.load(open(os.path.join(d, "manifest.json")))
    entries = man["entries"]
    per = {}
    for run in ("fetch", "write", "lds"):
        if os.path.isdir(os.path.join(d, run)):
            per[run] = _attribute(entries, _dispatches(os.path.join(d, run)))
    med = lambda run, k, c: float(np.median([x[4][c] for x in per[run][k]]))
    copy = next(k for k, e in enumerate(entries) if e["label"] == "copy")
    half = COPY_BYTES
    f_scale = half / (med("fetch", copy, "FETCH_SIZE") * 1024)
    w_scale = half / (med("write", copy, "WRITE_SIZE") * 1024)
    table = {}
    lines = []
    for k, e in enumerate(entries):
        fetch_kib, write_kib = med("fetch", k, "FETCH_SIZE"), med("write", k, "WRITE_SIZE")
        rd, wr = fetch_kib * 1024 * f_scale, write_kib * 1024 * w_scale
        need = e["algorithmic_bytes"] + e["scratch_bytes"]
        grid, wg = per["fetch"][k][0][2], per["fetch"][k][0][3]
        elems = e.get("elements", 0)
        row = {"kernel": e["kernel"], "workload": e["workload"], "grid": grid, "workgroup": wg,
               "fetch_kib": round(fetch_kib, 1), "write_kib": round(write_kib, 1), "scaled_bytes": int(rd + wr),
               "algorithmic_bytes": e["algorithmic_bytes"], "scratch_bytes": e["scratch_bytes"],
               "ratio": round((rd + wr) / need, 4),
               "bytes_per_element": round((rd + wr) / elems, 3) if elems else None}
        if "lds" in per:
            for c in ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS", "SQ_WAVES"):
                row[c] = med("lds", k, c)
        table[e["label"]] = row
        bpe = f"{row['bytes_per_element']:.2f}" if row["bytes_per_element"] else "-"
        lines.append(f"| {e['label']} | {e['kernel']} | {grid} / {wg} | {fetch_kib:.1f} | "
                     f"{write_kib:.1f} | {rd / 1e6:.2f} | {wr / 1e6:.2f} | {e['algorithmic_bytes'] / 1e6:.2f} | "
                     f"{e['scratch_bytes'] / 1e6:.2f} | {(rd + wr) / need:.3f} | {bpe} | "
                     + (" | ".join(f"{row[c]:.0f}" for c in ("SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE",
                                                               "SQ_INSTS_LDS")) if "lds" in per else "- | - | -")
                     + " |")
    print("| Launch | Kernel | Grid / workgroup (threads) | FETCH_SIZE (KiB) | "
          "WRITE_SIZE (KiB) | Read (MB) | Written (MB) | Algorithmic (MB) | Scratch (MB) | "
          "Moved / (algorithmic + scratch) | Moved bytes per element | SQ_LDS_BANK_CONFLICT | SQ_LDS_IDX_ACTIVE | "
          "SQ_INSTS_LDS |")
    print("|---|---|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|")
    print("\n".join(lines))
    print()
    print(f"Calibration: the copy reads and writes {COPY_BYTES} bytes; read bytes = FETCH_SIZE x 1024 x "
          f"{f_scale:.4f}, written bytes = WRITE_SIZE x 1024 x {w_scale:.4f}.")
    print()
    print("```json")
    print(json.dumps({"kernel_sha": man["kernel_sha"], "fetch_scale": round(f_scale, 5),
                      "write_scale": round(w_scale, 5), "entries": table}))
    print("```")


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): this path is measured on a single MI355X; "
              "multi-GPU sharding is described in the design notes, not run.", file=sys.stderr)
        sys.exit(2)
    # before torch initialises the GPU in this process
    ceiling = None if args.no_ceiling or args.counter_pass else stream_ceiling()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    import row_normalization_amd as rn

    if not os.path.exists(rn.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()
    torch.cuda.set_device(0)
    if args.counter_pass:
        counter_pass(args.counter_pass)
        return
    w = wl.RMS_WORKLOADS[args.workload]
    path = Path(w)
    overlapped = OverlappedSteps(path)
    schedules = {"overlapped_reduce": (overlapped.step, overlapped.join), "one_stream": (path.step, None)}
    step, join = schedules[args.schedule]
    for k in range(max(args.warmup, 1)):
        step(k)
    # then untimed steps until the clocks have settled (a short --warmup alone
    # leaves the timed steps inside the start-up ramp)
    settle_steps = settle(step)
    if join:
        join()
    torch.cuda.synchronize()

    t0 = time.perf_counter()
    sec_per_step = time_steps(step, args.steps, join)
    wall = time.perf_counter() - t0
    # the other schedule, for context: the same number of steps after its own settle
    other = "one_stream" if args.schedule == "overlapped_reduce" else "overlapped_reduce"
    o_step, o_join = schedules[other]
    settle(o_step)
    if o_join:
        o_join()
    sec_other = time_steps(o_step, args.steps, o_join)
    kern = {name: time_calls(fn, args.samples)
            for name, fn in (("fwd", path.fwd), ("bwd_rows", path.bwd_rows), ("dgamma_reduce", path.reduce))}

    b = wl.algorithmic_bytes(w.M, w.N, w.elsize)
    value = b["fwd_bwd"] / sec_per_step / 1e9
    t_rows = kern["bwd_rows"]["median_s"]
    achieved = b["bwd_rows"] / t_rows / 1e9
    h = kernel_hash()
    traffic_tab = traffic_table(h)
    traffic = traffic_tab.get(f"rms {args.workload} bwd_rows")
    copy_gbps = copy_reference(256 << 20, 50)
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle_steps,
        "ms_per_step": round(sec_per_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "gemma": w.gemma, "dx_in_place": w.dx_in_place,
                   "eps": w.eps, "io_dtype": w.dtype, "math": "fp32", "schedule": args.schedule},
        "pct_of_peak": round(100 * value / PEAK_HBM_GBPS, 2),
        "rows_per_s": round(w.M / sec_per_step, 1),
        "bytes_per_step": b["fwd_bwd"],
        "wall_s_timed": round(wall, 4),
        "schedules_ms_per_step": {args.schedule: round(sec_per_step * 1e3, 4), other: round(sec_other * 1e3, 4)},
        "kernels_us": {k: round(v["median_s"] * 1e6, 2) for k, v in kern.items()},
        "kernels_protocol": f"median of {args.samples} samples x {CALLS} back-to-back launches of the kernel alone",
        "kernels_gbps": {"fwd": round(b["fwd"] / kern["fwd"]["median_s"] / 1e9, 1),
                         "bwd_rows": round(achieved, 1),
                         "bwd": round(b["bwd"] / (kern["bwd_rows"]["median_s"] + kern["dgamma_reduce"]["median_s"])
                                      / 1e9, 1)},
        "partial_rows": path.partial_rows,
        "copy_ref_gbps": round(copy_gbps, 1),
        "roofline": {"bound": "hbm", "kernel": "rmsnorm_bwd_rows_kernel", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic, "algorithmic_bytes": b["bwd_rows"], "kernel_sha": h},
        "device": device_info(),
        "stream_ceiling": ceiling,
        "kernels_vs_ceiling": None if not ceiling else {
            "fwd": round(b["fwd"] / kern["fwd"]["median_s"] / 1e9 / ceiling["read1_write1"]["hot_gbps"], 4),
            "bwd_rows": round(achieved / ceiling["read2_write1"]["hot_gbps"], 4),
            "bwd_rows_vs_in_place": (round(achieved / ceiling["read2_write1_in_place"]["hot_gbps"], 4)
                                     if "read2_write1_in_place" in ceiling else None)},
    }
    del overlapped, path, schedules
    torch.cuda.empty_cache()
    out["configs"] = None if args.no_configs else {k: config_protocol(wl.RMS_WORKLOADS[k], args.samples)
                                                  for k in args.configs}
    out["layernorm"] = None if args.no_layernorm else layernorm_sweep(args.ln_samples, args.ln_ns)
    # calibrated HBM bytes per launch from the committed counter summary (None
    # where it holds no such launch or was taken on other kernel sources)
    for k, c in (out["configs"] or {}).items():
        c["traffic_bytes"] = {leg: traffic_tab.get(f"rms {k} {leg}") for leg in ("fwd", "bwd_rows", "reduce")}
    for pt in (out["layernorm"] or {}).get("points", []):
        pt["traffic_bytes"] = {leg: traffic_tab.get(f"ln {pt['N']} {leg}") for leg in ("fwd", "bwd_rows", "reduce")}
    for pt in (out["layernorm"] or {}).get("wide", {}).get("points", []):
        # the counter pass covers the 4096 x 32768 wide shape
        pt["traffic_bytes"] = {leg: traffic_tab.get(f"ln wide {leg}") if pt["N"] == 32768 else None
                               for leg in ("fwd", "bwd_rows", "reduce")}
    if args.no_elementwise:
        out["rope"] = out["swiglu"] = None
    else:
        out["rope"] = rope_leg(args.samples)
        out["rope"]["traffic_bytes"] = {leg: traffic_tab.get(f"rope {leg}") for leg in ("fwd", "bwd")}
        print(f"[rope] {out['rope']}", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
        out["swiglu"] = swiglu_leg(args.samples)
        out["swiglu"]["traffic_bytes"] = {leg: traffic_tab.get(f"swiglu {leg}") for leg in ("fwd", "bwd")}
        # each leg against the plain streaming rate of its own read/write mix
        if ceiling and "read3_write3" in ceiling:
            out["swiglu"]["vs_ceiling"] = {
                "fwd_vs_read2_write1": round(out["swiglu"]["fwd_gbps"] / ceiling["read2_write1"]["hot_gbps"], 4),
                "bwd_vs_read3_write3": round(out["swiglu"]["bwd_gbps"] / ceiling["read3_write3"]["hot_gbps"], 4)}
        print(f"[swiglu] {out['swiglu']}", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, args.cpu_all_cores_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

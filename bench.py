"""Benchmark of the in-place packed real FFT and the block-circulant layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline step: 4096 rows of p = 512, fp32, one forward and one inverse rdFFT
in place (one pass of the transform path over one batch).  Exactly W untimed
and K timed steps run.  The batch rotates over NBUF distinct copies (1 GiB in
total): step g transforms copy g mod NBUF forward and copy (g + NBUF/2) mod
NBUF back, so no step reads what the 256 MB last-level cache still holds;
every copy is resident in HBM before the timed region starts.  `value` =
algorithmic bytes (every row read once and written once, per transform) /
wall time of the K steps.

The JSON line also carries
  roofline      the forward kernel: algorithmic bytes per launch / its mean
                duration per launch in the timed region (HIP events around
                each run of back-to-back forward launches, on the launch
                stream, created without the system-scope fence a default
                event makes), against 8 TB/s HBM; beside it the average duration
                of the same dispatches in the committed kernel-trace summary;
  cpu_baseline  the fp64 oracle (numpy) on all host cores (up to 16) and on
                one thread, each on a bounded sample of the same workload, in
                the same unit;
  extra         the other transform sizes and the block-circulant layer
                workloads (tokens/s), each against its own roofline.
"""

from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import block_circulant_layers_amd as bcl  # noqa: E402
from block_circulant_layers_amd import synthetic as syn  # noqa: E402

IO_NAME = {"f32": "F32Io", "bf16": "Bf16Io", "f16": "F16Io"}
METRIC = "rdFFT GB/s + % HBM peak (p=512,4096); circulant fwd+bwd tokens/s"
HBM_PEAK_GBS = 8000.0
VALU_FP32_PEAK_TFS = 157.3
ROTATE_BYTES = 1 << 30
# timed regions of at most this many launches are queued as plain launches
MAX_QUEUED_LAUNCHES = 1024
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "block_circulant_layers_amd", "csrc")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


TRANSFORM_SOURCES = ("rdfft_device.hpp", "rdfft_kernels.hpp", "gen_twiddles.py")


def kernel_source_hash() -> str:
    """Hash of the transform kernels' sources; traffic figures taken from
    counters are only reported while the kernels they were measured on are
    unchanged."""
    h = hashlib.sha256()
    for name in TRANSFORM_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as fh:
            h.update(name.encode() + fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel_key: str):
    """HBM bytes per launch from the committed counter summary, or None."""
    path = os.path.join(PROFILES, "traffic.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m = re.search(r"source_hash:\s*(\w+)", txt)
    if not m or m.group(1) != kernel_source_hash():
        return None
    # table columns: kernel workload | dispatches | FETCH | WRITE | scaled bytes per launch | ...
    for line in txt.splitlines():
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) >= 5 and cells[0] == kernel_key:
            return float(cells[4])
    return None


def recorded_trace_ms(kernel: str):
    """The headline kernel's average duration (ms) over the timed region's
    dispatches in the committed kernel-trace summary of bench.py, or None when
    that summary was taken on other transform sources."""
    path = os.path.join(PROFILES, "kernel_trace_bench_default.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m = re.search(r"source_hash:\s*(\w+)", txt)
    if not m or m.group(1) != kernel_source_hash():
        return None
    want = kernel.replace(" ", "")
    for line in txt.split("timed region's dispatches only")[-1].splitlines():
        cells = [c.strip().strip("`") for c in line.strip().strip("|").split("|")]
        if len(cells) >= 3 and cells[0].replace(" ", "") == want:
            return float(cells[2]) * 1e-3
    return None


class Timer:
    """Events on the stream the kernels are launched on (torch's current stream)."""

    def __init__(self):
        self.a = torch.cuda.Event(enable_timing=True)
        self.b = torch.cuda.Event(enable_timing=True)

    def start(self):
        self.a.record()

    def stop(self) -> float:
        self.b.record()
        self.b.synchronize()
        return self.a.elapsed_time(self.b)


class MarkEvent:
    """A timing marker inside a timed region: a HIP event created with
    hipEventDisableSystemFence, recorded on torch's current stream.  A
    default event makes a system-scope memory fence when it is recorded (cache
    writeback and invalidation, which the HIP headers name as a cost on some
    AMD GPUs); measured on MI355X, three such markers inside 20 steps of the
    4096x512 fp32 forward + inverse added 0.75 us per step (10.45 against 9.65
    us with events only at the region's borders), and the markers' forward
    duration read 4.9 against 4.7 us.  Markers without the fence measure the
    launches between them and add nothing measurable.  The region's borders
    stay default events (Timer), and the results are read only after a full
    device synchronisation.  Where the runtime refuses the flag, the markers
    fall back to default events (MarkEvent.kind says which)."""

    _hip = None
    kind = None
    FLAG = 0x20000000  # hipEventDisableSystemFence

    @classmethod
    def _runtime(cls):
        if cls._hip is None:
            import ctypes

            # the HIP runtime torch has loaded (one runtime per process)
            hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = hip
        return cls._hip

    def __init__(self):
        import ctypes

        self.ev = None
        self.fallback = None
        if MarkEvent.kind != "default":
            hip = self._runtime()
            e = ctypes.c_void_p()
            if hip.hipEventCreateWithFlags(ctypes.byref(e), self.FLAG) == 0:
                self.ev = e
                MarkEvent.kind = "no system fence"
            else:
                MarkEvent.kind = "default"
        if self.ev is None:
            self.fallback = torch.cuda.Event(enable_timing=True)

    def record(self):
        if self.fallback is not None:
            self.fallback.record()
            return
        import ctypes

        st = self._hip.hipEventRecord(self.ev, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed: {st}")

    def elapsed_time(self, end: "MarkEvent") -> float:
        """Milliseconds from this marker to ``end`` (waits for ``end``)."""
        if self.fallback is not None:
            return self.fallback.elapsed_time(end.fallback)
        import ctypes

        ms = ctypes.c_float()
        if self._hip.hipEventSynchronize(end.ev) != 0 or \
                self._hip.hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def __del__(self):
        if self.ev is not None and self._hip is not None:
            self._hip.hipEventDestroy(self.ev)


_SLEEP_CYCLES_PER_MS = None


def hold_gpu(ms: float) -> None:
    """Keep the current stream busy for about ``ms`` milliseconds with torch's
    bounded spin kernel, so that the host queues the launches that follow
    before the GPU reaches them: events recorded after it then time GPU
    execution, not the host's launch rate."""
    global _SLEEP_CYCLES_PER_MS
    if _SLEEP_CYCLES_PER_MS is None:
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        torch.cuda._sleep(1_000_000)
        b.record()
        b.synchronize()
        _SLEEP_CYCLES_PER_MS = 1_000_000 / max(a.elapsed_time(b), 1e-3)
    torch.cuda._sleep(int(_SLEEP_CYCLES_PER_MS * ms))


# ---------------------------------------------------------------------------
# packed transform workloads
# ---------------------------------------------------------------------------


def _graph(fn):
    """Capture fn() (a sequence of library launches) into a HIP graph."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replayer(fn, eager):
    """fn's launches as one callable: replays of a HIP graph of them, or (eager)
    fn itself, so that a counter profiler sees ordinary dispatches."""
    if eager:
        return fn
    return _graph(fn).replay


def step_runs(g0, n, chunk):
    """Split the global steps [g0, g0 + n) into runs that never cross a
    multiple of ``chunk``: [(first step, length), ...]."""
    runs, g = [], g0
    while g < g0 + n:
        m = min(g0 + n, (g // chunk + 1) * chunk) - g
        runs.append((g, m))
        g += m
    return runs


def bench_rdfft(rows, p, dtype, steps, warmup, workload, index=0, eager=False):
    """Exactly ``warmup`` untimed and ``steps`` timed steps of one forward and
    one inverse transform in place, each on a 1 GiB rotation of nbuf copies of
    one batch: step g runs the forward on buffer g mod nbuf and the inverse on
    buffer (g + nbuf/2) mod nbuf, so a buffer's forward and its inverse are
    nbuf/2 steps (1 GiB of traffic) apart and neither reads from a cache.
    Steps run in runs of up to nbuf/2: the run's forwards, then its
    inverses, with events between them, giving the mean duration of a forward
    and of an inverse launch in the timed region.  A bounded spin kernel holds
    the GPU while the host queues the timed region, so the events time
    back-to-back GPU execution.  Timed regions of up to MAX_QUEUED_LAUNCHES
    launches are queued as plain launches; longer ones replay HIP graphs
    (cached per run position, all captured before the timed region), which
    cost about 10 us of GPU time per graph launch."""
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    eb = 4 if dtype == "f32" else 2
    nbytes = rows * p * eb
    nbuf = max(2, ROTATE_BYTES // nbytes)
    nbuf -= nbuf % 2
    half = nbuf // 2
    chunk = half
    base = syn.torch_normal((rows, p), workload, syn.T_X, index, dtype=tdt)
    bufs = [base.clone() for _ in range(nbuf)]
    graphs = {}
    # a short timed region is queued as plain launches behind the spin kernel
    # (no per-graph launch cost); a long one replays cached graphs
    queued = eager or 2 * steps <= MAX_QUEUED_LAUNCHES

    def run_fns(g, n, plain=False):
        fwd = lambda g=g, n=n: [bcl.rdfft_forward(bufs[(g + i) % nbuf]) for i in range(n)]  # noqa: E731
        inv = lambda g=g, n=n: [bcl.rdfft_inverse(bufs[(g + half + i) % nbuf]) for i in range(n)]  # noqa: E731
        if plain:
            return fwd, inv
        key = (g % nbuf, n)
        if key not in graphs:
            graphs[key] = (_replayer(fwd, False), _replayer(inv, False))
        return graphs[key]

    warm_runs = step_runs(0, warmup, chunk)
    timed_runs = step_runs(warmup, steps, chunk)
    if not queued:  # capture every run's graphs before anything is timed
        for g, n in warm_runs + timed_runs:
            run_fns(g, n)
    for g, n in warm_runs:
        f, i = run_fns(g, n, plain=queued)
        f()
        i()
    torch.cuda.synchronize()
    ev = [[MarkEvent() for _ in range(3)] for _ in timed_runs]
    tm = Timer()
    torch.cuda.synchronize()
    # hold the GPU while the host queues the timed region
    hold_gpu(2.0 + (0.04 * 2 * steps if queued else 0.15 * len(timed_runs)))
    tm.start()
    for (g, n), e in zip(timed_runs, ev):
        f, i = run_fns(g, n, plain=queued)
        e[0].record()
        f()
        e[1].record()
        i()
        e[2].record()
    ms = tm.stop()
    torch.cuda.synchronize()
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / max(1, steps)
    inv_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / max(1, steps)
    # a buffer that has had as many forwards as inverses holds its input again
    total = warmup + steps
    drift = None
    for b in range(nbuf):
        nops = sum(1 for g in range(total) if g % nbuf == b) + sum(1 for g in range(total) if (g + half) % nbuf == b)
        if nops % 2 == 0:
            drift = float((bufs[b].float() - base.float()).abs().max() / base.float().abs().max())
            break
    step_bytes = 2 * 2 * nbytes  # forward + inverse, each reads and writes every row once
    del bufs, graphs, base
    torch.cuda.empty_cache()
    return {
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": ms / max(1, steps),
        "gbs": step_bytes / (ms / max(1, steps)) / 1e6,
        "bytes_per_launch": 2 * nbytes,
        "fwd_ms": fwd_ms,
        "inv_ms": inv_ms,
        "nbuf": nbuf,
        "queued": queued,
        "roundtrip_drift": drift,
    }


def bench_spectrum(rows, p, steps, warmup):
    """rdfft_unpack then rdfft_pack over a rotating set: GB/s of each (bytes =
    packed rows read or written + complex bins written or read)."""
    nbytes = rows * p * 4
    nbuf = max(2, ROTATE_BYTES // (2 * nbytes))
    zs = [syn.torch_normal((rows, p), syn.WL_TEST, syn.T_X, i) for i in range(nbuf)]
    ss = [torch.empty(rows, p // 2 + 1, 2, device="cuda") for _ in range(nbuf)]
    out = {}
    for name, fn in (("unpack", lambda: [bcl.rdfft_unpack(z, s) for z, s in zip(zs, ss)]),
                     ("pack", lambda: [bcl.rdfft_pack(s, z) for z, s in zip(zs, ss)])):
        g = _replayer(fn, False)
        for _ in range(max(1, -(-warmup // nbuf))):
            g()
        reps = max(1, -(-steps // nbuf))
        tm = Timer()
        torch.cuda.synchronize()
        tm.start()
        for _ in range(reps):
            g()
        us = tm.stop() * 1e3 / (reps * nbuf)
        moved = nbytes + rows * (p + 2) * 4
        out[name] = {"us": round(us, 3), "gbs": round(moved / us / 1e3, 1)}
    del zs, ss
    torch.cuda.empty_cache()
    return out


def bench_rdfft2d(h, w, steps, warmup):
    """2D forward then inverse in place over a rotating set of h x w fp32
    arrays; GB/s on the algorithmic bytes (each array read and written once per
    transform), although the transform makes three passes over the array."""
    nbytes = h * w * 4
    nbuf = max(2, ROTATE_BYTES // nbytes)
    bufs = [syn.torch_normal((h, w), syn.WL_RDFFT_LARGE, syn.T_X, 50 + i) for i in range(nbuf)]
    gf = _replayer(lambda: [bcl.rdfft2d_forward(b) for b in bufs], False)
    gi = _replayer(lambda: [bcl.rdfft2d_inverse(b) for b in bufs], False)
    for _ in range(max(1, -(-warmup // nbuf))):
        gf()
        gi()
    reps = max(1, -(-steps // nbuf))
    ev = [[MarkEvent() for _ in range(3)] for _ in range(reps)]
    torch.cuda.synchronize()
    for r in range(reps):
        ev[r][0].record()
        gf()
        ev[r][1].record()
        gi()
        ev[r][2].record()
    torch.cuda.synchronize()
    fwd = sum(e[0].elapsed_time(e[1]) for e in ev) / (reps * nbuf)
    inv = sum(e[1].elapsed_time(e[2]) for e in ev) / (reps * nbuf)
    del bufs
    torch.cuda.empty_cache()
    return {"fwd_ms": round(fwd, 5), "inv_ms": round(inv, 5),
            "fwd_gbs_algorithmic": round(2 * nbytes / (fwd * 1e-3) / 1e9, 1),
            "inv_gbs_algorithmic": round(2 * nbytes / (inv * 1e-3) / 1e9, 1)}


def _stream_lib():
    import ctypes

    from block_circulant_layers_amd import build

    if not os.path.exists(build.PROBE_LIB):
        raise RuntimeError(f"{build.PROBE_LIB} is not built: run python -m block_circulant_layers_amd.build")
    lib = ctypes.CDLL(build.PROBE_LIB)
    lib.stream_probe.restype = ctypes.c_int
    lib.stream_probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                 ctypes.c_void_p]
    return lib


def bench_stream(nbytes, launches=512):
    """The in-place streaming pass of libstreamprobe.so (every float read once
    and written back once, scaled by 1: an in-place transform's HBM traffic
    with none of its arithmetic) over a 1 GiB rotation of nbytes buffers, for
    both cache policies and a few grid sizes.  Reported per policy: the mean
    time per launch of graph-replayed back-to-back launches, best grid."""
    lib = _stream_lib()
    n = nbytes // 4
    nbuf = max(2, ROTATE_BYTES // nbytes)
    bufs = [torch.zeros(n, device="cuda") for _ in range(nbuf)]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    chunks = -(-n // 4096)
    stream = lambda: torch.cuda.current_stream().cuda_stream  # noqa: E731
    out = {}
    for policy, name in ((0, "default_policy"), (1, "non_temporal")):
        best = None
        for grid in sorted({min(chunks, cus * r) for r in (2, 4, 8)} | {chunks}):
            def launch_all(grid=grid, policy=policy):
                for b in bufs:
                    if lib.stream_probe(b.data_ptr(), n, grid, policy, 1.0, stream()) != 0:
                        raise RuntimeError("stream_probe failed")
            g = _graph(launch_all)
            g.replay()
            reps = max(1, -(-launches // nbuf))
            tm = Timer()
            torch.cuda.synchronize()
            hold_gpu(1.0)
            tm.start()
            for _ in range(reps):
                g.replay()
            us = tm.stop() * 1e3 / (reps * nbuf)
            del g
            if best is None or us < best["us_per_launch"]:
                best = {"grid": grid, "us_per_launch": round(us, 3),
                        "pct_hbm_peak": round(100 * 2 * nbytes / us / 1e3 / HBM_PEAK_GBS, 2)}
        out[name] = best
    del bufs
    torch.cuda.empty_cache()
    return out


def bench_copy(nbytes, steps, warmup):
    """A plain device copy of nbytes (torch copy_, one read and one write of
    every byte) over the same 1 GiB rotation: the practical ceiling a transform
    of the same algorithmic bytes is compared with."""
    n = nbytes // 4
    nbuf = max(2, ROTATE_BYTES // nbytes)
    bufs = [torch.zeros(n, device="cuda") for _ in range(nbuf)]
    # buffer i is read half a rotation after it was last written: out of every cache
    g = _replayer(lambda: [bufs[(i + nbuf // 2) % nbuf].copy_(bufs[i]) for i in range(nbuf)], False)
    for _ in range(max(1, -(-warmup // nbuf))):
        g()
    reps = max(1, -(-steps // nbuf))
    tm = Timer()
    torch.cuda.synchronize()
    tm.start()
    for _ in range(reps):
        g()
    us = tm.stop() * 1e3 / (reps * nbuf)
    del bufs
    torch.cuda.empty_cache()
    return {"us_per_copy": round(us, 3), "gbs": round(2 * nbytes / us / 1e3, 1),
            "pct_hbm_peak": round(100 * 2 * nbytes / us / 1e3 / HBM_PEAK_GBS, 2)}


def torch_fft_circulant(x, c, real):
    """Context only, never a product path: the block-circulant layer in the
    form its baselines take on the pages (Paper-Notes, "实验关键数据"; scime,
    "Measured effects reported in the paper"): y_i = IFFT(sum_j FFT(c_ij) *
    FFT(x_j)) on torch.fft (rocFFT on this GPU), the per-block products
    broadcast before the block sum, differentiated by autograd.  ``real``
    picks rfft/irfft, else the complex fft/ifft."""
    b = x.shape[0]
    q, k, p = c.shape
    xs = x.view(b, 1, k, p)
    if real:
        yf = (torch.fft.rfft(xs, dim=-1) * torch.fft.rfft(c, dim=-1)).sum(dim=2)
        y = torch.fft.irfft(yf, n=p, dim=-1)
    else:
        yf = (torch.fft.fft(xs, dim=-1) * torch.fft.fft(c, dim=-1)).sum(dim=2)
        y = torch.fft.ifft(yf, dim=-1).real
    return y.reshape(b, q * p)


LAYER_FORMS = {
    "rdfft_layer": lambda x, c: bcl.BlockCirculantFunction.apply(x, c),
    "torch_rfft": lambda x, c: torch_fft_circulant(x, c, True),
    "torch_fft": lambda x, c: torch_fft_circulant(x, c, False),
}


def bench_layer_memory(batch, d, p, form="rdfft_layer"):
    """Peak device memory of one block-circulant forward + backward in fp32,
    counted from an empty allocator: parameters c, their gradient, x, y, dy
    and dx (the quantities a single-layer peak-memory figure holds), and what
    the step needed beyond those tensors (workspace).  ``form`` picks this
    library's layer or one of the torch.fft forms run as context."""
    fn = LAYER_FORMS[form]
    # earlier workloads' buffers held in reference cycles (a setup dict and
    # the step closure that refers to it) must not be freed inside the count
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    c = syn.torch_normal((d // p, d // p, p), syn.WL_TEST, syn.T_C, 99, scale=1 / np.sqrt(d)).requires_grad_(True)
    x = syn.torch_normal((batch, d), syn.WL_TEST, syn.T_X, 99).requires_grad_(True)
    dy = syn.torch_normal((batch, d), syn.WL_TEST, syn.T_DY, 99)
    y = fn(x, c)
    y.backward(dy)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    held = sum(-(-t.numel() * t.element_size() // 512) * 512 for t in (c, c.grad, x, x.grad, y, dy))
    out = {"peak_mib": round(peak / 2**20, 4), "workspace_bytes": int(peak - held)}
    del c, x, dy, y
    torch.cuda.empty_cache()
    return out


def bench_layer_eager(batch, d, p, form, steps=20, warmup=3, repeats=5):
    """Milliseconds per forward + backward of one fp32 layer through autograd,
    launched eagerly (no graph), for this library's layer and the torch.fft
    forms alike; the best of ``repeats`` timed runs of ``steps`` steps (host
    launch overhead makes single runs noisy)."""
    fn = LAYER_FORMS[form]
    c = syn.torch_normal((d // p, d // p, p), syn.WL_CIRC_LAYER, syn.T_C, p, scale=1 / 64.0).requires_grad_(True)
    x = syn.torch_normal((batch, d), syn.WL_CIRC_LAYER, syn.T_X, 0).requires_grad_(True)
    dy = syn.torch_normal((batch, d), syn.WL_CIRC_LAYER, syn.T_DY, 0)
    for _ in range(warmup):
        fn(x, c).backward(dy)
    tm = Timer()
    ms = float("inf")
    for _ in range(repeats):
        torch.cuda.synchronize()
        tm.start()
        for _ in range(steps):
            fn(x, c).backward(dy)
        ms = min(ms, tm.stop() / steps)
    del c, x, dy
    torch.cuda.empty_cache()
    return round(ms, 4)


def cpu_baseline_rdfft(rows, p, seconds=10.0):
    """The fp64 oracle, unmodified, on the headline workload: first on one
    thread for about seconds / 2, then with the batch split into row chunks
    run by a pool of threads, one per host core available (at most 16; numpy
    releases the GIL inside its FFTs), for about seconds / 2."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    from oracle import rdfft_oracle as ro

    t, ref = syn.cast_like_device(syn.normal((rows, p), syn.WL_RDFFT_512, syn.T_X), "f32")
    step_bytes = 2 * 2 * rows * p * 4

    def roundtrip(block):
        ro.rdfft_inverse(ro.rdfft_forward(block))

    def timed(run):
        reps = 0
        t0 = time.perf_counter()
        while True:
            run()
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds / 2:
                return reps, el

    reps1, el1 = timed(lambda: roundtrip(ref))
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    chunks = np.array_split(ref, 4 * cores)
    with ThreadPoolExecutor(cores) as pool:
        repsn, eln = timed(lambda: list(pool.map(roundtrip, chunks)))
    return {
        "value": round(step_bytes * repsn / eln / 1e9, 3),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{repsn} x (forward + inverse) of the full {rows}x{p} fp32 batch in {len(chunks)} row chunks on "
        f"{cores} threads, float64 numpy (pocketfft), {eln:.1f} s",
        "single_thread": {
            "value": round(step_bytes * reps1 / el1 / 1e9, 3),
            "cores": 1,
            "sample": f"{reps1} x (forward + inverse) of the full batch on one thread, {el1:.1f} s",
        },
    }


# ---------------------------------------------------------------------------
# block-circulant layer workloads
# ---------------------------------------------------------------------------


def circ_algorithmic(batch, d, p, eb):
    """Bytes and flops of one forward + backward at the algorithmic minimum:
    activations x, y, x, dy, dx once each; c twice, dc once (fp32)."""
    nbytes = 5 * batch * d * eb + 3 * (d * d // p) * 4
    lp = int(np.log2(p))
    flops = 5 * batch * 2.5 * d * lp + 3 * 2.5 * (d * d / p) * lp + 3 * 4 * batch * d * d / p
    return nbytes, flops


def circ_layer_setup(batch, d, p, nrot=32, spectra=False):
    """The single-layer workload as bench_circ_layer times it: nrot token
    batches (bf16), one c (fp32), and ``rot``, a rotation of nrot training
    steps.  After a rotation ys[j] and dxs[j] hold step j's outputs and dc the
    last step's gradient.  spectra: the steps keep the weight spectra in
    cs (circulant_fwd_step writes them, circulant_bwd_spec reads them)."""
    q = k = d // p
    w = {"xs": [syn.torch_normal((batch, d), syn.WL_CIRC_LAYER, syn.T_X, i, dtype=torch.bfloat16) for i in range(nrot)],
         "dys": [syn.torch_normal((batch, d), syn.WL_CIRC_LAYER, syn.T_DY, i, dtype=torch.bfloat16)
                 for i in range(nrot)],
         "c": syn.torch_normal((q, k, p), syn.WL_CIRC_LAYER, syn.T_C, p, scale=1 / 64.0)}
    w["ys"] = [torch.empty_like(x) for x in w["xs"]]
    w["dxs"] = [torch.empty_like(x) for x in w["xs"]]
    w["dc"] = torch.empty_like(w["c"])
    w["cs"] = torch.empty_like(w["c"])

    def rot():
        # a training step of the layer: the forward clears dc in its launch,
        # the backward adds the token sum into it (two launches per step)
        for j in range(nrot):
            if spectra:
                bcl.circulant_fwd_step(w["xs"][j], w["c"], w["cs"], w["ys"][j], dc=w["dc"])
                bcl.circulant_bwd_spec(w["xs"][j], w["cs"], w["dys"][j], dx=w["dxs"][j], dc=w["dc"], accumulate=True)
            else:
                bcl.circulant_fwd_zero(w["xs"][j], w["c"], w["dc"], w["ys"][j])
                bcl.circulant_bwd_acc(w["xs"][j], w["c"], w["dys"][j], w["dc"], dx=w["dxs"][j])

    w["rot"] = rot
    return w


def bench_circ_layer(batch, d, p, steps, warmup, nrot=32, spectra=False):
    w = circ_layer_setup(batch, d, p, nrot, spectra)  # kept alive: the graph holds raw pointers into it
    g = _graph(w["rot"])
    for _ in range(max(1, -(-warmup // nrot))):
        g.replay()
    reps = max(1, -(-steps // nrot))
    tm = Timer()
    torch.cuda.synchronize()
    hold_gpu(1.0)
    tm.start()
    for _ in range(reps):
        g.replay()
    ms = tm.stop() / (reps * nrot)
    nbytes, flops = circ_algorithmic(batch, d, p, 2)
    t_roof = max(nbytes / (HBM_PEAK_GBS * 1e9), flops / (VALU_FP32_PEAK_TFS * 1e12)) * 1e3
    return {
        "tokens_per_s": round(batch / (ms * 1e-3), 1),
        "ms_per_step": round(ms, 5),
        "roofline_ms": round(t_roof, 5),
        "frac_of_roofline": round(t_roof / ms, 4),
    }


def circ_adapters_setup(n_adapters=128, batch=2048, d=4096, p=1024, spectra=False):
    """The adapter workload as bench_circ_adapters times it: per adapter a
    token batch, an upstream gradient (bf16) and c (fp32), and ``step``: the
    forwards of all adapters in order, then the backwards in reverse.
    spectra: each adapter keeps its weight spectra from forward to backward."""
    q = k = d // p
    w = {"xs": [syn.torch_normal((batch, d), syn.WL_CIRC_ADAPTERS, syn.T_X, a, dtype=torch.bfloat16)
                for a in range(n_adapters)],
         "dys": [syn.torch_normal((batch, d), syn.WL_CIRC_ADAPTERS, syn.T_DY, a, dtype=torch.bfloat16)
                 for a in range(n_adapters)],
         "cs": [syn.torch_normal((q, k, p), syn.WL_CIRC_ADAPTERS, syn.T_C, a, scale=1 / 64.0) for a in range(n_adapters)]}
    w["ys"] = [torch.empty_like(x) for x in w["xs"]]
    w["dxs"] = [torch.empty_like(x) for x in w["xs"]]
    w["dcs"] = [torch.empty_like(c) for c in w["cs"]]
    w["specs"] = [torch.empty_like(c) for c in w["cs"]] if spectra else None

    def step():
        for a in range(n_adapters):
            if spectra:
                bcl.circulant_fwd_step(w["xs"][a], w["cs"][a], w["specs"][a], w["ys"][a], dc=w["dcs"][a])
            else:
                bcl.circulant_fwd_zero(w["xs"][a], w["cs"][a], w["dcs"][a], w["ys"][a])
        for a in reversed(range(n_adapters)):
            if spectra:
                bcl.circulant_bwd_spec(w["xs"][a], w["specs"][a], w["dys"][a], dx=w["dxs"][a], dc=w["dcs"][a],
                                       accumulate=True)
            else:
                bcl.circulant_bwd_acc(w["xs"][a], w["cs"][a], w["dys"][a], w["dcs"][a], dx=w["dxs"][a])

    w["step"] = step
    return w


def bench_circ_adapters(steps, warmup, n_adapters=128, batch=2048, d=4096, p=1024, spectra=False):
    w = circ_adapters_setup(n_adapters, batch, d, p, spectra)  # kept alive: the graph holds raw pointers into it
    g = _graph(w["step"])
    for _ in range(warmup):
        g.replay()
    tm = Timer()
    torch.cuda.synchronize()
    hold_gpu(1.0)
    tm.start()
    for _ in range(steps):
        g.replay()
    ms = tm.stop() / steps
    nbytes, flops = circ_algorithmic(batch, d, p, 2)
    nbytes *= n_adapters
    flops *= n_adapters
    t_roof = max(nbytes / (HBM_PEAK_GBS * 1e9), flops / (VALU_FP32_PEAK_TFS * 1e12)) * 1e3
    return {
        "tokens_per_s": round(batch / (ms * 1e-3), 1),
        "ms_per_step": round(ms, 4),
        "roofline_ms": round(t_roof, 4),
        "frac_of_roofline": round(t_roof / ms, 4),
    }


def bench_circ_forward_fixed(batch, d, p, spectra, steps=256, warmup=32, nrot=32):
    """Forwards only, with c fixed (inference): nrot token batches in rotation,
    from c (circulant_fwd) or from its spectra computed once beforehand
    (circulant_fwd_spec, the spectra launch outside the timed region)."""
    w = circ_layer_setup(batch, d, p, nrot)  # kept alive: the graph holds raw pointers into it
    bcl.circulant_weight_spectra(w["c"], w["cs"])

    def rot():
        for j in range(nrot):
            if spectra:
                bcl.circulant_fwd_spec(w["xs"][j], w["cs"], w["ys"][j])
            else:
                bcl.circulant_fwd(w["xs"][j], w["c"], w["ys"][j])

    g = _graph(rot)
    for _ in range(max(1, -(-warmup // nrot))):
        g.replay()
    reps = max(1, -(-steps // nrot))
    tm = Timer()
    torch.cuda.synchronize()
    hold_gpu(1.0)
    tm.start()
    for _ in range(reps):
        g.replay()
    ms = tm.stop() / (reps * nrot)
    return {"tokens_per_s": round(batch / (ms * 1e-3), 1), "ms_per_forward": round(ms, 5)}


def profile_circulant(reps=3):
    """Eager launches of the four circulant workloads (the zeroing forward, then
    the accumulating backward with dx and dc, as the timed steps run them; then
    the same from the weight spectra: the forward with fixed weights and the
    accumulating backward), for counter collection under a profiler: no
    graphs, no timing."""
    for name, (batch, d, p) in {"adapter": (2048, 4096, 1024), "p128": (256, 4096, 128), "p512": (256, 4096, 512),
                                "p4096": (256, 4096, 4096)}.items():
        q = k = d // p
        x = syn.torch_normal((batch, d), syn.WL_CIRC_LAYER, syn.T_X, 0, dtype=torch.bfloat16)
        dy = syn.torch_normal((batch, d), syn.WL_CIRC_LAYER, syn.T_DY, 0, dtype=torch.bfloat16)
        c = syn.torch_normal((q, k, p), syn.WL_CIRC_LAYER, syn.T_C, p, scale=1 / 64.0)
        dc = torch.empty_like(c)
        for _ in range(reps):
            bcl.circulant_fwd_zero(x, c, dc)
            bcl.circulant_bwd_acc(x, c, dy, dc)
        cs = bcl.circulant_weight_spectra(c)
        for _ in range(reps):
            bcl.circulant_fwd_spec(x, cs)
            bcl.circulant_bwd_spec(x, cs, dy, dc=dc, accumulate=True)
        torch.cuda.synchronize()
        log(f"profiled circulant {name}: B={batch} D={d} p={p}, {reps} x (forward, backward) from c and from its "
            "spectra")


def profile_api():
    """Every entry point of the library, on buffers allocated beforehand, once
    to warm up and once more between two of torch's spin kernels, for a HIP API
    trace (api_summary): the HIP calls on this thread between the two spin
    launches are the library's and the binding's alone."""
    a = syn.torch_normal((4096, 512), syn.WL_RDFFT_512, syn.T_X, 0)
    a2d = syn.torch_normal((1, 1024, 1024), syn.WL_RDFFT_LARGE, syn.T_X, 1)
    spec = torch.empty(4096, 257, 2, device=a.device)
    batch, d, p = 256, 4096, 128
    x = syn.torch_normal((batch, d), syn.WL_CIRC_LAYER, syn.T_X, 0, dtype=torch.bfloat16)
    dy = syn.torch_normal((batch, d), syn.WL_CIRC_LAYER, syn.T_DY, 0, dtype=torch.bfloat16)
    c = syn.torch_normal((d // p, d // p, p), syn.WL_CIRC_LAYER, syn.T_C, p, scale=1 / 64.0)
    y, dx = torch.empty_like(x), torch.empty_like(x)
    dc, cs = torch.empty_like(c), torch.empty_like(c)
    ws = torch.empty(bcl.circulant_bwd_det_workspace(batch, d, d, p, True) // 4, device=a.device)

    def calls():
        bcl.rdfft_forward(a)
        bcl.rdfft_inverse(a)
        bcl.rdfft2d_forward(a2d)
        bcl.rdfft2d_inverse(a2d)
        bcl.rdfft_unpack(a, spec)
        bcl.rdfft_pack(spec, a)
        bcl.circulant_fwd(x, c, y)
        bcl.circulant_bwd(x, c, dy, dx, dc)
        bcl.circulant_fwd_zero(x, c, dc, y)
        bcl.circulant_bwd_acc(x, c, dy, dc, dx)
        bcl.circulant_bwd_det_workspace(batch, d, d, p, True)
        bcl.circulant_bwd_det(x, c, dy, dx, dc, ws)
        bcl.circulant_bwd_det_noalloc(x, c, dy, dx, dc)
        bcl.circulant_weight_spectra(c, cs)
        bcl.circulant_fwd_step(x, c, cs, y, dc=dc)
        bcl.circulant_fwd_spec(x, cs, y, dc=dc)
        bcl.circulant_bwd_spec(x, cs, dy, dx, dc, accumulate=True)

    calls()
    torch.cuda.synchronize()
    torch.cuda._sleep(1000)
    calls()
    torch.cuda._sleep(1000)
    torch.cuda.synchronize()
    log("profiled the HIP API calls of every entry point (second pass between two spin kernels)")


API_ALLOC = re.compile(r"Malloc|Free|Memset|HostRegister|MemPool|MemAlloc|MemCreate|MemMap")


def api_summary(root: str) -> str:
    """Markdown summary of a rocprofv3 --hip-trace --kernel-trace run of
    --profile-api (csv under ``root``): the HIP API calls the calling thread
    made between the launches of the two spin kernels, by function, with the
    allocation and memset calls among them counted separately."""
    import csv
    import glob

    api = glob.glob(os.path.join(root, "**", "*hip_api_trace.csv"), recursive=True)
    ker = glob.glob(os.path.join(root, "**", "*kernel_trace.csv"), recursive=True)
    if not api or not ker:
        raise SystemExit(f"no hip_api_trace.csv / kernel_trace.csv under {root}")
    kernels = {r["Correlation_Id"]: r["Kernel_Name"] for r in csv.DictReader(open(ker[0]))}
    calls = sorted(csv.DictReader(open(api[0])), key=lambda r: int(r["Start_Timestamp"]))
    spins = [r for r in calls if "spin_kernel" in kernels.get(r["Correlation_Id"], "")]
    if len(spins) < 2:
        raise SystemExit("the trace holds fewer than two spin-kernel launches")
    a, b = spins[-2], spins[-1]
    t0, t1, tid = int(a["Start_Timestamp"]), int(b["Start_Timestamp"]), a["Thread_Id"]
    inside = [r for r in calls if r["Thread_Id"] == tid and t0 < int(r["Start_Timestamp"]) < t1]
    count = {}
    for r in inside:
        count[r["Function"]] = count.get(r["Function"], 0) + 1
    launches = [kernels[r["Correlation_Id"]] for r in inside if r["Correlation_Id"] in kernels]
    ours = sum(1 for k in launches if "rdfft::" in k)
    alloc = {f: n for f, n in count.items() if API_ALLOC.search(f)}
    rows = [f"| `{f}` | {n} |" for f, n in sorted(count.items(), key=lambda kv: (-kv[1], kv[0]))]
    return "\n".join([
        "# HIP API calls inside the library's entry points (rocprofv3 HIP trace)",
        "",
        "Command (repository root, one MI355X):",
        "",
        "```",
        "rocprofv3 --hip-trace --kernel-trace -d gpurun_out/api -o api --output-format csv -- python3 -u bench.py "
        "--profile-api",
        "python3 bench.py --api-summary gpurun_out/api",
        "```",
        "",
        "`--profile-api` calls every entry point (transforms, 2D, pack and unpack, every circulant call,",
        "the deterministic and allocation-free backwards, the weight-spectra calls) on buffers allocated",
        "beforehand: once to warm up, then once more between the launches of two of torch's spin kernels.",
        "Below: every HIP API call the calling thread made between those two launches, that is, the calls",
        "of the library and of its ctypes binding during the second pass.",
        "",
        f"Kernel launches in the window: {len(launches)}, of which {ours} of this library.",
        f"Allocation, free or memset calls in the window: {sum(alloc.values())}"
        + (f" ({', '.join(f'{f}: {n}' for f, n in alloc.items())})" if alloc else "") + ".",
        "",
        "| HIP function | calls |",
        "|---|---|",
        *rows,
    ]) + "\n"


def profile_2d(reps=3):
    """Eager 2D forward and inverse of one 4096x4096 fp32 array, for counter
    collection under a profiler: no graphs, no timing."""
    x = syn.torch_normal((1, 4096, 4096), syn.WL_RDFFT_LARGE, syn.T_X, 2)
    for _ in range(reps):
        bcl.rdfft2d_forward(x)
        bcl.rdfft2d_inverse(x)
    torch.cuda.synchronize()
    log(f"profiled 2D 4096x4096 fp32: {reps} x (forward, inverse)")


def trace_summary(trace_dir: str, steps: int, warmup: int, command: str) -> str:
    """Markdown summary of a ``rocprofv3 --kernel-trace --stats`` run of this
    script (csv output in ``trace_dir``): every kernel of this library by total
    time, and the headline forward kernel's average over the dispatches of the
    timed region alone (its dispatches warmup .. warmup + steps - 1 in launch
    order), the duration bench.py's roofline is to agree with."""
    import csv
    import glob

    stats = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    trace = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not stats or not trace:
        raise SystemExit(f"no kernel_stats.csv / kernel_trace.csv under {trace_dir}")
    short = lambda n: re.sub(r"rdfft::|^void ", "", n.replace("(anonymous namespace)::", "").split("(")[0])  # noqa: E731
    rows = [r for r in csv.DictReader(open(stats[0])) if "rdfft::" in r["Name"] or "stream_inplace" in r["Name"]]
    lines = [
        "# Kernel trace: bench.py",
        "",
        f"source_hash: {kernel_source_hash()}",
        "(hash of rdfft_device.hpp, rdfft_kernels.hpp and gen_twiddles.py as traced; bench.py reports",
        "`roofline.kernel_ms_traced` only while the current sources hash to this value)",
        "",
        "Command (repository root, one MI355X, libraries built with `python -m block_circulant_layers_amd.build`):",
        "",
        "```",
        command,
        "```",
        "",
        "This library's kernels (and the streaming reference pass), by total time; durations in microseconds,",
        "the tracer's start-to-end of each dispatch:",
        "",
        "| kernel | calls | avg us | min us | max us |",
        "|---|---|---|---|---|",
    ]
    for r in rows:
        lines.append(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} |")
    every = sorted(csv.DictReader(open(trace[0])), key=lambda r: int(r["Start_Timestamp"]))
    head = [i for i, r in enumerate(every) if "rdfft_fwd_kernel<512, rdfft::F32Io>" in r["Kernel_Name"]]
    timed = head[warmup: warmup + steps]
    if timed:
        d = [(int(every[i]["End_Timestamp"]) - int(every[i]["Start_Timestamp"])) / 1e3 for i in timed]
        # idle time before each timed launch: from the end of the dispatch before it
        idle = [(int(every[i]["Start_Timestamp"]) - int(every[i - 1]["End_Timestamp"])) / 1e3 for i in timed if i > 0]
        lines += ["", "Headline forward kernel, the timed region's dispatches only:", "",
                  "| kernel | timed dispatches | avg us | min us | max us | median idle before a launch, us |",
                  "|---|---|---|---|---|---|",
                  f"| rdfft_fwd_kernel<512, F32Io> | {len(d)} | {np.mean(d):.2f} | {min(d):.2f} | {max(d):.2f} | "
                  f"{float(np.median(idle)) if idle else 0.0:.1f} |",
                  "",
                  "bench.py queues the timed launches behind a spin kernel, so they run back to back (idle near 0).",
                  "Where the tracer's handling of each dispatch leaves the GPU idle between them, the launches",
                  "start on an idle GPU and take longer than in the untimed run."]
    return "\n".join(lines) + "\n"


CALIB_KIB = 262144.0  # the --calib-copy copy: 256 MiB read and 256 MiB written


def _counter_means(csv_path: str):
    """{kernel name: (mean counter value, dispatches)} of one rocprofv3 --pmc
    run, and the counter value of its first plain device copy (the
    --calib-copy copy of known size), in KiB."""
    import csv

    acc, calib = {}, None
    for r in csv.DictReader(open(csv_path)):
        name, v = r["Kernel_Name"], float(r["Counter_Value"])
        if name == "__amd_rocclr_copyBuffer" and calib is None:
            calib = v
        a = acc.setdefault(name, [0.0, 0])
        a[0] += v
        a[1] += 1
    return {k: (v[0] / v[1], v[1]) for k, v in acc.items()}, calib


def counter_summary(root: str):
    """Markdown summaries of the HBM counter runs under ``root`` (the layout of
    the commands quoted in them): (profiles/traffic.md text, profiles/
    traffic_circulant_d4096.md text).  FETCH_SIZE and WRITE_SIZE are scaled by
    the factor that maps the known copy onto its size."""
    import glob

    io = {"f32": "F32Io", "bf16": "Bf16Io", "f16": "F16Io"}
    rows_md = []
    calib_md = []
    for fdir in sorted(glob.glob(os.path.join(root, "pmc", "FETCH_SIZE_*"))):
        tag = os.path.basename(fdir)[len("FETCH_SIZE_"):]
        p, dt = tag.split("_")
        f, fcal = _counter_means(os.path.join(fdir, "pmc_counter_collection.csv"))
        w, wcal = _counter_means(os.path.join(root, "pmc", f"WRITE_SIZE_{tag}", "pmc_counter_collection.csv"))
        ff, wf = CALIB_KIB / fcal, CALIB_KIB / wcal
        calib_md.append(f"| 4096x{p} {dt} | {fcal:.1f} | {ff:.5f} | {wcal:.1f} | {wf:.5f} |")
        eb = 4 if dt == "f32" else 2
        algo = 2 * 4096 * int(p) * eb
        for kind in ("fwd", "inv"):
            key = next(k for k in f if f"rdfft_{kind}_kernel<{p}, rdfft::{io[dt]}>" in k)
            fk, n = f[key]
            wk, _ = w[key]
            scaled = (fk * ff + wk * wf) * 1024
            rows_md.append(f"| rdfft_{kind}_kernel<{p}, {io[dt]}> 4096x{p} | {n} | {fk:.1f} | {wk:.1f} | "
                           f"{scaled:.0f} | {algo} | {scaled / algo:.4f} |")
    tr = "\n".join([
        "# HBM traffic of the transform kernels (rocprofv3 counters)",
        "",
        f"source_hash: {kernel_source_hash()}",
        "(hash of rdfft_device.hpp, rdfft_kernels.hpp and gen_twiddles.py as measured; bench.py reports",
        "`roofline.traffic` only while the current sources hash to this value)",
        "",
        "Commands (one counter per run, repository root, one MI355X; `<p> <dtype>` = `512 f32`, `4096 f32`, "
        "`4096 bf16`):",
        "",
        "```",
        "rocprofv3 --pmc FETCH_SIZE -d gpurun_out/pmc/FETCH_SIZE_<p>_<dtype> -o pmc --output-format csv -- python3 -u "
        "bench.py --rows 4096 --p <p> --dtype <dtype> --steps 128 --warmup 1 --no-extra --no-cpu --calib-copy --eager",
        "rocprofv3 --pmc WRITE_SIZE -d gpurun_out/pmc/WRITE_SIZE_<p>_<dtype> -o pmc --output-format csv -- python3 -u "
        "bench.py --rows 4096 --p <p> --dtype <dtype> --steps 128 --warmup 1 --no-extra --no-cpu --calib-copy --eager",
        "python3 bench.py --counter-summary gpurun_out",
        "```",
        "",
        "`--calib-copy` first runs one plain 256 MiB device copy (`__amd_rocclr_copyBuffer`, the first copy dispatch",
        "of the run); `--eager` launches the transforms directly so that every dispatch is counted.  Values are KiB",
        "per dispatch, mean over all dispatches of the kernel.",
        "",
        "Calibration with the known-size copy (256 MiB = 262144 KiB read and written):",
        "",
        "| run | FETCH_SIZE of the copy | factor | WRITE_SIZE of the copy | factor |",
        "|---|---|---|---|---|",
        *calib_md,
        "",
        "Per launch (scaled; algorithmic = each row read once and written once):",
        "",
        "| kernel workload | dispatches | FETCH raw KiB | WRITE raw KiB | scaled bytes per launch | algorithmic | ratio |",
        "|---|---|---|---|---|---|---|",
        *rows_md,
    ]) + "\n"
    # circulant kernels of --profile-circulant (D=4096 bf16 workloads)
    ctr = os.path.join(root, "ctr")
    circ = None
    if os.path.isdir(os.path.join(ctr, "FETCH_SIZE")):
        f, fcal = _counter_means(os.path.join(ctr, "FETCH_SIZE", "pmc_counter_collection.csv"))
        w, wcal = _counter_means(os.path.join(ctr, "WRITE_SIZE", "pmc_counter_collection.csv"))
        if fcal is None or wcal is None:
            raise SystemExit("the circulant counter runs carry no calibration copy (take them with --calib-copy)")
        ff, wf = CALIB_KIB / fcal, CALIB_KIB / wcal
        kib = lambda b: b / 1024  # noqa: E731
        work = []  # (kernel, workload, algorithmic reads KiB, algorithmic writes KiB)
        for name, batch, pp in (("adapter", 2048, 1024), ("D=4096 B=256 p=128", 256, 128),
                                ("D=4096 B=256 p=512", 256, 512), ("D=4096 B=256 p=4096", 256, 4096)):
            act, cb = batch * 4096 * 2, 4096 * 4096 // pp * 4
            # a layer of one block (d = p) runs its forward on circ_one_kernel
            fwd = "circ_one_kernel" if pp == 4096 else "circ_tp_kernel"
            work += [
                (f"{fwd}<{pp}, false, rdfft::Bf16Io, false>", f"{name} forward", kib(act + cb),
                 kib(act + cb)),
                (f"circ_bwd_kernel<{pp}, rdfft::Bf16Io, false, false>", f"{name} backward (dx and dc)",
                 kib(2 * act + cb), kib(act + cb)),
                (f"{fwd}<{pp}, false, rdfft::Bf16Io, true>", f"{name} forward from the weight spectra",
                 kib(act + cb), kib(act)),
                (f"circ_bwd_kernel<{pp}, rdfft::Bf16Io, false, true>",
                 f"{name} backward from the weight spectra (dx and dc)", kib(2 * act + cb), kib(act + cb)),
            ]
        lines = []
        for kname, wl, ar, aw in work:
            key = next((k for k in f if kname in k), None)
            if key is None:
                continue
            fr, n = f[key]
            wr, _ = w[key]
            lines.append(f"| `{kname.replace('rdfft::', '')}` | {wl} | {n} | {ar:.0f} | {fr * ff:.0f} | "
                         f"{fr * ff / ar:.2f} | {aw:.0f} | {wr * wf:.0f} | {wr * wf / aw:.2f} |")
        circ = "\n".join([
            "# HBM traffic of the circulant kernels (rocprofv3 counters), D=4096 bf16 workloads",
            "",
            "Commands (repository root, one MI355X):",
            "",
            "```",
            "rocprofv3 --pmc FETCH_SIZE -d gpurun_out/ctr/FETCH_SIZE -o pmc --output-format csv -- python3 -u bench.py "
            "--profile-circulant --calib-copy",
            "rocprofv3 --pmc WRITE_SIZE -d gpurun_out/ctr/WRITE_SIZE -o pmc --output-format csv -- python3 -u bench.py "
            "--profile-circulant --calib-copy",
            "python3 bench.py --counter-summary gpurun_out",
            "```",
            "",
            f"Means over the dispatches of each kernel, KiB, scaled by the known-size copy (FETCH x {ff:.4f}, "
            f"WRITE x {wf:.4f}).  Algorithmic: activations once, `c` (or its spectra) once, `dc` once (fp32); "
            "the forward from `c` also writes the zeros of `dc`, which the backward then adds into; the "
            "forward from the spectra writes `y` alone.",
            "",
            "| kernel | workload | dispatches | algorithmic reads | measured reads | ratio | algorithmic writes | "
            "measured writes | ratio |",
            "|---|---|---|---|---|---|---|---|---|",
            *lines,
        ]) + "\n"
    return tr, circ


def _sq_means(csv_path: str):
    """{(kernel name, counter): mean value over its dispatches} of a rocprofv3 --pmc run."""
    import csv

    acc = {}
    for r in csv.DictReader(open(csv_path)):
        a = acc.setdefault((r["Kernel_Name"], r["Counter_Name"]), [0.0, 0])
        a[0] += float(r["Counter_Value"])
        a[1] += 1
    return {k: v[0] / v[1] for k, v in acc.items()}


def sq_summary(root: str, trace_dir: str) -> str:
    """Markdown summary of the SQ counter runs under ``root`` (cpmc/s1, cpmc/s2:
    the circulant workloads; rpmc/s<i>_<dtype>: the 4096x4096 transforms),
    with the traced durations of the same kernels from ``trace_dir``."""
    import csv
    import glob

    m = {}
    for path in glob.glob(os.path.join(root, "cpmc", "s*", "pmc_counter_collection.csv")) + \
            glob.glob(os.path.join(root, "rpmc", "s*", "pmc_counter_collection.csv")):
        m.update(_sq_means(path))
    stats = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    traced = {r["Name"]: float(r["AverageNs"]) / 1e3 for r in csv.DictReader(open(stats[0]))} if stats else {}
    clock, simds = 2.4e9, 1024
    rows = []
    kernels = sorted({k for k, _ in m if any(f"rdfft::{n}_" in k for n in ("circ", "rdfft", "col", "combine"))})
    for k in kernels:
        g = lambda c: m.get((k, c))  # noqa: E731
        if g("SQ_INSTS_VALU") is None or g("SQ_WAVE_CYCLES") is None:
            continue
        issue_us = g("SQ_INSTS_VALU") * 4 / (simds * clock) * 1e6
        dur = next((v for n, v in traced.items() if n.split("(")[0] == k.split("(")[0]), None)
        wait = g("SQ_WAIT_INST_ANY") / g("SQ_WAVE_CYCLES") if g("SQ_WAIT_INST_ANY") is not None else None
        bank = (g("SQ_LDS_BANK_CONFLICT") / g("SQ_ACTIVE_INST_LDS")
                if g("SQ_LDS_BANK_CONFLICT") is not None and g("SQ_ACTIVE_INST_LDS") else None)
        name = re.sub(r"rdfft::|^void ", "", k.split("(")[0])
        rows.append(f"| `{name}` | {g('SQ_WAVES'):.0f} | {g('SQ_INSTS_VALU') / 1e6:.2f} | {g('SQ_INSTS_LDS') / 1e6:.2f} | "
                    f"{issue_us:.1f} | {dur if dur is None else round(dur, 1)} | "
                    f"{'-' if dur is None else round(issue_us / dur, 2)} | "
                    f"{'-' if wait is None else round(wait, 2)} | {'-' if bank is None else round(bank, 2)} | "
                    f"{'-' if g('SQ_LDS_BANK_CONFLICT') is None else round(g('SQ_LDS_BANK_CONFLICT') / 1e6, 3)} |")
    return "\n".join([
        "# SQ counters of the circulant kernels, the 4096x4096 transforms, long rows and 2D (rocprofv3)",
        "",
        "Commands (repository root, one MI355X; `<set>` is one of the two counter sets below, `<i>` its number):",
        "",
        "```",
        "rocprofv3 --pmc <set> -d gpurun_out/cpmc/s<i> -o pmc --output-format csv -- python3 -u bench.py "
        "--profile-circulant",
        "rocprofv3 --pmc <set> -d gpurun_out/rpmc/s<i>_<dtype> -o pmc --output-format csv -- python3 -u bench.py "
        "--rows 4096 --p 4096 --dtype <dtype> --steps 64 --warmup 1 --no-extra --no-cpu --eager",
        "rocprofv3 --pmc <set> -d gpurun_out/rpmc/s<i>_long -o pmc --output-format csv -- python3 -u bench.py "
        "--rows 512 --p 32768 --steps 16 --warmup 1 --no-extra --no-cpu --eager",
        "rocprofv3 --pmc <set> -d gpurun_out/rpmc/s<i>_2d -o pmc --output-format csv -- python3 -u bench.py "
        "--profile-2d",
        "python3 bench.py --sq-summary gpurun_out",
        "```",
        "",
        "Set 1: `SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_INSTS_LDS "
        "SQ_WAIT_INST_LDS SQ_WAIT_ANY`;",
        "set 2: `SQ_INSTS_SALU SQ_ACTIVE_INST_LDS SQ_INST_CYCLES_VMEM SQ_WAIT_INST_ANY SQ_LDS_BANK_CONFLICT "
        "SQ_ACTIVE_INST_ANY GRBM_GUI_ACTIVE`.",
        "`--profile-circulant` launches each circulant workload three times eagerly (forward, then backward with",
        "dx and dc), from `c` and from its spectra (kernels instantiated with `true` last): one adapter of the",
        "128-adapter workload (4096x4096, p=1024, 2048 tokens) and the single layer D=4096, B=256 at",
        "p = 128, 512, 4096, all bf16.  `--profile-2d` runs the 2D forward and inverse of",
        "one 4096x4096 fp32 array three times.  Means over the dispatches of each kernel.",
        "",
        "*VALU issue time* = VALU wave-instructions x 4 cycles / (1024 SIMDs x 2.4 GHz): the time the",
        "chip's SIMDs need just to issue them (one unpacked fp32 wave64 instruction occupies a SIMD for 4",
        "cycles; the library is compiled with packed fp32 disabled).  *Traced duration* is the kernel's average in",
        "`kernel_trace_bench_default.md`.  *issue / duration* is the share of the kernel's time the VALUs are",
        "busy at best.  The last two columns are SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS and",
        "SQ_LDS_BANK_CONFLICT itself (cycles summed over the chip, per dispatch).",
        "",
        "| kernel | waves | VALU wave-instr (M) | LDS instr (M) | VALU issue time (us) | traced duration (us) | "
        "issue / duration | wait-for-issue / wave-cycles | bank-conflict cycles per LDS cycle | "
        "bank-conflict cycles (M) |",
        "|---|---|---|---|---|---|---|---|---|---|",
        *rows,
    ]) + "\n"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2048)
    ap.add_argument("--warmup", type=int, default=256)
    ap.add_argument("--no-extra", action="store_true", help="only the headline workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--cpu-seconds", type=float, default=20.0, help="oracle time, split between one thread and all cores")
    ap.add_argument("--rows", type=int, default=4096, help="transform rows of the timed workload")
    ap.add_argument("--p", type=int, default=512, help="row length of the timed workload")
    ap.add_argument("--dtype", choices=("f32", "bf16", "f16"), default="f32", help="storage type of the timed workload")
    ap.add_argument("--eager", action="store_true",
                    help="launch the timed transforms directly instead of from HIP graphs (for counter runs)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="first run one plain 256 MiB device copy (a known-size reference for HBM counters)")
    ap.add_argument("--profile-circulant", action="store_true",
                    help="only launch the circulant workloads eagerly, for counter collection, and exit")
    ap.add_argument("--profile-api", action="store_true",
                    help="only call every entry point twice (the second time between two spin kernels), for a "
                         "HIP API trace, and exit")
    ap.add_argument("--api-summary", metavar="ROOT",
                    help="write profiles/hip_api_library_calls.md from a HIP API trace of --profile-api under ROOT "
                         "and exit (no GPU needed)")
    ap.add_argument("--profile-2d", action="store_true",
                    help="only run the 2D forward and inverse of one 4096x4096 fp32 array eagerly, three times, for "
                         "counter collection, and exit")
    ap.add_argument("--counter-summary", metavar="ROOT",
                    help="write profiles/traffic.md and profiles/traffic_circulant_d4096.md from the FETCH_SIZE / "
                         "WRITE_SIZE runs under ROOT (see those files for the commands) and exit (no GPU needed)")
    ap.add_argument("--sq-summary", metavar="ROOT",
                    help="write profiles/counters_circulant_and_transforms.md from the SQ counter runs under ROOT "
                         "(and the kernel trace under ROOT/ktrace) and exit (no GPU needed)")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="write the markdown summary of a rocprofv3 kernel trace of this script (csv files under "
                         "DIR, taken with the same --steps/--warmup) to stdout and exit (no GPU needed)")
    args = ap.parse_args()
    if args.counter_summary:
        tr, circ = counter_summary(args.counter_summary)
        open(os.path.join(PROFILES, "traffic.md"), "w").write(tr)
        if circ:
            open(os.path.join(PROFILES, "traffic_circulant_d4096.md"), "w").write(circ)
        return
    if args.api_summary:
        open(os.path.join(PROFILES, "hip_api_library_calls.md"), "w").write(api_summary(args.api_summary))
        return
    if args.sq_summary:
        open(os.path.join(PROFILES, "counters_circulant_and_transforms.md"), "w").write(
            sq_summary(args.sq_summary, os.path.join(args.sq_summary, "ktrace")))
        return
    if args.trace_summary:
        cmd = (f"rocprofv3 --kernel-trace --stats -d {args.trace_summary} -o ktrace --output-format csv -- "
               f"python3 -u bench.py --steps {args.steps} --warmup {args.warmup}")
        sys.stdout.write(trace_summary(args.trace_summary, args.steps, args.warmup, cmd))
        return
    if args.gpus != 1:
        print(
            f"bench.py measures one GPU only (asked for {args.gpus}); the transform rows and the layer's "
            "tokens shard with no communication but dc's all-reduce, which is not built here.",
            file=sys.stderr,
        )
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    bcl.lib()
    if args.calib_copy:
        a = torch.ones(64 << 20, device="cuda:0")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    if args.profile_circulant:
        profile_circulant()
        return
    if args.profile_2d:
        profile_2d()
        return
    if args.profile_api:
        profile_api()
        return

    rows, p, dt = args.rows, args.p, args.dtype
    log(f"headline: rdfft {rows}x{p} {dt} fwd+inv, warmup {args.warmup}, steps {args.steps}")
    wl = syn.WL_RDFFT_512 if (rows, p) == (4096, 512) else syn.WL_RDFFT_LARGE
    h = bench_rdfft(rows, p, dt, args.steps, args.warmup, wl, eager=args.eager)
    kname = f"rdfft_fwd_kernel<{p}, {IO_NAME[dt]}>"
    achieved = h["bytes_per_launch"] / (h["fwd_ms"] * 1e-3) / 1e9
    traced = recorded_trace_ms(kname)
    out = {
        "metric": METRIC,
        "value": round(h["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": h["steps"],
        "warmup": h["warmup"],
        "ms_per_step": round(h["ms_per_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt,
        "data": "synthetic",
        "config": {
            "workload": f"rdFFT {rows} rows x p={p}, {dt}, forward then inverse in place",
            "rows": rows,
            "p": p,
            "rotating_buffers": h["nbuf"],
            "launch": ("plain launches queued behind a spin kernel" if h["queued"] else
                       "HIP graph replays, runs of up to rotating_buffers / 2 steps"),
            "roundtrip_drift": h["roundtrip_drift"],
            "pct_hbm_peak": round(100 * h["gbs"] / HBM_PEAK_GBS, 2),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic(f"{kname} {rows}x{p}"),
            "kernel": kname,
            "kernel_ms": round(h["fwd_ms"], 6),
            "duration": "mean per forward launch in the timed region (HIP events on the launch stream around "
                        "each run of back-to-back forward launches; markers: " + str(MarkEvent.kind) + ")",
            "kernel_ms_traced": traced,
            "frac_traced": None if traced is None else round(h["bytes_per_launch"] / (traced * 1e-3) / 1e9
                                                              / HBM_PEAK_GBS, 4),
            "inverse_kernel_ms": round(h["inv_ms"], 6),
        },
    }
    if not args.no_cpu and (rows, p, dt) == (4096, 512, "f32"):
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline_rdfft(rows, p, args.cpu_seconds)
    if not args.no_extra:
        extra = {}
        for (r, pp, dt) in ((4096, 4096, "f32"), (4096, 4096, "bf16"), (16384, 128, "f32"), (16384, 128, "bf16"),
                            (4096, 1024, "f32"), (4096, 2048, "f32"), (16384, 1024, "f32"), (4096, 4096, "f16"),
                            (2048, 8192, "f32"), (512, 32768, "f32")):
            log(f"extra: rdfft {r}x{pp} {dt}")
            e = bench_rdfft(r, pp, dt, max(256, args.steps // 4), max(32, args.warmup // 4), syn.WL_RDFFT_LARGE)
            extra[f"rdfft_{r}x{pp}_{dt}"] = {
                "gbs_fwd_plus_inv": round(e["gbs"], 1),
                "pct_hbm_peak": round(100 * e["gbs"] / HBM_PEAK_GBS, 2),
                "fwd_kernel_ms": round(e["fwd_ms"], 5),
                "inv_kernel_ms": round(e["inv_ms"], 5),
                "fwd_kernel_pct_hbm_peak": round(100 * e["bytes_per_launch"] / (e["fwd_ms"] * 1e-3) / 1e9
                                                 / HBM_PEAK_GBS, 2),
            }
        log("extra: 2D 4096x4096 f32")
        extra["rdfft2d_4096x4096_f32"] = bench_rdfft2d(4096, 4096, 256, 32)
        log("extra: unpack / pack 4096x512 f32")
        extra["spectrum_unpack_pack_4096x512_f32"] = bench_spectrum(4096, 512, 1024, 128)
        for mib in (4, 8, 16, 32, 64):
            if mib in (8, 64):
                log(f"extra: device copy {mib} MiB")
                extra[f"copy_ceiling_{mib}mib"] = bench_copy(mib << 20, 1024, 128)
            log(f"extra: in-place streaming pass {mib} MiB")
            extra[f"stream_ceiling_{mib}mib"] = bench_stream(mib << 20)
        for pp in (128, 512, 4096):
            log(f"extra: circulant layer D=4096 B=256 p={pp}")
            extra[f"circulant_d4096_b256_p{pp}_bf16"] = bench_circ_layer(256, 4096, pp, 256, 32)
            log(f"extra: circulant layer D=4096 B=256 p={pp}, weight spectra kept from forward to backward")
            extra[f"circulant_d4096_b256_p{pp}_bf16_weight_spectra"] = bench_circ_layer(256, 4096, pp, 256, 32,
                                                                                        spectra=True)
            log(f"extra: circulant forward D=4096 B=256 p={pp}, fixed weights, from c and from its spectra")
            extra[f"circulant_d4096_b256_p{pp}_bf16_forward_fixed_weights"] = {
                "from_c": bench_circ_forward_fixed(256, 4096, pp, False),
                "from_spectra": bench_circ_forward_fixed(256, 4096, pp, True)}
        log("extra: single-layer peak memory")
        mem = {}
        for (b, d, pp) in ((1, 4096, 128), (1, 4096, 512), (1, 4096, 1024), (1, 4096, 4096), (256, 4096, 128),
                           (256, 4096, 512), (256, 4096, 1024), (256, 4096, 4096), (1, 1024, 1024)):
            mem[f"d{d}_b{b}_p{pp}"] = bench_layer_memory(b, d, pp)
        extra["layer_peak_memory_f32"] = mem
        log("extra: torch.fft circulant forms beside the layer (context)")
        ctx = {"peak_mib": {}, "d4096_b256_f32_fwd_bwd_ms_eager": {}}
        for (b, d, pp) in ((1, 4096, 128), (1, 4096, 4096), (256, 4096, 128), (256, 4096, 512), (256, 4096, 4096),
                           (1, 1024, 1024)):
            ctx["peak_mib"][f"d{d}_b{b}_p{pp}"] = {
                form: (mem[f"d{d}_b{b}_p{pp}"] if form == "rdfft_layer" else bench_layer_memory(b, d, pp, form))["peak_mib"]
                for form in LAYER_FORMS
            }
        for pp in (128, 512, 4096):
            ctx["d4096_b256_f32_fwd_bwd_ms_eager"][f"p{pp}"] = {form: bench_layer_eager(256, 4096, pp, form)
                                                               for form in LAYER_FORMS}
        extra["torch_fft_context"] = ctx
        log("extra: 128 circulant adapters 4096x4096 p=1024, 2048 tokens")
        extra["circulant_128_adapters_d4096_p1024_b2048_bf16"] = bench_circ_adapters(10, 2)
        log("extra: 128 circulant adapters, weight spectra kept from forward to backward")
        extra["circulant_128_adapters_d4096_p1024_b2048_bf16_weight_spectra"] = bench_circ_adapters(10, 2,
                                                                                                   spectra=True)
        out["extra"] = extra
        # The pages' own operator timings (Paper-Notes page, "实验关键数据";
        # hardware, batch and precision unstated there), beside this run's
        # launches of the same lengths: context, not a comparison of equals.
        p4k = extra.get("rdfft_4096x4096_f32", {})
        out["pages_context"] = {
            "note": "pages: unnamed GPU, batch and dtype unstated; here: one MI355X, fp32, full batches",
            "rdfft_forward_p512_ms": {"pages": 0.0279, "here_4096_rows": round(h["fwd_ms"], 5)},
            "rdfft_inverse_p512_ms": {"pages": 0.0233, "here_4096_rows": round(h["inv_ms"], 5)},
            "rdfft_forward_p4096_ms": {"pages": 0.0687, "here_4096_rows": p4k.get("fwd_kernel_ms")},
            "circulant_tokens_per_s": {
                "pages_whole_7b_finetuning": 920,
                "here_128_adapters_only": extra["circulant_128_adapters_d4096_p1024_b2048_bf16"]["tokens_per_s"],
            },
        } if (rows, p, dt) == (4096, 512, "f32") else None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

"""Benchmark of the in-place packed real FFT and the block-circulant layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline step: 4096 rows of p = 512, fp32, forward then inverse rdFFT in
place (one pass of the transform path over one batch).  Each step works on
the next of NBUF distinct copies (>= 1 GiB in total) so the 256 MB last-level
cache cannot hold the data between steps; every buffer is resident in HBM
before the timed region starts.  `value` = algorithmic bytes (every row read
once and written once, per transform) / wall time of the K steps.

The JSON line also carries
  roofline      the forward kernel: algorithmic bytes per launch / its mean
                launch duration (HIP events around every launch in the timed
                region, on the launch stream), against 8 TB/s HBM;
  cpu_baseline  the fp64 oracle (numpy) on all host cores (up to 16) and on
                one thread, each on a bounded sample of the same workload, in
                the same unit;
  extra         the other transform sizes and the block-circulant layer
                workloads (tokens/s), each against its own roofline.
"""

from __future__ import annotations

import argparse
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


def bench_rdfft(rows, p, dtype, steps, warmup, workload, index=0, eager=False):
    """Steps of (forward, inverse) in place on one batch, the batch rotating
    over nbuf distinct copies.  Launches are replayed from two HIP graphs: all
    nbuf forwards, then all nbuf inverses (each buffer gets forward then
    inverse, as in a step).  Events around the forward graph give the forward
    kernel's mean launch duration."""
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    eb = 4 if dtype == "f32" else 2
    nbytes = rows * p * eb
    nbuf = max(2, ROTATE_BYTES // nbytes)
    base = syn.torch_normal((rows, p), workload, syn.T_X, index, dtype=tdt)
    bufs = [base.clone() for _ in range(nbuf)]
    g_fwd = _replayer(lambda: [bcl.rdfft_forward(b) for b in bufs], eager)
    g_inv = _replayer(lambda: [bcl.rdfft_inverse(b) for b in bufs], eager)
    reps_w = max(1, -(-warmup // nbuf))
    reps = max(1, -(-steps // nbuf))
    for _ in range(reps_w):
        g_fwd()
        g_inv()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    tm = Timer()
    torch.cuda.synchronize()
    tm.start()
    for r in range(reps):
        ev[r][0].record()
        g_fwd()
        ev[r][1].record()
        g_inv()
        ev[r][2].record()
    ms = tm.stop()
    torch.cuda.synchronize()
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / (reps * nbuf)
    inv_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / (reps * nbuf)
    # every buffer has been through (reps + reps_w) round trips: still the input
    drift = float((bufs[0].float() - base.float()).abs().max() / base.float().abs().max())
    nsteps = reps * nbuf
    step_bytes = 2 * 2 * nbytes  # forward + inverse, each reads and writes every row once
    del bufs, g_fwd, g_inv, base
    torch.cuda.empty_cache()
    return {
        "steps": nsteps,
        "warmup": reps_w * nbuf,
        "ms_per_step": ms / nsteps,
        "gbs": step_bytes / (ms / nsteps) / 1e6,
        "bytes_per_launch": 2 * nbytes,
        "fwd_ms": fwd_ms,
        "inv_ms": inv_ms,
        "nbuf": nbuf,
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
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
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


def bench_circ_layer(batch, d, p, steps, warmup, nrot=32):
    q = k = d // p
    xs = [syn.torch_normal((batch, d), syn.WL_CIRC_LAYER, syn.T_X, i, dtype=torch.bfloat16) for i in range(nrot)]
    dys = [syn.torch_normal((batch, d), syn.WL_CIRC_LAYER, syn.T_DY, i, dtype=torch.bfloat16) for i in range(nrot)]
    c = syn.torch_normal((q, k, p), syn.WL_CIRC_LAYER, syn.T_C, p, scale=1 / 64.0)
    ys = [torch.empty_like(x) for x in xs]
    dxs = [torch.empty_like(x) for x in xs]
    dc = torch.empty_like(c)

    def rot():
        for j in range(nrot):
            bcl.circulant_fwd(xs[j], c, ys[j])
            bcl.circulant_bwd(xs[j], c, dys[j], dx=dxs[j], dc=dc)

    g = _graph(rot)
    for _ in range(max(1, -(-warmup // nrot))):
        g.replay()
    reps = max(1, -(-steps // nrot))
    tm = Timer()
    torch.cuda.synchronize()
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


def bench_circ_adapters(steps, warmup, n_adapters=128, batch=2048, d=4096, p=1024):
    q = k = d // p
    xs = [syn.torch_normal((batch, d), syn.WL_CIRC_ADAPTERS, syn.T_X, a, dtype=torch.bfloat16) for a in range(n_adapters)]
    dys = [syn.torch_normal((batch, d), syn.WL_CIRC_ADAPTERS, syn.T_DY, a, dtype=torch.bfloat16) for a in range(n_adapters)]
    cs = [syn.torch_normal((q, k, p), syn.WL_CIRC_ADAPTERS, syn.T_C, a, scale=1 / 64.0) for a in range(n_adapters)]
    ys = [torch.empty_like(x) for x in xs]
    dxs = [torch.empty_like(x) for x in xs]
    dcs = [torch.empty_like(c) for c in cs]

    def step():
        for a in range(n_adapters):
            bcl.circulant_fwd(xs[a], cs[a], ys[a])
        for a in reversed(range(n_adapters)):
            bcl.circulant_bwd(xs[a], cs[a], dys[a], dx=dxs[a], dc=dcs[a])

    g = _graph(step)
    for _ in range(warmup):
        g.replay()
    tm = Timer()
    torch.cuda.synchronize()
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


def profile_circulant(reps=3):
    """Eager launches of the four circulant workloads (forward, then backward
    with dx and dc), for counter collection under a profiler: no graphs, no
    timing."""
    for name, (batch, d, p) in {"adapter": (2048, 4096, 1024), "p128": (256, 4096, 128), "p512": (256, 4096, 512),
                                "p4096": (256, 4096, 4096)}.items():
        q = k = d // p
        x = syn.torch_normal((batch, d), syn.WL_CIRC_LAYER, syn.T_X, 0, dtype=torch.bfloat16)
        dy = syn.torch_normal((batch, d), syn.WL_CIRC_LAYER, syn.T_DY, 0, dtype=torch.bfloat16)
        c = syn.torch_normal((q, k, p), syn.WL_CIRC_LAYER, syn.T_C, p, scale=1 / 64.0)
        for _ in range(reps):
            bcl.circulant_fwd(x, c)
            bcl.circulant_bwd(x, c, dy)
        torch.cuda.synchronize()
        log(f"profiled circulant {name}: B={batch} D={d} p={p}, {reps} x (forward, backward)")


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
    args = ap.parse_args()
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
    if args.profile_circulant:
        profile_circulant()
        return
    if args.calib_copy:
        a = torch.ones(64 << 20, device="cuda:0")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    rows, p, dt = args.rows, args.p, args.dtype
    log(f"headline: rdfft {rows}x{p} {dt} fwd+inv, warmup {args.warmup}, steps {args.steps}")
    wl = syn.WL_RDFFT_512 if (rows, p) == (4096, 512) else syn.WL_RDFFT_LARGE
    h = bench_rdfft(rows, p, dt, args.steps, args.warmup, wl, eager=args.eager)
    achieved = h["bytes_per_launch"] / (h["fwd_ms"] * 1e-3) / 1e9
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
            "launch": "eager launches" if args.eager else "HIP graph replays of the rotating set",
            "roundtrip_drift": h["roundtrip_drift"],
            "pct_hbm_peak": round(100 * h["gbs"] / HBM_PEAK_GBS, 2),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic(f"rdfft_fwd_kernel<{p}, {IO_NAME[dt]}> {rows}x{p}"),
            "kernel": f"rdfft_fwd_kernel<{p}, {IO_NAME[dt]}>",
            "kernel_ms": round(h["fwd_ms"], 6),
            "inverse_kernel_ms": round(h["inv_ms"], 6),
        },
    }
    if not args.no_cpu and (rows, p, dt) == (4096, 512, "f32"):
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline_rdfft(rows, p, args.cpu_seconds)
    if not args.no_extra:
        extra = {}
        for (r, pp, dt) in ((4096, 4096, "f32"), (4096, 4096, "bf16"), (16384, 128, "f32"), (16384, 128, "bf16")):
            log(f"extra: rdfft {r}x{pp} {dt}")
            e = bench_rdfft(r, pp, dt, max(256, args.steps // 4), max(32, args.warmup // 4), syn.WL_RDFFT_LARGE)
            ach = e["bytes_per_launch"] / (e["fwd_ms"] * 1e-3) / 1e9
            extra[f"rdfft_{r}x{pp}_{dt}"] = {
                "gbs_fwd_plus_inv": round(e["gbs"], 1),
                "pct_hbm_peak": round(100 * e["gbs"] / HBM_PEAK_GBS, 2),
                "fwd_kernel_gbs": round(ach, 1),
                "fwd_kernel_ms": round(e["fwd_ms"], 5),
                "inv_kernel_ms": round(e["inv_ms"], 5),
            }
        for (r, pp, dt) in ((4096, 1024, "f32"), (4096, 2048, "f32"), (16384, 1024, "f32"), (4096, 4096, "f16"),
                            (2048, 8192, "f32"), (512, 32768, "f32")):
            log(f"extra: rdfft {r}x{pp} {dt}")
            e = bench_rdfft(r, pp, dt, max(256, args.steps // 4), max(32, args.warmup // 4), syn.WL_RDFFT_LARGE)
            ach = e["bytes_per_launch"] / (e["fwd_ms"] * 1e-3) / 1e9
            extra[f"rdfft_{r}x{pp}_{dt}"] = {
                "gbs_fwd_plus_inv": round(e["gbs"], 1),
                "pct_hbm_peak": round(100 * e["gbs"] / HBM_PEAK_GBS, 2),
                "fwd_kernel_gbs": round(ach, 1),
                "fwd_kernel_ms": round(e["fwd_ms"], 5),
                "inv_kernel_ms": round(e["inv_ms"], 5),
            }
        log("extra: 2D 4096x4096 f32")
        extra["rdfft2d_4096x4096_f32"] = bench_rdfft2d(4096, 4096, 256, 32)
        log("extra: unpack / pack 4096x512 f32")
        extra["spectrum_unpack_pack_4096x512_f32"] = bench_spectrum(4096, 512, 1024, 128)
        for mib in (8, 64):
            log(f"extra: device copy {mib} MiB")
            extra[f"copy_ceiling_{mib}mib"] = bench_copy(mib << 20, 1024, 128)
        for pp in (128, 512, 4096):
            log(f"extra: circulant layer D=4096 B=256 p={pp}")
            extra[f"circulant_d4096_b256_p{pp}_bf16"] = bench_circ_layer(256, 4096, pp, 256, 32)
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

#!/usr/bin/env python3
"""Benchmark of the fused AdaLN forward+backward on one MI355X.

One step is the whole hot path over one batch of synthetic input already
resident in HBM: adaln_fwd, then the backward pass as adaln_bwd enqueues it
(adaln_bwd_fused, then adaln_bwd_finish), on torch's current stream.
For --workload mixed_schedule a step is one pass over all 64 buckets of the
mixed-length schedule in schedule order (each bucket a forward and a
backward); one input set per bucket shape is drawn and kept resident, since
the kernels' time does not depend on the values.  For the packed layouts
(--workload packed_mixed: one pack of mixed-length samples up to the
131072-token budget; mmdit_packed: text and video segments of 4 samples) a
step is adaln_fwd_segments then adaln_bwd_segments over the whole pack;
--unpacked runs the same samples as batched calls instead, one per run of
equal-length segments.  W untimed warm-up steps
run first; then exactly K steps are timed between two device
synchronisations.  Inside the timed region, HIP events recorded on the same
stream just before and after the backward's main kernel, on every fourth
step (--event-every), give that kernel's average duration (the roofline
line); each event record costs the step a few microseconds, so they are not
on every step.  The per-kernel breakdown comes from K further steps with an
event at every boundary, after the timed region.

Prints one JSON line:
  value         tokens/s over the timed steps (wall clock)
  hbm_gbps      algorithmic bytes of the step / step time
  kernels       per-call average duration, algorithmic bytes and GB/s
  roofline      the dominant kernel against the 8 TB/s HBM peak; `traffic`
                from the committed rocprofv3 counter summary when it was taken
                on the current kernel sources, else null
  cpu_baseline  the float64 CPU oracle on a bounded sample of the same
                workload, on this host's cores
  cold          each call timed alone after a 1 GiB write that evicts the
                caches, up to 20 times (median, p10, p90; --no-cold skips it)
Other modes print their own JSON line: --cost-model (shape benchmark and
cost-model fit of the bucket scheduler), --eager-reference (PyTorch's unfused
chain beside this library), --copy-probe, --traffic-from.
"""

from __future__ import annotations

import argparse
import hashlib
import glob
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("fused AdaLN fwd+bwd tokens/s and achieved HBM GB/s (% of peak), "
          "1 MI355X")
HBM_PEAK_GBPS = 8000.0


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# Sources that determine each kernel's code and launch shape.
_SHARED = ("common.hpp", "launch.hpp", "abi.hip")
KERNEL_SOURCES = {
    "fwd": ("fwd.hip", "fwd_wide.hip") + _SHARED,
    "bwd_fused": ("bwd_fused.hip", "bwd_wide.hip") + _SHARED,
    "bwd_finish": ("dmod.hip",) + _SHARED,
    "bwd": ("bwd_fused.hip", "bwd_wide.hip", "dmod.hip") + _SHARED,
    "bwd_dx": ("rows.hip",) + _SHARED,
    "bwd_dmod": ("dmod.hip",) + _SHARED,
}
# rocprofv3 kernel-name prefixes of each step component (one wavefront per
# row, or for wider rows several of them)
KERNEL_SYMBOLS = {
    "fwd": ("void adaln::fwd_rows_kernel", "void adaln::fwd_wide_kernel"),
    "bwd_fused": ("void adaln::bwd_stream_kernel",
                  "void adaln::bwd_wide_kernel"),
    "bwd_finish": ("void adaln::dmod_finish_kernel",),
}


# The streaming probes (bench_probe.hip): the operator's access pattern with
# no arithmetic, built beside this script, not part of the library.
PROBE_SRC = os.path.join(ROOT, "bench_probe.hip")
PROBE_LIB = os.path.join(ROOT, "bench_probe.so")
_probe_lib = None


def build_probe(verbose: bool = False) -> str:
    """Compile bench_probe.hip into bench_probe.so for gfx950."""
    import subprocess
    from adaln_fwd_amd import build as hip_build
    tmp = PROBE_LIB + ".tmp"
    cmd = [hip_build.hipcc(), *hip_build.FLAGS, "-shared", PROBE_SRC, "-o",
           tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, stdout=subprocess.PIPE,
                         stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def probe_lib():
    """ctypes handle of bench_probe.so (raises if it is not built)."""
    global _probe_lib
    if _probe_lib is None:
        import ctypes
        if not os.path.exists(PROBE_LIB):
            raise ImportError(f"{PROBE_LIB} is not built; run "
                              "__graft_entry__.build() first")
        lib = ctypes.CDLL(PROBE_LIB)
        vp = ctypes.c_void_p
        lib.bench_stream_probe.argtypes = [ctypes.c_int, vp, vp, vp,
                                           ctypes.c_int64, vp]
        lib.bench_stream_probe.restype = ctypes.c_int
        i = ctypes.c_int
        lib.bench_window_probe.argtypes = [i, vp, vp, vp, i, i, i, i, i, i,
                                           vp]
        lib.bench_window_probe.restype = ctypes.c_int
        _probe_lib = lib
    return _probe_lib


def run_probe(kind: int, a, dst, b=None, stream=None) -> None:
    """Enqueue a streaming probe on byte tensors of equal size (a multiple
    of 10240): kind 0 copies a into dst, kind 1 writes a XOR b."""
    import torch
    n = a.numel() * a.element_size()
    for t in (a, dst, b):
        if t is not None and (t.device.type != "cuda" or
                              not t.is_contiguous() or
                              t.numel() * t.element_size() != n):
            raise ValueError("probe buffers: contiguous GPU tensors of one "
                             "size")
    s = (stream or torch.cuda.current_stream(a.device)).cuda_stream
    rc = probe_lib().bench_stream_probe(int(kind), a.data_ptr(),
                                        None if b is None else b.data_ptr(),
                                        dst.data_ptr(), n, s)
    if rc != 0:
        raise ValueError(f"bench_stream_probe: code {rc}")


def run_window_probe(kind: int, a, dst, B: int, N: int, row_kib: int,
                     bps: int, grid: int, skew: int = 0, b=None,
                     stream=None) -> None:
    """Enqueue the windowed walk of bench_window_probe on byte tensors of
    B * N * row_kib KiB each: B sample windows of bps workgroups, `grid`
    workgroups, sample s's walk starting (s * skew) % N rows in."""
    import torch
    n = B * N * row_kib * 1024
    for t in (a, dst, b):
        if t is not None and (t.device.type != "cuda" or
                              not t.is_contiguous() or
                              t.numel() * t.element_size() != n):
            raise ValueError("window probe buffers: contiguous GPU tensors "
                             "of B * N * row_kib KiB")
    s = (stream or torch.cuda.current_stream(a.device)).cuda_stream
    rc = probe_lib().bench_window_probe(
        int(kind), a.data_ptr(), None if b is None else b.data_ptr(),
        dst.data_ptr(), int(B), int(N), int(row_kib), int(bps), int(grid),
        int(skew), s)
    if rc != 0:
        raise ValueError(f"bench_window_probe: code {rc}")


def kernel_source_hash(kernel: str = None) -> str:
    """Hash of the sources of one step component (all of them if None)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "adaln_fwd_amd", "csrc")
    if kernel is None:
        files = sorted(glob.glob(os.path.join(csrc, "*")))
    else:
        files = [os.path.join(csrc, f) for f in sorted(KERNEL_SOURCES[kernel])]
    files.append(os.path.join(ROOT, "include", "adaln.h"))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_from_counters(pmc_dir: str, workload: str, copy_bytes: int):
    """Per-launch HBM bytes of each step component from four rocprofv3
    --pmc runs under pmc_dir: fetch/ and write/ (FETCH_SIZE, WRITE_SIZE of
    bench.py) and copy_fetch/, copy_write/ (the same counters over the copy
    probe, which reads and writes copy_bytes each).  Each counter is scaled
    by the ratio of the copy's known size to what the counter read for it."""
    import csv

    def per_kernel(sub, counter):
        vals = {}
        path = os.path.join(pmc_dir, sub, "run_counter_collection.csv")
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    vals.setdefault(r["Kernel_Name"], []).append(
                        float(r["Counter_Value"]))
        return vals

    def copy_kib(sub, counter):
        vals = per_kernel(sub, counter)
        # the copy probe is the only kernel launched more than once
        name = max(vals, key=lambda k: len(vals[k]))
        v = vals[name]
        return name, sum(v) / len(v)

    cname, copy_fetch = copy_kib("copy_fetch", "FETCH_SIZE")
    _, copy_write = copy_kib("copy_write", "WRITE_SIZE")
    f_fetch = copy_bytes / (copy_fetch * 1024.0)
    f_write = copy_bytes / (copy_write * 1024.0)
    fetch = per_kernel("fetch", "FETCH_SIZE")
    write = per_kernel("write", "WRITE_SIZE")
    out = {}
    for comp, sym in KERNEL_SYMBOLS.items():
        fk = [v for k, v in fetch.items() if k.startswith(sym)]
        wk = [v for k, v in write.items() if k.startswith(sym)]
        if not fk or not wk:
            continue
        fa = sum(fk[0]) / len(fk[0])
        wa = sum(wk[0]) / len(wk[0])
        out[comp] = {
            "kernel": comp,
            "workload": workload,
            "fetch_kib_per_launch": round(fa, 3),
            "write_kib_per_launch": round(wa, 3),
            "copy_probe": {"kernel": cname, "bytes_read": copy_bytes,
                           "bytes_written": copy_bytes,
                           "fetch_kib": round(copy_fetch, 3),
                           "write_kib": round(copy_write, 3)},
            "fetch_scale": round(f_fetch, 6),
            "write_scale": round(f_write, 6),
            "hbm_bytes_per_launch": int(round(fa * 1024 * f_fetch
                                              + wa * 1024 * f_write)),
            "source_hash": kernel_source_hash(comp),
        }
    return out


def single_shape(synth, wl, bucket=None):
    """(B, N, D) of a single-shape workload, or of the mixed schedule's
    buckets of length `bucket` (B from the bucket rule)."""
    if bucket is not None:
        import adaln_fwd_amd as A
        B = A.bshape(bucket, synth.MIXED_M_MEM, synth.MIXED_M_COMP,
                     synth.MIXED_P)
        return B, bucket, wl.D
    return wl.shape


def workload_name(wl, bucket=None) -> str:
    """Name of a workload in profile file names."""
    return wl.name if bucket is None else f"{wl.name}_S{bucket}"


def algorithmic_bytes(B, N, D, esize, n_tiles, dmod_tiles=0):
    """Bytes each call must move at minimum (reads + writes); dmod_tiles is
    the n_tiles of the separate D-tile grid (adaln_bwd_dmod)."""
    T = B * N
    act = T * D * esize          # one [B, N, D] tensor
    stats = 4 * T                # one [B, N] float32 vector
    mod = B * D * esize          # one [B, D] modulation vector
    part = 2 * B * n_tiles * D * 4
    dpart = 2 * B * dmod_tiles * D * 4
    return {
        # the unfused backward: dx (read dy, x, stats, scale; write dx) and
        # the D-tile grid (read x, dy, stats; write, then read, its partial
        # sums; write dscale, dshift)
        "bwd_dx": 3 * act + mod + 2 * stats,
        "bwd_dmod": 2 * act + 2 * stats + 2 * dpart + 2 * B * D * 4,
        # read x, scale, shift; write y, mean, rstd
        "fwd": 2 * act + 2 * mod + 2 * stats,
        # read dy, x, scale, mean, rstd; write dx and the partial sums
        "bwd_fused": 3 * act + mod + 2 * stats + part,
        # read the partial sums; write dscale, dshift
        "bwd_finish": part + 2 * B * D * 4,
    }


def load_traffic(kernel: str, workload: str, src_hash: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was measured on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != src_hash:
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(inp, budget_s: float, sample_rows: int = 16384,
                 chunk_rows: int = 4096):
    """The oracle, untuned, on the first `sample_rows` token rows of the
    workload (converted to float64 once), in chunks of `chunk_rows`, cycling
    over the sample until about `budget_s` seconds of oracle time, on every
    host thread it may use; then the same on one thread for half the time
    (reported under "single_thread")."""
    import torch
    import oracle
    B, N, D = inp.x.shape
    R = min(B * N, sample_rows)
    rows = torch.arange(R)
    b = rows // N
    xs = inp.x.reshape(B * N, D)[:R].unsqueeze(1).double().numpy()
    gs = inp.dy.reshape(B * N, D)[:R].unsqueeze(1).double().numpy()
    ss = inp.scale[b].double().numpy()
    hs = inp.shift[b].double().numpy()

    def run(seconds, chunk):
        rows_done, spent, r0 = 0, 0.0, 0
        while spent < seconds:
            r1 = min(R, r0 + chunk)
            t0 = time.perf_counter()
            oracle.fwd(xs[r0:r1], ss[r0:r1], hs[r0:r1])
            oracle.bwd(gs[r0:r1], xs[r0:r1], ss[r0:r1])
            spent += time.perf_counter() - t0
            rows_done += r1 - r0
            r0 = r1 % R
        return rows_done, spent

    def describe(rows_done, spent, chunk):
        return (f"the first {R} token rows of {B}x{N}x{D}, in chunks of "
                f"{chunk} rows, forward + backward in float64, cycled for "
                f"{spent:.1f} s of oracle time ({rows_done} rows)")

    threads = oracle.num_threads()
    done, spent = run(budget_s, chunk_rows)
    rec = {
        "value": done / spent,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": describe(done, spent, chunk_rows),
    }
    oracle.set_num_threads(1)
    try:
        one_chunk = max(1, chunk_rows // 16)
        done1, spent1 = run(budget_s / 2, one_chunk)
    finally:
        oracle.set_num_threads(threads)
    rec["single_thread"] = {"value": done1 / spent1, "unit": "tokens/s",
                            "cores": 1,
                            "sample": describe(done1, spent1, one_chunk)}
    return rec


def copy_probe(nbytes: int, steps: int, warmup: int) -> int:
    """torch's copy kernel over `nbytes` (read nbytes + write nbytes)."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(warmup):
        dst.copy_(src)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(steps):
        dst.copy_(src)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    moved = 2 * src.numel() * 4
    print(json.dumps({"probe": "torch_copy", "bytes_per_launch": moved,
                      "avg_ms": round(ms, 5),
                      "gbps": round(moved / (ms * 1e-3) / 1e9, 1)}),
          flush=True)
    return 0


def segment_bytes(T, D, esize, nmod, part_bytes):
    """Algorithmic bytes of the packed calls (partial sums written by the
    stream kernel and read back by the finishing kernel)."""
    act = T * D * esize
    stats = 4 * T
    mod = nmod * D * esize
    return {
        "fwd": 2 * act + 2 * mod + 2 * stats,
        "bwd": 3 * act + mod + 2 * stats + 2 * part_bytes + 2 * nmod * D * 4,
    }


def packed_layout(synth, wl, seed):
    if wl.name == "mmdit_packed":
        lengths, mods = synth.mmdit_layout(wl.B)
        return lengths, mods, 2 * wl.B
    lengths = synth.pack_lengths(seed)
    return lengths, None, len(lengths)


def make_packed_job(A, torch, inp, dev, esize):
    job = {k: getattr(inp, k).to(dev) for k in ("x", "scale", "shift", "dy")}
    T, D = inp.x.shape
    nmod = inp.scale.shape[0]
    job["table"] = A.SegTable(inp.seg_offsets, inp.seg_mod)
    job["y"] = torch.empty_like(job["x"])
    job["dx"] = torch.empty_like(job["x"])
    job["mean"] = torch.empty(T, dtype=torch.float32, device=dev)
    job["rstd"] = torch.empty(T, dtype=torch.float32, device=dev)
    job["dscale"] = torch.empty(nmod, D, dtype=torch.float32, device=dev)
    job["dshift"] = torch.empty(nmod, D, dtype=torch.float32, device=dev)
    wbytes = A.bwd_segments_workspace_bytes(job["table"], D, inp.x.dtype)
    job["ws"] = torch.empty(max(wbytes, 1), dtype=torch.uint8, device=dev)
    job["tokens"] = T
    job["bytes"] = segment_bytes(T, D, esize, nmod, wbytes)
    return job


class _Batch:
    """x, scale, shift, dy of one batched call (host tensors)."""

    def __init__(self, x, scale, shift, dy):
        self.x, self.scale, self.shift, self.dy = x, scale, shift, dy


def unpacked_batches(inp):
    """The samples of a packed layout as batched calls: each run of
    consecutive segments of one length becomes one [B, L, D] call with the
    segments' modulation vectors gathered."""
    import torch
    off = [int(v) for v in inp.seg_offsets]
    mods = (list(range(len(off) - 1)) if inp.seg_mod is None
            else [int(m) for m in inp.seg_mod])
    by_len = {}
    for s in range(len(off) - 1):
        by_len.setdefault(off[s + 1] - off[s], []).append(s)
    out = []
    for L, segs in sorted(by_len.items()):
        if L == 0:
            continue
        x = torch.stack([inp.x[off[s]:off[s + 1]] for s in segs])
        dy = torch.stack([inp.dy[off[s]:off[s + 1]] for s in segs])
        idx = torch.tensor([mods[s] for s in segs])
        out.append(_Batch(x, inp.scale[idx], inp.shift[idx], dy))
    return out


def make_job(A, torch, inp, dev, esize):
    """Device buffers of one batch shape, plus its algorithmic bytes."""
    B, N, D = inp.x.shape
    dt = inp.x.dtype
    job = {k: getattr(inp, k).to(dev) for k in ("x", "scale", "shift", "dy")}
    job["y"] = torch.empty_like(job["x"])
    job["dx"] = torch.empty_like(job["x"])
    job["mean"] = torch.empty(B, N, dtype=torch.float32, device=dev)
    job["rstd"] = torch.empty(B, N, dtype=torch.float32, device=dev)
    job["dscale"] = torch.empty(B, D, dtype=torch.float32, device=dev)
    job["dshift"] = torch.empty(B, D, dtype=torch.float32, device=dev)
    wbytes = A.bwd_workspace_bytes(B, N, D, dt)
    job["ws"] = torch.empty(max(wbytes, 1), dtype=torch.uint8, device=dev)
    job["shape"] = (B, N, D)
    job["tokens"] = B * N
    part_rows = A.bwd_fused_plan(B, N, D, dt)["partial_rows"]
    job["bytes"] = algorithmic_bytes(
        B, N, D, esize, part_rows, A.plan("dmod", B, N, D, dt)["n_tiles"])
    return job


# Latent token counts of the pixel scan: 1, 3, 8, 15 and 21 frames of 30x52
# patches, and the schedule's 8190 and 16380 (all of them, like the
# schedule's lengths, not multiples of 128).
SWEEP_LENGTHS = (1560, 4680, 8190, 12480, 16380, 23400, 32760)
DP_GPUS = 8
REF_LENGTH = 16380


def cost_model(args) -> int:
    """Shape benchmark of the synthetic step, the cost-model fit and the
    bucket policies it implies; prints one JSON line."""
    import torch
    import adaln_fwd_amd as A
    from adaln_fwd_amd import sched
    import synth
    A.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    m_mem, m_comp, p_int = synth.MIXED_M_MEM, synth.MIXED_M_COMP, synth.MIXED_P
    D = synth.MIXED_SCHEDULE.D
    step = sched.SyntheticStep(D=D, heads=24)
    times = {}

    def measure(B, S):
        if (B, S) not in times:
            ms = step.run(B, S, iters=args.steps, warmup=args.warmup)
            times[(B, S)] = sorted(ms)[len(ms) // 2]
            log(f"B={B:3d} S={S:6d}: {times[(B, S)]:.3f} ms")
        return times[(B, S)]

    shapes = sched.sweep_shapes(SWEEP_LENGTHS, m_mem)
    log(f"shape benchmark: {len(shapes)} shapes, D={D}, 24 heads")
    for B, S in shapes:
        measure(B, S)
    Bs = [B for B, _ in shapes]
    Ss = [S for _, S in shapes]
    ts = [times[k] for k in shapes]
    model = sched.costfit(Bs, Ss, ts)
    mc = sched.m_comp_for(model.p, m_mem, REF_LENGTH)
    policies = {
        "token_equal": {S: max(1, m_mem // S) for S in synth.MIXED_LENGTHS},
        "dual_pages_constants": {S: A.bshape(S, m_mem, m_comp, p_int)
                                 for S in synth.MIXED_LENGTHS},
        "dual_fitted": sched.buckets(synth.MIXED_LENGTHS, m_mem, mc,
                                     model.p),
    }
    sched_draws = synth.mixed_schedule(args.seed)
    pol_out = {}
    for name, table in policies.items():
        # data-parallel estimate: the 64 draws dealt to DP_GPUS GPUs in
        # order, DP_GPUS buckets per step; a step lasts as long as its
        # slowest bucket
        steps_ms, steps_tok = [], []
        for i in range(0, len(sched_draws), DP_GPUS):
            group = sched_draws[i:i + DP_GPUS]
            steps_ms.append(max(measure(table[S], S) for S in group))
            steps_tok.append(sum(table[S] * S for S in group))
        t = [measure(B, S) for S, B in table.items()]
        tok = [B * S for S, B in table.items()]
        pol_out[name] = {
            "bucket_batch": {str(S): B for S, B in table.items()},
            "step_ms": {str(S): round(measure(B, S), 4)
                        for S, B in table.items()},
            "predicted_ms": {str(S): round(model.predict(B, S), 4)
                             for S, B in table.items()},
            "cv_step_time": round(sched.cv(t), 4),
            "dp_estimate": {
                "gpus": DP_GPUS,
                "tokens_per_s": round(sum(steps_tok) / (sum(steps_ms) * 1e-3),
                                      1),
                "busy_fraction": round(
                    sum(measure(table[S], S) for S in sched_draws)
                    / (DP_GPUS * sum(steps_ms)), 4),
            },
        }
    # attention's sensitivity to lengths that are multiples of 128
    aligned = {str(S): {"ms": round(measure(1, S), 4),
                        "ms_at_S-2": round(measure(1, S - 2), 4)}
               for S in (8192, 16384, 32768)}
    rec = {
        "metric": "cost model of the synthetic step (AdaLN fwd + fused "
                  "attention fwd and bwd + AdaLN bwd), 1 MI355X",
        "model": "t_ms = a + b * B * S^p",
        "fit": {"a": model.a, "b": model.b, "p": model.p, "rss": model.rss,
                "r2": model.r2},
        "samples": [{"B": B, "S": S, "ms": round(times[(B, S)], 4)}
                    for B, S in shapes],
        "pearson_r_token_equal_buckets": {
            "tokens": round(sched.pearson([m_mem // S * S for S in
                                           SWEEP_LENGTHS],
                                          [times[(m_mem // S, S)] for S in
                                           SWEEP_LENGTHS]), 4),
            "S^2": round(sched.pearson([S * S for S in SWEEP_LENGTHS],
                                       [times[(m_mem // S, S)] for S in
                                        SWEEP_LENGTHS]), 4),
        },
        "pearson_r": {
            "tokens": round(sched.pearson([B * S for B, S in shapes], ts), 4),
            "S^2": round(sched.pearson([S * S for S in Ss], ts), 4),
            "B*S^2": round(sched.pearson([B * S * S for B, S in shapes], ts),
                           4),
        },
        "m_comp": {"reference_length": REF_LENGTH, "fitted": mc,
                   "pages": m_comp,
                   "by_reference_length": {str(S): sched.m_comp_for(
                       model.p, m_mem, S) for S in synth.MIXED_LENGTHS}},
        "policies": pol_out,
        "alignment_probe_B1": aligned,
        "config": {"D": D, "heads": 24, "dtype": "bf16", "m_mem": m_mem,
                   "steps": args.steps, "warmup": args.warmup},
    }
    print(json.dumps(rec), flush=True)
    return 0


def eager_reference(args) -> int:
    """PyTorch's own unfused chain for the same workload -- layer_norm, then
    the modulation as separate elementwise ops, and its autograd backward --
    timed beside this library's calls (the analogue of the pages' unfused
    baseline); prints one JSON line."""
    import torch
    import torch.nn.functional as F
    import adaln_fwd_amd as A
    import synth
    A.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    wl = synth.BY_NAME[args.workload]
    if wl.B is None or wl in synth.PACKED:
        print("--eager-reference takes a batched workload", file=sys.stderr)
        return 2
    B, N, D = wl.shape
    inp = synth.make_inputs(wl, seed=args.seed)
    dev = torch.device("cuda", 0)
    x = inp.x.to(dev)
    dy = inp.dy.to(dev)
    scale = inp.scale.to(dev)
    shift = inp.shift.to(dev)

    def chain(x_, s_, h_):
        return (F.layer_norm(x_, (D,), eps=synth.EPS) * (1 + s_[:, None, :])
                + h_[:, None, :])

    def timed(fn, n):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * n)]
        for i in range(n):
            fn(ev[3 * i:3 * i + 3])
        torch.cuda.synchronize()
        fwd = [ev[3 * i].elapsed_time(ev[3 * i + 1]) for i in range(n)]
        bwd = [ev[3 * i + 1].elapsed_time(ev[3 * i + 2]) for i in range(n)]
        return sorted(fwd)[n // 2], sorted(bwd)[n // 2]

    xg = x.clone().requires_grad_(True)
    sg = scale.clone().requires_grad_(True)
    hg = shift.clone().requires_grad_(True)

    def torch_step(ev):
        ev[0].record()
        y = chain(xg, sg, hg)
        ev[1].record()
        torch.autograd.grad(y, (xg, sg, hg), dy)
        ev[2].record()

    y = torch.empty_like(x)
    dx = torch.empty_like(x)
    mean = torch.empty(B, N, device=dev)
    rstd = torch.empty(B, N, device=dev)
    ds = torch.empty(B, D, device=dev)
    dh = torch.empty(B, D, device=dev)
    ws = torch.empty(max(1, A.bwd_workspace_bytes(B, N, D, x.dtype)),
                     dtype=torch.uint8, device=dev)

    def lib_step(ev):
        ev[0].record()
        A.fwd(x, scale, shift, y=y, mean=mean, rstd=rstd)
        ev[1].record()
        A.bwd(dy, x, scale, mean, rstd, dx=dx, dscale=ds, dshift=dh,
              workspace=ws)
        ev[2].record()

    log(f"eager reference on {wl.name}: warm-up")
    timed(torch_step, args.warmup or 1)
    timed(lib_step, args.warmup or 1)
    log(f"timing {args.steps} steps each")
    t_fwd, t_bwd = timed(torch_step, args.steps)
    l_fwd, l_bwd = timed(lib_step, args.steps)

    # device memory a forward leaves allocated for its backward, beyond its
    # output y: autograd's saved tensors for the unfused chain, the saved
    # statistics (mean, rstd) for this library
    torch.cuda.synchronize()
    m0 = torch.cuda.memory_allocated()
    ye = chain(xg, sg, hg)
    torch.cuda.synchronize()
    eager_saved = torch.cuda.memory_allocated() - m0 - ye.numel() * \
        ye.element_size()
    del ye
    torch.cuda.synchronize()
    m0 = torch.cuda.memory_allocated()
    yl, ml, rl = A.fwd(x, scale, shift)
    torch.cuda.synchronize()
    lib_saved = torch.cuda.memory_allocated() - m0 - yl.numel() * \
        yl.element_size()
    del yl, ml, rl
    rec = {
        "metric": "median ms per call, PyTorch eager unfused chain vs this "
                  "library, 1 MI355X",
        "config": {"workload": wl.name, "B": B, "N": N, "D": D,
                   "dtype": wl.dtype},
        "torch_eager": {"fwd_ms": round(t_fwd, 4), "bwd_ms": round(t_bwd, 4)},
        "library": {"fwd_ms": round(l_fwd, 4), "bwd_ms": round(l_bwd, 4)},
        "speedup": {"fwd": round(t_fwd / l_fwd, 3),
                    "bwd": round(t_bwd / l_bwd, 3),
                    "fwd+bwd": round((t_fwd + t_bwd) / (l_fwd + l_bwd), 3)},
        "saved_for_backward_bytes": {"torch_eager": int(eager_saved),
                                     "library": int(lib_saved),
                                     "per_token_eager": round(
                                         eager_saved / (B * N), 2),
                                     "per_token_library": round(
                                         lib_saved / (B * N), 2)},
        "torch": torch.__version__,
    }
    print(json.dumps(rec), flush=True)
    return 0


def stream_probe(args) -> int:
    """The streaming probes (bench_probe.hip) on buffers of the workload's
    activation size; prints one JSON line."""
    import torch
    import adaln_fwd_amd as A
    import synth
    A.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    wl = synth.BY_NAME[args.workload]
    if wl.B is None:
        print("--probe takes a workload with one shape", file=sys.stderr)
        return 2
    esize = 4 if wl.dtype == "f32" else 2
    full = wl.B * wl.N * wl.D * esize
    n = full // 10240 * 10240
    fa = torch.empty(full, dtype=torch.uint8, device="cuda").random_()
    fb = torch.empty_like(fa).random_()
    fd = torch.empty_like(fa)
    a, b, d = fa[:n], fb[:n], fd[:n]
    out = {"probe": "bench_stream_probe", "workload": wl.name,
           "buffer_bytes": n}

    def timed(launch, nbytes, streams):
        for _ in range(args.warmup or 1):
            launch()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(args.steps):
            launch()
        ev[1].record()
        torch.cuda.synchronize()
        ms = ev[0].elapsed_time(ev[1]) / args.steps
        return {"avg_ms": round(ms, 5),
                "gbps": round(streams * nbytes / (ms * 1e-3) / 1e9, 1)}

    for kind, name, streams in ((0, "copy", 2), (1, "read2_write1", 3)):
        out[name] = timed(lambda: run_probe(kind, a, d, b=b), n, streams)
    out["read2_write1"]["result_ok"] = bool(torch.equal(d, a ^ b))

    # The same bytes walked in the kernels' sample windows (grid and bps of
    # the forward's plan for the copy, of the backward's for two reads + one
    # write), at several skews, beside one flat window over the batch.  The
    # forward of one-wavefront rows has no sample windows (bps 0): its grid
    # covers the rows, which the flat case with bps = grid walks the same way.
    row = wl.D * esize
    if row % 1024 == 0 and 1 <= row // 1024 <= 10:
        rk = row // 1024
        dt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
        wins = []
        for kind, name, streams, op in ((0, "copy", 2, "fwd"),
                                        (1, "read2_write1", 3, "bwd")):
            pl = A.plan(op, wl.B, wl.N, wl.D, dt)
            grid, bps = pl["workgroups"], pl["bps"]
            cases = [(1, wl.B * wl.N, grid, 0)]
            if wl.B > 1 and bps > 0:
                cases += [(wl.B, wl.N, bps, sk)
                          for sk in sorted({0, 64, 97, pl.get("skew", 0)})]
            for B_, N_, bps_, sk in cases:
                r = timed(lambda: run_window_probe(kind, fa, fd, B_, N_, rk,
                                                   bps_, grid, sk, b=fb),
                          full, streams)
                r.update({"pattern": name, "windows": B_, "grid": grid,
                          "bps": bps_, "skew": sk})
                want = fa ^ fb if kind == 1 else fa
                r["result_ok"] = bool(torch.equal(fd, want))
                wins.append(r)
        out["windows"] = wins
    print(json.dumps(out), flush=True)
    ok = out["read2_write1"]["result_ok"] and all(
        w["result_ok"] for w in out.get("windows", []))
    return 0 if ok else 1


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="large_model")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--event-every", type=int, default=4, metavar="K",
                    help="bracket the dominant kernel with HIP events on "
                         "every K-th timed step (default 4)")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle time for cpu_baseline (0: skip)")
    ap.add_argument("--traffic-from", metavar="DIR",
                    help="print per-kernel HBM traffic computed from the "
                         "rocprofv3 --pmc CSVs under DIR and exit")
    ap.add_argument("--bucket", type=int, default=None, metavar="S",
                    help="mixed_schedule: run only the buckets of length S "
                         "(one shape), as a single-shape workload")
    ap.add_argument("--unfused", action="store_true",
                    help="batched workloads: the backward as the pages' "
                         "separate kernels (adaln_bwd_dx, then adaln_bwd_dmod:"
                         " the (d_tile, n_tile) grid and its second stage) "
                         "instead of the fused single pass")
    ap.add_argument("--unpacked", action="store_true",
                    help="packed workloads: run the samples as batched "
                         "calls, one per segment length, instead")
    ap.add_argument("--cold", dest="cold", action="store_true",
                    default=True,
                    help="also time each call after evicting the caches, "
                         "up to 20 times each, after the timed region "
                         "(reported under 'cold'; single-call workloads; "
                         "the default)")
    ap.add_argument("--no-cold", dest="cold", action="store_false",
                    help="skip the cold-cache timings")
    ap.add_argument("--cost-model", action="store_true",
                    help="shape benchmark of the synthetic step, cost-model "
                         "fit and bucket policies (--steps/--warmup per shape)")
    ap.add_argument("--eager-reference", action="store_true",
                    help="time PyTorch's unfused eager chain (layer_norm, "
                         "modulation, autograd backward) beside this library "
                         "on the workload")
    ap.add_argument("--probe", action="store_true",
                    help="time the streaming probes of bench_probe.hip (copy; "
                         "2 reads + 1 write) on buffers of the workload's "
                         "activation size, flat and in the kernels' sample "
                         "windows")
    ap.add_argument("--copy-probe", action="store_true",
                    help="time torch's device copy of one workload-sized "
                         "tensor instead (achievable-bandwidth reference and "
                         "counter calibration)")
    args = ap.parse_args(argv)

    if args.traffic_from:
        import synth
        wl = synth.BY_NAME[args.workload]
        esize = 4 if wl.dtype == "f32" else 2
        B, N, D = single_shape(synth, wl, args.bucket)
        copy_bytes = B * N * D * esize
        print(json.dumps(traffic_from_counters(
            args.traffic_from, workload_name(wl, args.bucket), copy_bytes),
            indent=1))
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this operator is measured on a "
              "single MI355X and has no multi-GPU path (requested "
              f"--gpus {args.gpus}, WORLD_SIZE={world}).", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2
    if args.cost_model:
        return cost_model(args)
    if args.eager_reference:
        return eager_reference(args)
    if args.probe:
        return stream_probe(args)

    import torch
    import adaln_fwd_amd as A
    import synth

    A.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    wl = synth.BY_NAME[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    dt = synth.torch_dtype(wl.dtype)
    esize = torch.empty((), dtype=dt).element_size()

    packed = wl in synth.PACKED
    first_inp = None
    if packed:
        lengths, mods, nmod = packed_layout(synth, wl, args.seed)
        D = wl.D
        if args.copy_probe:
            return copy_probe(sum(lengths) * D * esize, args.steps,
                              args.warmup)
        log(f"packed workload {wl.name}: {len(lengths)} segments, "
            f"{sum(lengths)} tokens, D={D}, {nmod} modulation vectors")
        pinp = synth.make_packed(wl, lengths, mods, nmod=nmod, seed=args.seed)
        if args.unpacked:
            order = [make_job(A, torch, b, dev, esize)
                     for b in unpacked_batches(pinp)]
            packed = False
        else:
            order = [make_packed_job(A, torch, pinp, dev, esize)]
        del pinp
    elif wl.B is None:
        # the mixed-length schedule: one step = every bucket, in order
        sched = synth.mixed_schedule(args.seed)
        shapes = {S: A.bshape(S, synth.MIXED_M_MEM, synth.MIXED_M_COMP,
                              synth.MIXED_P) for S in sorted(set(sched))}
        D = wl.D
        if args.copy_probe:
            big = (shapes[args.bucket] * args.bucket if args.bucket in shapes
                   else max(b * S for S, b in shapes.items()))
            return copy_probe(big * D * esize, args.steps, args.warmup)
        if args.bucket is not None:
            # one bucket shape of the schedule on its own: a step is its
            # forward + backward
            if args.bucket not in shapes:
                print(f"--bucket must be one of {sorted(shapes)}",
                      file=sys.stderr)
                return 2
            S = args.bucket
            B, N = shapes[S], S
            log(f"bucket S={S} of the schedule: B={B} N={S} D={D}")
            first_inp = synth.make_inputs(synth.mixed_bucket(B, S),
                                          seed=args.seed,
                                          bucket=sched.index(S))
            order = [make_job(A, torch, first_inp, dev, esize)]
        else:
            log(f"schedule of {len(sched)} buckets, D={D}: drawing one input "
                f"set per bucket shape {shapes}")
            jobs = {}
            for S, Bk in shapes.items():
                inp = synth.make_inputs(synth.mixed_bucket(Bk, S),
                                        seed=args.seed, bucket=sched.index(S))
                jobs[S] = make_job(A, torch, inp, dev, esize)
                if S == sched[0]:
                    first_inp = inp  # the CPU baseline's sample
            order = [jobs[S] for S in sched]
    else:
        B, N, D = wl.shape
        if args.copy_probe:
            return copy_probe(B * N * D * esize, args.steps, args.warmup)
        log(f"workload {wl.name} B={B} N={N} D={D} {wl.dtype}: drawing inputs")
        first_inp = synth.make_inputs(wl, seed=args.seed)
        order = [make_job(A, torch, first_inp, dev, esize)]

    if packed:
        names = ("fwd", "bwd")
    elif args.unfused:
        names = ("fwd", "bwd_dx", "bwd_dmod")
    else:
        names = ("fwd", "bwd_fused", "bwd_finish")

    def job_calls(job):
        """The calls of one job's forward + backward, in order."""
        if packed:
            return [
                lambda: A.fwd_segments(
                    job["x"], job["scale"], job["shift"], job["table"],
                    y=job["y"], mean=job["mean"], rstd=job["rstd"],
                    stream=stream),
                lambda: A.bwd_segments(
                    job["dy"], job["x"], job["scale"], job["mean"],
                    job["rstd"], job["table"], dx=job["dx"],
                    dscale=job["dscale"], dshift=job["dshift"],
                    workspace=job["ws"], stream=stream)]
        if args.unfused:
            return [
                lambda: A.fwd(job["x"], job["scale"], job["shift"],
                              y=job["y"], mean=job["mean"], rstd=job["rstd"],
                              stream=stream),
                lambda: A.bwd_dx(job["dy"], job["x"], job["scale"],
                                 job["mean"], job["rstd"], dx=job["dx"],
                                 stream=stream),
                lambda: A.bwd_dmod(job["dy"], job["x"], job["mean"],
                                   job["rstd"], dscale=job["dscale"],
                                   dshift=job["dshift"], workspace=job["ws"],
                                   stream=stream)]
        return [
            lambda: A.fwd(job["x"], job["scale"], job["shift"], y=job["y"],
                          mean=job["mean"], rstd=job["rstd"], stream=stream),
            lambda: A.bwd_fused(job["dy"], job["x"], job["scale"],
                                job["mean"], job["rstd"], dx=job["dx"],
                                workspace=job["ws"], stream=stream),
            lambda: A.bwd_finish(job["ws"], *job["shape"], dt,
                                 dscale=job["dscale"], dshift=job["dshift"],
                                 stream=stream)]

    plan = [job_calls(job) for job in order]
    nk = len(names)

    def step(ev=None, at=()):
        """One step; ev[j][b] is recorded before call b of job j (b = nk:
        after its last call) for every boundary b in `at`."""
        for j, calls in enumerate(plan):
            for b, call in enumerate(calls):
                if ev is not None and b in at:
                    ev[j][b].record(stream)
                call()
            if ev is not None and nk in at:
                ev[j][nk].record(stream)

    calls = dict(zip(names, plan[0])) if len(order) == 1 else {}
    # The roofline's kernel: the backward's main pass (the largest), timed
    # inside the timed region with one event on each side; events on every
    # kernel boundary cost about 2% of the step (each record is a marker with
    # a cache flush), so the full per-kernel breakdown runs after it.
    dom = names.index("bwd" if packed else
                      "bwd_dx" if args.unfused else "bwd_fused")

    def new_events():
        return [[[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)]
                 for _ in order] for _ in range(args.steps)]

    log(f"warm-up {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    dom_events = new_events()
    log(f"timing {args.steps} steps")
    # HIP events bracket the dominant kernel on every `every`-th timed step
    # (each event record costs the step a few microseconds)
    every = max(1, min(args.event_every, args.steps))
    sampled = list(range(0, args.steps, every))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if i % every == 0:
            step(dom_events[i], at=(dom, dom + 1))
        else:
            step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = 1e3 * elapsed / args.steps

    log(f"per-kernel breakdown: {args.steps} more steps")
    events = new_events()
    for i in range(args.steps):
        step(events[i], at=tuple(range(nk + 1)))
    torch.cuda.synchronize()

    # per-kernel time and algorithmic bytes, summed over the jobs of a step
    tot_ms = {n: 0.0 for n in names}
    tot_bytes = {n: 0 for n in names}
    for j, job in enumerate(order):
        for i, n in enumerate(names):
            tot_ms[n] += sum(ev[j][i].elapsed_time(ev[j][i + 1])
                             for ev in events) / args.steps
            tot_bytes[n] += job["bytes"][n]
    launches = len(order)
    kernels = {n: {"avg_ms": round(tot_ms[n] / launches, 5),
                   "bytes": int(tot_bytes[n] / launches),
                   "gbps": round(tot_bytes[n] / (tot_ms[n] * 1e-3) / 1e9, 1)}
               for n in names}
    if launches == 1:
        # spread over the timed steps (one launch of each per step)
        for i, n in enumerate(names):
            d = sorted(ev[0][i].elapsed_time(ev[0][i + 1]) for ev in events)
            kernels[n]["p10_ms"] = round(d[len(d) // 10], 5)
            kernels[n]["median_ms"] = round(d[len(d) // 2], 5)
            kernels[n]["p90_ms"] = round(d[(9 * len(d)) // 10], 5)

    cold = None
    if args.cold and launches == 1:
        # each call after a 1 GiB write that evicts the caches (L2 and the
        # 256 MB memory-side cache), outside the timed region above
        scrub = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        per = {n: [] for n in names}
        cev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for _ in range(min(args.steps, 20)):
            for i, n in enumerate(names):
                scrub.fill_(1.0)
                cev[0].record(stream)
                calls[n]()
                cev[1].record(stream)
                torch.cuda.synchronize()
                per[n].append(cev[0].elapsed_time(cev[1]))
        del scrub
        cold = {}
        for n in names:
            d = sorted(per[n])
            b = order[0]["bytes"][n]
            cold[n] = {"median_ms": round(d[len(d) // 2], 5),
                       "p10_ms": round(d[len(d) // 10], 5),
                       "p90_ms": round(d[(9 * len(d)) // 10], 5),
                       "gbps": round(b / (d[len(d) // 2] * 1e-3) / 1e9, 1)}
    probe = None
    if launches == 1:
        # what HBM sustains for the dominant kernel's access pattern (two
        # read streams, one write stream) with no arithmetic, on buffers of
        # the workload's size; after the timed region, not part of `value`
        job = order[0]
        row = 10240
        n = (job["x"].numel() * job["x"].element_size()) // row * row
        if n > 0:
            a = job["x"].view(-1).view(torch.uint8)[:n]
            b = job["dy"].view(-1).view(torch.uint8)[:n]
            d = job["y"].view(-1).view(torch.uint8)[:n]
            for _ in range(3):
                run_probe(1, a, d, b=b, stream=stream)
            pev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            pev[0].record(stream)
            reps = 10
            for _ in range(reps):
                run_probe(1, a, d, b=b, stream=stream)
            pev[1].record(stream)
            torch.cuda.synchronize()
            pms = pev[0].elapsed_time(pev[1]) / reps
            probe = {"pattern": "2 reads + 1 write, nontemporal, no "
                                "arithmetic (bench_probe.hip, kind 1)",
                     "bytes": 3 * n, "avg_ms": round(pms, 5),
                     "gbps": round(3 * n / (pms * 1e-3) / 1e9, 1)}
    step_bytes = sum(tot_bytes.values())
    tokens = sum(job["tokens"] for job in order)
    gbps = step_bytes / (ms_step * 1e-3) / 1e9
    tokens_s = tokens / (ms_step * 1e-3)

    dname = names[dom]
    dom_ms = sum(dom_events[i][j][dom].elapsed_time(dom_events[i][j][dom + 1])
                 for i in sampled for j in range(len(order))) / len(sampled)
    src_hash = kernel_source_hash()
    achieved = tot_bytes[dname] / (dom_ms * 1e-3) / 1e9
    roofline = {
        "kernel": dname,
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4),
        "traffic": load_traffic(dname, workload_name(wl, args.bucket),
                                kernel_source_hash(dname)),
        "algorithmic_bytes_per_launch": int(tot_bytes[dname] / launches),
        "avg_launch_ms": round(dom_ms / launches, 5),
        "timed_launches": len(sampled) * launches,
    }
    if probe is not None:
        probe["kernel_frac_of_probe"] = round(achieved / probe["gbps"], 4)
        roofline["achievable_probe"] = probe
    if args.unfused and not packed:
        config_backward = "unfused: dx kernel, then the (d_tile, n_tile) grid"
    else:
        config_backward = None
    if wl in synth.PACKED:
        config = {"workload": wl.name, "layout": "batched per length"
                  if args.unpacked else "packed", "segments": len(lengths),
                  "calls": len(order), "D": D, "tokens": tokens,
                  "dtype": wl.dtype, "modulation_vectors": nmod,
                  "lengths": {str(L): lengths.count(L)
                              for L in sorted(set(lengths))}}
    elif wl.B is None and args.bucket is not None:
        config = {"workload": f"{wl.name} bucket S={args.bucket}", "B": B,
                  "N": N, "D": D, "dtype": wl.dtype}
    elif wl.B is None:
        config = {"workload": wl.name, "buckets": len(order), "D": D,
                  "tokens": tokens, "dtype": wl.dtype,
                  "bucket_batch": {str(S): b for S, b in shapes.items()}}
    else:
        config = {"workload": wl.name, "B": B, "N": N, "D": D,
                  "dtype": wl.dtype}

    if config_backward:
        config["backward"] = config_backward
    cpu = None
    if args.cpu_budget > 0 and first_inp is not None:
        log(f"cpu baseline: oracle for ~{args.cpu_budget:.0f} s")
        cpu = cpu_baseline(first_inp, args.cpu_budget)

    rec = {
        "metric": METRIC,
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": config,
        "hbm_gbps": round(gbps, 1),
        "hbm_frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "cold": cold,
        "kernel_source_hash": src_hash,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

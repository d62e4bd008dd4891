"""Benchmark of the fused BitDelta linear on one MI355X.

A step is one decode pass over one Llama-70B-shaped layer: the seven
projections (q, k, v, o 8192/1024-wide, gate/up 28672x8192, down 8192x28672)
at M = 1, 4 and 16 tokens, 21 fused-linear launches, each reading bf16 base
weights, packed signs and per-row α of its own projection, in M-major order
(the seven projections at M = 1, then 4, then 16).  Three full copies of the
layer's weights are rotated, so between two reads of one matrix at least
1.8 GB of other weights pass and nothing is served from the 256 MB MALL.  ``value`` is algorithmic bytes per step (base + signs + α +
x + y) x steps / wall time, in GB/s.

In the same run, outside the timed steps: the prefill path (the seven
projections at M = 2048, per-matrix α, TFLOP/s), the grouped path (one
8192x28672 base, 14 deltas, 256 tokens), the compression pass (gate,
per-row α), and the CPU oracle on a bounded sample (``cpu_baseline``).

Inputs are seeded synthetic tensors (bf16 base ~ N(0, 0.02^2), Laplace(0, 1e-3)
deltas, bf16 activations ~ N(0, 1)), generated on the GPU.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2516.6  # dense bf16 MFMA, TFLOP/s
ROTATE = 3
CALIB_BYTES = 1 << 30
# VALU issue peak: 256 CUs x 4 SIMDs at 2.4 GHz, 32 lanes per clock per SIMD,
# so a wave64 instruction every 2 clocks (the chip's 157.3 TFLOP/s fp32 vector
# figure is 256 x 4 x 2.4 GHz x 32 lanes x 2 flop of FMA).  Two waves of
# independent v_add_f32 on one SIMD were measured at 2.4 clocks per
# instruction; a single wave issues one every ~4.8 clocks.
VALU_PEAK_WAVE_INSTR_PER_S = 256 * 4 * 2.4e9 / 2


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def linear_bytes(M, N, K, per_row=True):
    return 2 * N * K + N * K // 8 + 4 * (N if per_row else 1) + 2 * M * K + 4 * M * N


class Call:
    """A pre-validated bd_linear call (pointer arguments resolved once) so the
    timed loop measures the GPU, not Python argument handling."""

    def __init__(self, lib, x, w, s, a, y, mode, stream):
        import torch
        self.fn = lib.bd_linear
        M, K = x.shape
        N = w.shape[0]
        nbytes = lib.bd_linear_workspace_bytes(M, N, K)
        self.ws = (torch.empty((nbytes + 15) // 16 * 4, dtype=torch.float32, device=x.device)
                   if nbytes else None)
        self.args = (ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(w.data_ptr()),
                     ctypes.c_void_p(s.data_ptr()), ctypes.c_void_p(a.data_ptr()), mode,
                     ctypes.c_void_p(y.data_ptr()), M, N, K,
                     ctypes.c_void_p(self.ws.data_ptr() if nbytes else 0), nbytes, stream)

    def __call__(self):
        st = self.fn(*self.args)
        if st != 0:
            raise RuntimeError("bd_linear failed with status %d" % st)


class GroupedCall:
    """A pre-validated bd_linear_grouped call: pointer arrays and workspace
    resolved once, so a loop of thousands of launches measures the GPU."""

    def __init__(self, lib, x, ids, w, signs, alphas, mode, y, ws, ws_bytes, stream, planned=False):
        G = len(signs)
        self.fn = lib.bd_linear_grouped_planned if planned else lib.bd_linear_grouped
        self.sp = (ctypes.c_void_p * G)(*[t.data_ptr() for t in signs])
        self.ap = (ctypes.c_void_p * G)(*[t.data_ptr() for t in alphas])
        M, K = x.shape
        N = w.shape[0]
        self.args = (ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(ids.data_ptr()),
                     ctypes.c_void_p(w.data_ptr()), self.sp, self.ap, mode, G,
                     ctypes.c_void_p(y.data_ptr()), M, N, K, ctypes.c_void_p(ws.data_ptr()),
                     ws_bytes, stream)

    def __call__(self):
        st = self.fn(*self.args)
        if st != 0:
            raise RuntimeError("bd_linear_grouped failed with status %d" % st)


def source_digest():
    """sha256 over the kernel sources; traffic figures taken from counters are
    reported only while the sources they were measured on are unchanged."""
    import hashlib
    h = hashlib.sha256()
    src = os.path.join(ROOT, "tenant_serving_amd", "csrc")
    for name in sorted(os.listdir(src)):
        if name.endswith((".hip", ".h", ".cpp")):
            h.update(name.encode())
            h.update(open(os.path.join(src, name), "rb").read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by the copy calibration), or None
    if there is none for this kernel or the sources changed since."""
    path = os.path.join(ROOT, "profiles", "traffic_decode_layer.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("source_sha256") != source_digest():
        return None
    for line in open(path):
        parts = line.split()
        if len(parts) >= 4 and parts[0] == "kernel" and parts[1] == kernel:
            return int(float(parts[3]))
    return None


def clock_snapshot():
    """Current shader (sclk) and memory (mclk) clock of the GPU, from the
    driver's DPM tables in sysfs (the level marked '*'); None where not
    readable."""
    import glob
    import re
    out = {}
    for card in sorted(glob.glob("/sys/class/drm/card*/device")):
        got = {}
        for key, fname in (("sclk_MHz", "pp_dpm_sclk"), ("mclk_MHz", "pp_dpm_mclk"), ("fclk_MHz", "pp_dpm_fclk")):
            try:
                for line in open(os.path.join(card, fname)):
                    if "*" in line:
                        m = re.search(r"(\d+)\s*[Mm]hz", line)
                        if m:
                            got[key] = int(m.group(1))
            except OSError:
                pass
        if got:
            out[os.path.basename(os.path.dirname(card))] = got
    return out or None


def committed_counters(fname, kernel):
    """Counters of `kernel` from a committed rocprofv3 summary under
    profiles/ (lines 'kernel <name> <counter> <value>'), or None if there is
    none or the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", fname)
    if not os.path.exists(path):
        return None
    sha = None
    res = {}
    for line in open(path):
        if line.startswith("source_sha256:"):
            sha = line.split(":", 1)[1].strip()
        parts = line.split()
        if len(parts) == 4 and parts[0] == "kernel" and parts[1] == kernel:
            res[parts[2]] = float(parts[3])
    if sha != source_digest() or not res:
        return None
    return res


def stream_read_regime(torch, dev, stream):
    """The achievable read rate, from libbdprobe.so (plain reads, no
    arithmetic): a grid-stride stream of 16-byte non-temporal loads over
    2 GiB, and over a 28672 x 8192 bf16 matrix two row patterns (1 KiB of a
    row per load instruction): two rows per wave walked in batches, and the
    one-token GEMV's present one, a 4-wave workgroup per row pair.
    Two buffers alternate so nothing is served from the 256 MB MALL.  Context
    for the decode fractions; the graded denominator stays 8 TB/s."""
    lib = ctypes.CDLL(os.path.join(ROOT, "tenant_serving_amd", "libbdprobe.so"))
    lib.bd_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    lib.bd_probe_stream_read.restype = ctypes.c_int32
    lib.bd_probe_stream_rows.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    lib.bd_probe_stream_rows.restype = ctypes.c_int32
    lib.bd_probe_stream_pairs.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                          ctypes.c_int32, ctypes.c_void_p]
    lib.bd_probe_stream_pairs.restype = ctypes.c_int32
    lib.bd_probe_stream_read_threads.argtypes = [ctypes.c_int32]
    lib.bd_probe_stream_read_threads.restype = ctypes.c_int64
    ncu = torch.cuda.get_device_properties(dev).multi_processor_count
    out = torch.empty(lib.bd_probe_stream_read_threads(ncu), dtype=torch.int32, device=dev)
    sh = ctypes.c_void_p(stream.cuda_stream)

    def measure(calls, nbytes):
        # 10 launches back to back (the buffers alternating) between one event
        # pair, three times; the best of the three.  An event pair per launch
        # would add its few microseconds to each 0.1-0.4 ms launch.
        for c in calls:
            if c() != 0:
                return None
        best = None
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(10):
                calls[i % len(calls)]()
            e1.record(stream)
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3 / 10
            best = t if best is None or t < best else best
        return round(nbytes / best / 1e9, 1)

    variants = {}
    nbytes = 2 << 30
    bufs = [torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev) for _ in range(2)]
    for wpc in (4, 8, 16):
        for loads in (4, 8):
            calls = [lambda b=b: lib.bd_probe_stream_read(ctypes.c_void_p(b.data_ptr()), nbytes,
                                                          ctypes.c_void_p(out.data_ptr()), ncu, wpc, loads, sh)
                     for b in bufs]
            r = measure(calls, nbytes)
            if r is None:
                return {"error": "probe launch failed"}
            variants["stream: %d wg/CU, %d loads/lane" % (wpc, loads)] = r
    del bufs
    rows, row_bytes = 28672, 8192 * 2
    bufs = [torch.ones(rows * row_bytes // 2, dtype=torch.bfloat16, device=dev) for _ in range(2)]
    for wpc in (4, 8, 16):
        for batch in (2, 4):
            calls = [lambda b=b: lib.bd_probe_stream_rows(ctypes.c_void_p(b.data_ptr()), rows, row_bytes,
                                                          ctypes.c_void_p(out.data_ptr()), ncu, wpc, batch, sh)
                     for b in bufs]
            r = measure(calls, rows * row_bytes)
            if r is None:
                return {"error": "probe launch failed"}
            variants["rows: %d wg/CU, %d KiB per row in flight" % (wpc, batch)] = r
    calls = [lambda b=b: lib.bd_probe_stream_pairs(ctypes.c_void_p(b.data_ptr()), rows, row_bytes,
                                                   ctypes.c_void_p(out.data_ptr()), ncu, sh)
             for b in bufs]
    r = measure(calls, rows * row_bytes)
    if r is None:
        return {"error": "probe launch failed"}
    variants["pairs: one 4-wave workgroup per row pair, whole rows at once"] = r
    del bufs, out
    torch.cuda.empty_cache()
    best = max(variants, key=lambda k: variants[k])
    log("stream read: %.1f GB/s (%s)" % (variants[best], best))
    return {"GB/s": variants[best], "frac": round(variants[best] / HBM_PEAK_GBS, 4), "best": best,
            "variants_GB/s": variants,
            "what": "plain reads, no arithmetic: a grid-stride stream of 16-byte non-temporal loads over 2 GiB, "
                    "and over a 28672x8192 bf16 matrix two row patterns (1 KiB of a row per load instruction): "
                    "two rows per wave walked in batches, and one 4-wave workgroup per row pair reading whole "
                    "rows at once (the one-token GEMV's); two buffers alternating, 10 launches back to back "
                    "per event pair, best of 3 and best launch shape; the practical read rate, context only"}


def timed_launches(torch, launches, reps, stream):
    """Run the list of callables `reps` times with a HIP event pair around each
    launch on `stream`; returns per-launch durations in seconds [reps][len]."""
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in launches] for _ in range(reps)]
    for r in range(reps):
        for i, fn in enumerate(launches):
            ev[r][i][0].record(stream)
            fn()
            ev[r][i][1].record(stream)
    torch.cuda.synchronize()
    return [[a.elapsed_time(b) * 1e-3 for a, b in row] for row in ev]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extra", action="store_true", help="skip every regime beside the decode step")
    ap.add_argument("--regimes", default="all",
                    help="comma list of regimes beside the decode step: prefill, grouped, compress, "
                         "cache, file, unfused, monosoup, stream, full_share (default: all)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=16.0,
                    help="CPU time budget of the oracle baseline, all samples together")
    ap.add_argument("--events", choices=("dominant", "all"), default="dominant",
                    help="in the timed steps, bracket only the dominant kernel's launches with "
                         "events (default) or every launch; consecutive marked launches share one "
                         "event pair")
    ap.add_argument("--event-every", type=int, default=4,
                    help="bracket launches with events in every n-th timed step (1 = every step)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB -> 1 GiB elementwise copy (torch.neg on bf16), "
                         "the reference dispatch for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE")
    ap.add_argument("--workload", choices=("decode-layer", "full-share"), default="decode-layer",
                    help="decode-layer (default): one 70B-shaped layer at M = 1, 4, 16; "
                         "full-share: 80 layers and 14 resident variants, a 512-token mixed "
                         "prefill and 64 mixed decode steps")
    ap.add_argument("--layers", type=int, default=80, help="full-share: layers")
    ap.add_argument("--decode-steps", type=int, default=64, help="full-share: decode steps")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the fused BitDelta linear runs and is measured on a "
              "single MI355X (each GPU would serve whole requests on its own copy of the base); "
              "there is no multi-GPU run.", file=sys.stderr)
        sys.exit(2)

    import torch
    import tenant_serving_amd as bd
    from tenant_serving_amd import synth

    lib = bd.library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    props = torch.cuda.get_device_properties(dev)
    log("device:", props.name, getattr(props, "gcnArchName", ""))

    if args.calib_copy:
        src = torch.ones(CALIB_BYTES // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
        log("copy calibration: 3 x torch.neg over %d bytes in, %d out" % (CALIB_BYTES, CALIB_BYTES))

    if args.workload == "full-share":
        print(json.dumps(full_share(args, torch, bd, synth, lib, dev, stream, sh)), flush=True)
        return

    clocks = {"before": clock_snapshot()}

    # ---------------------------------------------------------------- decode
    layer = synth.LLAMA70B_LAYER
    Ms = (1, 4, 16)
    copies = []
    seed = synth.SEEDS["decode"]
    for r in range(ROTATE):
        proj = {}
        for name, N, K in layer:
            w, d, _ = synth.projection(N, K, 1, seed=seed * 1000 + r * 10 + len(proj), device=dev)
            s, a = bd.bd_compress(d, bd.BD_ALPHA_PER_ROW)
            del d
            proj[name] = (w, s, a)
        copies.append(proj)
        torch.cuda.synchronize()
    xs = {K: synth.activations(synth.generator(seed, dev), 16, K, dev) for K in (8192, 28672)}
    ys = {(name, M): torch.empty((M, N), dtype=torch.float32, device=dev)
          for name, N, K in layer for M in Ms}
    # M-major order: the seven projections at M = 1, then at 4, then at 16,
    # so 1.8 GB of other weights pass between two reads of one matrix and no
    # launch finds its weights in the 256 MB MALL
    steps_calls = []
    for r in range(ROTATE):
        calls = []
        for M in Ms:
            for name, N, K in layer:
                w, s, a = copies[r][name]
                calls.append(((name, N, K, M), Call(lib, xs[K][:M], w, s, a, ys[(name, M)],
                                                      bd.BD_ALPHA_PER_ROW, sh)))
        steps_calls.append(calls)
    step_bytes = sum(linear_bytes(M, N, K) for _, N, K in layer for M in Ms)

    def run_step(i):
        for _, c in steps_calls[i % ROTATE]:
            c()

    for i in range(args.warmup):
        run_step(i)
    torch.cuda.synchronize()
    log("decode warmup done")

    # Per-launch durations of every projection, from a separate pass of
    # ROTATE * 2 steps with events around every launch (not timed for value).
    names = [(key, bd.bd_linear_path(key[3], key[1], key[2])) for key, _ in steps_calls[0]]
    prof_steps = 2 * ROTATE
    pev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in steps_calls[0]] for _ in range(prof_steps)]
    for i in range(prof_steps):
        for j, (_, c) in enumerate(steps_calls[i % ROTATE]):
            pev[i][j][0].record(stream)
            c()
            pev[i][j][1].record(stream)
    torch.cuda.synchronize()
    per_sym = {}
    per_proj = {}
    for i in range(prof_steps):
        for j, (key, sym) in enumerate(names):
            name, N, K, M = key
            dt = pev[i][j][0].elapsed_time(pev[i][j][1]) * 1e-3
            b = linear_bytes(M, N, K)
            e = per_sym.setdefault(sym, [0.0, 0, 0])
            e[0] += dt
            e[1] += 1
            e[2] += b
            p = per_proj.setdefault("%s M=%d" % (name, M), [0.0, 0, b])
            p[0] += dt
            p[1] += 1
    dominant = max(per_sym, key=lambda k: per_sym[k][0])

    # Timed region: exactly `steps` steps.  HIP events on the launch stream
    # bracket the dominant kernel's launches (all launches with --events all)
    # in every --event-every'th timed step, so its average duration is
    # measured live.  A run of consecutive marked launches (the seven M = 1
    # projections, say) shares one event pair: each recorded event holds the
    # queue for a few microseconds, which would otherwise be counted into the
    # kernel's time and lower the step rate it is meant to explain.
    every = args.events == "all"
    marked = [every or sym == dominant for _, sym in names]
    if args.event_every < 1:
        raise SystemExit("--event-every must be >= 1")
    dom = [sym == dominant for _, sym in names]
    runs = []  # (first launch, last launch) of each run of marked launches
    j = 0
    while j < len(names):
        if marked[j]:
            e = j
            while e + 1 < len(names) and marked[e + 1] and dom[e + 1] == dom[j] and (dom[j] or not every):
                e += 1
            runs.append((j, e))
            j = e + 1
        else:
            j += 1
    run_start = {a: r for r, (a, _) in enumerate(runs)}
    run_end = {b: r for r, (_, b) in enumerate(runs)}
    sampled = [i % args.event_every == 0 for i in range(args.steps)]
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in runs]
          if sampled[i] else None for i in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        row = ev[i]
        for j, (_, c) in enumerate(steps_calls[i % ROTATE]):
            if row is not None and j in run_start:
                row[run_start[j]][0].record(stream)
            c()
            if row is not None and j in run_end:
                row[run_end[j]][1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    clocks["right_after_timed_steps"] = clock_snapshot()
    wall = t1 - t0
    value = step_bytes * args.steps / wall / 1e9
    log("decode: %.1f GB/s over %d steps (%.3f ms/step)" % (value, args.steps, wall / args.steps * 1e3))

    tsum, count, bsum = 0.0, 0, 0
    for i in range(args.steps):
        if ev[i] is None:
            continue
        for r, (a, b) in enumerate(runs):
            if not dom[a]:
                continue  # --events all: only the dominant kernel's runs make the roofline
            tsum += ev[i][r][0].elapsed_time(ev[i][r][1]) * 1e-3
            for j in range(a, b + 1):
                key = names[j][0]
                count += 1
                bsum += linear_bytes(key[3], key[1], key[2])
    achieved = bsum / tsum / 1e9
    roofline = {
        "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(dominant),
        "kernel": dominant, "launches": count,
        "event_steps": "1 in %d timed steps" % args.event_every,
        "event_pairs_per_step": len(runs),
        "avg_launch_us": round(tsum / count * 1e6, 2),
        "bytes_per_launch": int(bsum / count),
    }
    breakdown = {k: {"us": round(v[0] / v[1] * 1e6, 2),
                     "GB/s": round(v[2] / (v[0] / v[1]) / 1e9, 1),
                     "frac": round(v[2] / (v[0] / v[1]) / 1e9 / HBM_PEAK_GBS, 4)}
                 for k, v in per_proj.items()}
    kernels = {k: {"avg_us": round(v[0] / v[1] * 1e6, 2), "launches": v[1],
                   "GB/s": round(v[2] / v[0] / 1e9, 1)} for k, v in per_sym.items()}

    # Context, not part of the metric: the same 21 projections through torch's
    # plain bf16 linear on the base weights alone (no delta, bf16 output), the
    # platform library's rate for the unfused base model.
    ref_steps = 10
    def ref_step(i):
        for M in Ms:
            for name, N, K in layer:
                torch.nn.functional.linear(xs[K][:M], copies[i % ROTATE][name][0])
    for i in range(3):
        ref_step(i)
    torch.cuda.synchronize()
    r0 = time.perf_counter()
    for i in range(ref_steps):
        ref_step(i)
    torch.cuda.synchronize()
    ref_wall = (time.perf_counter() - r0) / ref_steps
    ref_bytes = sum(2 * N * K + 2 * M * K + 2 * M * N for _, N, K in layer for M in Ms)
    torch_ref = {"ms_per_step": round(ref_wall * 1e3, 4), "GB/s": round(ref_bytes / ref_wall / 1e9, 1),
                 "fused_speedup": round(ref_wall / (wall / args.steps), 3),
                 "what": "torch.nn.functional.linear on the bf16 base weights only (no delta), "
                         "same 21 calls and weight rotation; context, not the metric"}
    log("torch bf16 base-only decode step: %.3f ms" % (ref_wall * 1e3))
    del copies, steps_calls
    torch.cuda.empty_cache()

    extra = {}
    if not args.no_extra:
        wanted = set(REGIMES) if args.regimes == "all" else set(args.regimes.split(","))
        unknown = wanted - set(REGIMES)
        if unknown:
            raise SystemExit("unknown regimes: %s" % ",".join(sorted(unknown)))
        extra = extra_regimes(torch, bd, synth, lib, dev, stream, sh, wanted)
        if "full_share" in wanted:
            try:
                extra["full_share"] = full_share(args, torch, bd, synth, lib, dev, stream, sh)
            except Exception as e:  # recorded, never fatal to the decode line
                extra["full_share"] = {"error": "%s: %s" % (type(e).__name__, str(e)[:300])}
            torch.cuda.empty_cache()
    clocks["after"] = clock_snapshot()

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(args.cpu_seconds)

    out = {
        "metric": "effective GB/s & % HBM peak (decode M<=16); TFLOP/s & % MFMA peak (prefill)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded: bf16 W_base~N(0,0.02^2), Laplace(0,1e-3) deltas, bf16 x~N(0,1))",
        "config": {"workload": "decode, one Llama-70B-shaped layer (q,k,v,o,gate,up,down), "
                               "M in {1,4,16}, per-row alpha, 21 fused-linear calls per step",
                   "bytes_per_step": step_bytes, "rotated_weight_copies": ROTATE},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "decode_kernels": kernels,
        "decode_breakdown": breakdown,
        "decode_torch_bf16_base_only": torch_ref,
        "breakdown_note": "decode_kernels/decode_breakdown: per-launch event timings from a separate "
                          "pass of %d steps with events around every launch" % prof_steps,
        "clocks": clocks,
        "regimes": extra,
    }
    print(json.dumps(out), flush=True)


REGIMES = ("prefill", "grouped", "compress", "cache", "file", "unfused", "monosoup", "stream", "full_share")


def extra_regimes(torch, bd, synth, lib, dev, stream, sh, wanted):
    res = {}
    if "stream" in wanted:
        res["stream_read"] = stream_read_regime(torch, dev, stream)
    if "prefill" in wanted:
        res["prefill"] = prefill_regime(torch, bd, synth, lib, dev, stream, sh)
    if "grouped" in wanted:
        res["grouped"] = grouped_regime(torch, bd, synth, dev, stream)
    if "compress" in wanted:
        res.update(compress_regimes(torch, synth, lib, dev, stream, sh))
    if "cache" in wanted:
        res["delta_cache"] = delta_cache_regime(torch, bd, synth, dev, stream)
    if "file" in wanted:
        res["delta_file"] = delta_file_regime(torch, bd, synth, dev, stream)
    if "unfused" in wanted:
        res["unfused"] = unfused_regime(torch, bd, synth, lib, dev, stream, sh)
    if "monosoup" in wanted:
        res["monosoup"] = monosoup_regime(torch, synth, dev, stream)
    return res


def prefill_regime(torch, bd, synth, lib, dev, stream, sh):
    """Seven projections at M = 2048, per-matrix α, each bd_linear call timed
    with HIP events (median of 5)."""
    M = 2048
    tot_flop = 0
    tot_t = 0.0
    ref_t = 0.0
    per = {}
    seed = synth.SEEDS["prefill"]
    for name, N, K in synth.LLAMA70B_LAYER:
        w, d, x = synth.projection(N, K, M, seed=seed, device=dev)
        s, a = bd.bd_compress(d, bd.BD_ALPHA_PER_MATRIX)
        del d
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
        c = Call(lib, x, w, s, a, y, bd.BD_ALPHA_PER_MATRIX, sh)
        for _ in range(2):
            c()
        dts = timed_launches(torch, [c], 5, stream)
        dt = sorted(r[0] for r in dts)[len(dts) // 2]
        flop = 2 * M * N * K
        per[name] = {"us": round(dt * 1e6, 1), "TFLOP/s": round(flop / dt / 1e12, 1),
                     "frac": round(flop / dt / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
        tot_flop += flop
        tot_t += dt
        # context: torch's plain bf16 GEMM on the base weights alone (no delta)
        ref = lambda: torch.nn.functional.linear(x, w)
        for _ in range(2):
            ref()
        rts = timed_launches(torch, [ref], 5, stream)
        rt = sorted(r[0] for r in rts)[len(rts) // 2]
        ref_t += rt
        per[name]["torch_bf16_base_only_TFLOP/s"] = round(flop / rt / 1e12, 1)
        del w, s, a, x, y
        torch.cuda.empty_cache()
    # roofline of the tiled kernel: the projection with the largest time
    # (gate/up); the call also runs the split tiles' sum kernel, whose share
    # the committed kernel trace gives
    big = max(per, key=lambda k: per[k]["us"])
    Nb, Kb = {n: (N_, K_) for n, N_, K_ in synth.LLAMA70B_LAYER}[big]
    flop_b = 2 * M * Nb * Kb
    ach = flop_b / (per[big]["us"] * 1e-6) / 1e12
    cnt = committed_counters("counters_prefill_grouped.txt", "prefill_kernel")
    roof = {"bound": "mfma", "kernel": "prefill_kernel", "projection": big,
            "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4), "avg_call_us": per[big]["us"],
            "flop_per_launch": flop_b,
            "scope": "one bd_linear call: prefill_kernel plus the sum kernel of its K-split tiles",
            "traffic": cnt.get("traffic_bytes") if cnt else None,
            "counters": cnt or None}
    out = {"TFLOP/s": round(tot_flop / tot_t / 1e12, 1),
           "frac_of_mfma_peak": round(tot_flop / tot_t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
           "layer_ms": round(tot_t * 1e3, 3), "per_projection": per, "roofline": roof,
           "torch_bf16_base_only_layer_ms": round(ref_t * 1e3, 3),
           "workload": "7 projections, x [2048, d_in], per-matrix alpha"}
    log("prefill: %.1f TFLOP/s" % out["TFLOP/s"])
    return out


def grouped_regime(torch, bd, synth, dev, stream):
    """One 8192x28672 base, 14 deltas, 256 tokens on ids drawn uniformly."""
    res = {}
    N, K, Mg, G = 8192, 28672, 256, 14
    gen = synth.generator(synth.SEEDS["grouped"], dev)
    w = synth.base_weight(gen, N, K, dev)
    scales = synth.variant_scales(gen, G, dev)
    sl, al = [], []
    for b in scales:
        d = synth.laplace_delta(gen, N, K, b, dev)
        s, a = bd.bd_compress(d, bd.BD_ALPHA_PER_ROW)
        sl.append(s)
        al.append(a)
        del d
    x = synth.activations(gen, Mg, K, dev)
    ids = synth.variant_ids(gen, Mg, G, dev)
    y = torch.empty((Mg, N), dtype=torch.float32, device=dev)
    fn = lambda: bd.bd_linear_grouped(x, ids, w, sl, al, bd.BD_ALPHA_PER_ROW, out=y)
    for _ in range(2):
        fn()
    dts = timed_launches(torch, [fn], 5, stream)
    dt = sorted(r[0] for r in dts)[len(dts) // 2]
    gbytes = 2 * N * K + G * (N * K // 8 + 4 * N) + 2 * Mg * K + 4 * Mg * N + 4 * Mg
    gflop = 2 * Mg * N * K
    kname = "grouped_stage_kernel"
    cnt = committed_counters("counters_prefill_grouped.txt", kname)
    bounds = {"hbm": round(gbytes / (HBM_PEAK_GBS * 1e9) * 1e6, 1),
              "mfma": round(gflop / (MFMA_BF16_PEAK_TFLOPS * 1e12) * 1e6, 1)}
    if cnt and "SQ_INSTS_VALU" in cnt:
        # VALU bound from the counted VALU wave instructions of one launch:
        # each takes 2 clocks of a SIMD, 1024 SIMDs at 2.4 GHz
        valu = cnt["SQ_INSTS_VALU"]
        bounds["valu_counted"] = round(valu / VALU_PEAK_WAVE_INSTR_PER_S * 1e6, 1)
    binding = max(bounds, key=lambda k: bounds[k])
    if binding == "valu_counted":
        ach = cnt["SQ_INSTS_VALU"] / dt
        roof = {"bound": "alu", "achieved": round(ach / 1e9, 1), "peak": VALU_PEAK_WAVE_INSTR_PER_S / 1e9,
                "unit": "G VALU wave-instr/s", "frac": round(ach / VALU_PEAK_WAVE_INSTR_PER_S, 4)}
    elif binding == "mfma":
        ach = gflop / dt / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4)}
    else:
        ach = gbytes / dt / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4)}
    roof.update({"kernel": kname, "avg_call_us": round(dt * 1e6, 1),
                 "traffic": cnt.get("traffic_bytes") if cnt else None, "counters": cnt or None})
    res = {
        "us": round(dt * 1e6, 1), "GB/s": round(gbytes / dt / 1e9, 1),
        "hbm_frac": round(gbytes / dt / 1e9 / HBM_PEAK_GBS, 4),
        "TFLOP/s": round(gflop / dt / 1e12, 2),
        "bounds_us": bounds, "binding_bound": binding, "roofline": roof,
        "workload": "8192x28672 base, 14 deltas (Laplace b in [5e-4,2e-3]), 256 tokens, per-row alpha",
    }
    log("grouped: %.1f us" % (dt * 1e6))
    del w, sl, al, x, y
    torch.cuda.empty_cache()
    return res


def compress_regimes(torch, synth, lib, dev, stream, sh):
    res = {}
    # compression: gate projection, per-row α
    N, K = 28672, 8192
    gen = synth.generator(synth.SEEDS["decode"], dev)
    d = synth.laplace_delta(gen, N, K, 1e-3, dev)
    s = torch.empty((N, K // 8), dtype=torch.uint8, device=dev)
    a = torch.empty((N,), dtype=torch.float32, device=dev)
    args = (ctypes.c_void_p(d.data_ptr()), N, K, 1, ctypes.c_void_p(s.data_ptr()),
            ctypes.c_void_p(a.data_ptr()), None, 0, sh)
    fn = lambda: lib.bd_compress(*args)
    for _ in range(2):
        fn()
    dts = timed_launches(torch, [fn], 5, stream)
    dt = sorted(r[0] for r in dts)[len(dts) // 2]
    cbytes = 4 * N * K + N * K // 8 + 4 * N
    res["compress"] = {"us": round(dt * 1e6, 1), "GB/s": round(cbytes / dt / 1e9, 1),
                       "frac": round(cbytes / dt / 1e9 / HBM_PEAK_GBS, 4),
                       "workload": "gate 28672x8192 fp32 delta, per-row alpha"}
    log("compress: %.1f GB/s" % res["compress"]["GB/s"])
    del d

    # compression from a (fine-tuned, base) bf16 pair, same shape: Δ formed on the device
    wb = synth.base_weight(gen, N, K, dev)
    wf = (wb.float() + 1e-3 * torch.randn((N, K), generator=gen, device=dev)).to(torch.bfloat16)
    args = (ctypes.c_void_p(wf.data_ptr()), ctypes.c_void_p(wb.data_ptr()), N, K, 1,
            ctypes.c_void_p(s.data_ptr()), ctypes.c_void_p(a.data_ptr()), None, 0, sh)
    fn = lambda: lib.bd_compress_pair(*args)
    for _ in range(2):
        fn()
    dts = timed_launches(torch, [fn], 5, stream)
    dt = sorted(r[0] for r in dts)[len(dts) // 2]
    pbytes = 4 * N * K + N * K // 8 + 4 * N
    res["compress_pair"] = {"us": round(dt * 1e6, 1), "GB/s": round(pbytes / dt / 1e9, 1),
                            "frac": round(pbytes / dt / 1e9 / HBM_PEAK_GBS, 4),
                            "workload": "gate 28672x8192 bf16 (W_ft, W_base) pair, per-row alpha"}
    log("compress_pair: %.1f GB/s" % res["compress_pair"]["GB/s"])
    del wb, wf, s, a
    torch.cuda.empty_cache()
    return res


def monosoup_regime(torch, synth, dev, stream):
    """MonoSoup merge of 4 checkpoints of one 8192x8192 projection at rank 64
    (randomized truncated SVD per task vector on the platform libraries)."""
    from tenant_serving_amd import monosoup
    N = K = 8192
    k, r = 4, 64
    gen = synth.generator(synth.SEEDS["full"] + 100, dev)
    base = synth.base_weight(gen, N, K, dev)
    ck = [(base.float() + synth.laplace_delta(gen, N, K, 1e-3, dev)).to(torch.bfloat16) for _ in range(k)]
    monosoup.merge(base, checkpoints=ck, rank=r)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(3):
        out = monosoup.merge(base, checkpoints=ck, rank=r)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / 3
    del base, ck, out
    torch.cuda.empty_cache()
    log("monosoup: %.2f ms for %d checkpoints of 8192x8192 at rank %d" % (ms, k, r))
    return {"ms": round(ms, 3), "checkpoints": k, "rank": r, "shape": [N, K],
            "what": "W_base + (1/k) sum of rank-r truncated SVDs of the task vectors; randomized range "
                    "finder (r + 8 columns, 2 power iterations), fp32, hipBLASLt / rocSOLVER via torch"}


def delta_file_regime(torch, bd, synth, dev, stream, layers=2):
    """A variant's delta set through the whole cold path: written as a
    delta-set file (safetensors) to the host's temporary directory, dropped
    from the page cache (fsync + POSIX_FADV_DONTNEED), read back into a pinned
    slot buffer in the cache's layout, then copied into an HBM slot by the
    cache.  `layers` layers of the 70B shapes, so the file stays small."""
    import tempfile
    from tenant_serving_amd import deltafile
    from tenant_serving_amd.cache import bd_cache
    mats = [("%d.%s" % (li, n), N, K) for li in range(layers) for n, N, K in synth.LLAMA70B_LAYER]
    layout, slot_bytes = deltafile.slot_layout(mats)
    gen = synth.generator(synth.SEEDS["full"] + 200, dev)
    entries = {}
    for name, N, K in mats:
        d = synth.laplace_delta(gen, N, K, 1e-3, dev)
        entries[name] = bd.bd_compress(d, bd.BD_ALPHA_PER_ROW)
        del d
    fd, path = tempfile.mkstemp(suffix=".safetensors")
    os.close(fd)
    try:
        deltafile.save_delta_set(path, entries, variant="bench")
        fbytes = os.path.getsize(path)
        with open(path, "rb") as f:
            os.fsync(f.fileno())
            dropped = hasattr(os, "posix_fadvise")
            if dropped:
                os.posix_fadvise(f.fileno(), 0, 0, os.POSIX_FADV_DONTNEED)
        host = torch.empty(slot_bytes, dtype=torch.uint8, pin_memory=True)
        t0 = time.perf_counter()
        deltafile.read_into(path, host, layout, {n: (d, k) for n, d, k in mats})
        t_read = time.perf_counter() - t0
    finally:
        os.unlink(path)
    slots = torch.empty(slot_bytes, dtype=torch.uint8, device=dev)
    c = bd_cache(1, 1, 0, 60.0, slot_bytes, slots, torch.cuda.Stream())
    c.bd_cache_set_source(0, host)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    c.bd_cache_acquire(0, 0.0, stream)
    e1.record(stream)
    c.bd_cache_release(0, stream)
    torch.cuda.synchronize()
    t_copy = e0.elapsed_time(e1) * 1e-3
    # the loaded slot holds exactly what compress produced
    views = deltafile.slot_views(slots, layout, {n: (N, K) for n, N, K in mats})
    same = all(torch.equal(views[n][0], entries[n][0]) and torch.equal(views[n][1], entries[n][1])
               for n, _, _ in mats)
    c.close()
    del host, slots, entries, views
    torch.cuda.empty_cache()
    full = 80 * sum(N * K // 8 + 4 * N for _, N, K in synth.LLAMA70B_LAYER)
    rd = fbytes / t_read / 1e9
    cp = slot_bytes / t_copy / 1e9
    out = {"layers": layers, "file_MB": round(fbytes / 1e6, 1), "page_cache_dropped": dropped,
           "file_to_pinned_GB/s": round(rd, 2), "pinned_to_hbm_GB/s": round(cp, 1),
           "slot_matches_compress": same,
           "projected_cold_start_ms_70B_variant": round((full / (rd * 1e9) + full / (cp * 1e9)) * 1e3, 1),
           "what": "safetensors delta-set file -> pinned slot buffer (host read, after dropping the file "
                   "from the page cache) -> HBM slot through the cache; projection for one 8.58 GB 70B "
                   "variant at these rates, unpipelined"}
    log("delta file: read %.2f GB/s, copy %.1f GB/s, slot matches: %s" % (rd, cp, same))
    return out


def unfused_regime(torch, bd, synth, lib, dev, stream, sh):
    """The post's serving flow without fusion, for comparison only: rebuild
    each variant's W_ft = W_base + α·sign(Δ) into HBM once (bf16, with torch
    ops written from the definition), then run torch's plain bf16 linear on it.
    One Llama-70B-shaped layer, per-row α: the rebuild's cost, the decode step
    (21 calls at M = 1, 4, 16) and a 2048-token prefill on the rebuilt
    weights, against the fused library on the same tensors."""
    layer = synth.LLAMA70B_LAYER
    Ms = (1, 4, 16)
    seed = synth.SEEDS["decode"]
    proj = {}
    for name, N, K in layer:
        w, d, _ = synth.projection(N, K, 1, seed=seed * 1000 + 500 + len(proj), device=dev)
        sg, a = bd.bd_compress(d, bd.BD_ALPHA_PER_ROW)
        del d
        proj[name] = (w, sg, a)
    shifts = torch.arange(8, dtype=torch.uint8, device=dev)

    def rebuild(w, sg, a):
        bits = (sg.unsqueeze(-1) >> shifts) & 1                       # [N, K/8, 8], LSB first
        pm = bits.view(w.shape).to(torch.float32).mul_(2.0).sub_(1.0)  # +1 / -1
        return (w.to(torch.float32) + a.unsqueeze(1) * pm).to(torch.bfloat16)

    for _ in range(2):
        weff = {n: rebuild(*proj[n]) for n, _, _ in layer}
        del weff
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    weff = {n: rebuild(*proj[n]) for n, _, _ in layer}
    e1.record(stream)
    torch.cuda.synchronize()
    rebuild_s = e0.elapsed_time(e1) * 1e-3
    nweights = sum(N * K for _, N, K in layer)
    xs = {K: synth.activations(synth.generator(seed, dev), 2048, K, dev) for K in (8192, 28672)}
    # sanity: the fused library and an fp32 product on the rebuilt weights
    # agree up to the summation order (torch's bf16 linear rounds y to bf16)
    worst = 0.0
    for name, N, K in layer:
        x = xs[K][:16]
        yf = bd.bd_linear(x, *proj[name], bd.BD_ALPHA_PER_ROW)
        yu = x.float() @ weff[name].float().t()
        worst = max(worst, ((yf - yu).norm() / yf.norm()).item())

    def decode_unfused():
        for M in Ms:
            for name, N, K in layer:
                torch.nn.functional.linear(xs[K][:M], weff[name])

    calls = [Call(lib, xs[K][:M].contiguous(), *proj[name],
                  torch.empty((M, N), dtype=torch.float32, device=dev), bd.BD_ALPHA_PER_ROW, sh)
             for M in Ms for name, N, K in layer]

    def decode_fused():
        for c in calls:
            c()

    def timed(fn, reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / reps

    dec_u = timed(decode_unfused, 10)
    dec_f = timed(decode_fused, 10)
    yp = {n: torch.empty((2048, N), dtype=torch.float32, device=dev) for n, N, _ in layer}
    pcalls = [Call(lib, xs[K], *proj[name], yp[name], bd.BD_ALPHA_PER_ROW, sh) for name, N, K in layer]
    pre_u = timed(lambda: [torch.nn.functional.linear(xs[K], weff[n]) for n, _, K in layer], 3)
    pre_f = timed(lambda: [c() for c in pcalls], 3)
    del weff, proj, calls, pcalls, yp, xs
    torch.cuda.empty_cache()
    out = {
        "rebuild_ms_per_layer": round(rebuild_s * 1e3, 3),
        "rebuild_ms_per_layer_at_hbm_peak": round(4.125 * nweights / (HBM_PEAK_GBS * 1e9) * 1e3, 3),
        "rebuild_ms_per_variant_80_layers": round(rebuild_s * 80 * 1e3, 1),
        "decode_step_ms": {"unfused_after_rebuild": round(dec_u * 1e3, 4), "fused": round(dec_f * 1e3, 4)},
        "prefill_2048_layer_ms": {"unfused_after_rebuild": round(pre_u * 1e3, 3),
                                  "unfused_with_rebuild": round((pre_u + rebuild_s) * 1e3, 3),
                                  "fused": round(pre_f * 1e3, 3)},
        "hbm_bytes_per_weight": {"fused_per_use": 2.125,
                                 "unfused_rebuild_once": 4.125, "unfused_per_use": 2.0},
        "resident_per_variant_GB_80_layers": {"unfused_W_ft": round(2 * nweights * 80 / 1e9, 1),
                                              "fused_signs_and_alpha": round(
                                                  80 * sum(N * K // 8 + 4 * N for _, N, K in layer) / 1e9, 2)},
        "fused_vs_fp32_on_rebuilt_rel_fro": float("%.3g" % worst),
        "what": "comparison only (torch ops, not the library): W_ft rebuilt into HBM per variant, then "
                "torch.nn.functional.linear; per-row alpha",
    }
    log("unfused: rebuild %.2f ms/layer; decode step %.3f ms (fused %.3f); prefill layer %.2f+%.2f ms "
        "(fused %.2f)" % (rebuild_s * 1e3, dec_u * 1e3, dec_f * 1e3, pre_u * 1e3, rebuild_s * 1e3,
                          pre_f * 1e3))
    return out


def delta_cache_regime(torch, bd, synth, dev, stream):
    """Cold start of one 70B variant through the delta cache: its whole delta
    set (80 layers of packed signs and per-row α, 8.58 GB) copied from pinned
    host memory into an HBM slot (the stand-in for the post's NVMe read), a
    second request joining that load, and a hit's host cost."""
    from tenant_serving_amd.cache import bd_cache
    layer = synth.LLAMA70B_LAYER
    per_layer = sum(N * K // 8 + 4 * N for _, N, K in layer)
    slot_bytes = 80 * per_layer
    try:
        host = torch.empty(slot_bytes, dtype=torch.uint8, pin_memory=True)
        slots = torch.empty(slot_bytes, dtype=torch.uint8, device=dev)
    except RuntimeError as e:
        return {"error": "allocation failed: %s" % str(e)[:200]}
    copy = torch.cuda.Stream()
    other = torch.cuda.Stream()
    c = bd_cache(2, 1, 0, 60.0, slot_bytes, slots, copy)
    c.bd_cache_set_source(0, host)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    t0 = time.perf_counter()
    _, a1, _, _ = c.bd_cache_acquire(0, 0.0, stream)
    t_call = time.perf_counter() - t0
    _, a2, _, _ = c.bd_cache_acquire(0, 0.0, other)   # arrives while loading
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t0
    load_s = e0.elapsed_time(e1) * 1e-3
    c.bd_cache_release(0, stream)
    c.bd_cache_release(0, other)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    hits = 1000
    for i in range(hits):
        _, a3, _, _ = c.bd_cache_acquire(0, 1.0 + i * 1e-3, stream)
        c.bd_cache_release(0, stream)
    t_hit = (time.perf_counter() - t0) / hits
    torch.cuda.synchronize()
    st = c.bd_cache_get_stats()
    c.close()
    del host, slots
    torch.cuda.empty_cache()
    out = {"variant_GB": round(slot_bytes / 1e9, 3), "cold_load_ms": round(load_s * 1e3, 2),
           "cold_load_GB/s": round(slot_bytes / load_s / 1e9, 1),
           "cold_load_wall_ms": round(t_wall * 1e3, 2), "acquire_call_us": round(t_call * 1e6, 1),
           "actions": [a1, a2, a3], "loads": st["loads"], "joins": st["joins"],
           "hit_acquire_release_us": round(t_hit * 1e6, 2),
           "post_cold_start": "about 200 ms for 8.75 GB (43.8 GB/s) from NVMe",
           "workload": "one 70B variant's delta set (80 layers of signs + per-row alpha), "
                       "pinned host -> HBM on a copy stream"}
    log("delta cache: cold load %.1f ms (%.1f GB/s), hit %.2f us"
        % (out["cold_load_ms"], out["cold_load_GB/s"], out["hit_acquire_release_us"]))
    return out


def full_share(args, torch, bd, synth, lib, dev, stream, sh):
    """The full single-GPU share: 80 Llama-70B-shaped layers (7 projections
    each, 136.9 GB of bf16 base) and 14 variants' packed signs and per-row α
    (14 x 8.58 GB), all resident in HBM.  16 requests, each on a variant drawn
    uniformly from the 14, send 32 prompt tokens (one grouped prefill pass of
    512 tokens through all 560 projections) and then decode 64 steps of one
    token each (560 grouped launches of 16 tokens per step).  Each projection
    takes a fixed synthetic input of its d_in (no attention, norm or activation
    between them).  The deltas are Laplace(0, b) with b drawn per variant,
    compressed on the GPU matrix by matrix."""
    L, G, R, P, D = args.layers, 14, 16, 32, args.decode_steps
    layer = synth.LLAMA70B_LAYER
    per_layer = sum(N * K for _, N, K in layer)
    gen = synth.generator(synth.SEEDS["full"], dev)
    scales = synth.variant_scales(gen, G, dev)
    req = synth.request_mix(gen, R, G, dev).cpu().tolist()
    present = sorted(set(req))
    local = {v: i for i, v in enumerate(present)}
    dec_ids = torch.tensor([local[v] for v in req], dtype=torch.int32, device=dev)
    pre_ids = dec_ids.repeat_interleave(P).contiguous()
    xs = {K: synth.activations(gen, R * P, K, dev) for K in (8192, 28672)}
    need = L * per_layer * 2 + G * L * (per_layer // 8 + 4 * sum(N for _, N, _ in layer))
    free, total = torch.cuda.mem_get_info(dev)
    log("full share: %d layers, %d variants, %.1f GB of weights and deltas; %.1f GB free of %.1f GB"
        % (L, G, need / 1e9, free / 1e9, total / 1e9))
    t0 = time.perf_counter()
    big = max(N * K for _, N, K in layer)
    tmp_a = torch.empty(big, dtype=torch.float32, device=dev)
    tmp_b = torch.empty(big, dtype=torch.float32, device=dev)
    # one allocation per layer of base weights and per variant of signs / α,
    # projections as views in layer order
    offs, o = {}, 0
    for name, N, K in layer:
        offs[name] = o
        o += N * K
    aoffs, o = {}, 0
    for name, N, K in layer:
        aoffs[name] = o
        o += N
    rows = o
    base = []
    for li in range(L):
        blob = torch.empty(per_layer, dtype=torch.bfloat16, device=dev)
        views = {}
        for name, N, K in layer:
            v = blob[offs[name]:offs[name] + N * K].view(N, K)
            synth.base_weight_into(gen, v, tmp_a)
            views[name] = v
        base.append((blob, views))
    sgn_blob = [torch.empty(L * per_layer // 8, dtype=torch.uint8, device=dev) for _ in range(G)]
    alp_blob = [torch.empty(L * rows, dtype=torch.float32, device=dev) for _ in range(G)]
    for g in range(G):
        for li in range(L):
            for name, N, K in layer:
                d = tmp_b[:N * K].view(N, K)
                synth.laplace_delta_into(gen, d, tmp_a, scales[g])
                so = (li * per_layer + offs[name]) // 8
                ao = li * rows + aoffs[name]
                st = lib.bd_compress(ctypes.c_void_p(d.data_ptr()), N, K, bd.BD_ALPHA_PER_ROW,
                                     ctypes.c_void_p(sgn_blob[g].data_ptr() + so),
                                     ctypes.c_void_p(alp_blob[g].data_ptr() + 4 * ao), None, 0, sh)
                if st != 0:
                    raise RuntimeError("bd_compress failed with status %d" % st)
        torch.cuda.synchronize()
        log("full share: variant %d of %d compressed (%.1f s)" % (g + 1, G, time.perf_counter() - t0))
    del tmp_a, tmp_b
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    t_setup = time.perf_counter() - t0
    log("full share: set up in %.1f s" % t_setup)

    def sv(g, li, name, N, K):
        so = (li * per_layer + offs[name]) // 8
        return sgn_blob[g][so:so + N * K // 8].view(N, K // 8)

    def av(g, li, name, N):
        ao = li * rows + aoffs[name]
        return alp_blob[g][ao:ao + N]

    ys = {(M, N): torch.empty((M, N), dtype=torch.float32, device=dev)
          for M in (R, R * P) for N in {n for _, n, _ in layer}}
    Gp = len(present)
    ws_bytes = max(lib.bd_linear_grouped_workspace_bytes(M, N, K, Gp)
                   for M in (R, R * P) for _, N, K in layer)
    ws = torch.empty(max(ws_bytes, 16) // 4 + 4, dtype=torch.float32, device=dev)

    # The token-by-variant bucketing is the same for all 560 launches of a
    # pass: it is planned once per pass (bd_linear_grouped_plan) and every
    # launch uses the plan.
    def calls(M, ids):
        out = []
        for li in range(L):
            for name, N, K in layer:
                out.append(GroupedCall(lib, xs[K][:M], ids, base[li][1][name],
                                       [sv(g, li, name, N, K) for g in present],
                                       [av(g, li, name, N) for g in present],
                                       bd.BD_ALPHA_PER_ROW, ys[(M, N)], ws, ws_bytes, sh, planned=True))
        return out

    def plan(M, ids):
        st = lib.bd_linear_grouped_plan(ctypes.c_void_p(ids.data_ptr()), M, Gp, ctypes.c_void_p(ws.data_ptr()),
                                        ws_bytes, sh)
        if st != 0:
            raise RuntimeError("bd_linear_grouped_plan failed with status %d" % st)

    pre_calls = calls(R * P, pre_ids)
    dec_calls = calls(R, dec_ids)
    # warm-up: one prefill pass and one decode step
    plan(R * P, pre_ids)
    for c in pre_calls:
        c()
    plan(R, dec_ids)
    for c in dec_calls:
        c()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(D + 2)]
    t_wall = time.perf_counter()
    ev[0].record(stream)
    plan(R * P, pre_ids)
    for c in pre_calls:
        c()
    ev[1].record(stream)
    for step in range(D):
        plan(R, dec_ids)
        for c in dec_calls:
            c()
        ev[step + 2].record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    pre_t = ev[0].elapsed_time(ev[1]) * 1e-3
    steps = [ev[i + 1].elapsed_time(ev[i + 2]) * 1e-3 for i in range(D)]
    dec_t = sum(steps)
    step_t = dec_t / D
    params = L * per_layer
    delta_bytes = L * (per_layer // 8 + 4 * rows)       # one variant's signs + α
    io = lambda M: L * sum(2 * M * K + 4 * M * N for _, N, K in layer)
    step_bytes = 2 * params + Gp * delta_bytes + io(R)
    pre_bytes = 2 * params + Gp * delta_bytes + io(R * P)
    pre_flop = 2 * R * P * params
    gbs = step_bytes / step_t / 1e9
    res = {
        "metric": "decode effective GB/s, full single-GPU share (80 layers, 14 variants resident, "
                  "M=16 mixed variants)",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": D, "warmup": 1,
        "ms_per_step": round(step_t * 1e3, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "full single-GPU share: %d layers x 7 Llama-70B projections "
                               "(bf16 base %.1f GB) + %d variants' signs and per-row alpha "
                               "(%.2f GB each), %d requests x %d prompt tokens, then %d decode "
                               "steps of one token per request" % (L, 2 * params / 1e9, G,
                                                                    delta_bytes / 1e9, R, P, D),
                   "variants_in_batch": Gp, "resident_GB": round(need / 1e9, 2)},
        "decode": {"step_ms": round(step_t * 1e3, 3),
                   "step_ms_min_max": [round(min(steps) * 1e3, 3), round(max(steps) * 1e3, 3)],
                   "tokens_per_s": round(R / step_t, 1),
                   "bytes_per_step": step_bytes, "hbm_bound_ms": round(step_bytes / 8e12 * 1e3, 3),
                   "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)},
        "prefill": {"ms": round(pre_t * 1e3, 3), "tokens": R * P,
                    "TFLOP/s": round(pre_flop / pre_t / 1e12, 1),
                    "frac_of_mfma_peak": round(pre_flop / pre_t / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                    "GB/s": round(pre_bytes / pre_t / 1e9, 1)},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "scope": "whole decode step (560 grouped launches)"},
        "cpu_baseline": None,
        "wall_s": round(t_wall, 3),
        "setup_s": round(t_setup, 1),
    }
    del pre_calls, dec_calls, base, sgn_blob, alp_blob, ys, ws, xs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    log("full share: decode step %.2f ms (%.1f GB/s), prefill %.1f ms" % (step_t * 1e3, gbs, pre_t * 1e3))
    return res


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(seconds):
    """The oracle as it stands (plain C, fp64, OpenMP over output rows), on the
    host cores, on bounded samples of the workloads, with all of the host's
    threads and with one.  The headline sample is the decode workload's q
    projection (8192x8192) at M = 1, in the metric's unit; the others are
    reported beside it.  Each sample repeats until its share of `seconds`
    has passed (at least once)."""
    import torch
    import oracle
    from tenant_serving_amd import synth

    lib_all = oracle.load()
    threads_all = oracle.num_threads(lib_all)

    def timed(fn, budget):
        reps, t0 = 0, time.perf_counter()
        while True:
            fn()
            reps += 1
            if time.perf_counter() - t0 >= budget:
                break
        return (time.perf_counter() - t0) / reps, reps

    share = seconds / 8.0
    samples = {}
    # decode q at M = 1 (the headline sample)
    N, K, M = 8192, 8192, 1
    w, d, x = synth.projection(N, K, M, seed=synth.SEEDS["decode"], device="cpu")
    s, a = oracle.compress(d, True)
    t, reps = timed(lambda: oracle.linear(x, w, s, a, True), 2 * share)
    headline = linear_bytes(M, N, K) / t / 1e9
    samples["decode_q_M1"] = {"GB/s": round(headline, 3), "s_per_run": round(t, 4), "runs": reps}
    # tiny: 256x512, 4 tokens, per-matrix alpha
    wt, dt_, xt = synth.tiny()
    st, at = oracle.compress(dt_, False)
    t, reps = timed(lambda: oracle.linear(xt, wt, st, at, False), 0.5 * share)
    samples["tiny"] = {"GB/s": round(linear_bytes(4, 256, 512, False) / t / 1e9, 3), "s_per_run": round(t, 6),
                       "runs": reps}
    # compress: q shape 8192x8192 fp32 delta, per-row alpha
    t, reps = timed(lambda: oracle.compress(d, True), share)
    samples["compress_q"] = {"GB/s": round((4 * N * K + N * K // 8 + 4 * N) / t / 1e9, 3),
                             "s_per_run": round(t, 4), "runs": reps}
    # prefill: 64 of the 2048 token rows of the q projection, extrapolated x32
    xp = synth.activations(synth.generator(synth.SEEDS["prefill"]), 64, K)
    t, reps = timed(lambda: oracle.linear(xp, w, s, a, True), share)
    samples["prefill_q_64_rows_extrapolated_x32"] = {
        "TFLOP/s": round(2 * 64 * N * K / t / 1e12, 5), "s_per_run_64_rows": round(t, 3),
        "s_extrapolated_2048_rows": round(32 * t, 2), "runs": reps}
    # grouped: 16 of the 256 tokens of the 14-variant workload on a 1024-row slice of its base
    Ng, Kg, G = 1024, 28672, 14
    wg, deltas, _, xg, ids = synth.grouped(Ng, Kg, 16, G)
    comp = [oracle.compress(dd, True) for dd in deltas]
    del deltas
    t, reps = timed(lambda: oracle.linear_grouped(xg, ids, wg, [c[0] for c in comp], [c[1] for c in comp], True),
                    share)
    gb = 2 * Ng * Kg + G * (Ng * Kg // 8 + 4 * Ng) + 2 * 16 * Kg + 4 * 16 * Ng
    samples["grouped_1024_rows_16_tokens"] = {"GB/s": round(gb / t / 1e9, 3), "s_per_run": round(t, 4),
                                              "runs": reps}
    # one thread: the headline sample again (the oracle's OpenMP runtime is the
    # process's libgomp, whose thread count is set for the calls below)
    one = None
    try:
        omp = ctypes.CDLL("libgomp.so.1")
        omp.omp_set_num_threads(1)
        try:
            t, reps = timed(lambda: oracle.linear(x, w, s, a, True), 2 * share)
            one = {"GB/s": round(linear_bytes(M, N, K) / t / 1e9, 3), "threads": oracle.num_threads(),
                   "s_per_run": round(t, 4), "runs": reps, "sample": "decode q 8192x8192, M=1"}
        finally:
            omp.omp_set_num_threads(threads_all)
    except OSError:
        one = None
    return {"value": round(headline, 3), "unit": "GB/s", "cores": threads_all, "kind": "oracle",
            "sample": "decode q projection 8192x8192, M=1, per-row alpha, %d runs" % samples["decode_q_M1"]["runs"],
            "cpu_model": _cpu_model(), "host_cpus": os.cpu_count(), "one_thread": one, "samples": samples}


if __name__ == "__main__":
    main()

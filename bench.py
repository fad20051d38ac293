#!/usr/bin/env python3
"""Throughput of the chunked gated delta rule forward on one MI355X.

A step is one full forward over the 64k-token, 32-head, K = V = 128 sequence
split into 4 contiguous segments: the carrying zero-state scan (phase 1), the
exclusive segment scan (phase 2) and the emitting scan (phase 3), i.e. every
entry point of the chunked path, on bf16 inputs with fp32 state, scheduled by
forward_segmented (segment 0 emitted from the initial state beside the
carrying pass of the middle segments; no carrying pass for segment 0's M or for
the last segment).  Inputs are seeded synthetic tensors already resident in HBM
when timing starts.

Prints one JSON line: tokens/s of that step, the roofline of its dominant
kernel (HIP events around that kernel's launches on its stream), the fp64 CPU
oracle timed on a bounded sample of the same workload on the host cores, and
secondary measurements (monolithic scan, 4k sequence, packed batch, decode).
"""
import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN fwd tokens/s at H=32,K=V=128,S=64k (1 GPU); % MFMA/HBM roofline"
PEAK_BF16_TFLOPS = 2500.0       # dense MFMA, MI355X
PEAK_F32_VALU_TFLOPS = 157.3    # fp32 vector, and fp32 dense MFMA
PEAK_HBM_GBS = 8000.0


def flops_per_token_head(C, K, V):
    """Canonical chunked work (dense tiles): the two C x C Gram matrices, T applied
    to [beta gamma K | beta V], the three K x V state products and attn @ delta."""
    return 2 * (2 * C * K + C * (K + V) + 3 * K * V + C * V)


def carry_flops_per_token_head(C, K, V):
    """Zero-state pass carrying X = [M | h]: Gram k k^T, T applied to
    [beta gamma K | beta V], and w X, k_tilde^T delta_X over K + V columns."""
    return 2 * C * K + 2 * C * (K + V) + 4 * K * (K + V)


def bwd_flops_per_token_head(C, K, V):
    """Dense work of the backward kernels (masked triangles counted dense, as in
    the forward): the Grams, T applied to [Kb | Vb], both state scans (delta and
    the state update; ddelta and the state-gradient update), and per chunk
    dattn, dw, dT, T^T dT T^T, dv, dq and the four parts of dk.  Per chunk-head
    18 C^2 K + 10 C^2 V + 16 C K V + 4 C^3 multiply-adds x 2, over C tokens."""
    return 2 * (9 * C * K + 5 * C * V + 8 * K * V + 2 * C * C)


def bytes_per_token_head(K, V, s_in, s_out):
    """q, k, v in, o out, g and beta fp32."""
    return (2 * K + V) * s_in + V * s_out + 8


def step_roofline(tokens, heads, ms, C=64, K=128, V=128, elem=2):
    """Whole-step rates of a forward over `tokens` real tokens and `heads` heads:
    canonical FLOPs against the bf16 MFMA peak and algorithmic bytes (states
    excluded) against HBM, each over the whole step's time."""
    t = ms * 1e-3
    fl = tokens * heads * flops_per_token_head(C, K, V)
    by = tokens * heads * bytes_per_token_head(K, V, elem, elem)
    return {"useful_tflops": fl / t / 1e12, "mfma_frac": fl / t / 1e12 / PEAK_BF16_TFLOPS,
            "hbm_frac": by / t / 1e9 / PEAK_HBM_GBS}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--segments", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the secondary measurements")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target duration of the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for the HBM byte counters)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_scan_mfma_seq64k_4seg.md")
# the sources of the scan kernels whose counters the traffic summary holds
KERNEL_SOURCES = [os.path.join(ROOT, "chunked_gated_delta_gdn_amd", "csrc", f)
                  for f in ("scan_mfma.hip", "mfma_tile.h", "dev_common.h")]
COPY_BYTES = 1 << 30


def kernel_source_digest():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None
    when there is none or the kernel sources changed since it was taken."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    src = re.search(r"kernel_source_digest:\s*([0-9a-f]+)", text)
    row = re.search(rf"traffic_bytes_per_launch\[{re.escape(kernel)}\]:\s*([0-9.e+]+)", text)
    if not src or not row or src.group(1) != kernel_source_digest():
        return None
    return float(row.group(1))


def measured_peaks(torch, dev):
    """Peaks measured on this GPU, quoted beside the datasheet ones: a dense bf16
    matrix-core loop (libgdn_probe.so: register operands, no memory traffic) and
    a 1 GiB device copy (read once, written once), each timed with HIP events
    over 5 launches after a warm-up."""
    import ctypes
    from chunked_gated_delta_gdn_amd import _build
    lib = ctypes.CDLL(_build.PROBE_LIB)
    for fn in (lib.gdn_probe_mfma_bf16, lib.gdn_probe_mfma_f32):
        fn.restype = ctypes.c_int32
        fn.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    n_blocks = 4 * torch.cuda.get_device_properties(dev).multi_processor_count
    iters = 4096
    out = torch.empty(n_blocks * 256, dtype=torch.float32, device=dev)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    def timed(fn, n=5):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e-3

    def probe(fn):
        if fn(ctypes.c_void_p(out.data_ptr()), n_blocks, iters, stream) != 0:
            raise RuntimeError("matrix-core probe failed")
    t_m = timed(lambda: probe(lib.gdn_probe_mfma_bf16))
    t_f = timed(lambda: probe(lib.gdn_probe_mfma_f32))
    flops = n_blocks * 4 * 4 * iters * 16 * 16 * 32 * 2
    flops_f = n_blocks * 4 * 4 * iters * 16 * 16 * 4 * 2
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    t_c = timed(lambda: torch.neg(src, out=dst))
    del src, dst, out
    return {"bf16_mfma_tflops": flops / t_m / 1e12, "f32_mfma_tflops": flops_f / t_f / 1e12,
            "hbm_copy_gbs": 2 * COPY_BYTES / t_c / 1e9,
            "how": f"MFMA loops ({n_blocks} workgroups x 4 waves x 4 chains x {iters} "
                   "v_mfma_f32_16x16x32_bf16, or v_mfma_f32_16x16x4_f32); 1 GiB device copy (read + write)"}


def copy_calibration(torch):
    """A plain device copy of COPY_BYTES, read once and written once per launch
    (elementwise negation, so it is an ordinary shader kernel that the counters see)."""
    dev = torch.device("cuda:0")
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": COPY_BYTES,
                      "copy_calibration_bytes_written": COPY_BYTES, "launches": 3,
                      "kernel_source_digest": kernel_source_digest()}), flush=True)


class StreamTimer:
    """HIP events recorded on the launching stream around named kernels."""

    def __init__(self, torch, only=None):
        self.torch = torch
        self.marks = {}
        self.only = only   # names to time (None: all)

    def around(self, name, fn, stream=None):
        if self.only is not None and name not in self.only:
            return fn()
        t = self.torch
        st = stream if stream is not None else t.cuda.current_stream()
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record(st)
        out = fn()
        b.record(st)
        self.marks.setdefault(name, []).append((a, b))
        return out

    def avg_ms(self):
        return {k: sum(a.elapsed_time(b) for a, b in v) / len(v) for k, v in self.marks.items()}


def time_steps(torch, step, steps, warmup, only=None, per_step=None):
    """Mean ms per step over `steps` steps after `warmup`, and the mean HIP-event
    time of each named kernel (only those in `only`, if given: every event pair
    recorded inside the timed steps costs the step a little).  With a list
    `per_step`, an event between consecutive steps gives each step's own time
    (appended to it)."""
    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    timer = StreamTimer(torch, only)
    st = torch.cuda.current_stream()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    marks[0].record(st)
    for i in range(steps):
        step(timer)
        marks[i + 1].record(st)
    torch.cuda.synchronize()
    if per_step is not None:
        per_step.extend(marks[i].elapsed_time(marks[i + 1]) for i in range(steps))
    return marks[0].elapsed_time(marks[steps]) / steps, timer.avg_ms()


def time_cold_steps(torch, step, steps, flush_bytes=1 << 30):
    """Per-step ms with the GPU's caches (L2 and the 256 MB MALL) flushed before
    each step by writing a buffer larger than them; only the step is timed."""
    dev = torch.cuda.current_device()
    junk = torch.empty(flush_bytes // 4, dtype=torch.float32, device=dev)
    out = []
    step(None)
    for _ in range(steps):
        junk.fill_(1.0)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step(None)
        b.record()
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b))
    del junk
    return out


def cpu_model():
    """The host CPU as /proc/cpuinfo names it, with its family, model and
    stepping numbers (a virtualised host may report only a generic name)."""
    fields = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" not in line:
                if fields:
                    break
                continue
            key, val = (x.strip() for x in line.split(":", 1))
            if key in ("model name", "cpu family", "model", "stepping") and key not in fields:
                fields[key] = val
    except OSError:
        return None
    if "model name" not in fields:
        return None
    ids = ", ".join(f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields)
    return f"{fields['model name']} ({ids})" if ids else fields["model name"]


def time_with_breakdown(torch, step, steps, warmup, stats=None):
    """Mean ms per step with no events inside the timed steps (events around
    each launch cost a short multi-launch step a large share), then the mean
    HIP-event time of each named kernel from a separate pass of up to 10 steps.
    With a dict `stats`, the median and the minimum of the steps' own times (an
    event between consecutive steps) are put in it."""
    per = []
    ms, _ = time_steps(torch, step, steps, warmup, only=set(), per_step=per)
    if stats is not None:
        stats["ms_median"] = float(statistics.median(per))
        stats["ms_min"] = float(min(per))
    _, kern = time_steps(torch, step, min(steps, 10), 1)
    return ms, kern


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 "
                                   "(sequence or head sharding across GPUs is not built)",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        copy_calibration(torch)
        return
    import chunked_gated_delta_gdn_amd as gdn
    from chunked_gated_delta_gdn_amd import binding
    from workloads import workload, make_decode_inputs

    binding.library()          # fail loudly before anything else if the library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bf = torch.bfloat16
    log = lambda m: print(m, file=sys.stderr, flush=True)

    # ---------------------------------------------------------------- headline workload
    log("bench: generating the 64k-token workload")
    x = workload(2)
    B, S, H, K, V, C = x.B, x.S, x.H, x.K, x.V, x.C
    R = args.segments
    q = torch.from_numpy(x.q).to(bf).to(dev)
    k = torch.from_numpy(x.k).to(bf).to(dev)
    v = torch.from_numpy(x.v).to(bf).to(dev)
    g = torch.from_numpy(x.g).to(dev)
    beta = torch.from_numpy(x.beta).to(dev)
    h0 = torch.from_numpy(x.h0).to(dev)
    backend = binding.gdn_scan_backend(gdn.problem_for(k, v, C, n_segments=R))

    def seg_step(timer):
        tm = timer.around if timer else (lambda _n, f, _s=None: f())
        if R == 1:
            return tm("scan_emit", lambda: gdn.scan_emit(q, k, v, g, beta, h_in=h0, chunk_size=C))
        return gdn.forward_segmented(q, k, v, g, beta, h0=h0, chunk_size=C, n_segments=R, timer=tm)

    log(f"bench: timing {args.steps} steps after {args.warmup} warm-up steps (R={R})")
    # the timed steps carry HIP events around the dominant kernel only (the roofline
    # kernel); a short second pass times every launch of the step for the breakdown
    dom_name = "scan_emit"
    step_ms = []
    ms, kern_dom = time_steps(torch, seg_step, args.steps, args.warmup, only={dom_name}, per_step=step_ms)
    _, kern = time_steps(torch, seg_step, min(args.steps, 10), 1)
    kern[dom_name] = kern_dom[dom_name]
    tokens = B * S
    value = tokens / (ms * 1e-3)

    # dominant kernel and its roofline.  Tokens per launch: segments 0 .. R-2 (segment
    # 0 emitted beside the carrying pass of 1 .. R-2, one launch), segments 1 .. R-1
    # (emitting).  The launch with the most algorithmic work is the emitting pass over
    # segments 1 .. R-1 (its time is within a few percent of the launch before it).
    dom = "scan_emit" if "scan_emit" in kern else max(kern, key=kern.get)
    th = tokens * H
    bnd = gdn.segment_bounds(S, C, R)
    n_tok = {"scan_emit_first": bnd[1], "scan_carry": bnd[R - 1] - bnd[1], "scan_head_carry": bnd[R - 1],
             "scan_emit": S - bnd[1] if R > 1 else S}
    n_seg = {"scan_emit_first": 1, "scan_carry": R - 2, "scan_head_carry": R - 1, "scan_emit": max(R - 1, 1)}
    if dom in ("scan_emit", "scan_emit_first"):
        flops = flops_per_token_head(C, K, V) * n_tok[dom] * H
        nbytes = bytes_per_token_head(K, V, 2, 2) * n_tok[dom] * H + (n_seg[dom] + 1) * H * K * V * 4
    elif dom == "scan_carry":
        flops = carry_flops_per_token_head(C, K, V) * n_tok[dom] * H
        nbytes = ((K + V) * 2 + 8) * n_tok[dom] * H + (R - 2) * H * K * (K + V) * 4
    else:
        flops = 2 * (R - 2) * H * K * K * V
        nbytes = (R - 2) * H * (K * K + 2 * K * V) * 4
    t_dom = kern[dom] * 1e-3
    if backend == 1:
        roof = {"bound": "mfma", "achieved": flops / t_dom / 1e12, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "alu", "achieved": flops / t_dom / 1e12, "peak": PEAK_F32_VALU_TFLOPS,
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(f"{dom}@{n_tok.get(dom, S)}x{H}")
    roof["kernel"] = dom
    # workgroups of the launch: two per (segment, head); the chip runs one per CU
    wgs = 2 * n_seg.get(dom, R) * H
    roof["workgroups"] = wgs
    roof["frac_of_occupied_cus"] = roof["frac"] * 256 / min(wgs, 256)
    roof["kernel_ms"] = kern[dom]
    roof["algorithmic_flops_per_launch"] = flops
    roof["algorithmic_bytes_per_launch"] = nbytes
    roof["hbm_frac_at_algorithmic_bytes"] = nbytes / t_dom / 1e9 / PEAK_HBM_GBS
    useful = flops_per_token_head(C, K, V) * th
    result = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "ms_per_step_median": float(np.median(step_ms)), "ms_per_step_min": float(np.min(step_ms)),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; q,k L2-normalised, beta sigmoid, g -softplus)",
        "config": {"workload": f"B{B} H{H} S{S} K{K} V{V} C{C}, {R} contiguous segments "
                               "(three-phase pass, overlapped schedule), bf16 q/k/v/o, "
                               "fp32 g/beta/state",
                   "B": B, "H": H, "S": S, "K": K, "V": V, "C": C, "segments": R,
                   "parallelism": "1 GPU"},
        "roofline": roof,
        "kernels_ms": kern,   # dominant kernel from the timed steps, the rest from the second pass
        "useful_tflops": useful / (ms * 1e-3) / 1e12,
        "step_roofline": step_roofline(tokens, H, ms, C, K, V),
        "scan_backend": "mfma" if backend == 1 else "valu",
    }
    if R > 2:
        # executed work: the canonical FLOPs of every token plus the carrying pass over
        # segments 1 .. R-2 (its Gram, T applied, and the products over the K + V
        # columns of [M | h]), against the bf16 MFMA peak
        executed = useful + carry_flops_per_token_head(C, K, V) * (bnd[R - 1] - bnd[1]) * H
        result["step_roofline"]["executed_tflops"] = executed / (ms * 1e-3) / 1e12
        result["step_roofline"]["executed_mfma_frac"] = executed / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS
    del seg_step
    peaks = measured_peaks(torch, dev)
    result["measured_peaks"] = peaks
    if roof["bound"] == "mfma":
        roof["frac_of_measured_peak"] = roof["achieved"] / peaks["bf16_mfma_tflops"]
    roof["hbm_frac_of_measured_copy"] = nbytes / t_dom / 1e9 / peaks["hbm_copy_gbs"]

    # ---------------------------------------------------------------- secondary lines
    extra = {}
    if not args.no_extra:
        def mono(timer):
            tm = timer.around if timer else (lambda _n, f: f())
            return tm("scan_emit", lambda: gdn.scan_emit(q, k, v, g, beta, h_in=h0, chunk_size=C))
        steps2 = max(5, args.steps // 2)
        st = {}
        ms1, k1 = time_with_breakdown(torch, mono, steps2, 2, st)
        extra["monolithic_64k"] = {"tokens_per_s": tokens / (ms1 * 1e-3), "ms": ms1, **st,
                                   "step_roofline": step_roofline(tokens, H, ms1)}

        # the plain three-phase pass: carrying pass over every segment, scan, emitting
        # pass over every segment
        def plain(timer):
            tm = timer.around if timer else (lambda _n, f: f())
            M, U = tm("scan_carry", lambda: gdn.scan_carry(k, v, g, beta, chunk_size=C, n_segments=R))
            h_in, _ = tm("segment_compose", lambda: gdn.segment_compose(M, U, h0))
            return tm("scan_emit", lambda: gdn.scan_emit(q, k, v, g, beta, h_in=h_in, chunk_size=C,
                                                         n_segments=R))
        if R > 1:
            st = {}
            ms_pl, k_pl = time_with_breakdown(torch, plain, steps2, 2, st)
            extra["segmented_64k_plain_schedule"] = {"tokens_per_s": tokens / (ms_pl * 1e-3), **st,
                                                     "step_roofline": step_roofline(tokens, H, ms_pl),
                                                     "ms": ms_pl, "kernels_ms": k_pl}

        # the same three-phase pass with the WY factors prepared once and reused by
        # both passes (the pages' own arrangement), for comparison
        def seg_wy(timer):
            tm = timer.around if timer else (lambda _n, f: f())
            wy = tm("chunk_prepare", lambda: gdn.chunk_prepare(k, v, g, beta, chunk_size=C))
            M, U = tm("scan_carry", lambda: gdn.scan_carry(k, v, g, beta, wy=wy, chunk_size=C,
                                                           n_segments=R))
            h_in, _ = tm("segment_compose", lambda: gdn.segment_compose(M, U, h0))
            return tm("scan_emit", lambda: gdn.scan_emit(q, k, v, g, beta, h_in=h_in, wy=wy,
                                                         chunk_size=C, n_segments=R))
        if R > 1:
            st = {}
            ms_w, k_w = time_with_breakdown(torch, seg_wy, steps2, 2, st)
            extra["segmented_64k_wy_reused"] = {"tokens_per_s": tokens / (ms_w * 1e-3), "ms": ms_w, **st,
                                                "step_roofline": step_roofline(tokens, H, ms_w),
                                                "kernels_ms": k_w}

        # grouped key heads: the same step with q and k on H/2 heads (value head h reads
        # key head h // 2), as in models whose linear attention has fewer key heads
        if R > 1 and H % 2 == 0:
            qg, kg = q[:, :, : H // 2].contiguous(), k[:, :, : H // 2].contiguous()

            def grouped(timer):
                tm = timer.around if timer else (lambda _n, f: f())
                return gdn.forward_segmented(qg, kg, v, g, beta, h0=h0, chunk_size=C, n_segments=R, timer=tm)
            st = {}
            ms_g, k_g = time_with_breakdown(torch, grouped, steps2, 2, st)
            extra[f"segmented_64k_hqk{H // 2}"] = {"tokens_per_s": tokens / (ms_g * 1e-3), "ms": ms_g, **st,
                                                  "step_roofline": step_roofline(tokens, H, ms_g), "kernels_ms": k_g}
            del qg, kg

        # per-chunk WY preparation (gdn_chunk_prepare) of the same workload: an HBM
        # stream of k, v, g, beta in and w, u out
        def prep(timer):
            tm = timer.around if timer else (lambda _n, f: f())
            return tm("chunk_prepare", lambda: gdn.chunk_prepare(k, v, g, beta, chunk_size=C))
        st_p = {}
        ms_p, k_p = time_with_breakdown(torch, prep, steps2, 2, st_p)
        prep_bytes = th * ((K + V) * 2 + 8 + (K + V) * 2)
        t_p = k_p["chunk_prepare"] * 1e-3
        extra["chunk_prepare_64k"] = {
            "tokens_per_s": tokens / (ms_p * 1e-3), "ms": ms_p, **st_p,
            "roofline": {"bound": "hbm", "achieved": prep_bytes / t_p / 1e9, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": prep_bytes / t_p / 1e9 / PEAK_HBM_GBS},
        }
        del q, k, v, g, beta, h0
        torch.cuda.empty_cache()

        # the 4k sequence and the packed batch: one emitting scan over whole
        # sequences, and the piece schedule (long sequences cut into pieces that
        # run as parallel chains; the cut chosen by plan_pieces)
        for wl, name in ((1, "seq4k_h16"), (3, "packed8_32k")):
            y = workload(wl)
            t = lambda a, dt=None: (torch.from_numpy(a).to(dt) if dt else torch.from_numpy(a)).to(dev)
            yq, yk, yv = t(y.q, bf), t(y.k, bf), t(y.v, bf)
            yg, yb, yh = t(y.g), t(y.beta), t(y.h0)
            cu = y.cu_seqlens if y.cu_seqlens is not None else np.array([0, y.q.shape[1]], dtype=np.int32)
            chunks = tuple(-(-(int(cu[n + 1]) - int(cu[n])) // 64) for n in range(len(cu) - 1))
            m = gdn.plan_pieces(chunks, y.q.shape[2], torch.cuda.get_device_properties(dev).multi_processor_count)
            for tag, mm in (("", 0), ("_pieces", m)):
                log(f"bench: {name}{tag} (max_piece_chunks {mm})")

                def fwd(timer, yq=yq, yk=yk, yv=yv, yg=yg, yb=yb, yh=yh, cu=cu, mm=mm):
                    return gdn.forward_packed(yq, yk, yv, yg, yb, cu, h0=yh, chunk_size=64, max_piece_chunks=mm,
                                              timer=timer.around if timer else None)
                st = {}
                ms2, k2 = time_with_breakdown(torch, fwd, steps2, 2, st)
                extra[name + tag] = {"tokens_per_s": y.real_tokens / (ms2 * 1e-3), "ms": ms2, **st,
                                     "max_piece_chunks": mm,
                                     "step_roofline": step_roofline(y.real_tokens, y.q.shape[2], ms2),
                                     "pieces": gdn.num_pieces(yk, yv, 64, cu, mm), "kernels_ms": k2}
                if wl == 1 and tag == "":
                    # the 4k-token inputs (48 MiB of bf16 q, k, v) fit the 256 MB MALL:
                    # the same step with every cache flushed first
                    cold = time_cold_steps(torch, fwd, steps2)
                    extra[name + "_cold_caches"] = {
                        "tokens_per_s": y.real_tokens / (float(np.median(cold)) * 1e-3),
                        "ms_median": float(np.median(cold)), "ms_min": float(np.min(cold)),
                        "how": "1 GiB buffer written before each step; each step timed alone"}
            del yq, yk, yv, yg, yb, yh

        # the steps beside the core at the 64k workload's size: the depthwise causal conv
        # over the q, k, v channels (16 key heads and 32 value heads of 128: 8,192
        # channels; 4 taps, SiLU, with the conv state) and the gated RMSNorm of the
        # 32 x 128 outputs of every token; both stream HBM once
        log("bench: causal conv1d and gated rmsnorm")
        gen = torch.Generator(device=dev).manual_seed(7)
        Tn, Dc, Wc = 65536, 2 * 16 * 128 + 32 * 128, 4
        xc = torch.randn((1, Tn, Dc), device=dev, generator=gen).to(bf)
        wc = (torch.randn((Dc, Wc), device=dev, generator=gen) * 0.5).to(bf)
        sc = torch.randn((1, Dc, Wc - 1), device=dev, generator=gen).to(bf)

        def conv(timer):
            tm = timer.around if timer else (lambda _n, f: f())
            return tm("causal_conv1d", lambda: gdn.causal_conv1d(xc, wc, sc))
        st_c = {}
        ms_c, k_c = time_with_breakdown(torch, conv, steps2, 2, st_c)
        conv_bytes = Tn * Dc * 2 * 2 + Dc * Wc * 2 + 2 * Dc * (Wc - 1) * 2
        t_c = k_c["causal_conv1d"] * 1e-3
        extra["causal_conv1d_64k"] = {
            "tokens_per_s": Tn / (ms_c * 1e-3), "ms": ms_c, **st_c, "channels": Dc, "taps": Wc,
            "roofline": {"bound": "hbm", "achieved": conv_bytes / t_c / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": conv_bytes / t_c / 1e9 / PEAK_HBM_GBS},
        }
        del xc, wc, sc
        on = torch.randn((Tn, H, V), device=dev, generator=gen).to(bf)
        zn = torch.randn((Tn, H, V), device=dev, generator=gen).to(bf)
        wn = torch.randn((V,), device=dev, generator=gen)

        def norm(timer):
            tm = timer.around if timer else (lambda _n, f: f())
            return tm("gated_rmsnorm", lambda: gdn.gated_rmsnorm(on, wn, zn))
        st_n = {}
        ms_n, k_n = time_with_breakdown(torch, norm, steps2, 2, st_n)
        norm_bytes = Tn * H * V * 2 * 3 + V * 4
        t_n = k_n["gated_rmsnorm"] * 1e-3
        extra["gated_rmsnorm_64k"] = {
            "tokens_per_s": Tn / (ms_n * 1e-3), "ms": ms_n, **st_n,
            "roofline": {"bound": "hbm", "achieved": norm_bytes / t_n / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": norm_bytes / t_n / 1e9 / PEAK_HBM_GBS},
        }
        del on, zn, wn
        torch.cuda.empty_cache()

        log("bench: decode")
        nsteps = 128
        d = make_decode_inputs(4, 256, 32, 128, 128, nsteps, dtype="bf16")
        dq, dk, dv = (torch.from_numpy(a).to(bf).to(dev) for a in (d.q, d.k, d.v))
        dg, db = torch.from_numpy(d.g).to(dev), torch.from_numpy(d.beta).to(dev)
        state = torch.from_numpy(d.state0).to(dev)
        dout = torch.empty((256, 32, 128), dtype=bf, device=dev)

        def dec(timer):
            for s_ in range(nsteps):
                if timer:
                    timer.around("decode_step", lambda: gdn.decode_step(
                        dq[s_], dk[s_], dv[s_], dg[s_], db[s_], state, out=dout))
                else:
                    gdn.decode_step(dq[s_], dk[s_], dv[s_], dg[s_], db[s_], state, out=dout)
        ms3, k3 = time_with_breakdown(torch, dec, 2, 1)
        # every step timed on its own: an event between consecutive steps
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(nsteps + 1)]
        torch.cuda.synchronize()
        marks[0].record()
        for s_ in range(nsteps):
            gdn.decode_step(dq[s_], dk[s_], dv[s_], dg[s_], db[s_], state, out=dout)
            marks[s_ + 1].record()
        torch.cuda.synchronize()
        per_step_us = [1e3 * marks[i].elapsed_time(marks[i + 1]) for i in range(nsteps)]
        step_bytes = 2 * 256 * 32 * 128 * 128 * 4 + 256 * 32 * ((2 * 128 + 128) * 2 + 128 * 2 + 8)
        t_step = k3["decode_step"] * 1e-3
        extra["decode_b256_h32"] = {
            "tokens_per_s": 256 * nsteps / (ms3 * 1e-3), "ms_per_128_steps": ms3,
            "us_per_step_kernel": t_step * 1e6,
            "us_per_step_median": float(np.median(per_step_us)), "us_per_step_min": float(np.min(per_step_us)),
            "ms_total_128_steps_each_timed": float(np.sum(per_step_us)) * 1e-3,
            "roofline": {"bound": "hbm", "achieved": step_bytes / t_step / 1e9,
                         "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": step_bytes / t_step / 1e9 / PEAK_HBM_GBS},
        }
        del dq, dk, dv, dg, db, state
        torch.cuda.empty_cache()

        # the backward pass (gradients of a loss through the forward): the 4k sequence
        # and the 64k workload.  Its products run as fp32 matrix-core tiles (the rest on
        # the fp32 vector ALU, whose peak is the same figure), so the roofline is the
        # fp32 peak against the dense work of its four kernels.
        log("bench: backward")
        for name, wl in (("backward_seq4k_h16", 1), ("backward_64k_h32", 2)):
            y = x if wl == 2 else workload(wl)
            t = lambda a, dt=None: (torch.from_numpy(a).to(dt) if dt else torch.from_numpy(a)).to(dev)
            bq, bk, bv, bg, bb, bh = t(y.q, bf), t(y.k, bf), t(y.v, bf), t(y.g), t(y.beta), t(y.h0)
            gen = torch.Generator(device=dev).manual_seed(11)
            bdo = torch.randn(bv.shape, device=dev, generator=gen).to(bf)
            bdh = torch.randn(bh.shape, device=dev, generator=gen)
            Sb, Hb = bq.shape[1], bq.shape[2]

            def bwd(timer):
                tm = timer.around if timer else (lambda _n, f: f())
                return tm("backward", lambda: gdn.backward(bq, bk, bv, bg, bb, bdo, h0=bh, dhT=bdh))
            st_b = {}
            ms_b, k_b = time_with_breakdown(torch, bwd, max(3, steps2 // 2), 1, st_b)
            fl = Sb * Hb * bwd_flops_per_token_head(C, K, V)
            t_b = k_b["backward"] * 1e-3
            extra[name] = {
                "tokens_per_s": Sb / (ms_b * 1e-3), "ms": ms_b, **st_b,
                "roofline": {"bound": "mfma", "achieved": fl / t_b / 1e12, "peak": PEAK_F32_VALU_TFLOPS,
                             "unit": "TFLOP/s", "frac": fl / t_b / 1e12 / PEAK_F32_VALU_TFLOPS,
                             "frac_of_measured_peak": fl / t_b / 1e12 / peaks["f32_mfma_tflops"]},
            }
            del bq, bk, bv, bg, bb, bh, bdo, bdh
            torch.cuda.empty_cache()
    result["extra"] = extra

    # ---------------------------------------------------------------- CPU oracle baseline
    if not args.no_cpu_baseline:
        import oracle
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
        nh = max(1, min(H, threads))
        log(f"bench: oracle baseline on {nh} heads, {threads} threads")
        probe = 256
        t0 = time.perf_counter()
        oracle.forward(x.q[:, :probe, :nh], x.k[:, :probe, :nh], x.v[:, :probe, :nh],
                       x.g[:, :probe, :nh], x.beta[:, :probe, :nh], h0=x.h0[:, :nh],
                       nthreads=min(threads, nh))
        dt = max(time.perf_counter() - t0, 1e-6)
        ns = int(min(S, max(probe, probe * args.cpu_seconds / dt)))
        # when the whole sequence takes less than the target, repeat it
        reps = 0
        t0 = time.perf_counter()
        while True:
            oracle.forward(x.q[:, :ns, :nh], x.k[:, :ns, :nh], x.v[:, :ns, :nh],
                           x.g[:, :ns, :nh], x.beta[:, :ns, :nh], h0=x.h0[:, :nh],
                           nthreads=min(threads, nh))
            reps += 1
            dt = time.perf_counter() - t0
            if dt >= 0.9 * args.cpu_seconds:
                break
        # one core: one head of the same tokens (about a sixteenth of the work above)
        n1 = ns
        t1 = time.perf_counter()
        oracle.forward(x.q[:, :n1, :1], x.k[:, :n1, :1], x.v[:, :n1, :1], x.g[:, :n1, :1],
                       x.beta[:, :n1, :1], h0=x.h0[:, :1], nthreads=1)
        d1 = time.perf_counter() - t1
        result["cpu_baseline"] = {
            "value": reps * ns * nh / H / dt, "unit": "tokens/s", "cores": min(threads, nh),
            "kind": "oracle",
            "sample": f"first {ns} tokens x {nh} of {H} heads of the 64k-token workload, "
                      f"{reps} pass(es), fp64 token recurrence, {dt:.1f} s; tokens/s counts "
                      f"whole {H}-head tokens",
            "cpu_model": cpu_model(),
            "host_cpus": {"os_cpu_count": os.cpu_count(),
                          "affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None},
            "single_core": {"value": n1 / H / d1, "unit": "tokens/s",
                            "sample": f"first {n1} tokens x 1 head, 1 thread, {d1:.1f} s"},
        }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

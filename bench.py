"""Benchmark of the FLARE / FLARE++ mixer hot path on one MI355X.

Default workload: FLARE encode + decode at mesh scale, bf16, B=1, H=8, D=32,
N=1,048,576 tokens, M=256 latents per head (K, V and Q ~ N(0, 1), seed 0).
One step = flare_encode (split-token kernel + logsumexp merge) followed by
flare_decode, on inputs already resident in HBM.  Prints ONE JSON line.

The roofline object also carries the shader clock measured live under the
dominant kernel (a one-wave sampler on a second stream), the matrix-core
fraction against the peak scaled to that clock, and the exponential unit's
share of its rate at that clock.

Also measured in the same run (reported under "extra"): the same workload
with sharp scores (Q x 40, which sends every split to the exact-softmax
rerun), FLARE++ attention, the backward pair, the whole FLARE++ mixer at the
same sizes (C = 256: four input projections, query synthesis, encode, decode,
output projection) via flare_mix and its variants, the smaller FLARE++
workloads, a sweep over the token count, and the oracle on a bounded sample
on the host cores ("cpu_baseline").

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu]
       python bench.py --copy-calibration   (plain device copy, for PMC scaling)
       python bench.py --write-traffic FETCH.csv WRITE.csv COPY_FETCH.csv COPY_WRITE.csv
           (host only: turns rocprofv3 FETCH_SIZE / WRITE_SIZE counter files of
            the bench kernels and of the copy into profiles/traffic_<kernel>.json)
       python bench.py --summarize NAME DIR [DIR ...]
           (host only: writes a profiles/*.md summary from rocprofv3 output)
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (published)
PEAK_CLOCK_GHZ = 2.4             # engine clock the published peaks assume
# v_exp_f32 retires one wave64 instruction per 8 cycles per SIMD (8.3 measured
# at 4 waves per SIMD, profiles/issue_rates.gfx950.md): 8 exponentials per
# cycle per SIMD, 1024 SIMDs.
EXP_PER_CYCLE = 8 * 1024
REALTIME_HZ = 1e8                # the 100 MHz real-time counter of gfx950
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E (published)
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-mix", action="store_true", help="skip the FLARE++ mixer measurement")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward measurement")
    ap.add_argument("--no-sweep", action="store_true", help="skip the sweep over the token count")
    ap.add_argument("--cpu-heads", type=int, default=4, help="heads in the oracle sample")
    ap.add_argument("--y-layout", choices=("token", "head"), default="token")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"))
    ap.add_argument("--summarize", nargs="+", metavar=("NAME", "INPUT"),
                    help="host only: write profiles/<NAME>.md from rocprofv3 output (NAME: units, "
                         "units_gemm, units_bwd, clock, stats TRACE_DIR [BENCH_LOG], xreuse TIMING.md PMC_DIR, "
                         "issue_rates TIMING.md "
                         "PMC_DIRS...)")
    return ap.parse_args()


def summarize(name, inputs):
    """Writes one committed profile summary from rocprofv3 output directories."""
    from rank_latent_routing_amd import profiling
    os.makedirs(PROFILES, exist_ok=True)
    if name == "units":
        b = profiling.write_units(os.path.join(PROFILES, "units.encdec_n1m.md"), inputs)
        for k, v in b.items():
            print(f"{k}: {v['cycles']:.0f} cycles per block, VALU issue {v['issue']:.0f}, none {v['idle']:.0f}")
    elif name == "units_gemm":
        profiling.write_units_gemm(os.path.join(PROFILES, "units_gemm.mix_n1m.md"), inputs, PROFILES)
    elif name == "issue_rates":
        profiling.write_issue_rates(os.path.join(PROFILES, "issue_rates.gfx950.md"), inputs[1:], inputs[0])
    elif name == "stats":
        profiling.write_stats(os.path.join(PROFILES, "kernel_stats.encdec_n1m.md"), inputs[0],
                              inputs[1] if len(inputs) > 1 else None)
    elif name == "clock":
        profiling.write_clock(os.path.join(PROFILES, "clock.encdec_n1m.md"), inputs)
    elif name == "units_bwd":
        profiling.write_units_bwd(os.path.join(PROFILES, "units_bwd.encdec_n1m.md"), inputs)
    elif name == "xreuse":
        profiling.write_xreuse(os.path.join(PROFILES, "xreuse.block_c5.md"), inputs[0], inputs[1], PROFILES)
    else:
        raise SystemExit(f"unknown summary {name}")


# Sources whose change invalidates a stored counter reading of a kernel
# (the kernel itself, shared device code, and the host code that picks its
# grid).
KERNEL_SOURCES = {
    "encode_bf16_kernel": ["encode_kernel.hpp", "encode_wide.hip", "encode.hip", "common.hpp", "launch.hpp", "api.cpp",
                           "plan.cpp"],
    "merge_kernel": ["encode_kernel.hpp", "encode_wide.hip", "encode.hip", "common.hpp", "launch.hpp", "api.cpp",
                     "plan.cpp"],
    "decode_bf16_kernel": ["decode.hip", "common.hpp", "launch.hpp", "api.cpp", "plan.cpp"],
}
COPY_BYTES = 1 << 30  # bytes read (and written) per launch of the calibration copy


class ClockSampler:
    """The shader clock while a kernel runs: a sampler kernel (the probes
    library's clock_sample, one wave on each XCD) spins on a second stream for
    WINDOW_MS of real time, reading the shader clock and the real-time
    counters, while the kernel is launched back to back on the main stream for
    about twice that long.  The sampler starts first on an idle GPU, so its
    window lies inside the kernel launches; it holds one wave slot of one
    compute unit per XCD.  under() returns the mean clock over the XCDs and
    the spread (min, max)."""
    WINDOW_MS = 2.0

    def __init__(self, torch):
        import ctypes
        from rank_latent_routing_amd.probes import run_probes
        if not os.path.exists(run_probes.LIB):
            raise RuntimeError(f"{run_probes.LIB} missing: run __graft_entry__.build()")
        self.torch = torch
        self.lib = ctypes.CDLL(run_probes.LIB)
        self.lib.clock_sample.argtypes = [ctypes.c_void_p, ctypes.c_ulonglong, ctypes.c_void_p]
        self.lib.clock_sample.restype = ctypes.c_int
        self.out = torch.zeros(32, dtype=torch.int64, device="cuda:0")
        self.side = torch.cuda.Stream()

    def under(self, launch, ms_per_launch):
        torch = self.torch
        torch.cuda.synchronize()
        n = int(2 * self.WINDOW_MS / max(ms_per_launch, 1e-3)) + 2
        rc = self.lib.clock_sample(self.out.data_ptr(), int(self.WINDOW_MS * 1e-3 * REALTIME_HZ),
                                   self.side.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"clock_sample failed ({rc})")
        for _ in range(n):
            launch()
        torch.cuda.synchronize()
        v = self.out.tolist()
        ghz = [(v[4 * i + 3] - v[4 * i + 2]) / ((v[4 * i + 1] - v[4 * i]) / REALTIME_HZ) / 1e9 for i in range(8)]
        return sum(ghz) / len(ghz), (min(ghz), max(ghz))


def _code_only(text):
    """The source without its comments, trailing blanks and empty lines: what
    a counter reading depends on.  (None of these sources has "//" or "/*"
    inside a string literal.)"""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", l).rstrip() for l in text.splitlines())
    return "\n".join(l for l in lines if l)


def kernel_source_sha(kernel):
    """Hash of a kernel's sources (code only) and of their per-source build flags."""
    from rank_latent_routing_amd import build as lib_build
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "rank_latent_routing_amd", "csrc", f)) as fh:
            h.update(_code_only(fh.read()).encode())
        h.update(" ".join(lib_build.SOURCE_FLAGS.get(f, [])).encode())
    return h.hexdigest()[:16]


def stored_traffic(kernels):
    """HBM bytes per launch (summed over the given kernels) from the committed
    counter summaries, if every one was taken on the current kernel source;
    else None."""
    total = 0.0
    for kernel in kernels:
        p = os.path.join(PROFILES, f"traffic_{kernel}.encdec_n1m.json")
        if not os.path.exists(p):
            return None
        d = json.load(open(p))
        if d.get("source_sha") != kernel_source_sha(kernel):
            return None
        total += d["bytes_per_launch"]
    return total


# Launches of each bench kernel in the timed steps of a counter run's metric
# step loop (`--steps 3 --warmup 1`: launches 1 .. 3); the warm-up and later
# launches of the same kernels (the clock samples, the sharp-score and
# FLARE++ extras, the backward leg's forward pass) are left out of the
# forward figures.
TRAFFIC_STEP_LAUNCHES = (1, 4)


def counter_means(path, counter, launches=None):
    """Mean over dispatches of one counter, per kernel (full demangled name),
    from a rocprofv3 counter_collection csv (rows of one dispatch are summed);
    with `launches` = (lo, hi), over dispatches lo .. hi - 1 of each kernel."""
    import csv
    import collections
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    for row in csv.DictReader(open(path)):
        if row["Counter_Name"] == counter:
            per[row["Kernel_Name"]][int(row["Dispatch_Id"])] += float(row["Counter_Value"])
    out = {}
    for k, v in per.items():
        vals = [x for _, x in sorted(v.items())]
        if launches is not None:
            vals = vals[launches[0]:launches[1]] or vals
        out[k] = sum(vals) / len(vals)
    return out


def library_kernel(means, kernel):
    """The value of our kernel `kernel` (any template instance) in `means`."""
    hits = [v for k, v in means.items() if f"flare::{kernel}" in k]
    return hits[0] if len(hits) == 1 else None


def write_traffic(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv):
    """HBM bytes per launch of the bench kernels from FETCH_SIZE / WRITE_SIZE
    (KiB per dispatch), each scaled by what the same counter reads for a
    plain 1 GiB device copy."""
    fetch = counter_means(fetch_csv, "FETCH_SIZE", TRAFFIC_STEP_LAUNCHES)
    write = counter_means(write_csv, "WRITE_SIZE", TRAFFIC_STEP_LAUNCHES)
    cf, cw = counter_means(copy_fetch_csv, "FETCH_SIZE"), counter_means(copy_write_csv, "WRITE_SIZE")
    copy_kernel = max(cf, key=cf.get)
    f_read = COPY_BYTES / (cf[copy_kernel] * 1024.0)
    f_write = COPY_BYTES / (cw[copy_kernel] * 1024.0)
    os.makedirs(PROFILES, exist_ok=True)
    for kernel in KERNEL_SOURCES:
        kf, kw = library_kernel(fetch, kernel), library_kernel(write, kernel)
        if kf is None or kw is None:
            continue
        d = {"kernel": kernel,
             "workload": "FLARE encode+decode, B=1, H=8, D=32, N=1048576, M=256, bf16 (bench.py default)",
             "source_sha": kernel_source_sha(kernel),
             "fetch_kib_per_dispatch": kf, "write_kib_per_dispatch": kw,
             "copy_kernel": copy_kernel, "copy_fetch_kib": cf[copy_kernel], "copy_write_kib": cw[copy_kernel],
             "copy_factor_read": f_read, "copy_factor_write": f_write,
             "bytes_read_per_launch": kf * 1024.0 * f_read,
             "bytes_written_per_launch": kw * 1024.0 * f_write,
             "bytes_per_launch": kf * 1024.0 * f_read + kw * 1024.0 * f_write}
        with open(os.path.join(PROFILES, f"traffic_{kernel}.encdec_n1m.json"), "w") as fh:
            json.dump(d, fh, indent=1)
        print(f"{kernel}: {d['bytes_per_launch'] / 1e9:.3f} GB per launch "
              f"(read {d['bytes_read_per_launch'] / 1e9:.3f}, written {d['bytes_written_per_launch'] / 1e9:.3f})")
    from rank_latent_routing_amd import profiling
    profiling.write_traffic_md(os.path.join(PROFILES, "traffic.encdec_n1m.md"), fetch_csv, write_csv, f_read, f_write,
                               (cf[copy_kernel], cw[copy_kernel]), TRAFFIC_STEP_LAUNCHES)


def copy_calibration():
    import torch
    n = 1 << 28  # 256 Mi fp32 = 1 GiB
    a = torch.ones(n, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 3}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU (asked for --gpus {args.gpus}); "
              "multi-GPU sharding of the encoder is a design note, not built.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        return copy_calibration()
    if args.write_traffic:
        return write_traffic(*args.write_traffic)
    if args.summarize:
        return summarize(args.summarize[0], args.summarize[1:])

    import numpy as np
    import torch
    import rank_latent_routing_amd as rl
    from rank_latent_routing_amd import costs, inputs

    dev = torch.device("cuda:0")
    w = inputs.WORKLOADS["encdec_bf16_n1m"]
    B, N, H, D, M = w.B, w.N, w.H, w.D, w.M
    x = inputs.make_encdec(w, seed=0, synth=True)  # q, k, v first; then eK, eV, seeds
    q = x["q"].to(dev)
    k = x["k"].permute(0, 2, 1, 3).contiguous().to(dev)   # head-major [B, H, N, D]
    v = x["v"].permute(0, 2, 1, 3).contiguous().to(dev)
    z = torch.empty((B, H, M, D), dtype=torch.bfloat16, device=dev)
    if args.y_layout == "token":
        y_store = torch.empty((B, N, H, D), dtype=torch.bfloat16, device=dev)
        y = y_store.permute(0, 2, 1, 3)
    else:
        y = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(rl.encode_workspace_size(B, H, M, N, D), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step():
        rl.flare_encode(q, k, v, z=z, workspace=ws, stream=stream)
        rl.flare_decode(k, q, z, y=y, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        rl.flare_encode(q, k, v, z=z, workspace=ws, stream=stream)
        ev[i][1].record(stream)
        rl.flare_decode(k, q, z, y=y, stream=stream)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    enc_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    dec_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))

    enc = costs.encode(B, H, N, M, D)
    dec = costs.decode(B, H, N, M, D)
    tokens = B * N
    value = tokens / (ms_step / 1e3)
    tflops_step = (enc.flops + dec.flops) / (ms_step / 1e3) / 1e12

    # Dominant kernel: the longer of the two calls.  The decode call is one
    # kernel; the encode call is the split kernel plus a small merge.
    if dec_ms >= enc_ms:
        kname, kms, kwork = "decode_bf16_kernel", dec_ms, dec
    else:
        kname, kms, kwork = "encode_bf16_kernel+merge_kernel", enc_ms, enc
    achieved = kwork.flops / (kms / 1e3) / 1e12
    roofline = {"bound": "mfma", "kernel": kname, "achieved": round(achieved, 2),
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": stored_traffic(kname.split("+")),
                "algorithmic_per_launch": {"flops": kwork.flops, "bytes": kwork.bytes,
                                           "unit": "per (token, head): 4*M*D flops, 4*D bytes",
                                           "units_per_launch": B * H * N},
                "hbm_algorithmic_GBs": round(kwork.bytes / (kms / 1e3) / 1e9, 1),
                "hbm_frac": round(kwork.bytes / (kms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}

    # The shader clock under each kernel (the chip runs below its 2.4 GHz
    # peak clock under this load), and the roofline again at that clock: the
    # matrix-core fraction against the peak scaled to the clock, and the
    # share of the exponential unit's rate at that clock.
    # The clock that prices the roofline is the one under the timed loop's
    # own pattern (encode and decode alternating); each kernel launched alone
    # back to back draws a different power, so its clock is reported apart.
    sampler = ClockSampler(torch)
    step_clk, step_spread = sampler.under(step, ms_step)
    enc_clk, enc_spread = sampler.under(lambda: rl.flare_encode(q, k, v, z=z, workspace=ws, stream=stream), enc_ms)
    dec_clk, dec_spread = sampler.under(lambda: rl.flare_decode(k, q, z, y=y, stream=stream), dec_ms)
    kclk = step_clk
    roofline["clock_GHz"] = round(kclk, 3)
    roofline["frac_at_clock"] = round(achieved / (MFMA_BF16_PEAK_TFLOPS * kclk / PEAK_CLOCK_GHZ), 4)
    roofline["exp_pipe_frac"] = round(kwork.exps / (kms / 1e3) / (EXP_PER_CYCLE * kclk * 1e9), 4)

    extra = {"encode_ms": round(enc_ms, 4), "decode_ms": round(dec_ms, 4),
             "clock_GHz": {"step": round(step_clk, 3), "encode_alone": round(enc_clk, 3),
                           "decode_alone": round(dec_clk, 3),
                           "xcd_min_max": {"step": [round(a, 3) for a in step_spread],
                                           "encode_alone": [round(a, 3) for a in enc_spread],
                                           "decode_alone": [round(a, 3) for a in dec_spread]}},
             "encode_frac_at_clock": round(enc.flops / (enc_ms / 1e3) / 1e12 /
                                           (MFMA_BF16_PEAK_TFLOPS * step_clk / PEAK_CLOCK_GHZ), 4),
             "encode_exp_pipe_frac": round(enc.exps / (enc_ms / 1e3) / (EXP_PER_CYCLE * step_clk * 1e9), 4),
             "decode_frac_at_clock": round(dec.flops / (dec_ms / 1e3) / 1e12 /
                                           (MFMA_BF16_PEAK_TFLOPS * step_clk / PEAK_CLOCK_GHZ), 4),
             "decode_exp_pipe_frac": round(dec.exps / (dec_ms / 1e3) / (EXP_PER_CYCLE * step_clk * 1e9), 4),
             "encode_tflops": round(enc.flops / (enc_ms / 1e3) / 1e12, 1),
             "decode_tflops": round(dec.flops / (dec_ms / 1e3) / 1e12, 1),
             "step_tflops": round(tflops_step, 1),
             "step_mfma_frac": round(tflops_step / MFMA_BF16_PEAK_TFLOPS, 4),
             "step_hbm_GBs": round((enc.bytes + dec.bytes) / (ms_step / 1e3) / 1e9, 1),
             "exps_per_s": (enc.exps + dec.exps) / (ms_step / 1e3)}

    # Parity spot check of this exact run against the oracle (two latents of
    # head 0 and a few tokens), so a broken kernel cannot report a number.
    import oracle
    qh = x["q"][0].double().numpy()
    kh = x["k"][0, :, 0].double().numpy()
    vh = x["v"][0, :, 0].double().numpy()
    zr = oracle.sdpa(qh, kh, vh)
    rows = np.arange(0, N, N // 64)
    yr = oracle.sdpa(kh[rows], qh, zr)
    zg = z[0, 0].double().cpu().numpy()
    yg = y[0, 0].double().cpu().numpy()[rows]
    rel = lambda a, b: float(np.linalg.norm(a - b) / np.linalg.norm(b))
    extra["parity_rel_l2"] = {"Z_head0": rel(zg, zr), "Y_head0_64_tokens": rel(yg, yr)}
    if extra["parity_rel_l2"]["Z_head0"] > 1e-2 or extra["parity_rel_l2"]["Y_head0_64_tokens"] > 1e-2:
        print("bench.py: parity check failed", extra["parity_rel_l2"], file=sys.stderr)
        sys.exit(3)

    # Sharp scores: the same workload with Q x 40 (rounded to bf16 once), so
    # that a latent's scores span hundreds of units in base 2.  The fast
    # softmax's range check then fails in every split and token group and the
    # exact running-maximum pass reruns them: "default" is that cost, next to
    # FLARE_FLAG_EXACT_SOFTMAX (the exact pass alone) and the metric workload.
    q40 = (q.float() * 40.0).to(torch.bfloat16)

    def timed(f, n):
        for _ in range(2):
            f()
        torch.cuda.synchronize()
        t0e, t1e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0e.record(stream)
        for _ in range(n):
            f()
        t1e.record(stream)
        torch.cuda.synchronize()
        return t0e.elapsed_time(t1e) / n

    def sharp(flags):
        def f():
            rl.flare_encode(q40, k, v, z=z, workspace=ws, flags=flags, stream=stream)
            rl.flare_decode(k, q40, z, y=y, flags=flags, stream=stream)
        return f
    sn = max(3, args.steps // 2)
    sharp_ms = timed(sharp(0), sn)
    exact_ms = timed(sharp(rl.FLARE_FLAG_EXACT_SOFTMAX), sn)
    extra["sharp_q40"] = {
        "config": "metric workload with Q x 40 (scores of a few hundred in base 2): every split and token group "
                  "fails the fast softmax's range check and reruns with the exact running maximum",
        "ms": round(sharp_ms, 4), "exact_flag_ms": round(exact_ms, 4), "metric_ms": round(ms_step, 4),
        "fallback_cost": round(sharp_ms / ms_step, 3), "over_exact": round(sharp_ms / exact_ms, 3)}
    del q40

    # FLARE++ attention at the same sizes: the query synthesis Q(X) =
    # SDPA(seeds, eK, eV) over separate eK, eV ~ N(0, 1), then the encode and
    # decode with Q(X) (the metric workload with the synthesis added; no
    # projections).
    ek = x["ek"].permute(0, 2, 1, 3).contiguous().to(dev)
    ev = x["ev"].permute(0, 2, 1, 3).contiguous().to(dev)
    seeds = x["seeds"].to(dev)
    qx = torch.empty((B, H, M, D), dtype=torch.float32, device=dev)

    def pp_step():
        rl.flare_route_queries(seeds, ek, ev, qx=qx, workspace=ws, stream=stream)
        rl.flare_encode(qx, k, v, z=z, workspace=ws, stream=stream)
        rl.flare_decode(k, qx, z, y=y, stream=stream)

    for _ in range(max(2, args.warmup // 2)):
        pp_step()
    torch.cuda.synchronize()
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record(stream)
    for _ in range(args.steps):
        pp_step()
    p1.record(stream)
    torch.cuda.synchronize()
    pp_ms = p0.elapsed_time(p1) / args.steps
    pp_flops = 3 * enc.flops
    extra["flarepp_encdec"] = {
        "config": "FLARE++ attention: query synthesis from seeds over eK, eV, then encode and decode; "
                  "B=1, H=8, D=32, N=1048576, M=256, bf16, no projections",
        "ms": round(pp_ms, 4), "tokens_per_s": tokens / (pp_ms / 1e3),
        "tflops": round(pp_flops / (pp_ms / 1e3) / 1e12, 1),
        "mfma_frac": round(pp_flops / (pp_ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "over_flare": round(pp_ms / ms_step, 3)}
    del ek, ev, seeds, qx

    if not args.no_bwd:
        # Backward of the same encode + decode pair: decoder gradient (dK, dQ,
        # dZ), then the encoder's (dQ, dK accumulated, dV), from the forward
        # normalisers; fp32 gradients, upstream gradient ~ N(0, 1).
        zf, lse_e = rl.flare_encode(q, k, v, want_lse=True, z_dtype=torch.float32, stream=stream)
        yb, lse_d = rl.flare_decode(k, q, zf, want_lse=True, stream=stream)
        dy = torch.randn((B, H, N, D), generator=torch.Generator(device=dev).manual_seed(0), device=dev,
                         dtype=torch.float32).to(torch.bfloat16)
        dk_b = torch.empty((B, H, N, D), dtype=torch.float32, device=dev)
        dv_b = torch.empty_like(dk_b)
        dq_b = torch.empty((B, H, M, D), dtype=torch.float32, device=dev)
        dz_b = torch.empty_like(dq_b)
        wsd = torch.empty(rl.lib().flare_decode_backward_workspace_size(B, H, M, N, D), dtype=torch.uint8,
                          device=dev)
        wse = torch.empty(rl.lib().flare_encode_backward_workspace_size(B, H, M, N, D), dtype=torch.uint8,
                          device=dev)
        wsp = torch.empty(rl.lib().flare_encdec_backward_workspace_size(B, H, M, N, D), dtype=torch.uint8,
                          device=dev)
        acc = rl.FLARE_ACCUMULATE_DQ | rl.FLARE_ACCUMULATE_DK

        def pair():
            rl.flare_encdec_backward(q, k, v, zf, lse_e, yb, lse_d, dy, dq=dq_b, dk=dk_b, dv=dv_b,
                                     workspace=wsp, stream=stream)

        def two_calls():
            rl.flare_decode_backward(k, q, zf, yb, lse_d, dy, dk=dk_b, dq=dq_b, dz=dz_b, workspace=wsd,
                                     stream=stream)
            rl.flare_encode_backward(q, k, v, zf, lse_e, dz_b, dq=dq_b, dk=dk_b, dv=dv_b, flags=acc,
                                     workspace=wse, stream=stream)

        def time_bwd(f):
            for _ in range(max(2, args.warmup // 2)):
                f()
            torch.cuda.synchronize()
            b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            bsteps = max(3, args.steps // 2)
            b0.record(stream)
            for _ in range(bsteps):
                f()
            b1.record(stream)
            torch.cuda.synchronize()
            return b0.elapsed_time(b1) / bsteps
        bms = time_bwd(pair)
        sms = time_bwd(two_calls)
        dk_h = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=dev)
        dv_h = torch.empty_like(dk_h)

        def pair_bf16():
            rl.flare_encdec_backward(q, k, v, zf, lse_e, yb, lse_d, dy, dq=dq_b, dk=dk_h, dv=dv_h,
                                     workspace=wsp, stream=stream)

        hms = time_bwd(pair_bf16)
        del dk_h, dv_h
        bwk = costs.encdec_backward(B, H, N, M, D)
        extra["encdec_backward"] = {
            "config": "gradients of FLARE encode+decode (dQ, dK, dV) at the bench sizes, bf16 inputs, "
                      "fp32 gradients, one flare_encdec_backward call",
            "ms": round(bms, 4), "tokens_per_s": tokens / (bms / 1e3),
            "tflops": round(bwk.flops / (bms / 1e3) / 1e12, 1),
            "over_forward": round(bms / ms_step, 3),
            "two_calls_ms": round(sms, 4),
            "bf16_gradients_ms": round(hms, 4)}
        del zf, yb, dy, dk_b, dv_b, dq_b, dz_b, wsd, wse, wsp

    if not args.no_mix:
        # FLARE++ forward mixer at the same sizes: C = 256, all projections.
        mw = inputs.Workload("mix_n1m", "mix", 1, N, H, D, M, "bf16", dynamic=True, has_wo=True)
        del k, v
        m = {n: t.to(dev) for n, t in inputs.make_mix(mw, seed=0).items()}
        out = torch.empty_like(m["x"])
        mws = torch.empty(rl.mix_workspace_size(1, N, mw.C, H, M, True, True), dtype=torch.uint8,
                          device=dev)

        msteps = max(3, args.steps // 2)

        def time_mix(**kw):
            def run():
                rl.flare_mix(m["x"], m["w_k"], m["w_v"], m["qs"], H, w_o=m["w_o"], out=out, workspace=mws,
                             stream=stream, **kw)
            for _ in range(max(2, args.warmup // 2)):
                run()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(msteps):
                run()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / msteps

        def mix_entry(what, ms, wk):
            return {"config": f"{what} with all projections, B=1, N=1048576, C=256, H=8, D=32, M=256, bf16",
                    "ms": round(ms, 4), "tokens_per_s": N / (ms / 1e3),
                    "tflops": round(wk.flops / (ms / 1e3) / 1e12, 1)}
        # FLARE++ (synthesis with its own eK/eV projections), FLARE++ with
        # shared projections (the synthesis attends over K and V), and FLARE
        # (fixed learned queries), for the cost ratios the pages discuss.
        mms = time_mix(w_ek=m["w_ek"], w_ev=m["w_ev"])
        sms = time_mix(w_ek=m["w_k"], w_ev=m["w_v"])
        fms = time_mix()
        mwk = costs.mixer(1, N, mw.C, H, M, dynamic=True, has_wo=True)
        fwk = costs.mixer(1, N, mw.C, H, M, dynamic=False, has_wo=True)
        swk = costs.mixer(1, N, mw.C, H, M, dynamic=True, has_wo=True, shared=True)
        extra["flarepp_mixer"] = mix_entry("FLARE++ mixer", mms, mwk)
        extra["flarepp_shared_mixer"] = mix_entry("FLARE++ mixer, shared projections (eK = K, eV = V)", sms, swk)
        extra["flare_mixer"] = mix_entry("FLARE mixer", fms, fwk)
        extra["flarepp_over_flare"] = {"time": round(mms / fms, 3),
                                       "operations": round(mwk.flops / fwk.flops, 3),
                                       "shared_time": round(sms / fms, 3),
                                       "shared_operations": round(swk.flops / fwk.flops, 3)}
        del m, out, mws

        # The small FLARE++ mixer (B=8, N=4096, C=128, H=8, D=16, M=64): a
        # dozen short launches per call, so launch overhead matters; timed as
        # eager calls and as replays of one captured HIP graph.
        sw = inputs.WORKLOADS["mix_bf16_n4k_c128"]
        sm = {n: t.to(dev) for n, t in inputs.make_mix(sw, seed=0).items()}
        sout = torch.empty_like(sm["x"])
        sws = torch.empty(rl.mix_workspace_size(sw.B, sw.N, sw.C, sw.H, sw.M, True, False), dtype=torch.uint8,
                          device=dev)

        def small_mix(s=stream):
            rl.flare_mix(sm["x"], sm["w_k"], sm["w_v"], sm["qs"], sw.H, w_ek=sm["w_ek"], w_ev=sm["w_ev"],
                         out=sout, workspace=sws, stream=s)
        reps = 50
        for _ in range(5):
            small_mix()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        h0 = time.perf_counter()
        for _ in range(reps):
            small_mix()
        eager_host_us = (time.perf_counter() - h0) / reps * 1e6
        e1.record(stream)
        torch.cuda.synchronize()
        eager_ms = e0.elapsed_time(e1) / reps
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()  # capture needs a side stream; replays go on the launch stream
        with torch.cuda.graph(graph, stream=cap):
            small_mix(cap)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            graph.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        h0 = time.perf_counter()
        with torch.cuda.stream(stream):
            for _ in range(reps):
                graph.replay()
        graph_host_us = (time.perf_counter() - h0) / reps * 1e6
        e1.record(stream)
        torch.cuda.synchronize()
        graph_ms = e0.elapsed_time(e1) / reps
        # Ten calls captured in one graph: the per-replay cost of a graph
        # launch is paid once per ten calls.
        graph10 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph10, stream=cap):
            for _ in range(10):
                small_mix(cap)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            graph10.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        with torch.cuda.stream(stream):
            for _ in range(reps // 10):
                graph10.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        graph10_ms = e0.elapsed_time(e1) / (10 * (reps // 10))
        extra["small_flarepp_mixer"] = {
            "config": "FLARE++ mixer, B=8, N=4096, C=128, H=8, D=16, M=64, bf16, no W_O",
            "eager_ms": round(eager_ms, 4), "graph_ms": round(graph_ms, 4),
            "graph_10_calls_per_replay_ms": round(graph10_ms, 4),
            # host time to issue one call / one replay: both below the GPU
            # time per call, so the launch loop never starves the GPU
            "eager_host_us_per_call": round(eager_host_us, 1), "graph_host_us_per_replay": round(graph_host_us, 1),
            "tokens_per_s_graph": sw.B * sw.N / (graph_ms / 1e3)}
        del graph, graph10, sm, sout, sws

        # The two other FLARE++ mixer workloads at full size: the sequence
        # workload (B=32, N=4096, C=256, M=128, no W_O) and the block workload
        # (B=4, N=262144, C=256, M=512, with W_O).
        for key, label in (("seq_bf16_b32_n4k", "FLARE++ sequence mixer"), ("block_bf16_n256k", "FLARE++ block")):
            ww = inputs.WORKLOADS[key]
            wm = {n: t.to(dev) for n, t in inputs.make_mix(ww, seed=0).items()}
            wout = torch.empty_like(wm["x"])
            wws = torch.empty(rl.mix_workspace_size(ww.B, ww.N, ww.C, ww.H, ww.M, True, ww.has_wo),
                              dtype=torch.uint8, device=dev)

            def run_w(flags=0):
                rl.flare_mix(wm["x"], wm["w_k"], wm["w_v"], wm["qs"], ww.H, w_ek=wm["w_ek"], w_ev=wm["w_ev"],
                             w_o=wm.get("w_o"), out=wout, workspace=wws, flags=flags, stream=stream)

            def time_w(flags=0):
                for _ in range(3):
                    run_w(flags)
                torch.cuda.synchronize()
                e0.record(stream)
                for _ in range(10):
                    run_w(flags)
                e1.record(stream)
                torch.cuda.synchronize()
                return e0.elapsed_time(e1) / 10
            wms = time_w()
            wk = costs.mixer(ww.B, ww.N, ww.C, ww.H, ww.M, dynamic=True, has_wo=ww.has_wo)
            extra[key] = {"config": f"{label}, B={ww.B}, N={ww.N}, C={ww.C}, H={ww.H}, D={ww.D}, M={ww.M}, bf16"
                                    + (", with W_O" if ww.has_wo else ""),
                          "ms": round(wms, 4), "tokens_per_s": ww.B * ww.N / (wms / 1e3),
                          "tflops": round(wk.flops / (wms / 1e3) / 1e12, 1)}
            if ww.has_wo:
                # the output projection in the decoder's epilogue instead of a
                # second pass over Y (FLARE_MIX_FUSED_WO; the faster form is
                # the default)
                fms = time_w(rl.FLARE_MIX_FUSED_WO)
                extra[key]["fused_wo_ms"] = round(fms, 4)
                extra[key]["fused_over_two_pass"] = round(fms / wms, 3)
            del wm, wout, wws

    if not args.no_sweep:
        # Time and memory against the token count, three orders of magnitude
        # and more (H=8, D=32, M=256, bf16, B=1): FLARE encode+decode, and the
        # whole FLARE++ mixer with all projections at C=256.  Memory is the peak
        # of device memory allocated for the call's inputs, outputs and
        # workspace.
        sweep = []
        for n_tok in (1 << 10, 1 << 12, 1 << 14, 1 << 16, 1 << 18, 1 << 20, 1 << 22):
            torch.cuda.empty_cache()
            torch.cuda.reset_peak_memory_stats()
            base_mem = torch.cuda.memory_allocated()
            sw_ = inputs.Workload("sweep", "encdec", 1, n_tok, H, D, M, "bf16")
            sx = inputs.make_encdec(sw_, seed=1)
            sq = sx["q"].to(dev)
            sk = sx["k"].to(dev).permute(0, 2, 1, 3).contiguous()
            sv = sx["v"].to(dev).permute(0, 2, 1, 3).contiguous()
            del sx
            sz = torch.empty((1, H, M, D), dtype=torch.bfloat16, device=dev)
            syt = torch.empty((1, n_tok, H, D), dtype=torch.bfloat16, device=dev)
            sy = syt.permute(0, 2, 1, 3)
            sws = torch.empty(rl.encode_workspace_size(1, H, M, n_tok, D), dtype=torch.uint8, device=dev)

            def encdec():
                rl.flare_encode(sq, sk, sv, z=sz, workspace=sws, stream=stream)
                rl.flare_decode(sk, sq, sz, y=sy, stream=stream)
            reps = max(5, min(200, (1 << 24) // n_tok))
            for _ in range(3):
                encdec()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                encdec()
            e1.record(stream)
            torch.cuda.synchronize()
            ems = e0.elapsed_time(e1) / reps
            emem = (torch.cuda.max_memory_allocated() - base_mem) / 1e9
            # the pair backward at the same size (one call, fp32 gradients);
            # its memory is the peak of the forward and backward buffers
            szf, sle = rl.flare_encode(sq, sk, sv, want_lse=True, z_dtype=torch.float32, workspace=sws,
                                       stream=stream)
            syb, sld = rl.flare_decode(sk, sq, szf, want_lse=True, stream=stream)
            sdy = torch.randn(syb.shape, generator=torch.Generator(device=dev).manual_seed(1), device=dev,
                              dtype=torch.float32).to(torch.bfloat16)
            sdq = torch.empty((1, H, M, D), dtype=torch.float32, device=dev)
            sdk = torch.empty((1, H, n_tok, D), dtype=torch.float32, device=dev)
            sdv = torch.empty_like(sdk)
            swb = torch.empty(rl.lib().flare_encdec_backward_workspace_size(1, H, M, n_tok, D), dtype=torch.uint8,
                              device=dev)

            def pair_bwd():
                rl.flare_encdec_backward(sq, sk, sv, szf, sle, syb, sld, sdy, dq=sdq, dk=sdk, dv=sdv,
                                         workspace=swb, stream=stream)
            breps = max(3, reps // 3)
            for _ in range(2):
                pair_bwd()
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(breps):
                pair_bwd()
            e1.record(stream)
            torch.cuda.synchronize()
            bms_ = e0.elapsed_time(e1) / breps
            bmem = (torch.cuda.max_memory_allocated() - base_mem) / 1e9
            del sq, sk, sv, sz, syt, sy, sws, szf, sle, syb, sld, sdy, sdq, sdk, sdv, swb
            torch.cuda.empty_cache()
            torch.cuda.reset_peak_memory_stats()
            base_mem = torch.cuda.memory_allocated()
            mw_ = inputs.Workload("sweep_mix", "mix", 1, n_tok, H, D, M, "bf16", dynamic=True, has_wo=True)
            mm = {nm: t.to(dev) for nm, t in inputs.make_mix(mw_, seed=1).items()}
            mout = torch.empty_like(mm["x"])
            mws2 = torch.empty(rl.mix_workspace_size(1, n_tok, mw_.C, H, M, True, True), dtype=torch.uint8,
                               device=dev)

            def mixer():
                rl.flare_mix(mm["x"], mm["w_k"], mm["w_v"], mm["qs"], H, w_ek=mm["w_ek"], w_ev=mm["w_ev"],
                             w_o=mm["w_o"], out=mout, workspace=mws2, stream=stream)
            for _ in range(3):
                mixer()
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(reps):
                mixer()
            e1.record(stream)
            torch.cuda.synchronize()
            mms_ = e0.elapsed_time(e1) / reps
            mmem = (torch.cuda.max_memory_allocated() - base_mem) / 1e9
            del mm, mout, mws2
            sweep.append({"N": n_tok, "encdec_ms": round(ems, 4), "encdec_tokens_per_s": n_tok / (ems / 1e3),
                          "encdec_mem_GB": round(emem, 4), "backward_ms": round(bms_, 4),
                          "backward_tokens_per_s": n_tok / (bms_ / 1e3), "fwd_bwd_mem_GB": round(bmem, 4),
                          "flarepp_mixer_ms": round(mms_, 4),
                          "flarepp_mixer_tokens_per_s": n_tok / (mms_ / 1e3), "flarepp_mixer_mem_GB": round(mmem, 4)})
        extra["n_sweep"] = {"config": "B=1, H=8, D=32, M=256, bf16; FLARE encode+decode, its one-call backward "
                                      "(fp32 dK, dV), and the FLARE++ mixer with all projections at C=256; "
                                      "memory = peak device memory of inputs, outputs, gradients and workspace",
                            "points": sweep}

    cpu = None
    if not args.no_cpu:
        import oracle
        nh = max(1, min(H, args.cpu_heads))
        q64 = x["q"].double().numpy()
        k64 = x["k"].double().numpy().reshape(B, N, H * D)
        v64 = x["v"].double().numpy().reshape(B, N, H * D)
        c0 = time.perf_counter()
        oracle.flare_encdec(q64, k64, v64, H, heads=(0, nh))
        csec = time.perf_counter() - c0
        cpu = {"value": tokens / (csec * H / nh), "unit": "tokens/s", "cores": oracle.max_threads(),
               "kind": "oracle",
               "sample": f"fp64 oracle encode+decode of heads 0..{nh - 1} of {H} over all {N} tokens "
                         f"({csec:.1f} s); rate scaled by {H}/{nh} to the whole workload"}

    rec = {"metric": "mixer fwd tokens/s at N=1M,H=8,M=256,D=32 bf16; % MFMA peak",
           "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "FLARE encode+decode, B=1, H=8, D=32, N=1048576, M=256, bf16 "
                                  "(K, V head-major [B,H,N,D]; Y " + args.y_layout + "-major)",
                      "global_batch": B, "seq_len": N, "parallelism": "single-gpu"},
           "roofline": roofline, "cpu_baseline": cpu, "extra": extra}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()

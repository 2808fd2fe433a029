"""Issue-rate probes of the gfx950 instructions the mixer's inner loops use.

Builds ``issue.hip`` (with ``clock.hip``, the shader-clock sampler bench.py
uses, and ``xreuse.hip``, the X-reuse probe of run_xreuse.py) into
``_build/libflare_probes.so`` (also built by
``__graft_entry__.build()``) and runs each instruction mix on one workgroup
per compute unit with 1, 2 or 4 waves per SIMD.  Prints a markdown table of
SIMD cycles per loop iteration (median over waves, from the shader clock each
wave reads around its loop) and the shader clock rate (shader-clock ticks over
the 100 MHz real-time counter).

    python -m rank_latent_routing_amd.probes.run_probes [--iters N]
"""
import argparse
import ctypes
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
LIB = os.path.join(PKG, "_build", "libflare_probes.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

MIX = {"mfma": 0, "mul": 1, "exp": 2, "cvt": 3, "dot2": 4, "mul+exp": 5, "mfma+4mul": 6,
       "mfma+8mul": 7, "mfma+16mul": 8, "mfma+4exp": 9, "mfma+8exp": 10, "mfma+16exp": 11,
       "block": 12, "block-nomul": 13, "block-nodot": 14, "block-dep": 15, "idle": 16,
       "agpr+8mul": 17, "agpr+16exp": 18, "mfma16": 19, "mfma16+8mul": 20, "mfma16+16exp": 21,
       "block-agpr": 22, "block-hilo": 23, "block-hilo-agpr": 24, "block-nomul-agpr": 25, "agpr": 26}
# instructions per loop iteration: (mfma, mul, exp, cvt, dot2)
COUNTS = {"mfma": (8, 0, 0, 0, 0), "mul": (0, 32, 0, 0, 0), "exp": (0, 0, 32, 0, 0),
          "cvt": (0, 0, 0, 16, 0), "dot2": (0, 0, 0, 0, 16), "mul+exp": (0, 16, 16, 0, 0),
          "mfma+4mul": (8, 32, 0, 0, 0), "mfma+8mul": (8, 64, 0, 0, 0),
          "mfma+16mul": (8, 128, 0, 0, 0), "mfma+4exp": (8, 0, 32, 0, 0),
          "mfma+8exp": (8, 0, 64, 0, 0), "mfma+16exp": (8, 0, 128, 0, 0),
          "block": (4, 16, 16, 8, 8), "block-nomul": (4, 0, 16, 8, 8),
          "block-nodot": (4, 16, 16, 8, 0), "block-dep": (4, 16, 16, 8, 8), "idle": (0, 0, 0, 0, 0),
          "agpr": (8, 0, 0, 0, 0), "agpr+8mul": (8, 64, 0, 0, 0), "agpr+16exp": (8, 0, 128, 0, 0),
          # 16x16x32 products counted as half a 32x32x16 product (same flops per pair)
          "mfma16": (8, 0, 0, 0, 0), "mfma16+8mul": (8, 64, 0, 0, 0), "mfma16+16exp": (8, 0, 128, 0, 0),
          "block-agpr": (4, 16, 16, 8, 8), "block-hilo": (6, 0, 16, 8, 8),
          "block-hilo-agpr": (6, 0, 16, 8, 8), "block-nomul-agpr": (4, 0, 16, 8, 8)}


# mixes with AGPR weighted sums run at most two waves per SIMD
AGPR_BLOCKS = ("block-agpr", "block-hilo-agpr", "block-nomul-agpr")


def build(verbose=False):
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-x", "hip", os.path.join(HERE, "issue.hip"), os.path.join(HERE, "clock.hip"),
           os.path.join(HERE, "xreuse.hip"), "-o", LIB + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("building the probes failed:\n" + r.stderr)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--iters", type=int, default=20000)
    ap.add_argument("--mixes", default="", help="comma-separated mixes to run (default: all)")
    ap.add_argument("--wps", default="1,2,4", help="comma-separated waves per SIMD")
    ap.add_argument("--no-split", action="store_true", help="skip the split-role table")
    args = ap.parse_args()
    wps_list = [int(w) for w in args.wps.split(",")]
    import torch
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} missing: run __graft_entry__.build()")
    L = ctypes.CDLL(LIB)
    L.probe_run.argtypes = [ctypes.c_int] * 6 + [ctypes.c_void_p] * 3
    L.probe_run.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    blocks = torch.cuda.get_device_properties(0).multi_processor_count

    def run(mix0, mix1, wps, role_shift):
        """Median over compute units of the span from the first wave's start
        to the last wave's end, in shader cycles per loop iteration; the
        same for each role's waves alone; and the shader clock rate."""
        threads = 256 * wps
        nw = threads // 64
        out = torch.empty(blocks * threads, dtype=torch.float32, device=dev)
        cyc = torch.zeros(4 * blocks * nw, dtype=torch.int64, device=dev)
        for iters in (max(args.iters // 20, 1), args.iters):  # warm-up, then measured
            rc = L.probe_run(MIX[mix0], MIX[mix1], blocks, threads, iters, role_shift,
                             out.data_ptr(), cyc.data_ptr(), stream)
            if rc != 0:
                raise RuntimeError(f"probe {mix0}/{mix1}: hipError {rc}")
            torch.cuda.synchronize()
        c = cyc.view(blocks, nw, 4).cpu().double()
        waves = torch.arange(nw)
        second = ((waves >> role_shift) & 1) == 1 if role_shift >= 0 else torch.zeros(nw, dtype=torch.bool)

        def span(sel):
            if not bool(sel.any()):
                return None
            t0 = c[:, sel, 0].min(dim=1).values
            t1 = c[:, sel, 1].max(dim=1).values
            return float((t1 - t0).median()) / args.iters

        dt, dr = (c[..., 1] - c[..., 0]).flatten(), (c[..., 3] - c[..., 2]).flatten()
        busy = dr > 1000  # waves that ran a loop (idle roles do not)
        ghz = float((dt[busy] / dr[busy]).median()) * 0.1
        return span(torch.ones(nw, dtype=torch.bool)), span(~second), span(second), ghz

    print(f"device: {torch.cuda.get_device_name(0)}, {blocks} compute units, {args.iters} iterations")
    print()
    print("Cycles are shader-clock cycles per loop iteration of the whole compute unit: from the first")
    print("wave's start to the last wave's end (median over compute units), divided by the iterations.")
    print("Per-instruction figures divide that by the instructions every SIMD issues per iteration")
    print("(waves per SIMD x the mix's count).")
    print()
    print("| mix | waves/SIMD | CU cycles/iter | MFMA | mul | exp | cvt | dot2 | SIMD cycles per MFMA | "
          "SIMD cycles per VALU instr. | shader clock (GHz) |")
    print("|---|---|---|---|---|---|---|---|---|---|---|")
    names = ["mfma", "mul", "exp", "cvt", "dot2", "mul+exp", "mfma+4mul", "mfma+8mul", "mfma+16mul",
             "mfma+4exp", "mfma+8exp", "mfma+16exp", "agpr", "agpr+8mul", "agpr+16exp", "mfma16",
             "mfma16+8mul", "mfma16+16exp", "block", "block-dep", "block-nomul", "block-nodot",
             "block-agpr", "block-nomul-agpr", "block-hilo", "block-hilo-agpr"]
    if args.mixes:
        names = [n for n in args.mixes.split(",")]
    for name in names:
        for wps in [w for w in wps_list if not (name in AGPR_BLOCKS and w > 2)]:
            per, _, _, ghz = run(name, name, wps, -1)
            n = COUNTS[name]
            nv = sum(n[1:])
            per_mfma = f"{per / (wps * n[0]):.2f}" if n[0] else "-"
            per_valu = f"{per / (wps * nv):.2f}" if nv else "-"
            print(f"| {name} | {wps} | {per:.1f} | {n[0]} | {n[1]} | {n[2]} | {n[3]} | {n[4]} | "
                  f"{per_mfma} | {per_valu} | {ghz:.2f} |")
    if args.no_split:
        return
    print()
    print("Split roles, two waves per SIMD: wave w runs the second mix when bit `shift` of w is set")
    print("(which shift pairs the two roles on one SIMD depends on how waves map to SIMDs).  Spans as")
    print("above, for all waves and for each role's waves alone.")
    print()
    print("| first mix | second mix | shift | CU cycles/iter, all | first role | second role | "
          "shader clock (GHz) |")
    print("|---|---|---|---|---|---|---|")
    for a, b in [("mfma", "idle"), ("exp", "idle"), ("mul", "idle"), ("mfma", "exp"), ("mfma", "mul"),
                 ("exp", "mul")]:
        for shift in (0, 2):
            per, p0, p1, ghz = run(a, b, 2, shift)
            f = lambda v: f"{v:.1f}" if v is not None else "-"
            print(f"| {a} | {b} | {shift} | {f(per)} | {f(p0)} | {f(p1)} | {ghz:.2f} |")
    sys.stdout.flush()


if __name__ == "__main__":
    main()

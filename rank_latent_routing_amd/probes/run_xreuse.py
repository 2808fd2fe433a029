"""X reuse across heads (see xreuse.hip): times the probe kernel in its three
dispatch orders over the FLARE++ block workload's projection input (X [B*N, C]
bf16 with B=4, N=262144, C=256, H=8: 537 MB) and prints a markdown table.

    python -m rank_latent_routing_amd.probes.run_xreuse [--reps N]

Each order reads X once per head (8 x 537 MB of loads); a read of X once (one
head) is timed beside them.  Under ``rocprofv3 --pmc FETCH_SIZE`` the same run
gives the bytes each order fetches past L2 (``bench.py --summarize xreuse``).
"""
import argparse
import ctypes
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from rank_latent_routing_amd.probes.run_probes import LIB  # noqa: E402

B, N, C, H = 4, 262144, 256, 8
ROWS_PER_BLOCK = 128
WARMUP = 2
# (label, heads, order), in the order the runs happen (the counter summary
# relies on it)
RUNS = [("X read once (1 head)", 1, 0), ("head-major", H, 0), ("head-interleaved", H, 1),
        ("head-interleaved per XCD", H, 2)]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--reps", type=int, default=10)
    args = ap.parse_args()
    import torch
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} missing: run __graft_entry__.build()")
    L = ctypes.CDLL(LIB)
    L.xreuse_run.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                             ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.xreuse_run.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    R = B * N
    x = torch.randn((R, C), generator=torch.Generator(device=dev).manual_seed(0), device=dev).to(torch.bfloat16)
    nrb = (R + ROWS_PER_BLOCK - 1) // ROWS_PER_BLOCK
    out = torch.empty(nrb * H * 4, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    xbytes = R * C * 2
    print(f"X [{R}, {C}] bf16, {xbytes / 1e6:.0f} MB; {ROWS_PER_BLOCK}-row blocks ({nrb}), {args.reps} timed "
          f"launches per order after {WARMUP} warm-up\n")
    print("| order | heads | us per launch | X loads per launch (GB) | load rate (TB/s) |")
    print("|---|---|---|---|---|")
    for label, heads, order in RUNS:
        def run():
            rc = L.xreuse_run(x.data_ptr(), R, C, heads, order, ROWS_PER_BLOCK, out.data_ptr(), stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"xreuse_run failed ({rc})")
        for _ in range(WARMUP):
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.reps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / args.reps * 1e3
        loads = heads * xbytes
        print(f"| {label} | {heads} | {us:.1f} | {loads / 1e9:.3f} | {loads / (us * 1e-6) / 1e12:.2f} |", flush=True)


if __name__ == "__main__":
    main()

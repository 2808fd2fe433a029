"""GPU tier: the measurement probes the bench and the profiles rely on.

The shader-clock sampler must report a clock in the chip's range on every
XCD, and the X-reuse probe must visit every (row block, head) pair exactly
once in each of its three dispatch orders (its per-wave sums, weighted by
head + 1, must add up to (1 + ... + H) times the sum of X).
"""
import ctypes
import os

import pytest
import torch

from rank_latent_routing_amd.probes import run_probes

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _lib():
    if not os.path.exists(run_probes.LIB):
        pytest.fail(f"{run_probes.LIB} missing: run __graft_entry__.build()")
    L = ctypes.CDLL(run_probes.LIB)
    L.clock_sample.argtypes = [ctypes.c_void_p, ctypes.c_ulonglong, ctypes.c_void_p]
    L.clock_sample.restype = ctypes.c_int
    L.xreuse_run.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                             ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.xreuse_run.restype = ctypes.c_int
    return L


def test_clock_sampler_reads_a_plausible_clock_on_every_xcd():
    L = _lib()
    out = torch.zeros(32, dtype=torch.int64, device=DEV)
    stream = torch.cuda.current_stream()
    assert L.clock_sample(out.data_ptr(), 20000, stream.cuda_stream) == 0  # 0.2 ms
    torch.cuda.synchronize()
    v = out.tolist()
    for i in range(8):
        r0, r1, c0, c1 = v[4 * i:4 * i + 4]
        assert r1 - r0 >= 20000
        ghz = (c1 - c0) / ((r1 - r0) / 1e8) / 1e9
        print(f"  XCD {i}: {ghz:.3f} GHz", flush=True)
        assert 0.3 < ghz < 3.5
    # out-of-range requests are refused before any launch
    assert L.clock_sample(out.data_ptr(), 0, stream.cuda_stream) != 0
    assert L.clock_sample(out.data_ptr(), 10 ** 8, stream.cuda_stream) != 0


@pytest.mark.parametrize("C,H,rows", [(256, 8, 128), (128, 3, 64)])
def test_xreuse_orders_visit_every_block_and_head_once(C, H, rows):
    L = _lib()
    nrb = 64  # order 2 needs a multiple of 8 row blocks
    R = nrb * rows
    g = torch.Generator(device=DEV).manual_seed(3)
    x = torch.randn((R, C), generator=g, device=DEV).to(torch.bfloat16)
    weight = H * (H + 1) / 2
    want = float(x.double().sum()) * weight
    tol = 1e-5 * float(x.double().abs().sum()) * weight + 1e-3
    out = torch.empty(nrb * H * 4, dtype=torch.float32, device=DEV)
    stream = torch.cuda.current_stream()
    for order in (0, 1, 2):
        out.fill_(float("nan"))
        assert L.xreuse_run(x.data_ptr(), R, C, H, order, rows, out.data_ptr(), stream.cuda_stream) == 0
        torch.cuda.synchronize()
        got = float(out.double().sum())
        assert abs(got - want) <= tol, (order, got, want)
    # order 2 with a row-block count that is not a multiple of 8 is refused
    assert L.xreuse_run(x.data_ptr(), R - rows, C, H, 2, rows, out.data_ptr(), stream.cuda_stream) != 0

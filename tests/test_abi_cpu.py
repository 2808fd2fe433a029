"""CPU tier: the C-ABI library loads, exports what include/flare.h declares,
and rejects bad arguments before touching any device (no compute calls)."""
import ctypes
import os
import re

import pytest

from rank_latent_routing_amd import binding as fb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flare.h")

needs_lib = pytest.mark.skipif(not os.path.exists(fb.LIB_PATH), reason="HIP library not built")

# A fake but well-aligned device address: validation never dereferences it,
# and every call below fails validation before any launch.
FAKE = 0x7F0000000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flare_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for f in ("flare_route_queries", "flare_encode", "flare_decode", "flare_mix"):
        assert f in names
    assert set(names) == set(fb.EXPORTS)


@needs_lib
def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(fb.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name


@needs_lib
def test_status_strings_and_version():
    assert fb.status_string(0) == "ok"
    assert "workspace" in fb.status_string(fb.FLARE_E_WORKSPACE)
    assert fb.status_string(12345) == "unknown status"
    assert re.fullmatch(r"\d+\.\d+\.\d+", fb.version())


def T(dtype=fb.FLARE_BF16, sb=0, sh=8, sl=8, data=FAKE):
    return fb.FlareTensor(data, dtype, 0, sb, sh, sl)


def call_encode(Q=None, K=None, V=None, Z=None, B=1, H=2, M=32, N=100, D=32, scale=0.0,
                flags=0, ws=FAKE, ws_bytes=1 << 40, lse=None):
    L = fb.lib()
    r = lambda t: ctypes.byref(t) if t is not None else None
    Q = T() if Q is None else Q
    K = T(sb=N * 8 * H) if K is None else K
    V = T(sb=N * 8 * H) if V is None else V
    Z = T() if Z is None else Z
    return L.flare_encode(r(Q), r(K), r(V), r(Z), lse, B, H, M, N, D, scale, flags,
                          ctypes.c_void_p(ws), ws_bytes, None)


@needs_lib
def test_encode_rejects_bad_arguments_without_a_device():
    E = fb
    assert call_encode(K=fb.FlareTensor(0, 1, 0, 0, 8, 8)) == E.FLARE_E_INVALID  # null data
    assert call_encode(B=0) == E.FLARE_E_INVALID
    assert call_encode(N=0) == E.FLARE_E_INVALID
    assert call_encode(M=0) == E.FLARE_E_INVALID
    assert call_encode(B=300, H=300) == E.FLARE_E_INVALID                  # B*H above the grid's y limit
    assert call_encode(D=24) == E.FLARE_E_UNSUPPORTED
    assert call_encode(D=64) == E.FLARE_E_UNSUPPORTED
    assert call_encode(M=513) == E.FLARE_E_UNSUPPORTED
    assert call_encode(K=T(data=FAKE + 2)) == E.FLARE_E_INVALID       # misaligned rows
    assert call_encode(V=T(sl=12)) == E.FLARE_E_INVALID                # stride not a multiple of 8
    assert call_encode(V=T(dtype=fb.FLARE_F32)) == E.FLARE_E_INVALID   # K, V dtypes differ
    assert call_encode(Q=T(dtype=7)) == E.FLARE_E_INVALID               # unknown dtype
    assert call_encode(scale=float("nan")) == E.FLARE_E_INVALID
    assert call_encode(flags=0x80) == E.FLARE_E_INVALID
    assert call_encode(ws=0) == E.FLARE_E_WORKSPACE
    assert call_encode(ws_bytes=16) == E.FLARE_E_WORKSPACE


@needs_lib
def test_decode_and_route_reject_bad_arguments():
    L = fb.lib()
    r = ctypes.byref
    ok = T()
    assert L.flare_decode(None, r(ok), r(ok), r(ok), None, 1, 1, 8, 10, 32, 0.0, 0, None) == fb.FLARE_E_INVALID
    assert L.flare_decode(r(ok), r(ok), r(ok), r(ok), None, 1, 1, 8, 10, 8, 0.0, 0, None) == fb.FLARE_E_UNSUPPORTED
    assert L.flare_decode(r(ok), r(ok), r(ok), r(T(data=FAKE + 8)), None, 1, 1, 8, 10, 32, 0.0, 0,
                          None) == fb.FLARE_E_INVALID
    assert L.flare_decode(r(ok), r(ok), r(ok), r(ok), ctypes.c_void_p(FAKE + 2), 1, 1, 8, 10, 32, 0.0,
                          0, None) == fb.FLARE_E_INVALID
    assert L.flare_route_queries(r(ok), r(ok), r(ok), r(ok), None, 1, 1, 8, 10, 32, 0.0, 0, None, 0,
                                 None) == fb.FLARE_E_WORKSPACE


@needs_lib
def test_mix_and_project_reject_bad_arguments():
    L = fb.lib()
    p = ctypes.c_void_p(FAKE)
    n = None
    # C not divisible by H
    assert L.flare_mix(p, p, p, n, n, p, n, p, 1, 1, 10, 100, 3, 8, 0.0, 0, p, 1 << 40, n) == fb.FLARE_E_INVALID
    # fp32 mixer not built
    assert L.flare_mix(p, p, p, n, n, p, n, p, 0, 1, 10, 64, 2, 8, 0.0, 0, p, 1 << 40, n) == fb.FLARE_E_UNSUPPORTED
    # only one of the two synthesis weights
    assert L.flare_mix(p, p, p, p, n, p, n, p, 1, 1, 10, 64, 2, 8, 0.0, 0, p, 1 << 40, n) == fb.FLARE_E_INVALID
    # workspace too small
    assert L.flare_mix(p, p, p, p, p, p, n, p, 1, 1, 10, 64, 2, 8, 0.0, 0, p, 64, n) == fb.FLARE_E_WORKSPACE
    warr = (ctypes.c_void_p * 1)(FAKE)
    assert L.flare_project(p, warr, warr, 1, 10, 48, 64, 0, 1, 0, p, 1 << 30, n) == fb.FLARE_E_UNSUPPORTED
    assert L.flare_project(p, warr, warr, 1, 10, 64, 64, 1, 3, 32, p, 1 << 30, n) == fb.FLARE_E_INVALID
    assert L.flare_project(p, warr, warr, 1, 10, 64, 64, 0, 1, 0, p, 16, n) == fb.FLARE_E_WORKSPACE


@needs_lib
def test_workspace_sizes():
    small = fb.encode_workspace_size(1, 8, 256, 4096, 32)
    big = fb.encode_workspace_size(1, 8, 256, 1 << 20, 32)
    assert 0 < small <= big
    assert fb.encode_workspace_size(1, 8, 256, 1 << 20, 24) == 0
    assert fb.project_workspace_size(256, 256, 4) == 4 * 256 * 256 * 2
    m1 = fb.mix_workspace_size(4, 1 << 18, 256, 8, 512, True, True)
    m0 = fb.mix_workspace_size(4, 1 << 18, 256, 8, 512, False, False)
    assert m1 > m0 > 4 * (1 << 18) * 256 * 2 * 2
    assert fb.mix_workspace_size(1, 10, 100, 3, 8, True, False) == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(fb, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(fb, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        fb.lib()


@needs_lib
def test_backward_calls_reject_bad_arguments():
    L = fb.lib()
    r = ctypes.byref
    ok, f32 = T(), T(dtype=fb.FLARE_F32, sh=4, sl=4)
    p = ctypes.c_void_p(FAKE)
    ws = ctypes.c_void_p(FAKE)
    need = L.flare_decode_backward_workspace_size(1, 1, 8, 10, 32)
    assert need > 0 and L.flare_encode_backward_workspace_size(1, 1, 8, 10, 32) > 0
    # token-side inputs must be bf16; token-side gradients fp32 or bf16 (one
    # dtype for dK and dV), nothing else
    assert L.flare_decode_backward(r(f32), r(ok), r(ok), r(ok), p, r(ok), r(f32), p, p, 0, 1, 1, 8, 10, 32,
                                   0.0, ws, need, None) == fb.FLARE_E_UNSUPPORTED
    bad_dtype = T(dtype=5)
    assert L.flare_decode_backward(r(ok), r(ok), r(ok), r(ok), p, r(ok), r(bad_dtype), p, p, 0, 1, 1, 8, 10,
                                   32, 0.0, ws, need, None) == fb.FLARE_E_INVALID
    # the normaliser is required; sizes; workspace
    assert L.flare_decode_backward(r(ok), r(ok), r(ok), r(ok), None, r(ok), r(f32), p, p, 0, 1, 1, 8, 10, 32,
                                   0.0, ws, need, None) == fb.FLARE_E_INVALID
    assert L.flare_decode_backward(r(ok), r(ok), r(ok), r(ok), p, r(ok), r(f32), p, p, 0, 1, 1, 8, 10, 8,
                                   0.0, ws, need, None) == fb.FLARE_E_UNSUPPORTED
    assert L.flare_decode_backward(r(ok), r(ok), r(ok), r(ok), p, r(ok), r(f32), p, p, 0, 1, 1, 8, 10, 32,
                                   0.0, ws, need - 1, None) == fb.FLARE_E_WORKSPACE
    # unknown flag bits
    assert L.flare_decode_backward(r(ok), r(ok), r(ok), r(ok), p, r(ok), r(f32), p, p, 8, 1, 1, 8, 10, 32,
                                   0.0, ws, need, None) == fb.FLARE_E_INVALID
    need = L.flare_encode_backward_workspace_size(1, 1, 8, 10, 32)
    assert L.flare_encode_backward(r(ok), r(ok), r(ok), r(ok), p, p, p, r(f32), r(f32), 8, 1, 1, 8, 10, 32,
                                   0.0, ws, need, None) == fb.FLARE_E_INVALID
    # dK bf16 with dV fp32: the two gradients must share one dtype
    assert L.flare_encode_backward(r(ok), r(ok), r(ok), r(ok), p, p, p, r(ok), r(f32), 0, 1, 1, 8, 10, 32,
                                   0.0, ws, need, None) == fb.FLARE_E_UNSUPPORTED
    assert L.flare_encode_backward(r(ok), r(ok), r(ok), r(ok), p, p, p, r(f32), r(f32), 0, 1, 1, 8, 10, 32,
                                   float("nan"), ws, need, None) == fb.FLARE_E_INVALID
    # the fused pair: same rules
    need = L.flare_encdec_backward_workspace_size(1, 1, 8, 10, 32)
    assert need >= L.flare_decode_backward_workspace_size(1, 1, 8, 10, 32)
    pair = lambda **kw: L.flare_encdec_backward(
        r(ok), r(kw.get("k", ok)), r(ok), r(ok), kw.get("lse", p), r(ok), p, r(ok), p, r(kw.get("dk", f32)),
        r(f32), kw.get("flags", 0), 1, 1, 8, 10, kw.get("D", 32), 0.0, ws, kw.get("ws", need), None)
    assert pair(k=f32) == fb.FLARE_E_UNSUPPORTED
    assert pair(dk=ok) == fb.FLARE_E_UNSUPPORTED
    assert pair(lse=None) == fb.FLARE_E_INVALID
    assert pair(flags=8) == fb.FLARE_E_INVALID
    assert pair(D=8) == fb.FLARE_E_UNSUPPORTED
    assert pair(ws=need - 1) == fb.FLARE_E_WORKSPACE


def test_binding_rejects_strided_or_misshaped_arrays():
    # lse, dQ and dZ cross the C ABI as plain arrays: the binding must refuse
    # a view whose memory is not that array, or host memory, instead of
    # passing its pointer
    import torch
    good = torch.zeros(2, 3, 4, 32)
    with pytest.raises(ValueError, match="on the GPU"):  # right layout, but host memory
        fb._f32_ptr(good, (2, 3, 4, 32), "dz")
    with pytest.raises(ValueError, match="strided"):
        fb._f32_ptr(torch.zeros(2, 3, 4, 40)[..., :32], (2, 3, 4, 32), "dz")
    with pytest.raises(ValueError, match="shape"):
        fb._f32_ptr(good, (3, 4, 32), "dq")
    with pytest.raises(ValueError, match="float32"):
        fb._f32_ptr(good.double(), (2, 3, 4, 32), "dz")


def test_binding_refuses_host_tensors():
    # every tensor the kernels touch must be in GPU memory: a host tensor is
    # refused before the call (never handed to a kernel)
    import torch
    k = torch.zeros(1, 2, 16, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="on the GPU"):
        fb.describe(k)
    with pytest.raises(ValueError, match="on the GPU"):
        fb._dev(torch.zeros(4), "workspace")


def test_binding_checks_extents_before_any_call():
    # extents that disagree with the sizes the binding passes are refused
    # before the library is called (shape checks come before the device check)
    import torch
    bf = torch.bfloat16
    k = torch.zeros(2, 3, 64, 32, dtype=bf)
    with pytest.raises(ValueError, match="q must be"):
        fb.flare_encode(torch.zeros(3, 8, 16, dtype=bf), k, k)           # D of q differs
    with pytest.raises(ValueError, match="q must be"):
        fb.flare_encode(torch.zeros(1, 3, 8, 32, dtype=bf), k, k)        # [1, H, M, D] with B = 2
    with pytest.raises(ValueError, match="v must be"):
        fb.flare_encode(torch.zeros(3, 8, 32, dtype=bf), k, k[:, :, :32])
    with pytest.raises(ValueError, match="y must be"):
        fb.flare_decode(k, torch.zeros(3, 8, 32, dtype=bf), torch.zeros(2, 3, 8, 32),
                        y=torch.zeros(2, 3, 63, 32, dtype=bf))
    with pytest.raises(ValueError, match="weight 1"):
        fb.flare_project(torch.zeros(2, 10, 64, dtype=bf), [torch.zeros(64, 64, dtype=bf),
                                                             torch.zeros(64, 32, dtype=bf)])
    with pytest.raises(ValueError, match="qs must be"):
        fb.flare_mix(torch.zeros(1, 10, 64, dtype=bf), torch.zeros(64, 64, dtype=bf),
                     torch.zeros(64, 64, dtype=bf), torch.zeros(2, 8, 16, dtype=bf), 2)

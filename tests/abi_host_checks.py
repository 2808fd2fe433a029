"""Host-side checks of the C ABI of include/flare.h: argument checks, planning,
workspace carving and the mapping of launch errors to FLARE_E_HIP.

They drive the host-only build of the library (``libflare_host.so``: the same
host code as the gfx950 library, with stand-ins for the kernel launchers that
record what they would launch and return a status the check chooses).
Pointers are fake addresses that nothing dereferences, so no device is
needed and none is touched.

tests/test_abi_cpu.py runs every ``check_*`` function here.  Run as a script,
``python tests/abi_host_checks.py LIB`` runs them all against LIB and prints
one line per check; the CPU suite runs it that way on the build with
AddressSanitizer and UndefinedBehaviorSanitizer, in a process that preloads
the sanitizer runtime.  This module imports no torch (and not the package,
whose binding does): it loads the ctypes declarations from their file.
"""
import ctypes
import importlib.util
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _load_cabi():
    path = os.path.join(ROOT, "rank_latent_routing_amd", "cabi.py")
    spec = importlib.util.spec_from_file_location("flare_cabi", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


cabi = _load_cabi()
OK, E_INVALID, E_UNSUPPORTED = cabi.FLARE_OK, cabi.FLARE_E_INVALID, cabi.FLARE_E_UNSUPPORTED
E_WORKSPACE, E_HIP = cabi.FLARE_E_WORKSPACE, cabi.FLARE_E_HIP
BF16, F32 = cabi.FLARE_BF16, cabi.FLARE_F32

FAKE = 0x7F0000000000   # fake tensor base (256-byte aligned)
WS = 0x100000000000     # fake workspace base, far from the tensors
OUT = FAKE + (1 << 36)  # the mixer's output
(ENC_PART_O, ENC_PART_L, BWD_DQ, BWD_DZ, SUM_PART, SWIZZLED, GEMM_OUT, ENC_K, ENC_V, WO_LAT, WO_T,
 DEC_ZPART) = range(1, 13)
WRITTEN = (ENC_PART_O, ENC_PART_L, BWD_DQ, BWD_DZ, SWIZZLED, GEMM_OUT, WO_LAT, WO_T)
HIP_ERRORS = (1, 2, 98, 719)  # invalid value, out of memory, invalid device function, launch failure


def load(path=None):
    """Open a host-only build and declare its test hooks."""
    L = cabi.load(path or cabi.HOST_LIB_PATH)
    L.flare_stub_set_launch_status.argtypes = [ctypes.c_int]
    L.flare_stub_reset.argtypes = []
    L.flare_stub_launches.restype = ctypes.c_long
    L.flare_stub_last_launch.restype = ctypes.c_char_p
    L.flare_stub_ranges.argtypes = [ctypes.POINTER(ctypes.c_ulonglong), ctypes.c_int]
    L.flare_stub_ranges.restype = ctypes.c_int
    return L


def ranges(L):
    buf = (ctypes.c_ulonglong * (4 * 256))()
    n = L.flare_stub_ranges(buf, 256)
    assert n <= 256
    return [tuple(buf[4 * i:4 * i + 4]) for i in range(n)]


def T(dtype=BF16, sb=0, sh=8, sl=8, data=FAKE):
    return cabi.FlareTensor(data, dtype, 0, sb, sh, sl)


def tok(B, H, N, D, dtype=BF16, data=FAKE):
    """A head-major [B, H, N, D] token-side view."""
    return T(dtype, H * N * D, N * D, D, data)


def lat(H, M, D, dtype=BF16, B=1, data=FAKE):
    return T(dtype, H * M * D if B > 1 else 0, M * D, D, data)


r = ctypes.byref
vp = ctypes.c_void_p


# ------------------------------------------------------- calls by entry point
# Each helper makes one call with valid arguments for the given sizes; keyword
# overrides replace single arguments.

def encode(L, B, H, M, N, D, ws=WS, ws_bytes=None, fn="flare_encode", **kw):
    need = L.flare_encode_workspace_size(B, H, M, N, D)
    Q = kw.get("Q", lat(H, M, D))
    K = kw.get("K", tok(B, H, N, D))
    V = kw.get("V", tok(B, H, N, D))
    Z = kw.get("Z", lat(H, M, D, F32, B))
    return getattr(L, fn)(r(Q), r(K), r(V), r(Z), kw.get("lse"), B, H, M, N, D, kw.get("scale", 0.0),
                          kw.get("flags", 0), vp(ws), need if ws_bytes is None else ws_bytes, None)


def decode(L, B, H, M, N, D, dtype=BF16, **kw):
    K, Y = tok(B, H, N, D, dtype), tok(B, H, N, D, dtype)
    Q, Z = lat(H, M, D), lat(H, M, D, F32, B)
    return L.flare_decode(r(K), r(Q), r(Z), r(Y), kw.get("lse"), B, H, M, N, D, 0.0, kw.get("flags", 0), None)


def project(L, R, Cin, Cout, n, head_major=0, B=1, hd=0, ws=WS, ws_bytes=None):
    need = L.flare_project_workspace_size(Cin, Cout, n)
    W = (vp * n)(*[FAKE + i * (1 << 24) for i in range(n)])
    Y = (vp * n)(*[FAKE + (i + 1) * (1 << 40) for i in range(n)])
    return L.flare_project(vp(FAKE), W, Y, n, R, Cin, Cout, head_major, B, hd, vp(ws),
                           need if ws_bytes is None else ws_bytes, None)


def mix(L, B, N, C, H, M, dynamic=True, shared=False, wo=True, ws=WS, ws_bytes=None, flags=0):
    need = L.flare_mix_workspace_size(B, N, C, H, M, int(dynamic), int(wo))
    p = lambda i: vp(FAKE + i * (1 << 24))
    wk, wv = p(1), p(2)
    ek, ev = (wk, wv) if shared else (p(3), p(4))
    if not dynamic:
        ek = ev = None
    return L.flare_mix(p(0), wk, wv, ek, ev, p(5), p(6) if wo else None, vp(OUT), BF16, B, N, C,
                       H, M, 0.0, flags, vp(ws), need if ws_bytes is None else ws_bytes, None)


def decode_backward(L, B, H, M, N, D, ws=WS, ws_bytes=None, **kw):
    need = L.flare_decode_backward_workspace_size(B, H, M, N, D)
    t, q, z, dk = tok(B, H, N, D), lat(H, M, D), lat(H, M, D, F32, B), kw.get("dK", tok(B, H, N, D, F32))
    return L.flare_decode_backward(r(t), r(q), r(z), r(t), kw.get("lse", vp(FAKE)), r(t), r(dk), vp(FAKE),
                                   vp(FAKE), kw.get("flags", 0), B, H, M, N, D, kw.get("scale", 0.0), vp(ws),
                                   need if ws_bytes is None else ws_bytes, None)


def encode_backward(L, B, H, M, N, D, ws=WS, ws_bytes=None, **kw):
    need = L.flare_encode_backward_workspace_size(B, H, M, N, D)
    t, q, z = tok(B, H, N, D), lat(H, M, D), lat(H, M, D, F32, B)
    dk, dv = kw.get("dK", tok(B, H, N, D, F32)), kw.get("dV", tok(B, H, N, D, F32))
    return L.flare_encode_backward(r(q), r(t), r(t), r(z), vp(FAKE), vp(FAKE), vp(FAKE), r(dk), r(dv),
                                   kw.get("flags", 0), B, H, M, N, D, kw.get("scale", 0.0), vp(ws),
                                   need if ws_bytes is None else ws_bytes, None)


def encdec_backward(L, B, H, M, N, D, ws=WS, ws_bytes=None, **kw):
    need = L.flare_encdec_backward_workspace_size(B, H, M, N, D)
    t, q, z = tok(B, H, N, D), lat(H, M, D), lat(H, M, D, F32, B)
    k = kw.get("K", t)
    dk, dv = kw.get("dK", tok(B, H, N, D, F32)), tok(B, H, N, D, F32)
    return L.flare_encdec_backward(r(q), r(k), r(t), r(z), kw.get("lse", vp(FAKE)), r(t), vp(FAKE), r(t),
                                   vp(FAKE), r(dk), r(dv), kw.get("flags", 0), B, H, M, N, D,
                                   kw.get("scale", 0.0), vp(ws), need if ws_bytes is None else ws_bytes, None)


def valid_calls(B=2, H=4, M=64, N=1000, D=32):
    """(name, call) pairs that each make one valid call of an entry point."""
    C = H * D
    return [
        ("encode", lambda L, **kw: encode(L, B, H, M, N, D, **kw)),
        ("route_queries", lambda L, **kw: encode(L, B, H, M, N, D, fn="flare_route_queries", **kw)),
        ("encode_f32", lambda L, **kw: encode(L, B, H, M, N, D, K=tok(B, H, N, D, F32), V=tok(B, H, N, D, F32),
                                              **kw)),
        ("decode", lambda L, **kw: decode(L, B, H, M, N, D, **kw)),
        ("decode_f32", lambda L, **kw: decode(L, B, H, M, N, D, F32, **kw)),
        ("project", lambda L, **kw: project(L, B * N, 64, 128, 3, **kw)),
        ("project_head_major", lambda L, **kw: project(L, B * N, C, C, 2, 1, B, D, **kw)),
        ("mix_dynamic", lambda L, **kw: mix(L, B, N, C, H, M, **kw)),
        ("mix_shared", lambda L, **kw: mix(L, B, N, C, H, M, shared=True, **kw)),
        ("mix_static_no_wo", lambda L, **kw: mix(L, B, N, C, H, M, dynamic=False, wo=False, **kw)),
        ("mix_fused_wo", lambda L, **kw: mix(L, B, N, C, H, M, flags=cabi.FLARE_MIX_FUSED_WO, **kw)),
        ("decode_backward", lambda L, **kw: decode_backward(L, B, H, M, N, D, **kw)),
        ("encode_backward", lambda L, **kw: encode_backward(L, B, H, M, N, D, **kw)),
        ("encdec_backward", lambda L, **kw: encdec_backward(L, B, H, M, N, D, **kw)),
    ]


NEEDS_WORKSPACE = {"encode", "route_queries", "encode_f32", "project", "project_head_major", "mix_dynamic",
                   "mix_shared", "mix_static_no_wo", "mix_fused_wo", "decode_backward", "encode_backward",
                   "encdec_backward"}
LAST_LAUNCH = {"encode": "merge", "route_queries": "merge", "encode_f32": "merge", "decode": "decode_bf16",
               "decode_f32": "decode_f32", "project": "gemm_bf16", "project_head_major": "gemm_bf16",
               "mix_dynamic": "gemm_bf16", "mix_shared": "gemm_bf16", "mix_static_no_wo": "decode_bf16",
               "mix_fused_wo": "decode_wo"}


def _workspace_need(L, name, B, H, M, N, D):
    C = H * D
    return {
        "encode": lambda: L.flare_encode_workspace_size(B, H, M, N, D),
        "route_queries": lambda: L.flare_encode_workspace_size(B, H, M, N, D),
        "encode_f32": lambda: L.flare_encode_workspace_size(B, H, M, N, D),
        "project": lambda: L.flare_project_workspace_size(64, 128, 3),
        "project_head_major": lambda: L.flare_project_workspace_size(C, C, 2),
        "mix_dynamic": lambda: L.flare_mix_workspace_size(B, N, C, H, M, 1, 1),
        "mix_shared": lambda: L.flare_mix_workspace_size(B, N, C, H, M, 1, 1),
        "mix_static_no_wo": lambda: L.flare_mix_workspace_size(B, N, C, H, M, 0, 0),
        "mix_fused_wo": lambda: L.flare_mix_workspace_size(B, N, C, H, M, 1, 1),
        "decode_backward": lambda: L.flare_decode_backward_workspace_size(B, H, M, N, D),
        "encode_backward": lambda: L.flare_encode_backward_workspace_size(B, H, M, N, D),
        "encdec_backward": lambda: L.flare_encdec_backward_workspace_size(B, H, M, N, D),
    }[name]()


# ------------------------------------------------------------------ checks

def check_encode_rejects_bad_arguments(L):
    e = lambda **kw: encode(L, 1, 2, 32, 100, 32, **kw)
    assert e() == OK
    assert e(K=cabi.FlareTensor(0, BF16, 0, 0, 8, 8)) == E_INVALID          # null data
    assert encode(L, 0, 2, 32, 100, 32) == E_INVALID
    assert encode(L, 1, 2, 32, 0, 32) == E_INVALID
    assert encode(L, 1, 2, 0, 100, 32) == E_INVALID
    assert encode(L, 300, 300, 32, 100, 32) == E_INVALID                     # B*H above the grid's y limit
    assert encode(L, 1, 2, 32, 100, 24) == E_UNSUPPORTED
    assert encode(L, 1, 2, 32, 100, 64) == E_UNSUPPORTED
    assert encode(L, 1, 2, 513, 100, 32) == E_UNSUPPORTED
    assert e(K=T(data=FAKE + 2)) == E_INVALID                                # misaligned rows
    assert e(V=T(sl=12)) == E_INVALID                                        # stride not a multiple of 8
    assert e(V=T(sl=1 << 22)) == E_INVALID                                   # beyond 32-bit tile offsets
    assert e(V=T(sh=-8)) == E_INVALID                                        # negative stride
    assert e(V=T(dtype=F32)) == E_INVALID                                    # K, V dtypes differ
    assert e(Q=T(dtype=7)) == E_INVALID                                      # unknown dtype
    assert e(Q=T(data=FAKE + 1)) == E_INVALID                                # misaligned latent element
    assert e(scale=float("nan")) == E_INVALID
    assert e(scale=float("inf")) == E_INVALID
    assert e(flags=0x80) == E_INVALID
    assert e(lse=vp(FAKE + 2)) == E_INVALID
    assert e(ws=0) == E_WORKSPACE
    assert e(ws=WS + 8) == E_WORKSPACE                                       # misaligned workspace
    assert e(ws_bytes=16) == E_WORKSPACE


def check_decode_and_route_reject_bad_arguments(L):
    ok = T()
    assert L.flare_decode(None, r(ok), r(ok), r(ok), None, 1, 1, 8, 10, 32, 0.0, 0, None) == E_INVALID
    assert L.flare_decode(r(ok), r(ok), r(ok), r(ok), None, 1, 1, 8, 10, 8, 0.0, 0, None) == E_UNSUPPORTED
    assert L.flare_decode(r(ok), r(ok), r(ok), r(T(data=FAKE + 8)), None, 1, 1, 8, 10, 32, 0.0, 0,
                          None) == E_INVALID
    assert L.flare_decode(r(ok), r(ok), r(ok), r(ok), vp(FAKE + 2), 1, 1, 8, 10, 32, 0.0, 0, None) == E_INVALID
    assert L.flare_decode(r(ok), r(ok), r(ok), r(ok), None, 1, 1, 8, 10, 32, 0.0, 2, None) == E_INVALID
    assert L.flare_route_queries(r(ok), r(ok), r(ok), r(ok), None, 1, 1, 8, 10, 32, 0.0, 0, None, 0,
                                 None) == E_WORKSPACE


def check_mix_and_project_reject_bad_arguments(L):
    p, n = vp(FAKE), None
    # C not divisible by H
    assert L.flare_mix(p, p, p, n, n, p, n, p, 1, 1, 10, 100, 3, 8, 0.0, 0, p, 1 << 40, n) == E_INVALID
    # fp32 mixer not built
    assert L.flare_mix(p, p, p, n, n, p, n, p, 0, 1, 10, 64, 2, 8, 0.0, 0, p, 1 << 40, n) == E_UNSUPPORTED
    # only one of the two synthesis weights
    assert L.flare_mix(p, p, p, p, n, p, n, p, 1, 1, 10, 64, 2, 8, 0.0, 0, p, 1 << 40, n) == E_INVALID
    # workspace too small, or not 256-byte aligned
    assert L.flare_mix(p, p, p, p, p, p, n, p, 1, 1, 10, 64, 2, 8, 0.0, 0, p, 64, n) == E_WORKSPACE
    assert L.flare_mix(p, p, p, p, p, p, n, p, 1, 1, 10, 64, 2, 8, 0.0, 0, vp(WS + 16), 1 << 40, n) == E_WORKSPACE
    # flag bits other than the exact softmax and the fused output projection
    assert mix(L, 1, 10, 64, 2, 8, flags=4) == E_INVALID
    assert mix(L, 1, 10, 64, 2, 8, flags=cabi.FLARE_MIX_FUSED_WO | 1) == OK
    assert encode(L, 1, 2, 32, 100, 32, flags=cabi.FLARE_MIX_FUSED_WO) == E_INVALID  # a mixer-only flag
    warr = (vp * 1)(FAKE)
    assert L.flare_project(p, warr, warr, 1, 10, 48, 64, 0, 1, 0, p, 1 << 30, n) == E_UNSUPPORTED
    assert L.flare_project(p, warr, warr, 1, 10, 64, 64, 1, 3, 32, p, 1 << 30, n) == E_INVALID
    assert L.flare_project(p, warr, warr, 1, 10, 64, 64, 0, 1, 0, p, 16, n) == E_WORKSPACE
    assert L.flare_project(p, warr, warr, 6, 10, 64, 64, 0, 1, 0, p, 1 << 30, n) == E_INVALID


def check_backward_calls_reject_bad_arguments(L):
    f32, bad = T(dtype=F32, sh=4, sl=4), T(dtype=5)
    db = lambda **kw: decode_backward(L, 1, 1, 8, 10, 32, **kw)
    assert db() == OK
    assert db(dK=bad) == E_INVALID
    assert db(lse=None) == E_INVALID                    # the normaliser is required
    assert decode_backward(L, 1, 1, 8, 10, 8) == E_UNSUPPORTED
    need = L.flare_decode_backward_workspace_size(1, 1, 8, 10, 32)
    assert need > 0 and db(ws_bytes=need - 1) == E_WORKSPACE
    assert db(flags=8) == E_INVALID                     # unknown flag bits
    eb = lambda **kw: encode_backward(L, 1, 1, 8, 10, 32, **kw)
    assert eb() == OK
    assert eb(flags=8) == E_INVALID
    assert eb(dK=tok(1, 1, 10, 32)) == E_UNSUPPORTED    # dK bf16 with dV fp32: one dtype for both
    assert eb(scale=float("nan")) == E_INVALID
    pair = lambda **kw: encdec_backward(L, 1, 1, 8, 10, kw.pop("D", 32), **kw)
    need = L.flare_encdec_backward_workspace_size(1, 1, 8, 10, 32)
    assert need >= L.flare_decode_backward_workspace_size(1, 1, 8, 10, 32)
    assert pair() == OK
    assert pair(K=f32) == E_UNSUPPORTED
    assert pair(dK=tok(1, 1, 10, 32)) == E_UNSUPPORTED
    assert pair(lse=None) == E_INVALID
    assert pair(flags=8) == E_INVALID
    assert pair(D=8) == E_UNSUPPORTED
    assert pair(ws_bytes=need - 1) == E_WORKSPACE


def check_workspace_sizes(L):
    small = L.flare_encode_workspace_size(1, 8, 256, 4096, 32)
    big = L.flare_encode_workspace_size(1, 8, 256, 1 << 20, 32)
    assert 0 < small <= big
    assert L.flare_encode_workspace_size(1, 8, 256, 1 << 20, 24) == 0
    assert L.flare_project_workspace_size(256, 256, 4) == 4 * 256 * 256 * 2
    assert L.flare_project_workspace_size(48, 256, 1) == 0
    m1 = L.flare_mix_workspace_size(4, 1 << 18, 256, 8, 512, 1, 1)
    m0 = L.flare_mix_workspace_size(4, 1 << 18, 256, 8, 512, 0, 0)
    assert m1 > m0 > 4 * (1 << 18) * 256 * 2 * 2
    assert L.flare_mix_workspace_size(1, 10, 100, 3, 8, 1, 0) == 0
    for f in (L.flare_decode_backward_workspace_size, L.flare_encode_backward_workspace_size,
              L.flare_encdec_backward_workspace_size):
        assert f(1, 1, 8, 10, 32) > 0 and f(1, 1, 8, 10, 8) == 0 and f(0, 1, 8, 10, 32) == 0


def check_status_strings(L):
    text = lambda s: L.flare_status_string(s).decode()
    assert text(OK) == "ok"
    assert "workspace" in text(E_WORKSPACE)
    assert text(12345) == "unknown status"
    assert len({text(s) for s in (OK, E_INVALID, E_UNSUPPORTED, E_WORKSPACE, E_HIP, cabi.FLARE_E_SCRATCH)}) == 6


def check_valid_calls_launch(L):
    for name, call in valid_calls():
        L.flare_stub_reset()
        assert call(L) == OK, name
        assert L.flare_stub_launches() >= 1, name
        if name in LAST_LAUNCH:
            assert L.flare_stub_last_launch().decode() == LAST_LAUNCH[name], name


def check_launch_failure_maps_to_hip_error(L):
    """Any launcher error ends the call with FLARE_E_HIP and nothing more is launched."""
    try:
        for status in HIP_ERRORS:
            for name, call in valid_calls():
                L.flare_stub_reset()
                L.flare_stub_set_launch_status(status)
                assert call(L) == E_HIP, (name, status)
                assert L.flare_stub_launches() == 1, (name, status, L.flare_stub_launches())
    finally:
        L.flare_stub_reset()


def check_short_workspace_is_refused(L):
    for name, call in valid_calls():
        if name not in NEEDS_WORKSPACE:
            continue
        need = _workspace_need(L, name, 2, 4, 64, 1000, 32)
        L.flare_stub_reset()
        assert need > 0, name
        assert call(L, ws_bytes=need - 1) == E_WORKSPACE, name
        assert call(L, ws=0) == E_WORKSPACE, name
        assert L.flare_stub_launches() == 0, name


def check_small_mixer_merges_in_the_decoder(L):
    """The mixer lets the decoder merge small split sets of its encoder (no
    merge launch for them: weight rearrangement, projections, synthesis
    encoder and merge, encoder, decoder), the decoder reads exactly the split
    results that encoder wrote, and large split sets keep their merge launch.
    Small weight sets on few rows need no rearrangement launch: the
    projection kernel lays them out itself."""
    for (B, H, M, N, D), fold in (((2, 4, 64, 1000, 16), True), ((8, 8, 64, 4096, 16), True),
                                  ((32, 8, 128, 4096, 32), True), ((1, 8, 512, 1 << 20, 32), False)):
        L.flare_stub_reset()
        assert mix(L, B, N, H * D, H, M, wo=False) == OK, (B, H, M, N, D)
        rs = ranges(L)
        C = H * D
        preload = (B * N + 255) // 256 < 512 and 4 * C * C * 2 <= 128 * 1024
        assert preload == (C <= 128), (B, H, M, N, D)
        assert bool([x for x in rs if x[3] == SWIZZLED]) != preload, (B, H, M, N, D)
        expected = (6 if fold else 7) - (1 if preload else 0)
        assert L.flare_stub_launches() == expected, (B, H, M, N, D, L.flare_stub_launches())
        zp = [x for x in rs if x[3] == DEC_ZPART]
        assert bool(zp) == fold, (B, H, M, N, D, rs)
        if fold:
            enc_o = [x for x in rs if x[3] == ENC_PART_O]
            enc_l = [x for x in rs if x[3] == ENC_PART_L]
            assert zp[0][:2] == enc_o[-1][:2] and zp[1][:2] == enc_l[-1][:2], (zp, enc_o, enc_l)
            assert zp[0][2] == enc_o[-1][2] + 1  # the launch right after that encoder


def _overlap(a, b):
    return a[0] < b[0] + b[1] and b[0] < a[0] + a[1]


def workspace_carving(L, B, H, M, N, D):
    """Every buffer carved from the workspace lies inside it, with no overlap
    between buffers that one launch writes, or that a launch writes while it
    reads another (encoder partials vs. K/V in the workspace, projection
    outputs vs. the swizzled weights)."""
    for name, call in valid_calls(B, H, M, N, D):
        if name not in NEEDS_WORKSPACE:
            continue
        need = _workspace_need(L, name, B, H, M, N, D)
        if need == 0:  # sizes outside this entry point (mix: C = H*D)
            continue
        L.flare_stub_reset()
        assert call(L) == OK, (name, B, H, M, N, D)
        rs = ranges(L)
        inside = lambda x: WS <= x[0] and x[0] + x[1] <= WS + need
        for addr, nbytes, launch, tag in rs:
            in_ws = tag in (ENC_PART_O, ENC_PART_L, BWD_DQ, BWD_DZ, SUM_PART, SWIZZLED, WO_LAT, WO_T, DEC_ZPART)
            if name.startswith("mix"):
                # projections and encoder inputs live in the workspace, except
                # the output projection's result, which is the caller's
                in_ws = in_ws or tag in (ENC_K, ENC_V) or (tag == GEMM_OUT and addr != OUT)
            if in_ws:
                assert nbytes > 0 and inside((addr, nbytes)), (name, tag, hex(addr), nbytes, hex(need))
            assert addr % 16 == 0, (name, tag, hex(addr))
        for i, a in enumerate(rs):
            for b in rs[i + 1:]:
                same = a[2] == b[2]
                if same and a[3] in WRITTEN and b[3] in WRITTEN:
                    assert not _overlap(a, b), (name, a, b)
                if same and {a[3], b[3]} & {ENC_PART_O, ENC_PART_L} and {a[3], b[3]} & {ENC_K, ENC_V}:
                    assert not _overlap(a, b), (name, a, b)
                if {a[3], b[3]} == {SWIZZLED, GEMM_OUT}:
                    assert not _overlap(a, b), (name, a, b)


CARVING_SHAPES = [(1, 1, 1, 1, 16), (1, 2, 32, 100, 32), (2, 3, 17, 4097, 16), (4, 8, 256, 65536, 32),
                  (1, 8, 512, 1 << 20, 32), (16, 16, 512, 1 << 22, 32), (300, 200, 8, 300, 16)]


def check_workspace_carving(L):
    for shape in CARVING_SHAPES:
        workspace_carving(L, *shape)


def run_all(L):
    names = sorted(n for n in globals() if n.startswith("check_"))
    for n in names:
        globals()[n](L)
        print(f"ok {n}", flush=True)
    return len(names)


if __name__ == "__main__":
    count = run_all(load(sys.argv[1] if len(sys.argv) > 1 else None))
    print(f"passed {count}", flush=True)

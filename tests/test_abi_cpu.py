"""CPU tier of the C ABI (include/flare.h).

The gfx950 library is only opened here: it loads and exports every declared
symbol, and its two pure-host functions (status strings, version) answer.  No
compute entry point of it is called, so no pointer ever reaches a kernel.
Argument checks, planning, workspace carving and the mapping of launch errors
run against the host-only build (same host code, stand-in launchers), through
tests/abi_host_checks.py, and once more under AddressSanitizer and
UndefinedBehaviorSanitizer in a child process.
"""
import ctypes
import os
import re
import subprocess
import sys

import pytest
from hypothesis import given, settings, strategies as st

from rank_latent_routing_amd import binding as fb
from rank_latent_routing_amd import cabi

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import abi_host_checks as hc  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flare.h")

needs_lib = pytest.mark.skipif(not os.path.exists(cabi.LIB_PATH), reason="HIP library not built")
needs_host = pytest.mark.skipif(not os.path.exists(cabi.HOST_LIB_PATH), reason="host-only library not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flare_[a-z_]+)\s*\(", text)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for f in ("flare_route_queries", "flare_encode", "flare_decode", "flare_mix"):
        assert f in names
    assert set(names) == set(cabi.EXPORTS)


@needs_lib
def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(cabi.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name


@needs_lib
def test_library_status_strings_and_version():
    L = cabi.load(cabi.LIB_PATH)
    assert L.flare_status_string(0).decode() == "ok"
    assert "workspace" in L.flare_status_string(cabi.FLARE_E_WORKSPACE).decode()
    assert L.flare_status_string(12345).decode() == "unknown status"
    assert re.fullmatch(r"\d+\.\d+\.\d+", L.flare_version().decode())


@pytest.fixture(scope="module")
def host():
    L = hc.load(cabi.HOST_LIB_PATH)
    L.flare_stub_reset()
    yield L
    L.flare_stub_reset()


@needs_host
def test_host_build_exports_the_host_entry_points(host):
    for name in cabi.EXPORTS:
        if name not in cabi.DEVICE_ONLY:
            assert hasattr(host, name), name


@needs_host
@pytest.mark.parametrize("check", sorted(n for n in dir(hc) if n.startswith("check_")))
def test_host_check(host, check):
    getattr(hc, check)(host)


@needs_host
@settings(max_examples=150, deadline=None)
@given(B=st.integers(1, 64), H=st.integers(1, 32), M=st.integers(1, 512),
       logN=st.floats(0.0, 24.0), D=st.sampled_from([16, 32]))
def test_workspace_carving_property(host, B, H, M, logN, D):
    hc.workspace_carving(host, B, H, M, max(1, int(2.0 ** logN)), D)


@needs_host
def test_host_checks_under_address_and_undefined_behaviour_sanitizers():
    lib = cabi.HOST_SAN_LIB_PATH
    if not os.path.exists(lib):
        pytest.skip("sanitized host-only library not built")
    asan = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("AddressSanitizer runtime not found")
    env = dict(os.environ)
    env["LD_PRELOAD"] = asan + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([sys.executable, os.path.join(ROOT, "tests", "abi_host_checks.py"), lib],
                       capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    n = len([x for x in dir(hc) if x.startswith("check_")])
    assert f"passed {n}" in r.stdout, out[-4000:]


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(fb, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(fb, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        fb.lib()


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

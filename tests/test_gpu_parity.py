"""GPU tier: the HIP library through its C ABI against the fp64 oracle.

Tolerances (stated for the two number paths of the library):
  * bf16 inputs, matrix cores, fp32 accumulation: relative L2 error of the
    whole output tensor <= 1e-2 (also checked per (batch, head));
  * fp32 path: normwise max relative error ||y - r||_inf / ||r||_inf <= 1e-4.
The oracle reads exactly the rounded inputs the GPU reads, widened to fp64.
"Sharp" cases scale the queries so that scores span tens of units, which
also drives the kernels' exact-softmax fallback; FLARE_FLAG_EXACT_SOFTMAX
forces that path everywhere.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import rank_latent_routing_amd as rl
from rank_latent_routing_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF16_TOL = 1e-2
F32_TOL = 1e-4
EXACT = rl.FLARE_FLAG_EXACT_SOFTMAX


def f64(t):
    return t.detach().double().cpu().numpy()


def rel_l2(a, b):
    return float(np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300))


def max_rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def elementwise_max_rel(a, b, floor=1e-3):
    """max |a_i - b_i| / |b_i| over the outputs with |b_i| >= floor * ||b||_inf (an elementwise
    ratio on outputs near zero would measure their conditioning, not the kernel)."""
    big = np.abs(b) >= floor * np.max(np.abs(b))
    return float(np.max(np.abs(a - b)[big] / np.abs(b)[big]))


def check_f32(got, ref, what):
    """Normwise max-rel within the fp32 bar; the elementwise max-rel over the outputs above
    1e-3 of the largest is reported, and held to the bound the normwise bar implies."""
    e, ee = max_rel(got, ref), elementwise_max_rel(got, ref)
    say(f"  {what}: max-rel (normwise) {e:.2e}, elementwise over |r| >= 1e-3 max|r|: {ee:.2e}")
    assert e <= F32_TOL, what
    assert ee <= F32_TOL / 1e-3, what


def say(*a):
    print(*a, flush=True)


def hm(t):
    """[B, N, H, D] -> [B, H, N, D] view."""
    return t.permute(0, 2, 1, 3)


def check_bf16(got, ref, what, per_bh_axes=None):
    e = rel_l2(got, ref)
    say(f"  {what}: rel-L2 {e:.3e}")
    assert e <= BF16_TOL, what
    if per_bh_axes is not None:
        B, H = ref.shape[0], ref.shape[1]
        for b in range(B):
            for h in range(H):
                assert rel_l2(got[b, h], ref[b, h]) <= BF16_TOL, (what, b, h)


# (B, H, N, D, M, layout, q_mult, flags, per_batch_q, z_dtype)
ENCDEC_CASES = [
    (1, 8, 5000, 32, 256, "token", 1.0, 0, False, torch.float32),
    (2, 4, 3001, 32, 64, "head", 8.0, 0, True, torch.bfloat16),
    (2, 4, 3001, 32, 64, "head", 8.0, EXACT, True, torch.float32),
    (1, 2, 1, 32, 32, "token", 1.0, 0, False, torch.float32),
    (1, 2, 63, 16, 17, "token", 4.0, 0, False, torch.float32),
    (3, 2, 700, 16, 64, "head", 1.0, 0, False, torch.float32),
    (1, 1, 2000, 32, 1, "token", 2.0, 0, False, torch.float32),
    (1, 2, 4096, 32, 512, "head", 1.0, 0, False, torch.float32),
    (1, 2, 4096, 16, 512, "token", 8.0, 0, False, torch.float32),
    (2, 3, 1500, 32, 128, "token", 8.0, EXACT, False, torch.float32),
    (1, 1, 70000, 32, 48, "head", 30.0, 0, False, torch.float32),
    (1, 2, 20000, 32, 200, "token", 1.0, EXACT, False, torch.float32),
]


@pytest.mark.parametrize("case", ENCDEC_CASES, ids=lambda c: "B{}H{}N{}D{}M{}-{}-q{}-f{}-pb{}".format(*c[:9]))
def test_encode_decode_bf16(case):
    B, H, N, D, M, layout, qm, flags, pbq, zdt = case
    say(f"case {case}")
    w = inputs.Workload("t", "encdec", B, N, H, D, M, "bf16")
    x = inputs.make_encdec(w, seed=N + M, q_mult=qm, per_batch_q=pbq)
    q = x["q"].to(DEV)
    if layout == "head":
        k = hm(x["k"]).contiguous().to(DEV)
        v = hm(x["v"]).contiguous().to(DEV)
        kv, vv = k, v
        y = torch.empty_like(k)
        yv = y
    else:
        k, v = x["k"].to(DEV), x["v"].to(DEV)
        kv, vv = hm(k), hm(v)
        y = torch.empty_like(k)
        yv = hm(y)
    z, lse = rl.flare_encode(q, kv, vv, want_lse=True, flags=flags, z_dtype=zdt)
    rl.flare_decode(kv, q, z, y=yv, flags=flags)
    torch.cuda.synchronize()
    qo = f64(x["q"])
    ko, vo = f64(hm(x["k"])), f64(hm(x["v"]))
    zr, lr = oracle.encode(qo, ko, vo)
    yr = oracle.decode(ko, qo, zr)
    check_bf16(f64(z), zr, "Z", per_bh_axes=True)
    el = float(np.max(np.abs(f64(lse) - lr)))
    say(f"  lse: max abs err {el:.3e}")
    assert el <= 1e-2 * max(1.0, float(np.max(np.abs(lr))))
    check_bf16(f64(yv), yr, "Y", per_bh_axes=True)


def test_decode_alone_with_oracle_latents():
    # The decoder fed the oracle's own latent values (rounded to fp32): its
    # error is then the decoder's alone.
    B, H, N, D, M = 2, 3, 3000, 32, 96
    w = inputs.Workload("t", "encdec", B, N, H, D, M, "bf16")
    x = inputs.make_encdec(w, seed=5, q_mult=3.0)
    ko, vo, qo = f64(hm(x["k"])), f64(hm(x["v"])), f64(x["q"])
    zr, _ = oracle.encode(qo, ko, vo)
    z32 = torch.from_numpy(zr).float()
    yr = oracle.decode(ko, qo, f64(z32))
    k = hm(x["k"]).contiguous().to(DEV)
    y = rl.flare_decode(k, x["q"].to(DEV), z32.to(DEV))
    torch.cuda.synchronize()
    check_bf16(f64(y), yr, "Y(decode only)", per_bh_axes=True)


@pytest.mark.parametrize("z_dtype", [torch.float32, torch.bfloat16])
def test_decode_large_latent_values(z_dtype):
    # Head 0: latent values near 1e15 and a common score offset of about 55
    # (feature 0 of every key 8, of every query 39), so the unscaled weights
    # sum to about e^60 (inside the fast pass's accepted normaliser range) and
    # the unnormalised outputs overflow fp32: the kernel must notice and redo
    # the head with the row maximum subtracted.  Head 1: the same magnitudes
    # without the offset (fast result kept).  Head 2: ordinary values.
    B, H, N, D, M = 1, 3, 1500, 32, 80
    w = inputs.Workload("t", "encdec", B, N, H, D, M, "bf16")
    x = inputs.make_encdec(w, seed=11)
    q, k = x["q"].clone(), x["k"].clone()
    q[0, :, 0] = 39.0
    k[:, :, 0, 0] = 8.0
    z = inputs.normal_tensor((B, H, M, D), "f32", seed=12)
    z[:, :2] *= 1e15
    z = z.to(z_dtype)
    qo, ko = f64(q), f64(hm(k))
    yr = oracle.decode(ko, qo, f64(z))
    y = rl.flare_decode(hm(k).contiguous().to(DEV), q.to(DEV), z.to(DEV))
    torch.cuda.synchronize()
    got = f64(y)
    assert np.all(np.isfinite(got))
    check_bf16(got, yr, "Y(large latents)", per_bh_axes=True)


@pytest.mark.parametrize("qm", [1.0, 6.0])
def test_route_queries_shared_seeds(qm):
    B, H, N, D, M = 3, 4, 2500, 32, 64
    w = inputs.Workload("t", "encdec", B, N, H, D, M, "bf16")
    x = inputs.make_encdec(w, seed=7, q_mult=qm, synth=True)
    ek, ev = hm(x["ek"]).to(DEV), hm(x["ev"]).to(DEV)
    qx = rl.flare_route_queries(x["seeds"].to(DEV), ek, ev)
    torch.cuda.synchronize()
    qr, _ = oracle.encode(f64(x["seeds"]), f64(hm(x["ek"])), f64(hm(x["ev"])))
    check_bf16(f64(qx), qr, "Q(X)", per_bh_axes=True)


@pytest.mark.parametrize("flags", [0, EXACT])
def test_fp32_path_encdec_n1k(flags):
    # FLARE encode/decode in fp32: B=1, H=4, D=16, N=1024, M=32, seed 0.
    w = inputs.WORKLOADS["encdec_f32_n1k"]
    x = inputs.make_encdec(w, seed=0)
    q = x["q"].to(DEV)
    k, v = x["k"].to(DEV), x["v"].to(DEV)
    z, lse = rl.flare_encode(q, hm(k), hm(v), want_lse=True, flags=flags)
    y = torch.empty_like(k)
    rl.flare_decode(hm(k), q, z, y=hm(y), flags=flags)
    torch.cuda.synchronize()
    yr, zr, lr = oracle.flare_encdec(f64(x["q"]), f64(x["k"]).reshape(1, 1024, 64),
                                     f64(x["v"]).reshape(1, 1024, 64), 4, want_latents=True)
    check_f32(f64(z), zr, "Z")
    check_f32(f64(y).reshape(1, 1024, 64), yr, "Y")
    el = float(np.max(np.abs(f64(lse) - lr)))
    say(f"  lse abs {el:.2e}")
    assert el <= 1e-4


def test_fp32_path_ragged_and_sharp():
    B, H, N, D, M = 2, 3, 777, 32, 40
    w = inputs.Workload("t", "encdec", B, N, H, D, M, "f32")
    x = inputs.make_encdec(w, seed=3, q_mult=6.0)
    q, k, v = x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV)
    z = rl.flare_encode(q, hm(k), hm(v))
    y = torch.empty_like(k)
    rl.flare_decode(hm(k), q, z, y=hm(y))
    torch.cuda.synchronize()
    ko, vo, qo = f64(hm(x["k"])), f64(hm(x["v"])), f64(x["q"])
    zr, _ = oracle.encode(qo, ko, vo)
    yr = oracle.decode(ko, qo, zr)
    check_f32(f64(z), zr, "Z")
    check_f32(f64(hm(y)), yr, "Y")


@pytest.mark.parametrize("R,Cin,Cout,nproj,head_dim", [
    (1000, 128, 128, 4, 16), (4096, 256, 256, 2, 32), (333, 256, 256, 5, None),
    (64, 64, 96, 1, None), (2048, 32, 64, 3, 32),
    # row-major outputs with paired column blocks and two row tiles per wave
    # (R of at least 512 workgroups), ragged last rows
    (140001, 256, 256, 1, None), (131331, 128, 192, 2, None), (140000, 64, 96, 1, None)])
def test_projection_gemm(R, Cin, Cout, nproj, head_dim):
    B = 2 if head_dim and R % 2 == 0 else 1
    xs = inputs.normal_tensor((B, R // B, Cin), "bf16", seed=R)
    ws = [inputs.normal_tensor((Cin, Cout), "bf16", seed=100 + i, std=1 / math.sqrt(Cin))
          for i in range(nproj)]
    outs = rl.flare_project(xs.to(DEV), [w.to(DEV) for w in ws], head_dim=head_dim)
    torch.cuda.synchronize()
    x2 = f64(xs).reshape(R, Cin)
    for i, w in enumerate(ws):
        ref = oracle.matmul(x2, f64(w))
        got = f64(outs[i])
        if head_dim:
            Hh = Cout // head_dim
            got = got.reshape(B, Hh, R // B, head_dim).transpose(0, 2, 1, 3).reshape(R, Cout)
        check_bf16(got, ref, f"projection {i}")


def _oracle_mix(m, H, batches=None):
    sel = (lambda a: a[batches]) if batches is not None else (lambda a: a)
    return oracle.flare_mix(sel(f64(m["x"])), f64(m["w_k"]), f64(m["w_v"]), f64(m["qs"]), H,
                            w_ek=f64(m["w_ek"]) if "w_ek" in m else None,
                            w_ev=f64(m["w_ev"]) if "w_ev" in m else None,
                            w_o=f64(m["w_o"]) if "w_o" in m else None)[0]


def _gpu_mix(m, H, flags=0):
    g = {n: t.to(DEV) for n, t in m.items()}
    out = rl.flare_mix(g["x"], g["w_k"], g["w_v"], g["qs"], H, w_ek=g.get("w_ek"),
                       w_ev=g.get("w_ev"), w_o=g.get("w_o"), flags=flags)
    torch.cuda.synchronize()
    return f64(out)


@pytest.mark.parametrize("qm", [1.0, 8.0])
def test_mix_flarepp_n4k_c128(qm):
    # FLARE++ mixer, B=8, C=128, H=8 (D=16), N=4096, M=64, full size.
    w = inputs.WORKLOADS["mix_bf16_n4k_c128"]
    m = inputs.make_mix(w, seed=0, q_mult=qm)
    check_bf16(_gpu_mix(m, w.H), _oracle_mix(m, w.H), f"FLARE++ mix (seed x{qm})")


def test_mix_seq_b32_sampled_batches():
    # Sequence-shaped FLARE++ (B=32, N=4096, C=256, M=128) at full size; the
    # oracle checks batch elements 0 and 31 (batch elements are independent).
    w = inputs.WORKLOADS["seq_bf16_b32_n4k"]
    m = inputs.make_mix(w, seed=0)
    got = _gpu_mix(m, w.H)
    check_bf16(got[[0, 31]], _oracle_mix(m, w.H, batches=[0, 31]), "FLARE++ seq mix")


# (B, N, C, H, M, q_mult): the small mixer itself, M not a multiple of 32 with
# 4-wave encoder workgroups, and 300 latents in two latent blocks.
WORKSPACE_CASES = [(8, 4096, 128, 8, 64, 8.0), (3, 1000, 64, 4, 100, 2.0), (2, 700, 256, 8, 300, 1.0)]


@pytest.mark.parametrize("case", WORKSPACE_CASES, ids=lambda c: "B{}N{}C{}H{}M{}-q{}".format(*c))
def test_mix_ignores_workspace_contents(case):
    # Nothing the mixer reads from its workspace is left over from before the
    # call: a workspace full of stale bytes, and one reused by the next call,
    # give the same output bit for bit as a zeroed one, and that output
    # matches the oracle.
    B, N, C, H, M, qm = case
    w = inputs.Workload("t", "mix", B, N, H, C // H, M, "bf16", dynamic=True, has_wo=False)
    m = inputs.make_mix(w, seed=N + M, q_mult=qm)
    g = {n: t.to(DEV) for n, t in m.items()}
    need = rl.mix_workspace_size(B, N, C, H, M, True, False)
    outs = []
    ws = None
    for fill in (0, 0x7F, 0xFF, None):  # None: the previous call's workspace as it was left
        if fill is not None:
            ws = torch.full((need,), fill, dtype=torch.uint8, device=DEV)
        say(f"  workspace fill {fill}")
        outs.append(rl.flare_mix(g["x"], g["w_k"], g["w_v"], g["qs"], H, w_ek=g["w_ek"], w_ev=g["w_ev"],
                                 workspace=ws))
        torch.cuda.synchronize()
    for o in outs[1:]:
        assert torch.equal(o, outs[0])
    check_bf16(f64(outs[0]), _oracle_mix(m, H), f"mix on a stale workspace {case}")


@pytest.mark.parametrize("dynamic,has_wo,qm,flags", [
    (True, True, 1.0, 0), (True, True, 8.0, 0), (False, True, 2.0, 0), (False, False, 1.0, EXACT),
    (True, False, 8.0, EXACT)])
def test_mix_block_reduced(dynamic, has_wo, qm, flags):
    # The block workload's shape (C=256, H=8, M=512) at N = 3000 tokens.
    w = inputs.Workload("t", "mix", 2, 3000, 8, 32, 512, "bf16", dynamic=dynamic, has_wo=has_wo)
    m = inputs.make_mix(w, seed=2, q_mult=qm)
    check_bf16(_gpu_mix(m, w.H, flags), _oracle_mix(m, w.H), f"mix dyn={dynamic} wo={has_wo}")


FUSED = rl.FLARE_MIX_FUSED_WO


# (B, N, C, H, M, dynamic, q_mult, flags): the output projection in the
# decoder's epilogue; ragged token windows (N not a multiple of 384), M not a
# multiple of 32, C = 128 (4 heads), sharp seeds that send heads to the exact
# fallback, and the exact softmax forced.
FUSED_CASES = [
    (2, 3000, 256, 8, 512, True, 1.0, FUSED),
    (2, 3000, 256, 8, 512, True, 8.0, FUSED),
    (1, 777, 128, 4, 200, False, 2.0, FUSED),
    (2, 1000, 256, 8, 100, True, 30.0, FUSED),
    (1, 500, 256, 8, 64, False, 1.0, FUSED | EXACT),
    (3, 1, 256, 8, 32, True, 1.0, FUSED),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=lambda c: "B{}N{}C{}H{}M{}-dyn{}-q{}-f{}".format(*c))
def test_mix_fused_output_projection(case):
    B, N, C, H, M, dyn, qm, flags = case
    w = inputs.Workload("t", "mix", B, N, H, C // H, M, "bf16", dynamic=dyn, has_wo=True)
    m = inputs.make_mix(w, seed=N + M, q_mult=qm)
    fused = _gpu_mix(m, H, flags)
    check_bf16(fused, _oracle_mix(m, H), f"fused W_O mix {case}")
    # the two-pass form computes the same Y (bf16) and sums the projection in
    # another order
    plain = _gpu_mix(m, H, flags & ~FUSED)
    e = rel_l2(fused, plain)
    say(f"  fused vs two-pass: rel-L2 {e:.2e}")
    assert e <= 1e-2


@pytest.mark.parametrize("qm", [1.0, 8.0])
def test_mix_shared_projections(qm):
    # FLARE++ with shared projections (the synthesis attends over K and V):
    # the same weight tensors passed for both pairs; the oracle runs the
    # general mixer with eK = K, eV = V.
    w = inputs.Workload("t", "mix", 2, 3000, 8, 32, 128, "bf16", dynamic=True, has_wo=True)
    m = inputs.make_mix(w, seed=4, q_mult=qm)
    g = {n: t.to(DEV) for n, t in m.items()}
    out = rl.flare_mix(g["x"], g["w_k"], g["w_v"], g["qs"], w.H, w_ek=g["w_k"], w_ev=g["w_v"], w_o=g["w_o"])
    torch.cuda.synchronize()
    ref = oracle.flare_mix(f64(m["x"]), f64(m["w_k"]), f64(m["w_v"]), f64(m["qs"]), w.H,
                           w_ek=f64(m["w_k"]), w_ev=f64(m["w_v"]), w_o=f64(m["w_o"]))[0]
    check_bf16(f64(out), ref, f"FLARE++ shared projections (seed x{qm})")


def test_deterministic_repeat():
    w = inputs.Workload("t", "encdec", 1, 4000, 4, 32, 256, "bf16")
    x = inputs.make_encdec(w, seed=9, q_mult=2.0)
    q, k, v = x["q"].to(DEV), hm(x["k"]).to(DEV), hm(x["v"]).to(DEV)
    outs = []
    for _ in range(2):
        z = rl.flare_encode(q, k, v, z_dtype=torch.float32)
        outs.append((z.clone(), rl.flare_decode(k, q, z).clone()))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_metric_workload_full_size_sampled():
    # FLARE encode/decode at N = 1,048,576, H=8, D=32, M=256 (bf16), in the
    # launch configuration the benchmark times.  The oracle computes every
    # latent of heads 0 and 5 and 4096 sampled tokens of their decode.
    w = inputs.WORKLOADS["encdec_bf16_n1m"]
    x = inputs.make_encdec(w, seed=0)
    q = x["q"].to(DEV)
    k = hm(x["k"]).contiguous().to(DEV)
    v = hm(x["v"]).contiguous().to(DEV)
    z = rl.flare_encode(q, k, v, z_dtype=torch.bfloat16)
    y = rl.flare_decode(k, q, z)
    torch.cuda.synchronize()
    rows = np.random.default_rng(0).choice(w.N, 4096, replace=False)
    for h in (0, 5):
        kh = f64(x["k"][0, :, h])
        vh = f64(x["v"][0, :, h])
        qh = f64(x["q"][h])
        zr = oracle.sdpa(qh, kh, vh)
        check_bf16(f64(z[0, h]), zr, f"Z head {h}")
        yr = oracle.sdpa(kh[rows], qh, zr)
        check_bf16(f64(y[0, h])[rows], yr, f"Y head {h} (4096 sampled tokens)")


@pytest.mark.parametrize("flags", [0, rl.FLARE_MIX_FUSED_WO], ids=["two-pass", "fused-wo"])
def test_block_workload_full_size_sampled(flags):
    # FLARE++ block with all projections (B=4, N=262,144, C=256, H=8, M=512)
    # at full size; the oracle computes batch element 3 at 2048 sampled output
    # tokens from oracle primitives (projections, the three SDPA calls per
    # head, the output projection).
    w = inputs.WORKLOADS["block_bf16_n256k"]
    m = inputs.make_mix(w, seed=0)
    got = _gpu_mix(m, w.H, flags)
    b = 3
    X = f64(m["x"][b])
    K, V, eK, eV = (oracle.matmul(X, f64(m[n])) for n in ("w_k", "w_v", "w_ek", "w_ev"))
    rows = np.sort(np.random.default_rng(1).choice(w.N, 2048, replace=False))
    D = w.D
    Y = np.empty((len(rows), w.C))
    for h in range(w.H):
        sl = slice(h * D, (h + 1) * D)
        Qh = oracle.sdpa(f64(m["qs"][h]), eK[:, sl], eV[:, sl])
        Zh = oracle.sdpa(Qh, K[:, sl], V[:, sl])
        Y[:, sl] = oracle.sdpa(K[rows, sl], Qh, Zh)
    ref = oracle.matmul(Y, f64(m["w_o"]))
    check_bf16(got[b][rows], ref, "FLARE++ block out (sampled)")


# ---------------------------------------------------------------- backward
# Gradients of the two SDPA calls (standard SDPA backward, recomputed from the
# forward normalisers) against the oracle's fp64 gradients on the same
# bf16-rounded inputs.

BWD_CASES = [
    # B, H, N, D, M, q_mult, layout, per-batch q
    (1, 2, 1000, 32, 64, 1.0, "head", False),
    (2, 3, 777, 32, 200, 4.0, "token", False),
    (1, 2, 333, 16, 48, 2.0, "head", True),
    (1, 1, 5000, 32, 256, 8.0, "head", False),
    (2, 2, 64, 32, 17, 1.0, "token", True),
    (1, 1, 1, 32, 32, 1.0, "head", False),
    (1, 2, 3000, 16, 512, 2.0, "head", False),
]


def check_grad(got, ref, what, scale_ref):
    """rel-L2 within the bf16 bar; a gradient that is exactly zero in real
    arithmetic (one token: the softmax weight is 1 and dS = dP - delta
    cancels) is held to 1e-2 of a well-scaled gradient of the same call."""
    nr = float(np.linalg.norm(ref.ravel()))
    if nr <= 1e-12 * float(np.linalg.norm(scale_ref.ravel())):
        e = float(np.linalg.norm(got.ravel())) / float(np.linalg.norm(scale_ref.ravel()))
        say(f"  {what}: zero in exact arithmetic, |got| / |scale| {e:.3e}")
        assert e <= BF16_TOL, what
    else:
        check_bf16(got, ref, what)


def _bwd_inputs(case):
    B, H, N, D, M, qm, layout, pbq = case
    w = inputs.Workload("t", "encdec", B, N, H, D, M, "bf16")
    x = inputs.make_encdec(w, seed=N + 3 * M, q_mult=qm, per_batch_q=pbq)
    g = inputs.normal_tensor((B, N, H, D), "bf16", seed=N + M + 7)
    return x, g


def _dev_view(t, layout):
    """[B, N, H, D] CPU tensor -> device [B, H, N, D] view in the given layout."""
    if layout == "head":
        return hm(t).contiguous().to(DEV)
    return hm(t.to(DEV))


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "B{}H{}N{}D{}M{}-q{}-{}-pb{}".format(*c))
def test_decode_backward(case):
    B, H, N, D, M, qm, layout, pbq = case
    say(f"case {case}")
    x, dy_t = _bwd_inputs(case)
    q = x["q"].to(DEV)
    k = _dev_view(x["k"], layout)
    zr = inputs.normal_tensor((B, H, M, D), "bf16", seed=M + 11)  # any latent values
    z = zr.to(DEV)
    dy = _dev_view(dy_t, layout)
    y, lse = rl.flare_decode(k, q, z, want_lse=True)
    dk, dq, dz = rl.flare_decode_backward(k, q, z, y, lse, dy)
    torch.cuda.synchronize()
    dkr, dqr, dzr = oracle.decode_backward(f64(hm(x["k"])), f64(x["q"]), f64(zr), f64(hm(dy_t)))
    check_grad(f64(dk), dkr, "dK (decoder)", dzr)
    check_grad(f64(dq), dqr, "dQ (decoder)", dzr)
    check_bf16(f64(dz), dzr, "dZ (decoder)")


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "B{}H{}N{}D{}M{}-q{}-{}-pb{}".format(*c))
def test_encode_backward(case):
    B, H, N, D, M, qm, layout, pbq = case
    say(f"case {case}")
    x, _ = _bwd_inputs(case)
    q = x["q"].to(DEV)
    k, v = _dev_view(x["k"], layout), _dev_view(x["v"], layout)
    z, lse = rl.flare_encode(q, k, v, want_lse=True, z_dtype=torch.float32)
    dz = inputs.normal_tensor((B, H, M, D), "f32", seed=M + 5).to(DEV)
    dq, dk, dv = rl.flare_encode_backward(q, k, v, z, lse, dz)
    torch.cuda.synchronize()
    dqr, dkr, dvr = oracle.encode_backward(f64(x["q"]), f64(hm(x["k"])), f64(hm(x["v"])), f64(dz))
    check_grad(f64(dq), dqr, "dQ (encoder)", dvr)
    check_grad(f64(dk), dkr, "dK (encoder)", dvr)
    check_bf16(f64(dv), dvr, "dV (encoder)")


@pytest.mark.parametrize("case", BWD_CASES[:5], ids=lambda c: "B{}H{}N{}D{}M{}-q{}-{}-pb{}".format(*c))
def test_flare_backward_chain(case):
    # the chain rule through both calls: decoder gradient first (its dZ drives
    # the encoder's), the encoder's dQ and dK accumulated onto the decoder's
    B, H, N, D, M, qm, layout, pbq = case
    say(f"case {case}")
    x, dy_t = _bwd_inputs(case)
    q = x["q"].to(DEV)
    k, v = _dev_view(x["k"], layout), _dev_view(x["v"], layout)
    dy = _dev_view(dy_t, layout)
    z, lse_e = rl.flare_encode(q, k, v, want_lse=True, z_dtype=torch.float32)
    y, lse_d = rl.flare_decode(k, q, z, want_lse=True)
    dk, dq, dz = rl.flare_decode_backward(k, q, z, y, lse_d, dy)
    dq, dk, dv = rl.flare_encode_backward(q, k, v, z, lse_e, dz, dq=dq, dk=dk,
                                          flags=rl.FLARE_ACCUMULATE_DQ | rl.FLARE_ACCUMULATE_DK)
    torch.cuda.synchronize()
    dqr, dkr, dvr = oracle.flare_encdec_backward(f64(x["q"]), f64(hm(x["k"])), f64(hm(x["v"])),
                                                 f64(hm(dy_t)))
    check_bf16(f64(dq), dqr, "dQ")
    check_bf16(f64(dk), dkr, "dK")
    check_bf16(f64(dv), dvr, "dV")


PAIR_CASES = BWD_CASES + [(2, 2, 900, 32, 300, 2.0, "head", False), (1, 2, 700, 16, 512, 4.0, "token", True)]


@pytest.mark.parametrize("case", PAIR_CASES, ids=lambda c: "B{}H{}N{}D{}M{}-q{}-{}-pb{}".format(*c))
def test_flare_pair_backward(case):
    # flare_encdec_backward: the whole FLARE pair's gradient in one call (a
    # shared token pass for M <= 256, the two calls above that)
    B, H, N, D, M, qm, layout, pbq = case
    say(f"case {case}")
    x, dy_t = _bwd_inputs(case)
    q = x["q"].to(DEV)
    k, v = _dev_view(x["k"], layout), _dev_view(x["v"], layout)
    dy = _dev_view(dy_t, layout)
    z, lse_e = rl.flare_encode(q, k, v, want_lse=True, z_dtype=torch.float32)
    y, lse_d = rl.flare_decode(k, q, z, want_lse=True)
    dq, dk, dv = rl.flare_encdec_backward(q, k, v, z, lse_e, y, lse_d, dy)
    torch.cuda.synchronize()
    dqr, dkr, dvr = oracle.flare_encdec_backward(f64(x["q"]), f64(hm(x["k"])), f64(hm(x["v"])),
                                                 f64(hm(dy_t)))
    check_grad(f64(dq), dqr, "dQ", dvr)
    check_grad(f64(dk), dkr, "dK", dvr)
    check_bf16(f64(dv), dvr, "dV")


@pytest.mark.parametrize("M", [64, 320])
def test_flare_pair_backward_flags(M):
    # batch-summed dQ for shared queries, and accumulation into given dQ / dK
    B, H, N, D = 3, 2, 1200, 32
    w = inputs.Workload("t", "encdec", B, N, H, D, M, "bf16")
    x = inputs.make_encdec(w, seed=M, q_mult=3.0)
    dy_t = inputs.normal_tensor((B, N, H, D), "bf16", seed=M + 1)
    q = x["q"].to(DEV)
    k, v, dy = hm(x["k"]).contiguous().to(DEV), hm(x["v"]).contiguous().to(DEV), hm(dy_t).contiguous().to(DEV)
    z, lse_e = rl.flare_encode(q, k, v, want_lse=True, z_dtype=torch.float32)
    y, lse_d = rl.flare_decode(k, q, z, want_lse=True)
    dq0 = inputs.normal_tensor((H, M, D), "f32", seed=5).to(DEV)
    dk0 = inputs.normal_tensor((B, H, N, D), "f32", seed=6).to(DEV)
    dq, dk = dq0.clone(), dk0.clone()
    rl.flare_encdec_backward(q, k, v, z, lse_e, y, lse_d, dy, dq=dq, dk=dk,
                             flags=rl.FLARE_SUM_DQ_OVER_BATCH | rl.FLARE_ACCUMULATE_DQ | rl.FLARE_ACCUMULATE_DK)
    torch.cuda.synchronize()
    dqr, dkr, _ = oracle.flare_encdec_backward(f64(x["q"]), f64(hm(x["k"])), f64(hm(x["v"])), f64(hm(dy_t)))
    check_bf16(f64(dq) - f64(dq0), dqr.sum(0), "dQ added, summed over the batch")
    check_bf16(f64(dk) - f64(dk0), dkr, "dK added")


@pytest.mark.parametrize("case", [(2, 3, 777, 32, 200, 4.0, "token", False),
                                  (3, 2, 1500, 16, 40, 2.0, "head", False)],
                         ids=lambda c: "B{}H{}N{}D{}M{}-q{}-{}".format(*c[:7]))
def test_flare_backward_shared_queries(case):
    # FLARE's learned queries are shared by the batch: both calls sum their dQ
    # over b in the split reduction, the encoder's onto the decoder's
    B, H, N, D, M, qm, layout, _ = case
    say(f"case {case}")
    x, dy_t = _bwd_inputs(case)
    q = x["q"].to(DEV)
    assert q.dim() == 3
    k, v = _dev_view(x["k"], layout), _dev_view(x["v"], layout)
    dy = _dev_view(dy_t, layout)
    z, lse_e = rl.flare_encode(q, k, v, want_lse=True, z_dtype=torch.float32)
    y, lse_d = rl.flare_decode(k, q, z, want_lse=True)
    dk, dq, dz = rl.flare_decode_backward(k, q, z, y, lse_d, dy, flags=rl.FLARE_SUM_DQ_OVER_BATCH)
    assert tuple(dq.shape) == (H, M, D)
    dq, dk, dv = rl.flare_encode_backward(
        q, k, v, z, lse_e, dz, dq=dq, dk=dk,
        flags=rl.FLARE_ACCUMULATE_DQ | rl.FLARE_ACCUMULATE_DK | rl.FLARE_SUM_DQ_OVER_BATCH)
    torch.cuda.synchronize()
    dqr, dkr, dvr = oracle.flare_encdec_backward(f64(x["q"]), f64(hm(x["k"])), f64(hm(x["v"])),
                                                 f64(hm(dy_t)))
    check_bf16(f64(dq), dqr.sum(0), "dQ (summed over the batch)")
    check_bf16(f64(dk), dkr, "dK")
    check_bf16(f64(dv), dvr, "dV")


@pytest.mark.parametrize("B,H,N,D,M,qm", [(2, 2, 1000, 32, 64, 2.0), (3, 1, 700, 16, 40, 4.0),
                                          (1, 2, 4096, 32, 128, 1.0)])
def test_flarepp_backward_chain(B, H, N, D, M, qm):
    # FLARE++ end to end: synthesis Q(X) = SDPA(seeds, eK, eV), encode and
    # decode with Q(X), then the three backward calls in reverse order; the
    # seeds' gradient is summed over the batch
    say(f"case B{B} H{H} N{N} D{D} M{M} q{qm}")
    w = inputs.Workload("t", "encdec", B, N, H, D, M, "bf16")
    x = inputs.make_encdec(w, seed=N + M, q_mult=qm, synth=True)
    dy_t = inputs.normal_tensor((B, N, H, D), "bf16", seed=N + 2 * M)
    seeds = x["seeds"].to(DEV)
    ek, ev = hm(x["ek"]).contiguous().to(DEV), hm(x["ev"]).contiguous().to(DEV)
    k, v = hm(x["k"]).contiguous().to(DEV), hm(x["v"]).contiguous().to(DEV)
    dy = hm(dy_t).contiguous().to(DEV)
    qx, lse_s = rl.flare_route_queries(seeds, ek, ev, want_lse=True)
    z, lse_e = rl.flare_encode(qx, k, v, want_lse=True, z_dtype=torch.float32)
    y, lse_d = rl.flare_decode(k, qx, z, want_lse=True)
    dk, dqx, dz = rl.flare_decode_backward(k, qx, z, y, lse_d, dy)
    dqx, dk, dv = rl.flare_encode_backward(qx, k, v, z, lse_e, dz, dq=dqx, dk=dk,
                                           flags=rl.FLARE_ACCUMULATE_DQ | rl.FLARE_ACCUMULATE_DK)
    dseeds, dek, dev = rl.flare_encode_backward(seeds, ek, ev, qx, lse_s, dqx,
                                                flags=rl.FLARE_SUM_DQ_OVER_BATCH)
    torch.cuda.synchronize()
    ref = oracle.flarepp_backward(f64(x["seeds"]), f64(hm(x["ek"])), f64(hm(x["ev"])),
                                  f64(hm(x["k"])), f64(hm(x["v"])), f64(hm(dy_t)))
    for got, r, what in zip((dseeds, dek, dev, dk, dv), ref, ("dseeds", "deK", "deV", "dK", "dV")):
        check_bf16(f64(got), r, what)


def test_backward_metric_workload_full_size_one_head():
    # The backward of the FLARE pair at N = 1,048,576, H=8, D=32, M=256 (bf16),
    # in the calls and launch configuration the benchmark times (decoder
    # backward, then encoder backward accumulating dQ and dK).  The oracle's
    # chain rule runs on head 3 over all tokens (about 15-30 s of fp64 work);
    # the head's dQ, and its dK and dV for every token, are compared.
    w = inputs.WORKLOADS["encdec_bf16_n1m"]
    x = inputs.make_encdec(w, seed=0)
    dy_t = inputs.normal_tensor((w.B, w.N, w.H, w.D), "bf16", seed=77)
    q = x["q"].to(DEV)
    k = hm(x["k"]).contiguous().to(DEV)
    v = hm(x["v"]).contiguous().to(DEV)
    dy = hm(dy_t).contiguous().to(DEV)
    z, lse_e = rl.flare_encode(q, k, v, want_lse=True, z_dtype=torch.float32)
    y, lse_d = rl.flare_decode(k, q, z, want_lse=True)
    dk, dq, dz = rl.flare_decode_backward(k, q, z, y, lse_d, dy)
    dq, dk, dv = rl.flare_encode_backward(q, k, v, z, lse_e, dz, dq=dq, dk=dk,
                                          flags=rl.FLARE_ACCUMULATE_DQ | rl.FLARE_ACCUMULATE_DK)
    torch.cuda.synchronize()
    h = 3
    say("oracle: chain-rule gradients of head 3 over all tokens")
    dqr, dkr, dvr = oracle.flare_encdec_backward(f64(x["q"][h:h + 1]), f64(hm(x["k"][:, :, h:h + 1])),
                                                 f64(hm(x["v"][:, :, h:h + 1])), f64(hm(dy_t[:, :, h:h + 1])))
    check_bf16(f64(dq[:, h:h + 1]), dqr, "dQ head 3")
    check_bf16(f64(dk[:, h:h + 1]), dkr, "dK head 3")
    check_bf16(f64(dv[:, h:h + 1]), dvr, "dV head 3")


def _sweep_cases(count=12, seed=2024):
    """Seeded random shapes: ragged N, M on and off the 32-latent chunk, both
    head dims and layouts, shared or per-batch queries, mild to sharp scores."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        B, H = int(rng.integers(1, 4)), int(rng.choice([1, 2, 3, 5]))
        D = int(rng.choice([16, 32]))
        M = int(rng.choice([1, 2, 31, 32, 33, 63, 100, 255, 256, 257, 384, 511, 512]))
        N = int(rng.integers(1, 6000))
        if B * H * N * M > 2e7:
            continue
        layout = str(rng.choice(["head", "token"]))
        qm = float(rng.choice([0.5, 1.0, 3.0, 10.0]))
        pbq = bool(rng.integers(0, 2))
        out.append((B, H, N, D, M, layout, qm, pbq))
    return out


@pytest.mark.parametrize("case", _sweep_cases(), ids=lambda c: "B{}H{}N{}D{}M{}-{}-q{}-pb{}".format(*c))
def test_sweep_forward_and_pair_backward(case):
    # forward (encode, decode) and the pair's gradient on seeded random shapes
    B, H, N, D, M, layout, qm, pbq = case
    say(f"case {case}")
    w = inputs.Workload("t", "encdec", B, N, H, D, M, "bf16")
    x = inputs.make_encdec(w, seed=7 * N + M, q_mult=qm, per_batch_q=pbq)
    dy_t = inputs.normal_tensor((B, N, H, D), "bf16", seed=N + 3)
    q = x["q"].to(DEV)
    k, v, dy = _dev_view(x["k"], layout), _dev_view(x["v"], layout), _dev_view(dy_t, layout)
    z, lse_e = rl.flare_encode(q, k, v, want_lse=True, z_dtype=torch.float32)
    y, lse_d = rl.flare_decode(k, q, z, want_lse=True)
    dq, dk, dv = rl.flare_encdec_backward(q, k, v, z, lse_e, y, lse_d, dy)
    torch.cuda.synchronize()
    qo, ko, vo = f64(x["q"]), f64(hm(x["k"])), f64(hm(x["v"]))
    zr, _ = oracle.encode(qo, ko, vo)
    check_bf16(f64(z), zr, "Z")
    check_bf16(f64(y), oracle.decode(ko, qo, zr), "Y")
    dqr, dkr, dvr = oracle.flare_encdec_backward(qo, ko, vo, f64(hm(dy_t)))
    check_grad(f64(dq), dqr, "dQ", dvr)
    check_grad(f64(dk), dkr, "dK", dvr)
    check_bf16(f64(dv), dvr, "dV")


@pytest.mark.parametrize("D,M", [(32, 40), (16, 300)])
def test_negative_scale_forward_and_backward(D, M):
    # a negative softmax scale is legal SDPA (weights favour the lowest
    # scores); padded rows and ragged tokens must still get weight 0
    B, H, N, scale = 2, 2, 777, -0.3
    w = inputs.Workload("t", "encdec", B, N, H, D, M, "bf16")
    x = inputs.make_encdec(w, seed=M + 1, q_mult=3.0)
    dy_t = inputs.normal_tensor((B, N, H, D), "bf16", seed=M + 2)
    q = x["q"].to(DEV)
    k, v, dy = hm(x["k"]).contiguous().to(DEV), hm(x["v"]).contiguous().to(DEV), hm(dy_t).contiguous().to(DEV)
    z, lse_e = rl.flare_encode(q, k, v, want_lse=True, z_dtype=torch.float32, scale=scale)
    y, lse_d = rl.flare_decode(k, q, z, want_lse=True, scale=scale)
    dq, dk, dv = rl.flare_encdec_backward(q, k, v, z, lse_e, y, lse_d, dy, scale=scale)
    dk1, dq1, dz1 = rl.flare_decode_backward(k, q, z, y, lse_d, dy, scale=scale)
    dq1, dk1, dv1 = rl.flare_encode_backward(q, k, v, z, lse_e, dz1, dq=dq1, dk=dk1, scale=scale,
                                             flags=rl.FLARE_ACCUMULATE_DQ | rl.FLARE_ACCUMULATE_DK)
    torch.cuda.synchronize()
    qo, ko, vo = f64(x["q"]), f64(hm(x["k"])), f64(hm(x["v"]))
    zr, _ = oracle.encode(qo, ko, vo, scale)
    check_bf16(f64(z), zr, "Z")
    check_bf16(f64(y), oracle.decode(ko, qo, zr, scale), "Y")
    dqr, dkr, dvr = oracle.flare_encdec_backward(qo, ko, vo, f64(hm(dy_t)), scale)
    for tag, (a, b_, c_) in (("one call", (dq, dk, dv)), ("two calls", (dq1, dk1, dv1))):
        check_bf16(f64(a), dqr, f"dQ ({tag})")
        check_bf16(f64(b_), dkr, f"dK ({tag})")
        check_bf16(f64(c_), dvr, f"dV ({tag})")


def test_pair_backward_token_major_gradients():
    # dK, dV written into token-major [B, N, H, D] fp32 views (strided per head),
    # through the one-call and the two-call backward
    B, H, N, D, M = 2, 3, 1100, 32, 96
    w = inputs.Workload("t", "encdec", B, N, H, D, M, "bf16")
    x = inputs.make_encdec(w, seed=31, q_mult=2.0)
    dy_t = inputs.normal_tensor((B, N, H, D), "bf16", seed=32)
    q = x["q"].to(DEV)
    k, v, dy = hm(x["k"].to(DEV)), hm(x["v"].to(DEV)), hm(dy_t.to(DEV))
    z, lse_e = rl.flare_encode(q, k, v, want_lse=True, z_dtype=torch.float32)
    y, lse_d = rl.flare_decode(k, q, z, want_lse=True)
    tm = lambda: hm(torch.full((B, N, H, D), float("nan"), dtype=torch.float32, device=DEV))
    dk, dv = tm(), tm()
    dq, _, _ = rl.flare_encdec_backward(q, k, v, z, lse_e, y, lse_d, dy, dk=dk, dv=dv)
    dk2, dv2 = tm(), tm()
    _, dq2, dz2 = rl.flare_decode_backward(k, q, z, y, lse_d, dy, dk=dk2)
    dq2, _, _ = rl.flare_encode_backward(q, k, v, z, lse_e, dz2, dq=dq2, dk=dk2, dv=dv2,
                                         flags=rl.FLARE_ACCUMULATE_DQ | rl.FLARE_ACCUMULATE_DK)
    torch.cuda.synchronize()
    dqr, dkr, dvr = oracle.flare_encdec_backward(f64(x["q"]), f64(hm(x["k"])), f64(hm(x["v"])),
                                                 f64(hm(dy_t)))
    for tag, (a, b_, c_) in (("one call", (dq, dk, dv)), ("two calls", (dq2, dk2, dv2))):
        check_bf16(f64(a), dqr, f"dQ ({tag})")
        check_bf16(f64(b_), dkr, f"dK ({tag})")
        check_bf16(f64(c_), dvr, f"dV ({tag})")


def test_padded_strides_forward_and_backward():
    # Every tensor a view into a larger buffer: token rows padded (row stride
    # H*48 elements for D = 32, batch stride with 3 spare rows), latent rows
    # padded to 40.  Padding that is read holds NaN, so a kernel that used it
    # would fail; padding of outputs holds a sentinel that must survive.
    B, H, N, D, M = 2, 3, 900, 32, 72
    w = inputs.Workload("t", "encdec", B, N, H, D, M, "bf16")
    x = inputs.make_encdec(w, seed=41, q_mult=3.0)
    dy_t = inputs.normal_tensor((B, N, H, D), "bf16", seed=42)

    def tok_in(t):
        buf = torch.full((B, N + 3, H, 48), float("nan"), dtype=t.dtype, device=DEV)
        buf[:, :N, :, :D] = t.to(DEV)
        return hm(buf[:, :N, :, :D])

    def tok_out(dtype):
        buf = torch.full((B, N + 3, H, 48), 12345.0, dtype=dtype, device=DEV)
        return buf, hm(buf[:, :N, :, :D])

    def lat_out():
        buf = torch.full((B, H, M, 40), 12345.0, dtype=torch.float32, device=DEV)
        return buf, buf[..., :D]

    qbuf = torch.full((H, M, 40), float("nan"), dtype=torch.bfloat16, device=DEV)
    qbuf[..., :D] = x["q"].to(DEV)
    q = qbuf[..., :D]
    k, v, dy = tok_in(x["k"]), tok_in(x["v"]), tok_in(dy_t)
    zbuf, z = lat_out()
    z, lse_e = rl.flare_encode(q, k, v, z=z, want_lse=True)
    ybuf, y = tok_out(torch.bfloat16)
    y, lse_d = rl.flare_decode(k, q, z, y=y, want_lse=True)
    dkb, dk = tok_out(torch.float32)
    dvb, dv = tok_out(torch.float32)
    dq, _, _ = rl.flare_encdec_backward(q, k, v, z, lse_e, y, lse_d, dy, dk=dk, dv=dv)
    dkb2, dk2 = tok_out(torch.float32)
    dvb2, dv2 = tok_out(torch.float32)
    _, dq2, dz = rl.flare_decode_backward(k, q, z, y, lse_d, dy, dk=dk2)
    dq2, _, _ = rl.flare_encode_backward(q, k, v, z, lse_e, dz, dq=dq2, dk=dk2, dv=dv2,
                                         flags=rl.FLARE_ACCUMULATE_DQ | rl.FLARE_ACCUMULATE_DK)
    torch.cuda.synchronize()
    qo, ko, vo = f64(x["q"]), f64(hm(x["k"])), f64(hm(x["v"]))
    zr, _ = oracle.encode(qo, ko, vo)
    check_bf16(f64(z), zr, "Z (padded views)")
    check_bf16(f64(y), oracle.decode(ko, qo, f64(z)), "Y (padded views)")
    dqr, dkr, dvr = oracle.flare_encdec_backward(qo, ko, vo, f64(hm(dy_t)))
    for tag, (a, b_, c_) in (("one call", (dq, dk, dv)), ("two calls", (dq2, dk2, dv2))):
        check_bf16(f64(a), dqr, f"dQ ({tag}, padded views)")
        check_bf16(f64(b_), dkr, f"dK ({tag}, padded views)")
        check_bf16(f64(c_), dvr, f"dV ({tag}, padded views)")
    for name, buf in (("Y", ybuf), ("dK", dkb), ("dV", dvb), ("dK2", dkb2), ("dV2", dvb2)):
        assert torch.all(buf[:, :N, :, D:] == 12345.0), name
        assert torch.all(buf[:, N:] == 12345.0), name
    assert torch.all(zbuf[..., D:] == 12345.0), "Z"


def test_concurrent_calls_on_two_streams():
    # The library holds no mutable state: two different workloads issued on
    # two streams at once, each with its own workspace, give the results each
    # gives alone (bit for bit: same kernels, same launch shapes).
    def setup(B, H, N, D, M, seed):
        w = inputs.Workload("t", "encdec", B, N, H, D, M, "bf16")
        x = inputs.make_encdec(w, seed=seed, q_mult=3.0)
        dy = hm(inputs.normal_tensor((B, N, H, D), "bf16", seed=seed + 1)).contiguous().to(DEV)
        return x["q"].to(DEV), hm(x["k"]).contiguous().to(DEV), hm(x["v"]).contiguous().to(DEV), dy

    cases = [setup(2, 4, 20000, 32, 128, 51), setup(1, 3, 30000, 16, 300, 52)]
    # workspaces live until the end: a stream may still use one after the call returns
    wss = []
    for q, k, _, _ in cases:
        B, H, N, D = k.shape
        M = q.shape[-2]
        wss.append((torch.empty(rl.encode_workspace_size(B, H, M, N, D), dtype=torch.uint8, device=DEV),
                    torch.empty(rl.lib().flare_encdec_backward_workspace_size(B, H, M, N, D), dtype=torch.uint8,
                                device=DEV)))

    def run(i, stream):
        q, k, v, dy = cases[i]
        ws, wsb = wss[i]
        with torch.cuda.stream(stream):
            z, le = rl.flare_encode(q, k, v, want_lse=True, z_dtype=torch.float32, workspace=ws, stream=stream)
            y, ld = rl.flare_decode(k, q, z, want_lse=True, stream=stream)
            dq, dk, dv = rl.flare_encdec_backward(q, k, v, z, le, y, ld, dy, workspace=wsb, stream=stream)
        return z, y, dq, dk, dv

    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    alone = []
    for i in range(2):
        alone.append(run(i, s1))
        torch.cuda.synchronize()
    a = run(0, s1)
    b = run(1, s2)
    torch.cuda.synchronize()
    for ref, got in zip(alone, (a, b)):
        for r_, g_ in zip(ref, got):
            assert torch.equal(r_, g_)
    say("  two streams: both workloads equal to their runs alone")


def test_largest_batch_times_heads():
    # B * H = 65535, the largest grid the calls accept (one workgroup row per
    # batch*head), with a ragged handful of tokens and latents per head:
    # forward and the one-call backward against the oracle.
    B, H, N, D, M = 255, 257, 5, 16, 3
    w = inputs.Workload("t", "encdec", B, N, H, D, M, "bf16")
    x = inputs.make_encdec(w, seed=61, q_mult=2.0, per_batch_q=True)
    dy_t = inputs.normal_tensor((B, N, H, D), "bf16", seed=62)
    q = x["q"].to(DEV)
    k, v, dy = hm(x["k"]).contiguous().to(DEV), hm(x["v"]).contiguous().to(DEV), hm(dy_t).contiguous().to(DEV)
    z, le = rl.flare_encode(q, k, v, want_lse=True, z_dtype=torch.float32)
    y, ld = rl.flare_decode(k, q, z, want_lse=True)
    dq, dk, dv = rl.flare_encdec_backward(q, k, v, z, le, y, ld, dy)
    torch.cuda.synchronize()
    qo, ko, vo = f64(x["q"]), f64(hm(x["k"])), f64(hm(x["v"]))
    zr, _ = oracle.encode(qo, ko, vo)
    check_bf16(f64(z), zr, "Z (B*H = 65535)")
    check_bf16(f64(y), oracle.decode(ko, qo, f64(z)), "Y (B*H = 65535)")
    dqr, dkr, dvr = oracle.flare_encdec_backward(qo, ko, vo, f64(hm(dy_t)))
    check_bf16(f64(dq), dqr, "dQ (B*H = 65535)")
    check_bf16(f64(dk), dkr, "dK (B*H = 65535)")
    check_bf16(f64(dv), dvr, "dV (B*H = 65535)")


@pytest.mark.parametrize("case", ["zero_queries", "equal_keys", "zero_values"])
def test_degenerate_inputs(case):
    # Degenerate cases of the method, forward and one-call backward:
    # zero queries (every score 0: uniform weights in both calls), every key
    # equal (the encoder weights every token alike, so Z is the mean of V),
    # zero values (Z = 0, so Y = 0 and every gradient through Z vanishes).
    B, H, N, D, M = 2, 3, 1000, 32, 48
    w = inputs.Workload("t", "encdec", B, N, H, D, M, "bf16")
    x = inputs.make_encdec(w, seed=71, q_mult=3.0)
    q, k, v = x["q"].clone(), x["k"].clone(), x["v"].clone()
    if case == "zero_queries":
        q.zero_()
    elif case == "equal_keys":
        k[:] = k[:, :1]
    else:
        v.zero_()
    dy_t = inputs.normal_tensor((B, N, H, D), "bf16", seed=72)
    qd = q.to(DEV)
    kd, vd, dy = hm(k).contiguous().to(DEV), hm(v).contiguous().to(DEV), hm(dy_t).contiguous().to(DEV)
    z, le = rl.flare_encode(qd, kd, vd, want_lse=True, z_dtype=torch.float32)
    y, ld = rl.flare_decode(kd, qd, z, want_lse=True)
    dq, dk, dv = rl.flare_encdec_backward(qd, kd, vd, z, le, y, ld, dy)
    torch.cuda.synchronize()
    qo, ko, vo = f64(q), f64(hm(k)), f64(hm(v))
    zr, _ = oracle.encode(qo, ko, vo)
    yr = oracle.decode(ko, qo, zr)
    dqr, dkr, dvr = oracle.flare_encdec_backward(qo, ko, vo, f64(hm(dy_t)))
    if case == "zero_values":
        # exact zeros: no weight times zero values can be anything but zero
        assert not torch.any(z) and not torch.any(y) and not torch.any(dq) and not torch.any(dk)
        check_bf16(f64(dv), dvr, f"dV ({case})")
        return
    if case == "equal_keys":
        # Z[m] = mean over tokens of V, whatever the query (within bf16 of V's mean)
        np.testing.assert_allclose(zr, np.broadcast_to(vo.mean(axis=2, keepdims=True), zr.shape), atol=1e-12)
    check_bf16(f64(z), zr, f"Z ({case})")
    check_bf16(f64(y), yr, f"Y ({case})")
    for name, got, ref in (("dQ", dq, dqr), ("dK", dk, dkr), ("dV", dv, dvr)):
        nr = float(np.linalg.norm(ref))
        if nr < 1e-9:
            # zero in exact arithmetic: held to 1e-2 of the upstream gradient's scale
            e = float(np.linalg.norm(f64(got))) / float(np.linalg.norm(f64(dy)))
            say(f"  {name} ({case}): zero in exact arithmetic, |got| / |dY| {e:.3e}")
            assert e <= BF16_TOL
        else:
            check_bf16(f64(got), ref, f"{name} ({case})")


@pytest.mark.parametrize("B,H,N,D,M,qm", [(2, 3, 777, 32, 200, 4.0), (1, 2, 1000, 16, 64, 2.0),
                                           (1, 2, 900, 32, 300, 3.0)])
def test_backward_bf16_gradients(B, H, N, D, M, qm):
    # dK, dV written in bf16 (formed in fp32, rounded once; accumulation in
    # the two-call chain, and over the 256-latent blocks at M = 300, adds in
    # fp32 before rounding): against the oracle at the bf16 bar, and against
    # the same calls' fp32 gradients within a few bf16 roundings
    w = inputs.Workload("t", "encdec", B, N, H, D, M, "bf16")
    x = inputs.make_encdec(w, seed=N + M, q_mult=qm)
    dy_t = inputs.normal_tensor((B, N, H, D), "bf16", seed=N + 1)
    q = x["q"].to(DEV)
    k, v, dy = hm(x["k"]).contiguous().to(DEV), hm(x["v"]).contiguous().to(DEV), hm(dy_t).contiguous().to(DEV)
    z, le = rl.flare_encode(q, k, v, want_lse=True, z_dtype=torch.float32)
    y, ld = rl.flare_decode(k, q, z, want_lse=True)
    acc = rl.FLARE_ACCUMULATE_DQ | rl.FLARE_ACCUMULATE_DK
    res = {}
    for gd in (torch.float32, torch.bfloat16):
        one = rl.flare_encdec_backward(q, k, v, z, le, y, ld, dy, grad_dtype=gd)
        dk2, dq2, dz2 = rl.flare_decode_backward(k, q, z, y, ld, dy, grad_dtype=gd)
        two = rl.flare_encode_backward(q, k, v, z, le, dz2, dq=dq2, dk=dk2, flags=acc, grad_dtype=gd)
        res[gd] = (one, two)
    torch.cuda.synchronize()
    dqr, dkr, dvr = oracle.flare_encdec_backward(f64(x["q"]), f64(hm(x["k"])), f64(hm(x["v"])), f64(hm(dy_t)))
    for form in (0, 1):
        tag = ("one call", "two calls")[form]
        g16, g32 = res[torch.bfloat16][form], res[torch.float32][form]
        assert g16[1].dtype == torch.bfloat16 and g16[2].dtype == torch.bfloat16
        for name, i, ref in (("dQ", 0, dqr), ("dK", 1, dkr), ("dV", 2, dvr)):
            check_bf16(f64(g16[i]), ref, f"{name} ({tag}, bf16 gradients)")
        for name, i in (("dK", 1), ("dV", 2)):
            e = rel_l2(f64(g16[i]), f64(g32[i]))
            say(f"  {name} ({tag}): bf16 against fp32 gradients rel-L2 {e:.2e}")
            assert e <= 6e-3


def test_graph_capture_replays_match_eager():
    # flare_mix (FLARE++, B=8, N=4096, C=128, M=64) and the pair backward
    # captured into HIP graphs: the library issues only kernel launches on the
    # caller's stream (no memset, allocation or synchronisation), so every
    # replay, with eager work and synchronisations between replays, must equal
    # the eager result bit for bit
    w = inputs.WORKLOADS["mix_bf16_n4k_c128"]
    m = inputs.make_mix(w, seed=3, q_mult=4.0)
    g = {n: t.to(DEV) for n, t in m.items()}
    B, N, C, H, M = w.B, w.N, w.C, w.H, w.M
    out = torch.empty_like(g["x"])
    ws = torch.empty(rl.mix_workspace_size(B, N, C, H, M, True, False), dtype=torch.uint8, device=DEV)
    mix = lambda s: rl.flare_mix(g["x"], g["w_k"], g["w_v"], g["qs"], H, w_ek=g["w_ek"], w_ev=g["w_ev"],
                                 out=out, workspace=ws, stream=s)
    D = C // H
    e = inputs.make_encdec(inputs.Workload("t", "encdec", 2, 3000, 4, 32, 100, "bf16"), seed=5, q_mult=2.0)
    q = e["q"].to(DEV)
    k, v = hm(e["k"]).contiguous().to(DEV), hm(e["v"]).contiguous().to(DEV)
    dy = hm(inputs.normal_tensor((2, 3000, 4, 32), "bf16", seed=6)).contiguous().to(DEV)
    z, lse_e = rl.flare_encode(q, k, v, want_lse=True, z_dtype=torch.float32)
    y, lse_d = rl.flare_decode(k, q, z, want_lse=True)
    dq = torch.empty((4, 100, 32), dtype=torch.float32, device=DEV)
    dk = torch.empty((2, 4, 3000, 32), dtype=torch.float32, device=DEV)
    dv = torch.empty_like(dk)
    wsb = torch.empty(rl.lib().flare_encdec_backward_workspace_size(2, 4, 100, 3000, 32), dtype=torch.uint8,
                      device=DEV)
    bwd = lambda s: rl.flare_encdec_backward(q, k, v, z, lse_e, y, lse_d, dy, dq=dq, dk=dk, dv=dv,
                                             flags=rl.FLARE_SUM_DQ_OVER_BATCH, workspace=wsb, stream=s)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        mix(stream)
        bwd(stream)
    torch.cuda.synchronize()
    ref = [out.clone(), dq.clone(), dk.clone(), dv.clone()]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        mix(stream)
        bwd(stream)
    for i in range(4):
        for t in (out, dq, dk, dv):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [out, dq, dk, dv]
        for r, gt, name in zip(ref, got, ("out", "dQ", "dK", "dV")):
            assert torch.equal(r, gt), (i, name)
        _ = (g["x"].float() * 2).sum().item()  # eager work between replays
    say(f"  4 replays equal to the eager run (D={D})")


@pytest.mark.parametrize("qm,flags", [(40.0, 0), (3.0, EXACT)])
def test_backward_after_exact_forward(qm, flags):
    # scores far outside the range-checked fast softmax (queries x40: exponents
    # in the hundreds) send the forward calls through their exact
    # running-maximum path, whose normalisers the backward then uses; the
    # same with the exact path forced on ordinary scores
    B, H, N, D, M = 1, 2, 2000, 32, 64
    w = inputs.Workload("t", "encdec", B, N, H, D, M, "bf16")
    x = inputs.make_encdec(w, seed=41, q_mult=qm)
    dy_t = inputs.normal_tensor((B, N, H, D), "bf16", seed=42)
    q = x["q"].to(DEV)
    k, v, dy = hm(x["k"]).contiguous().to(DEV), hm(x["v"]).contiguous().to(DEV), hm(dy_t).contiguous().to(DEV)
    z, lse_e = rl.flare_encode(q, k, v, want_lse=True, z_dtype=torch.float32, flags=flags)
    y, lse_d = rl.flare_decode(k, q, z, want_lse=True, flags=flags)
    dq, dk, dv = rl.flare_encdec_backward(q, k, v, z, lse_e, y, lse_d, dy)
    torch.cuda.synchronize()
    qo, ko, vo = f64(x["q"]), f64(hm(x["k"])), f64(hm(x["v"]))
    zr, lr = oracle.encode(qo, ko, vo)
    check_bf16(f64(z), zr, "Z")
    yr = oracle.decode(ko, qo, zr)
    check_bf16(f64(y), yr, "Y")
    _, ld = oracle.sdpa(ko[0, 0], qo[0], zr[0, 0], return_lse=True)
    el = float(np.max(np.abs(f64(lse_d)[0, 0] - ld)))
    say(f"  decoder lse (head 0): max abs err {el:.3e}, max |lse| {np.max(np.abs(ld)):.1f}")
    assert el <= 1e-2 * max(1.0, float(np.max(np.abs(ld))))
    dqr, dkr, dvr = oracle.flare_encdec_backward(qo, ko, vo, f64(hm(dy_t)))
    check_grad(f64(dq), dqr, "dQ", dvr)
    check_grad(f64(dk), dkr, "dK", dvr)
    check_bf16(f64(dv), dvr, "dV")


# ------------------------------------------------ fast softmax acceptance range
# The first pass of the encoder forms weights 2^x with no running maximum and
# keeps a split when every latent's normaliser l (a sum of n weights) lies in
# [n 2^-102, 2^100].  The exponential returns 0 for results below 2^-126, so
# a split whose weights mostly fall just below that threshold loses up to
# n 2^-126 of its mass; the lower end scales with n so that this loss stays
# below fp32 rounding and any split beyond it is recomputed exactly.

def _flush_band_inputs(N, H, D, M):
    """One head-major block [1, H, N, D] of keys and values and [H, M, D]
    queries.  With scale ln 2 (base-2 scores s = q.k), latents j < 4 score
    every token but the last one at s = -126.125 - 0.125 j (weights just below
    the flush threshold) and the last token at s = -99.875 + 0.125 j.  Those
    latents weigh only features 0..3 of the keys, where the bulk tokens hold
    (1, 0, 1, 0) and the last one (0, 1, 0, 1); features 4.. of the bulk keys,
    the other latents and the values are random, so every other softmax is an
    ordinary one.  The designed scores are exact in bf16 arithmetic.  The bulk
    values have mean zero: a large mean shared by every latent's Z would leave
    the decoder's gradient dependent on differences between Z rows far below
    bf16 resolution (Z enters the decoder's matrix products in bf16)."""
    g = np.random.default_rng(4242)
    k = np.zeros((1, H, N, D), np.float32)
    k[..., :-1, 4:] = g.standard_normal((1, H, N - 1, D - 4), dtype=np.float32)
    k[..., :-1, 0] = 1.0
    k[..., :-1, 2] = 1.0          # bulk tokens: s = q0 + q2
    k[..., -1, 1] = 1.0
    k[..., -1, 3] = 1.0           # last token: s = q1 + q3
    ramp = np.arange(D, dtype=np.float32) / 64.0
    v = np.empty((1, H, N, D), np.float32)
    v[..., :-1, :] = 0.5 * g.standard_normal((1, H, N - 1, D), dtype=np.float32)
    v[..., -1, :] = 1.0 - ramp
    q = (g.standard_normal((H, M, D)) * 0.5).astype(np.float32)
    for j in range(4):
        q[:, j, :] = 0.0
        q[:, j, 0] = -126.0
        q[:, j, 2] = -0.125 * (j + 1)
        q[:, j, 1] = -96.0
        q[:, j, 3] = -3.875 + 0.125 * j
    to = lambda a: torch.from_numpy(a).to(torch.bfloat16)
    return to(q), to(k), to(v)


def test_fast_softmax_long_split_near_flush_threshold():
    # B*H = 1024 gives one split per (batch, head): every workgroup sums all
    # 2^20 tokens.  The batch shares one block of keys and values (stride 0),
    # so all B results equal the oracle's per-head result.
    B, H, N, D, M = 128, 8, 1 << 20, 32, 32
    scale = math.log(2.0)
    qt, kt, vt = _flush_band_inputs(N, H, D, M)
    parts = B * H * 1 * M
    ws_one_split = (parts * D * 4 + 255) // 256 * 256 + (parts * 4 + 255) // 256 * 256
    assert rl.encode_workspace_size(B, H, M, N, D) == ws_one_split
    say(f"encode B={B} H={H} N={N} D={D} M={M}, one split per head")
    q = qt.to(DEV)
    k1 = kt.to(DEV)
    v1 = vt.to(DEV)
    k = k1.expand(B, H, N, D)
    v = v1.expand(B, H, N, D)
    z, lse = rl.flare_encode(q, k, v, want_lse=True, scale=scale, z_dtype=torch.float32)
    torch.cuda.synchronize()
    zr, lr = oracle.encode(f64(qt), f64(kt), f64(vt), scale)
    # Every latent within the bf16 bar.  The flush-band latents' weights take
    # two values (bulk and last token), each rounded once to bf16, which moves
    # their ratio r ~ 1e-2 by at most 2^-8 relative: an error near 1e-4 of Z.
    # They are held to 1e-3; flushing the bulk mass unseen would cost r / (1 + r),
    # 0.8 to 1.3 %.
    for b in (0, B - 1):
        for h in range(H):
            for m in range(M):
                e = rel_l2(f64(z[b, h, m]), zr[0, h, m])
                assert e <= (1e-3 if m < 4 else BF16_TOL), (b, h, m, e)
        check_bf16(f64(lse[b]), lr[0], f"lse batch {b}")
    worst = max(rel_l2(f64(z[0, h, j]), zr[0, h, j]) for h in range(H) for j in range(4))
    say(f"  flush-band latents: worst per-latent rel-L2 {worst:.3e}")

    # The backward of the pair on one batch element, from this forward's Z and
    # lse (the encoder's normalisers of the long split), against the oracle's
    # chain rule on heads 0 and 1.
    zb, lseb = z[0:1].contiguous(), lse[0:1].contiguous()
    y, lse_d = rl.flare_decode(k1, q, zb, want_lse=True, scale=scale)
    dy_t = inputs.normal_tensor((1, N, H, D), "bf16", seed=91)
    dy = hm(dy_t).contiguous().to(DEV)
    dq, dk, dv = rl.flare_encdec_backward(q, k1, v1, zb, lseb, y, lse_d, dy, scale=scale)
    torch.cuda.synchronize()
    say("oracle: chain-rule gradients of heads 0 and 1 over all tokens")
    dqr, dkr, dvr = oracle.flare_encdec_backward(f64(qt[0:2]), f64(kt[:, 0:2]), f64(vt[:, 0:2]),
                                                 f64(hm(dy_t)[:, 0:2]), scale)
    check_grad(f64(dq[:, 0:2]), dqr, "dQ heads 0-1", dqr)
    check_grad(f64(dk[:, 0:2]), dkr, "dK heads 0-1", dkr)
    check_grad(f64(dv[:, 0:2]), dvr, "dV heads 0-1", dvr)

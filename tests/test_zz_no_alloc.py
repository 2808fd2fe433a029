"""GPU tier: flare_encode_static (no workspace; split partials in the
library's static per-GPU scratch) against flare_encode through the C ABI.

Two calls in a row, the second with a smaller input than the first, so the
second runs on scratch that still holds the first call's partials.  Where the
encoder's own split plan fits the scratch both entry points run the same
kernels on the same plan, so the results must agree bit for bit; where the
scratch caps the split count, the merged result may differ by rounding and is
held to the bf16 bar (relative L2 <= 1e-2) against flare_encode and against
the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import rank_latent_routing_amd as rl
from rank_latent_routing_amd import binding, inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
BF16_TOL = 1e-2


def f64(t):
    return t.detach().double().cpu().numpy()


def rel_l2(a, b):
    return float(np.linalg.norm((a - b).ravel()) / max(np.linalg.norm(b.ravel()), 1e-300))


def _case(B, H, N, D, M, dtype, seed, qm=2.0):
    w = inputs.Workload("t", "encdec", B, N, H, D, M, dtype)
    x = inputs.make_encdec(w, seed=seed, q_mult=qm)
    q = x["q"].to(DEV)
    k = x["k"].permute(0, 2, 1, 3).contiguous().to(DEV)
    v = x["v"].permute(0, 2, 1, 3).contiguous().to(DEV)
    return x, q, k, v


def _both(q, k, v, flags=0):
    z0, l0 = rl.flare_encode(q, k, v, want_lse=True, z_dtype=torch.float32, flags=flags)
    z1, l1 = binding.flare_encode_static(q, k, v, want_lse=True, z_dtype=torch.float32, flags=flags)
    torch.cuda.synchronize()
    return z0, l0, z1, l1


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_static_encode_equals_workspace_encode_two_calls(dtype):
    print(f"no-alloc encode, {dtype}: large call then smaller call", flush=True)
    # first call: B=2, H=4, N=20000, M=256 (the planner's 78 splits fit the scratch)
    _, q, k, v = _case(2, 4, 20000, 32, 256, dtype, seed=5)
    z0, l0, z1, l1 = _both(q, k, v)
    assert torch.equal(z0, z1) and torch.equal(l0, l1)
    # second call, smaller: B=1, H=2, N=3001, D=16, M=40, sharp queries
    _, q, k, v = _case(1, 2, 3001, 16, 40, dtype, seed=6, qm=8.0)
    z0, l0, z1, l1 = _both(q, k, v)
    assert torch.equal(z0, z1) and torch.equal(l0, l1)
    # and once more with the exact softmax forced
    z0, l0, z1, l1 = _both(q, k, v, flags=rl.FLARE_FLAG_EXACT_SOFTMAX)
    assert torch.equal(z0, z1) and torch.equal(l0, l1)


def test_static_encode_caps_splits_to_fit():
    # B*H = 8, M = 512: the planner's 128 splits need 69 MB of partials, more
    # than the scratch; the static call runs fewer, longer splits.
    print("no-alloc encode: split count capped by the scratch, then a smaller call", flush=True)
    B, H, N, D, M = 2, 4, 40000, 32, 512
    assert rl.encode_workspace_size(B, H, M, N, D) > binding.encode_static_scratch_bytes()
    x, q, k, v = _case(B, H, N, D, M, "bf16", seed=7, qm=4.0)
    z0, l0, z1, l1 = _both(q, k, v)
    assert rel_l2(f64(z1), f64(z0)) <= BF16_TOL
    assert rel_l2(f64(l1), f64(l0)) <= BF16_TOL
    zr, lr = oracle.encode(f64(x["q"]), f64(x["k"].permute(0, 2, 1, 3)), f64(x["v"].permute(0, 2, 1, 3)))
    assert rel_l2(f64(z1), zr) <= BF16_TOL
    assert rel_l2(f64(l1), lr) <= BF16_TOL
    # a smaller call right after (fits without capping): bit-identical again
    _, q, k, v = _case(1, 3, 777, 32, 64, "bf16", seed=8)
    z0, l0, z1, l1 = _both(q, k, v)
    assert torch.equal(z0, z1) and torch.equal(l0, l1)


def test_static_encode_rejects_sizes_beyond_the_scratch():
    # one split per (batch, head) at B*H = 1024, M = 512, D = 32 needs
    # 1024 * 512 * 33 * 4 bytes > 64 MiB: rejected before any launch.
    B, H, N, D, M = 128, 8, 256, 32, 512
    k1 = torch.zeros((1, H, N, D), dtype=torch.bfloat16, device=DEV)
    k = k1.expand(B, H, N, D)
    q = torch.zeros((H, M, D), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(rl.FlareError) as e:
        binding.flare_encode_static(q, k, k, z_dtype=torch.float32)
    assert e.value.status == binding.FLARE_E_SCRATCH

"""Seeded synthetic inputs for the FLARE / FLARE++ mixer.

This module holds only random draws and their shapes: none of the method's
arithmetic.  Both the HIP path and the fp64 oracle receive exactly these
tensors, so the two never depend on each other for an input.

Draws use numpy ``Generator(PCG64(seed))`` in float32, in the fixed order each
recipe lists, and are then rounded once to the run dtype (bf16 by torch's
round-to-nearest-even).  The oracle reads the rounded values widened to
float64, so comparisons measure the kernels, not the input rounding.

Workloads (named by what they are; sizes as in the scale claims of the
FLARE and FLARE++ pages, tokens as i.i.d. Gaussian "token clouds"):

* ``encdec_f32_n1k``   FLARE encode/decode, fp32: B=1, H=4, D=16, N=1024, M=32;
  draws Q [H, M, D], K, V [B, N, H, D] ~ N(0, 1).
* ``mix_bf16_n4k_c128`` FLARE++ mixer, bf16: B=8, C=128, H=8 (D=16), N=4096,
  M=64; draws X [B, N, C] ~ N(0, 1), W_K, W_V, W_eK, W_eV [C, C] ~ N(0, 1/C),
  seeds [H, M, D] ~ N(0, 1).
* ``encdec_bf16_n1m``  FLARE encode/decode at mesh scale, bf16: B=1, H=8, D=32,
  N=1,048,576, M=256; draws Q [H, M, D], K, V [B, N, H, D] ~ N(0, 1).
* ``seq_bf16_b32_n4k`` FLARE++ on sequence-shaped input, bf16: B=32, N=4096,
  C=256, H=8 (D=32), M=128; draws an embedding table E [256, C] ~ N(0, 1), token
  ids [B, N] uniform on {0..255}, X = E[ids], four weights ~ N(0, 1/C), seeds.
* ``block_bf16_n256k`` FLARE++ block with the output projection, bf16: B=4,
  N=262,144, C=256, H=8 (D=32), M=512; X ~ N(0, 1), W_K, W_V, W_eK, W_eV, W_O ~
  N(0, 1/C), seeds ~ N(0, 1).

"Sharp" variants multiply the latent queries (or seeds) by ``q_mult`` so that
routing is far from uniform (score std of several units); with the plain
recipes the synthesized queries are small and routing is nearly uniform.
"""
from dataclasses import dataclass, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str          # "encdec" (K, V given) or "mix" (projections from X)
    B: int
    N: int
    H: int
    D: int
    M: int
    dtype: str         # "f32" or "bf16"
    dynamic: bool = False   # FLARE++ query synthesis
    has_wo: bool = False    # output projection
    tokens: str = "gaussian"  # or "vocab" (embedded random integer tokens)

    @property
    def C(self) -> int:
        return self.H * self.D

    def with_n(self, n: int) -> "Workload":
        return replace(self, N=n)

    def with_b(self, b: int) -> "Workload":
        return replace(self, B=b)


WORKLOADS = {
    "encdec_f32_n1k": Workload("encdec_f32_n1k", "encdec", 1, 1024, 4, 16, 32, "f32"),
    "mix_bf16_n4k_c128": Workload("mix_bf16_n4k_c128", "mix", 8, 4096, 8, 16, 64, "bf16",
                                  dynamic=True),
    "encdec_bf16_n1m": Workload("encdec_bf16_n1m", "encdec", 1, 1 << 20, 8, 32, 256, "bf16"),
    "seq_bf16_b32_n4k": Workload("seq_bf16_b32_n4k", "mix", 32, 4096, 8, 32, 128, "bf16",
                                 dynamic=True, tokens="vocab"),
    "block_bf16_n256k": Workload("block_bf16_n256k", "mix", 4, 1 << 18, 8, 32, 512, "bf16",
                                 dynamic=True, has_wo=True),
}

VOCAB = 256


def torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def _normal(rng, shape, std=1.0):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _cast(a: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(a).to(torch_dtype(dtype))


def make_encdec(w: Workload, seed: int = 0, q_mult: float = 1.0, synth: bool = False,
                per_batch_q: bool = False):
    """Inputs of an encode/decode workload, token-major.

    Returns a dict of CPU tensors: q [H, M, D] (or [B, H, M, D] with
    per_batch_q), k, v [B, N, H, D]; with
    ``synth`` also ek, ev [B, N, H, D] and seeds [H, M, D] (drawn after q, k, v)
    for the variant that synthesizes the queries first.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _normal(rng, (w.B, w.H, w.M, w.D) if per_batch_q else (w.H, w.M, w.D))
    k = _normal(rng, (w.B, w.N, w.H, w.D))
    v = _normal(rng, (w.B, w.N, w.H, w.D))
    if q_mult != 1.0:
        q *= np.float32(q_mult)
    out = {"q": _cast(q, w.dtype), "k": _cast(k, w.dtype), "v": _cast(v, w.dtype)}
    if synth:
        ek = _normal(rng, (w.B, w.N, w.H, w.D))
        ev = _normal(rng, (w.B, w.N, w.H, w.D))
        seeds = _normal(rng, (w.H, w.M, w.D))
        if q_mult != 1.0:
            seeds *= np.float32(q_mult)
        out.update(ek=_cast(ek, w.dtype), ev=_cast(ev, w.dtype), seeds=_cast(seeds, w.dtype))
    return out


def make_mix(w: Workload, seed: int = 0, q_mult: float = 1.0):
    """Inputs of a mixer workload: x [B, N, C]; w_k, w_v (and w_ek, w_ev when
    dynamic, w_o when has_wo) [C, C] with y = x W; qs [H, M, D] (the learned
    queries, or the seeds when dynamic)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    C = w.C
    if w.tokens == "vocab":
        table = _normal(rng, (VOCAB, C))
        ids = rng.integers(0, VOCAB, size=(w.B, w.N))
        x = table[ids]
    else:
        x = _normal(rng, (w.B, w.N, C))
    std = 1.0 / np.sqrt(C)
    out = {"x": _cast(x, w.dtype)}
    out["w_k"] = _cast(_normal(rng, (C, C), std), w.dtype)
    out["w_v"] = _cast(_normal(rng, (C, C), std), w.dtype)
    if w.dynamic:
        out["w_ek"] = _cast(_normal(rng, (C, C), std), w.dtype)
        out["w_ev"] = _cast(_normal(rng, (C, C), std), w.dtype)
    if w.has_wo:
        out["w_o"] = _cast(_normal(rng, (C, C), std), w.dtype)
    qs = _normal(rng, (w.H, w.M, w.D))
    if q_mult != 1.0:
        qs *= np.float32(q_mult)
    out["qs"] = _cast(qs, w.dtype)
    return out


def normal_tensor(shape, dtype: str, seed: int, std: float = 1.0) -> torch.Tensor:
    """A standalone N(0, std^2) tensor (edge-case tests)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return _cast(_normal(rng, tuple(shape), std), dtype)

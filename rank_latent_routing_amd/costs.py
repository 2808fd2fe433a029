"""Algorithmic work of the mixer: flops, exponentials and HBM bytes.

These are the counts the method itself requires (not what a kernel happens
to execute), used to turn measured times into TFLOP/s, GB/s and roofline
fractions.  The operation model follows "FLARE++: Low-Rank Attention with
Dynamic Attention Routing", section 3, "Computational complexity": a
pointwise projection costs O(N C^2), a token-latent SDPA call O(N M C);
FLARE uses three projections and two calls, FLARE++ five projections and
three calls.

Per SDPA call, per (batch, head) token: scores q.k cost 2*M*D flops, the
weighted sum of values another 2*M*D, and there are M exponentials.  A
projection costs 2*C*C flops per token.
"""
from dataclasses import dataclass

BF16 = 2
F32 = 4


@dataclass
class Work:
    flops: float
    exps: float
    bytes: float

    def __add__(self, o):
        return Work(self.flops + o.flops, self.exps + o.exps, self.bytes + o.bytes)


def sdpa_call(B, H, N, M, D, elem=BF16, token_bytes_per_head=None) -> Work:
    """One token-latent SDPA call over N tokens and M latents per (b, h).

    Bytes: the token-side streams only (two D-vectors per token and head:
    K and V for an encode, K in and Y out for a decode); the latent-side
    tensors are O(B H M D) and counted separately by callers when wanted.
    """
    tb = 2 * D * elem if token_bytes_per_head is None else token_bytes_per_head
    return Work(4.0 * B * H * N * M * D, 1.0 * B * H * N * M, 1.0 * B * H * N * tb)


def encode(B, H, N, M, D, elem=BF16) -> Work:
    return sdpa_call(B, H, N, M, D, elem)


def decode(B, H, N, M, D, elem=BF16) -> Work:
    return sdpa_call(B, H, N, M, D, elem)


def projection(B, N, C, n_proj, elem=BF16, read_x=True) -> Work:
    """n_proj C x C projections of the same X: X read once, outputs written once."""
    byts = (B * N * C * elem if read_x else 0) + n_proj * B * N * C * elem
    return Work(2.0 * B * N * C * C * n_proj, 0.0, float(byts))


def mixer(B, N, C, H, M, dynamic: bool, has_wo: bool, elem=BF16, shared: bool = False) -> Work:
    """Whole mixer: projections + SDPA calls (+ output projection).  With
    ``shared`` (FLARE++ whose synthesis reuses K and V) the eK, eV
    projections drop out."""
    D = C // H
    n_proj, calls = primitives(dynamic, has_wo)
    n_in = n_proj - (1 if has_wo else 0) - (2 if dynamic and shared else 0)
    w = projection(B, N, C, n_in, elem)
    for _ in range(calls):
        w = w + sdpa_call(B, H, N, M, D, elem)
    if has_wo:
        w = w + projection(B, N, C, 1, elem)
    return w


def primitives(dynamic: bool, has_wo: bool = True):
    """(number of C x C projections, number of SDPA calls) in one mixer:
    FLARE projects K, V (and the output), FLARE++ adds eK, eV and one call."""
    n_proj = (4 if dynamic else 2) + (1 if has_wo else 0)
    return n_proj, (3 if dynamic else 2)


def mixer_op_ratio(C: int, M: int) -> float:
    """FLARE++ / FLARE operation count in the pages' unit-cost model (a
    projection costs C^2 per token, an SDPA call M C per token), output
    projection included in both: (5 C^2 + 3 M C) / (3 C^2 + 2 M C)."""
    p1, c1 = primitives(False)
    p2, c2 = primitives(True)
    return (p2 * C * C + c2 * M * C) / (p1 * C * C + c1 * M * C)


def encdec_backward(B, H, N, M, D, elem=BF16) -> Work:
    """Gradients of one FLARE encode + decode pair: each SDPA call's backward
    is five products of 2 N M D flops (scores recomputed, dP, dq, dk, dv) and
    N M exponentials; bytes are the token-side reads (K, V, Y, dY) and writes
    (dK, dV in fp32) per (token, head)."""
    per = B * H * N
    flops = 2 * 5 * 2.0 * M * D * per
    exps = 2.0 * M * per
    bytes_ = per * D * (4 * elem + 2 * 4)
    return Work(flops, exps, bytes_)

"""CPU tier: property tests of the fp64 oracle on random shapes and values.

Each property is fixed by the mathematics of the operator the pages state
("FLARE++: Low-Rank Attention with Dynamic Attention Routing", section 3:
"FLARE: fixed-query latent routing" for the encode/decode pair, "Multi-GPU
context parallelism" for the split merge), not by the oracle's own code, so a
dropped term, a wrong axis or a transposed operand in the oracle fails one of
them on some drawn input:

  * a softmax row is invariant to a shift of its scores: adding a vector u to
    every key (encoder) or to every latent query (decoder) adds q.u (k.u) to a
    whole row of scores and leaves the output unchanged;
  * every output row is a convex combination of value rows;
  * the output is linear in the values;
  * scale enters only through scale * q: (q, scale) and (a q, scale / a) agree;
  * the token-split encoder merged by logsumexp equals the unsplit one, for
    any split points (empty splits included), and so does its lse;
  * the materialised mixing matrix has rows summing to 1, rank at most M, and
    W V equals the factored encode-then-decode result;
  * permuting the tokens permutes the decoder output and leaves the latents;
  * the gradients of a softmax row sum to zero along the row, so the key
    gradient of the encoder sums to zero over tokens, and the query gradient
    of the decoder sums to zero over latents; the value gradient of the
    encoder sums (over tokens) to the sum of the output gradient (over
    latents).
"""
import numpy as np
from hypothesis import given, settings, strategies as st

import oracle

SETTINGS = settings(max_examples=60, deadline=None)


@st.composite
def head(draw, max_n=40, max_m=12, sharp=3.0):
    """One head: q [M, D], k [N, D], v [N, Dv] with scores of moderate to sharp size."""
    N = draw(st.integers(1, max_n))
    M = draw(st.integers(1, max_m))
    D = draw(st.sampled_from([1, 2, 4, 8, 16]))
    Dv = draw(st.sampled_from([1, 3, 8]))
    seed = draw(st.integers(0, 2**31 - 1))
    qm = draw(st.floats(0.0, sharp))
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((M, D)) * qm
    k = rng.standard_normal((N, D))
    v = rng.standard_normal((N, Dv))
    return q, k, v, rng


def close(a, b, tol=1e-9):
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    return float(np.max(np.abs(a - b))) <= tol * scale if a.size else True


@SETTINGS
@given(head())
def test_encoder_is_invariant_to_a_common_key_shift(h):
    q, k, v, rng = h
    u = rng.standard_normal(k.shape[1]) * 2.0
    assert close(oracle.sdpa(q, k + u, v), oracle.sdpa(q, k, v))


@SETTINGS
@given(head())
def test_decoder_is_invariant_to_a_common_latent_query_shift(h):
    q, k, v, rng = h
    z = oracle.sdpa(q, k, v)
    u = rng.standard_normal(q.shape[1]) * 2.0
    assert close(oracle.sdpa(k, q + u, z), oracle.sdpa(k, q, z))


@SETTINGS
@given(head(sharp=20.0))
def test_outputs_are_convex_combinations_of_values(h):
    q, k, v, _ = h
    z = oracle.sdpa(q, k, v)
    eps = 1e-12 * max(1.0, float(np.max(np.abs(v))))
    assert np.all(z >= v.min(axis=0) - eps) and np.all(z <= v.max(axis=0) + eps)
    y = oracle.sdpa(k, q, z)
    assert np.all(y >= z.min(axis=0) - eps) and np.all(y <= z.max(axis=0) + eps)


@SETTINGS
@given(head(), st.floats(-3.0, 3.0), st.floats(-3.0, 3.0))
def test_encoder_is_linear_in_the_values(h, a, b):
    q, k, v, rng = h
    v2 = rng.standard_normal(v.shape)
    assert close(oracle.sdpa(q, k, a * v + b * v2), a * oracle.sdpa(q, k, v) + b * oracle.sdpa(q, k, v2))


@SETTINGS
@given(head(), st.floats(0.125, 8.0))
def test_scale_acts_through_scale_times_q(h, a):
    q, k, v, _ = h
    s = oracle.default_scale(q.shape[1])
    assert close(oracle.sdpa(a * q, k, v, scale=s / a), oracle.sdpa(q, k, v, scale=s), 1e-8)


@SETTINGS
@given(head(max_n=60, sharp=10.0), st.lists(st.integers(0, 60), max_size=6))
def test_split_merge_equals_unsplit_encoder(h, cuts):
    q, k, v, _ = h
    N = k.shape[0]
    bounds = [0] + sorted(min(c, N) for c in cuts) + [N]
    z, lse = oracle.sharded_encode(q, k, v, bounds)
    zr, lr = oracle.sdpa(q, k, v, return_lse=True)
    assert close(z, zr) and close(lse, lr)


@SETTINGS
@given(head(max_n=24, max_m=6))
def test_mixing_matrix_rows_rank_and_factorisation(h):
    q, k, v, _ = h
    N, M = k.shape[0], q.shape[0]
    w, wd, we = oracle.mixing_matrix(q, k)
    assert close(w.sum(axis=1), np.ones(N))
    assert np.linalg.matrix_rank(w, tol=1e-10) <= M
    y = oracle.sdpa(k, q, oracle.sdpa(q, k, v))
    assert close(w @ v, y)
    assert close(wd @ we, w)


@SETTINGS
@given(head())
def test_token_permutation_permutes_outputs_and_keeps_latents(h):
    q, k, v, rng = h
    p = rng.permutation(k.shape[0])
    z = oracle.sdpa(q, k, v)
    zp = oracle.sdpa(q, k[p], v[p])
    assert close(zp, z)
    assert close(oracle.sdpa(k[p], q, zp), oracle.sdpa(k, q, z)[p])


@SETTINGS
@given(head(sharp=5.0))
def test_softmax_gradients_sum_to_zero_along_the_row(h):
    q, k, v, rng = h
    # encoder: rows are latents, the softmax runs over tokens
    dz = rng.standard_normal((q.shape[0], v.shape[1]))
    dq, dk, dv = oracle.sdpa_backward(q, k, v, dz)
    assert close(dk.sum(axis=0), np.zeros(k.shape[1]), 1e-9)
    assert close(dv.sum(axis=0), dz.sum(axis=0), 1e-9)
    # decoder: rows are tokens, the softmax runs over latents
    z = oracle.sdpa(q, k, v)
    dy = rng.standard_normal((k.shape[0], z.shape[1]))
    dk2, dq2, dz2 = oracle.sdpa_backward(k, q, z, dy)
    assert close(dq2.sum(axis=0), np.zeros(q.shape[1]), 1e-9)
    assert close(dz2.sum(axis=0), dy.sum(axis=0), 1e-9)

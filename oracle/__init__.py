"""fp64 CPU oracle for the FLARE / FLARE++ token mixer (test infrastructure).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product library never calls it, and it shares no code with
the HIP path.  The arithmetic lives in ``flare_oracle.c`` (plain C, fp64,
libm exp/log); this module only marshals numpy arrays to it.

Every function takes and returns float64 numpy arrays.  Citations name the
page and section the computation follows:

* [P1] "FLARE++: Low-Rank Attention with Dynamic Attention Routing", section 3
  (Method): "Full self-attention", "FLARE: fixed-query latent routing"
  (equation 5), "FLARE++: dynamic token routing" (equations 7, 8),
  "Computational complexity", "Multi-GPU context parallelism".

Parity status: every function here is pinned by tests in
``tests/test_oracle_pins.py`` (library SDPA, closed forms, invariants, brute
force).  The full FLARE++ composition ``flare_mix`` is pinned by the
composition of pinned parts, by token-permutation equivariance, and by the
special cases where zero synthesis values or keys reduce it to closed forms;
beyond those its values are parity unpinned: the pages print no worked
example of the mixer.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_build", "liboracle.so")
_lib = None

_d = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_sdpa.argtypes = [_d, _i64, _d, _i64, _d, _i64, _d, _i64, _d,
                                _i64, _i64, ctypes.c_int, ctypes.c_int,
                                ctypes.c_double]
    lib.oracle_sdpa_backward.argtypes = [_d, _i64, _d, _i64, _d, _i64, _d, _i64, _d, _i64,
                                         _d, _i64, _d, _i64, _i64, _i64, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_double]
    lib.oracle_matmul.argtypes = [_d, _i64, _d, _i64, _d, _i64, _i64,
                                  ctypes.c_int, ctypes.c_int]
    lib.oracle_merge.argtypes = [_d, _i64, _d, ctypes.c_int, _i64, ctypes.c_int,
                                 _d, _d]
    lib.oracle_sharded_encode.argtypes = [_d, _i64, _d, _i64, _d, _i64,
                                          ctypes.POINTER(ctypes.c_int64),
                                          ctypes.c_int, _d, _d, _i64,
                                          ctypes.c_int, ctypes.c_int,
                                          ctypes.c_double]
    lib.oracle_mixing_matrix.argtypes = [_d, _i64, _d, _i64, _i64, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_double, _d, _d, _d]
    lib.oracle_flare_encdec.argtypes = [_d, _i64, _d, _d, _d, _d, _d,
                                        ctypes.c_int, _i64, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int,
                                        ctypes.c_double, ctypes.c_int,
                                        ctypes.c_int]
    lib.oracle_flare_mix.argtypes = [_d, _d, _d, _d, _d, _d, _d, _d, _d, _d,
                                     ctypes.c_int, _i64, ctypes.c_int,
                                     ctypes.c_int, ctypes.c_int, ctypes.c_double]
    for f in ("oracle_sdpa", "oracle_sdpa_backward", "oracle_matmul", "oracle_merge",
              "oracle_sharded_encode", "oracle_mixing_matrix",
              "oracle_flare_encdec", "oracle_flare_mix"):
        getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


def max_threads() -> int:
    """OpenMP threads the oracle runs with (OMP_NUM_THREADS, else all cores)."""
    return _load().oracle_max_threads()


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a):
    if a is None:
        return None
    return a.ctypes.data_as(_d)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"oracle {what} failed with code {rc}")


def default_scale(D: int) -> float:
    """1/sqrt(D), the scale of every SDPA call ([P1] "Full self-attention")."""
    return 1.0 / np.sqrt(D)


def sdpa(q, k, v, scale=None, return_lse=False):
    """One scaled dot-product attention call: rows of ``q`` [Lq, D] attend
    over keys ``k`` [Lk, D] and values ``v`` [Lk, Dv]; returns o [Lq, Dv]
    (and the natural-log row normaliser lse [Lq])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    Lq, D = q.shape
    Lk = k.shape[0]
    Dv = v.shape[1]
    assert k.shape == (Lk, D) and v.shape[0] == Lk
    if scale is None:
        scale = default_scale(D)
    o = np.empty((Lq, Dv))
    lse = np.empty(Lq) if return_lse else None
    dummy = np.zeros((1, max(D, Dv)))
    kp = k if Lk else dummy
    vp = v if Lk else dummy
    _check(_load().oracle_sdpa(_p(q), D, _p(kp), D, _p(vp), Dv, _p(o), Dv,
                               _p(lse), Lq, Lk, D, Dv, float(scale)), "sdpa")
    return (o, lse) if return_lse else o


def sdpa_backward(q, k, v, do, scale=None):
    """Gradients (dq, dk, dv) of sum(do * sdpa(q, k, v)) for q [Lq, D],
    k [Lk, D], v [Lk, Dv], do [Lq, Dv] (the standard SDPA gradient, which is
    what the encoder and decoder calls need in training)."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    Lq, D = q.shape
    Lk, Dv = v.shape
    assert k.shape == (Lk, D) and do.shape == (Lq, Dv)
    if scale is None:
        scale = default_scale(D)
    dq, dk, dv = np.empty((Lq, D)), np.empty((Lk, D)), np.empty((Lk, Dv))
    _check(_load().oracle_sdpa_backward(_p(q), D, _p(k), D, _p(v), Dv, _p(do), Dv,
                                        _p(dq), D, _p(dk), D, _p(dv), Dv, Lq, Lk, D, Dv,
                                        float(scale)), "sdpa_backward")
    return dq, dk, dv


def encode_backward(q, k, v, dz, scale=None):
    """Gradients of sum(dz * encode(q, k, v)) for q [B|1, H, M, D] or [H, M, D],
    k, v [B, H, N, D], dz [B, H, M, D].  Returns (dq [B, H, M, D] per batch
    element, dk, dv [B, H, N, D]); a batch-shared q gets the sum over b."""
    q = _f64(q)
    if q.ndim == 3:
        q = q[None]
    k, v, dz = _f64(k), _f64(v), _f64(dz)
    B, H, N, D = k.shape
    dq = np.empty(dz.shape)
    dk = np.empty(k.shape)
    dv = np.empty(v.shape)
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = sdpa_backward(q[b if q.shape[0] > 1 else 0, h], k[b, h],
                                                         v[b, h], dz[b, h], scale)
    return dq, dk, dv


def decode_backward(k, q, z, dy, scale=None):
    """Gradients of sum(dy * decode(k, q, z)) for k [B, H, N, D], q, z
    [B|1, H, M, D] or [H, M, D], dy [B, H, N, D].  Returns (dk [B, H, N, D],
    dq, dz [B, H, M, D] per batch element)."""
    k, dy = _f64(k), _f64(dy)
    q, z = _f64(q), _f64(z)
    if q.ndim == 3:
        q = q[None]
    if z.ndim == 3:
        z = z[None]
    B, H, N, D = k.shape
    M = q.shape[2]
    dk = np.empty(k.shape)
    dq = np.empty((B, H, M, D))
    dz = np.empty((B, H, M, z.shape[3]))
    for b in range(B):
        for h in range(H):
            dk[b, h], dq[b, h], dz[b, h] = sdpa_backward(k[b, h], q[b if q.shape[0] > 1 else 0, h],
                                                         z[b if z.shape[0] > 1 else 0, h], dy[b, h], scale)
    return dk, dq, dz


def flare_encdec_backward(q, k, v, dy, scale=None):
    """Gradients of sum(dy * Y) for the FLARE pair Z = SDPA(Q, K, V),
    Y = SDPA(K, Q, Z) with head-major k, v, dy [B, H, N, D] and q
    [B|1, H, M, D] or [H, M, D].  The chain rule through the two calls:
    the decoder's gradient gives dK, dQ and dZ; dZ drives the encoder's
    gradient, whose dQ and dK add to the decoder's.  Returns (dq per batch
    element [B, H, M, D], dk, dv)."""
    z, _ = encode(q, k, v, scale)
    dk1, dq1, dz = decode_backward(k, q, z, dy, scale)
    dq2, dk2, dv = encode_backward(q, k, v, dz, scale)
    return dq1 + dq2, dk1 + dk2, dv


def flarepp_backward(seeds, ek, ev, k, v, dy, scale=None):
    """Gradients of sum(dy * Y) for FLARE++'s three calls ([P1] "FLARE++:
    dynamic token routing", equation 8, then "FLARE: fixed-query latent
    routing"): Q(X) = SDPA(seeds, eK, eV), Z = SDPA(Q(X), K, V),
    Y = SDPA(K, Q(X), Z), with seeds [H, M, D] shared by the batch and
    head-major ek, ev, k, v, dy [B, H, N, D].  The chain rule: the decoder
    and the encoder give dQ(X), dK, dV as in flare_encdec_backward; dQ(X)
    drives the synthesis gradient, whose seed part is summed over the batch.
    Returns (dseeds [H, M, D], dek, dev, dk, dv)."""
    qx, _ = encode(seeds, ek, ev, scale)
    dqx, dk, dv = flare_encdec_backward(qx, k, v, dy, scale)
    dseeds_b, dek, dev = encode_backward(seeds, ek, ev, dqx, scale)
    return dseeds_b.sum(0), dek, dev, dk, dv


def matmul(x, w):
    """y = x W for x [R, Cin], W [Cin, Cout] (pointwise projection)."""
    x, w = _f64(x), _f64(w)
    R, Cin = x.shape
    Cout = w.shape[1]
    y = np.empty((R, Cout))
    _check(_load().oracle_matmul(_p(x), Cin, _p(w), Cout, _p(y), Cout, R, Cin,
                                 Cout), "matmul")
    return y


def merge(o_parts, l_parts):
    """Exact logsumexp merge of shard results ([P1] "Multi-GPU context
    parallelism"): o_parts [R, Lq, Dv], l_parts [R, Lq] -> (z, lse)."""
    o_parts, l_parts = _f64(o_parts), _f64(l_parts)
    R, Lq, Dv = o_parts.shape
    z = np.empty((Lq, Dv))
    lse = np.empty(Lq)
    _check(_load().oracle_merge(_p(o_parts), Lq * Dv, _p(l_parts), R, Lq, Dv,
                                _p(z), _p(lse)), "merge")
    return z, lse


def sharded_encode(q, k, v, bounds, scale=None):
    """Encoder applied per token shard [bounds[r], bounds[r+1]) and merged."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    Lq, D = q.shape
    Dv = v.shape[1]
    if scale is None:
        scale = default_scale(D)
    b = np.ascontiguousarray(np.asarray(bounds, dtype=np.int64))
    assert b[0] == 0 and b[-1] == k.shape[0]
    z = np.empty((Lq, Dv))
    lse = np.empty(Lq)
    _check(_load().oracle_sharded_encode(
        _p(q), D, _p(k), D, _p(v), Dv,
        b.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), len(b) - 1,
        _p(z), _p(lse), Lq, D, Dv, float(scale)), "sharded_encode")
    return z, lse


def mixing_matrix(q, k, scale=None):
    """Materialised W_eff = W_dec W_enc [N, N] of one head (tiny N only).
    Returns (W, W_dec [N, M], W_enc [M, N])."""
    q, k = _f64(q), _f64(k)
    M, D = q.shape
    N = k.shape[0]
    if scale is None:
        scale = default_scale(D)
    w = np.empty((N, N))
    wd = np.empty((N, M))
    we = np.empty((M, N))
    _check(_load().oracle_mixing_matrix(_p(q), D, _p(k), D, N, M, D,
                                        float(scale), _p(w), _p(wd), _p(we)),
           "mixing_matrix")
    return w, wd, we


# ----- batched forms used by the parity tests (head-major numpy layouts) -----

def encode(q, k, v, scale=None):
    """Z[b,h] = SDPA(Q[b,h], K[b,h], V[b,h]) for q [B|1, H, M, D] (a leading 1
    or a 3-d [H, M, D] means one set shared by the batch), k, v [B, H, N, D].
    Returns (z [B, H, M, D], lse [B, H, M]).  ([P1] equation 5; the FLARE++
    query synthesis of equation 8 is this call with the seeds as q.)"""
    q = _f64(q)
    if q.ndim == 3:
        q = q[None]
    k, v = _f64(k), _f64(v)
    B, H, N, D = k.shape
    M = q.shape[2]
    z = np.empty((B, H, M, v.shape[3]))
    lse = np.empty((B, H, M))
    for b in range(B):
        for h in range(H):
            z[b, h], lse[b, h] = sdpa(q[b if q.shape[0] > 1 else 0, h], k[b, h],
                                      v[b, h], scale, return_lse=True)
    return z, lse


def decode(k, q, z, scale=None):
    """Y[b,h] = SDPA(K[b,h], Q[b,h], Z[b,h]) for k [B, H, N, D], q and z
    [B|1, H, M, D]; returns y [B, H, N, D]  ([P1] "FLARE: fixed-query latent
    routing", the decoder call)."""
    k = _f64(k)
    q, z = _f64(q), _f64(z)
    if q.ndim == 3:
        q = q[None]
    if z.ndim == 3:
        z = z[None]
    B, H, N, D = k.shape
    y = np.empty((B, H, N, z.shape[3]))
    for b in range(B):
        for h in range(H):
            y[b, h] = sdpa(k[b, h], q[b if q.shape[0] > 1 else 0, h],
                           z[b if z.shape[0] > 1 else 0, h], scale)
    return y


def flare_encdec(q, k, v, H, scale=None, heads=None, want_latents=False):
    """FLARE encode then decode for token-major k, v [B, N, H*D]; q is
    [H, M, D] (shared) or [B, H, M, D].  Returns y [B, N, H*D] (heads outside
    ``heads`` = (lo, hi) stay zero), plus (z, lse) when want_latents."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, N, C = k.shape
    D = C // H
    M = q.shape[-2]
    q_bs = 0 if q.ndim == 3 else H * M * D
    if scale is None:
        scale = default_scale(D)
    lo, hi = heads if heads is not None else (0, H)
    y = np.zeros((B, N, C))
    z = np.zeros((B, H, M, D)) if want_latents else None
    lse = np.zeros((B, H, M)) if want_latents else None
    _check(_load().oracle_flare_encdec(_p(q), q_bs, _p(k), _p(v), _p(y), _p(z),
                                       _p(lse), B, N, H, M, D, float(scale),
                                       lo, hi), "flare_encdec")
    return (y, z, lse) if want_latents else y


def flare_mix(x, w_k, w_v, qs, H, w_ek=None, w_ev=None, w_o=None, scale=None):
    """Whole mixer on x [B, N, C]: FLARE when w_ek is None (qs = learned
    queries [H, M, D]), FLARE++ otherwise (qs = seeds).  Returns
    (out [B, N, C], qx [B, H, M, D], z [B, H, M, D])."""
    x = _f64(x)
    B, N, C = x.shape
    D = C // H
    qs = _f64(qs)
    M = qs.shape[1]
    if scale is None:
        scale = default_scale(D)
    args = [_f64(w) if w is not None else None for w in (w_k, w_v, w_ek, w_ev, w_o)]
    out = np.empty((B, N, C))
    qx = np.empty((B, H, M, D))
    z = np.empty((B, H, M, D))
    _check(_load().oracle_flare_mix(_p(x), _p(args[0]), _p(args[1]),
                                    _p(args[2]), _p(args[3]), _p(qs),
                                    _p(args[4]), _p(out), _p(qx), _p(z), B, N,
                                    C, H, M, float(scale)), "flare_mix")
    return out, qx, z

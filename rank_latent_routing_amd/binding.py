"""ctypes binding of the C ABI in include/flare.h.

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the mixer runs in the library's gfx950 kernels.  The
library must be built (``__graft_entry__.build()`` or
``python rank_latent_routing_amd/build.py``); without it every call raises.

Tensor arguments are 4-d ``[B, H, L, D]`` views (any strides with a
contiguous last axis), or 3-d ``[H, L, D]`` for a block shared by the batch.
``token_major(x, H)`` turns a ``[B, N, H*D]`` activation into such a view
without copying.
"""
import ctypes

import torch

from .cabi import (EXPORTS, FLARE_ACCUMULATE_DK, FLARE_ACCUMULATE_DQ,  # noqa: F401
                   FLARE_BF16, FLARE_E_HIP, FLARE_E_INVALID, FLARE_E_SCRATCH,
                   FLARE_E_UNSUPPORTED, FLARE_E_WORKSPACE, FLARE_F32,
                   FLARE_FLAG_EXACT_SOFTMAX, FLARE_MIX_FUSED_WO, FLARE_OK, FLARE_SUM_DQ_OVER_BATCH,
                   LIB_PATH, FlareTensor)
from . import cabi as _cabi


class FlareError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


_lib = None


def lib():
    """The loaded gfx950 library; raises if it has not been built."""
    global _lib
    if _lib is None:
        _lib = _cabi.load(LIB_PATH)
    return _lib


def status_string(s: int) -> str:
    return lib().flare_status_string(int(s)).decode()


def version() -> str:
    return lib().flare_version().decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return FLARE_F32
    if t.dtype == torch.bfloat16:
        return FLARE_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t, what="tensor"):
    """The raw pointer of a tensor in GPU memory (the library's kernels read
    and write what they are given: a host pointer would fault the device)."""
    if not t.is_cuda:
        raise ValueError(f"{what} must be a tensor on the GPU, got device {t.device}")
    return ctypes.c_void_p(t.data_ptr())


def _opt_dev(t, what):
    return _dev(t, what) if t is not None else ctypes.c_void_p(None)


def describe(t: torch.Tensor) -> FlareTensor:
    """flare_tensor of a [B, H, L, D] (or shared [H, L, D]) view in GPU memory."""
    if t.dim() == 3:
        sb, (sh, sl, sd) = 0, t.stride()
    elif t.dim() == 4:
        sb, sh, sl, sd = t.stride()
    else:
        raise ValueError("expected a [B, H, L, D] or [H, L, D] tensor")
    if sd != 1 and t.shape[-1] > 1:
        raise ValueError("the last axis must be contiguous")
    return FlareTensor(_dev(t).value, _dtype_code(t), 0, sb, sh, sl)


def token_major(x: torch.Tensor, H: int) -> torch.Tensor:
    """[B, N, H*D] -> [B, H, N, D] view (no copy)."""
    B, N, C = x.shape
    return x.view(B, N, H, C // H).permute(0, 2, 1, 3)


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(status: int, what: str):
    if status != FLARE_OK:
        raise FlareError(status, what)


def _dims(k: torch.Tensor):
    if k.dim() != 4:
        raise ValueError(f"keys must be [B, H, N, D], got shape {tuple(k.shape)}")
    B, H, N, D = k.shape
    return B, H, N, D


# The C ABI sees pointers and strides only: every extent below must match the
# sizes passed with them, or a kernel would read or write past the tensor.
def _token(t, B, H, N, D, what):
    if tuple(t.shape) != (B, H, N, D):
        raise ValueError(f"{what} must be [B, H, N, D] = {(B, H, N, D)}, got {tuple(t.shape)}")


def _latent(t, B, H, M, D, what, shared=True):
    """[B, H, M, D], or with ``shared`` one [H, M, D] block for the whole batch."""
    s = tuple(t.shape)
    if s != (B, H, M, D) and not (shared and s == (H, M, D)):
        raise ValueError(f"{what} must be [B, H, M, D] = {(B, H, M, D)}"
                         + (f" or shared [H, M, D] = {(H, M, D)}" if shared else "") + f", got {s}")


def _plain(t, shape, what, dtype=torch.bfloat16):
    """A contiguous tensor of the given shape and dtype (passed as a raw array)."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{what} must be a contiguous {dtype} tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)}{'' if t.is_contiguous() else ' (strided)'}")


def encode_workspace_size(B, H, M, N, D) -> int:
    return lib().flare_encode_workspace_size(B, H, M, N, D)


def _workspace(nbytes: int, device, workspace):
    if workspace is not None:
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def flare_encode(q, k, v, z=None, want_lse=False, scale=0.0, flags=0, workspace=None,
                 stream=None, z_dtype=None):
    """Z = SDPA(Q, K, V) over [B, H, N, D] keys/values; q is [B, H, M, D] or
    shared [H, M, D].  Returns z (and lse [B, H, M] fp32 when want_lse)."""
    B, H, N, D = _dims(k)
    M = q.shape[-2]
    _latent(q, B, H, M, D, "q")
    _token(v, B, H, N, D, "v")
    if z is None:
        z = torch.empty((B, H, M, D), dtype=z_dtype or k.dtype, device=k.device)
    _latent(z, B, H, M, D, "z", shared=False)
    lse = torch.empty((B, H, M), dtype=torch.float32, device=k.device) if want_lse else None
    ws = _workspace(encode_workspace_size(B, H, M, N, D), k.device, workspace)
    s = lib().flare_encode(describe(q), describe(k), describe(v), describe(z),
                           _opt_dev(lse, "lse"),
                           B, H, M, N, D, float(scale), int(flags),
                           _dev(ws, "workspace"), ws.numel() * ws.element_size(),
                           _stream(stream))
    _check(s, "flare_encode")
    return (z, lse) if want_lse else z


def flare_encode_static(q, k, v, z=None, want_lse=False, scale=0.0, flags=0, stream=None,
                        z_dtype=None):
    """flare_encode without a workspace: the split partials live in the
    library's static per-GPU scratch (see include/flare.h), so nothing is
    allocated for them.  Calls that overlap on one GPU share that scratch and
    must be ordered by the caller."""
    B, H, N, D = _dims(k)
    M = q.shape[-2]
    _latent(q, B, H, M, D, "q")
    _token(v, B, H, N, D, "v")
    if z is None:
        z = torch.empty((B, H, M, D), dtype=z_dtype or k.dtype, device=k.device)
    _latent(z, B, H, M, D, "z", shared=False)
    lse = torch.empty((B, H, M), dtype=torch.float32, device=k.device) if want_lse else None
    s = lib().flare_encode_static(describe(q), describe(k), describe(v), describe(z),
                                  _opt_dev(lse, "lse"), B, H, M, N, D, float(scale), int(flags),
                                  _stream(stream))
    _check(s, "flare_encode_static")
    return (z, lse) if want_lse else z


def encode_static_scratch_bytes() -> int:
    return lib().flare_encode_static_scratch_bytes()


def flare_route_queries(seeds, ek, ev, qx=None, scale=0.0, flags=0, workspace=None,
                        stream=None, want_lse=False):
    """Q(X) = SDPA(seeds, eK, eV); seeds [H, M, D]; returns qx [B, H, M, D] fp32
    (and the per-query normaliser lse [B, H, M] fp32 when want_lse)."""
    B, H, N, D = _dims(ek)
    M = seeds.shape[-2]
    _latent(seeds, B, H, M, D, "seeds")
    _token(ev, B, H, N, D, "ev")
    if qx is None:
        qx = torch.empty((B, H, M, D), dtype=torch.float32, device=ek.device)
    _latent(qx, B, H, M, D, "qx", shared=False)
    lse = torch.empty((B, H, M), dtype=torch.float32, device=ek.device) if want_lse else None
    ws = _workspace(encode_workspace_size(B, H, M, N, D), ek.device, workspace)
    s = lib().flare_route_queries(describe(seeds), describe(ek), describe(ev), describe(qx),
                                  _opt_dev(lse, "lse"),
                                  B, H, M, N, D, float(scale), int(flags),
                                  _dev(ws, "workspace"), ws.numel() * ws.element_size(),
                                  _stream(stream))
    _check(s, "flare_route_queries")
    return (qx, lse) if want_lse else qx


def flare_decode(k, q, z, y=None, scale=0.0, flags=0, stream=None, want_lse=False):
    """Y = SDPA(K, Q, Z); k [B, H, N, D]; q, z [B, H, M, D] or shared.  Returns
    y (and the per-token normaliser lse [B, H, N] fp32 when want_lse)."""
    B, H, N, D = _dims(k)
    M = q.shape[-2]
    _latent(q, B, H, M, D, "q")
    _latent(z, B, H, M, D, "z")
    if y is None:
        y = torch.empty((B, H, N, D), dtype=k.dtype, device=k.device)
    _token(y, B, H, N, D, "y")
    lse = torch.empty((B, H, N), dtype=torch.float32, device=k.device) if want_lse else None
    s = lib().flare_decode(describe(k), describe(q), describe(z), describe(y),
                           _opt_dev(lse, "lse"),
                           B, H, M, N, D, float(scale), int(flags), _stream(stream))
    _check(s, "flare_decode")
    return (y, lse) if want_lse else y


def _f32_ptr(t, shape, what):
    """The raw pointer of a contiguous fp32 tensor of the given shape (the C
    ABI takes these operands as plain arrays, so their layout is fixed)."""
    if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what} must be a contiguous float32 tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)}{'' if t.is_contiguous() else ' (strided)'}")
    return _dev(t, what)


def _dq_shape(B, H, M, D, flags):
    return (H, M, D) if flags & FLARE_SUM_DQ_OVER_BATCH else (B, H, M, D)


def flare_decode_backward(k, q, z, y, lse, dy, dk=None, dq=None, dz=None, flags=0, scale=0.0,
                          workspace=None, stream=None, grad_dtype=torch.float32):
    """Gradients (dk [B, H, N, D] in grad_dtype (fp32 or bf16), dq, dz
    [B, H, M, D] fp32) of sum(dy * Y) for Y = flare_decode(k, q, z) with its
    lse.  ``flags``: FLARE_ACCUMULATE_DQ / _DK add into the given dq / dk;
    FLARE_SUM_DQ_OVER_BATCH makes dq [H, M, D], summed over the batch."""
    B, H, N, D = _dims(k)
    M = q.shape[-2]
    dev = k.device
    dk = dk if dk is not None else torch.empty((B, H, N, D), dtype=grad_dtype, device=dev)
    dq = dq if dq is not None else torch.empty(_dq_shape(B, H, M, D, flags), dtype=torch.float32,
                                               device=dev)
    dz = dz if dz is not None else torch.empty((B, H, M, D), dtype=torch.float32, device=dev)
    _latent(q, B, H, M, D, "q")
    _latent(z, B, H, M, D, "z")
    for name, tt in (("y", y), ("dy", dy), ("dk", dk)):
        _token(tt, B, H, N, D, name)
    ws = _workspace(lib().flare_decode_backward_workspace_size(B, H, M, N, D), dev, workspace)
    s = lib().flare_decode_backward(describe(k), describe(q), describe(z), describe(y),
                                    _f32_ptr(lse, (B, H, N), "lse"), describe(dy), describe(dk),
                                    _f32_ptr(dq, _dq_shape(B, H, M, D, flags), "dq"),
                                    _f32_ptr(dz, (B, H, M, D), "dz"),
                                    int(flags), B, H, M, N, D, float(scale), _dev(ws, "workspace"),
                                    ws.numel() * ws.element_size(), _stream(stream))
    _check(s, "flare_decode_backward")
    return dk, dq, dz


def flare_encode_backward(q, k, v, z, lse, dz, dq=None, dk=None, dv=None, flags=0,
                          scale=0.0, workspace=None, stream=None, grad_dtype=torch.float32):
    """Gradients (dq [B, H, M, D] fp32, dk, dv [B, H, N, D] in grad_dtype, fp32
    or bf16) of sum(dz * Z) for Z = flare_encode(q, k, v) (or
    flare_route_queries) with its lse.
    ``flags``: FLARE_ACCUMULATE_DQ / _DK add into the given dq / dk;
    FLARE_SUM_DQ_OVER_BATCH makes dq [H, M, D], summed over the batch."""
    B, H, N, D = _dims(k)
    M = q.shape[-2]
    dev = k.device
    dq = dq if dq is not None else torch.empty(_dq_shape(B, H, M, D, flags), dtype=torch.float32,
                                               device=dev)
    dk = dk if dk is not None else torch.empty((B, H, N, D), dtype=grad_dtype, device=dev)
    dv = dv if dv is not None else torch.empty((B, H, N, D), dtype=dk.dtype, device=dev)
    _latent(q, B, H, M, D, "q")
    _latent(z, B, H, M, D, "z")
    for name, tt in (("v", v), ("dk", dk), ("dv", dv)):
        _token(tt, B, H, N, D, name)
    ws = _workspace(lib().flare_encode_backward_workspace_size(B, H, M, N, D), dev, workspace)
    s = lib().flare_encode_backward(describe(q), describe(k), describe(v), describe(z),
                                    _f32_ptr(lse, (B, H, M), "lse"), _f32_ptr(dz, (B, H, M, D), "dz"),
                                    _f32_ptr(dq, _dq_shape(B, H, M, D, flags), "dq"), describe(dk), describe(dv),
                                    int(flags), B, H, M, N, D, float(scale),
                                    _dev(ws, "workspace"), ws.numel() * ws.element_size(),
                                    _stream(stream))
    _check(s, "flare_encode_backward")
    return dq, dk, dv


def flare_encdec_backward(q, k, v, z, lse_enc, y, lse_dec, dy, dq=None, dk=None, dv=None, flags=0,
                          scale=0.0, workspace=None, stream=None, grad_dtype=torch.float32):
    """Gradients (dq fp32, dk, dv [B, H, N, D] in grad_dtype, fp32 or bf16) of
    sum(dy * Y) through the FLARE pair Z = flare_encode(q, k, v),
    Y = flare_decode(k, q, z), given both calls' outputs and normalisers.
    ``flags`` as for the two calls."""
    B, H, N, D = _dims(k)
    M = q.shape[-2]
    dev = k.device
    dq = dq if dq is not None else torch.empty(_dq_shape(B, H, M, D, flags), dtype=torch.float32,
                                               device=dev)
    dk = dk if dk is not None else torch.empty((B, H, N, D), dtype=grad_dtype, device=dev)
    dv = dv if dv is not None else torch.empty((B, H, N, D), dtype=dk.dtype, device=dev)
    _latent(q, B, H, M, D, "q")
    _latent(z, B, H, M, D, "z")
    for name, tt in (("v", v), ("y", y), ("dy", dy), ("dk", dk), ("dv", dv)):
        _token(tt, B, H, N, D, name)
    ws = _workspace(lib().flare_encdec_backward_workspace_size(B, H, M, N, D), dev, workspace)
    s = lib().flare_encdec_backward(describe(q), describe(k), describe(v), describe(z),
                                    _f32_ptr(lse_enc, (B, H, M), "lse_enc"), describe(y),
                                    _f32_ptr(lse_dec, (B, H, N), "lse_dec"), describe(dy),
                                    _f32_ptr(dq, _dq_shape(B, H, M, D, flags), "dq"),
                                    describe(dk), describe(dv), int(flags), B, H, M, N, D, float(scale),
                                    _dev(ws, "workspace"), ws.numel() * ws.element_size(),
                                    _stream(stream))
    _check(s, "flare_encdec_backward")
    return dq, dk, dv


def project_workspace_size(C_in, C_out, n_proj) -> int:
    return lib().flare_project_workspace_size(C_in, C_out, n_proj)


def flare_project(x, weights, outs=None, head_dim=None, workspace=None, stream=None):
    """Y_p = X W_p for x [B, N, C_in] (or [R, C_in]) bf16, weights [C_in, C_out].
    With head_dim the outputs are head-major [B, H, N, head_dim]."""
    x2 = x.reshape(-1, x.shape[-1]).contiguous()
    R, Cin = x2.shape
    Cout = weights[0].shape[1]
    B = x.shape[0] if x.dim() == 3 else 1
    n = len(weights)
    for i, w in enumerate(weights):
        _plain(w, (Cin, Cout), f"weight {i}", x.dtype)
    if head_dim:
        if Cout % head_dim or R % B:
            raise ValueError("head-major outputs need C_out divisible by head_dim and R by B")
        oshape = (B, Cout // head_dim, R // B, head_dim)
    else:
        oshape = (R, Cout)
    if outs is None:
        outs = [torch.empty(oshape, dtype=x.dtype, device=x.device) for _ in range(n)]
    for i, o in enumerate(outs):
        # row-major outputs may also carry x's leading shape, [..., C_out]
        shape = oshape
        if not head_dim and tuple(o.shape) == tuple(x.shape[:-1]) + (Cout,):
            shape = tuple(o.shape)
        _plain(o, shape, f"output {i}", x.dtype)
    ws = _workspace(project_workspace_size(Cin, Cout, n), x.device, workspace)
    warr = (ctypes.c_void_p * n)(*[_dev(w, "weight").value for w in weights])
    yarr = (ctypes.c_void_p * n)(*[_dev(o, "output").value for o in outs])
    s = lib().flare_project(_dev(x2, "x"), warr, yarr, n, R, Cin, Cout,
                            1 if head_dim else 0, B, head_dim or 0,
                            _dev(ws, "workspace"), ws.numel() * ws.element_size(),
                            _stream(stream))
    _check(s, "flare_project")
    return outs


def mix_workspace_size(B, N, C, H, M, dynamic, has_wo) -> int:
    return lib().flare_mix_workspace_size(B, N, C, H, M, int(bool(dynamic)), int(bool(has_wo)))


def flare_mix(x, w_k, w_v, qs, H, w_ek=None, w_ev=None, w_o=None, out=None, scale=0.0,
              flags=0, workspace=None, stream=None):
    """The whole mixer on x [B, N, C] bf16: FLARE with learned queries qs
    [H, M, D] when w_ek is None, FLARE++ (qs = seeds) otherwise; optional
    output projection.  Returns out [B, N, C]."""
    B, N, C = x.shape
    M = qs.shape[1]
    if C % H:
        raise ValueError(f"C = {C} is not divisible by H = {H}")
    _plain(x, (B, N, C), "x", x.dtype)
    for name, w in (("w_k", w_k), ("w_v", w_v), ("w_ek", w_ek), ("w_ev", w_ev), ("w_o", w_o)):
        if w is not None:
            _plain(w, (C, C), name, x.dtype)
    _plain(qs, (H, M, C // H), "qs", x.dtype)
    if out is None:
        out = torch.empty_like(x)
    _plain(out, (B, N, C), "out", x.dtype)
    dyn, has_wo = w_ek is not None, w_o is not None
    ws = _workspace(mix_workspace_size(B, N, C, H, M, dyn, has_wo), x.device, workspace)
    ptr = lambda t: _opt_dev(t, "mixer operand")
    s = lib().flare_mix(ptr(x), ptr(w_k), ptr(w_v), ptr(w_ek), ptr(w_ev), ptr(qs), ptr(w_o),
                        ptr(out), _dtype_code(x), B, N, C, H, M, float(scale), int(flags),
                        _dev(ws, "workspace"), ws.numel() * ws.element_size(),
                        _stream(stream))
    _check(s, "flare_mix")
    return out

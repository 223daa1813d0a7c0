"""MI355X (gfx950) GEMM-epilogue chain: GEMM -> residual -> RMSNorm -> GEMM(+SwiGLU).

Thin Python binding over the C ABI of ``libcoda.so`` (declared in ``include/coda.h``).
Every step of the chain runs in the library's HIP kernels; this module only marshals
torch device tensors (memory) and the current HIP stream into the C calls.  If the
library is missing, importing the binding's functions raises: there is no CPU path.

    h, P = gemm_resid_partialrms(A, Wo_t, x_res)          # first GEMM + epilogue
    r    = rowscale_reduce(P, N=d, eps=1e-5)               # light reduction
    y    = gemm_rowscale_swiglu(h, Wp_t, r, act=SWIGLU)   # second GEMM + epilogue
"""

from __future__ import annotations

import torch

from . import _lib
from ._lib import CODA_ACT_NONE, CODA_ACT_SWIGLU, CODA_BF16, CODA_E4M3, CodaError  # noqa: F401

NONE = CODA_ACT_NONE
SWIGLU = CODA_ACT_SWIGLU

__all__ = ["NONE", "SWIGLU", "CodaError", "prepare_weight_bf16", "quantize_e4m3",
           "partials_per_row", "gemm_resid_partialrms", "rowscale_reduce",
           "gemm_rowscale_swiglu", "rope_table", "gemm_rowscale_rope", "ce_partials_per_row",
           "gemm_rowscale_ce", "ce_reduce", "rowscale_from_h", "transpose_bf16", "gemm_swiglu_bwd", "rmsnorm_bwd_reduce",
           "gemm_rmsnorm_bwd", "mlpin_bwd", "wgrad_partials_rows", "gemm_wgrad", "colsum_reduce",
           "mlpin_wgrad", "gemm_bf16", "chain_bwd", "wgrad_workspace_bytes", "gemm_rowscale_swiglu_save",
           "swiglu_bwd_saved", "gemm_rowscale_gfold", "gemm_wgrad_tok", "gemm_wgrad_tok_noalloc", "rope_bwd", "qkv_rope_bwd", "gemm_ce_bwd",
           "lmhead_ce_bwd", "chain",
           "version"]


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"expected a device (GPU) tensor, got one on {t.device}")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


# Storage kinds the library reads and writes: bf16 codes (2 bytes), e4m3 codes (1 byte),
# fp32 and int32.  The library sees plain pointers, so every tensor a caller hands in is
# checked here -- shape, element type, contiguity, device -- before any call is made: a
# mismatched buffer would otherwise be read or written out of bounds on the GPU.
B16 = (torch.bfloat16, torch.int16, torch.uint16)
B8 = (torch.uint8, torch.int8, torch.float8_e4m3fn)
F32 = (torch.float32,)
I32 = (torch.int32,)


def _dims(t, name, nd):
    """The shape of a caller's operand whose sizes define the problem (ndim checked)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch tensor, got {type(t).__name__}")
    if t.dim() != nd:
        raise ValueError(f"{name}: expected {nd} dimensions, got shape {tuple(t.shape)}")
    return tuple(t.shape)


def _need(t, name, shape, kinds, dev, optional=True):
    """Raise ValueError unless tensor ``t`` has exactly ``shape`` (None: any), a dtype in
    ``kinds``, is contiguous and sits on device ``dev`` (the call's first operand's); ``t``
    may be None when ``optional``.  That the device is a GPU is checked last, when the
    pointers are taken (``_ptr``), after every operand's shape has been checked."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name}: required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch tensor, got {type(t).__name__}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype not in kinds:
        raise ValueError(f"{name}: expected dtype in {[str(k) for k in kinds]}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    if dev is not None and t.device != dev:
        raise ValueError(f"{name}: on {t.device}, the other operands on {dev}")


def _scalar(t, name, dev):
    """A device fp32 scalar (a one-element tensor, or a longer one whose first element is used)."""
    if t is None:
        return
    _need(t, name, None, F32, dev)
    if t.numel() < 1:
        raise ValueError(f"{name}: expected at least one fp32 element")


def version() -> str:
    return _lib.load().coda_version().decode()


def partials_per_row(N: int) -> int:
    return int(_lib.load().coda_partials_per_row(N))


def prepare_weight_bf16(W_t, gamma=None, out=None, stream=None):
    """Wp[n,k] = bf16(gamma[k] * W[n,k]);  W_t [N, K] bf16, gamma [K] fp32."""
    N, K = _dims(W_t, "W_t", 2)
    dev = W_t.device
    _need(W_t, "W_t", (N, K), B16, dev)
    _need(gamma, "gamma", (K,), F32, dev)
    _need(out, "out", (N, K), B16, dev)
    out = torch.empty((N, K), dtype=torch.bfloat16, device=dev) if out is None else out
    _lib.check("coda_prepare_weight_bf16", _lib.load().coda_prepare_weight_bf16(
        N, K, _ptr(W_t), _ptr(gamma), _ptr(out), _stream(stream)))
    return out


def quantize_e4m3(X, gamma=None, out=None, amax_scale=None, stream=None):
    """Per-tensor e4m3 quantisation (gamma folded first if given).

    Returns (Q uint8 [N, K], amax_scale fp32 [2] = {amax, scale})."""
    N, K = _dims(X, "X", 2)
    dev = X.device
    _need(X, "X", (N, K), B16, dev)
    _need(gamma, "gamma", (K,), F32, dev)
    _need(out, "out", (N, K), B8, dev)
    _need(amax_scale, "amax_scale", (2,), F32, dev)
    out = torch.empty((N, K), dtype=torch.uint8, device=dev) if out is None else out
    if amax_scale is None:
        amax_scale = torch.empty(2, dtype=torch.float32, device=dev)
    _lib.check("coda_quantize_e4m3", _lib.load().coda_quantize_e4m3(
        N, K, _ptr(X), _ptr(gamma), _ptr(out), _ptr(amax_scale), _stream(stream)))
    return out, amax_scale


def gemm_resid_partialrms(A, W, x_res=None, a_scale=None, w_scale=None, h=None,
                          partials=None, stream=None):
    """h = bf16(sa*sw*A.W^T + x_res);  P[m,t] = sum of h^2 over N-tile t.

    A [M, K] and W [N, K] both bf16 (2-byte) or both e4m3 (1-byte, scales required)."""
    M, K = _dims(A, "A", 2)
    N, KW = _dims(W, "W", 2)
    if KW != K:
        raise ValueError("A and W disagree on K")
    dev = A.device
    fp8 = A.element_size() == 1
    kinds = B8 if fp8 else B16
    _need(A, "A", (M, K), kinds, dev)
    _need(W, "W", (N, K), kinds, dev)
    _need(x_res, "x_res", (M, N), B16, dev)
    _scalar(a_scale, "a_scale", dev)
    _scalar(w_scale, "w_scale", dev)
    T = partials_per_row(N)
    _need(h, "h", (M, N), B16, dev)
    _need(partials, "partials", (M, T), F32, dev)
    if h is None:
        h = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    if partials is None:
        partials = torch.empty((M, T), dtype=torch.float32, device=dev)
    _lib.check("coda_gemm_resid_partialrms", _lib.load().coda_gemm_resid_partialrms(
        M, N, K, _ptr(A), CODA_E4M3 if fp8 else CODA_BF16, _ptr(a_scale), _ptr(W), _ptr(w_scale),
        _ptr(x_res), _ptr(h), _ptr(partials), _stream(stream)))
    return h, partials


def rowscale_reduce(partials, N: int, eps: float, r=None, stream=None):
    """r[m] = 1/sqrt(sum_t P[m,t]/N + eps)."""
    M, _ = _dims(partials, "partials", 2)
    dev = partials.device
    _need(partials, "partials", (M, partials_per_row(N)), F32, dev)
    _need(r, "r", (M,), F32, dev)
    r = torch.empty(M, dtype=torch.float32, device=dev) if r is None else r
    _lib.check("coda_rowscale_reduce", _lib.load().coda_rowscale_reduce(
        M, N, _ptr(partials), float(eps), _ptr(r), _stream(stream)))
    return r


def _second_gemm_operands(h, W, r, w_scale):
    """Shapes and checks shared by the second-GEMM calls: h [M, K] bf16, W [n_w, K] bf16
    or e4m3, r [M] fp32, w_scale a device fp32 scalar."""
    M, K = _dims(h, "h", 2)
    n_w, KW = _dims(W, "W", 2)
    if KW != K:
        raise ValueError("h and W disagree on K")
    dev = h.device
    _need(h, "h", (M, K), B16, dev)
    _need(W, "W", (n_w, K), B8 if W.element_size() == 1 else B16, dev)
    _need(r, "r", (M,), F32, dev, optional=False)
    _scalar(w_scale, "w_scale", dev)
    return M, K, n_w, dev


def gemm_rowscale_swiglu(h, W, r, act=SWIGLU, w_scale=None, y=None, stream=None):
    """y = act(r * sw * h.W^T); W [2F, K] (SwiGLU: gate rows then up rows) or [N, K]."""
    M, K, n_w, dev = _second_gemm_operands(h, W, r, w_scale)
    fp8 = W.element_size() == 1
    if act == SWIGLU and n_w % 2:
        raise ValueError("W: a SwiGLU weight needs an even number of rows")
    n_out = n_w // 2 if act == SWIGLU else n_w
    _need(y, "y", (M, n_out), B16, dev)
    y = torch.empty((M, n_out), dtype=torch.bfloat16, device=dev) if y is None else y
    _lib.check("coda_gemm_rowscale_swiglu", _lib.load().coda_gemm_rowscale_swiglu(
        M, n_out, K, act, _ptr(h), _ptr(W), CODA_E4M3 if fp8 else CODA_BF16, _ptr(w_scale),
        _ptr(r), _ptr(y), _stream(stream)))
    return y


def rope_table(rows, base=500000.0, cos=None, sin=None, stream=None):
    """cos / sin [rows, 32] fp32 of the angles p * base^(-2i/64) (RoPE, heads of 64)."""
    dev = torch.device("cuda") if cos is None else cos.device
    _need(cos, "cos", (rows, 32), F32, dev)
    _need(sin, "sin", (rows, 32), F32, dev)
    cos = torch.empty((rows, 32), dtype=torch.float32, device=dev) if cos is None else cos
    sin = torch.empty((rows, 32), dtype=torch.float32, device=dev) if sin is None else sin
    _lib.check("coda_rope_table", _lib.load().coda_rope_table(rows, float(base), _ptr(cos), _ptr(sin),
                                                               _stream(stream)))
    return cos, sin


def _rope_operands(M, pos, cos, sin, dev):
    """Positions [M] int32 (or None) and the angle table cos / sin [rows, 32] fp32."""
    _need(pos, "pos", (M,), I32, dev)
    rows = 0 if cos is None else _dims(cos, "cos", 2)[0]
    _need(cos, "cos", (rows, 32), F32, dev)
    _need(sin, "sin", (rows, 32), F32, dev, optional=cos is None)
    if cos is None and sin is not None:
        raise ValueError("cos: required with sin")
    return rows


def gemm_rowscale_rope(h, W, r, pos, cos, sin, rot_cols, w_scale=None, y=None, stream=None):
    """y = RoPE(r * sw * h.W^T): W [N_out, K]; the first rot_cols columns (Q and K heads
    of 64) turn by the angles of their row's position pos [M] (int32) from the cos / sin
    table [rows, 32]; the rest (V) pass."""
    M, K, n_out, dev = _second_gemm_operands(h, W, r, w_scale)
    fp8 = W.element_size() == 1
    rows = _rope_operands(M, pos, cos, sin, dev)
    _need(y, "y", (M, n_out), B16, dev)
    y = torch.empty((M, n_out), dtype=torch.bfloat16, device=dev) if y is None else y
    _lib.check("coda_gemm_rowscale_rope", _lib.load().coda_gemm_rowscale_rope(
        M, n_out, K, _ptr(h), _ptr(W), CODA_E4M3 if fp8 else CODA_BF16, _ptr(w_scale), _ptr(r),
        _ptr(pos), _ptr(cos), _ptr(sin), rows, rot_cols, _ptr(y), _stream(stream)))
    return y


def ce_partials_per_row(V: int) -> int:
    return int(_lib.load().coda_ce_partials_per_row(V))


def gemm_rowscale_ce(h, W, r, targets, w_scale=None, partials=None, tgt_logit=None, stream=None):
    """LM-head GEMM with the block log-sum-exp epilogue: W [V, K]; returns (partials
    [M, T, 2] = per-tile (max, sum exp(z - max)), tgt_logit [M] = z[m, targets[m]])."""
    M, K, V, dev = _second_gemm_operands(h, W, r, w_scale)
    _need(targets, "targets", (M,), I32, dev, optional=False)
    T = ce_partials_per_row(V)
    _need(partials, "partials", (M, T, 2), F32, dev)
    _need(tgt_logit, "tgt_logit", (M,), F32, dev)
    partials = torch.empty((M, T, 2), dtype=torch.float32, device=dev) if partials is None else partials
    tgt_logit = torch.empty(M, dtype=torch.float32, device=dev) if tgt_logit is None else tgt_logit
    fp8 = W.element_size() == 1
    _lib.check("coda_gemm_rowscale_ce", _lib.load().coda_gemm_rowscale_ce(
        M, V, K, _ptr(h), _ptr(W), CODA_E4M3 if fp8 else CODA_BF16, _ptr(w_scale), _ptr(r), _ptr(targets),
        _ptr(partials), _ptr(tgt_logit), _stream(stream)))
    return partials, tgt_logit


def ce_reduce(partials, targets, tgt_logit, V, lse=None, loss=None, stream=None):
    """(lse [M], loss [M]) from the LM-head GEMM's partials (loss 0 for ignored rows)."""
    M = _dims(partials, "partials", 3)[0]
    dev = partials.device
    _need(partials, "partials", (M, ce_partials_per_row(V), 2), F32, dev)
    _need(targets, "targets", (M,), I32, dev, optional=False)
    _need(tgt_logit, "tgt_logit", (M,), F32, dev, optional=False)
    _need(lse, "lse", (M,), F32, dev)
    _need(loss, "loss", (M,), F32, dev)
    lse = torch.empty(M, dtype=torch.float32, device=dev) if lse is None else lse
    loss = torch.empty(M, dtype=torch.float32, device=dev) if loss is None else loss
    _lib.check("coda_ce_reduce", _lib.load().coda_ce_reduce(
        M, V, _ptr(partials), _ptr(targets), _ptr(tgt_logit), _ptr(lse), _ptr(loss), _stream(stream)))
    return lse, loss


def rowscale_from_h(h, eps, r=None, stream=None):
    """r [M] = 1/sqrt(mean(h^2) + eps) of a stored bf16 h [M, N]."""
    M, N = _dims(h, "h", 2)
    dev = h.device
    _need(h, "h", (M, N), B16, dev)
    _need(r, "r", (M,), F32, dev)
    r = torch.empty(M, dtype=torch.float32, device=dev) if r is None else r
    _lib.check("coda_rowscale_from_h", _lib.load().coda_rowscale_from_h(M, N, _ptr(h), eps, _ptr(r), _stream(stream)))
    return r


def transpose_bf16(src, out=None, stream=None):
    """out [C, R] = src [R, C]^T (bf16)."""
    R, C = _dims(src, "src", 2)
    dev = src.device
    _need(src, "src", (R, C), B16, dev)
    _need(out, "out", (C, R), B16, dev)
    out = torch.empty((C, R), dtype=src.dtype, device=dev) if out is None else out
    _lib.check("coda_transpose_bf16", _lib.load().coda_transpose_bf16(R, C, _ptr(src), _ptr(out), _stream(stream)))
    return out


def gemm_swiglu_bwd(h, W, r, dy, dz=None, partials=None, stream=None):
    """Recompute h.W'^T and apply the SwiGLU backward: returns (dz [M, 2F] = r * dL/dz,
    partials [M, T] of dL/dr).  W [2F, K] (gate rows, then up rows), dy [M, F]."""
    M, K, F2, dev = _second_gemm_operands(h, W, r, None)
    _need(W, "W", (F2, K), B16, dev)
    if F2 % 2:
        raise ValueError("W: a SwiGLU weight needs an even number of rows")
    F = F2 // 2
    T = int(_lib.load().coda_swiglu_bwd_partials_per_row(F))
    _need(dy, "dy", (M, F), B16, dev, optional=False)
    _need(dz, "dz", (M, F2), B16, dev)
    _need(partials, "partials", (M, T), F32, dev)
    dz = torch.empty((M, F2), dtype=torch.bfloat16, device=dev) if dz is None else dz
    partials = torch.empty((M, T), dtype=torch.float32, device=dev) if partials is None else partials
    _lib.check("coda_gemm_swiglu_bwd", _lib.load().coda_gemm_swiglu_bwd(
        M, F, K, _ptr(h), _ptr(W), _ptr(r), _ptr(dy), _ptr(dz), _ptr(partials), _stream(stream)))
    return dz, partials


def rmsnorm_bwd_reduce(partials, r, N, F, q=None, stream=None):
    """q [M] = -(r^3 / N) * sum_t partials."""
    M = _dims(partials, "partials", 2)[0]
    dev = partials.device
    _need(partials, "partials", (M, int(_lib.load().coda_swiglu_bwd_partials_per_row(F))), F32, dev)
    _need(r, "r", (M,), F32, dev, optional=False)
    _need(q, "q", (M,), F32, dev)
    q = torch.empty(M, dtype=torch.float32, device=dev) if q is None else q
    _lib.check("coda_rmsnorm_bwd_reduce", _lib.load().coda_rmsnorm_bwd_reduce(
        M, N, F, _ptr(partials), _ptr(r), _ptr(q), _stream(stream)))
    return q


def gemm_rmsnorm_bwd(dz, Wt, h, q, dh_res=None, dh=None, stream=None):
    """dh [M, N] = dz . Wt^T + q * h (+ dh_res); Wt [N, K] = W'^T."""
    M, K = _dims(dz, "dz", 2)
    N, KW = _dims(Wt, "Wt", 2)
    if KW != K:
        raise ValueError("dz and Wt disagree on K")
    dev = dz.device
    _need(dz, "dz", (M, K), B16, dev)
    _need(Wt, "Wt", (N, K), B16, dev)
    _need(h, "h", (M, N), B16, dev)
    _need(q, "q", (M,), F32, dev)
    _need(dh_res, "dh_res", (M, N), B16, dev)
    _need(dh, "dh", (M, N), B16, dev)
    dh = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if dh is None else dh
    _lib.check("coda_gemm_rmsnorm_bwd", _lib.load().coda_gemm_rmsnorm_bwd(
        M, N, K, _ptr(dz), _ptr(Wt), _ptr(h), _ptr(q), _ptr(dh_res), _ptr(dh), _stream(stream)))
    return dh


def mlpin_bwd(h, Wp, Wpt, r, dy, dh_res=None, out=None, stream=None):
    """The three backward calls in order: returns (dh, dz, partials, q)."""
    out = out or {}
    dz, P = gemm_swiglu_bwd(h, Wp, r, dy, out.get("dz"), out.get("partials"), stream)
    q = rmsnorm_bwd_reduce(P, r, h.shape[1], Wp.shape[0] // 2, out.get("q"), stream)
    dh = gemm_rmsnorm_bwd(dz, Wpt, h, q, dh_res, out.get("dh"), stream)
    return dh, dz, P, q


def gemm_rowscale_gfold(h, W, gamma, r, act=SWIGLU, y=None, stream=None):
    """The second GEMM from the raw bf16 weight W with gamma folded in on chip
    (bit-identical to gemm_rowscale_swiglu with prepare_weight_bf16(W, gamma))."""
    M, K, n_w, dev = _second_gemm_operands(h, W, r, None)
    _need(W, "W", (n_w, K), B16, dev)
    _need(gamma, "gamma", (K,), F32, dev, optional=False)
    if act == SWIGLU and n_w % 2:
        raise ValueError("W: a SwiGLU weight needs an even number of rows")
    N_out = n_w // 2 if act == SWIGLU else n_w
    _need(y, "y", (M, N_out), B16, dev)
    y = torch.empty((M, N_out), dtype=torch.bfloat16, device=dev) if y is None else y
    _lib.check("coda_gemm_rowscale_gfold", _lib.load().coda_gemm_rowscale_gfold(
        M, N_out, K, act, _ptr(h), _ptr(W), _ptr(gamma), _ptr(r), _ptr(y), _stream(stream)))
    return y


def gemm_rowscale_swiglu_save(h, W, r, y=None, z=None, stream=None):
    """The SwiGLU second GEMM (bf16 W [2F, K]) that also keeps the pre-activation:
    returns (y [M, F], z [M, 2F] = r * (h . W^T) in bf16)."""
    M, K, F2, dev = _second_gemm_operands(h, W, r, None)
    _need(W, "W", (F2, K), B16, dev)
    if F2 % 2:
        raise ValueError("W: a SwiGLU weight needs an even number of rows")
    F = F2 // 2
    _need(y, "y", (M, F), B16, dev)
    _need(z, "z", (M, 2 * F), B16, dev)
    y = torch.empty((M, F), dtype=torch.bfloat16, device=dev) if y is None else y
    z = torch.empty((M, 2 * F), dtype=torch.bfloat16, device=dev) if z is None else z
    _lib.check("coda_gemm_rowscale_swiglu_save", _lib.load().coda_gemm_rowscale_swiglu_save(
        M, F, K, _ptr(h), _ptr(W), _ptr(r), _ptr(y), _ptr(z), _stream(stream)))
    return y, z


def swiglu_bwd_saved(z, dy, r, dz=None, dzt=None, partials=None, transpose=True, stream=None):
    """SwiGLU backward from the saved z [M, 2F]: returns (dz [M, 2F] = r * dL/dz,
    dzt [2F, M] (its transpose; None with transpose=False), partials [M, T])."""
    M, F2 = _dims(z, "z", 2)
    dev = z.device
    if F2 % 2:
        raise ValueError("z needs an even number of columns (gate, then up)")
    F = F2 // 2
    T = int(_lib.load().coda_swiglu_bwd_partials_per_row(F))
    _need(z, "z", (M, F2), B16, dev)
    _need(dy, "dy", (M, F), B16, dev, optional=False)
    _need(r, "r", (M,), F32, dev, optional=False)
    _need(dz, "dz", (M, F2), B16, dev)
    _need(dzt if transpose else None, "dzt", (F2, M), B16, dev)
    _need(partials, "partials", (M, T), F32, dev)
    dz = torch.empty((M, F2), dtype=torch.bfloat16, device=dev) if dz is None else dz
    if transpose and dzt is None:
        dzt = torch.empty((F2, M), dtype=torch.bfloat16, device=dev)
    partials = torch.empty((M, T), dtype=torch.float32, device=dev) if partials is None else partials
    _lib.check("coda_swiglu_bwd_saved", _lib.load().coda_swiglu_bwd_saved(
        M, F, _ptr(z), _ptr(dy), _ptr(r), _ptr(dz), _ptr(dzt if transpose else None), _ptr(partials),
        _stream(stream)))
    return dz, (dzt if transpose else None), partials


def rope_bwd(dy, y, r, pos, cos, sin, rot_cols, dz=None, partials=None, stream=None):
    """Backward of the RoPE epilogue from the forward's output y [M, N]: returns (dz
    [M, N] = r * RoPE^T(dy) in bf16, partials [M, T] = per 128-column tile
    (1/r) * sum of dy * y, the layout rmsnorm_bwd_reduce takes with F = N)."""
    M, N = _dims(dy, "dy", 2)
    dev = dy.device
    _need(dy, "dy", (M, N), B16, dev)
    _need(y, "y", (M, N), B16, dev, optional=False)
    _need(r, "r", (M,), F32, dev, optional=False)
    rows = _rope_operands(M, pos, cos, sin, dev)
    T = int(_lib.load().coda_swiglu_bwd_partials_per_row(N))
    _need(dz, "dz", (M, N), B16, dev)
    _need(partials, "partials", (M, T), F32, dev)
    dz = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if dz is None else dz
    partials = torch.empty((M, T), dtype=torch.float32, device=dev) if partials is None else partials
    _lib.check("coda_rope_bwd", _lib.load().coda_rope_bwd(
        M, N, _ptr(dy), _ptr(y), _ptr(r), _ptr(pos), _ptr(cos), _ptr(sin), rows, rot_cols, _ptr(dz),
        _ptr(partials), _stream(stream)))
    return dz, partials


def qkv_rope_bwd(h, r, Wpt, W, gamma, dy, y, pos, cos, sin, rot_cols, dh_res=None, out=None, stream=None):
    """Backward of the QKV block y = RoPE(RMSNorm(h) . W^T) from the forward's h, r and y:
    the RoPE backward, the row coefficient, the input-gradient GEMM (Wpt = W'^T [d, N])
    and the weight / gamma gradients on dz and h as stored.  Returns dict(dh, dW [N, d]
    fp32, dgamma [d] fp32, dz, q)."""
    out = out or {}
    dz, P = rope_bwd(dy, y, r, pos, cos, sin, rot_cols, out.get("dz"), out.get("partials"), stream)
    q = rmsnorm_bwd_reduce(P, r, h.shape[1], dy.shape[1], out.get("q"), stream)
    dh = gemm_rmsnorm_bwd(dz, Wpt, h, q, dh_res, out.get("dh"), stream)
    dW, dgam = mlpin_wgrad(dz, h, gamma, W, out=out, stream=stream)
    return dict(dh=dh, dW=dW, dgamma=dgam, dz=dz, q=q)


def gemm_ce_bwd(h, W, r, targets, lse, g, dz=None, partials=None, stream=None):
    """The LM-head product recomputed with the cross-entropy backward in its epilogue:
    returns (dz [M, V] = r * g * (softmax - onehot) in bf16 (zero rows for ignored
    targets), partials [M, T] = per 128 columns sum of dL/dz * acc, the layout
    rmsnorm_bwd_reduce takes with F = V).  W [V, K] is the gamma-folded weight."""
    M, K, V, dev = _second_gemm_operands(h, W, r, None)
    _need(W, "W", (V, K), B16, dev)
    _need(targets, "targets", (M,), I32, dev, optional=False)
    _need(lse, "lse", (M,), F32, dev, optional=False)
    _need(g, "g", (M,), F32, dev, optional=False)
    T = int(_lib.load().coda_swiglu_bwd_partials_per_row(V))
    _need(dz, "dz", (M, V), B16, dev)
    _need(partials, "partials", (M, T), F32, dev)
    dz = torch.empty((M, V), dtype=torch.bfloat16, device=dev) if dz is None else dz
    partials = torch.empty((M, T), dtype=torch.float32, device=dev) if partials is None else partials
    _lib.check("coda_gemm_ce_bwd", _lib.load().coda_gemm_ce_bwd(
        M, V, K, _ptr(h), _ptr(W), _ptr(r), _ptr(targets), _ptr(lse), _ptr(g), _ptr(dz), _ptr(partials),
        _stream(stream)))
    return dz, partials


def lmhead_ce_bwd(h, r, Wp, Wpt, W, gamma, targets, lse, g, dh_res=None, out=None, stream=None):
    """Backward of the LM-head block from the forward's h, r and lse: the recomputed
    product with the loss backward, the row coefficient, the input-gradient GEMM (Wpt =
    W'^T [d, V]) and the weight / gamma gradients on dz and h as stored.  Returns dict(dh,
    dW [V, d] fp32, dgamma [d] fp32, dz, q)."""
    out = out or {}
    dz, P = gemm_ce_bwd(h, Wp, r, targets, lse, g, out.get("dz"), out.get("partials"), stream)
    q = rmsnorm_bwd_reduce(P, r, h.shape[1], Wp.shape[0], out.get("q"), stream)
    dh = gemm_rmsnorm_bwd(dz, Wpt, h, q, dh_res, out.get("dh"), stream)
    dW, dgam = mlpin_wgrad(dz, h, gamma, W, out=out, stream=stream)
    return dict(dh=dh, dW=dW, dgamma=dgam, dz=dz, q=q)


def gemm_bf16(A, Bt, c_res=None, C=None, stream=None):
    """C [M, N] = A [M, K] . Bt [N, K]^T (+ c_res) in bf16 (fp32 sums)."""
    M, K = _dims(A, "A", 2)
    N, KB = _dims(Bt, "Bt", 2)
    if KB != K:
        raise ValueError("A and Bt disagree on K")
    dev = A.device
    _need(A, "A", (M, K), B16, dev)
    _need(Bt, "Bt", (N, K), B16, dev)
    _need(c_res, "c_res", (M, N), B16, dev)
    _need(C, "C", (M, N), B16, dev)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if C is None else C
    _lib.check("coda_gemm_bf16", _lib.load().coda_gemm_bf16(
        M, N, K, _ptr(A), _ptr(Bt), _ptr(c_res), _ptr(C), _stream(stream)))
    return C


def wgrad_partials_rows(NR: int) -> int:
    return int(_lib.load().coda_wgrad_partials_rows(NR))


def wgrad_workspace_bytes(NR: int, NC: int, K: int) -> int:
    return int(_lib.load().coda_wgrad_workspace_bytes(NR, NC, K))


def _wgrad_outputs(NR, NC, gamma, W, dW, partials, workspace, dev):
    """Checks shared by the weight-gradient calls; returns (dW, partials) allocated where
    the caller gave none."""
    _need(gamma, "gamma", (NC,), F32, dev)
    _need(W, "W", (NR, NC), B16, dev)
    _need(dW, "dW", (NR, NC), F32, dev)
    TW = wgrad_partials_rows(NR)
    _need(partials if W is not None else None, "partials", (TW, NC), F32, dev)
    if workspace is not None and not isinstance(workspace, str):
        _need(workspace, "workspace", None, (torch.uint8,), dev)
    dW = torch.empty((NR, NC), dtype=torch.float32, device=dev) if dW is None else dW
    if W is not None and partials is None:
        partials = torch.empty((TW, NC), dtype=torch.float32, device=dev)
    return dW, partials


def gemm_wgrad(At, Bt, gamma=None, W=None, dW=None, partials=None, workspace=None, stream=None):
    """dW [NR, NC] fp32 = gamma * (At . Bt^T), a sum over the K tokens of At [NR, K] and
    Bt [NC, K]; with the raw weight W [NR, NC] also the per-256-row-tile partials of the
    gamma gradient sum_j W[j,k] * G[j,k] (else partials is None).  A device
    ``workspace`` (uint8 tensor) of wgrad_workspace_bytes(NR, NC, K) bytes, when that is
    nonzero, lets the tokens be split over more blocks; workspace="auto" allocates it."""
    NR, K = _dims(At, "At", 2)
    NC, KB = _dims(Bt, "Bt", 2)
    if KB != K:
        raise ValueError("At and Bt disagree on K")
    dev = At.device
    _need(At, "At", (NR, K), B16, dev)
    _need(Bt, "Bt", (NC, K), B16, dev)
    dW, partials = _wgrad_outputs(NR, NC, gamma, W, dW, partials, workspace, dev)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be a tensor, None or 'auto'")
        n = wgrad_workspace_bytes(NR, NC, K)
        workspace = torch.empty(n, dtype=torch.uint8, device=dev) if n > 0 else None
    _lib.check("coda_gemm_wgrad", _lib.load().coda_gemm_wgrad(
        NR, NC, K, _ptr(At), _ptr(Bt), _ptr(gamma), _ptr(W), _ptr(dW),
        _ptr(partials) if W is not None else None, _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream)))
    return dW, (partials if W is not None else None)


def gemm_wgrad_tok(X, Y, gamma=None, W=None, dW=None, partials=None, workspace=None, NR=None, NC=None,
                   stream=None):
    """dW [NR, NC] fp32 = gamma * (X^T . Y), the sum over the K token rows of the token-major
    X [K, lda] (its first NR columns, default all) and Y [K, ldb] (first NC columns): the
    weight gradient without transposed copies.  W, partials and workspace as gemm_wgrad."""
    K, lda = _dims(X, "X", 2)
    KY, ldb = _dims(Y, "Y", 2)
    if KY != K:
        raise ValueError("X and Y disagree on the token count")
    dev = X.device
    _need(X, "X", (K, lda), B16, dev)
    _need(Y, "Y", (K, ldb), B16, dev)
    NR = lda if NR is None else NR
    NC = ldb if NC is None else NC
    if not (0 < NR <= lda and 0 < NC <= ldb):
        raise ValueError(f"NR, NC = {NR}, {NC} must lie in (0, {lda}] and (0, {ldb}]")
    dW, partials = _wgrad_outputs(NR, NC, gamma, W, dW, partials, workspace, dev)
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be a tensor, None or 'auto'")
        n = int(_lib.load().coda_wgrad_tok_workspace_bytes(NR, NC, K, lda, ldb))
        workspace = torch.empty(n, dtype=torch.uint8, device=dev) if n > 0 else None
    _lib.check("coda_gemm_wgrad_tok", _lib.load().coda_gemm_wgrad_tok(
        NR, NC, K, _ptr(X), lda, _ptr(Y), ldb, _ptr(gamma), _ptr(W), _ptr(dW),
        _ptr(partials) if W is not None else None, _ptr(workspace),
        0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream)))
    return dW, (partials if W is not None else None)


def gemm_wgrad_tok_noalloc(X, Y, gamma=None, W=None, dW=None, partials=None, NR=None, NC=None, stream=None):
    """gemm_wgrad_tok for callers that cannot allocate: the token split (when taken) runs
    in the library's static per-device scratch instead of a workspace.  Bit-identical
    to gemm_wgrad_tok with a sufficient workspace; calls that overlap on one GPU race."""
    K, lda = _dims(X, "X", 2)
    KY, ldb = _dims(Y, "Y", 2)
    if KY != K:
        raise ValueError("X and Y disagree on the token count")
    dev = X.device
    _need(X, "X", (K, lda), B16, dev)
    _need(Y, "Y", (K, ldb), B16, dev)
    NR = lda if NR is None else NR
    NC = ldb if NC is None else NC
    if not (0 < NR <= lda and 0 < NC <= ldb):
        raise ValueError(f"NR, NC = {NR}, {NC} must lie in (0, {lda}] and (0, {ldb}]")
    dW, partials = _wgrad_outputs(NR, NC, gamma, W, dW, partials, None, dev)
    _lib.check("coda_gemm_wgrad_tok_noalloc", _lib.load().coda_gemm_wgrad_tok_noalloc(
        NR, NC, K, _ptr(X), lda, _ptr(Y), ldb, _ptr(gamma), _ptr(W), _ptr(dW),
        _ptr(partials) if W is not None else None, _stream(stream)))
    return dW, (partials if W is not None else None)


def colsum_reduce(partials, out=None, stream=None):
    """out [NC] = sum over the rows of partials [T, NC] (fixed order, fp64 inside)."""
    T, NC = _dims(partials, "partials", 2)
    dev = partials.device
    _need(partials, "partials", (T, NC), F32, dev)
    _need(out, "out", (NC,), F32, dev)
    out = torch.empty(NC, dtype=torch.float32, device=dev) if out is None else out
    _lib.check("coda_colsum_reduce", _lib.load().coda_colsum_reduce(T, NC, _ptr(partials), _ptr(out), _stream(stream)))
    return out


def mlpin_wgrad(dz, h, gamma, W, dzt=None, ht=None, out=None, stream=None):
    """Weight gradients of the MLP-input block from the backward's dz = r * dL/dz [M, 2F]
    and the block input h [M, d]: returns (dW [2F, d], dgamma [d]) for the raw weight
    W [2F, d] and gamma [d].  The GEMM reads dz and h as stored (token-major); with both
    dzt and ht given it reads those transposed copies instead."""
    out = out or {}
    ws = out.get("wws", "auto")      # a token split when the weight has few 256-row tiles
    if dzt is not None and ht is not None:
        dW, P = gemm_wgrad(dzt, ht, gamma, W, out.get("dW"), out.get("wpartials"), ws, stream=stream)
    else:
        dW, P = gemm_wgrad_tok(dz, h, gamma, W, out.get("dW"), out.get("wpartials"), ws, stream=stream)
    dgam = colsum_reduce(P, out.get("dgamma"), stream)
    return dW, dgam


def chain_bwd(A, WoT, h, r, Wp, Wpt, W, gamma, dy, dres=None, z=None, out=None, stream=None):
    """Backward of the whole chain h = x_res + A . Wo^T -> r -> y = SwiGLU(r (h . W'^T))
    from the forward's saved h and r: returns dict(dh (also the gradient of x_res), dA,
    dWo [d, K1] fp32, dW [2F, d] fp32, dgamma [d] fp32).  WoT = Wo^T [K1, d] and
    Wpt = W'^T [d, 2F] are the weight transposes (once per weight update); W is the raw
    second weight, gamma the RMSNorm weight; dres the gradient reaching h through the
    residual stream (None = 0).  With the pre-activation z saved by
    gemm_rowscale_swiglu_save the gate/up product is not recomputed (Wp unused)."""
    out = out or {}
    if z is None:
        dh, dz, _, _ = mlpin_bwd(h, Wp, Wpt, r, dy, dres, out, stream)
    else:
        dz, _, P = swiglu_bwd_saved(z, dy, r, out.get("dz"), None, out.get("partials"), False, stream)
        q = rmsnorm_bwd_reduce(P, r, h.shape[1], z.shape[1] // 2, out.get("q"), stream)
        dh = gemm_rmsnorm_bwd(dz, Wpt, h, q, dres, out.get("dh"), stream)
    # the weight gradients read dz, h, dh and A as stored (token-major): no transposes
    dW, dgam = mlpin_wgrad(dz, h, gamma, W, out=out, stream=stream)
    dA = gemm_bf16(dh, WoT, None, out.get("dA"), stream)
    dWo, _ = gemm_wgrad_tok(dh, A, None, None, out.get("dWo"), None, out.get("ws", "auto"), stream=stream)
    return dict(dh=dh, dA=dA, dWo=dWo, dW=dW, dgamma=dgam)


def chain(A, Wo_t, x_res, Wp_t, eps, act=SWIGLU, a_scale=None, wo_scale=None, wp_scale=None,
          out=None, stream=None, save_z=False):
    """The three calls in order on one stream.  Returns (h, P, r, y), and z last with
    save_z=True (bf16 SwiGLU only: the pre-activation a backward can start from).

    ``out`` may hold preallocated h, partials, r, y, z tensors (dict)."""
    out = out or {}
    h, P = gemm_resid_partialrms(A, Wo_t, x_res, a_scale, wo_scale, out.get("h"),
                                 out.get("partials"), stream)
    r = rowscale_reduce(P, Wo_t.shape[0], eps, out.get("r"), stream)
    if save_z:
        if act != SWIGLU or wp_scale is not None:
            raise ValueError("save_z needs the bf16 SwiGLU chain")
        y, z = gemm_rowscale_swiglu_save(h, Wp_t, r, out.get("y"), out.get("z"), stream)
        return h, P, r, y, z
    y = gemm_rowscale_swiglu(h, Wp_t, r, act, wp_scale, out.get("y"), stream)
    return h, P, r, y

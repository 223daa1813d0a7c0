"""ctypes wrapper around the fp64 C oracle (``coda_oracle.c``).

TEST INFRASTRUCTURE ONLY (tests, smoke check, the bench's CPU-baseline leg).

The C file is compiled with gcc on first use (or by ``build()``) into
``oracle/liborcl.so``; no part of the HIP library is involved.
"""

from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "coda_oracle.c")
# ORC_LIB: a separately built copy (the sanitizer build of the tests) is loaded as is
_LIB = os.environ.get("ORC_LIB") or os.path.join(_HERE, "liborcl.so")

BF16 = 0
E4M3 = 1
ACT_NONE = 0
ACT_SWIGLU = 1

__all__ = ["build", "lib", "max_threads", "bf16_decode", "bf16_encode", "e4m3_decode",
           "e4m3_encode", "fold_bf16", "quant_e4m3", "rope", "rope_transpose", "cross_entropy", "mlpin_bwd",
           "mlpin_wgrad", "chain_bwd", "qkv_rope_bwd", "lmhead_ce_bwd", "chain", "chain_textbook", "prepare", "BF16", "E4M3",
           "ACT_NONE", "ACT_SWIGLU"]


def build(force: bool = True) -> str:
    """Compile the oracle (plain C, fp64, OpenMP, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                               "-std=c11", "-Wall", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.environ.get("ORC_LIB"):
            build(force=False)
        L = C.CDLL(_LIB)
        P = C.c_void_p
        i64 = C.c_int64
        L.orc_max_threads.restype = C.c_int
        L.orc_bf16_decode.restype = C.c_double
        L.orc_bf16_decode.argtypes = [C.c_uint16]
        L.orc_bf16_encode_rne.restype = C.c_uint16
        L.orc_bf16_encode_rne.argtypes = [C.c_double]
        L.orc_e4m3_decode.restype = C.c_double
        L.orc_e4m3_decode.argtypes = [C.c_uint8]
        L.orc_e4m3_encode_sat_rne.restype = C.c_uint8
        L.orc_e4m3_encode_sat_rne.argtypes = [C.c_double]
        for f in ("orc_bf16_decode_n", "orc_bf16_encode_n", "orc_e4m3_decode_n", "orc_e4m3_encode_n"):
            getattr(L, f).restype = None
            getattr(L, f).argtypes = [i64, P, P]
        L.orc_fold_bf16.restype = None
        L.orc_fold_bf16.argtypes = [i64, i64, P, P, P]
        L.orc_quant_e4m3.restype = None
        L.orc_quant_e4m3.argtypes = [i64, i64, P, P, P, P, P]
        L.orc_mlpin_bwd.restype = C.c_int
        L.orc_mlpin_bwd.argtypes = [i64, P, i64, i64, P, P, P, C.c_int, C.c_double, P, C.c_double, P, P, P]
        L.orc_mlpin_wgrad.restype = C.c_int
        L.orc_mlpin_wgrad.argtypes = [i64, i64, i64, P, P, P, C.c_int, C.c_double, P, P, C.c_double,
                                      i64, P, i64, P, P, P, P, P]
        L.orc_cross_entropy.restype = C.c_int
        L.orc_cross_entropy.argtypes = [i64, i64, P, P, P, P]
        L.orc_rope.restype = C.c_int
        L.orc_rope.argtypes = [i64, i64, P, P, C.c_double, i64, i64]
        L.orc_chain.restype = C.c_int
        L.orc_chain.argtypes = [i64, P, i64, i64, i64, C.c_int,
                                P, C.c_int, C.c_double,
                                P, C.c_int, C.c_double,
                                P, P, P, C.c_int, C.c_double, C.c_double,
                                P, P, P, P, P]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def max_threads() -> int:
    return int(lib().orc_max_threads())


def bf16_decode(c) -> np.ndarray:
    c = np.ascontiguousarray(c, dtype=np.uint16)
    out = np.empty(c.shape, np.float64)
    lib().orc_bf16_decode_n(c.size, _p(c), _p(out))
    return out


def bf16_encode(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    lib().orc_bf16_encode_n(x.size, _p(x), _p(out))
    return out


def e4m3_decode(c) -> np.ndarray:
    c = np.ascontiguousarray(c, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().orc_e4m3_decode_n(c.size, _p(c), _p(out))
    return out


def e4m3_encode(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint8)
    lib().orc_e4m3_encode_n(x.size, _p(x), _p(out))
    return out


def fold_bf16(W_t: np.ndarray, gamma: np.ndarray | None) -> np.ndarray:
    """W'[n,k] = bf16_rne(fl32(gamma[k] * W[n,k])), W_t [N, K] bf16 bits."""
    W_t = np.ascontiguousarray(W_t, dtype=np.uint16)
    N, K = W_t.shape
    g = None if gamma is None else np.ascontiguousarray(gamma, dtype=np.float32)
    out = np.empty((N, K), np.uint16)
    lib().orc_fold_bf16(N, K, _p(W_t), _p(g), _p(out))
    return out


def quant_e4m3(W_t: np.ndarray, gamma: np.ndarray | None):
    """Per-tensor e4m3 quantisation of fl32(gamma*W) (gamma None: of W itself).

    Returns (codes uint8 [N, K], amax float32, scale float32)."""
    W_t = np.ascontiguousarray(W_t, dtype=np.uint16)
    N, K = W_t.shape
    g = None if gamma is None else np.ascontiguousarray(gamma, dtype=np.float32)
    out = np.empty((N, K), np.uint8)
    amax = np.zeros(1, np.float32)
    scale = np.zeros(1, np.float32)
    lib().orc_quant_e4m3(N, K, _p(W_t), _p(g), _p(out), _p(amax), _p(scale))
    return out, np.float32(amax[0]), np.float32(scale[0])


def prepare(inputs: dict, dtype: str) -> dict:
    """The oracle's own weight/activation preparation for a workload.

    bf16: Wp = fold_bf16(W_t, gamma); scales 1.
    e4m3: A, Wo_t quantised per tensor; Wp = quant_e4m3(W_t, gamma) (fold first).
    Returns dict(A, a_dt, a_scale, Wo, wo_dt, wo_scale, Wp, wp_dt, wp_scale)."""
    if dtype == "bf16":
        return dict(A=inputs["A"], a_dt=BF16, a_scale=1.0, Wo=inputs["Wo_t"], wo_dt=BF16,
                    wo_scale=1.0, Wp=fold_bf16(inputs["W_t"], inputs["gamma"]), wp_dt=BF16,
                    wp_scale=1.0)
    if dtype == "e4m3":
        qa, _, sa = quant_e4m3(inputs["A"], None)
        qo, _, so = quant_e4m3(inputs["Wo_t"], None)
        qw, _, sw = quant_e4m3(inputs["W_t"], inputs["gamma"])
        return dict(A=qa, a_dt=E4M3, a_scale=float(sa), Wo=qo, wo_dt=E4M3, wo_scale=float(so),
                    Wp=qw, wp_dt=E4M3, wp_scale=float(sw))
    raise ValueError(dtype)


def chain(prep: dict, x_res, gamma, act: int, eps: float, rows=None, M: int | None = None):
    """Run the unfused fp64 chain on the listed rows (default: all M rows).

    ``prep`` is the output of :func:`prepare`.  Returns dict(h, hb, S, r, y) with one
    entry per computed row: h fp64 [R, d] (unrounded), hb uint16 [R, d] (bf16 bits),
    S fp64 [R] = sum hb^2, r fp64 [R], y fp64 [R, n_out]."""
    A = np.ascontiguousarray(prep["A"])
    Wo = np.ascontiguousarray(prep["Wo"])
    Wp = np.ascontiguousarray(prep["Wp"])
    M = A.shape[0] if M is None else M
    K1 = A.shape[1]
    d = Wo.shape[0]
    N2w = Wp.shape[0]
    if Wo.shape[1] != K1 or Wp.shape[1] != d:
        raise ValueError("shape mismatch")
    if rows is None:
        rows_a = None
        R = M
    else:
        rows_a = np.ascontiguousarray(rows, dtype=np.int64)
        R = rows_a.size
    n_out = N2w // 2 if act == ACT_SWIGLU else N2w
    xr = None if x_res is None else np.ascontiguousarray(x_res, dtype=np.uint16)
    g = np.ascontiguousarray(gamma, dtype=np.float32)
    h = np.empty((R, d), np.float64)
    hb = np.empty((R, d), np.uint16)
    S = np.empty(R, np.float64)
    r = np.empty(R, np.float64)
    y = np.empty((R, n_out), np.float64)
    rc = lib().orc_chain(R, _p(rows_a), K1, d, N2w, act,
                         _p(A), prep["a_dt"], prep["a_scale"],
                         _p(Wo), prep["wo_dt"], prep["wo_scale"],
                         _p(xr), _p(g), _p(Wp), prep["wp_dt"], prep["wp_scale"], eps,
                         _p(h), _p(hb), _p(S), _p(r), _p(y))
    if rc != 0:
        raise RuntimeError(f"oracle chain failed ({rc})")
    return dict(h=h, hb=hb, S=S, r=r, y=y)


def chain_textbook(inputs: dict, act: int, eps: float, rows=None, round_h: bool = False) -> dict:
    """The chain as a model defines it, before any reparameterisation or preparation:
    the raw second weight, gamma inside RMSNorm, and (by default) no rounding of the
    residual stream -- the reference the pages' numerics claim is about (kucoin page,
    section "Resultados del experimento", last paragraph: the reparameterised chain's
    error is comparable to the unfused PyTorch chain's, sometimes lower).  Plain fp64
    numpy on the decoded bf16 inputs (the pre-quantisation ones for an 8-bit workload),
    in the order the pages give the chain (kucoin, section "CODA: El epilogo esconde un
    tesoro"):
      t = A . Wo^T,  h = x_res + t            (round_h: h = bf16_rne(h), as the chain stores it)
      r = 1 / sqrt(mean_n(h^2) + eps),  n = h * r * gamma
      z = n . W^T                             (W the raw second weight, [N2w, d])
      NONE: y = z;  SWIGLU: y = silu(z[:, :F]) * z[:, F:],  silu(g) = g / (1 + exp(-g))
    Returns dict(h, r, y) for the listed rows (all rows by default)."""
    A = inputs["A"] if rows is None else inputs["A"][rows]
    xr = inputs["x_res"] if rows is None else inputs["x_res"][rows]
    a = bf16_decode(A)
    wo = bf16_decode(inputs["Wo_t"])
    h = bf16_decode(xr) + a @ wo.T
    if round_h:
        h = bf16_decode(bf16_encode(h))
    d = h.shape[1]
    r = 1.0 / np.sqrt((h * h).sum(1) / d + eps)
    n = h * r[:, None] * inputs["gamma"].astype(np.float64)[None, :]
    z = n @ bf16_decode(inputs["W_t"]).T
    if act == ACT_SWIGLU:
        F = z.shape[1] // 2
        g, u = z[:, :F], z[:, F:]
        with np.errstate(over="ignore"):          # exp(-g) = inf for g << 0 gives silu = -0
            y = g / (1.0 + np.exp(-g)) * u
    else:
        y = z
    return dict(h=h, r=r, y=y)


def rope(y: np.ndarray, pos, base: float, head_dim: int, rot_cols: int) -> np.ndarray:
    """RoPE of the chain output: a rotated copy of ``y`` (fp64 [R, ncols]), row i at
    position ``pos[i]``; columns [0, rot_cols) are heads of ``head_dim`` values (pair
    i, i + head_dim/2 rotated by pos * base^(-2i/head_dim)), the rest pass through."""
    out = np.array(y, dtype=np.float64, order="C", copy=True)
    p = np.ascontiguousarray(pos, dtype=np.int32)
    if out.ndim != 2 or p.shape != (out.shape[0],):
        raise ValueError("y must be [R, ncols] and pos [R]")
    rc = lib().orc_rope(out.shape[0], out.shape[1], _p(out), _p(p), float(base), int(head_dim), int(rot_cols))
    if rc != 0:
        raise ValueError("bad RoPE layout")
    return out


def rope_transpose(dy: np.ndarray, pos, base: float, head_dim: int, rot_cols: int) -> np.ndarray:
    """The transpose of the RoPE rotation applied to ``dy`` (fp64 [R, ncols]): the
    gradient with respect to RoPE's input given the gradient ``dy`` of its output.  Per
    rotated head, for i < head_dim/2 with angle a = pos * base^(-2i/head_dim):
      forward   y_i = x_i cos a - x_{i+h} sin a,   y_{i+h} = x_{i+h} cos a + x_i sin a
      transpose dx_i = dy_i cos a + dy_{i+h} sin a,   dx_{i+h} = dy_{i+h} cos a - dy_i sin a
    (h = head_dim/2); columns [rot_cols, ncols) pass through.  Plain fp64 numpy."""
    g = np.array(dy, dtype=np.float64, copy=True)
    p = np.asarray(pos, dtype=np.float64)
    if g.ndim != 2 or p.shape != (g.shape[0],) or rot_cols % head_dim or rot_cols > g.shape[1]:
        raise ValueError("bad RoPE layout")
    half = head_dim // 2
    i = np.arange(half, dtype=np.float64)
    a = p[:, None] * base ** (-2.0 * i / head_dim)[None, :]            # [R, half]
    c, s = np.cos(a), np.sin(a)
    for h0 in range(0, rot_cols, head_dim):
        lo, hi = dy[:, h0:h0 + half].astype(np.float64), dy[:, h0 + half:h0 + head_dim].astype(np.float64)
        g[:, h0:h0 + half] = lo * c + hi * s
        g[:, h0 + half:h0 + head_dim] = hi * c - lo * s
    return g


def qkv_rope_bwd(hb, gamma, Wp, wp_scale: float, W_raw, dy, pos, base: float, head_dim: int,
                 rot_cols: int, eps: float, rows=None, js=None, ks=None, rss=False):
    """Backward of the QKV block  y = RoPE( RMSNorm(hb) . W_or^T )  (kucoin page, section
    "CODA: El epilogo esconde un tesoro", last paragraph: the reparameterisation covers
    RoPE and holds for the backward pass).  The chain rule in reverse order, plain fp64:
      forward   r = 1/sqrt(mean(hb^2) + eps),  n = hb r gamma,  z = n . W_or^T,
                y = RoPE(z)                      (W_or = Wp * wp_scale / gamma, the weight
                                                  the prepared Wp stands for)
      RoPE      dz = RoPE^T(dy)                  (:func:`rope_transpose`)
      GEMM      dn = dz . W_or;   dW[j, k] = sum_m dz[m, j] n[m, k]   (the raw weight's)
      RMSNorm   dhb[k] = r gamma[k] dn[k] - (r^3 / d) hb[k] sum_k' gamma[k'] dn[k'] hb[k']
                dgamma[k] = sum_m sum_j dz[m, j] W_raw[j, k] hb[m, k] r[m]
    hb uint16 [M, d] and dy uint16 [M, N] bf16 codes, gamma fp32 [d], Wp uint16 [N, d]
    (bf16 codes of the gamma-folded weight), W_raw uint16 [N, d], pos int [M].

    Returns dict(dh [R, d], r [R], dz [R, N]) for the listed rows (default all), dW
    [nj, nk] summed over all M tokens at rows js of W (default all N) and columns ks
    (default all d), dgamma [nk] when js covers every row (else None), and with rss=True
    the root-sum-squares over the tokens of the summed terms, rss [nj, nk] (gamma left
    out) and rss_gamma [nk] (full js only)."""
    hbv = bf16_decode(np.asarray(hb, dtype=np.uint16))
    dyv = bf16_decode(np.asarray(dy, dtype=np.uint16))
    g = np.asarray(gamma, dtype=np.float64)
    wor = bf16_decode(np.asarray(Wp, dtype=np.uint16)) * float(wp_scale) / g[None, :]
    wraw = bf16_decode(np.asarray(W_raw, dtype=np.uint16))
    M, d = hbv.shape
    N = wor.shape[0]
    if wor.shape != (N, d) or wraw.shape != (N, d) or dyv.shape != (M, N) or g.shape != (d,):
        raise ValueError("shape mismatch")
    r = 1.0 / np.sqrt((hbv * hbv).sum(axis=1) / d + eps)               # [M]
    dz_all = rope_transpose(dyv, pos, base, head_dim, rot_cols)      # [M, N]
    rr = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    dz = dz_all[rr]
    dn = dz @ wor                                                    # [R, d]
    hr, rv = hbv[rr], r[rr]
    c = (g[None, :] * dn * hr).sum(axis=1)
    dh = rv[:, None] * g[None, :] * dn - (rv ** 3 / d)[:, None] * hr * c[:, None]
    j = np.arange(N) if js is None else np.asarray(js, dtype=np.int64)
    k = np.arange(d) if ks is None else np.asarray(ks, dtype=np.int64)
    t = dz_all[:, j]                                                 # [M, nj]
    hk = hbv[:, k] * r[:, None]                                      # [M, nk]: hb r
    dW = (t.T @ hk) * g[k][None, :]
    dgam = None
    if js is None:
        dgam = ((dz_all @ wraw[:, k]) * hk).sum(axis=0)
    out = dict(dh=dh, r=rv, dz=dz, dW=dW, dgamma=dgam)
    if rss:
        out["rss"] = np.sqrt((t * t).T @ (hk * hk))
        out["rss_gamma"] = None
        if js is None:
            out["rss_gamma"] = np.sqrt((((dz_all * dz_all) @ (wraw[:, k] * wraw[:, k])) * hk * hk).sum(axis=0))
    return out


def lmhead_ce_bwd(hb, gamma, Wp, wp_scale: float, W_raw, targets, g, eps: float, rows=None, js=None, ks=None,
                  rss=False):
    """Backward of the LM-head block  loss_m = CE( RMSNorm(hb) . W_or^T, t_m )  weighted by
    g[m] = d(total loss)/d(loss_m) (kucoin page, section "CODA: El epilogo esconde un
    tesoro", last paragraph: the reparameterisation covers the cross-entropy loss and
    holds for the backward pass).  The chain rule in reverse order, plain fp64:
      forward   r = 1/sqrt(mean(hb^2) + eps),  n = hb r gamma,  z = n . W_or^T,
                lse = log sum_v exp z_v,  loss = lse - z_t   (0 for t outside [0, V))
      loss      dz_v = g (softmax(z)_v - [v == t])           (0 for an ignored row)
      GEMM      dn = dz . W_or;   dW[j, k] = sum_m dz[m, j] n[m, k]   (the raw weight's)
      RMSNorm   dhb[k] = r gamma[k] dn[k] - (r^3 / d) hb[k] sum_k' gamma[k'] dn[k'] hb[k']
                dgamma[k] = sum_m sum_j dz[m, j] W_raw[j, k] hb[m, k] r[m]
    (W_or = Wp * wp_scale / gamma.)  hb uint16 [M, d] bf16 codes, gamma fp32 [d], Wp and
    W_raw uint16 [V, d], targets int [M], g float [M].

    Returns dict(dh [R, d], r [R], dz [R, V], lse [R]) for the listed rows (default all);
    with js given (a list of weight rows, or "all") also dW [nj, nk] summed over all M
    tokens at columns ks (default all d), dgamma [nk] for js == "all", and with rss=True
    the root-sum-squares of their terms (rss [nj, nk] with gamma left out, rss_gamma).
    The weight gradient needs the softmax of every token's logits (M V d operations)."""
    hbv = bf16_decode(np.asarray(hb, dtype=np.uint16))
    g_ = np.asarray(gamma, dtype=np.float64)
    wor = bf16_decode(np.asarray(Wp, dtype=np.uint16)) * float(wp_scale) / g_[None, :]
    wraw = bf16_decode(np.asarray(W_raw, dtype=np.uint16))
    t = np.asarray(targets, dtype=np.int64)
    gw = np.asarray(g, dtype=np.float64)
    M, d = hbv.shape
    V = wor.shape[0]
    if wor.shape != (V, d) or wraw.shape != (V, d) or t.shape != (M,) or gw.shape != (M,) or g_.shape != (d,):
        raise ValueError("shape mismatch")
    r_all = 1.0 / np.sqrt((hbv * hbv).sum(axis=1) / d + eps)

    def dlogits(idx):
        n = hbv[idx] * r_all[idx, None] * g_[None, :]
        z = n @ wor.T
        mx = z.max(axis=1, keepdims=True)
        lse = mx[:, 0] + np.log(np.exp(z - mx).sum(axis=1))
        p = np.exp(z - lse[:, None])
        ti = t[idx]
        valid = (ti >= 0) & (ti < V)
        p[valid, ti[valid]] -= 1.0
        return p * (gw[idx] * valid)[:, None], lse

    rr = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    dz, lse = dlogits(rr)
    dn = dz @ wor
    hr, rv = hbv[rr], r_all[rr]
    c = (g_[None, :] * dn * hr).sum(axis=1)
    dh = rv[:, None] * g_[None, :] * dn - (rv ** 3 / d)[:, None] * hr * c[:, None]
    out = dict(dh=dh, r=rv, dz=dz, lse=lse)
    if js is not None:
        full = isinstance(js, str)
        j = np.arange(V) if full else np.asarray(js, dtype=np.int64)
        k = np.arange(d) if ks is None else np.asarray(ks, dtype=np.int64)
        dz_all, _ = dlogits(np.arange(M))
        tj = dz_all[:, j]
        hk = hbv[:, k] * r_all[:, None]
        out["dW"] = (tj.T @ hk) * g_[k][None, :]
        out["dgamma"] = ((dz_all @ wraw[:, k]) * hk).sum(axis=0) if full else None
        if rss:
            out["rss"] = np.sqrt((tj * tj).T @ (hk * hk))
            out["rss_gamma"] = (np.sqrt((((dz_all * dz_all) @ (wraw[:, k] * wraw[:, k])) * hk * hk).sum(axis=0))
                                if full else None)
    return out


def cross_entropy(z: np.ndarray, targets):
    """(lse, loss) per row of the logits ``z`` (fp64 [R, V]): lse = log sum exp z,
    loss = lse - z[target] (0 for a target outside [0, V), an ignored row)."""
    zz = np.ascontiguousarray(z, dtype=np.float64)
    t = np.ascontiguousarray(targets, dtype=np.int32)
    if zz.ndim != 2 or t.shape != (zz.shape[0],):
        raise ValueError("z must be [R, V] and targets [R]")
    lse = np.empty(zz.shape[0], np.float64)
    loss = np.empty(zz.shape[0], np.float64)
    if lib().orc_cross_entropy(zz.shape[0], zz.shape[1], _p(zz), _p(t), _p(lse), _p(loss)) != 0:
        raise ValueError("empty vocabulary")
    return lse, loss


def mlpin_bwd(hb, gamma, Wp, wp_dt: int, wp_scale: float, dy, eps: float, rows=None):
    """Input gradient of y = SwiGLU(RMSNorm(hb) . W_or^T) for the listed rows (default
    all): hb uint16 [M, d] bf16 codes, gamma fp32 [d], Wp [2F, d] prepared second weight
    codes (bf16 or e4m3, with wp_scale), dy uint16 [M, F] bf16 codes of the upstream
    gradient.  Returns dict(dh [R, d], r [R], dz [R, 2F]) in fp64."""
    hb = np.ascontiguousarray(hb, dtype=np.uint16)
    dy = np.ascontiguousarray(dy, dtype=np.uint16)
    g = np.ascontiguousarray(gamma, dtype=np.float32)
    Wp = np.ascontiguousarray(Wp)
    M, d = hb.shape
    F2 = Wp.shape[0]
    F = F2 // 2
    if F2 % 2 or Wp.shape[1] != d or dy.shape != (M, F) or g.shape != (d,):
        raise ValueError("shape mismatch")
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    R = M if rows is None else rows_a.size
    dh = np.empty((R, d), np.float64)
    r = np.empty(R, np.float64)
    dz = np.empty((R, F2), np.float64)
    rc = lib().orc_mlpin_bwd(R, _p(rows_a), d, F, _p(hb), _p(g), _p(Wp), wp_dt, float(wp_scale), _p(dy),
                             float(eps), _p(dh), _p(r), _p(dz))
    if rc != 0:
        raise RuntimeError(f"oracle backward failed ({rc})")
    return dict(dh=dh, r=r, dz=dz)


def mlpin_wgrad(hb, gamma, Wp, wp_dt: int, wp_scale: float, W_raw, dy, eps: float, js=None, ks=None,
                rss=False):
    """Weight gradients of y = SwiGLU(RMSNorm(hb) . W^T) summed over all tokens: dW [nj, nk]
    at the listed rows js of W (default all 2F) and columns ks (default all d); dgamma
    [nk] only when js covers every row (else None).  Inputs as :func:`mlpin_bwd` plus
    the raw weight W_raw [2F, d] (bf16 codes).

    rss=True also returns the root-sum-square over the tokens of the summed terms,
    (dW, dgamma, rss [nj, nk] (gamma left out), rss_gamma [nk] or None): the scale of a
    sum's error when each of its terms carries an independent relative rounding."""
    hb = np.ascontiguousarray(hb, dtype=np.uint16)
    dy = np.ascontiguousarray(dy, dtype=np.uint16)
    g = np.ascontiguousarray(gamma, dtype=np.float32)
    Wp = np.ascontiguousarray(Wp)
    Wr = np.ascontiguousarray(W_raw, dtype=np.uint16)
    M, d = hb.shape
    F2 = Wp.shape[0]
    F = F2 // 2
    if F2 % 2 or Wp.shape[1] != d or Wr.shape != Wp.shape or dy.shape != (M, F):
        raise ValueError("shape mismatch")
    j = np.arange(F2, dtype=np.int64) if js is None else np.ascontiguousarray(js, dtype=np.int64)
    k = np.arange(d, dtype=np.int64) if ks is None else np.ascontiguousarray(ks, dtype=np.int64)
    full = js is None
    dW = np.empty((j.size, k.size), np.float64)
    dgam = np.empty(k.size, np.float64) if full else None
    sq = np.empty((j.size, k.size), np.float64) if rss else None
    sqg = np.empty(k.size, np.float64) if rss and full else None
    rc = lib().orc_mlpin_wgrad(M, d, F, _p(hb), _p(g), _p(Wp), wp_dt, float(wp_scale), _p(Wr), _p(dy), float(eps),
                               j.size, _p(j), k.size, _p(k), _p(dW), _p(dgam), _p(sq), _p(sqg))
    if rc != 0:
        raise RuntimeError(f"oracle weight gradient failed ({rc})")
    return (dW, dgam, sq, sqg) if rss else (dW, dgam)


def chain_bwd(prep: dict, x_res, gamma, W_raw, dy, eps: float, dres=None, rows=None, rss=False):
    """Backward of the whole chain  h = x_res + A . Wo^T,  y = SwiGLU(RMSNorm(h) . W^T)
    (kucoin page, section "CODA: El epilogo esconde un tesoro": the backward keeps the
    forward's structure; section "Resultados del experimento": the backward of
    GEMM-Residual-PartialRMS-GEMM).  bf16 operands (``prep`` from :func:`prepare`).

    The chain rule in reverse order, fp64:
      dh     = d/dh of the MLP-input block (:func:`mlpin_bwd`, at the rounded hb the
               forward stores) + dres (the gradient reaching h through the residual
               stream; None = 0).  The bf16 rounding of h passes the gradient unchanged.
      dx_res = dh;   dA = dh . Wo;   dWo[n, k] = sum_m dh[m, n] A[m, k]
      dW, dgamma of the second weight and of gamma (:func:`mlpin_wgrad`).
    Returns dict(dh [R, d], dA [R, K1], and with rows=None also dWo [d, K1], dW [2F, d],
    dgamma [d]).  rss=True adds the root-sum-square of the summed terms of each entry of
    dA (over n), dWo (over m), dW (gamma left out, as :func:`mlpin_wgrad`) and dgamma
    (``rss_*``) for rounding-error bounds."""
    if prep["a_dt"] != BF16 or prep["wo_dt"] != BF16 or prep["wp_dt"] != BF16:
        raise ValueError("the backward is defined for bf16 operands")
    M = prep["A"].shape[0]
    sel = np.arange(M) if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    fwd = chain(prep, x_res, gamma, ACT_SWIGLU, eps, rows=None if rows is None else sel)
    hb = fwd["hb"]
    dyr = np.ascontiguousarray(np.asarray(dy)[sel])
    b = mlpin_bwd(hb, gamma, prep["Wp"], BF16, 1.0, dyr, eps)
    dh = b["dh"] + (0.0 if dres is None else bf16_decode(np.asarray(dres)[sel]))
    A = bf16_decode(prep["A"])
    Wo = bf16_decode(prep["Wo"])
    out = dict(dh=dh, dA=dh @ Wo)
    if rss:
        out["rss_dA"] = np.sqrt((dh * dh) @ (Wo * Wo))
    if rows is None:
        out["dWo"] = dh.T @ A
        wg = mlpin_wgrad(hb, gamma, prep["Wp"], BF16, 1.0, W_raw, dyr, eps, rss=rss)
        out["dW"], out["dgamma"] = wg[0], wg[1]
        if rss:
            out["rss_dWo"] = np.sqrt((dh * dh).T @ (A * A))
            out["rss_dW"], out["rss_dgamma"] = wg[2], wg[3]
    return out

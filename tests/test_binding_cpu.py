"""The Python binding checks every caller-provided tensor -- shape, dtype, contiguity,
device -- against the sizes the call derives, and raises ValueError before anything
reaches the library.  The library only sees pointers, so an unchecked buffer of the
wrong size would be read or written out of bounds on the GPU.

Runs on the CPU: the library handle is replaced by a stand-in that answers the sizing
queries (partials per row and the like) from the real library and fails the test on
any other call.  Tensors are CPU tensors, so a case whose shapes are all right still
stops at the device check -- which shows the shape checks let the right shapes pass.
"""

import pytest
import torch

import gemm_epilogue_transformer_amd as coda
from gemm_epilogue_transformer_amd import _lib

SIZING = {"coda_partials_per_row", "coda_ce_partials_per_row", "coda_swiglu_bwd_partials_per_row",
          "coda_wgrad_partials_rows", "coda_wgrad_workspace_bytes", "coda_wgrad_tok_workspace_bytes",
          "coda_status_string", "coda_last_hip_error", "coda_version"}


class _NoLaunch:
    def __init__(self, real):
        self._real = real

    def __getattr__(self, name):
        if name in SIZING:
            return getattr(self._real, name)

        def launched(*a):
            raise AssertionError(f"{name} was called: the binding let a bad argument through")
        return launched


@pytest.fixture(autouse=True)
def no_launch(monkeypatch):
    real = _lib.load()
    monkeypatch.setattr(_lib, "load", lambda: _NoLaunch(real))


bf = lambda *s: torch.zeros(s, dtype=torch.bfloat16)  # noqa: E731
f32 = lambda *s: torch.zeros(s, dtype=torch.float32)  # noqa: E731
i32 = lambda *s: torch.zeros(s, dtype=torch.int32)  # noqa: E731
u8 = lambda *s: torch.zeros(s, dtype=torch.uint8)  # noqa: E731

M, K, N, F, V = 40, 64, 48, 28, 72      # all sizes distinct (2F = 56)


def _tb(n):
    return int(_lib.load().coda_swiglu_bwd_partials_per_row(n))


# (call, good keyword arguments, {argument: bad value})
def cases():
    T = coda.partials_per_row(N)
    Tce = coda.ce_partials_per_row(V)
    TW = coda.wgrad_partials_rows(2 * F)
    return [
        ("prepare_weight_bf16", coda.prepare_weight_bf16, dict(W_t=bf(N, K), gamma=f32(K), out=bf(N, K)),
         {"gamma": f32(K + 1), "out": bf(N, K + 8)}),
        ("quantize_e4m3", coda.quantize_e4m3, dict(X=bf(N, K), gamma=f32(K), out=u8(N, K), amax_scale=f32(2)),
         {"out": bf(N, K), "amax_scale": f32(1), "gamma": torch.zeros(K, dtype=torch.float64)}),
        ("gemm_resid_partialrms", coda.gemm_resid_partialrms,
         dict(A=bf(M, K), W=bf(N, K), x_res=bf(M, N), h=bf(M, N), partials=f32(M, T)),
         {"x_res": bf(M, N + 8), "h": bf(M - 1, N), "partials": f32(M, T + 1), "W": bf(N, K + 8),
          "A": bf(M, K, 1)}),
        ("rowscale_reduce", coda.rowscale_reduce, dict(partials=f32(M, T), N=N, eps=1e-5, r=f32(M)),
         {"partials": f32(M, T + 2), "r": f32(M + 1)}),
        ("gemm_rowscale_swiglu", coda.gemm_rowscale_swiglu,
         dict(h=bf(M, K), W=bf(2 * F, K), r=f32(M), act=coda.SWIGLU, y=bf(M, F)),
         {"r": f32(M - 1), "y": bf(M, 2 * F), "W": bf(2 * F + 1, K), "h": f32(M, K)}),
        ("gemm_rowscale_swiglu e4m3", coda.gemm_rowscale_swiglu,
         dict(h=bf(M, K), W=u8(2 * F, K), r=f32(M), act=coda.SWIGLU, w_scale=f32(1), y=bf(M, F)),
         {"w_scale": torch.zeros(1, dtype=torch.float64)}),
        ("gemm_rowscale_rope", coda.gemm_rowscale_rope,
         dict(h=bf(M, K), W=bf(N, K), r=f32(M), pos=i32(M), cos=f32(16, 32), sin=f32(16, 32), rot_cols=0,
              y=bf(M, N)),
         {"pos": torch.zeros(M, dtype=torch.int64), "sin": f32(15, 32), "cos": f32(16, 33), "y": bf(M, N - 8)}),
        ("gemm_rowscale_ce", coda.gemm_rowscale_ce,
         dict(h=bf(M, K), W=bf(V, K), r=f32(M), targets=i32(M), partials=f32(M, Tce, 2), tgt_logit=f32(M)),
         {"targets": i32(M + 1), "partials": f32(M, Tce + 1, 2), "tgt_logit": f32(M, 1)}),
        ("ce_reduce", coda.ce_reduce,
         dict(partials=f32(M, Tce, 2), targets=i32(M), tgt_logit=f32(M), V=V, lse=f32(M), loss=f32(M)),
         {"partials": f32(M, Tce, 3), "lse": f32(M - 1), "loss": bf(M), "targets": f32(M)}),
        ("rowscale_from_h", coda.rowscale_from_h, dict(h=bf(M, N), eps=1e-5, r=f32(M)), {"r": f32(M + 1)}),
        ("transpose_bf16", coda.transpose_bf16, dict(src=bf(M, N), out=bf(N, M)), {"out": bf(M, N)}),
        ("gemm_swiglu_bwd", coda.gemm_swiglu_bwd,
         dict(h=bf(M, K), W=bf(2 * F, K), r=f32(M), dy=bf(M, F), dz=bf(M, 2 * F), partials=f32(M, _tb(F))),
         {"dy": bf(M, 2 * F), "dz": bf(M, F), "partials": f32(M, _tb(F) + 1), "W": u8(2 * F, K)}),
        ("rmsnorm_bwd_reduce", coda.rmsnorm_bwd_reduce, dict(partials=f32(M, _tb(F)), r=f32(M), N=N, F=F, q=f32(M)),
         {"partials": f32(M, _tb(F) + 1), "q": f32(M + 1), "r": f32(M - 1)}),
        ("gemm_rmsnorm_bwd", coda.gemm_rmsnorm_bwd,
         dict(dz=bf(M, K), Wt=bf(N, K), h=bf(M, N), q=f32(M), dh_res=bf(M, N), dh=bf(M, N)),
         {"h": bf(M, K), "q": f32(M + 1), "dh_res": bf(M + 1, N), "dh": f32(M, N)}),
        ("gemm_rowscale_gfold", coda.gemm_rowscale_gfold,
         dict(h=bf(M, K), W=bf(2 * F, K), gamma=f32(K), r=f32(M), act=coda.SWIGLU, y=bf(M, F)),
         {"gamma": f32(2 * F), "y": bf(M, 2 * F)}),
        ("gemm_rowscale_swiglu_save", coda.gemm_rowscale_swiglu_save,
         dict(h=bf(M, K), W=bf(2 * F, K), r=f32(M), y=bf(M, F), z=bf(M, 2 * F)),
         {"y": bf(M, 2 * F), "z": bf(M, F)}),
        ("swiglu_bwd_saved", coda.swiglu_bwd_saved,
         dict(z=bf(M, 2 * F), dy=bf(M, F), r=f32(M), dz=bf(M, 2 * F), dzt=bf(2 * F, M), partials=f32(M, _tb(F))),
         {"dzt": bf(M, 2 * F), "dy": bf(M, 2 * F), "partials": f32(M + 1, _tb(F))}),
        ("rope_bwd", coda.rope_bwd,
         dict(dy=bf(M, N), y=bf(M, N), r=f32(M), pos=i32(M), cos=f32(16, 32), sin=f32(16, 32), rot_cols=0,
              dz=bf(M, N), partials=f32(M, _tb(N))),
         {"y": bf(M, N + 8), "partials": f32(M, _tb(N) + 1), "pos": i32(M - 1)}),
        ("gemm_ce_bwd", coda.gemm_ce_bwd,
         dict(h=bf(M, K), W=bf(V, K), r=f32(M), targets=i32(M), lse=f32(M), g=f32(M), dz=bf(M, V),
              partials=f32(M, _tb(V))),
         {"lse": f32(M + 1), "g": bf(M), "dz": bf(M, V + 8), "partials": f32(M, 1 + _tb(V))}),
        ("gemm_bf16", coda.gemm_bf16, dict(A=bf(M, K), Bt=bf(N, K), c_res=bf(M, N), C=bf(M, N)),
         {"c_res": bf(N, M), "C": f32(M, N), "Bt": bf(N, K + 8)}),
        ("gemm_wgrad", coda.gemm_wgrad,
         dict(At=bf(2 * F, M), Bt=bf(N, M), gamma=f32(N), W=bf(2 * F, N), dW=f32(2 * F, N),
              partials=f32(TW, N), workspace=u8(64)),
         {"gamma": f32(2 * F), "W": bf(N, 2 * F), "dW": f32(2 * F, N + 1), "partials": f32(TW + 1, N),
          "workspace": f32(16)}),
        ("gemm_wgrad_tok", coda.gemm_wgrad_tok,
         dict(X=bf(M, 2 * F), Y=bf(M, N), gamma=f32(N), W=bf(2 * F, N), dW=f32(2 * F, N), partials=f32(TW, N)),
         {"Y": bf(M + 1, N), "dW": f32(N, 2 * F), "NR": 2 * F + 8, "gamma": f32(N + 8)}),
        ("colsum_reduce", coda.colsum_reduce, dict(partials=f32(3, N), out=f32(N)), {"out": f32(N + 1)}),
    ]


CASES = cases()


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_right_shapes_stop_only_at_the_device_check(case):
    _, fn, good, _ = case
    with pytest.raises(ValueError, match="device"):
        fn(**good)


@pytest.mark.parametrize("case,arg", [(c, a) for c in CASES for a in c[3]],
                         ids=[f"{c[0]}:{a}" for c in CASES for a in c[3]])
def test_bad_argument_is_rejected_before_any_call(case, arg):
    _, fn, good, bad = case
    kw = dict(good, **{arg: bad[arg]})
    with pytest.raises(ValueError) as e:
        fn(**kw)
    msg = str(e.value)
    assert "device" not in msg or arg in msg, msg
    # the message names the offending operand, or (for the sizes that define the
    # problem) the disagreement it caused
    assert arg in msg or "disagree" in msg or "dimensions" in msg or "must lie" in msg, msg


def test_non_contiguous_output_is_rejected():
    y = torch.empty_strided((M, 2 * F), (1, M), dtype=torch.bfloat16)     # right shape, column-major
    with pytest.raises(ValueError, match="y: expected a contiguous"):
        coda.gemm_rowscale_swiglu(bf(M, K), bf(2 * F, K), f32(M), coda.NONE, y=y)


def test_mixed_devices_are_rejected():
    meta = torch.empty((M, N), dtype=torch.bfloat16, device="meta")
    with pytest.raises(ValueError, match="x_res: on meta"):
        coda.gemm_resid_partialrms(bf(M, K), bf(N, K), meta)

"""The C ABI library loads, exports every symbol include/coda.h declares, and rejects
invalid arguments with the documented status codes before enqueuing anything.

No compute call is made here.  The validation cases pass fake (but aligned) addresses;
they only run on hosts WITHOUT a GPU so that a validation mistake could never turn into
a launch on fake pointers.
"""

import ctypes as C
import os
import re

import pytest
import torch

from gemm_epilogue_transformer_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "coda.h")

OK, NULL, SHAPE, DTYPE, VALUE, ALIAS, HIP, ALIGN = range(8)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(coda_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_chain_calls():
    names = declared_functions()
    for n in ("coda_gemm_resid_partialrms", "coda_rowscale_reduce", "coda_gemm_rowscale_swiglu"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = C.CDLL(_lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(_lib.SIGNATURES)


def test_utilities():
    L = _lib.load()
    assert b"gfx950" in L.coda_version()
    for s in range(8):
        assert L.coda_status_string(s)
    assert L.coda_partials_per_row(0) == -1
    assert L.coda_partials_per_row(1) == 1
    T = L.coda_partials_per_row(2048)
    assert T >= 1 and 2048 % T == 0


no_gpu = pytest.mark.skipif(torch.cuda.is_available(),
                            reason="fake-pointer validation cases run on GPU-less hosts only")

# fake, 16-byte aligned, far apart device addresses
P1, P2, P3, P4, P5, P6 = (0x10000000 * (i + 1) for i in range(6))


@no_gpu
def test_gemm1_validation():
    f = _lib.load().coda_gemm_resid_partialrms
    # M, N, K, A, dt, sa, W, sw, x, h, P, stream
    assert f(16, 64, 64, None, 0, None, P2, None, P3, P4, P5, None) == NULL
    assert f(16, 64, 64, P1, 0, None, P2, None, P3, None, P5, None) == NULL
    assert f(16, 64, 64, P1, 1, None, P2, P6, P3, P4, P5, None) == NULL     # e4m3 needs scales
    assert f(16, 64, 64, P1, 7, None, P2, None, P3, P4, P5, None) == DTYPE
    assert f(-1, 64, 64, P1, 0, None, P2, None, P3, P4, P5, None) == SHAPE
    assert f(16, 0, 64, P1, 0, None, P2, None, P3, P4, P5, None) == SHAPE
    assert f(16, 64, 0, P1, 0, None, P2, None, P3, P4, P5, None) == SHAPE
    assert f(16, 60, 64, P1, 0, None, P2, None, P3, P4, P5, None) == SHAPE  # N % 8
    assert f(16, 64, 60, P1, 0, None, P2, None, P3, P4, P5, None) == SHAPE  # K % 8
    assert f(16, 64, 24, P1, 1, P6, P2, P6, P3, P4, P5, None) == SHAPE      # e4m3 K % 16
    assert f(1 << 31, 64, 64, P1, 0, None, P2, None, P3, P4, P5, None) == SHAPE
    assert f(16, 64, (1 << 22) + 8, P1, 0, None, P2, None, P3, P4, P5, None) == SHAPE  # row cap
    assert f(16, (1 << 22) + 8, 64, P1, 0, None, P2, None, P3, P4, P5, None) == SHAPE
    assert f(16, 64, 64, P1 + 8, 0, None, P2, None, P3, P4, P5, None) == ALIGN
    assert f(16, 64, 64, P1, 0, None, P2, None, P3, P4, P5 + 4, None) == ALIGN
    assert f(16, 64, 64, P1, 0, None, P2, None, P3, P1, P5, None) == ALIAS   # h over A
    assert f(16, 64, 64, P1, 0, None, P2, None, P3, P4, P4 + 16, None) == ALIAS  # P over h
    assert f(16, 64, 64, P1, 0, None, P2, None, P4 + 16, P4, P5, None) == ALIAS  # partial alias
    # the exact alias h == x_res is allowed; M == 0 enqueues nothing and succeeds
    assert f(0, 64, 64, P1, 0, None, P2, None, P4, P4, P5, None) == OK


@no_gpu
def test_rowscale_validation():
    f = _lib.load().coda_rowscale_reduce
    assert f(16, 64, None, 1e-5, P2, None) == NULL
    assert f(16, 0, P1, 1e-5, P2, None) == SHAPE
    assert f(16, 64, P1, -1.0, P2, None) == VALUE
    assert f(16, 64, P1, float("nan"), P2, None) == VALUE
    assert f(16, 64, P1, float("inf"), P2, None) == VALUE
    assert f(16, 64, P1, 1e-5, P1, None) == ALIAS
    assert f(16, 64, P1 + 4, 1e-5, P2, None) == ALIGN
    assert f(0, 64, P1, 1e-5, P2, None) == OK


@no_gpu
def test_gemm2_validation():
    f = _lib.load().coda_gemm_rowscale_swiglu
    # M, N_out, K, act, h, W, wdt, sw, r, y, stream
    assert f(16, 64, 64, 1, None, P2, 0, None, P3, P4, None) == NULL
    assert f(16, 64, 64, 1, P1, P2, 1, None, P3, P4, None) == NULL           # e4m3 needs scale
    assert f(16, 64, 64, 2, P1, P2, 0, None, P3, P4, None) == DTYPE
    assert f(16, 64, 64, 1, P1, P2, 3, None, P3, P4, None) == DTYPE
    assert f(16, 60, 64, 1, P1, P2, 0, None, P3, P4, None) == SHAPE
    assert f(16, 64, 8, 1, P1, P2, 1, P5, P3, P4, None) == SHAPE             # e4m3 K % 16
    assert f(16, 1 << 30, 64, 1, P1, P2, 0, None, P3, P4, None) == SHAPE     # 2F too large
    assert f(16, 64, (1 << 22) + 8, 1, P1, P2, 0, None, P3, P4, None) == SHAPE  # row cap
    assert f(16, 64, 64, 1, P1, P2, 0, None, P3, P1, None) == ALIAS          # y over h
    assert f(16, 64, 64, 1, P1, P2, 0, None, P3, P3, None) == ALIAS          # y over r
    assert f(16, 64, 64, 1, P1, P2, 0, None, P3 + 8, P4, None) == ALIGN
    assert f(0, 64, 64, 1, P1, P2, 0, None, P3, P4, None) == OK


@no_gpu
def test_prepare_validation():
    L = _lib.load()
    assert L.coda_prepare_weight_bf16(8, 64, None, None, P2, None) == NULL
    assert L.coda_prepare_weight_bf16(8, 60, P1, None, P2, None) == SHAPE
    assert L.coda_prepare_weight_bf16(8, 64, P1, None, P1, None) == ALIAS
    assert L.coda_prepare_weight_bf16(8, 64, P1, P3 + 4, P2, None) == ALIGN
    assert L.coda_quantize_e4m3(8, 64, P1, None, P2, None, None) == NULL
    assert L.coda_quantize_e4m3(8, 40, P1, None, P2, P3, None) == SHAPE
    assert L.coda_quantize_e4m3(8, 64, P1, None, P2, P2, None) == ALIAS
    assert L.coda_quantize_e4m3(8, 64, P1, None, P2, P1 + 16, None) == ALIAS


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        _lib.load()


@no_gpu
def test_rope_validation():
    L = _lib.load()
    t = L.coda_rope_table
    assert t(0, 500000.0, P1, P2, None) == SHAPE
    assert t(1 << 24, 500000.0, P1, P2, None) == SHAPE
    assert t(16, 1.0, P1, P2, None) == VALUE
    assert t(16, float("inf"), P1, P2, None) == VALUE
    assert t(16, 500000.0, None, P2, None) == NULL
    assert t(16, 500000.0, P1 + 4, P2, None) == ALIGN
    assert t(16, 500000.0, P1, P1 + 16, None) == ALIAS
    f = L.coda_gemm_rowscale_rope
    # M, N_out, K, h, W, wdt, sw, r, pos, cos, sin, rows, rot_cols, y, stream
    assert f(16, 128, 64, P1, P2, 2, None, P3, P4, P5, P6, 8, 64, P6 + 4096, None) == DTYPE
    assert f(16, 128, 64, P1, P2, 0, None, P3, P4, P5, P6, 8, 32, P6 + 4096, None) == SHAPE   # not whole heads
    assert f(16, 128, 64, P1, P2, 0, None, P3, P4, P5, P6, 8, 192, P6 + 4096, None) == SHAPE  # > N_out
    assert f(16, 128, 64, P1, P2, 0, None, P3, P4, P5, P6, 0, 64, P6 + 4096, None) == SHAPE   # no table
    assert f(16, 124, 64, P1, P2, 0, None, P3, P4, P5, P6, 8, 64, P6 + 4096, None) == SHAPE   # N_out % 8
    assert f(16, 128, 64, P1, P2, 0, None, P3, None, P5, P6, 8, 64, P6 + 4096, None) == NULL
    assert f(16, 128, 64, P1, P2, 1, None, P3, P4, P5, P6, 8, 64, P6 + 4096, None) == NULL    # e4m3 scale
    assert f(16, 128, 64, P1, P2, 0, None, P3, P4 + 4, P5, P6, 8, 64, P6 + 4096, None) == ALIGN
    assert f(16, 128, 64, P1, P2, 0, None, P3, P4, P5, P6, 8, 64, P4, None) == ALIAS          # y over pos
    assert f(16, 128, 64, P1, P2, 0, None, P3, P4, P5, P6, 8, 64, P5, None) == ALIAS          # y over cos
    # rot_cols == 0: no table, positions or angles needed; M == 0 enqueues nothing
    assert f(0, 128, 64, P1, P2, 0, None, P3, None, None, None, 0, 0, P6 + 4096, None) == OK
    assert f(0, 128, 64, P1, P2, 0, None, P3, P4, P5, P6, 8, 64, P6 + 4096, None) == OK


@no_gpu
def test_cross_entropy_validation():
    L = _lib.load()
    assert L.coda_ce_partials_per_row(0) == -1
    assert L.coda_ce_partials_per_row(256) == 1 and L.coda_ce_partials_per_row(257) == 2
    assert L.coda_ce_partials_per_row(128256) == 501
    f = L.coda_gemm_rowscale_ce
    # M, V, K, h, W, wdt, sw, r, targets, partials, tgt_logit, stream
    Q = P6 + 0x1000000
    assert f(16, 100, 64, P1, P2, 2, None, P3, P4, P5, Q, None) == DTYPE
    assert f(16, 0, 64, P1, P2, 0, None, P3, P4, P5, Q, None) == SHAPE
    assert f(16, 100, 60, P1, P2, 0, None, P3, P4, P5, Q, None) == SHAPE          # K % 8
    assert f(16, (1 << 22) + 1, 64, P1, P2, 0, None, P3, P4, P5, Q, None) == SHAPE
    assert f(16, 100, 64, P1, P2, 0, None, P3, None, P5, Q, None) == NULL
    assert f(16, 100, 64, P1, P2, 1, None, P3, P4, P5, Q, None) == NULL          # e4m3 scale
    assert f(16, 100, 64, P1, P2, 0, None, P3, P4, P5 + 4, Q, None) == ALIGN
    assert f(16, 100, 64, P1, P2, 0, None, P3, P4, P5, P5 + 16, None) == ALIAS   # outputs overlap
    assert f(16, 100, 64, P1, P2, 0, None, P3, P4, P4, Q, None) == ALIAS         # partials over targets
    assert f(0, 100, 64, None, None, 0, None, None, None, None, None, None) == OK
    g = L.coda_ce_reduce
    # M, V, partials, targets, tgt_logit, lse, loss, stream
    assert g(16, 0, P1, P2, P3, P4, P5, None) == SHAPE
    assert g(16, 100, P1, P2, P3, None, P5, None) == NULL
    assert g(16, 100, P1, P2, P3, P4 + 8, P5, None) == ALIGN
    assert g(16, 100, P1, P2, P3, P4, P4, None) == ALIAS
    assert g(16, 100, P1, P2, P3, P1, P5, None) == ALIAS                          # lse over partials
    assert g(0, 100, None, None, None, None, None, None) == OK


@no_gpu
def test_backward_validation():
    L = _lib.load()
    assert L.coda_swiglu_bwd_partials_per_row(0) == -1
    assert L.coda_swiglu_bwd_partials_per_row(8192) == 64 and L.coda_swiglu_bwd_partials_per_row(129) == 2
    rs = L.coda_rowscale_from_h
    assert rs(16, 60, P1, 1e-5, P2, None) == SHAPE
    assert rs(16, 64, P1, -1.0, P2, None) == VALUE
    assert rs(16, 64, None, 1e-5, P2, None) == NULL
    assert rs(16, 64, P1, 1e-5, P1 + 64, None) == ALIAS
    t = L.coda_transpose_bf16
    assert t(0, 8, P1, P2, None) == SHAPE
    assert t(8, 8, P1, P1 + 64, None) == ALIAS
    assert t(8, 8, P1 + 2, P2, None) == ALIGN
    f = L.coda_gemm_swiglu_bwd
    # M, F, K, h, W, r, dy, dz, partials, stream
    assert f(16, 60, 64, P1, P2, P3, P4, P5, P6, None) == SHAPE          # F % 8
    assert f(16, 64, 60, P1, P2, P3, P4, P5, P6, None) == SHAPE          # K % 8
    assert f(16, 64, 64, P1, P2, P3, None, P5, P6, None) == NULL
    assert f(16, 64, 64, P1, P2, P3, P4, P5, P5 + 16, None) == ALIAS     # partials over dz
    assert f(16, 64, 64, P1, P2, P3, P4, P4, P6, None) == ALIAS          # dz over dy
    assert f(0, 64, 64, None, None, None, None, None, None, None) == OK
    g = L.coda_rmsnorm_bwd_reduce
    assert g(16, 0, 64, P1, P2, P3, None) == SHAPE
    assert g(16, 64, 64, P1, P2, P2, None) == ALIAS
    b = L.coda_gemm_rmsnorm_bwd
    # M, N, K, dz, Wt, h, q, dh_res, dh, stream
    assert b(16, 60, 64, P1, P2, P3, P4, None, P5, None) == SHAPE
    assert b(16, 64, 64, P1, P2, P3, P4, None, P3, None) == ALIAS        # dh over h
    assert b(16, 64, 64, P1, P2, P3, P4, P5 + 16, P5, None) == ALIAS     # partial overlap with dh_res
    assert b(16, 64, 64, P1, P2, P3, None, None, P5, None) == NULL
    assert b(0, 64, 64, None, None, None, None, None, None, None) == OK


@no_gpu
def test_weight_gradient_validation():
    L = _lib.load()
    assert L.coda_wgrad_partials_rows(0) == -1
    assert L.coda_wgrad_partials_rows(256) == 1 and L.coda_wgrad_partials_rows(257) == 2
    w = L.coda_gemm_wgrad
    # NR, NC, K, At, Bt, gamma, W, dW, partials, workspace, workspace_bytes, stream
    assert w(64, 60, 64, P1, P2, P3, P4, P5, P6, None, 0, None) == SHAPE          # NC % 8
    assert w(64, 64, 60, P1, P2, P3, P4, P5, P6, None, 0, None) == SHAPE          # K % 8 (the tokens)
    assert w(0, 64, 64, P1, P2, P3, P4, P5, P6, None, 0, None) == SHAPE
    assert w(64, 64, 64, P1, P2, P3, P4, P5, None, None, 0, None) == NULL         # W without partials
    assert w(64, 64, 64, None, P2, P3, P4, P5, P6, None, 0, None) == NULL
    assert w(64, 64, 0, None, None, None, None, None, None, None, 0, None) == NULL  # no tokens still writes dW
    assert w(64, 64, 64, P1, P2, P3 + 4, P4, P5, P6, None, 0, None) == ALIGN      # gamma read 16 bytes at a time
    assert w(64, 64, 64, P1, P2, P3, P4, P5, P5 + 64, None, 0, None) == ALIAS     # partials over dW
    assert w(64, 64, 64, P1, P2, P3, P4, P1 + 16, P6, None, 0, None) == ALIAS     # dW over At
    assert w(64, 64, 64, P1, P2, P3, P4, P5, P4, None, 0, None) == ALIAS          # partials over W
    # NR, NC, K, At, Bt, gamma, W, dW, partials, workspace, workspace_bytes, stream
    assert w(64, 64, 64, P1, P2, P3, None, P5, None, None, 64, None) == VALUE      # bytes without a workspace
    assert w(64, 64, 64, P1, P2, P3, None, P5, None, P6, -1, None) == VALUE
    assert w(64, 64, 64, P1, P2, P3, None, P5, None, P6 + 8, 64, None) == ALIGN
    assert w(64, 64, 64, P1, P2, P3, None, P5, None, P5 + 64, 64, None) == ALIAS    # workspace over dW
    assert w(64, 64, 64, P1, P2, P3, None, P5, None, P1 + 64, 64, None) == ALIAS    # workspace over At
    assert L.coda_wgrad_workspace_bytes(0, 64, 64) == -1
    assert L.coda_wgrad_workspace_bytes(16384, 2048, 16384) == 0                # 512 tiles: no split
    # 64 tiles: 4 splits, each a dW slice and the partial rows of its 8 row tiles
    assert L.coda_wgrad_workspace_bytes(2048, 2048, 16384) == 4 * (2048 + 8) * 2048 * 4
    assert L.coda_wgrad_workspace_bytes(2048, 2048, 2048) == 0                  # too few tokens to split
    c = L.coda_colsum_reduce
    assert c(0, 64, P1, P2, None) == SHAPE
    assert c(4, 64, None, P2, None) == NULL
    assert c(4, 64, P1, P1 + 128, None) == ALIAS


@no_gpu
def test_plain_gemm_validation():
    L = _lib.load()
    g = L.coda_gemm_bf16
    # M, N, K, A, Bt, c_res, C, stream
    assert g(16, 60, 64, P1, P2, None, P3, None) == SHAPE             # N % 8
    assert g(16, 64, 60, P1, P2, None, P3, None) == SHAPE             # K % 8
    assert g(16, 64, 64, None, P2, None, P3, None) == NULL
    assert g(16, 64, 64, P1 + 8, P2, None, P3, None) == ALIGN
    assert g(16, 64, 64, P1, P2, None, P1 + 16, None) == ALIAS        # C over A
    assert g(16, 64, 64, P1, P2, P3 + 16, P3, None) == ALIAS          # partial overlap with c_res
    assert g(0, 64, 64, None, None, None, None, None) == OK


@no_gpu
def test_saved_pre_activation_validation():
    L = _lib.load()
    f = L.coda_gemm_rowscale_swiglu_save
    # M, F, K, h, W, r, y, z, stream
    assert f(16, 60, 64, P1, P2, P3, P4, P5, None) == SHAPE             # F % 8
    assert f(16, 64, 64, P1, P2, P3, P4, None, None) == NULL
    assert f(16, 64, 64, P1, P2, P3, P4, P4 + 64, None) == ALIAS         # z over y
    assert f(16, 64, 64, P1, P2, P3, P4, P1, None) == ALIAS              # z over h
    assert f(0, 64, 64, None, None, None, None, None, None) == OK
    b = L.coda_swiglu_bwd_saved
    # M, F, z, dy, r, dz, dzt, partials, stream
    assert b(16, 60, P1, P2, P3, P4, P5, P6, None) == SHAPE              # F % 8
    assert b(12, 64, P1, P2, P3, P4, P5, P6, None) == SHAPE              # transposed rows need M % 8
    assert b(16, 64, P1, P2, P3, None, P5, P6, None) == NULL
    assert b(16, 64, P1, P2, P3, P4, P5 + 8, P6, None) == ALIGN
    assert b(16, 64, P1, P2, P3, P4, P4 + 64, P6, None) == ALIAS         # dzt over dz
    assert b(16, 64, P1, P2, P3, P4, P5, P1, None) == ALIAS              # partials over z
    assert b(0, 64, None, None, None, None, None, None, None) == OK


@no_gpu
def test_on_chip_fold_validation():
    L = _lib.load()
    f = L.coda_gemm_rowscale_gfold
    # M, N_out, K, act, h, W, gamma, r, y, stream
    assert f(16, 64, 64, 7, P1, P2, P3, P4, P5, None) == DTYPE
    assert f(16, 60, 64, 1, P1, P2, P3, P4, P5, None) == SHAPE
    assert f(16, 64, 64, 1, P1, P2, None, P4, P5, None) == NULL
    assert f(16, 64, 64, 1, P1, P2, P3 + 4, P4, P5, None) == ALIGN
    assert f(16, 64, 64, 1, P1, P2, P3, P4, P3, None) == ALIAS              # y over gamma
    assert f(0, 64, 64, 1, None, None, None, None, None, None) == OK


@no_gpu
def test_token_major_weight_gradient_validation():
    L = _lib.load()
    w = L.coda_gemm_wgrad_tok
    # NR, NC, K, X, lda, Y, ldb, gamma, W, dW, partials, workspace, workspace_bytes, stream
    assert w(64, 60, 64, P1, 64, P2, 64, None, None, P5, None, None, 0, None) == SHAPE     # NC % 8
    assert w(64, 64, 64, P1, 60, P2, 64, None, None, P5, None, None, 0, None) == SHAPE     # lda % 8
    assert w(72, 64, 64, P1, 64, P2, 64, None, None, P5, None, None, 0, None) == SHAPE     # lda < NR
    # rows are addressed per 64-token k-tile: the LM head's 4.2 GB dz [16384, 128256] needs
    # no split (4008 tiles), the split is the time model's alone, as on transposed operands
    assert L.coda_wgrad_tok_workspace_bytes(128256, 2048, 16384, 128256, 2048) == 0
    assert L.coda_wgrad_tok_workspace_bytes(16384, 2048, 16384, 16384, 2048) == 0     # 512 tiles
    ws = L.coda_wgrad_workspace_bytes(2048, 2048, 16384)                                # 64 tiles: split
    assert ws > 0 and L.coda_wgrad_tok_workspace_bytes(2048, 2048, 16384, 2048, 2048) == ws
    assert L.coda_wgrad_tok_workspace_bytes(64, 64, 64, 32, 64) == -1                   # lda < NR
    assert L.coda_wgrad_tok_workspace_bytes(64, 64, 64, (1 << 22) + 8, 64) == -1        # lda > 2^22
    assert w(64, 64, 13, None, 64, P2, 64, None, None, P5, None, None, 0, None) == NULL
    assert w(64, 64, 13, P1, 64, P2, 64, None, None, P1 + 64, None, None, 0, None) == ALIAS  # dW over X
    assert w(64, 64, 13, P1, 64, P2 + 8, 64, None, None, P5, None, None, 0, None) == ALIGN


@no_gpu
def test_rope_backward_validation():
    L = _lib.load()
    f = L.coda_rope_bwd
    DZ, PT = P6 + 0x1000000, P6 + 0x2000000
    # M, N, dy, y, r, pos, cos, sin, table_rows, rot_cols, dz, partials, stream
    assert f(16, 60, P1, P2, P3, P4, P5, P6, 8, 0, DZ, PT, None) == SHAPE       # N % 8
    assert f(16, 128, P1, P2, P3, P4, P5, P6, 8, 96, DZ, PT, None) == SHAPE     # whole heads
    assert f(16, 128, P1, P2, P3, P4, P5, P6, 8, 192, DZ, PT, None) == SHAPE    # rot_cols > N
    assert f(16, 128, P1, P2, P3, P4, P5, P6, 0, 64, DZ, PT, None) == SHAPE     # empty table
    assert f(16, 128, P1, P2, P3, None, P5, P6, 8, 64, DZ, PT, None) == NULL    # positions needed
    # without rotation no table is read: a later check (alignment) is the one that fails
    assert f(16, 128, P1 + 8, P2, P3, None, None, None, 0, 0, DZ, PT, None) == ALIGN
    assert f(16, 128, P1, P2, P3, P4, P5, P6, 8, 64, None, PT, None) == NULL
    assert f(16, 128, P1, P2, P3, P4, P5 + 4, P6, 8, 64, DZ, PT, None) == ALIGN  # cos 16-byte aligned
    assert f(16, 128, P1 + 8, P2, P3, P4, P5, P6, 8, 64, DZ, PT, None) == ALIGN
    assert f(16, 128, P1, P2, P3, P4, P5, P6, 8, 64, DZ, DZ + 64, None) == ALIAS  # partials over dz
    assert f(16, 128, P1, P2, P3, P4, P5, P6, 8, 64, P2, PT, None) == ALIAS      # dz over y
    assert f(16, 128, P1, P2, P3, P4, P5, P6, 8, 64, DZ, P6 + 64, None) == ALIAS  # partials over sin
    assert f(0, 128, None, None, None, None, None, None, 0, 0, None, None, None) == OK     # empty batch


@no_gpu
def test_cross_entropy_backward_validation():
    L = _lib.load()
    f = L.coda_gemm_ce_bwd
    DZ, PT = P6 + 0x1000000, P6 + 0x2000000
    # M, V, K, h, W, r, targets, lse, g, dz, partials, stream
    assert f(16, 100, 64, P1, P2, P3, P4, P5, P6, DZ, PT, None) == SHAPE        # V % 8
    assert f(16, 128, 60, P1, P2, P3, P4, P5, P6, DZ, PT, None) == SHAPE        # K % 8
    assert f(16, 1 << 22, 64, P1, P2, P3, P4, P5, P6, DZ, PT, None) == SHAPE    # V past 2^21
    assert f(16, 128, 64, P1, P2, P3, None, P5, P6, DZ, PT, None) == NULL       # targets
    assert f(16, 128, 64, P1, P2, P3, P4, None, P6, DZ, PT, None) == NULL       # lse
    assert f(16, 128, 64, P1, P2, P3, P4, P5, None, DZ, PT, None) == NULL       # g
    assert f(16, 128, 64, P1 + 8, P2, P3, P4, P5, P6, DZ, PT, None) == ALIGN
    assert f(16, 128, 64, P1, P2, P3, P4, P5, P6, DZ, DZ + 64, None) == ALIAS   # partials over dz
    assert f(16, 128, 64, P1, P2, P3, P4, P5, P6, P2, PT, None) == ALIAS        # dz over W
    assert f(16, 128, 64, P1, P2, P3, P4, P5, P6, DZ, P5, None) == ALIAS        # partials over lse
    assert f(0, 128, 64, None, None, None, None, None, None, None, None, None) == OK

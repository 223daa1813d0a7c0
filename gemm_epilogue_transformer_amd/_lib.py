"""ctypes declarations of the C ABI in ``include/coda.h`` (libcoda.so, built in-tree).

Loading fails loudly when the library has not been built: there is no fallback path.
"""

from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.environ.get("CODA_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcoda.so")

CODA_OK = 0
STATUS_NAMES = {0: "CODA_OK", 1: "CODA_ERR_NULL", 2: "CODA_ERR_SHAPE", 3: "CODA_ERR_DTYPE",
                4: "CODA_ERR_VALUE", 5: "CODA_ERR_ALIAS", 6: "CODA_ERR_HIP", 7: "CODA_ERR_ALIGN"}
CODA_BF16, CODA_E4M3 = 0, 1
CODA_ACT_NONE, CODA_ACT_SWIGLU = 0, 1

# (name, restype, argtypes) for every symbol the header declares
_P, _I64, _F, _I = C.c_void_p, C.c_int64, C.c_float, C.c_int
SIGNATURES = {
    "coda_prepare_weight_bf16": (_I, [_I64, _I64, _P, _P, _P, _P]),
    "coda_quantize_e4m3": (_I, [_I64, _I64, _P, _P, _P, _P, _P]),
    "coda_partials_per_row": (_I64, [_I64]),
    "coda_gemm_resid_partialrms": (_I, [_I64, _I64, _I64, _P, _I, _P, _P, _P, _P, _P, _P, _P]),
    "coda_rowscale_reduce": (_I, [_I64, _I64, _P, _F, _P, _P]),
    "coda_gemm_rowscale_swiglu": (_I, [_I64, _I64, _I64, _I, _P, _P, _I, _P, _P, _P, _P]),
    "coda_rope_table": (_I, [_I64, C.c_double, _P, _P, _P]),
    "coda_gemm_rowscale_rope": (_I, [_I64, _I64, _I64, _P, _P, _I, _P, _P, _P, _P, _P, _I64, _I64, _P, _P]),
    "coda_ce_partials_per_row": (_I64, [_I64]),
    "coda_gemm_rowscale_ce": (_I, [_I64, _I64, _I64, _P, _P, _I, _P, _P, _P, _P, _P, _P]),
    "coda_ce_reduce": (_I, [_I64, _I64, _P, _P, _P, _P, _P, _P]),
    "coda_rowscale_from_h": (_I, [_I64, _I64, _P, _F, _P, _P]),
    "coda_transpose_bf16": (_I, [_I64, _I64, _P, _P, _P]),
    "coda_swiglu_bwd_partials_per_row": (_I64, [_I64]),
    "coda_gemm_swiglu_bwd": (_I, [_I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P]),
    "coda_rmsnorm_bwd_reduce": (_I, [_I64, _I64, _I64, _P, _P, _P, _P]),
    "coda_gemm_rmsnorm_bwd": (_I, [_I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P]),
    "coda_gemm_rowscale_gfold": (_I, [_I64, _I64, _I64, _I, _P, _P, _P, _P, _P, _P]),
    "coda_gemm_rowscale_swiglu_save": (_I, [_I64, _I64, _I64, _P, _P, _P, _P, _P, _P]),
    "coda_swiglu_bwd_saved": (_I, [_I64, _I64, _P, _P, _P, _P, _P, _P, _P]),
    "coda_rope_bwd": (_I, [_I64, _I64, _P, _P, _P, _P, _P, _P, _I64, _I64, _P, _P, _P]),
    "coda_gemm_ce_bwd": (_I, [_I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "coda_wgrad_tok_workspace_bytes": (_I64, [_I64, _I64, _I64, _I64, _I64]),
    "coda_gemm_bf16": (_I, [_I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "coda_wgrad_partials_rows": (_I64, [_I64]),
    "coda_wgrad_workspace_bytes": (_I64, [_I64, _I64, _I64]),
    "coda_gemm_wgrad": (_I, [_I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P, _I64, _P]),
    "coda_gemm_wgrad_tok": (_I, [_I64, _I64, _I64, _P, _I64, _P, _I64, _P, _P, _P, _P, _P, _I64, _P]),
    "coda_gemm_wgrad_tok_noalloc": (_I, [_I64, _I64, _I64, _P, _I64, _P, _I64, _P, _P, _P, _P, _P]),
    "coda_colsum_reduce": (_I, [_I64, _I64, _P, _P, _P]),
    "coda_status_string": (C.c_char_p, [_I]),
    "coda_last_hip_error": (_I, []),
    "coda_version": (C.c_char_p, []),
}

_lib = None


class CodaError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str = ""):
        self.status = status
        super().__init__(f"{fn} -> {STATUS_NAMES.get(status, status)}: {detail}")


def load():
    """Load libcoda.so (raises if it is missing: build it with
    ``python -m gemm_epilogue_transformer_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"HIP library not built: {LIB_PATH} is missing "
                              "(run python -m gemm_epilogue_transformer_amd.build)")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def check(fn: str, status: int) -> None:
    if status != CODA_OK:
        L = load()
        detail = L.coda_status_string(status).decode()
        if status == 6:
            detail += f" (hipError {L.coda_last_hip_error()})"
        raise CodaError(fn, status, detail)

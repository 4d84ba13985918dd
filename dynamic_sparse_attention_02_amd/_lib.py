"""ctypes loader of libsa.so and the C struct/enum mirrors of include/sa.h.

No fallback: if the shared library is missing or fails to load, every entry
point raises.  Build it with ``python -m dynamic_sparse_attention_02_amd.build``.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("SA_LIBRARY", os.path.join(PKG, "libsa.so"))

# enums (sa.h)
SA_OK = 0
SA_ERR_INVALID_ARGUMENT = 1
SA_ERR_UNSUPPORTED = 2
SA_ERR_CAPACITY = 3
SA_ERR_WORKSPACE = 4
SA_ERR_HIP = 5

SA_F32 = 0
SA_BF16 = 1

SA_OP_INDEX_SCORES = 0
SA_OP_SELECT = 1
SA_OP_SPARSE_DECODE = 2
SA_OP_PREFILL_SELECT = 3
SA_OP_DECODE_STEP = 4
SA_OP_SPARSE_DECODE_RLA = 5
SA_OP_ATTENTION_MASS = 6
SA_OP_PREFILL_QUERY = 7
SA_OP_PBS_IMPORTANCE = 8
SA_OP_PBS_SELECT = 9
SA_OP_PREFILL_ORACLE = 10
SA_OP_DECODE_STEP_PAGES = 11
SA_OP_DECODE_STEP_RLA = 12


class SaShape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("idx_rank", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_pages", ctypes.c_int32),
        ("max_len", ctypes.c_int32),
        ("n_pool_pages", ctypes.c_int64),
    ]


class SaPages(ctypes.Structure):
    _fields_ = [("page_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t
_SH = ctypes.POINTER(SaShape)
_PG = ctypes.POINTER(SaPages)

# name -> (restype, argtypes); mirrors include/sa.h
SIGNATURES = {
    "sa_workspace_size": (_SZ, [ctypes.c_int, _SH, _I64]),
    "sa_index_append": (ctypes.c_int, [_SH, _P, _P, ctypes.c_int, _P, _I32, _P, _P]),
    "sa_page_stats": (ctypes.c_int, [_SH, _P, ctypes.c_int, _P, _P, _I32, _P, _P]),
    "sa_index_scores": (ctypes.c_int, [_SH, _PG, _P, _P, _P, ctypes.c_int, _F, _P, _I64, _P, _SZ, _P]),
    "sa_page_scores": (ctypes.c_int, [_SH, _PG, _P, _P, ctypes.c_int, _F, _P, _I64, _P]),
    "sa_select_topp": (ctypes.c_int, [_SH, _PG, _P, _I64, _F, _I32, _I32, _P, _P, _I32, _P, _SZ, _P]),
    "sa_select_topk": (ctypes.c_int, [_SH, _PG, _P, _I64, _I32, _I32, _I32, _I32, _P, _P, _I32, _P, _SZ, _P]),
    "sa_sparse_decode": (ctypes.c_int, [_SH, _PG, _P, _P, _P, ctypes.c_int, _P, _P, _I32, _F, _P,
                                        ctypes.c_int, _P, _P, _SZ, _P]),
    "sa_sparse_decode_rla": (ctypes.c_int, [_SH, _PG, _P, _P, _P, ctypes.c_int, _P, _P, _I32, _F,
                                            _P, ctypes.c_int, _P, _P, _P, _P, _P, _SZ, _P]),
    "sa_rla_state": (ctypes.c_int, [_SH, _PG, _P, _P, ctypes.c_int, _I32, _P, _P]),
    "sa_attention_mass": (ctypes.c_int, [_SH, _PG, _P, _P, ctypes.c_int, _F, _P, _I64, _P, _SZ, _P]),
    "sa_support_coverage": (ctypes.c_int, [_SH, _PG, _P, _I64, _P, _P, _I32, _P, _P, _I32, _P, _P,
                                           _P]),
    "sa_decode_step": (ctypes.c_int, [_SH, _PG, _P, _P, _P, _P, _P, ctypes.c_int, _F, _F, _F, _I32,
                                      _I32, _I32, _P, _I64, _P, _P, _I32, _P, ctypes.c_int, _P, _P,
                                      _SZ, _P]),
    "sa_decode_step_rla": (ctypes.c_int, [_SH, _PG, _P, _P, _P, _P, _P, ctypes.c_int, _F, _F, _F,
                                          _I32, _I32, _I32, _P, _I64, _P, _P, _I32, _P,
                                          ctypes.c_int, _P, _P, _P, _P, _P, _SZ, _P]),
    "sa_decode_step_noalloc": (ctypes.c_int, [_SH, _PG, _P, _P, _P, _P, _P, ctypes.c_int, _F, _F,
                                              _F, _I32, _I32, _I32, _P, _I64, _P, _P, _I32, _P,
                                              ctypes.c_int, _P, _P]),
    "sa_decode_step_pages": (ctypes.c_int, [_SH, _PG, _P, _P, _P, _P, ctypes.c_int, _F, _I32, _P,
                                            _I64, _P, _P, _I32, _P, ctypes.c_int, _P, _P, _SZ, _P]),
    "sa_select_prefill_topk": (ctypes.c_int, [_SH, _PG, _I32, _P, _P, _P, ctypes.c_int, _F, _I32,
                                              _I32, _P, _P, _I32, _P, _SZ, _P]),
    "sa_select_prefill_topk_probs": (ctypes.c_int, [_SH, _PG, _I32, _P, _P, _P, ctypes.c_int, _F,
                                                    _I32, _I32, _P, _P, _I32, _P, _SZ, _P]),
    "sa_sparse_prefill_query": (ctypes.c_int, [_SH, _PG, _I32, _P, _P, _P, ctypes.c_int, _P, _P,
                                               _I32, _F, _P, ctypes.c_int, _P, _P, _SZ, _P]),
    "sa_select_prefill_oracle": (ctypes.c_int, [_SH, _PG, _I32, _P, _P, ctypes.c_int, _F, _I32,
                                                _I32, _P, _P, _I32, _P, _SZ, _P]),
    "sa_pbs_importance": (ctypes.c_int, [_SH, _PG, _I32, _P, _P, ctypes.c_int, _F, _I32, _P, _P,
                                         _SZ, _P]),
    "sa_pbs_permutation": (ctypes.c_int, [_SH, _P, _I32, _I32, _P, _P]),
    "sa_pbs_select": (ctypes.c_int, [_SH, _PG, _I32, _P, _P, ctypes.c_int, _P, _I32, _I32, _I32, _P,
                                     _P, _I32, _P, _SZ, _P]),
    "sa_sparse_prefill": (ctypes.c_int, [_SH, _PG, _I32, _P, _P, _P, ctypes.c_int, _P, _P, _I32,
                                         _I32, _F, _P, ctypes.c_int, _P, _P]),
    "sa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "sa_last_error": (ctypes.c_char_p, []),
    "sa_version": (ctypes.c_char_p, []),
}

_lib = None


class SAError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        super().__init__(f"{fn}: status {status}: {msg}")
        self.status = status


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libsa.so once (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(
            f"libsa.so not found at {p}; build it with "
            "`python -m dynamic_sparse_attention_02_amd.build` (hipcc, gfx950)")
    try:
        import torch  # noqa: F401  (load torch's HIP runtime first)
    except ImportError:
        pass
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def check(status: int, fn: str) -> None:
    if status != SA_OK:
        lib = load()
        msg = lib.sa_last_error().decode()
        raise SAError(status, fn, msg)

"""ctypes view of libtsa.so (declared in include/tsa.h).

Argument marshalling only: every step of the op runs in the library's HIP
kernels.  Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libtsa.so")
PROBE_PATH = os.path.join(PKG, "libtsa_probe.so")

TSA_OK, TSA_ERR_INVALID_ARG, TSA_ERR_UNSUPPORTED, TSA_ERR_WORKSPACE, TSA_ERR_HIP = range(5)
TSA_F32, TSA_BF16 = 0, 1
TSA_FLAG_NONCAUSAL_PROXY, TSA_FLAG_PER_HEAD_BUDGET, TSA_FLAG_KEEP_WINDOW = 1, 2, 4

# Every symbol include/tsa.h declares.
EXPORTS = ["tsa_status_string", "tsa_last_error", "tsa_version", "tsa_workspace_bytes",
           "tsa_forward_workspace_bytes", "tsa_score", "tsa_budget", "tsa_select", "tsa_gather",
           "tsa_attention", "tsa_scatter", "tsa_forward", "tsa_fused_workspace_bytes",
           "tsa_attention_indexed", "tsa_forward_fused", "tsa_zero_unselected",
           "tsa_block_mask_words", "tsa_attention_block_sparse", "tsa_attention_qo_indexed",
           "tsa_forward_fused_noalloc", "tsa_gather_kv"]


class TsaProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("L", ctypes.c_int32), ("d", ctypes.c_int32), ("w", ctypes.c_int32),
                ("tau", ctypes.c_float), ("dtype", ctypes.c_int32), ("flags", ctypes.c_int32)]


_P = ctypes.POINTER(TsaProblem)
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_i32 = ctypes.c_int32

_SIGNATURES = {
    "tsa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "tsa_last_error": (ctypes.c_char_p, []),
    "tsa_version": (ctypes.c_char_p, []),
    "tsa_workspace_bytes": (_sz, [_P]),
    "tsa_forward_workspace_bytes": (_sz, [_P]),
    "tsa_score": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _sz, _vp]),
    "tsa_budget": (ctypes.c_int, [_P, _vp, _vp, _vp, _sz, _vp]),
    "tsa_select": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "tsa_gather": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "tsa_attention": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _i32, _vp, _vp]),
    "tsa_scatter": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp]),
    "tsa_forward": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "tsa_fused_workspace_bytes": (_sz, [_P]),
    "tsa_attention_indexed": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "tsa_attention_qo_indexed": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "tsa_forward_fused": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "tsa_zero_unselected": (ctypes.c_int, [_P, _vp, _vp, _vp]),
    "tsa_block_mask_words": (_sz, [_P]),
    "tsa_attention_block_sparse": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp]),
    "tsa_forward_fused_noalloc": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "tsa_gather_kv": (ctypes.c_int, [_P, _vp, _vp, _vp, _vp, _vp, _vp]),
}

NOALLOC_SCRATCH_BYTES = 128 << 20    # TSA_NOALLOC_SCRATCH_BYTES in include/tsa.h
FORWARD_FUSED_MAX_L = 32768          # tsa_forward runs the fused kernels up to this L (include/tsa.h)

_lib = None


def load() -> ctypes.CDLL:
    """Load libtsa.so once; raise if it is missing (there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m token_sparse_attention_proxy_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


# include/tsa_probe.h: the bf16 MFMA ceiling probe, a library of its own.
PROBE_EXPORTS = ["tsa_probe_sink_bytes", "tsa_probe_mfma_bf16"]
_PROBE_SIGNATURES = {
    "tsa_probe_sink_bytes": (_sz, []),
    "tsa_probe_mfma_bf16": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, _vp, _sz,
                                           ctypes.POINTER(ctypes.c_double), _vp]),
}
_probe = None


def load_probe() -> ctypes.CDLL:
    """Load libtsa_probe.so once; raise if it is missing."""
    global _probe
    if _probe is None:
        if not os.path.exists(PROBE_PATH):
            raise RuntimeError(
                f"{PROBE_PATH} is not built; run `python -m token_sparse_attention_proxy_amd.build`")
        lib = ctypes.CDLL(PROBE_PATH)
        for name, (res, args) in _PROBE_SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _probe = lib
    return _probe


class TsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        self.status = status
        self.name = lib.tsa_status_string(status).decode()
        self.detail = lib.tsa_last_error().decode()
        super().__init__(f"{where}: {self.name}: {self.detail}")


def check(status: int, where: str) -> None:
    if status != TSA_OK:
        raise TsaError(status, where)

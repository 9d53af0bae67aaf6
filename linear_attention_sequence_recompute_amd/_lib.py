"""ctypes loader for libgdn.so: symbol signatures and status codes.

The library is built in-tree by ``build.build_library()``. Loading fails loudly
when it is missing: there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libgdn.so")

GDN_OK, GDN_EINVAL, GDN_EUNSUPPORTED, GDN_EWORKSPACE, GDN_EHIP = 0, -1, -2, -3, -4
GDN_BF16, GDN_F32 = 0, 1
GDN_NOALLOC_WORKSPACE_BYTES = 64 << 20  # include/gdn.h

# (name, restype, argtypes) for every entry point declared in include/*.h
_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t
SIGNATURES = {
    "gdn_chunk_fwd_workspace_bytes": (_SZ, [_I, _I64, _I, _I, _I, _I]),
    "gdn_chunk_fwd_plan": (_I, [_I, _I64, _I64, _I, _I, _I, _I, _P, _P]),
    "gdn_chunk_fwd": (_I, [_P, _P, _P, _P, _P, _P, _I, _I64, _I, _I, _I, _F, _I, _I,
                           _P, _P, _P, _P, _P, _I64, _P, _P, _SZ, _P]),
    "gdn_chunk_fwd_profiled": (_I, [_P, _P, _P, _P, _P, _P, _I, _I64, _I, _I, _I, _F, _I, _I,
                                    _P, _P, _P, _P, _P, _I64, _P, _P, _SZ, _P, _P]),
    "gdn_chunk_fwd_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _I, _I64, _I, _I, _I, _F, _I, _I,
                                   _P, _P, _P, _P, _P, _I64, _P, _P]),
    "gdn_recurrent_step": (_I, [_P, _P, _P, _P, _P, _P, _I64, _P, _P, _I, _I, _I, _I, _F, _I, _I, _P]),
    "gdn_recurrent_step_kda": (_I, [_P, _P, _P, _P, _P, _P, _I64, _P, _P, _I, _I, _I, _I, _F, _I, _I, _P]),
    "gdn_recurrent_verify": (_I, [_P, _P, _P, _P, _P, _P, _I64, _P, _I, _P, _P, _I, _I, _I, _I, _I, _F, _I, _I,
                                  _P]),
    "gdn_kda_gate": (_I, [_P, _P, _P, _P, _F, _I, _P, _P, _I, _I, _I, _P]),
    "gdn_fp8_quant": (_I, [_P, _P, _P, _I64, _I64, _I, _P]),
    "gdn_decode_prologue": (_I, [_P, _P, _P, _P, _I64, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P]),
    "gdn_decode_prologue_verify": (_I, [_P, _P, _P, _P, _I64, _P, _I, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I,
                                        _P]),
    "gdn_decode_layer": (_I, [_P, _P, _P, _P, _I64, _P, _P, _P, _I, _P, _I64, _P, _P, _F, _P, _I, _I, _I, _I, _F,
                              _P]),
    "gdn_gated_rmsnorm": (_I, [_P, _P, _P, _F, _P, _I, _I, _I, _I, _P]),
    "gdn_chunk_fwd_kda_workspace_bytes": (_SZ, [_I, _I64, _I, _I]),
    "gdn_chunk_fwd_kda": (_I, [_P, _P, _P, _P, _P, _P, _I, _I64, _I, _I, _I, _F, _I, _I,
                               _P, _P, _P, _P, _P, _I64, _P, _P, _SZ, _P]),
    "gdn_chunk_fwd_kda_profiled": (_I, [_P, _P, _P, _P, _P, _P, _I, _I64, _I, _I, _I, _F, _I, _I,
                                        _P, _P, _P, _P, _P, _I64, _P, _P, _SZ, _P, _P]),
    "gdn_status_string": (ctypes.c_char_p, [_I]),
    # measurement probes (include/gdn_probe.h)
    "gdn_probe_mfma_bf16": (_I, [_P, _I, _I, _P]),
    "gdn_probe_copy": (_I, [_P, _P, _I64, _P]),
    "gdn_probe_write": (_I, [_P, _I64, _P]),
    "gdn_probe_read": (_I, [_P, _P, _I64, _P]),
}


class GdnError(RuntimeError):
    """A non-zero status returned by the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m linear_attention_sequence_recompute_amd.build` (there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().gdn_status_string(status).decode()


def check(status: int, where: str) -> None:
    if status != GDN_OK:
        raise GdnError(status, where)

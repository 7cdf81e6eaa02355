"""ctypes handle on liblinattn.so (the C ABI of include/lin_attn.h).

Loading fails loudly when the library has not been built: there is no other
implementation behind this package.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblinattn.so")

LA_OK, LA_EINVAL, LA_EUNSUPPORTED, LA_ERANGE, LA_EHIP = 0, 1, 2, 3, 4
LA_BF16, LA_FP32 = 0, 1
LA_GATE_LOG, LA_GATE_BOUNDED_LOGIT = 0, 1

# Every symbol include/lin_attn.h declares, with its ctypes signature.
_P, _I, _F, _LL = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_longlong
SIGNATURES = {
    "lin_attn_chunk_fwd": (_I, [_P, _P, _P, _P, _I, _F, _P, _P, _P, _P,
                                _I, _I, _I, _I, _I, _I, _P, _LL, _P]),
    "lin_attn_chunk_fwd_workspace_size": (_LL, [_I, _I, _I, _I, _I, _I]),
    "lin_attn_chunk_fwd_noalloc": (_I, [_P, _P, _P, _P, _I, _F, _P, _P, _P, _P,
                                        _I, _I, _I, _I, _I, _I, _P]),
    "lin_attn_chunk_fwd_raw": (_I, [_P, _P, _P, _P, _I, _F, _P, _P, _P, _P,
                                    _I, _I, _I, _I, _I, _I, _P, _LL, _P]),
    "lin_attn_chunk_fwd_raw_affine": (_I, [_P, _P, _P, _P, _F, _P, _P, _P, _P, _P, _P,
                                           _I, _I, _I, _I, _I, _I, _P, _LL, _P]),
    "lin_attn_chunk_fwd_channel": (_I, [_P, _P, _P, _P, _I, _F, _P, _P, _P, _P,
                                        _I, _I, _I, _I, _I, _I, _P, _LL, _P]),
    "lin_attn_chunk_fwd_channel_workspace_size": (_LL, [_I, _I, _I, _I, _I, _I]),
    "lin_attn_chunk_fwd_channel_varlen": (_I, [_P, _P, _P, _P, _I, _F, _P, _P, _P, _P, _P, _I,
                                               _I, _I, _I, _I, _I, _P, _LL, _P]),
    "lin_attn_chunk_fwd_channel_varlen_workspace_size": (_LL, [_I, _I, _I, _I, _I, _I]),
    "lin_attn_chunk_fwd_varlen": (_I, [_P, _P, _P, _P, _I, _F, _P, _P, _P, _P, _P, _I,
                                       _I, _I, _I, _I, _I, _P, _LL, _P]),
    "lin_attn_chunk_fwd_varlen_workspace_size": (_LL, [_I, _I, _I, _I, _I, _I]),
    "lin_attn_chunk_fwd_varlen_raw": (_I, [_P, _P, _P, _P, _I, _F, _P, _P, _P, _P, _P, _I,
                                           _I, _I, _I, _I, _I, _P, _LL, _P]),
    "lin_attn_chunk_fwd_varlen_raw_affine": (_I, [_P, _P, _P, _P, _F, _P, _P, _P, _P, _P, _P,
                                                  _P, _I, _I, _I, _I, _I, _I, _P, _LL, _P]),
    "lin_attn_chunk_bwd": (_I, [_P, _P, _P, _P, _I, _F, _P, _P, _P, _P,
                                _P, _P, _P, _P, _P, _P,
                                _I, _I, _I, _I, _I, _I, _P, _LL, _P]),
    "lin_attn_chunk_bwd_workspace_size": (_LL, [_I, _I, _I, _I, _I, _I]),
    "lin_attn_chunk_bwd_segmented": (_I, [_P, _P, _P, _P, _I, _F, _P, _P, _P, _P,
                                          _P, _P, _P, _P, _P, _P,
                                          _I, _I, _I, _I, _I, _I, _I, _P, _LL, _P]),
    "lin_attn_chunk_bwd_segmented_workspace_size": (_LL, [_I, _I, _I, _I, _I, _I, _I]),
    "lin_attn_chunk_bwd_varlen": (_I, [_P, _P, _P, _P, _I, _F, _P, _P, _P, _P,
                                       _P, _P, _P, _P, _P, _P, _P,
                                       _I, _I, _I, _I, _I, _I, _P, _LL, _P]),
    "lin_attn_chunk_bwd_varlen_workspace_size": (_LL, [_I, _I, _I, _I, _I, _I]),
    "lin_attn_decode_step": (_I, [_P, _P, _P, _P, _I, _F, _P, _P, _P,
                                  _I, _I, _I, _I, _I, _P]),
    "lin_attn_decode_step_channel": (_I, [_P, _P, _P, _P, _I, _F, _P, _P, _P,
                                          _I, _I, _I, _I, _I, _P]),
    "lin_attn_gate": (_I, [_P, _F, _P, _LL, _P]),
    "lin_attn_check_inputs": (_I, [_P, _P, _P, _P, _I, _F, _P, _P, _LL, _I, _I, _I, _I, _I, _I,
                                   _P, _P]),
    "lin_attn_last_error": (ctypes.c_char_p, []),
    "lin_attn_version": (_I, []),
}

_lib = None


class LinAttnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"lin_attn error {code}: {msg}")
        self.code = code


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m chunked_gated_linear_amd.build`"
                " (or __graft_entry__.build()); there is no fallback implementation")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def check(code: int) -> None:
    if code != LA_OK:
        raise LinAttnError(code, lib().lin_attn_last_error().decode())

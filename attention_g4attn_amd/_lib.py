"""Locate and open libg4attn.so; declare the C signatures of include/g4attn.h.

There is no fallback: if the library is missing the first call raises.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libg4attn.so")
_LIB = None

# names and argtypes, in the order include/g4attn.h declares them
P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "g4attn_prefill_workspace_bytes": ([I, I, I, I, F, I], Z),
    "g4attn_local_prefill": ([P, P, P, P, P, I, I, I, I, I, I, F, F, I, I, P, Z, P], I),
    "g4attn_global_prefill": ([P, P, P, P, I, I, I, I, I, I, F, F, I, I, P, Z, P], I),
    "g4attn_vision_prefill": ([P, P, P, P, P, P, I, I, I, I, I, F, I, I, P, Z, P], I),
    "g4attn_decode": ([P, P, P, P, P, I, I, I, I, I, I, F, F, I, I, P, Z, P], I),
    "g4attn_decode_workspace_bytes": ([I, I, I, I, I, I], Z),
    "g4attn_decode_noalloc": ([P, P, P, P, P, I, I, I, I, I, I, F, F, I, I, P], I),
    "g4attn_decode_multi": ([P, P, P, P, P, I, I, I, I, I, I, I, F, F, I, I, P, Z, P], I),
    "g4attn_decode_multi_workspace_bytes": ([I, I, I, I, I, I, I], Z),
    "g4attn_fill_cache": ([P, P, P, I, I, I, I, P, P, I, I, F, F, I, P], I),
    "g4attn_fill_cache_fp8": ([P, P, P, P, P, I, I, I, I, P, P, I, I, F, F, I, P], I),
    "g4attn_decode_fp8": ([P, P, P, P, P, P, P, I, I, I, I, I, I, I, F, F, I, P, Z, P], I),
    "g4attn_decode_fp8_workspace_bytes": ([I, I, I, I, I, I, I], Z),
    "g4attn_strerror": ([I], ctypes.c_char_p),
    "g4attn_last_hip_error": ([], I),
}


def lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m attention_g4attn_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.argtypes = args
            fn.restype = res
        _LIB = h
    return _LIB

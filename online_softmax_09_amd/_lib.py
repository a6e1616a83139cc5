"""ctypes loader for libmi355attn.so (the C ABI declared in include/mi355attn.h).

Loading the library does not touch the GPU; the HIP runtime initialises on the first
kernel launch.  There is no fallback: if the library is missing, every call raises.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# The in-tree library.  MI355ATTN_LIB_PATH names another build of the same C ABI (the
# tests use it for a host-only AddressSanitizer build of the argument checks).
LIB_PATH = os.environ.get("MI355ATTN_LIB_PATH") or os.path.join(_HERE, "libmi355attn.so")

# Return codes, as in include/mi355attn.h (FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED,
# FA_ERR_HIP).
OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED = -2
ERR_HIP = -3

# Bytes of device scratch fa_fwd_splitkv_noalloc holds per device.
SPLITKV_SCRATCH_BYTES = 32 << 20

# Every symbol the header declares, with (restype, argtypes).
_c_int, _c_i64, _c_f, _vp = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
SIGNATURES = {
    "fa_fwd": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_f, _c_int, _vp]),
    "fa_fwd_f16": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_f, _c_int, _vp]),
    "fa_fwd_f32": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_f, _c_int, _vp]),
    "online_softmax_rows": (_c_int, [_vp, _vp, _c_i64, _c_i64, _vp]),
    "fa_bwd": (_c_int, [_vp] * 10 + [_c_int, _c_int, _c_int, _c_int, _c_f, _c_int, _vp]),
    "fa_bwd_workspace_bytes": (_c_i64, [_c_int, _c_int, _c_int]),
    "fa_fwd_splitkv": (_c_int, [_vp] * 6 + [_c_int] * 5 + [_c_f, _c_int, _c_int, _vp]),
    "fa_fwd_splitkv_workspace_bytes": (_c_i64, [_c_int] * 5),
    "fa_fwd_splitkv_noalloc": (_c_int, [_vp] * 5 + [_c_int] * 5 + [_c_f, _c_int, _c_int, _vp]),
    "attn_merge_states": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_i64, _c_int, _vp]),
    "fused_add_rmsnorm": (_c_int, [_vp] * 5 + [_c_i64, _c_i64, _c_f, _vp]),
    "fused_add_layernorm": (_c_int, [_vp] * 6 + [_c_i64, _c_i64, _c_f, _vp]),
    "fa_strerror": (ctypes.c_char_p, [_c_int]),
    "mi355attn_strerror": (ctypes.c_char_p, [_c_int]),
    "mi355attn_last_hip_error": (_c_int, []),
    "mi355attn_version": (_c_int, []),
}

_lib = None


def load():
    """The loaded library, with argument and return types set.  Raises if not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m online_softmax_09_amd.build` first")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def strerror(code):
    return load().fa_strerror(int(code)).decode()


def check(code, what):
    if code != OK:
        detail = ""
        if code == ERR_HIP:
            detail = f" (hipError_t {load().mi355attn_last_hip_error()})"
        raise RuntimeError(f"{what}: {strerror(code)}{detail}")

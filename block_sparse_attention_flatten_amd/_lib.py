"""ctypes view of libnabla's C ABI (include/nabla.h).

Only the raw symbols and their signatures live here; ``api.py`` adds the
torch-tensor marshalling.  Loading fails loudly when the library has not been
built: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnabla.so")

NABLA_OK = 0
STATUS = {
    0: "NABLA_OK", -1: "NABLA_E_NULL", -2: "NABLA_E_SHAPE", -3: "NABLA_E_DTYPE",
    -4: "NABLA_E_HEAD_DIM", -5: "NABLA_E_PATCH", -6: "NABLA_E_THR", -7: "NABLA_E_STA",
    -8: "NABLA_E_WORKSPACE", -9: "NABLA_E_LAYOUT", -10: "NABLA_E_HIP", -11: "NABLA_E_SCALE",
    -12: "NABLA_E_TOO_LARGE",
}
DTYPE_F32, DTYPE_BF16 = 0, 1
LAYOUT_THW, LAYOUT_BLOCKED = 0, 1
MAX_BLOCKS = 4096
WORKSPACE_PARTS = 7


class nabla_geom(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int64), ("heads", ctypes.c_int64),
        ("T", ctypes.c_int32), ("H", ctypes.c_int32), ("W", ctypes.c_int32),
        ("P", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("layout", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
    ]


_P = ctypes.c_void_p
_G = ctypes.POINTER(nabla_geom)
_I32P = ctypes.POINTER(ctypes.c_int32)
_SZP = ctypes.POINTER(ctypes.c_size_t)

SIGNATURES = {
    "nabla_num_blocks": ([_G, ctypes.POINTER(ctypes.c_int64)], ctypes.c_int),
    "nabla_flatten": ([_G, _P, _P, _P], ctypes.c_int),
    "nabla_unflatten": ([_G, _P, _P, _P], ctypes.c_int),
    "nabla_pool": ([_G, _P, _P, _P, _P, _P], ctypes.c_int),
    "nabla_mask": ([_G, _P, _P, ctypes.c_float, _I32P, _P, _P, _P, _P], ctypes.c_int),
    "nabla_compact": ([_G, _P, _P, _P, _P, _P], ctypes.c_int),
    "nabla_mask_build": ([_G, _P, _P, ctypes.c_float, _I32P, _P, _P, _P, _P, _P, _P, _P, _P],
                         ctypes.c_int),
    "nabla_attn_fwd": ([_G, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P], ctypes.c_int),
    "nabla_transpose_v": ([_G, _P, _P, _P], ctypes.c_int),
    "nabla_attn_fwd_vt": ([_G, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P], ctypes.c_int),
    "nabla_dense_attn_fwd": ([_G, _P, _P, _P, ctypes.c_float, _P, _P, _P], ctypes.c_int),
    "nabla_qkv_split": ([_G, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "nabla_attn_fwd_lse": ([_G, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P], ctypes.c_int),
    "nabla_attn_fwd_vt_lse": ([_G, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P],
                              ctypes.c_int),
    "nabla_mask_transpose": ([_G, _P, _P, _P, _P], ctypes.c_int),
    "nabla_attn_bwd_dq": ([_G, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P],
                          ctypes.c_int),
    "nabla_attn_bwd_dkdv": ([_G, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P],
                            ctypes.c_int),
    "nabla_forward_workspace_size": ([_G, _SZP, _SZP], ctypes.c_int),
    "nabla_forward": ([_G, _P, _P, _P, ctypes.c_float, _I32P, ctypes.c_float, _P, _P,
                       ctypes.c_size_t, _P], ctypes.c_int),
    "nabla_forward_noalloc": ([_G, _P, _P, _P, ctypes.c_float, _I32P, ctypes.c_float, _P, _P],
                              ctypes.c_int),
    "nabla_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "nabla_last_hip_error": ([], ctypes.c_int),
    "nabla_abi_version": ([], ctypes.c_int),
}

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libnabla once and attach the signatures of every exported call."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"libnabla is not built ({path} missing); run "
            "`python -m block_sparse_attention_flatten_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (args, res) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib

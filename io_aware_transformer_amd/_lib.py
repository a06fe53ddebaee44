"""ctypes loader for libfa.so and the C ABI declared in include/fa.h.

Loading fails loudly (``LibraryNotBuilt``) when the library is missing:
there is no fallback implementation of any entry point.
"""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

# include/fa.h: block-sparse map blocks and sequence limit
FA_SPARSE_BLOCK = 128
FA_SPARSE_MAX_N = 65536
# include/fa.h: largest B * H_q * N of fa_bwd_noalloc
FA_NOALLOC_MAX_ROWS = 1 << 21

# enum fa_dtype
FA_BF16 = 0
FA_FP32 = 1

# enum fa_status
STATUS = {
    0: "FA_OK",
    -1: "FA_ERR_NULL",
    -2: "FA_ERR_SHAPE",
    -3: "FA_ERR_HEADDIM",
    -4: "FA_ERR_DTYPE",
    -5: "FA_ERR_ALIGN",
    -6: "FA_ERR_WORKSPACE",
    -7: "FA_ERR_UNSUPPORTED",
    -8: "FA_ERR_HIP",
    -9: "FA_ERR_ARG",
}
STATUS_CODE = {v: k for k, v in STATUS.items()}

# every symbol include/fa.h declares
EXPORTS = (
    "fa_fwd",
    "fa_bwd",
    "fa_bwd_workspace_size",
    "fa_status_str",
    "fa_last_hip_error",
    "fa_version",
    "fa_fwd_split_parts",
    "fa_fwd_split_workspace_size",
    "fa_fwd_split",
    "fa_lse_merge",
    "fa_fwd_window",
    "fa_bwd_window",
    "fa_fwd_varlen",
    "fa_bwd_varlen_workspace_size",
    "fa_bwd_varlen",
    "fa_bwd_noalloc",
    "fa_fwd_blocksparse",
    "fa_bwd_blocksparse",
    "fa_fwd_dropout",
    "fa_bwd_dropout",
)


class LibraryNotBuilt(RuntimeError):
    pass


class FAError(RuntimeError):
    def __init__(self, status, where, hip_error=0):
        self.status = status
        self.hip_error = hip_error
        name = STATUS.get(status, str(status))
        extra = f" (hipError_t {hip_error})" if status == STATUS_CODE["FA_ERR_HIP"] else ""
        super().__init__(f"{where} failed: {name}{extra}")


_lib = None

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float


def load():
    """Load libfa.so once and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise LibraryNotBuilt(
            f"{LIB_PATH} is missing: build it with `python -m io_aware_transformer_amd.build`"
        )
    lib = ctypes.CDLL(LIB_PATH)
    lib.fa_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _vp]
    lib.fa_fwd.restype = _i
    lib.fa_bwd.argtypes = [_vp] * 10 + [ctypes.c_size_t, _i, _i, _i, _i, _i, _f, _i, _i, _vp]
    lib.fa_bwd.restype = _i
    lib.fa_bwd_workspace_size.argtypes = [_i, _i, _i, _i, _i, _i]
    lib.fa_bwd_workspace_size.restype = ctypes.c_size_t
    lib.fa_status_str.argtypes = [_i]
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_last_hip_error.argtypes = []
    lib.fa_last_hip_error.restype = _i
    lib.fa_version.argtypes = []
    lib.fa_version.restype = _i
    lib.fa_fwd_split_parts.argtypes = [_i] * 7
    lib.fa_fwd_split_parts.restype = _i
    lib.fa_fwd_split_workspace_size.argtypes = [_i] * 8
    lib.fa_fwd_split_workspace_size.restype = ctypes.c_size_t
    lib.fa_fwd_split.argtypes = [_vp] * 5 + [_i] * 6 + [_f, _i, _i, _vp, ctypes.c_size_t, _i, _vp]
    lib.fa_fwd_split.restype = _i
    lib.fa_lse_merge.argtypes = [_vp, _vp, _i, ctypes.c_longlong, _i, _vp, _vp, _i, _vp]
    lib.fa_lse_merge.restype = _i
    lib.fa_fwd_window.argtypes = [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _i, _vp]
    lib.fa_fwd_window.restype = _i
    lib.fa_bwd_window.argtypes = [_vp] * 10 + [ctypes.c_size_t, _i, _i, _i, _i, _i, _f, _i, _i, _i, _vp]
    lib.fa_bwd_window.restype = _i
    # Q K V O LSE cu | batch total max_seqlen H_q H_kv d | scale | causal dtype | stream
    lib.fa_fwd_varlen.argtypes = [_vp] * 6 + [_i] * 6 + [_f, _i, _i, _vp]
    lib.fa_fwd_varlen.restype = _i
    lib.fa_bwd_varlen_workspace_size.argtypes = [_i] * 5
    lib.fa_bwd_varlen_workspace_size.restype = ctypes.c_size_t
    # Q K V O dO LSE dQ dK dV workspace | bytes | cu | batch total max_seqlen H_q H_kv d | scale | causal dtype | stream
    lib.fa_bwd_varlen.argtypes = [_vp] * 10 + [ctypes.c_size_t, _vp] + [_i] * 6 + [_f, _i, _i, _vp]
    lib.fa_bwd_varlen.restype = _i
    # Q K V O dO LSE dQ dK dV | B H_q H_kv N d | scale | causal dtype | stream
    lib.fa_bwd_noalloc.argtypes = [_vp] * 9 + [_i] * 5 + [_f, _i, _i, _vp]
    lib.fa_bwd_noalloc.restype = _i
    # Q K V O LSE mask | B H_q H_kv N d | scale | causal dtype | stream
    lib.fa_fwd_blocksparse.argtypes = [_vp] * 6 + [_i] * 5 + [_f, _i, _i, _vp]
    lib.fa_fwd_blocksparse.restype = _i
    # Q K V O dO LSE dQ dK dV workspace | bytes | mask | B H_q H_kv N d | scale | causal dtype | stream
    lib.fa_bwd_blocksparse.argtypes = [_vp] * 10 + [ctypes.c_size_t, _vp] + [_i] * 5 + [_f, _i, _i, _vp]
    lib.fa_bwd_blocksparse.restype = _i
    _u64, _u32 = ctypes.c_ulonglong, ctypes.c_uint
    # Q K V O LSE | B H_q H_kv N d | scale | causal | p seed offset | dtype stream
    lib.fa_fwd_dropout.argtypes = [_vp] * 5 + [_i] * 5 + [_f, _i, _f, _u64, _u32, _i, _vp]
    lib.fa_fwd_dropout.restype = _i
    # Q K V O dO LSE dQ dK dV workspace | bytes | B H_q H_kv N d | scale | causal | p seed offset | dtype stream
    lib.fa_bwd_dropout.argtypes = [_vp] * 10 + [ctypes.c_size_t] + [_i] * 5 + [_f, _i, _f, _u64, _u32, _i, _vp]
    lib.fa_bwd_dropout.restype = _i
    _lib = lib
    return lib


def check(status, where):
    if status != 0:
        hip = load().fa_last_hip_error() if status == STATUS_CODE["FA_ERR_HIP"] else 0
        raise FAError(status, where, hip)

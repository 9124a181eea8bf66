"""ctypes declarations of libcp_attn.so (the C ABI in include/cp_attn.h).

Loading fails loudly when the library has not been built: there is no other
implementation to fall back to.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcp_attn.so")

CP_OK, CP_ERR_INVALID, CP_ERR_UNSUPPORTED, CP_ERR_ALIAS, CP_ERR_HIP = range(5)
CP_DTYPE_BF16, CP_DTYPE_F32 = 0, 1
# scratch bytes of cp_attn_bwd_noalloc per device (CP_ATTN_BWD_NOALLOC_MAX_BYTES)
CP_ATTN_BWD_NOALLOC_MAX_BYTES = 32 << 20

# (name, restype, argtypes) of every exported entry point
c_i64, c_i32, c_vp, c_f = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_float


class AttnArgs(ctypes.Structure):
    """Mirror of cp_attn_args_t."""

    _fields_ = [
        ("batch", c_i64), ("seqlen_q", c_i64), ("seqlen_k", c_i64), ("heads_q", c_i64),
        ("heads_kv", c_i64), ("head_dim", c_i64), ("dtype", c_i32), ("causal", c_i32),
        ("q_offset", c_i64), ("k_offset", c_i64), ("q_pos", c_vp), ("k_pos", c_vp),
        ("q_seg", c_vp), ("k_seg", c_vp), ("window", c_i64), ("softmax_scale", c_f),
    ]


class RelayoutArgs(ctypes.Structure):
    """Mirror of cp_relayout_args_t."""

    _fields_ = [
        ("groups", c_i64), ("P", c_i64), ("batch", c_i64), ("seqlen", c_i64), ("heads", c_i64),
        ("head_dim", c_i64), ("elem_bytes", c_i64), ("rep", c_i64), ("inverse", c_i32),
    ]


SIGNATURES = {
    "cp_attn_fwd": (c_i32, [ctypes.POINTER(AttnArgs), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "cp_attn_fwd_merge": (c_i32, [ctypes.POINTER(AttnArgs), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "cp_attn_fwd_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(AttnArgs)]),
    "cp_attn_fwd_ws": (c_i32, [ctypes.POINTER(AttnArgs), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, ctypes.c_size_t,
                               c_vp]),
    "cp_attn_bwd_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(AttnArgs)]),
    "cp_attn_check_args": (c_i32, [ctypes.POINTER(AttnArgs), c_vp, c_vp]),
    "cp_attn_bwd": (c_i32, [ctypes.POINTER(AttnArgs), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                            c_vp, c_i32, c_vp, ctypes.c_size_t, c_vp]),
    "cp_attn_bwd_rows_ready": (c_i32, [ctypes.POINTER(AttnArgs), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                            c_vp, c_i32, c_vp, ctypes.c_size_t, c_vp]),
    "cp_attn_bwd_noalloc": (c_i32, [ctypes.POINTER(AttnArgs), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp,
                                    c_vp, c_i32, c_vp]),
    "cp_lse_merge": (c_i32, [c_i64, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_i32, c_vp]),
    "cp_ulysses_relayout": (c_i32, [c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_i64, c_i64, c_vp]),
    "cp_ulysses_relayout_inv": (c_i32, [c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_i64, c_i64, c_vp]),
    "cp_zigzag_reorder": (c_i32, [c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, c_i32, c_i32, c_vp]),
    "cp_ulysses_relayout_ex": (c_i32, [ctypes.POINTER(RelayoutArgs), c_vp, c_vp, c_vp]),
    "cp_pad_rows": (c_i32, [c_vp, c_vp, c_i64, c_i64, c_i64, c_i64, ctypes.c_uint32, c_vp]),
    "cp_prof_enable": (None, [c_i32]),
    "cp_prof_reset": (None, []),
    "cp_prof_kernel_count": (c_i32, []),
    "cp_prof_kernel_name": (ctypes.c_char_p, [c_i32]),
    "cp_prof_read": (c_i32, [c_i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]),
    "cp_status_string": (ctypes.c_char_p, [c_i32]),
    "cp_last_error": (ctypes.c_char_p, []),
}

_lib = None


def load():
    """The loaded library (built by ``python -m context_cp_attn_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m context_cp_attn_amd.build` "
                "(the HIP library is the only implementation)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class CpError(ValueError):
    """A call rejected by libcp_attn (status != CP_OK)."""

    def __init__(self, status: int, message: str):
        self.status = status
        name = load().cp_status_string(status).decode()
        super().__init__(f"{name}: {message}")


def check(status: int) -> None:
    if status != CP_OK:
        raise CpError(status, load().cp_last_error().decode())


class KernelTrace:
    """Per-kernel durations from the library's HIP-event tracing.

        with KernelTrace() as tr:
            ...launches...
        tr.results  # {kernel name: (total_ms, launches)}
    """

    def __enter__(self):
        lib = load()
        lib.cp_prof_reset()
        lib.cp_prof_enable(1)
        return self

    def __exit__(self, *exc):
        lib = load()
        lib.cp_prof_enable(0)
        self.results = {}
        for i in range(lib.cp_prof_kernel_count()):
            ms, n = ctypes.c_double(), ctypes.c_int64()
            check(lib.cp_prof_read(i, ctypes.byref(ms), ctypes.byref(n)))
            if n.value:
                self.results[lib.cp_prof_kernel_name(i).decode()] = (ms.value, n.value)
        lib.cp_prof_reset()
        return False

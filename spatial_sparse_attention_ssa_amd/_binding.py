"""ctypes view of the C ABI declared in include/ssa.h.

Argument marshalling only: every computation runs inside libssa.so.  If the
shared library has not been built the import of the package still succeeds,
but every call raises, so no code path can silently run without the HIP
kernels.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libssa.so")

SSA_OK = 0
SSA_ERR_INVALID_ARGUMENT = 1
SSA_ERR_UNSUPPORTED = 2
SSA_ERR_WORKSPACE = 3
SSA_ERR_DEVICE = 4

SSA_F32 = 0
SSA_BF16 = 1

SSA_ROUTE_SCORE = 0
SSA_ROUTE_GEOMETRIC = 1

SSA_COUNT_NB = 0
SSA_COUNT_NW = 1
SSA_COUNT_INVALID = 2
SSA_COUNT_MAX_BLK = 3
SSA_COUNT_MAX_WIN = 4
SSA_COUNT_KEY_BITS = 5
SSA_COUNTS = 8
SSA_STAGES = 12
SSA_NOALLOC_SCRATCH_BYTES = 64 << 20

# every symbol include/ssa.h declares
EXPORTED = (
    "ssa_build_blocks_workspace",
    "ssa_build_blocks",
    "ssa_forward_workspace",
    "ssa_forward",
    "ssa_forward_timed",
    "ssa_forward_noalloc",
    "ssa_stage_name",
    "ssa_forward_train",
    "ssa_backward_workspace",
    "ssa_backward",
    "ssa_backward_timed",
    "ssa_backward_stage_name",
    "ssa_status_string",
    "ssa_last_error",
    "ssa_version",
)


class SsaGeometry(ctypes.Structure):
    _fields_ = [("grid_res", ctypes.c_int32), ("m_cmp", ctypes.c_int32), ("m_win", ctypes.c_int32),
                ("win_shift", ctypes.c_int32)]


class SsaBlocks(ctypes.Structure):
    _fields_ = [
        ("perm", ctypes.c_void_p),
        ("blk_off", ctypes.c_void_p),
        ("win_off", ctypes.c_void_p),
        ("win_blk_off", ctypes.c_void_p),
        ("seq_blk_off", ctypes.c_void_p),
        ("seq_win_off", ctypes.c_void_p),
        ("counts", ctypes.c_void_p),
        ("n_tokens", ctypes.c_int64),
        ("batch", ctypes.c_int32),
        ("nb", ctypes.c_int32),
        ("nw", ctypes.c_int32),
        ("max_blk_tokens", ctypes.c_int32),
        ("max_win_tokens", ctypes.c_int32),
        ("geo", SsaGeometry),
        ("coords", ctypes.c_void_p),
    ]


class SsaAttn(ctypes.Structure):
    _fields_ = [
        ("h_q", ctypes.c_int32),
        ("h_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("dtype", ctypes.c_int),
        ("routing", ctypes.c_int32),
    ]


class SsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded libssa.so; raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"libssa.so not found at {LIB_PATH}: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
    L.ssa_build_blocks_workspace.argtypes = [i64, i32, ctypes.POINTER(SsaGeometry)]
    L.ssa_build_blocks_workspace.restype = sz
    L.ssa_build_blocks.argtypes = [vp, vp, i64, i32, ctypes.POINTER(SsaGeometry),
                                   ctypes.POINTER(SsaBlocks), ctypes.c_int, vp, sz, vp]
    L.ssa_build_blocks.restype = ctypes.c_int
    L.ssa_forward_workspace.argtypes = [ctypes.POINTER(SsaBlocks), ctypes.POINTER(SsaAttn)]
    L.ssa_forward_workspace.restype = sz
    L.ssa_forward.argtypes = [ctypes.POINTER(SsaBlocks), ctypes.POINTER(SsaAttn), vp, vp, vp, vp, vp,
                              vp, vp, vp, vp, sz, vp]
    L.ssa_forward.restype = ctypes.c_int
    L.ssa_forward_timed.argtypes = [ctypes.POINTER(SsaBlocks), ctypes.POINTER(SsaAttn), vp, vp, vp, vp,
                                    vp, vp, vp, vp, vp, sz, vp, ctypes.POINTER(ctypes.c_float),
                                    ctypes.POINTER(i32)]
    L.ssa_forward_timed.restype = ctypes.c_int
    L.ssa_forward_noalloc.argtypes = [ctypes.POINTER(SsaBlocks), ctypes.POINTER(SsaAttn), vp, vp, vp, vp, vp,
                                      vp, vp, vp, vp]
    L.ssa_forward_noalloc.restype = ctypes.c_int
    L.ssa_stage_name.argtypes = [ctypes.POINTER(SsaAttn), i32]
    L.ssa_stage_name.restype = ctypes.c_char_p
    L.ssa_forward_train.argtypes = [ctypes.POINTER(SsaBlocks), ctypes.POINTER(SsaAttn), vp, vp, vp, vp, vp,
                                    vp, vp, vp, sz, vp]
    L.ssa_forward_train.restype = ctypes.c_int
    L.ssa_backward_workspace.argtypes = [ctypes.POINTER(SsaBlocks), ctypes.POINTER(SsaAttn)]
    L.ssa_backward_workspace.restype = sz
    bwd = [ctypes.POINTER(SsaBlocks), ctypes.POINTER(SsaAttn), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
           vp, vp, sz, vp]
    L.ssa_backward.argtypes = bwd
    L.ssa_backward.restype = ctypes.c_int
    L.ssa_backward_timed.argtypes = bwd + [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(i32)]
    L.ssa_backward_timed.restype = ctypes.c_int
    L.ssa_backward_stage_name.argtypes = [ctypes.POINTER(SsaAttn), i32]
    L.ssa_backward_stage_name.restype = ctypes.c_char_p
    L.ssa_status_string.argtypes = [ctypes.c_int]
    L.ssa_status_string.restype = ctypes.c_char_p
    L.ssa_last_error.argtypes = []
    L.ssa_last_error.restype = ctypes.c_char_p
    L.ssa_version.argtypes = []
    L.ssa_version.restype = i32
    _LIB = L
    return L


def check(status: int) -> None:
    if status != SSA_OK:
        L = lib()
        msg = L.ssa_last_error().decode() or L.ssa_status_string(status).decode()
        raise SsaError(status, msg)

"""ctypes declarations of libvsa_h3.so and thin wrappers with the C ABI's names.

Argument marshalling only: every step of the forward runs in the library's
HIP kernels.  There is no fallback: a missing library raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvsa_h3.so")

VSA_OK, VSA_E_ARG, VSA_E_LAYOUT, VSA_E_POSITIONS = 0, -1, -2, -3
VSA_E_UNSUPPORTED, VSA_E_WORKSPACE, VSA_E_HIP = -4, -5, -6
STATUS_NAMES = {0: "VSA_OK", -1: "VSA_E_ARG", -2: "VSA_E_LAYOUT", -3: "VSA_E_POSITIONS",
                -4: "VSA_E_UNSUPPORTED", -5: "VSA_E_WORKSPACE", -6: "VSA_E_HIP"}
VSA_BF16, VSA_F32 = 0, 1
VSA_TAG_TEXT, VSA_TAG_COND, VSA_TAG_AUDIO, VSA_TAG_VIDEO = 0, 1, 2, 3

EXPORTED = (
    "vsa_h3_topk", "vsa_h3_plan_create", "vsa_h3_plan_info", "vsa_h3_plan_set_chunk_tiles",
    "vsa_h3_plan_layout",
    "vsa_h3_plan_tables", "vsa_h3_plan_upload", "vsa_h3_forward", "vsa_h3_forward_timed",
    "vsa_h3_oneshot_workspace_bytes", "vsa_h3_forward_oneshot", "vsa_h3_plan_destroy",
    "vsa_h3_last_error", "vsa_h3_version", "vsa_h3_plan_set_qk_prep", "vsa_h3_forward_qk_prep",
    "vsa_h3_plan_set_qk_fp8", "vsa_h3_plan_set_ref_keep", "vsa_h3_plan_set_io_dtype",
    "vsa_h3_forward_noalloc",
)


class VsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class Dims3(ctypes.Structure):
    _fields_ = [("t", ctypes.c_int32), ("h", ctypes.c_int32), ("w", ctypes.c_int32)]


class Info(ctypes.Structure):
    _fields_ = [("L", ctypes.c_int64), ("num_prefix_tiles", ctypes.c_int64),
                ("num_video_tiles", ctypes.c_int64), ("num_tiles", ctypes.c_int64),
                ("topk", ctypes.c_int64), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("workspace_bytes", ctypes.c_uint64),
                ("chunk_tiles", ctypes.c_int32), ("num_chunks", ctypes.c_int32),
                ("num_ref_tiles", ctypes.c_int64), ("topk_ref", ctypes.c_int64),
                ("ref_keep", ctypes.c_double), ("tile_tokens", ctypes.c_int32),
                ("num_blocks", ctypes.c_int32)]


class WsLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in ("perm", "valid", "kt", "vt", "qp", "kp", "vp",
                                               "scores", "coarse", "sel", "total")] + \
               [("scores_row_stride", ctypes.c_int64), ("chunk_offsets", ctypes.c_uint64),
                ("state", ctypes.c_uint64), ("qt", ctypes.c_uint64), ("kt8", ctypes.c_uint64),
                ("kscale", ctypes.c_uint64), ("kind", ctypes.c_uint64),
                ("visit", ctypes.c_uint64), ("order", ctypes.c_uint64),
                ("kt_lo", ctypes.c_uint64), ("vt_lo", ctypes.c_uint64),
                ("qt_lo", ctypes.c_uint64)]


_lib = None
_lib_lock = threading.Lock()
_P = ctypes.c_void_p
_I64P = ctypes.POINTER(ctypes.c_int64)
_I32P = ctypes.POINTER(ctypes.c_int32)


def lib() -> ctypes.CDLL:
    """Load libvsa_h3.so once.  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m video_dit_block_amd.build` (no fallback path exists)")
        L = ctypes.CDLL(LIB_PATH)
        L.vsa_h3_topk.argtypes = [ctypes.c_int64, ctypes.c_double]
        L.vsa_h3_topk.restype = ctypes.c_int64
        L.vsa_h3_plan_create.argtypes = [_I64P, _I64P, ctypes.c_int64, Dims3, Dims3,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_double,
                                         ctypes.POINTER(_P)]
        L.vsa_h3_plan_info.argtypes = [_P, ctypes.POINTER(Info)]
        L.vsa_h3_plan_set_chunk_tiles.argtypes = [_P, ctypes.c_int32]
        L.vsa_h3_plan_layout.argtypes = [_P, ctypes.POINTER(WsLayout)]
        L.vsa_h3_plan_tables.argtypes = [_P, _I32P, _I32P, _I32P]
        L.vsa_h3_plan_upload.argtypes = [_P, _P, ctypes.c_uint64, _P]
        L.vsa_h3_forward.argtypes = [_P, _P, _P, _P, _P, ctypes.c_int, _P, _P, _P,
                                     ctypes.c_uint64, _P]
        L.vsa_h3_forward_timed.argtypes = [_P, _P, _P, _P, _P, ctypes.c_int, _P, _P, _P,
                                           ctypes.c_uint64, _P, ctypes.POINTER(_P)]
        L.vsa_h3_oneshot_workspace_bytes.argtypes = [_I64P, _I64P, ctypes.c_int64, Dims3, Dims3,
                                                     ctypes.c_int32, ctypes.c_int32,
                                                     ctypes.c_double, ctypes.c_int,
                                                     ctypes.POINTER(ctypes.c_uint64)]
        L.vsa_h3_forward_oneshot.argtypes = [_P, _P, _P, _P, _I64P, _I64P, ctypes.c_int64,
                                             ctypes.c_int32, ctypes.c_int32, Dims3,
                                             ctypes.c_double, Dims3, ctypes.c_int, _P, _P, _P,
                                             ctypes.c_uint64, _P]
        L.vsa_h3_plan_set_qk_prep.argtypes = [_P, ctypes.c_int32]
        L.vsa_h3_plan_set_qk_fp8.argtypes = [_P, ctypes.c_int32]
        L.vsa_h3_plan_set_ref_keep.argtypes = [_P, ctypes.c_double]
        L.vsa_h3_plan_set_io_dtype.argtypes = [_P, ctypes.c_int]
        L.vsa_h3_forward_noalloc.argtypes = [_P, _P, _P, _P, _P, ctypes.c_int, _P, _P, _P]
        L.vsa_h3_forward_qk_prep.argtypes = [_P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P,
                                             ctypes.c_int, _P, _P, _P, ctypes.c_uint64, _P,
                                             ctypes.POINTER(_P)]
        L.vsa_h3_plan_destroy.argtypes = [_P]
        L.vsa_h3_plan_destroy.restype = None
        L.vsa_h3_last_error.restype = ctypes.c_char_p
        L.vsa_h3_version.restype = ctypes.c_char_p
        for name in EXPORTED:
            if name not in ("vsa_h3_topk", "vsa_h3_plan_destroy", "vsa_h3_last_error",
                            "vsa_h3_version"):
                getattr(L, name).restype = ctypes.c_int
        _lib = L
        return L


def check(status: int) -> None:
    if status != VSA_OK:
        raise VsaError(status, lib().vsa_h3_last_error().decode())


def _i64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


def _ptr64(a: np.ndarray):
    return a.ctypes.data_as(_I64P)


# ---------------------------------------------------------------- same-name wrappers
def vsa_h3_topk(num_video_tiles: int, sparsity: float) -> int:
    return int(lib().vsa_h3_topk(int(num_video_tiles), float(sparsity)))


def vsa_h3_plan_create(token_tags, position_ids, grid, tile, heads, head_dim, sparsity) -> int:
    """Returns an opaque plan handle (int).  token_tags [L], position_ids [L, 3]: host int64."""
    tags = _i64(token_tags).reshape(-1)
    pos = _i64(position_ids).reshape(-1, 3)
    if pos.shape[0] != tags.shape[0]:
        raise VsaError(VSA_E_ARG, "position_ids must be [L, 3] with L = len(token_tags)")
    handle = _P()
    check(lib().vsa_h3_plan_create(_ptr64(tags), _ptr64(pos), tags.shape[0], Dims3(*grid),
                                   Dims3(*tile), int(heads), int(head_dim), float(sparsity),
                                   ctypes.byref(handle)))
    return handle.value


def vsa_h3_plan_info(plan: int) -> Info:
    info = Info()
    check(lib().vsa_h3_plan_info(plan, ctypes.byref(info)))
    return info


def vsa_h3_plan_set_chunk_tiles(plan: int, chunk_tiles: int) -> None:
    check(lib().vsa_h3_plan_set_chunk_tiles(plan, int(chunk_tiles)))


def vsa_h3_plan_layout(plan: int) -> WsLayout:
    lo = WsLayout()
    check(lib().vsa_h3_plan_layout(plan, ctypes.byref(lo)))
    return lo


def vsa_h3_plan_tables(plan: int):
    """Host copies: perm int32 [Nt, tile_tokens], valid int32 [Nt], tile_slot int32 [L]."""
    info = vsa_h3_plan_info(plan)
    perm = np.empty((info.num_tiles, info.tile_tokens), np.int32)
    valid = np.empty(info.num_tiles, np.int32)
    ts = np.empty(info.L, np.int32)
    check(lib().vsa_h3_plan_tables(plan, perm.ctypes.data_as(_I32P), valid.ctypes.data_as(_I32P),
                                   ts.ctypes.data_as(_I32P)))
    return perm, valid, ts


def vsa_h3_plan_upload(plan: int, workspace_ptr: int, workspace_bytes: int, stream: int) -> None:
    check(lib().vsa_h3_plan_upload(plan, workspace_ptr, workspace_bytes, stream))


def vsa_h3_forward(plan: int, q_ptr: int, k_ptr: int, v_ptr: int, gate_ptr: int, io_dtype: int,
                   out_ptr: int, sel_ptr, workspace_ptr: int, workspace_bytes: int,
                   stream: int) -> None:
    check(lib().vsa_h3_forward(plan, q_ptr, k_ptr, v_ptr, gate_ptr, io_dtype, out_ptr, sel_ptr,
                               workspace_ptr, workspace_bytes, stream))


def vsa_h3_forward_timed(plan: int, q_ptr: int, k_ptr: int, v_ptr: int, gate_ptr: int,
                         io_dtype: int, out_ptr: int, sel_ptr, workspace_ptr: int,
                         workspace_bytes: int, stream: int, events) -> None:
    """``events``: 4 hipEvent_t handles (ints) recorded at the stage boundaries."""
    arr = (_P * 4)(*events) if events is not None else None
    check(lib().vsa_h3_forward_timed(plan, q_ptr, k_ptr, v_ptr, gate_ptr, io_dtype, out_ptr,
                                     sel_ptr, workspace_ptr, workspace_bytes, stream, arr))


def vsa_h3_forward_noalloc(plan: int, q_ptr: int, k_ptr: int, v_ptr: int, gate_ptr: int,
                           io_dtype: int, out_ptr: int, sel_ptr, stream: int) -> None:
    """The forward with the library's own device workspace (no allocation)."""
    check(lib().vsa_h3_forward_noalloc(plan, q_ptr, k_ptr, v_ptr, gate_ptr, io_dtype, out_ptr,
                                       sel_ptr, stream))


def vsa_h3_plan_set_qk_prep(plan: int, enable: bool) -> None:
    check(lib().vsa_h3_plan_set_qk_prep(plan, 1 if enable else 0))


def vsa_h3_plan_set_qk_fp8(plan: int, enable: bool) -> None:
    check(lib().vsa_h3_plan_set_qk_fp8(plan, 1 if enable else 0))


def vsa_h3_plan_set_ref_keep(plan: int, keep: float) -> None:
    check(lib().vsa_h3_plan_set_ref_keep(plan, float(keep)))


def vsa_h3_plan_set_io_dtype(plan: int, io_dtype: int) -> None:
    check(lib().vsa_h3_plan_set_io_dtype(plan, int(io_dtype)))


def vsa_h3_forward_qk_prep(plan: int, q_ptr: int, k_ptr: int, v_ptr: int, gate_ptr: int,
                           q_norm_weight_ptr: int, k_norm_weight_ptr: int, eps: float,
                           rope_cos_ptr: int, rope_sin_ptr: int, io_dtype: int, out_ptr: int,
                           sel_ptr, workspace_ptr: int, workspace_bytes: int, stream: int,
                           events=None) -> None:
    arr = (_P * 4)(*events) if events is not None else None
    check(lib().vsa_h3_forward_qk_prep(plan, q_ptr, k_ptr, v_ptr, gate_ptr, q_norm_weight_ptr,
                                       k_norm_weight_ptr, float(eps), rope_cos_ptr, rope_sin_ptr,
                                       io_dtype, out_ptr, sel_ptr, workspace_ptr,
                                       workspace_bytes, stream, arr))


def vsa_h3_oneshot_workspace_bytes(token_tags, position_ids, grid, tile, heads, head_dim,
                                   sparsity, io_dtype: int = VSA_BF16) -> int:
    tags = _i64(token_tags).reshape(-1)
    pos = _i64(position_ids).reshape(-1, 3)
    n = ctypes.c_uint64()
    check(lib().vsa_h3_oneshot_workspace_bytes(_ptr64(tags), _ptr64(pos), tags.shape[0],
                                               Dims3(*grid), Dims3(*tile), int(heads),
                                               int(head_dim), float(sparsity), int(io_dtype),
                                               ctypes.byref(n)))
    return n.value


def vsa_h3_forward_oneshot(q_ptr, k_ptr, v_ptr, gate_ptr, token_tags, position_ids, heads,
                           head_dim, grid, sparsity, tile, io_dtype, out_ptr, sel_ptr,
                           workspace_ptr, workspace_bytes, stream) -> None:
    tags = _i64(token_tags).reshape(-1)
    pos = _i64(position_ids).reshape(-1, 3)
    check(lib().vsa_h3_forward_oneshot(q_ptr, k_ptr, v_ptr, gate_ptr, _ptr64(tags), _ptr64(pos),
                                       tags.shape[0], int(heads), int(head_dim), Dims3(*grid),
                                       float(sparsity), Dims3(*tile), io_dtype, out_ptr, sel_ptr,
                                       workspace_ptr, workspace_bytes, stream))


def vsa_h3_plan_destroy(plan: int) -> None:
    if plan:
        lib().vsa_h3_plan_destroy(plan)


def vsa_h3_last_error() -> str:
    return lib().vsa_h3_last_error().decode()


def vsa_h3_version() -> str:
    return lib().vsa_h3_version().decode()

"""VSA-H3 attention forward on AMD Instinct MI355X (gfx950).

Video Sparse Attention as used by the FastH3 / MiniMax-H3 video DiT: packed
[text | cond | audio | video] tokens are cut into 64-token tiles, a coarse
branch scores mean-pooled tiles and produces a gated compression output, each
video query tile keeps its top-k video key tiles (plus every prefix tile), and
a block-sparse flash attention computes the fine branch.  The OmniRef variant
(128-token tiles, a reference keep ratio for the cond tiles) is a plan option.
All of it runs in hand-written HIP kernels behind the C ABI of
``include/vsa_h3.h``; this module only marshals arguments (PyTorch provides
device memory and the stream).

    import video_dit_block_amd as vsa
    out = vsa.forward(q, k, v, gate, token_tags, position_ids, grid=(T, H, W),
                      sparsity=0.8)
"""
from __future__ import annotations

import contextlib
import hashlib
import os
import threading
from collections import OrderedDict

import numpy as np

from ._abi import (  # noqa: F401  (re-exported: same names as the C ABI)
    EXPORTED, LIB_PATH, VSA_BF16, VSA_F32, VSA_TAG_AUDIO, VSA_TAG_COND, VSA_TAG_TEXT,
    VSA_TAG_VIDEO, VsaError, lib, vsa_h3_forward, vsa_h3_forward_oneshot, vsa_h3_forward_timed,
    vsa_h3_last_error,
    vsa_h3_oneshot_workspace_bytes, vsa_h3_plan_create, vsa_h3_plan_destroy, vsa_h3_plan_info,
    vsa_h3_plan_layout, vsa_h3_plan_set_chunk_tiles, vsa_h3_plan_tables, vsa_h3_plan_upload,
    vsa_h3_topk, vsa_h3_version, vsa_h3_plan_set_qk_prep, vsa_h3_forward_qk_prep,
    vsa_h3_plan_set_qk_fp8, vsa_h3_plan_set_ref_keep, vsa_h3_plan_set_io_dtype,
    vsa_h3_forward_noalloc,
)

__all__ = ["Plan", "forward", "forward_qk_prep", "VsaError", "vsa_h3_topk",
           "vsa_h3_version", "io_dtype_code", "get_plan", "plan_cache_bytes",
           "set_plan_cache_bytes"] + list(EXPORTED)


def io_dtype_code(dtype) -> int:
    """VSA_BF16 or VSA_F32 for a torch dtype, "bf16" / "f32", or the code itself."""
    if isinstance(dtype, int):
        if dtype not in (VSA_BF16, VSA_F32):
            raise VsaError(-1, f"unknown io dtype code {dtype}")
        return dtype
    name = str(dtype).replace("torch.", "")
    if name in ("bf16", "bfloat16"):
        return VSA_BF16
    if name in ("f32", "fp32", "float32", "float"):
        return VSA_F32
    raise VsaError(-1, f"unsupported io dtype {dtype}")


def _host_i64(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu").numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.int64))


class Plan:
    """Tile geometry for one packed layout (host), plus per-device workspaces."""

    def __init__(self, token_tags, position_ids, grid, heads, head_dim, sparsity,
                 tile=(4, 4, 4), chunk_tiles: int = 0, qk_prep: bool = False,
                 qk_fp8: bool = False, ref_keep: float = 1.0, io_dtype="bf16"):
        self.token_tags = _host_i64(token_tags).reshape(-1)
        self.position_ids = _host_i64(position_ids).reshape(-1, 3)
        self.grid = tuple(int(g) for g in grid)
        self.tile = tuple(int(t) for t in tile)
        self.sparsity = float(sparsity)
        self.handle = vsa_h3_plan_create(self.token_tags, self.position_ids, self.grid,
                                         self.tile, heads, head_dim, sparsity)
        if chunk_tiles:
            vsa_h3_plan_set_chunk_tiles(self.handle, chunk_tiles)
        if qk_prep:
            vsa_h3_plan_set_qk_prep(self.handle, True)
        self.qk_prep = bool(qk_prep)
        if qk_fp8:
            vsa_h3_plan_set_qk_fp8(self.handle, True)
        self.qk_fp8 = bool(qk_fp8)
        if ref_keep != 1.0:
            vsa_h3_plan_set_ref_keep(self.handle, ref_keep)
        self.ref_keep = float(ref_keep)
        # fp32 I/O needs the low-part regions of the workspace.
        self.io_dtype = io_dtype_code(io_dtype)
        if self.io_dtype == VSA_F32:
            vsa_h3_plan_set_io_dtype(self.handle, VSA_F32)
        self.info = vsa_h3_plan_info(self.handle)
        self.layout = vsa_h3_plan_layout(self.handle)
        self._ws = {}
        self._ws_lock = threading.Lock()

    # geometry
    @property
    def L(self): return self.info.L
    @property
    def heads(self): return self.info.heads
    @property
    def head_dim(self): return self.info.head_dim
    @property
    def num_prefix_tiles(self): return self.info.num_prefix_tiles
    @property
    def num_video_tiles(self): return self.info.num_video_tiles
    @property
    def num_tiles(self): return self.info.num_tiles
    @property
    def topk(self): return self.info.topk
    @property
    def topk_ref(self): return self.info.topk_ref
    @property
    def num_ref_tiles(self): return self.info.num_ref_tiles
    @property
    def sel_width(self): return self.info.topk_ref + self.info.topk
    @property
    def tile_tokens(self): return self.info.tile_tokens
    @property
    def num_blocks(self): return self.info.num_blocks
    @property
    def workspace_bytes(self): return self.info.workspace_bytes
    @property
    def chunk_tiles(self): return self.info.chunk_tiles
    @property
    def num_chunks(self): return self.info.num_chunks

    def tables(self):
        """(perm [Nt, tile_tokens], valid [Nt], tile_slot [L]) as host int32 arrays."""
        return vsa_h3_plan_tables(self.handle)

    def workspace(self, device, stream=None):
        """The plan's workspace for work on ``stream`` (a raw stream handle;
        default: the device's current stream) of ``device``: a torch uint8
        tensor, created and filled with the plan's tables on first use.

        Every (device, stream) pair has its own workspace, so forwards that
        share this plan on different streams never share scratch memory.  It
        is allocated with that stream current, so once the plan lets go of it
        (``release_workspaces``, or the plan cache evicting the plan) the
        caching allocator hands the memory out again only in that stream's
        order, after the forwards already queued there."""
        import torch
        device = torch.device(device)
        dev = device.index if device.index is not None else torch.cuda.current_device()
        cur = torch.cuda.current_stream(dev)
        s = cur.cuda_stream if stream is None else int(stream)
        key = (dev, s)
        with self._ws_lock:
            ws = self._ws.get(key)
            if ws is None:
                cuda = torch.device("cuda", dev)
                ctx = (contextlib.nullcontext() if s == cur.cuda_stream else
                       torch.cuda.stream(torch.cuda.ExternalStream(s, device=cuda)))
                with ctx:
                    ws = torch.empty(self.workspace_bytes, dtype=torch.uint8, device=cuda)
                vsa_h3_plan_upload(self.handle, ws.data_ptr(), self.workspace_bytes, s)
                self._ws[key] = ws
            return ws

    def resident_bytes(self) -> int:
        """Device bytes held by this plan's workspaces."""
        with self._ws_lock:
            return sum(int(w.numel()) for w in self._ws.values())

    def release_workspaces(self) -> None:
        """Drop every workspace (each is freed in its own stream's order)."""
        with self._ws_lock:
            self._ws.clear()

    def view(self, ws, name: str, dtype, shape):
        """A typed view of one workspace region (for tests and tools)."""
        import torch
        off = getattr(self.layout, name)
        n = int(np.prod(shape))
        itemsize = torch.empty((), dtype=dtype).element_size()
        return ws[off:off + n * itemsize].view(dtype).view(*shape)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h:
            try:
                vsa_h3_plan_destroy(h)
            except Exception:  # pragma: no cover
                pass
            self.handle = None


_plans: "OrderedDict[tuple, Plan]" = OrderedDict()
_plans_lock = threading.Lock()
_PLAN_CACHE_MAX_PLANS = 8
_plan_cache_bytes = int(os.environ.get("VSA_H3_PLAN_CACHE_BYTES", 16 << 30))


def plan_cache_bytes() -> int:
    """Most device bytes the workspaces of cached plans may hold between calls."""
    return _plan_cache_bytes


def set_plan_cache_bytes(n: int) -> None:
    """Set the byte budget of the plan cache (default 16 GiB, or the
    VSA_H3_PLAN_CACHE_BYTES environment variable) and trim the cache to it."""
    global _plan_cache_bytes
    if int(n) < 0:
        raise VsaError(-1, "the plan cache budget must be >= 0 bytes")
    _plan_cache_bytes = int(n)
    _trim_plan_cache()


def _trim_plan_cache() -> None:
    """Evict least recently used plans until the cache holds at most
    _PLAN_CACHE_MAX_PLANS plans whose workspaces total at most the byte
    budget.  A plan is evicted whole: the cache drops its reference, and its
    workspaces are freed once no caller holds the plan either."""
    with _plans_lock:
        sizes = {key: p.resident_bytes() for key, p in _plans.items()}
        total = sum(sizes.values())
        for key in list(_plans):
            if total <= _plan_cache_bytes and len(_plans) <= _PLAN_CACHE_MAX_PLANS:
                break
            total -= sizes[key]
            del _plans[key]


def get_plan(token_tags, position_ids, grid, heads, head_dim, sparsity, tile=(4, 4, 4),
             qk_prep: bool = False, ref_keep: float = 1.0, io_dtype="bf16") -> Plan:
    """Cached Plan for this exact layout (keyed by a digest of tags and
    positions).  The cache keeps at most 8 plans, and between calls their
    workspaces hold at most ``plan_cache_bytes()`` of device memory: the
    forward calls trim it once their work is queued."""
    tags = _host_i64(token_tags).reshape(-1)
    pos = _host_i64(position_ids).reshape(-1, 3)
    digest = hashlib.sha256(tags.tobytes() + b"|" + pos.tobytes()).hexdigest()
    io = io_dtype_code(io_dtype)
    key = (digest, tuple(grid), tuple(tile), int(heads), int(head_dim), float(sparsity),
           bool(qk_prep), float(ref_keep), io)
    with _plans_lock:
        p = _plans.get(key)
        if p is not None:
            _plans.move_to_end(key)
            return p
    p = Plan(tags, pos, grid, heads, head_dim, sparsity, tile, qk_prep=qk_prep,
             ref_keep=ref_keep, io_dtype=io)
    with _plans_lock:
        p = _plans.setdefault(key, p)
        _plans.move_to_end(key)
    _trim_plan_cache()
    return p


def forward(q, k, v, gate, token_tags=None, position_ids=None, grid=None, sparsity=None,
            tile=(4, 4, 4), *, ref_keep: float = 1.0, plan: Plan | None = None, out=None,
            return_sel: bool = False):
    """VSA-H3 forward.  q, k, v, gate: CUDA tensors [L, heads, head_dim], contiguous,
    all bfloat16 or all float32.  ``tile`` is the video tile box (64 or 128 grid
    cells) and ``ref_keep`` the reference keep ratio (1 visits every reference
    tile).  Returns out (same shape and dtype), and the selected key tiles
    int32 [heads, NV, topk_ref + topk] if ``return_sel``."""
    import torch
    if not (q.is_cuda and k.is_cuda and v.is_cuda and gate.is_cuda):
        raise VsaError(-1, "q, k, v and gate must be GPU tensors (there is no CPU path)")
    if not (q.shape == k.shape == v.shape == gate.shape) or q.dim() != 3:
        raise VsaError(-1, "q, k, v and gate must share one [L, heads, head_dim] shape")
    if not (q.dtype == k.dtype == v.dtype == gate.dtype):
        raise VsaError(-1, "q, k, v and gate must share one dtype")
    if q.dtype == torch.bfloat16:
        io = VSA_BF16
    elif q.dtype == torch.float32:
        io = VSA_F32
    else:
        raise VsaError(-1, f"unsupported dtype {q.dtype}")
    for t in (q, k, v, gate):
        if not t.is_contiguous():
            raise VsaError(-1, "tensors must be contiguous")
    L, H, D = q.shape
    if plan is None:
        plan = get_plan(token_tags, position_ids, grid, H, D, sparsity, tile, ref_keep=ref_keep,
                        io_dtype=io)
    if (plan.L, plan.heads, plan.head_dim) != (L, H, D):
        raise VsaError(-1, "plan does not match the tensors' [L, heads, head_dim]")
    if io == VSA_F32 and plan.io_dtype != VSA_F32:
        raise VsaError(-1, "float32 tensors need a plan built with io_dtype='f32'")
    dev = q.device
    stream = torch.cuda.current_stream(dev).cuda_stream
    ws = plan.workspace(dev, stream)
    if out is None:
        out = torch.empty_like(q)
    sel = None
    if return_sel:
        sel = torch.empty((H, plan.num_video_tiles, plan.sel_width), dtype=torch.int32,
                          device=dev)
    vsa_h3_forward(plan.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), gate.data_ptr(), io,
                   out.data_ptr(), sel.data_ptr() if sel is not None and sel.numel() else None,
                   ws.data_ptr(), plan.workspace_bytes, stream)
    _trim_plan_cache()
    return (out, sel) if return_sel else out


def forward_qk_prep(q, k, v, gate, q_norm_weight, k_norm_weight, eps, rope_cos, rope_sin,
                    token_tags=None, position_ids=None, grid=None, sparsity=None,
                    tile=(4, 4, 4), *, ref_keep: float = 1.0, plan: Plan | None = None,
                    out=None, return_sel: bool = False):
    """VSA-H3 forward with QK RMS norm and RoPE applied to q and k while they
    are gathered into tile order.  q, k, v, gate as for ``forward`` (q and k
    before the norm); q_norm_weight, k_norm_weight: float32 CUDA [head_dim];
    rope_cos, rope_sin: float32 CUDA [L, head_dim // 2] in packed order."""
    import torch
    if not (q.is_cuda and k.is_cuda and v.is_cuda and gate.is_cuda):
        raise VsaError(-1, "q, k, v and gate must be GPU tensors (there is no CPU path)")
    if not (q.shape == k.shape == v.shape == gate.shape) or q.dim() != 3:
        raise VsaError(-1, "q, k, v and gate must share one [L, heads, head_dim] shape")
    if not (q.dtype == k.dtype == v.dtype == gate.dtype):
        raise VsaError(-1, "q, k, v and gate must share one dtype")
    io = VSA_BF16 if q.dtype == torch.bfloat16 else (VSA_F32 if q.dtype == torch.float32 else None)
    if io is None:
        raise VsaError(-1, f"unsupported dtype {q.dtype}")
    L, H, D = q.shape
    for name, t, shape in (("q_norm_weight", q_norm_weight, (D,)),
                           ("k_norm_weight", k_norm_weight, (D,)),
                           ("rope_cos", rope_cos, (L, D // 2)), ("rope_sin", rope_sin, (L, D // 2))):
        if not (t.is_cuda and t.dtype == torch.float32 and t.is_contiguous()
                and tuple(t.shape) == shape):
            raise VsaError(-1, f"{name} must be a contiguous float32 GPU tensor of shape {shape}")
    for t in (q, k, v, gate):
        if not t.is_contiguous():
            raise VsaError(-1, "tensors must be contiguous")
    if plan is None:
        plan = get_plan(token_tags, position_ids, grid, H, D, sparsity, tile, qk_prep=True,
                        ref_keep=ref_keep, io_dtype=io)
    if not plan.qk_prep:
        raise VsaError(-1, "plan was built without qk_prep=True")
    if io == VSA_F32 and plan.io_dtype != VSA_F32:
        raise VsaError(-1, "float32 tensors need a plan built with io_dtype='f32'")
    if (plan.L, plan.heads, plan.head_dim) != (L, H, D):
        raise VsaError(-1, "plan does not match the tensors' [L, heads, head_dim]")
    dev = q.device
    stream = torch.cuda.current_stream(dev).cuda_stream
    ws = plan.workspace(dev, stream)
    if out is None:
        out = torch.empty_like(q)
    sel = None
    if return_sel:
        sel = torch.empty((H, plan.num_video_tiles, plan.sel_width), dtype=torch.int32,
                          device=dev)
    vsa_h3_forward_qk_prep(plan.handle, q.data_ptr(), k.data_ptr(), v.data_ptr(),
                           gate.data_ptr(), q_norm_weight.data_ptr(), k_norm_weight.data_ptr(),
                           float(eps), rope_cos.data_ptr(), rope_sin.data_ptr(), io,
                           out.data_ptr(),
                           sel.data_ptr() if sel is not None and sel.numel() else None,
                           ws.data_ptr(), plan.workspace_bytes, stream)
    _trim_plan_cache()
    return (out, sel) if return_sel else out

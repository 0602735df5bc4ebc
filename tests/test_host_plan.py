"""Host-side tests of the C ABI (no GPU needed): the library loads and exports
every function include/vsa_h3.h declares, plan geometry matches the oracle's
independent geometry, error codes, and workspace layout."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import video_dit_block_amd as vsa
from video_dit_block_amd import _abi
from workloads import AUDIO, COND, TEXT, WORKLOADS, Workload, make_layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vsa_h3.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(vsa_h3_\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = _abi.lib()
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_abi.EXPORTED)
    assert vsa.vsa_h3_version().startswith("vsa_h3")


def test_topk_matches_golden_and_oracle():
    path = os.path.join(ROOT, "tests", "golden", "topk_cases.txt")
    for line in open(path):
        if line.strip() and not line.startswith("#"):
            n, s, k = line.split()[:3]
            assert vsa.vsa_h3_topk(int(n), float(s)) == int(k)
    for n in (1, 3, 8, 216, 1260, 1764):
        for s in np.linspace(0, 1, 41):
            assert vsa.vsa_h3_topk(n, float(s)) == oracle.topk_count(n, float(s))
    assert vsa.vsa_h3_topk(0, 0.5) == 0
    assert vsa.vsa_h3_topk(10, 1.5) == -1
    assert vsa.vsa_h3_topk(10, float("nan")) == -1


LAYOUTS = [
    ("tiny", WORKLOADS["tiny"], "raster"),
    ("odd", Workload("odd", 3, 64, "f32", ((TEXT, 70), (COND, 20), (AUDIO, 33)), (5, 6, 7), 0.5), "shuffled"),
    ("odd2", Workload("odd2", 2, 128, "bf16", ((AUDIO, 1),), (9, 2, 13), 0.3), "shuffled"),
    ("video_only", Workload("vo", 2, 64, "f32", (), (4, 8, 8), 0.5), "raster"),
    ("prefix_only", Workload("po", 2, 64, "f32", ((TEXT, 100),), (0, 0, 0), 0.5), "raster"),
    ("480p5s", WORKLOADS["480p5s"], "raster"),
    ("768p10s", WORKLOADS["768p10s"], "raster"),
]


@pytest.mark.parametrize("name,w,order", LAYOUTS, ids=[l[0] for l in LAYOUTS])
def test_plan_geometry_matches_oracle(name, w, order):
    tags, pos = make_layout(w, order, seed=11)
    p = vsa.Plan(tags, pos, w.grid, w.heads, w.head_dim, w.sparsity)
    g = oracle.geometry(tags.numpy(), pos.numpy(), w.grid)
    assert (p.num_prefix_tiles, p.num_video_tiles, p.num_tiles) == (g.P, g.NV, g.Nt)
    assert p.topk == oracle.topk_count(g.NV, w.sparsity)
    perm, valid, tile_slot = p.tables()
    assert np.array_equal(valid, g.valid)
    assert np.array_equal(perm, g.perm())
    expect_ts = g.tile_of_token() * 64 + g.slot_of_token()
    assert np.array_equal(tile_slot, expect_ts)


def test_plan_sizes_768p10s_and_768p15s():
    for name, P, NV, topk, n32 in (("768p10s", 16, 1260, 252, 252), ("768p15s_smooth", 48, 1764, 177, 0)):
        w = WORKLOADS[name]
        tags, pos = make_layout(w)
        p = vsa.Plan(tags, pos, w.grid, w.heads, w.head_dim, w.sparsity)
        assert (p.num_prefix_tiles, p.num_video_tiles, p.topk) == (P, NV, topk)
        _, valid, _ = p.tables()
        if name == "768p10s":
            assert (valid[P:] == 32).sum() == 252 and (valid[P:] == 64).sum() == 1008
        else:
            assert (valid[P:] == 48).sum() == 252 and (valid[P:] == 64).sum() == 1512


def test_workspace_layout_aligned_disjoint_and_64bit():
    w = WORKLOADS["768p15s_smooth"]
    tags, pos = make_layout(w)
    p = vsa.Plan(tags, pos, w.grid, w.heads, w.head_dim, w.sparsity)
    lo = p.layout
    H, D, Nt, NV, k = w.heads, w.head_dim, p.num_tiles, p.num_video_tiles, p.topk
    ns = (Nt + 3) // 4 * 4
    regions = [("perm", Nt * 64 * 4), ("valid", Nt * 4), ("kt", H * Nt * 64 * D * 2),
               ("vt", H * Nt * 64 * D * 2), ("qp", H * Nt * D * 4), ("kp", H * Nt * D * 4),
               ("vp", H * Nt * D * 4), ("scores", H * Nt * ns * 4), ("coarse", H * Nt * D * 4),
               ("sel", H * NV * k * 4), ("chunk_offsets", H * NV * (p.num_chunks + 1) * 4),
               ("state", H * Nt * 2 * 64 * (D // 2 + 4) * 4)]
    assert p.num_chunks > 1
    spans = []
    for n, size in regions:
        off = getattr(lo, n)
        assert off % 256 == 0
        spans.append((off, off + size))
    spans.sort()
    for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
        assert a1 <= b0
    assert spans[-1][1] <= lo.total == p.workspace_bytes
    assert lo.scores_row_stride == ns
    assert lo.total > 2 ** 32          # 64-bit offsets are needed at this size


@pytest.mark.parametrize("name,chunk_tiles,num_chunks", [
    ("768p10s", 319, 4),          # 1,276 tiles, head_dim 128: at most 320 tiles (10 MiB) per chunk
    ("768p15s_smooth", 302, 6),   # 1,812 tiles
    ("480p5s", 236, 1),           # 236 tiles: one chunk
    ("tiny", 9, 1),               # 9 tiles, head_dim 64: one chunk
])
def test_default_key_chunks(name, chunk_tiles, num_chunks):
    w = WORKLOADS[name]
    tags, pos = make_layout(w)
    p = vsa.Plan(tags, pos, w.grid, w.heads, w.head_dim, w.sparsity)
    assert (p.chunk_tiles, p.num_chunks) == (chunk_tiles, num_chunks)
    assert p.chunk_tiles * 2 * 64 * w.head_dim * 2 <= 10 << 20
    assert (p.num_chunks - 1) * p.chunk_tiles < p.num_tiles <= p.num_chunks * p.chunk_tiles
    if num_chunks == 1:
        # a single launch needs neither the chunk offsets nor the running state
        assert p.layout.total <= p.layout.state + 256


def test_set_chunk_tiles_resizes_the_workspace_and_checks_its_argument():
    w = Workload("c", 2, 128, "bf16", ((TEXT, 130),), (8, 12, 16), 0.5)   # 3 + 24 tiles
    tags, pos = make_layout(w)
    p = vsa.Plan(tags, pos, w.grid, w.heads, w.head_dim, w.sparsity)
    assert p.num_chunks == 1
    base = p.workspace_bytes
    for ch, nc in ((1, 27), (2, 14), (26, 2), (27, 1), (1000, 1)):
        vsa.vsa_h3_plan_set_chunk_tiles(p.handle, ch)
        info = vsa.vsa_h3_plan_info(p.handle)
        assert (info.chunk_tiles, info.num_chunks) == (min(ch, 27), nc)
        lo = vsa.vsa_h3_plan_layout(p.handle)
        if nc > 1:
            state_bytes = 2 * 27 * 2 * 64 * (128 // 2 + 4) * 4
            assert info.workspace_bytes >= base + state_bytes
            assert lo.state + state_bytes <= lo.total
        else:
            assert info.workspace_bytes == base
    with pytest.raises(vsa.VsaError):
        vsa.vsa_h3_plan_set_chunk_tiles(p.handle, -1)
    big = WORKLOADS["768p10s"]
    tags, pos = make_layout(big)
    p2 = vsa.Plan(tags, pos, big.grid, big.heads, big.head_dim, big.sparsity)
    with pytest.raises(vsa.VsaError):     # 1,276 chunks > 63
        vsa.vsa_h3_plan_set_chunk_tiles(p2.handle, 1)
    assert _abi.lib().vsa_h3_plan_set_chunk_tiles(None, 4) == _abi.VSA_E_ARG


def _raw_create(tags, pos, grid, tile=(4, 4, 4), heads=2, D=64, s=0.5):
    return _abi.lib().vsa_h3_plan_create(
        np.ascontiguousarray(tags, np.int64).ctypes.data_as(_abi._I64P),
        np.ascontiguousarray(pos, np.int64).ctypes.data_as(_abi._I64P),
        len(tags), _abi.Dims3(*grid), _abi.Dims3(*tile), heads, D, s, ctypes.byref(ctypes.c_void_p()))


@pytest.mark.parametrize("case,status", [
    ("ok", 0), ("video_first", -2), ("badtag", -2), ("dup", -3), ("outside", -3),
    ("count", -3), ("sparsity", -1), ("sparsity_nan", -1), ("heads", -1), ("head_dim", -4),
    ("tile", -4), ("neg_grid", -1)])
def test_plan_error_codes(case, status):
    w = Workload("e", 2, 64, "f32", ((TEXT, 10),), (4, 4, 4), 0.5)
    tags, pos = make_layout(w)
    tags, pos = tags.numpy().copy(), pos.numpy().copy()
    kw = {}
    grid = w.grid
    if case == "video_first":
        tags[[0, 20]] = tags[[20, 0]]
    elif case == "badtag":
        tags[2] = 7
    elif case == "dup":
        pos[20] = pos[21]
    elif case == "outside":
        pos[20, 1] = -1
    elif case == "count":
        grid = (4, 4, 5)
    elif case == "sparsity":
        kw["s"] = 1.5
    elif case == "sparsity_nan":
        kw["s"] = float("nan")
    elif case == "heads":
        kw["heads"] = 0
    elif case == "head_dim":
        kw["D"] = 96
    elif case == "tile":
        kw["tile"] = (2, 2, 2)
    elif case == "neg_grid":
        grid = (-1, 4, 4)
    st = _raw_create(tags, pos, grid, **kw)
    assert st == status, _abi.vsa_h3_last_error()
    if status:
        assert _abi.vsa_h3_last_error()
        with pytest.raises(vsa.VsaError):
            vsa.Plan(tags, pos, grid, kw.get("heads", 2), kw.get("D", 64), kw.get("s", 0.5),
                     kw.get("tile", (4, 4, 4)))


def test_forward_argument_errors_before_any_device_work():
    w = WORKLOADS["tiny"]
    tags, pos = make_layout(w)
    p = vsa.Plan(tags, pos, w.grid, w.heads, w.head_dim, w.sparsity)
    L = _abi.lib()
    fake = 1 << 40  # never dereferenced: every call below fails its checks first
    assert L.vsa_h3_forward(p.handle, fake, fake, fake, fake, 0, fake + (1 << 30), None,
                            None, 0, None) == _abi.VSA_E_WORKSPACE
    assert L.vsa_h3_forward(p.handle, fake, fake, fake, fake, 0, fake + (1 << 30), None,
                            fake + 8, p.workspace_bytes, None) == _abi.VSA_E_WORKSPACE
    assert L.vsa_h3_forward(p.handle, fake, fake, fake, fake, 0, fake + (1 << 30), None,
                            fake, p.workspace_bytes - 1, None) == _abi.VSA_E_WORKSPACE
    assert L.vsa_h3_forward(p.handle, fake, fake, fake, fake, 7, fake + (1 << 30), None,
                            fake, p.workspace_bytes, None) == _abi.VSA_E_ARG
    assert L.vsa_h3_forward(p.handle, None, fake, fake, fake, 0, fake + (1 << 30), None,
                            fake, p.workspace_bytes, None) == _abi.VSA_E_ARG
    # out aliasing an input
    assert L.vsa_h3_forward(p.handle, fake, fake, fake, fake, 0, fake + 64, None,
                            fake, p.workspace_bytes, None) == _abi.VSA_E_ARG
    assert L.vsa_h3_forward(None, fake, fake, fake, fake, 0, fake, None, fake, 1,
                            None) == _abi.VSA_E_ARG


def test_oneshot_workspace_bytes_matches_plan():
    w = WORKLOADS["480p5s"]
    tags, pos = make_layout(w)
    p = vsa.Plan(tags, pos, w.grid, w.heads, w.head_dim, w.sparsity)
    n = vsa.vsa_h3_oneshot_workspace_bytes(tags.numpy(), pos.numpy(), w.grid, (4, 4, 4), w.heads,
                                           w.head_dim, w.sparsity)
    assert n == p.workspace_bytes


def test_empty_sequence_plan():
    p = vsa.Plan(np.zeros(0, np.int64), np.zeros((0, 3), np.int64), (0, 0, 0), 2, 64, 0.5)
    assert (p.L, p.num_tiles, p.topk) == (0, 0, 0)


def test_python_forward_refuses_cpu_tensors():
    import torch
    w = WORKLOADS["tiny"]
    tags, pos = make_layout(w)
    x = torch.zeros((w.L, w.heads, w.head_dim))
    with pytest.raises(vsa.VsaError):
        vsa.forward(x, x, x, x, tags, pos, w.grid, w.sparsity)


def test_more_than_4096_tiles_per_head_is_rejected():
    ok = Workload("ok", 1, 64, "f32", (), (64, 64, 64), 0.5)          # 4,096 tiles
    tags, pos = make_layout(ok)
    assert vsa.Plan(tags, pos, ok.grid, 1, 64, 0.5).num_tiles == 4096
    big = Workload("big", 1, 64, "f32", ((TEXT, 1),), (64, 64, 64), 0.5)   # 4,097 tiles
    tags, pos = make_layout(big)
    assert _raw_create(tags.numpy(), pos.numpy(), big.grid, heads=1, D=64) == _abi.VSA_E_UNSUPPORTED


def test_qk_prep_plan_region_and_argument_errors():
    w = WORKLOADS["tiny"]
    tags, pos = make_layout(w)
    p = vsa.Plan(tags, pos, w.grid, w.heads, w.head_dim, w.sparsity)
    base = p.workspace_bytes
    L = _abi.lib()
    fake = 1 << 40   # never dereferenced: every call below fails its checks first
    args = [fake, fake + (1 << 30), fake + (2 << 30), fake + (3 << 30)]
    tabs = [fake + (4 << 30), fake + (5 << 30), fake + (6 << 30), fake + (7 << 30)]
    # no QK-prep region in the plan
    assert L.vsa_h3_forward_qk_prep(p.handle, *args, tabs[0], tabs[1], 1e-6, tabs[2], tabs[3], 0,
                                    fake + (8 << 30), None, fake + (9 << 30), base, None,
                                    None) == _abi.VSA_E_ARG
    p2 = vsa.Plan(tags, pos, w.grid, w.heads, w.head_dim, w.sparsity, qk_prep=True)
    Nt, D, H = p2.num_tiles, w.head_dim, w.heads
    assert p2.workspace_bytes >= base + H * Nt * 64 * D * 2
    lo = p2.layout
    assert lo.qt % 256 == 0 and lo.qt + H * Nt * 64 * D * 2 <= lo.total
    ws = fake + (9 << 30)
    n = p2.workspace_bytes
    assert L.vsa_h3_forward_qk_prep(p2.handle, *args, None, tabs[1], 1e-6, tabs[2], tabs[3], 0,
                                    fake + (8 << 30), None, ws, n, None, None) == _abi.VSA_E_ARG
    assert L.vsa_h3_forward_qk_prep(p2.handle, *args, tabs[0], tabs[1], -1.0, tabs[2], tabs[3], 0,
                                    fake + (8 << 30), None, ws, n, None, None) == _abi.VSA_E_ARG
    assert L.vsa_h3_forward_qk_prep(p2.handle, *args, tabs[0], tabs[1], float("nan"), tabs[2],
                                    tabs[3], 0, fake + (8 << 30), None, ws, n, None,
                                    None) == _abi.VSA_E_ARG
    assert L.vsa_h3_forward_qk_prep(p2.handle, *args, tabs[0] + 2, tabs[1], 1e-6, tabs[2],
                                    tabs[3], 0, fake + (8 << 30), None, ws, n, None,
                                    None) == _abi.VSA_E_ARG
    assert L.vsa_h3_forward_qk_prep(p2.handle, *args, tabs[0], tabs[1], 1e-6, tabs[2], tabs[3], 0,
                                    fake + (8 << 30), None, ws, n - 1, None,
                                    None) == _abi.VSA_E_WORKSPACE
    vsa.vsa_h3_plan_set_qk_prep(p2.handle, False)
    assert vsa.vsa_h3_plan_info(p2.handle).workspace_bytes == base


def test_default_key_chunks_follow_the_key_format():
    # FP8 keys are one byte per element: a 10 MiB chunk holds 64*128*(1+2) = 24 KB tiles
    w = WORKLOADS["768p10s"]
    tags, pos = make_layout(w)
    p = vsa.Plan(tags, pos, w.grid, w.heads, w.head_dim, w.sparsity, qk_fp8=True)
    assert (p.chunk_tiles, p.num_chunks) == (426, 3)
    assert p.chunk_tiles * 64 * w.head_dim * 3 <= 10 << 20
    lo = p.layout
    assert lo.kt8 % 256 == 0 and lo.kscale % 256 == 0
    assert lo.kscale + w.heads * p.num_tiles * 64 * 4 <= lo.total
    # an explicit chunk length is kept when the key format changes
    p2 = vsa.Plan(tags, pos, w.grid, w.heads, w.head_dim, w.sparsity, chunk_tiles=200, qk_fp8=True)
    assert (p2.chunk_tiles, p2.num_chunks) == (200, 7)
    vsa.vsa_h3_plan_set_qk_fp8(p.handle, False)
    info = vsa.vsa_h3_plan_info(p.handle)
    assert (info.chunk_tiles, info.num_chunks) == (319, 4)


def test_fp32_io_plan_regions_and_errors():
    """A plan laid out for fp32 I/O holds the low bf16 parts of the tile-ordered
    keys and values (and of Qt with QK-norm + RoPE; no key low parts with FP8
    keys); an fp32 forward on a bf16 plan is refused before any device work."""
    w = WORKLOADS["tiny"]
    tags, pos = make_layout(w)
    p = vsa.Plan(tags, pos, w.grid, w.heads, w.head_dim, w.sparsity)
    base = p.workspace_bytes
    H, Nb, D = w.heads, p.num_blocks, w.head_dim
    tok = H * Nb * 64 * D * 2
    L = _abi.lib()
    fake = 1 << 40   # never dereferenced: the call fails its checks first
    ins = [fake, fake + (1 << 30), fake + (2 << 30), fake + (3 << 30)]
    assert L.vsa_h3_forward(p.handle, *ins, _abi.VSA_F32, fake + (4 << 30), None,
                            fake + (5 << 30), base, None) == _abi.VSA_E_ARG
    assert "vsa_h3_plan_set_io_dtype" in vsa.vsa_h3_last_error()
    f = vsa.Plan(tags, pos, w.grid, w.heads, w.head_dim, w.sparsity, io_dtype="f32")
    lo = f.layout
    assert f.workspace_bytes >= base + 2 * tok
    for off in (lo.kt_lo, lo.vt_lo):
        assert off % 256 == 0 and off + tok <= lo.total
    assert p.layout.kt_lo == p.layout.vt_lo == p.layout.qt_lo  # empty regions in a bf16 plan
    fp = vsa.Plan(tags, pos, w.grid, w.heads, w.head_dim, w.sparsity, qk_prep=True,
                  io_dtype="f32")
    assert fp.layout.qt_lo % 256 == 0 and fp.layout.qt_lo + tok <= fp.layout.total
    f8 = vsa.Plan(tags, pos, w.grid, w.heads, w.head_dim, w.sparsity, qk_fp8=True,
                  io_dtype="f32")
    assert f8.layout.vt_lo + tok <= f8.layout.total
    assert f8.workspace_bytes < f8.layout.vt_lo + 2 * tok   # no key low parts with FP8 keys
    # back to bf16: the low-part regions go
    vsa.vsa_h3_plan_set_io_dtype(f.handle, vsa.VSA_BF16)
    assert vsa.vsa_h3_plan_info(f.handle).workspace_bytes == base
    assert L.vsa_h3_plan_set_io_dtype(f.handle, 7) == _abi.VSA_E_ARG
    # the one-call form sizes its workspace by the I/O dtype
    n16 = vsa.vsa_h3_oneshot_workspace_bytes(tags.numpy(), pos.numpy(), w.grid, (4, 4, 4), H, D,
                                             w.sparsity, vsa.VSA_BF16)
    n32 = vsa.vsa_h3_oneshot_workspace_bytes(tags.numpy(), pos.numpy(), w.grid, (4, 4, 4), H, D,
                                             w.sparsity, vsa.VSA_F32)
    assert (n16, n32) == (base, vsa.Plan(tags, pos, w.grid, H, D, w.sparsity,
                                         io_dtype="f32").workspace_bytes)


def test_plan_cache_is_bounded_by_workspace_bytes():
    # workspaces stand in as host tensors (no GPU here): the cache evicts the
    # least recently used plans until what it pins fits the byte budget
    import torch
    old = vsa.plan_cache_bytes()
    vsa._plans.clear()
    try:
        vsa.set_plan_cache_bytes(2500)
        plans = []
        for n in range(3):
            w = Workload(f"c{n}", 2, 64, "f32", ((TEXT, 10 + n),), (4, 4, 4), 0.5)
            tags, pos = make_layout(w)
            p = vsa.get_plan(tags, pos, w.grid, w.heads, w.head_dim, w.sparsity)
            p._ws[(0, n)] = torch.empty(1000, dtype=torch.uint8)
            plans.append(p)
            vsa._trim_plan_cache()
        cached = list(vsa._plans.values())
        assert cached == plans[1:]                      # the oldest went first
        assert sum(p.resident_bytes() for p in cached) <= 2500
        # a plan used again moves to the back of the eviction order
        w = Workload("c1", 2, 64, "f32", ((TEXT, 11),), (4, 4, 4), 0.5)
        tags, pos = make_layout(w)
        assert vsa.get_plan(tags, pos, w.grid, w.heads, w.head_dim, w.sparsity) is plans[1]
        vsa.set_plan_cache_bytes(1500)
        assert list(vsa._plans.values()) == [plans[1]]
        # a plan whose own workspaces exceed the budget is not kept either
        plans[1]._ws[(0, 9)] = torch.empty(1000, dtype=torch.uint8)
        vsa._trim_plan_cache()
        assert not vsa._plans
        with pytest.raises(vsa.VsaError):
            vsa.set_plan_cache_bytes(-1)
    finally:
        vsa._plans.clear()
        vsa.set_plan_cache_bytes(old)

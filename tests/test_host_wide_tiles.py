"""Host-side tests (no GPU) of 128-token tiles and the reference keep ratio:
plan geometry against the oracle's geometry, the keep rule against the
oracle's rule, argument errors and the workspace regions."""
import ctypes

import numpy as np
import pytest

import oracle
import video_dit_block_amd as vsa
from video_dit_block_amd import _abi
from workloads import AUDIO, COND, TEXT, WORKLOADS, Workload, make_layout

WIDE = [
    ("omniref_small", WORKLOADS["omniref_small"], "raster"),
    ("omniref768p10s", WORKLOADS["omniref768p10s"], "raster"),
    ("t844_odd", Workload("a", 2, 64, "f32", ((COND, 300), (TEXT, 64), (COND, 65)), (9, 8, 13),
                          0.6, tile=(8, 4, 4)), "shuffled"),
    ("t288_odd", Workload("b", 2, 128, "bf16", ((TEXT, 10), (AUDIO, 129)), (5, 17, 9), 0.8,
                          tile=(2, 8, 8)), "shuffled"),
    ("t1_1_128", Workload("c", 1, 64, "f32", ((TEXT, 1),), (3, 2, 300), 0.5,
                          tile=(1, 1, 128)), "shuffled"),
    ("video_only", Workload("d", 2, 64, "f32", (), (8, 16, 8), 0.5, tile=(4, 8, 4)), "raster"),
]


@pytest.mark.parametrize("name,w,order", WIDE, ids=[x[0] for x in WIDE])
def test_wide_plan_geometry_matches_oracle(name, w, order):
    tags, pos = make_layout(w, order, seed=5)
    p = vsa.Plan(tags, pos, w.grid, w.heads, w.head_dim, w.sparsity, w.tile)
    g = oracle.geometry(tags.numpy(), pos.numpy(), w.grid, w.tile)
    assert (p.num_prefix_tiles, p.num_video_tiles, p.num_tiles) == (g.P, g.NV, g.Nt)
    assert p.tile_tokens == 128 and p.num_blocks == 2 * g.Nt
    assert p.topk == oracle.topk_count(g.NV, w.sparsity)
    assert p.num_ref_tiles == int(np.sum(g.tile_tag == COND))
    perm, valid, tile_slot = p.tables()
    assert perm.shape == (g.Nt, 128)
    assert np.array_equal(valid, g.valid)
    assert np.array_equal(perm, g.perm())
    assert np.array_equal(tile_slot, g.tile_of_token() * 128 + g.slot_of_token())


def test_ref_keep_count_matches_oracle_rule():
    w = Workload("r", 2, 64, "f32", ((TEXT, 64), (COND, 64 * 25), (AUDIO, 64)), (4, 4, 4), 0.5)
    tags, pos = make_layout(w)
    for keep in (0.01, 0.1, 0.28, 0.5, 0.96, 0.999999):
        p = vsa.Plan(tags, pos, w.grid, 2, 64, 0.5, ref_keep=keep)
        assert p.num_ref_tiles == 25
        assert p.topk_ref == oracle.ref_keep_count(25, keep), keep
        assert p.sel_width == p.topk_ref + p.topk
        assert p.info.ref_keep == keep
    assert oracle.ref_keep_count(25, 0.28) == 8          # 0.28 * 25 rounds above 7 in double
    p = vsa.Plan(tags, pos, w.grid, 2, 64, 0.5)
    assert (p.topk_ref, p.info.ref_keep) == (0, 1.0)


def test_ref_keep_without_reference_tiles_keeps_the_base_layout():
    w = Workload("n", 2, 64, "f32", ((TEXT, 100),), (4, 8, 8), 0.5)
    tags, pos = make_layout(w)
    a = vsa.Plan(tags, pos, w.grid, 2, 64, 0.5, ref_keep=0.1)
    b = vsa.Plan(tags, pos, w.grid, 2, 64, 0.5)
    assert a.topk_ref == 0 and a.workspace_bytes == b.workspace_bytes


@pytest.mark.parametrize("keep", [0.0, -0.1, 1.5, float("nan"), float("inf")])
def test_ref_keep_out_of_range_is_an_argument_error(keep):
    w = WORKLOADS["omniref_small"]
    tags, pos = make_layout(w)
    p = vsa.Plan(tags, pos, w.grid, 2, 128, 0.7, w.tile)
    assert _abi.lib().vsa_h3_plan_set_ref_keep(p.handle, ctypes.c_double(keep)) == -1
    assert "keep" in _abi.vsa_h3_last_error()
    with pytest.raises(vsa.VsaError):
        vsa.Plan(tags, pos, w.grid, 2, 128, 0.7, w.tile, ref_keep=keep)
    assert _abi.lib().vsa_h3_plan_set_ref_keep(None, ctypes.c_double(0.5)) == -1


@pytest.mark.parametrize("tile", [(4, 4, 2), (3, 3, 3), (4, 8, 8), (0, 8, 16), (-4, -8, 4)])
def test_other_tile_volumes_are_unsupported(tile):
    w = Workload("v", 2, 64, "f32", ((TEXT, 10),), (4, 8, 8), 0.5)
    tags, pos = make_layout(w)
    st = _abi.lib().vsa_h3_plan_create(
        np.ascontiguousarray(tags.numpy(), np.int64).ctypes.data_as(_abi._I64P),
        np.ascontiguousarray(pos.numpy(), np.int64).ctypes.data_as(_abi._I64P), w.L,
        _abi.Dims3(*w.grid), _abi.Dims3(*tile), 2, 64, 0.5, ctypes.byref(ctypes.c_void_p()))
    assert st == -4 and "64 or 128" in _abi.vsa_h3_last_error()


def test_wide_workspace_regions_sized_and_disjoint():
    w = WORKLOADS["omniref768p10s"]
    tags, pos = make_layout(w)
    p = vsa.Plan(tags, pos, w.grid, w.heads, w.head_dim, w.sparsity, w.tile, ref_keep=w.ref_keep)
    lo = p.layout
    H, D, Nt, Nb, NV = w.heads, w.head_dim, p.num_tiles, p.num_blocks, p.num_video_tiles
    assert (Nt, Nb, NV, p.topk, p.topk_ref) == (670, 1340, 630, 63, 4)
    V = (p.num_prefix_tiles - p.num_ref_tiles) + p.topk_ref + p.topk
    assert V == 8 + 4 + 63
    ns = (Nt + 3) // 4 * 4
    regions = [("perm", Nb * 64 * 4), ("valid", Nb * 4), ("kind", Nt * 4),
               ("kt", H * Nb * 64 * D * 2), ("vt", H * Nb * 64 * D * 2),
               ("qp", H * Nt * D * 4), ("kp", H * Nt * D * 4), ("vp", H * Nt * D * 4),
               ("scores", H * Nt * ns * 4), ("coarse", H * Nt * D * 4),
               ("sel", H * NV * (p.topk_ref + p.topk) * 4), ("visit", H * NV * V * 4),
               ("chunk_offsets", H * NV * (p.num_chunks + 1) * 4),
               ("state", H * Nb * 2 * 64 * (D // 2 + 4) * 4)]
    assert p.num_chunks > 1
    spans = sorted((getattr(lo, n), getattr(lo, n) + size) for n, size in regions)
    for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
        assert a0 % 256 == 0 and a1 <= b0
    assert spans[-1][1] <= lo.total == p.workspace_bytes
    # a 128-token tile's K+V is 64 KiB at head_dim 128: at most 512 tiles per
    # 32 MiB chunk, balanced: 670 tiles in 2 chunks of 335
    assert (p.chunk_tiles, p.num_chunks) == (335, 2)
    assert p.chunk_tiles * 128 * D * 4 <= 32 << 20
    assert (p.num_chunks - 1) * p.chunk_tiles < Nt <= p.num_chunks * p.chunk_tiles

"""Pins of the oracle's 128-token tiles and reference keep ratio.

Each check compares the oracle with something other than itself: closed-form
tile counts, an exhaustive Python sort, torch SDPA in float64 over a token
mask built here from the scores, or the method without the keep ratio.
"""
import math

import numpy as np
import pytest
import torch

from oracle import vsa_h3 as O
from workloads import TEXT, COND, AUDIO, VIDEO, Workload, make_inputs, make_layout


def _sdpa64(q, k, v, mask=None):
    qt = torch.as_tensor(np.asarray(q, np.float64)).permute(1, 0, 2).unsqueeze(0)
    kt = torch.as_tensor(np.asarray(k, np.float64)).permute(1, 0, 2).unsqueeze(0)
    vt = torch.as_tensor(np.asarray(v, np.float64)).permute(1, 0, 2).unsqueeze(0)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    return o[0].permute(1, 0, 2).numpy()


def _f32(x):
    return x.to(torch.float32).numpy()


def _inputs(grid, prefix, sparsity=0.5, heads=2, D=16, seed=0, order="raster"):
    w = Workload("w", heads, D, "f32", prefix, grid, sparsity)
    return w, make_inputs(w, seed=seed, video_order=order)


# ----------------------------------------------------------------- keep count
def test_ref_keep_count_closed_form():
    assert O.ref_keep_count(32, 0.1) == 4        # ceil(3.2)
    assert O.ref_keep_count(10, 0.1) == 1
    assert O.ref_keep_count(3, 0.99) == 3        # ceil(2.97)
    assert O.ref_keep_count(5, 1.0) == 5
    assert O.ref_keep_count(1, 0.01) == 1        # at least one
    assert O.ref_keep_count(0, 0.1) == 0         # nothing to keep
    # evaluated in double as written: 0.28 * 25 = 7.000000000000001 -> 8
    assert 0.28 * 25 > 7.0
    assert O.ref_keep_count(25, 0.28) == 8
    for n in (1, 4, 33):
        ks = [O.ref_keep_count(n, r / 50) for r in range(1, 51)]
        assert all(1 <= k <= n for k in ks) and ks[-1] == n
        assert all(a <= b for a, b in zip(ks, ks[1:]))


# ----------------------------------------------------------------- geometry
@pytest.mark.parametrize("tile", [(4, 8, 4), (8, 4, 4), (2, 8, 8)])
def test_geometry_128_closed_form(tile):
    grid = (6, 11, 9)
    prefix = ((TEXT, 150), (COND, 200), (AUDIO, 20))
    w = Workload("w", 1, 8, "f32", prefix, grid, 0.5)
    tags, pos = make_layout(w, "shuffled", seed=2)
    g = O.geometry(tags.numpy(), pos.numpy(), grid, tile)
    assert g.tile_tokens == 128
    # prefix runs cut into 128-token chunks: text 128 + 22, cond 128 + 72, audio 20
    assert g.P == 5 and list(g.valid[:5]) == [128, 22, 128, 72, 20]
    assert list(g.tile_tag[:5]) == [TEXT, TEXT, COND, COND, AUDIO]
    ext = [[min(b, n - b * i) for i in range(-(-n // b))] for n, b in zip(grid, tile)]
    assert g.NV == len(ext[0]) * len(ext[1]) * len(ext[2])
    assert list(g.valid[5:]) == [a * b * c for a in ext[0] for b in ext[1] for c in ext[2]]
    allidx = np.sort(np.concatenate(g.tiles))
    assert np.array_equal(allidx, np.arange(w.L))
    P = pos.numpy()
    nh, nw = len(ext[1]), len(ext[2])
    for j in range(5, g.Nt):
        tyx = P[g.tiles[j]]
        assert [tuple(r) for r in tyx] == sorted(tuple(r) for r in tyx)
        boxes = {(t // tile[0], y // tile[1], x // tile[2]) for t, y, x in tyx}
        assert len(boxes) == 1
        (bt, by, bx), = boxes
        assert j - 5 == (bt * nh + by) * nw + bx
    assert g.perm().shape == (g.Nt, 128)


@pytest.mark.parametrize("tile", [(4, 4, 2), (3, 3, 3), (4, 4, 16), (0, 8, 8)])
def test_geometry_rejects_other_tile_volumes(tile):
    w = Workload("w", 1, 8, "f32", ((TEXT, 10),), (4, 4, 4), 0.5)
    tags, pos = make_layout(w)
    with pytest.raises(O.GeometryError):
        O.geometry(tags.numpy(), pos.numpy(), w.grid, tile)


def test_pool_128_constant_tiles_exact_and_float64_bound():
    w = Workload("w", 1, 8, "f32", ((TEXT, 300),), (5, 10, 9), 0.5)
    tags, pos = make_layout(w, "shuffled", seed=1)
    g = O.geometry(tags.numpy(), pos.numpy(), w.grid, (4, 8, 4))
    rng = np.random.default_rng(1)
    vals = np.round(rng.standard_normal((g.Nt, 8)) * 64) / 64      # dyadic: exact sums
    x = np.zeros((w.L, 8), np.float32)
    for j, idx in enumerate(g.tiles):
        x[idx] = vals[j]
    assert np.array_equal(O.pool_canonical(x, g), vals.astype(np.float32))
    x = rng.standard_normal((w.L, 8)).astype(np.float32)
    p = O.pool_canonical(x, g)
    u = 2.0 ** -24
    for j, idx in enumerate(g.tiles):
        exact = x[idx].astype(np.float64).mean(axis=0)
        n = len(idx)
        bound = (n * u) * np.abs(x[idx]).astype(np.float64).sum(axis=0) / n + u * np.abs(exact)
        assert np.all(np.abs(p[j] - exact) <= bound * 1.01 + 1e-30)
    assert max(len(t) for t in g.tiles) == 128


def test_pool_128_sums_past_slot_64_in_slot_order():
    # 1 in slot 0, then 127 terms of 2^-24: each one is lost against the running
    # sum in slot order (ties to even), so the mean is exactly 1/128; any order
    # that adds a half-tile partial sum first would keep them.
    idx = np.arange(128)
    g = O.Geometry(L=128, P=1, NV=0, tiles=[idx], tile_tag=np.array([TEXT]), grid=(0, 0, 0),
                   tile_dims=(4, 8, 4))
    x = np.full((128, 1), 2.0 ** -24, np.float32)
    x[0] = 1.0
    assert O.pool_canonical(x, g)[0, 0] == np.float32(1.0 / 128)
    g2 = O.Geometry(L=128, P=1, NV=0, tiles=[idx[::-1].copy()], tile_tag=np.array([TEXT]),
                    grid=(0, 0, 0), tile_dims=(4, 8, 4))
    assert O.pool_canonical(x, g2)[0, 0] > np.float32(1.0 / 128)


# ----------------------------------------------------------------- reference selection
def test_select_ref_matches_exhaustive_sort_over_cond_tiles_only():
    rng = np.random.default_rng(4)
    tags = np.array([TEXT, COND, COND, AUDIO, COND, TEXT, COND] + [VIDEO] * 30, np.int64)
    g = O.Geometry(L=0, P=7, NV=30, tiles=[np.zeros(1)] * 37, tile_tag=tags, grid=(0, 0, 0))
    S = rng.integers(-4, 4, size=(37, 37)).astype(np.float32)    # many exact ties
    S[S == 0] = -0.0
    ref = [1, 2, 4, 6]
    for kr in (1, 2, 4):
        rs = O.select_ref(S, g, kr)
        assert rs.shape == (30, kr)
        for i in range(30):
            row = {j: float(S[7 + i, j]) for j in ref}
            best = sorted(ref, key=lambda j: (-row[j], j))[:kr]
            assert list(rs[i]) == sorted(best)


def test_ref_ties_go_to_the_lower_tile_index():
    w, x = _inputs((8, 8, 8), ((TEXT, 64), (COND, 256)), sparsity=0.5, heads=1)
    g = O.geometry(x["token_tags"], x["position_ids"], w.grid, (4, 8, 4))
    assert list(g.tile_tag[:g.P]) == [TEXT, COND, COND]
    k = x["k"].clone()
    k[torch.as_tensor(g.tiles[2])] = k[torch.as_tensor(g.tiles[1])]   # equal pooled keys
    r = O.forward_head(x["q"], k, x["v"], x["gate"], g, O.topk_count(g.NV, 0.5), 0,
                       with_fine=False, ref_keep=0.5)
    assert r.ref_sel.shape == (g.NV, 1)
    assert np.all(r.ref_sel[:, 0] == 1)
    assert np.all(r.S[g.P:, 1] == r.S[g.P:, 2])


def _masked_reference(x, g, S, topk, kr, h):
    """Token-level mask built here from the scores: prefix query rows see every
    token; a video query tile sees the text and audio tiles, its kr best
    reference tiles and its topk best video tiles (ties to the lower index)."""
    ref = [j for j in range(g.P) if g.tile_tag[j] == COND]
    allowed = np.zeros((g.Nt, g.Nt), bool)
    allowed[:g.P, :] = True
    for i in range(g.P, g.Nt):
        row = [float(s) for s in S[i]]
        for j in range(g.P):
            if g.tile_tag[j] != COND:
                allowed[i, j] = True
        for j in sorted(ref, key=lambda j: (-row[j], j))[:kr]:
            allowed[i, j] = True
        for j in sorted(range(g.P, g.Nt), key=lambda j: (-row[j], j))[:topk]:
            allowed[i, j] = True
    tile = g.tile_of_token()
    mask = torch.as_tensor(allowed[tile][:, tile])
    return _sdpa64(_f32(x["q"])[:, h:h + 1], _f32(x["k"])[:, h:h + 1], _f32(x["v"])[:, h:h + 1],
                   mask=mask)[:, 0]


@pytest.mark.parametrize("tile,keep", [((4, 8, 4), 0.3), ((8, 4, 4), 0.5), ((4, 4, 4), 0.2)])
def test_fine_with_ref_keep_equals_token_level_masked_attention(tile, keep):
    w, x = _inputs((9, 10, 8), ((TEXT, 70), (COND, 500), (AUDIO, 40), (COND, 130)),
                   sparsity=0.7, order="shuffled")
    g = O.geometry(x["token_tags"], x["position_ids"], w.grid, tile)
    topk = O.topk_count(g.NV, 0.7)
    nref = int(np.sum(g.tile_tag == COND))
    kr = O.ref_keep_count(nref, keep)
    assert 0 < kr < nref
    for h in range(2):
        r = O.forward_head(x["q"], x["k"], x["v"], x["gate"], g, topk, h, ref_keep=keep)
        ref = _masked_reference(x, g, r.S, topk, kr, h)
        assert np.max(np.abs(r.o - ref)) < 1e-12
        assert r.ref_sel.shape == (g.NV, kr)


def test_keep_that_keeps_every_reference_tile_equals_the_method_without_it():
    w, x = _inputs((8, 9, 8), ((TEXT, 64), (COND, 300), (AUDIO, 30)), sparsity=0.6)
    g = O.geometry(x["token_tags"], x["position_ids"], w.grid, (4, 8, 4))
    nref = int(np.sum(g.tile_tag == COND))
    assert nref == 3 and O.ref_keep_count(nref, 0.99) == 3
    topk = O.topk_count(g.NV, 0.6)
    for h in range(2):
        a = O.forward_head(x["q"], x["k"], x["v"], x["gate"], g, topk, h, ref_keep=0.99)
        b = O.forward_head(x["q"], x["k"], x["v"], x["gate"], g, topk, h)
        assert b.ref_sel is None and a.ref_sel.shape == (g.NV, 3)
        assert np.max(np.abs(a.out - b.out)) < 1e-12
        assert np.array_equal(a.c, b.c)


def test_sparsity0_128_tiles_equals_sdpa():
    w, x = _inputs((5, 9, 7), ((TEXT, 70), (COND, 20), (AUDIO, 33)), sparsity=0.0, D=32,
                   order="shuffled")
    res = O.forward(x["q"], x["k"], x["v"], torch.zeros_like(x["gate"]), x["token_tags"],
                    x["position_ids"], w.grid, 0.0, tile=(4, 8, 4))
    ref = _sdpa64(_f32(x["q"]), _f32(x["k"]), _f32(x["v"]))
    for h in range(2):
        assert np.max(np.abs(res["heads"][h].o - ref[:, h, :])) < 1e-12


def test_ref_keep_leaves_prefix_rows_dense_and_coarse_unchanged():
    w, x = _inputs((8, 8, 12), ((TEXT, 64), (COND, 400), (AUDIO, 50)), sparsity=0.8)
    g = O.geometry(x["token_tags"], x["position_ids"], w.grid, (4, 8, 4))
    ref = _sdpa64(_f32(x["q"]), _f32(x["k"]), _f32(x["v"]))
    npre = 514
    topk = O.topk_count(g.NV, 0.8)
    for h in range(2):
        a = O.forward_head(x["q"], x["k"], x["v"], x["gate"], g, topk, h, ref_keep=0.25)
        b = O.forward_head(x["q"], x["k"], x["v"], x["gate"], g, topk, h)
        assert np.max(np.abs(a.o[:npre] - ref[:npre, h, :])) < 1e-12
        assert np.array_equal(a.c, b.c) and np.array_equal(a.sel, b.sel)
        # video rows genuinely see fewer reference tiles
        assert np.max(np.abs(a.o[npre:] - b.o[npre:])) > 1e-3


def test_ref_keep_out_of_range_is_rejected():
    w, x = _inputs((4, 8, 4), ((COND, 64),), heads=1)
    g = O.geometry(x["token_tags"], x["position_ids"], w.grid)
    for r in (0.0, -0.5, 1.5, math.nan):
        with pytest.raises(ValueError):
            O.forward_head(x["q"], x["k"], x["v"], x["gate"], g, 1, 0, with_fine=False,
                           ref_keep=r)

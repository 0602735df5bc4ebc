"""Pins of the CPU oracle against what the pages and mathematics fix.

None of these compares the oracle with itself: each check uses a closed form,
a library routine (torch SDPA in float64), an exhaustive sort, or an
independent token-level formulation.  All run on the CPU in seconds.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import vsa_h3 as O
from workloads import TEXT, COND, AUDIO, VIDEO, WORKLOADS, Workload, make_inputs, make_layout

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _sdpa64(q, k, v, mask=None):
    """torch SDPA in float64 on the packed sequence, per head: [L, H, D]."""
    qt = torch.as_tensor(np.asarray(q, np.float64)).permute(1, 0, 2).unsqueeze(0)
    kt = torch.as_tensor(np.asarray(k, np.float64)).permute(1, 0, 2).unsqueeze(0)
    vt = torch.as_tensor(np.asarray(v, np.float64)).permute(1, 0, 2).unsqueeze(0)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
    return o[0].permute(1, 0, 2).numpy()


def _f32(x):
    return x.to(torch.float32).numpy()


def small_workload(grid=(5, 6, 7), prefix=((TEXT, 70), (AUDIO, 40)), heads=2, D=32,
                   sparsity=0.5):
    return Workload("t", heads, D, "f32", prefix, grid, sparsity)


# ----------------------------------------------------------------- top-k rule
def test_topk_golden_cases():
    rows = []
    with open(os.path.join(GOLDEN, "topk_cases.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                n, s, k = line.split()[:3]
                rows.append((int(n), float(s), int(k)))
    assert len(rows) >= 10
    for n, s, k in rows:
        assert O.topk_count(n, s) == k, (n, s)


def test_topk_bounds_and_monotone():
    for n in (1, 2, 7, 64, 1260):
        ks = [O.topk_count(n, s / 100) for s in range(101)]
        assert ks[0] == n and ks[-1] == 1
        assert all(1 <= k <= n for k in ks)
        assert all(a >= b for a, b in zip(ks, ks[1:]))
    assert O.topk_count(0, 0.5) == 0


# ----------------------------------------------------------------- geometry
def test_geometry_odd_grid_closed_form():
    w = small_workload(grid=(5, 6, 7))
    tags, pos = make_layout(w)
    g = O.geometry(tags.numpy(), pos.numpy(), w.grid)
    # prefix: text 70 -> 64 + 6, audio 40 -> 40
    assert g.P == 3 and list(g.valid[:3]) == [64, 6, 40]
    assert list(g.tile_tag[:3]) == [TEXT, TEXT, AUDIO]
    # video: ceil(5/4) * ceil(6/4) * ceil(7/4) = 2 * 2 * 2 tiles
    assert g.NV == 8
    ext = lambda n: [min(4, n - 4 * b) for b in range(-(-n // 4))]
    expect = [a * b * c for a in ext(5) for b in ext(6) for c in ext(7)]
    assert list(g.valid[3:]) == expect
    # every token in exactly one tile; video slot order is the (t, y, x) raster
    allidx = np.sort(np.concatenate(g.tiles))
    assert np.array_equal(allidx, np.arange(w.L))
    P = pos.numpy()
    for j in range(3, 11):
        tyx = P[g.tiles[j]]
        key = [tuple(r) for r in tyx]
        assert key == sorted(key)
        tb = {(t // 4, y // 4, x // 4) for t, y, x in tyx}
        assert len(tb) == 1
        (bt, by, bx), = tb
        assert j - 3 == (bt * 2 + by) * 2 + bx


def test_geometry_shuffled_order_same_tiles():
    w = small_workload(grid=(6, 5, 9))
    t1, p1 = make_layout(w, "raster")
    t2, p2 = make_layout(w, "shuffled", seed=3)
    g1 = O.geometry(t1.numpy(), p1.numpy(), w.grid)
    g2 = O.geometry(t2.numpy(), p2.numpy(), w.grid)
    assert g1.P == g2.P and g1.NV == g2.NV
    for a, b in zip(g1.tiles, g2.tiles):
        assert np.array_equal(p1.numpy()[a], p2.numpy()[b])


@pytest.mark.parametrize("case", ["video_first", "dup", "outside", "count", "badtag"])
def test_geometry_rejects(case):
    w = small_workload(grid=(4, 4, 4), prefix=((TEXT, 10),))
    tags, pos = make_layout(w)
    tags, pos = tags.numpy().copy(), pos.numpy().copy()
    grid = w.grid
    if case == "video_first":
        tags[[0, 20]] = tags[[20, 0]]
    elif case == "dup":
        pos[20] = pos[21]
    elif case == "outside":
        pos[20, 2] = 4
    elif case == "count":
        grid = (4, 4, 5)
    elif case == "badtag":
        tags[3] = 9
    with pytest.raises(O.GeometryError):
        O.geometry(tags, pos, grid)


# ----------------------------------------------------------------- pooling
def test_pool_constant_tiles_exact():
    w = small_workload(grid=(5, 6, 7), heads=1, D=8)
    tags, pos = make_layout(w)
    g = O.geometry(tags.numpy(), pos.numpy(), w.grid)
    vals = np.random.default_rng(1).standard_normal((g.Nt, 8)).astype(np.float32)
    x = np.zeros((w.L, 8), np.float32)
    for j, idx in enumerate(g.tiles):
        x[idx] = vals[j]
    # n copies of a value summed in fp32 then divided by n: exact for n <= 64
    # only when the partial sums are exact; use dyadic values to make them so.
    vals = np.round(vals * 64) / 64
    for j, idx in enumerate(g.tiles):
        x[idx] = vals[j]
    assert np.array_equal(O.pool_canonical(x, g), vals)


def test_pool_vs_float64_mean_bound():
    w = small_workload(grid=(9, 8, 7), heads=1, D=16)
    tags, pos = make_layout(w)
    g = O.geometry(tags.numpy(), pos.numpy(), w.grid)
    x = np.random.default_rng(2).standard_normal((w.L, 16)).astype(np.float32)
    p = O.pool_canonical(x, g)
    u = 2.0 ** -24
    for j, idx in enumerate(g.tiles):
        exact = x[idx].astype(np.float64).mean(axis=0)
        n = len(idx)
        bound = (n * u) * np.abs(x[idx]).astype(np.float64).sum(axis=0) / n + u * np.abs(exact) + 1e-30
        assert np.all(np.abs(p[j] - exact) <= bound * 1.01)


def test_pool_sequential_order_is_slot_order():
    # values chosen so that the fp32 result depends on summation order:
    # 1 + 2^-24 + 2^-24 ... in slot order loses the small terms one by one.
    g = O.Geometry(L=3, P=1, NV=0, tiles=[np.array([0, 1, 2])], tile_tag=np.array([0]),
                   grid=(0, 0, 0))
    x = np.array([[1.0], [2.0 ** -24], [2.0 ** -24]], np.float32)
    assert O.pool_canonical(x, g)[0, 0] == np.float32(1.0) / np.float32(3.0)
    g2 = O.Geometry(L=3, P=1, NV=0, tiles=[np.array([1, 2, 0])], tile_tag=np.array([0]),
                    grid=(0, 0, 0))
    assert O.pool_canonical(x, g2)[0, 0] == np.float32(1.0 + 2.0 ** -23) / np.float32(3.0)


# ----------------------------------------------------------------- scores
def test_scores_vs_float64_error_bound():
    rng = np.random.default_rng(3)
    qp = rng.standard_normal((20, 128)).astype(np.float32)
    kp = rng.standard_normal((30, 128)).astype(np.float32)
    S = O.scores_canonical(qp, kp)
    exact = qp.astype(np.float64) @ kp.astype(np.float64).T
    u = 2.0 ** -24
    gam = 128 * u / (1 - 128 * u)
    bound = gam * (np.abs(qp).astype(np.float64) @ np.abs(kp).astype(np.float64).T)
    assert np.all(np.abs(S - exact) <= bound)
    assert S.dtype == np.float32


def test_scores_fixed_order_no_fma():
    # term 1: a*b = 2^-24 * (1 + 2^-36) exactly, which rounds to 2^-24 as a
    # product.  Separately rounded: fl(1 + 2^-24) is a tie -> 1.0 (even).
    # A fused multiply-add would see the 2^-60 excess and give 1 + 2^-23.
    b1 = np.float32(2.0 ** -24 * (1 - 2.0 ** -12 + 2.0 ** -24))
    assert float(b1) == 2.0 ** -24 * (1 - 2.0 ** -12 + 2.0 ** -24)
    qp = np.array([[1.0, 1.0 + 2.0 ** -12]], np.float32)
    kp = np.array([[1.0, b1]], np.float32)
    assert O.scores_canonical(qp, kp)[0, 0] == np.float32(1.0)
    from fractions import Fraction as F
    exact = F(1) + F(1.0 + 2.0 ** -12) * F(float(b1))
    assert exact > F(1) + F(2.0 ** -24)     # a single rounding would round up to 1 + 2^-23
    # order d = 0, 1, 2: ((1 + 2^-24) + 2^-24) -> 1; the reverse order gives 1 + 2^-23
    qo = np.array([[1.0, 2.0 ** -24, 2.0 ** -24]], np.float32)
    ko = np.ones((1, 3), np.float32)
    assert O.scores_canonical(qo, ko)[0, 0] == np.float32(1.0)
    # integer-valued operands: every partial sum is exact
    qi = np.arange(12, dtype=np.float32).reshape(3, 4)
    ki = np.arange(8, dtype=np.float32).reshape(2, 4) - 3
    assert np.array_equal(O.scores_canonical(qi, ki), (qi.astype(np.int64) @ ki.astype(np.int64).T))


# ----------------------------------------------------------------- selection
def test_select_matches_exhaustive_sort_with_ties():
    rng = np.random.default_rng(4)
    g = O.Geometry(L=0, P=3, NV=40, tiles=[np.zeros(1)] * 43, tile_tag=np.zeros(43, np.int64),
                   grid=(0, 0, 0))
    S = rng.integers(-5, 5, size=(43, 43)).astype(np.float32)   # many exact ties
    S[S == 0] = -0.0                                            # mix -0 and +0
    S[::2][S[::2] == -0.0] = 0.0
    for topk in (1, 7, 40):
        sel = O.select_topk(S, g, topk)
        for i in range(40):
            row = [float(S[3 + i, 3 + j]) for j in range(40)]
            best = sorted(range(40), key=lambda j: (-row[j], j))[:topk]
            assert list(sel[i]) == sorted(b + 3 for b in best)


def _tiny_f32(heads=2, D=32, grid=(8, 8, 8), prefix=((TEXT, 64),), sparsity=0.5, seed=0,
              order="raster"):
    w = Workload("t", heads, D, "f32", prefix, grid, sparsity)
    return w, make_inputs(w, seed=seed, video_order=order)


def test_select_forced_ties_lower_index_wins():
    w, x = _tiny_f32(heads=1, D=16, sparsity=0.75)          # 8 video tiles, topk 2
    g = O.geometry(x["token_tags"], x["position_ids"], w.grid)
    k = x["k"].clone()
    # make video tiles 2, 5 and 6 identical copies of each other (same slot order)
    for dst in (5, 6):
        k[torch.as_tensor(g.tiles[g.P + dst])] = k[torch.as_tensor(g.tiles[g.P + 2])]
    r = O.forward_head(x["q"], k, x["v"], x["gate"], g, O.topk_count(g.NV, 0.75), 0,
                       with_fine=False)
    hit = 0
    for i in range(g.NV):
        row = r.S[g.P + i, g.P:]
        assert row[2] == row[5] == row[6]
        best = sorted(range(g.NV), key=lambda j: (-float(row[j]), j))[:2]
        assert list(r.sel[i]) == sorted(b + g.P for b in best)
        tied = [t for t in (2, 5, 6) if t + g.P in r.sel[i]]
        assert tied == [2, 5, 6][:len(tied)]
        hit += len(tied) in (1, 2)
    assert hit > 0          # the tie actually decided some rows


# ----------------------------------------------------------------- fine branch
@pytest.mark.parametrize("order", ["raster", "shuffled"])
def test_fine_at_sparsity0_equals_sdpa(order):
    w, x = _tiny_f32(heads=2, D=32, grid=(5, 6, 7), prefix=((TEXT, 70), (COND, 20), (AUDIO, 33)),
                     sparsity=0.0, order=order)
    res = O.forward(x["q"], x["k"], x["v"], torch.zeros_like(x["gate"]), x["token_tags"],
                    x["position_ids"], w.grid, 0.0)
    ref = _sdpa64(_f32(x["q"]), _f32(x["k"]), _f32(x["v"]))
    for h in range(2):
        o = res["heads"][h].o
        assert np.max(np.abs(o - ref[:, h, :])) < 1e-12


def test_prefix_rows_dense_at_any_sparsity():
    w, x = _tiny_f32(heads=2, D=32, grid=(8, 8, 12), prefix=((TEXT, 64), (AUDIO, 50)),
                     sparsity=0.8)
    g = O.geometry(x["token_tags"], x["position_ids"], w.grid)
    ref = _sdpa64(_f32(x["q"]), _f32(x["k"]), _f32(x["v"]))
    npre = 114
    for h in range(2):
        r = O.forward_head(x["q"], x["k"], x["v"], x["gate"], g, O.topk_count(g.NV, 0.8), h)
        assert np.max(np.abs(r.o[:npre] - ref[:npre, h, :])) < 1e-12
        # video rows genuinely differ from dense at this sparsity
        assert np.max(np.abs(r.o[npre:] - ref[npre:, h, :])) > 1e-3


def test_fine_equals_token_level_masked_attention():
    """Independent formulation: full L x L boolean mask from the selection,
    masked dense softmax attention (torch SDPA, float64)."""
    w, x = _tiny_f32(heads=2, D=16, grid=(6, 9, 5), prefix=((TEXT, 64), (COND, 10)),
                     sparsity=0.6, order="shuffled")
    g = O.geometry(x["token_tags"], x["position_ids"], w.grid)
    topk = O.topk_count(g.NV, 0.6)
    tile = g.tile_of_token()
    for h in range(2):
        r = O.forward_head(x["q"], x["k"], x["v"], x["gate"], g, topk, h)
        allowed = np.zeros((g.Nt, g.Nt), bool)
        allowed[:g.P, :] = True
        allowed[:, :g.P] = True
        for i in range(g.NV):
            allowed[g.P + i, r.sel[i]] = True
        mask = torch.as_tensor(allowed[tile][:, tile])
        ref = _sdpa64(_f32(x["q"])[:, h:h + 1], _f32(x["k"])[:, h:h + 1], _f32(x["v"])[:, h:h + 1],
                      mask=mask)[:, 0]
        assert np.max(np.abs(r.o - ref)) < 1e-12
        assert all(len(r.sel[i]) == topk for i in range(g.NV))


# ----------------------------------------------------------------- coarse + combine
def _tile_constant_inputs(heads=2, D=16, grid=(8, 8, 8), prefix=((TEXT, 128),), seed=5):
    w = Workload("c", heads, D, "f32", prefix, grid, 0.0)
    tags, pos = make_layout(w, "shuffled", seed=seed)
    g = O.geometry(tags.numpy(), pos.numpy(), w.grid)
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(3):
        vals = rng.standard_normal((g.Nt, heads, D)).astype(np.float32)
        x = np.zeros((w.L, heads, D), np.float32)
        for j, idx in enumerate(g.tiles):
            x[idx] = vals[j]
        out.append(torch.from_numpy(x))
    return w, g, tags, pos, out


def test_coarse_closed_form_tile_constant_equals_dense():
    """With q, k, v constant inside every (full) tile, dense attention of any
    token of tile i equals softmax_j(qp_i . kp_j / sqrt(D)) @ vp_j -- which is
    the compression branch.  Pins the scale, the all-tile softmax domain and
    the unweighted (one term per tile) form."""
    w, g, tags, pos, (q, k, v) = _tile_constant_inputs()
    assert np.all(g.valid == 64)
    dense = _sdpa64(q.numpy(), k.numpy(), v.numpy())
    tile = g.tile_of_token()
    for h in range(2):
        r = O.forward_head(q, k, v, torch.zeros_like(q), g, g.NV, h, with_fine=False)
        assert np.max(np.abs(r.c[tile] - dense[:, h, :])) < 2e-6  # fp32 pooled scores


def test_combine_gate_closed_forms():
    w, g, tags, pos, (q, k, v) = _tile_constant_inputs(heads=1, D=8)
    dense = _sdpa64(q.numpy(), k.numpy(), v.numpy())[:, 0, :]
    # gate 0 -> out == o exactly
    r0 = O.forward_head(q, k, v, torch.zeros_like(q), g, g.NV, 0)
    assert np.array_equal(r0.out, r0.o)
    # per-channel gate alpha_d, tile-constant inputs at sparsity 0:
    # out = dense + alpha_d * dense
    alpha = torch.linspace(-1.0, 2.0, 8).view(1, 1, 8).expand(w.L, 1, 8).contiguous()
    r1 = O.forward_head(q, k, v, alpha, g, g.NV, 0)
    assert np.max(np.abs(r1.out - dense * (1.0 + alpha[:, 0, :].numpy()))) < 1e-5


def test_coarse_equal_keys_gives_mean_of_pooled_values():
    rng = np.random.default_rng(6)
    S = np.full((5, 7), 0.3125, np.float32)
    vp = rng.standard_normal((7, 4)).astype(np.float32)
    c = O.coarse(S, vp, 1 / math.sqrt(4))
    assert np.max(np.abs(c - vp.astype(np.float64).mean(axis=0))) < 1e-15


# ----------------------------------------------------------------- invariants
def test_packed_order_permutation_invariance():
    w, x1 = _tiny_f32(heads=2, D=16, grid=(5, 6, 7), sparsity=0.5, order="raster")
    _, x2 = _tiny_f32(heads=2, D=16, grid=(5, 6, 7), sparsity=0.5, order="shuffled")
    # carry the same per-position values into the shuffled packing
    p1, p2 = x1["position_ids"].numpy(), x2["position_ids"].numpy()
    npre = w.n_prefix_tokens
    T, H, W = w.grid
    cell = lambda p: (p[:, 0] * H + p[:, 1]) * W + p[:, 2]
    src = np.empty(w.L, np.int64)
    src[:npre] = np.arange(npre)
    inv1 = np.empty(T * H * W, np.int64)
    inv1[cell(p1[npre:])] = np.arange(npre, w.L)
    src[npre:] = inv1[cell(p2[npre:])]
    xs = {n: x1[n][torch.as_tensor(src)] for n in ("q", "k", "v", "gate")}
    r1 = O.forward(x1["q"], x1["k"], x1["v"], x1["gate"], x1["token_tags"], p1, w.grid, 0.5)
    r2 = O.forward(xs["q"], xs["k"], xs["v"], xs["gate"], x2["token_tags"], p2, w.grid, 0.5)
    for h in range(2):
        assert np.array_equal(r1["heads"][h].sel, r2["heads"][h].sel)
    assert np.array_equal(r1["out"][src], r2["out"])


def test_head_independence():
    w, x = _tiny_f32(heads=3, D=16, grid=(8, 4, 8), sparsity=0.5)
    r1 = O.forward(x["q"], x["k"], x["v"], x["gate"], x["token_tags"], x["position_ids"], w.grid, 0.5)
    x2 = {n: x[n].clone() for n in ("q", "k", "v", "gate")}
    for n in x2:
        x2[n][:, 1] = torch.randn_like(x2[n][:, 1])
    r2 = O.forward(x2["q"], x2["k"], x2["v"], x2["gate"], x["token_tags"], x["position_ids"], w.grid, 0.5)
    for h in (0, 2):
        assert np.array_equal(r1["out"][:, h], r2["out"][:, h])
        assert np.array_equal(r1["heads"][h].sel, r2["heads"][h].sel)


# ----------------------------------------------------------------- rounding
def test_round_bf16_single_rounding():
    # exactly representable in fp32: must equal torch's fp32 -> bf16 RNE
    xs = np.random.default_rng(7).standard_normal(10000).astype(np.float32)
    xs = np.concatenate([xs, np.float32([0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8,
                                         3.0e38, -3.0e38, 1e-40, 2.0 ** -133])])
    ref = torch.from_numpy(xs).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16_from_f64(xs.astype(np.float64))
    assert np.array_equal(got, ref)
    # a float64 value just above a bf16 tie: a detour through fp32 would land
    # exactly on the tie and round to even (1.0); one rounding gives 1 + 2^-7
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert O.round_bf16_from_f64(np.array([x]))[0] == 1.0 + 2.0 ** -7
    assert np.isinf(O.round_bf16_from_f64(np.array([3.5e38]))[0])


def test_tiny_workload_end_to_end_shapes():
    w = WORKLOADS["tiny"]
    x = make_inputs(w)
    res = oracle.forward(x["q"], x["k"], x["v"], x["gate"], x["token_tags"], x["position_ids"],
                         w.grid, w.sparsity)
    g = res["geom"]
    assert (g.P, g.NV, res["topk"]) == (1, 8, 4)
    assert res["out"].shape == (576, 2, 64) and np.all(np.isfinite(res["out"]))
    for h in range(2):
        sel = res["heads"][h].sel
        assert sel.shape == (8, 4) and np.all(np.diff(sel, axis=1) > 0)
        assert sel.min() >= 1 and sel.max() <= 8


def _pooled_f64(x, g, h):
    """Per-tile float64 mean of head h (an independent pooling for the checks below)."""
    a = _f32(x[:, h, :]).astype(np.float64)
    return np.stack([a[idx].mean(axis=0) for idx in g.tiles])


def test_coarse_equals_sdpa_over_pooled_tokens():
    """Library special case: the compression branch is plain softmax attention
    in which each tile is one token (pooled q, k, v)."""
    w, x = _tiny_f32(heads=2, D=32, grid=(5, 6, 7), prefix=((TEXT, 70), (AUDIO, 40)),
                     sparsity=0.5, order="shuffled")
    g = O.geometry(x["token_tags"], x["position_ids"], w.grid)
    for h in range(2):
        r = O.forward_head(x["q"], x["k"], x["v"], x["gate"], g, O.topk_count(g.NV, 0.5), h,
                           with_fine=False)
        qp, kp, vp = (_pooled_f64(x[n], g, h) for n in ("q", "k", "v"))
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.as_tensor(qp)[None], torch.as_tensor(kp)[None], torch.as_tensor(vp)[None])[0]
        assert np.max(np.abs(r.c - ref.numpy())) < 1e-5


def test_combine_with_independent_branches():
    """out = o + gate * c[tile(r)], with o from masked dense SDPA and c from
    SDPA over pooled tokens (both float64 library calls), on random inputs
    where o and c differ."""
    w, x = _tiny_f32(heads=1, D=16, grid=(6, 8, 5), prefix=((TEXT, 64), (COND, 12)),
                     sparsity=0.5, order="shuffled")
    g = O.geometry(x["token_tags"], x["position_ids"], w.grid)
    r = O.forward_head(x["q"], x["k"], x["v"], x["gate"], g, O.topk_count(g.NV, 0.5), 0)
    tile = g.tile_of_token()
    allowed = np.zeros((g.Nt, g.Nt), bool)
    allowed[:g.P, :] = True
    allowed[:, :g.P] = True
    for i in range(g.NV):
        allowed[g.P + i, r.sel[i]] = True
    o_ref = _sdpa64(_f32(x["q"]), _f32(x["k"]), _f32(x["v"]),
                    mask=torch.as_tensor(allowed[tile][:, tile]))[:, 0]
    qp, kp, vp = (_pooled_f64(x[n], g, 0) for n in ("q", "k", "v"))
    c_ref = torch.nn.functional.scaled_dot_product_attention(
        torch.as_tensor(qp)[None], torch.as_tensor(kp)[None], torch.as_tensor(vp)[None])[0].numpy()
    gate = _f32(x["gate"])[:, 0].astype(np.float64) * 10.0      # make the gated term visible
    out = O.combine(r.o, gate, r.c, g)
    assert np.max(np.abs(o_ref - c_ref[tile])) > 1e-2            # o and c really differ
    assert np.max(np.abs(out - (o_ref + gate * c_ref[tile]))) < 1e-5


# ----------------------------------------------------------------- QK-norm + RoPE (optional upstream step)
def _ident_tables(L, D):
    return np.ones((L, D // 2), np.float32), np.zeros((L, D // 2), np.float32)


def test_qk_norm_hand_computed_row():
    # x = (3, 4), unit weights, eps 0: mean square 12.5, y = x / sqrt(12.5)
    x = np.array([[3.0, 4.0]], np.float32)
    c, s = _ident_tables(1, 2)
    y = oracle.qk_norm_rope(x, np.ones(2, np.float32), 0.0, c, s)
    want = np.array([3.0, 4.0]) / math.sqrt(12.5)
    assert np.allclose(y[0].astype(np.float64), want, rtol=3e-7, atol=0)
    # the weight scales each channel afterwards
    y2 = oracle.qk_norm_rope(x, np.array([2.0, 0.5], np.float32), 0.0, c, s)
    assert np.allclose(y2[0].astype(np.float64), want * [2.0, 0.5], rtol=3e-7, atol=0)


def test_qk_norm_power_of_two_scale_invariance_exact():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, 64)).astype(np.float32)
    w = rng.uniform(0.5, 1.5, 64).astype(np.float32)
    c, s = _ident_tables(50, 64)
    base = oracle.qk_norm_rope(x, w, 0.0, c, s)
    for k in (-6, -1, 3, 10):
        assert np.array_equal(oracle.qk_norm_rope(x * np.float32(2.0 ** k), w, 0.0, c, s), base)


def test_qk_norm_unit_rms_with_unit_weights():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((40, 128)) * rng.uniform(0.1, 30, (40, 1))).astype(np.float32)
    c, s = _ident_tables(40, 128)
    y = oracle.qk_norm_rope(x, np.ones(128, np.float32), 0.0, c, s).astype(np.float64)
    assert np.allclose(np.sqrt((y ** 2).mean(axis=1)), 1.0, rtol=2e-6, atol=0)
    # eps shrinks a small row toward zero exactly as 1/sqrt(ms + eps) says
    tiny = np.full((1, 4), 1e-3, np.float32)
    y = oracle.qk_norm_rope(tiny, np.ones(4, np.float32), 1e-6, *_ident_tables(1, 4))
    assert np.allclose(y[0], 1e-3 / math.sqrt(1e-6 + 1e-6), rtol=1e-6)


def test_rope_identity_and_quarter_turn():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((8, 16)).astype(np.float32)
    w = np.ones(16, np.float32)
    c, s = _ident_tables(8, 16)
    y = oracle.qk_norm_rope(x, w, 0.0, c, s)
    # a quarter turn maps each pair (a, b) to (-b, a) exactly
    q = oracle.qk_norm_rope(x, w, 0.0, np.zeros_like(c), np.ones_like(s))
    assert np.array_equal(q[:, 0::2], -y[:, 1::2]) and np.array_equal(q[:, 1::2], y[:, 0::2])


def test_rope_pair_is_complex_multiplication():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((6, 8)).astype(np.float32)
    w = np.ones(8, np.float32)
    theta = rng.uniform(-math.pi, math.pi, (6, 4))
    c, s = np.cos(theta).astype(np.float32), np.sin(theta).astype(np.float32)
    base = oracle.qk_norm_rope(x, w, 0.0, *_ident_tables(6, 8)).astype(np.float64)
    y = oracle.qk_norm_rope(x, w, 0.0, c, s).astype(np.float64)
    for r in range(6):
        for i in range(4):
            z = complex(base[r, 2 * i], base[r, 2 * i + 1]) * complex(float(c[r, i]), float(s[r, i]))
            assert abs(y[r, 2 * i] - z.real) <= 4e-7 * (abs(z) + 1e-30)
            assert abs(y[r, 2 * i + 1] - z.imag) <= 4e-7 * (abs(z) + 1e-30)
        # rotation keeps every pair's length
        n0 = np.hypot(base[r, 0::2], base[r, 1::2])
        n1 = np.hypot(y[r, 0::2], y[r, 1::2])
        assert np.allclose(n0, n1, rtol=1e-6)


def test_rope_scores_depend_only_on_position_difference():
    # q and k rotated by angles p*f and p'*f: q'.k' equals q rotated by (p - p')*f against k
    rng = np.random.default_rng(4)
    D = 32
    freqs = 1.0 / (10000.0 ** (np.arange(D // 2) * 2.0 / D))
    q = rng.standard_normal((1, D)).astype(np.float32)
    k = rng.standard_normal((1, D)).astype(np.float32)
    w = np.ones(D, np.float32)

    def rot(x, p):
        ang = (p * freqs)[None, :]
        return oracle.qk_norm_rope(x, w, 0.0, np.cos(ang).astype(np.float32),
                                   np.sin(ang).astype(np.float32)).astype(np.float64)
    for p, pp in ((7, 3), (40, 2), (5, 5), (0, 11)):
        lhs = float((rot(q, p) @ rot(k, pp).T).item())
        rhs = float((rot(q, p - pp) @ rot(k, 0).T).item())
        assert abs(lhs - rhs) < 2e-5 * D


def test_rope_rotates_adjacent_channel_pairs_of_the_input():
    # identity tables give the normalised input in its own channel order
    # (float64 formula), and a table that turns only pair i changes only
    # input channels 2i and 2i+1
    rng = np.random.default_rng(5)
    D = 16
    x = rng.standard_normal((3, D)).astype(np.float32)
    w = rng.uniform(0.5, 1.5, D).astype(np.float32)
    c, s = _ident_tables(3, D)
    y = oracle.qk_norm_rope(x, w, 1e-6, c, s).astype(np.float64)
    x64 = x.astype(np.float64)
    ref = x64 / np.sqrt((x64 ** 2).mean(axis=1, keepdims=True) + 1e-6) * w
    assert np.allclose(y, ref, rtol=1e-6, atol=0)
    for i in (0, 3, 7):
        c2, s2 = c.copy(), s.copy()
        c2[:, i], s2[:, i] = 0.0, 1.0
        z = oracle.qk_norm_rope(x, w, 1e-6, c2, s2).astype(np.float64)
        other = [d for d in range(D) if d not in (2 * i, 2 * i + 1)]
        assert np.array_equal(z[:, other], y[:, other])
        assert np.array_equal(z[:, 2 * i], -y[:, 2 * i + 1])
        assert np.array_equal(z[:, 2 * i + 1], y[:, 2 * i])


def test_prep_qk_per_head_weights_rotation_and_io_rounding_closed_form():
    """prep_qk's own steps (R14-R17 over every head): q uses q_weight and k uses
    k_weight, each head and token separately, and the result is rounded to the
    I/O dtype -- bf16 nearest-even for bf16 inputs, left exact for fp32 ones.
    Rows of +-s (s a power of two) normalise to exactly +-1 with eps 0, so the
    expected values follow by hand: y_d = sign_d * w_d, then the token's turn
    of each pair (identity, a quarter turn of pair 0, a half turn)."""
    u = 2.0 ** -10
    qw = np.array([1 + u, 1.5, 3.0, 1 + 2 ** -8 + u], np.float32)      # not all bf16 values
    kw = np.array([2.0, 1 + 2 ** -9, 0.75, 1.0 + 2 ** -7], np.float32)
    sign = np.array([[1.0, -1.0, 1.0, 1.0], [-1.0, 1.0, 1.0, -1.0]])    # per head
    L, H, D = 3, 2, 4
    scale = np.array([[0.5, 4.0], [2.0, 0.125], [1.0, 8.0]])           # per token and head
    x = (scale[:, :, None] * sign[None, :, :]).astype(np.float32)
    cos = np.array([[1, 1], [0, 1], [-1, -1]], np.float32)             # [L, D/2]
    sin = np.array([[0, 0], [1, 0], [0, 0]], np.float32)

    def by_hand(w):
        out = np.empty((L, H, D))
        for h in range(H):
            y = sign[h] * w.astype(np.float64)                         # normalised and weighted
            out[0, h] = y                                              # identity
            out[1, h] = [-y[1], y[0], y[2], y[3]]                      # pair 0 quarter turn
            out[2, h] = -y                                             # half turn of both pairs
        return out

    def bf16_by_hand(v):
        # nearest-even to 8 significant bits, written out for these magnitudes
        m, e = np.frexp(np.abs(v))
        return np.sign(v) * np.ldexp(np.round(np.ldexp(m, 8)), e - 8)

    q32, k32 = oracle.prep_qk(x, x * 3.0, qw, kw, 0.0, cos, sin)
    assert q32.dtype == np.float32 and q32.shape == (L, H, D)
    assert np.array_equal(q32, by_hand(qw))                            # fp32: exact, no rounding
    assert np.array_equal(k32, by_hand(kw))                            # k: its own weights
    xb = torch.from_numpy(x).to(torch.bfloat16)
    assert torch.equal(xb.float(), torch.from_numpy(x))                # inputs exact in bf16
    qb, kb = oracle.prep_qk(xb, xb, qw, kw, 0.0, cos, sin)
    want_q = bf16_by_hand(by_hand(qw))
    assert np.array_equal(qb, want_q)
    assert np.array_equal(kb, bf16_by_hand(by_hand(kw)))
    # the rounding decided these: 1 + 2^-10 -> 1, 1 + 2^-8 + 2^-10 -> 1 + 2^-7 (above the tie)
    assert want_q[0, 0, 0] == 1.0 and want_q[0, 0, 3] == 1 + 2 ** -7
    assert kb[0, 0, 1] == -1.0 and kb[0, 1, 1] == 1.0                  # +-(1 + 2^-9) -> +-1


# ----------------------------------------------------------------- FP8 (OCP E4M3) Q/K for the fine branch
def test_e4m3_decode_printed_codes():
    # values fixed by the OCP FP8 definition: bias 7, 3 mantissa bits, subnormals, max 448
    table = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x3F: 1.875, 0x40: 2.0, 0x7E: 448.0, 0x77: 240.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in table.items():
        assert oracle.e4m3_decode(np.array([c]))[0] == v, hex(c)
    assert np.isnan(oracle.e4m3_decode(np.array([0x7F, 0xFF]))).all()
    assert np.signbit(oracle.e4m3_decode(np.array([0x80]))[0])


def test_e4m3_round_trip_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = oracle.e4m3_decode(codes)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)
    assert np.all(np.diff(vals[:127]) > 0)            # monotone magnitudes 0..448


def test_e4m3_midpoints_round_to_even_code_exactly():
    from fractions import Fraction
    vals = oracle.e4m3_decode(np.arange(127))
    for c in range(126):
        mid = (Fraction(vals[c]) + Fraction(vals[c + 1])) / 2
        got = int(oracle.e4m3_encode(np.array([float(mid)]))[0])
        assert float(mid) == mid                        # exactly representable in float64
        assert got == (c if c % 2 == 0 else c + 1), (c, float(mid), got)
        # just off the midpoint: the nearer value wins
        assert oracle.e4m3_encode(np.array([float(mid) * (1 - 2 ** -40)]))[0] == c
        assert oracle.e4m3_encode(np.array([float(mid) * (1 + 2 ** -40)]))[0] == c + 1


def test_e4m3_matches_torch_cast_in_range_and_saturates():
    rng = np.random.default_rng(6)
    x = np.concatenate([rng.standard_normal(20000) * 30, rng.standard_normal(2000) * 1e-2,
                        rng.uniform(-463.9, 463.9, 2000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_encode(x.astype(np.float64)), ref)
    assert list(oracle.e4m3_encode(np.array([464.0, 1e4, -1e9]))) == [0x7E, 0x7E, 0xFE]


def test_quantize_rows_scale_max_and_error_bound():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((64, 128)) * rng.uniform(0.01, 50, (64, 1))).astype(np.float32)
    x[3] = 0.0
    codes, s = oracle.quantize_rows(x)
    assert s[3] == 0 and not codes[3].any()
    deq = oracle.dequantize_rows(codes, s)
    rows = [r for r in range(64) if r != 3]
    for r in rows:
        j = int(np.argmax(np.abs(x[r])))
        assert codes[r, j] & 0x7F == 0x7E                # the largest element becomes +-448
        assert s[r] == np.float32(np.abs(x[r]).max() / np.float32(448.0))
    # relative error of a normal code is at most 2^-4 (half of the 2^-3 mantissa step),
    # plus the fp32 roundings of the scaling
    normal = np.abs(oracle.e4m3_decode(codes)) >= 2.0 ** -6
    err = np.abs(deq - x.astype(np.float64))
    assert np.all(err[normal] <= (2.0 ** -4 + 1e-6) * np.abs(x.astype(np.float64))[normal])


def test_fp8_fine_branch_close_to_full_precision_and_exact_on_representable_inputs():
    # inputs whose rows already are exact FP8 multiples of a power-of-two scale
    # (every |x| <= 448 * 2^-k on the E4M3 grid with the row max at 448 * 2^-k)
    # quantise without error, so the FP8 fine branch equals the bf16 one
    w = small_workload(D=32)
    x = make_inputs(w, seed=2)
    rng = np.random.default_rng(8)
    L, H, D = w.L, w.heads, w.head_dim
    codes = rng.integers(0, 126, (L, H, D)).astype(np.uint8) | rng.choice([0, 0x80], (L, H, D)).astype(np.uint8)
    codes[:, :, 0] = 0x7E
    qe = (oracle.e4m3_decode(codes) * 2.0 ** -6).astype(np.float32)
    codes2 = rng.integers(0, 126, (L, H, D)).astype(np.uint8)
    codes2[:, :, 5] = 0x7E
    ke = (oracle.e4m3_decode(codes2) * 2.0 ** -5).astype(np.float32)
    g = oracle.geometry(x["token_tags"], x["position_ids"], w.grid)
    topk = oracle.topk_count(g.NV, w.sparsity)
    for h in range(H):
        a = oracle.forward_head(qe, ke, x["v"], x["gate"], g, topk, h)
        b = oracle.forward_head(qe, ke, x["v"], x["gate"], g, topk, h, qk_fp8=True)
        assert np.array_equal(a.sel, b.sel)
        assert np.allclose(a.out, b.out, rtol=0, atol=1e-12)
    # and on N(0,1) inputs the FP8 branch stays within a few per cent of full precision
    r0 = oracle.forward_head(x["q"], x["k"], x["v"], x["gate"], g, topk, 0)
    r1 = oracle.forward_head(x["q"], x["k"], x["v"], x["gate"], g, topk, 0, qk_fp8=True)
    rel = np.linalg.norm(r1.out - r0.out) / np.linalg.norm(r0.out)
    assert 1e-4 < rel < 5e-2

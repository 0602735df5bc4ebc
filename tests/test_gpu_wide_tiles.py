"""GPU parity of 128-token tiles and the reference keep ratio against the oracle.

Bar as for the base method: pooled q/k/v and the selection (reference and
video tiles) bit-exact, the visit list and chunk offsets exact, the output
within max-abs 2e-2 and relative L2 5e-3.  Small layouts are compared on every
row; the full-size OmniRef layout runs in the benchmark's launch configuration
and is compared on sampled heads and query tiles.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import video_dit_block_amd as vsa
from tests.gpu_helpers import (assert_close, check_dispatch_order, errors, intermediates,
                               oracle_prep, out_f64, require_gpu, run, run_qk_prep, say)
from workloads import AUDIO, COND, TEXT, WORKLOADS, Workload, make_inputs, make_qk_prep_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _bf16_bits(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16).view(torch.int16)


def _expected_lists(g, ref_sel, sel):
    """Per video query tile: the visit list (fixed prefix tiles, selected
    reference tiles, selected video tiles, ascending) when reference tiles
    are selected, else the selected video tiles (prefix tiles are implicit)."""
    if ref_sel is None:
        return sel
    fixed = np.nonzero(g.tile_tag[:g.P] != COND)[0]
    return np.stack([np.sort(np.concatenate([fixed, ref_sel[i], sel[i]]))
                     for i in range(g.NV)]).astype(np.int32)


def _check_lists(plan, ws, g, lists_by_head):
    """The visit list (if any) and the chunk offsets over the fine branch's list."""
    H, NV = plan.heads, plan.num_video_tiles
    if plan.topk_ref > 0:
        V = lists_by_head[0].shape[1]
        got = plan.view(ws, "visit", torch.int32, (H, NV, V)).cpu().numpy()
        for h, want in lists_by_head.items():
            assert np.array_equal(got[h], want), f"visit list head {h}"
    if plan.num_chunks > 1 and NV:
        C = plan.num_chunks
        co = plan.view(ws, "chunk_offsets", torch.int32, (H, NV, C + 1)).cpu().numpy()
        bounds = np.minimum(np.arange(C + 1) * plan.chunk_tiles, plan.num_tiles)
        for h, lst in lists_by_head.items():
            want = (lst[:, :, None] < bounds[None, None, :]).sum(axis=1)
            assert np.array_equal(co[h], want), f"chunk offsets head {h}"
        if len(lists_by_head) == H:
            check_dispatch_order(plan, ws, co, 0 if plan.topk_ref > 0 else plan.num_prefix_tiles)


def wide_check(w: Workload, x, plan=None, heads=None, check_tiles=True, qk_fp8=False,
               chunk_tiles=0):
    out, sel, plan, ws = run(x, w.grid, w.sparsity, plan=plan, tile=w.tile,
                             ref_keep=w.ref_keep, qk_fp8=qk_fp8, chunk_tiles=chunk_tiles)
    H = w.heads
    heads = list(range(H)) if heads is None else heads
    g = oracle.geometry(x["token_tags"], x["position_ids"], w.grid, w.tile)
    topk = oracle.topk_count(g.NV, w.sparsity)
    nref = int(np.sum(g.tile_tag == COND))
    kr = oracle.ref_keep_count(nref, w.ref_keep) if w.ref_keep < 1 else 0
    assert (plan.topk, plan.topk_ref, plan.tile_tokens) == (topk, kr, g.tile_tokens)
    assert plan.num_blocks == g.Nt * g.tile_tokens // 64
    assert tuple(sel.shape) == (H, g.NV, kr + topk)
    inter = intermediates(plan, ws)
    sel_h = sel.cpu().numpy()
    got = out_f64(out)
    is_bf16 = w.io_dtype == "bf16"
    lists = {}
    for h in heads:
        r = oracle.forward_head(x["q"], x["k"], x["v"], x["gate"], g, topk, h,
                                qk_fp8=qk_fp8, ref_keep=w.ref_keep)
        assert np.array_equal(inter["qp"][h], r.qp), f"pooled q head {h}"
        assert np.array_equal(inter["kp"][h], r.kp), f"pooled k head {h}"
        assert np.array_equal(inter["vp"][h], r.vp), f"pooled v head {h}"
        want_sel = r.sel if r.ref_sel is None else np.concatenate([r.ref_sel, r.sel], axis=1)
        assert np.array_equal(sel_h[h], want_sel), f"selection head {h}"
        lists[h] = _expected_lists(g, r.ref_sel, r.sel)
        ma, _ = errors(inter["coarse"][h], r.c)
        assert ma < 1e-5 * max(1.0, float(np.abs(r.c).max())) + 1e-6, ("coarse", h, ma)
        ref = oracle.round_bf16_from_f64(r.out) if is_bf16 else r.out.astype(np.float32)
        assert_close(got[:, h, :], ref, f"out head {h}")
        if check_tiles and not qk_fp8:
            perm = g.perm().reshape(-1, 64)          # blocks of 64 slots
            kt_ref = torch.zeros((perm.shape[0], 64, w.head_dim), dtype=torch.int16)
            vt_ref = torch.zeros_like(kt_ref)
            for b in range(perm.shape[0]):
                idx = torch.as_tensor(perm[b][perm[b] >= 0])
                kt_ref[b, :len(idx)] = _bf16_bits(x["k"][idx, h])
                vt_ref[b, :len(idx)] = _bf16_bits(x["v"][idx, h])
            assert torch.equal(inter["kt"][h], kt_ref), f"K blocks head {h}"
            cols = [(p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1) for p in range(64)]
            vt_cols = vt_ref.transpose(1, 2)[:, :, cols]
            vt_halves = vt_cols.reshape(perm.shape[0], w.head_dim, 2, 32).permute(0, 2, 1, 3)
            assert torch.equal(inter["vt"][h], vt_halves), f"V^T blocks head {h}"
    _check_lists(plan, ws, g, lists)
    assert torch.isfinite(out).all()
    return out, sel, plan, ws


def test_omniref_small_full_parity():
    w = WORKLOADS["omniref_small"]
    say(f"case omniref_small: {w.description}")
    wide_check(w, make_inputs(w))


LAYOUTS = [
    # name, heads, D, io, prefix, grid, sparsity, tile, keep, order
    ("t484_keep1_f32_d64", 3, 64, "f32", ((TEXT, 70), (COND, 130), (AUDIO, 33)), (5, 9, 7),
     0.5, (4, 8, 4), 1.0, "shuffled"),
    ("t844_keep03_bf16", 4, 128, "bf16", ((COND, 300), (TEXT, 64), (COND, 65)), (9, 8, 12),
     0.6, (8, 4, 4), 0.3, "shuffled"),
    ("t288_keep05_d64", 8, 64, "bf16", ((TEXT, 10), (COND, 400)), (6, 16, 16), 0.8,
     (2, 8, 8), 0.5, "raster"),
    ("t444_keep02", 4, 128, "bf16", ((TEXT, 64), (COND, 600), (AUDIO, 40)), (8, 8, 12), 0.7,
     (4, 4, 4), 0.2, "shuffled"),
    ("t484_keep01_no_ref", 2, 128, "bf16", ((TEXT, 200), (AUDIO, 64)), (8, 8, 8), 0.5,
     (4, 8, 4), 0.1, "raster"),
    ("t484_keep_all_refs", 2, 128, "bf16", ((COND, 300),), (6, 8, 8), 0.5, (4, 8, 4), 0.99,
     "raster"),
    ("t484_s0_video_only", 2, 128, "bf16", (), (8, 16, 8), 0.0, (4, 8, 4), 1.0, "raster"),
    ("t484_single_short_tile", 2, 64, "f32", ((COND, 3),), (1, 2, 3), 0.5, (4, 8, 4), 0.5,
     "raster"),
]


@pytest.mark.parametrize("name,H,D,io,prefix,grid,s,tile,keep,order", LAYOUTS,
                         ids=[l[0] for l in LAYOUTS])
def test_wide_layouts_full_parity(name, H, D, io, prefix, grid, s, tile, keep, order):
    w = Workload(name, H, D, io, prefix, grid, s, tile=tile, ref_keep=keep)
    say(f"case {name}: L={w.L} heads={H} D={D} {io} grid={grid} s={s} tile={tile} "
        f"keep={keep} {order}")
    wide_check(w, make_inputs(w, seed=4, video_order=order))


CHUNKED = [("omniref_small", 1), ("omniref_small", 3), ("t844_keep03_bf16", 2),
           ("t484_s0_video_only", 5)]


@pytest.mark.parametrize("name,ch", CHUNKED, ids=[f"{n}-ch{c}" for n, c in CHUNKED])
def test_wide_key_chunks_match_oracle_and_single_launch(name, ch):
    if name in WORKLOADS:
        w = WORKLOADS[name]
        x = make_inputs(w, seed=6)
    else:
        _, H, D, io, prefix, grid, s, tile, keep, order = {l[0]: l for l in LAYOUTS}[name]
        w = Workload(name, H, D, io, prefix, grid, s, tile=tile, ref_keep=keep)
        x = make_inputs(w, seed=6, video_order=order)
    say(f"case {name}: chunk_tiles={ch}")
    out, sel, plan, _ = wide_check(w, x, chunk_tiles=ch)
    assert plan.num_chunks == -(-plan.num_tiles // ch)
    out1, sel1, single, _ = run(x, w.grid, w.sparsity, tile=w.tile, ref_keep=w.ref_keep,
                                chunk_tiles=plan.num_tiles)
    assert single.num_chunks == 1
    assert torch.equal(sel, sel1) and torch.equal(out, out1)


def test_omniref_small_fp8_qk_parity():
    w = WORKLOADS["omniref_small"]
    say("case omniref_small with FP8 q/k")
    wide_check(w, make_inputs(w, seed=2), qk_fp8=True)


FP8_WIDE = [
    # FP8 keys at head_dim 64 do not split over four waves: two-wave blocks
    ("d64_bf16_keep04", Workload("f64", 3, 64, "bf16", ((TEXT, 90), (COND, 300), (AUDIO, 20)),
                                 (6, 16, 12), 0.6, tile=(4, 8, 4), ref_keep=0.4), 0),
    ("d64_f32_chunked", Workload("f64c", 2, 64, "f32", ((COND, 200), (TEXT, 64)), (9, 8, 12),
                                 0.5, tile=(8, 4, 4), ref_keep=0.5), 3),
    ("d128_f32_keep1", Workload("f128", 2, 128, "f32", ((TEXT, 100), (AUDIO, 70)), (6, 9, 8),
                                0.5, tile=(2, 8, 8)), 0),
    ("d128_bf16_chunked", Workload("f128c", 4, 128, "bf16", ((TEXT, 64), (COND, 400)),
                                   (10, 16, 8), 0.7, tile=(4, 8, 4), ref_keep=0.3), 4),
]


@pytest.mark.parametrize("name,w,ch", FP8_WIDE, ids=[f[0] for f in FP8_WIDE])
def test_wide_fp8_qk_instances(name, w, ch):
    """FP8 q/k on 128-token tiles in each kernel instance: two-wave blocks at
    head_dim 64, four-wave tiles at 128, both I/O types, one and several key
    chunks."""
    say(f"case {name}: L={w.L} {w.io_dtype} D={w.head_dim} tile={w.tile} keep={w.ref_keep} "
        f"chunk_tiles={ch}")
    out, _, plan, _ = wide_check(w, make_inputs(w, seed=12, video_order="shuffled"),
                                 qk_fp8=True, chunk_tiles=ch)
    if ch:
        assert plan.num_chunks > 1


def test_wide_tiles_sparsity0_keep1_equals_dense_sdpa():
    w = Workload("dense", 2, 64, "f32", ((TEXT, 70), (COND, 140)), (6, 9, 8), 0.0,
                 tile=(4, 8, 4))
    x = make_inputs(w, seed=9)
    x["gate"] = torch.zeros_like(x["gate"])
    out, _, plan, _ = run(x, w.grid, 0.0, tile=w.tile)
    assert plan.topk == plan.num_video_tiles
    q, k, v = (x[n].to(torch.float64).permute(1, 0, 2)[None] for n in ("q", "k", "v"))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v)[0].permute(1, 0, 2).numpy()
    assert_close(out_f64(out), ref, "128-token tiles s=0 vs SDPA")


def test_fp8_zero_query_rows_in_partial_tiles():
    """A query row of zeros has an FP8 scale of 0 and all-zero logits: its
    softmax is uniform over the valid keys, also next to masked pad keys."""
    w = Workload("zq", 2, 128, "bf16", ((TEXT, 70), (AUDIO, 20)), (6, 5, 7), 0.5)
    x = make_inputs(w, seed=8)
    x["q"][::7] = 0
    wide_check(w, x, qk_fp8=True)


WIDE_PREP = [
    Workload("prep_d128_keep03", 4, 128, "bf16", ((TEXT, 90), (COND, 300), (AUDIO, 40)),
             (6, 16, 12), 0.6, tile=(4, 8, 4), ref_keep=0.3),
    Workload("prep_d64_f32", 2, 64, "f32", ((COND, 150), (TEXT, 64)), (9, 8, 8), 0.5,
             tile=(8, 4, 4), ref_keep=0.6),
]


@pytest.mark.parametrize("w", WIDE_PREP, ids=[w.name for w in WIDE_PREP])
def test_wide_tiles_with_qk_norm_rope(w):
    """QK-norm + RoPE fused into the gather of 128-token tiles: Qt and Kt per
    64-slot block bit-exact, pooled values over all 128 slots, selection with
    reference keep, and the output."""
    say(f"case {w.name} + qk prep: L={w.L} {w.io_dtype} D={w.head_dim} tile={w.tile}")
    x = make_inputs(w, seed=14, video_order="shuffled")
    prep = make_qk_prep_inputs(w, x["position_ids"], seed=14)
    out, sel, plan, ws = run_qk_prep(x, prep, w.grid, w.sparsity, tile=w.tile,
                                     ref_keep=w.ref_keep, chunk_tiles=3)
    assert plan.num_chunks > 1
    q2, k2 = oracle_prep(x, prep)
    g = oracle.geometry(x["token_tags"], x["position_ids"], w.grid, w.tile)
    topk = oracle.topk_count(g.NV, w.sparsity)
    H, D = w.heads, w.head_dim
    inter = intermediates(plan, ws)
    Nb = plan.num_blocks
    qt = plan.view(ws, "qt", torch.int16, (H, Nb, 64, D)).cpu()
    perm = g.perm().reshape(-1, 64)
    got = out_f64(out)
    sel_h = sel.cpu().numpy()
    for h in range(H):
        for name, x2, reg in (("Qt", q2, qt[h]), ("Kt", k2, inter["kt"][h])):
            src = torch.from_numpy(np.ascontiguousarray(x2[:, h, :])).to(torch.bfloat16)
            ref = torch.zeros((Nb, 64, D), dtype=torch.int16)
            for b in range(Nb):
                idx = perm[b][perm[b] >= 0]
                ref[b, :len(idx)] = src.view(torch.int16)[torch.as_tensor(idx)]
            assert torch.equal(reg, ref), f"{name} head {h}"
        r = oracle.forward_head(q2, k2, x["v"], x["gate"], g, topk, h, ref_keep=w.ref_keep)
        assert np.array_equal(inter["qp"][h], r.qp), f"pooled q head {h}"
        assert np.array_equal(inter["kp"][h], r.kp), f"pooled k head {h}"
        assert np.array_equal(sel_h[h], np.concatenate([r.ref_sel, r.sel], axis=1)), h
        ref = (oracle.round_bf16_from_f64(r.out) if w.io_dtype == "bf16"
               else r.out.astype(np.float32))
        assert_close(got[:, h, :], ref, f"out head {h}")


def test_wide_tiles_oneshot_equals_plan_forward():
    """The one-call form with a 128-cell box builds the same plan and gives
    the same output and selection, bit for bit."""
    w = WORKLOADS["omniref_small"].with_(ref_keep=1.0)
    x = make_inputs(w, seed=15)
    out1, sel1, plan, _ = run(x, w.grid, w.sparsity, tile=w.tile)
    xd = {n: x[n].cuda() for n in ("q", "k", "v", "gate")}
    nbytes = vsa.vsa_h3_oneshot_workspace_bytes(x["token_tags"], x["position_ids"], w.grid,
                                                w.tile, w.heads, w.head_dim, w.sparsity,
                                                vsa.VSA_BF16)
    assert nbytes == plan.workspace_bytes
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out2 = torch.empty_like(xd["q"])
    sel2 = torch.empty_like(sel1)
    vsa.vsa_h3_forward_oneshot(xd["q"].data_ptr(), xd["k"].data_ptr(), xd["v"].data_ptr(),
                               xd["gate"].data_ptr(), x["token_tags"].numpy(),
                               x["position_ids"].numpy(), w.heads, w.head_dim, w.grid,
                               w.sparsity, w.tile, vsa.VSA_BF16, out2.data_ptr(),
                               sel2.data_ptr(), ws.data_ptr(), nbytes,
                               torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(sel1, sel2)


# ----------------------------------------------------------------- full-size OmniRef layout
def test_omniref768p10s_sampled_parity():
    w = WORKLOADS["omniref768p10s"]
    heads = [0, 37]
    say(f"case omniref768p10s: {w.description}; oracle heads {heads}")
    x = make_inputs(w)
    out, sel, plan, ws = run(x, w.grid, w.sparsity, tile=w.tile, ref_keep=w.ref_keep)
    g = oracle.geometry(x["token_tags"], x["position_ids"], w.grid, w.tile)
    topk = oracle.topk_count(g.NV, w.sparsity)
    nref = int(np.sum(g.tile_tag == COND))
    kr = oracle.ref_keep_count(nref, w.ref_keep)
    assert (plan.topk, plan.topk_ref, plan.num_chunks > 1) == (topk, kr, True)
    sel_all = sel.cpu().numpy()
    assert sel_all.shape == (w.heads, g.NV, kr + topk)
    assert np.all(np.diff(sel_all, axis=2) > 0)
    ref_ids = set(np.nonzero(g.tile_tag == COND)[0].tolist())
    assert all(int(t) in ref_ids for t in np.unique(sel_all[:, :, :kr]))
    assert sel_all[:, :, kr:].min() >= g.P and sel_all.max() < g.Nt
    assert torch.isfinite(out).all()
    inter = intermediates(plan, ws)
    rng = np.random.default_rng(321)
    scale = 1.0 / math.sqrt(w.head_dim)
    lists = {}
    for h in heads:
        r = oracle.forward_head(x["q"], x["k"], x["v"], x["gate"], g, topk, h, with_fine=False,
                                ref_keep=w.ref_keep)
        assert np.array_equal(inter["qp"][h], r.qp), h
        assert np.array_equal(inter["kp"][h], r.kp), h
        assert np.array_equal(sel_all[h], np.concatenate([r.ref_sel, r.sel], axis=1)), h
        lists[h] = _expected_lists(g, r.ref_sel, r.sel)
        ma, _ = errors(inter["coarse"][h], r.c)
        assert ma < 1e-5 * max(1.0, float(np.abs(r.c).max())) + 1e-6, ("coarse", h, ma)
        short = [j for j in range(g.P, g.Nt) if g.valid[j] <= 64]
        items = sorted({0, g.P - 1, g.P, g.Nt - 1, short[0], short[-1],
                        *[int(v) for v in rng.choice(np.arange(g.P, g.Nt), 8, replace=False)]})
        q64 = oracle.to_f32(x["q"][:, h, :]).astype(np.float64)
        k64 = oracle.to_f32(x["k"][:, h, :]).astype(np.float64)
        v64 = oracle.to_f32(x["v"][:, h, :]).astype(np.float64)
        gate = oracle.to_f32(x["gate"][:, h, :]).astype(np.float64)
        got_rows, ref_rows = [], []
        for i in items:
            o = oracle.fine_item(q64, k64, v64, g, r.sel, i, scale, r.ref_sel)
            rows = g.tiles[i]
            ref_rows.append(oracle.round_bf16_from_f64(o + gate[rows] * r.c[i]))
            got_rows.append(out[torch.as_tensor(rows), h, :].to(torch.float64).cpu().numpy())
        assert_close(np.concatenate(got_rows), np.concatenate(ref_rows),
                     f"out head {h} ({len(items)} query tiles)")
    _check_lists(plan, ws, g, lists)

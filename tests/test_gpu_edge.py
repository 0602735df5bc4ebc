"""GPU edge cases through the C ABI against the CPU oracle: the largest plan
the kernels take (4,096 tiles per head), logits large enough to move the
running maximum often, exact score ties (the lower tile index wins), a
one-token video, and query tiles of at most 32 tokens (one of the query
item's two waves then holds only pad rows), also where no key tile has more
than 32 keys."""
import math

import numpy as np
import pytest
import torch

import oracle
import video_dit_block_amd as vsa
from tests.gpu_helpers import (F32_MAX_ABS, F32_REL_L2, assert_close, intermediates, out_f64,
                               require_gpu, run, say)
from workloads import TEXT, Workload, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def test_max_tiles_4096_sampled():
    # 64x64x64 video grid: 4,096 video tiles, no prefix; 262,144 tokens
    w = Workload("max4096", 2, 64, "bf16", (), (64, 64, 64), 0.95)
    say(f"case max tiles: L={w.L} heads=2 D=64 grid=(64,64,64) s=0.95")
    x = make_inputs(w, seed=4)
    out, sel, plan, ws = run(x, w.grid, w.sparsity)
    assert plan.num_tiles == 4096 and plan.topk == oracle.topk_count(4096, w.sparsity) == 205
    g = oracle.geometry(x["token_tags"], x["position_ids"], w.grid)
    inter = intermediates(plan, ws)
    sel_h = sel.cpu().numpy()
    rng = np.random.default_rng(9)
    scale = 1.0 / math.sqrt(w.head_dim)
    for h in range(2):
        r = oracle.forward_head(x["q"], x["k"], x["v"], x["gate"], g, plan.topk, h,
                                with_fine=False)
        assert np.array_equal(sel_h[h], r.sel), h
        assert np.array_equal(inter["qp"][h], r.qp), h
        q64 = oracle.to_f32(x["q"][:, h, :]).astype(np.float64)
        k64 = oracle.to_f32(x["k"][:, h, :]).astype(np.float64)
        v64 = oracle.to_f32(x["v"][:, h, :]).astype(np.float64)
        gate = oracle.to_f32(x["gate"][:, h, :]).astype(np.float64)
        got, ref = [], []
        for i in sorted(set([0, 4095] + list(rng.choice(4096, 6, replace=False)))):
            o = oracle.fine_item(q64, k64, v64, g, r.sel, int(i), scale)
            rows = g.tiles[int(i)]
            ref.append(oracle.round_bf16_from_f64(o + gate[rows] * r.c[int(i)]))
            got.append(out[torch.as_tensor(rows), h, :].to(torch.float64).cpu().numpy())
        assert_close(np.concatenate(got), np.concatenate(ref), f"out head {h}")


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_large_logits_move_the_running_max(io):
    # q, k scaled up: logits reach thousands, so the lazily raised running
    # maximum moves often and rescales O.  Both I/O types are held against the
    # oracle itself: with fp32 I/O the fine branch forms every product from
    # bf16 high and low parts, so its logits carry fp32-level error even here.
    w = Workload("large", 4, 128, io, ((TEXT, 100),), (8, 12, 12), 0.5)
    say(f"case large logits ({io})")
    x = make_inputs(w, seed=6, video_order="shuffled")
    L = w.L
    ramp = torch.linspace(0.5, 6.0, L).reshape(L, 1, 1)
    x["q"] = (x["q"].float() * 6.0 * ramp).to(x["q"].dtype)
    x["k"] = (x["k"].float() * 4.0 * ramp.flip(0)).to(x["k"].dtype)
    out, sel, plan, ws = run(x, w.grid, w.sparsity)
    assert torch.isfinite(out).all()
    ref = oracle.forward(x["q"], x["k"], x["v"], x["gate"], x["token_tags"], x["position_ids"],
                         w.grid, w.sparsity)
    for h in range(w.heads):
        assert np.array_equal(sel[h].cpu().numpy(), ref["heads"][h].sel), h
    # the logits do reach the thousands
    g, h0 = ref["geom"], ref["heads"][0]
    i = g.P + 3
    q64 = oracle.to_f32(x["q"][:, 0, :]).astype(np.float64)[g.tiles[i]]
    k64 = oracle.to_f32(x["k"][:, 0, :]).astype(np.float64)
    keys = np.concatenate([g.tiles[j] for j in oracle.key_tiles(g, h0.sel, i)])
    assert np.abs(q64 @ k64[keys].T).max() / math.sqrt(w.head_dim) > 1000.0
    assert_close(out_f64(out), ref["out"], "large logits")


def test_exact_score_ties_lower_tile_wins():
    # every video tile holds the same k rows (so every pooled k and every
    # score ties) except a few that are scaled up; the kept set is the scaled
    # ones plus the lowest-indexed of the tied rest
    w = Workload("ties", 2, 64, "f32", ((TEXT, 64),), (8, 8, 16), 0.5)   # 1 + 16 tiles, topk 8
    say("case exact score ties")
    x = make_inputs(w, seed=7)
    g = oracle.geometry(x["token_tags"], x["position_ids"], w.grid)
    base = x["k"][g.tiles[g.P]].clone()
    for j in range(g.P, g.Nt):
        x["k"][torch.as_tensor(g.tiles[j])] = base
    boosted = [g.P + 3, g.P + 11, g.P + 14]
    for j in boosted:
        x["k"][torch.as_tensor(g.tiles[j])] = base * 2.0
    out, sel, plan, ws = run(x, w.grid, w.sparsity)
    ref = oracle.forward(x["q"], x["k"], x["v"], x["gate"], x["token_tags"], x["position_ids"],
                         w.grid, w.sparsity)
    sel_h = sel.cpu().numpy()
    for h in range(w.heads):
        assert np.array_equal(sel_h[h], ref["heads"][h].sel), h
        row_sets = {tuple(r) for r in sel_h[h]}
        assert len(row_sets) <= 2          # every query tile ties the same way up to sign of q.k
    assert_close(out_f64(out), ref["out"], "ties")


def test_one_token_video():
    w = Workload("one", 2, 64, "f32", ((TEXT, 3),), (1, 1, 1), 0.5)
    x = make_inputs(w, seed=8)
    out, sel, plan, ws = run(x, w.grid, w.sparsity)
    assert (plan.num_tiles, plan.topk) == (2, 1)
    ref = oracle.forward(x["q"], x["k"], x["v"], x["gate"], x["token_tags"], x["position_ids"],
                         w.grid, w.sparsity)
    assert np.array_equal(sel.cpu().numpy()[:, :, 0], np.full((2, 1), 1))
    assert_close(out_f64(out), ref["out"], "one-token video")


SHORT_CASES = [
    # every tile holds 32 tokens: no key tile has a second half
    (Workload("short_all32", 4, 128, "bf16", (), (2, 8, 12), 0.5), 2),
    (Workload("short_all32_f32", 2, 64, "f32", (), (2, 8, 12), 0.5), 3),
    # a text prefix plus a last tile row of 2 frames: 32-token query tiles
    # meet key tiles of 64 and of 32 tokens
    (Workload("short_mixed", 4, 128, "bf16", ((TEXT, 64),), (6, 8, 12), 0.6), 4),
    # a last tile row of 1 frame: 16-token query tiles, pad keys in the first half
    (Workload("short_16", 2, 128, "bf16", ((TEXT, 40),), (5, 8, 8), 0.5), 3),
]


@pytest.mark.parametrize("w,ch", SHORT_CASES, ids=[c[0].name for c in SHORT_CASES])
def test_query_tiles_of_at_most_32_tokens(w, ch):
    say(f"case {w.name}: grid={w.grid} {w.io_dtype}, and chunk_tiles={ch}")
    x = make_inputs(w, seed=12, video_order="shuffled")
    out, sel, plan, ws = run(x, w.grid, w.sparsity)
    ref = oracle.forward(x["q"], x["k"], x["v"], x["gate"], x["token_tags"], x["position_ids"],
                         w.grid, w.sparsity)
    g = ref["geom"]
    assert any(len(t) <= 32 for t in g.tiles[g.P:])
    for h in range(w.heads):
        assert np.array_equal(sel[h].cpu().numpy(), ref["heads"][h].sel), h
    if w.io_dtype == "bf16":
        assert_close(out_f64(out), ref["out"], w.name)
    else:
        assert_close(out_f64(out), ref["out"], w.name, F32_MAX_ABS, F32_REL_L2)
    # key chunks pass the running state on bit for bit
    chunked = vsa.Plan(x["token_tags"], x["position_ids"], w.grid, w.heads, w.head_dim,
                       w.sparsity, chunk_tiles=ch, io_dtype=x["q"].dtype)
    assert chunked.num_chunks > 1
    out2, sel2, _, _ = run(x, w.grid, w.sparsity, plan=chunked)
    assert torch.equal(sel2, sel)
    assert torch.equal(out2, out)


def _crafted_scores_inputs(values_per_head, seed):
    """fp32 inputs whose pooled video-tile scores are exactly the given values:
    every video query row is e0 (so each pooled query is e0); in video tile j
    the first key row is 64 * values[h][j] * e0 and the other rows are zero, so
    the fixed-order sum is exact and the pooled key is values[h][j] * e0, and
    the fixed-order score of any video query tile against it is values[h][j]
    (a product of +-0 adds to the +0 start as +0)."""
    H = len(values_per_head)
    w = Workload("crafted", H, 64, "f32", ((TEXT, 64),), (8, 8, 16), 0.5)   # 1 + 16 tiles, topk 8
    x = make_inputs(w, seed=seed)
    g = oracle.geometry(x["token_tags"], x["position_ids"], w.grid)
    assert g.NV == 16
    for j in range(g.P, g.Nt):
        rows = torch.as_tensor(g.tiles[j])
        x["q"][rows] = 0.0
        x["q"][rows, :, 0] = 1.0
        x["k"][rows] = 0.0
        for h in range(H):
            x["k"][rows[0], h, 0] = 64.0 * float(values_per_head[h][j - g.P])
    return w, x, g


def test_topk_ties_straddling_the_kth_rank_low_bit_decisions_and_zero_scores():
    """Selections decided by the top-k kernel's hardest cases: a cluster of
    equal scores straddling the k-th rank (lower indices win), the k-th and
    (k+1)-th scores differing only in the last bit of the fp32 mantissa (the
    bitwise search reaches count == k only there), every score equal, and a
    cluster of zero scores (from keys of either sign of zero) around the k-th
    rank."""
    u = 2.0 ** -23
    perm = np.random.default_rng(3).permutation(16)
    vals = [
        # 2 scores of 3, then 7 of 2 at scattered indices: 6 of the 2s fit
        [2, 1, 3, 2, 0.5, 2, 1, 2, 3, 2, -1, 2, 0.25, 2, 1, 0],
        # 1 + m*2^-23 for m = 13..28: kept m = 21..28; 21 and 20 differ in bit 0 only
        [1.0 + (13 + int(m)) * u for m in perm],
        # all equal: the 8 lowest indices
        [1.5] * 16,
        # 10 zeros of either sign, 6 negatives: the 8 lowest-indexed zeros
        [-0.0, 0.0, -1, 0.0, -0.0, -2, 0.0, -0.5, -0.0, 0.0, -3, -0.0, 0.0, -0.25, -4, -8],
    ]
    w, x, g = _crafted_scores_inputs(vals, seed=17)
    out, sel, plan, ws = run(x, w.grid, w.sparsity)
    ref = oracle.forward(x["q"], x["k"], x["v"], x["gate"], x["token_tags"], x["position_ids"],
                         w.grid, w.sparsity)
    inter = intermediates(plan, ws)
    want = [
        [0, 2, 3, 5, 7, 8, 9, 11],
        sorted(int(j) for j in np.nonzero(perm + 13 >= 21)[0]),
        list(range(8)),
        [0, 1, 3, 4, 6, 8, 9, 11],
    ]
    # the k-th and (k+1)-th scores of head 1 differ in the last mantissa bit only
    top = np.sort(np.float32(vals[1]))[::-1]
    assert int(top[7].view(np.uint32)) ^ int(top[8].view(np.uint32)) == 1
    sel_h = sel.cpu().numpy()
    for h in range(w.heads):
        assert np.array_equal(inter["kp"][h, g.P:, 0], np.float32(vals[h])), h
        assert np.array_equal(ref["heads"][h].sel[0], np.array(want[h]) + g.P), h   # oracle
        assert np.array_equal(sel_h[h], ref["heads"][h].sel), h                     # GPU
        assert (sel_h[h] == sel_h[h][0]).all(), h     # every query tile ties the same way
    assert_close(out_f64(out), ref["out"], "crafted scores", F32_MAX_ABS, F32_REL_L2)

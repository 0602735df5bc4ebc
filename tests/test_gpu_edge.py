"""GPU edge cases through the C ABI against the CPU oracle: the largest plan
the kernels take (4,096 tiles per head), logits large enough to move the
running maximum often, exact score ties (the lower tile index wins), and a
one-token video."""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import assert_close, intermediates, out_f64, require_gpu, run, say
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
    # maximum moves often and rescales O.  With fp32 I/O the fine branch's MFMA
    # operands are q, k, v rounded to bf16 (nearest even), which at these
    # logits moves the softmax weights by far more than the bar; that case is
    # held against the oracle's fine branch fed the same bf16-rounded operands
    # (selection and coarse branch stay fp32 on both sides)
    w = Workload("large", 4, 128, io, ((TEXT, 100),), (8, 12, 12), 0.5)
    say(f"case large logits ({io})")
    x = make_inputs(w, seed=6, video_order="shuffled")
    L = w.L
    ramp = torch.linspace(0.5, 6.0, L).reshape(L, 1, 1)
    x["q"] = (x["q"].float() * 6.0 * ramp).to(x["q"].dtype)
    x["k"] = (x["k"].float() * 4.0 * ramp.flip(0)).to(x["k"].dtype)
    out, sel, plan, ws = run(x, w.grid, w.sparsity)
    assert torch.isfinite(out).all()
    g = oracle.geometry(x["token_tags"], x["position_ids"], w.grid)
    topk = oracle.topk_count(g.NV, w.sparsity)
    scale = 1.0 / math.sqrt(w.head_dim)
    ref = np.empty((L, w.heads, w.head_dim))
    for h in range(w.heads):
        r = oracle.forward_head(x["q"], x["k"], x["v"], x["gate"], g, topk, h, with_fine=False)
        assert np.array_equal(sel[h].cpu().numpy(), r.sel), h
        q64, k64, v64 = (oracle.to_f32(x[n][:, h, :].to(torch.bfloat16)).astype(np.float64)
                         for n in ("q", "k", "v"))
        o = oracle.fine(q64, k64, v64, g, r.sel, scale)
        full = oracle.combine(o, oracle.to_f32(x["gate"][:, h, :]), r.c, g)
        ref[:, h, :] = (oracle.round_bf16_from_f64(full) if io == "bf16"
                        else full.astype(np.float32).astype(np.float64))
    assert_close(out_f64(out), ref, "large logits")


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

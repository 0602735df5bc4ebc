"""GPU parity of the forward with QK RMS norm + RoPE fused into the tile
gather, through the C ABI, against the CPU oracle.

Bar: the normalised, rotated q and k in tile order (Qt, Kt), the pooled
q/k/v and the selection bit-exact; the output within max-abs 2e-2 and
relative L2 5e-3.  Norm weights, eps and cos/sin tables are synthetic (the H3
values are not published).
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import (assert_close, check_all_heads_selection, errors, intermediates,
                               oracle_prep, out_f64,
                               require_gpu, run_qk_prep, say)
from workloads import AUDIO, COND, TEXT, WORKLOADS, Workload, make_inputs, make_qk_prep_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _tile_bits(x2, g, h, D):
    """bf16 bits of x2[:, h, :] gathered into tile order, pad rows zero."""
    perm = g.perm()
    ref = torch.zeros((g.Nt, 64, D), dtype=torch.int16)
    src = torch.from_numpy(np.ascontiguousarray(x2[:, h, :])).to(torch.bfloat16).view(torch.int16)
    for j in range(g.Nt):
        idx = perm[j][perm[j] >= 0]
        ref[j, :len(idx)] = src[torch.as_tensor(idx)]
    return ref


def prep_check(w, x, prep, sparsity, heads=None, check_tiles=True, chunk_tiles=0):
    out, sel, plan, ws = run_qk_prep(x, prep, w.grid, sparsity, chunk_tiles=chunk_tiles)
    q2, k2 = oracle_prep(x, prep)
    g = oracle.geometry(x["token_tags"], x["position_ids"], w.grid)
    topk = oracle.topk_count(g.NV, sparsity)
    H, D = w.heads, w.head_dim
    heads = list(range(H)) if heads is None else heads
    inter = intermediates(plan, ws)
    qt = plan.view(ws, "qt", torch.int16, (H, g.Nt, 64, D)).cpu()
    sel_h = sel.cpu().numpy()
    got = out_f64(out)
    for h in heads:
        r = oracle.forward_head(q2, k2, x["v"], x["gate"], g, topk, h)
        if check_tiles:
            assert torch.equal(qt[h], _tile_bits(q2, g, h, D)), f"Qt head {h}"
            assert torch.equal(inter["kt"][h], _tile_bits(k2, g, h, D)), f"Kt head {h}"
        assert np.array_equal(inter["qp"][h], r.qp), f"pooled q head {h}"
        assert np.array_equal(inter["kp"][h], r.kp), f"pooled k head {h}"
        assert np.array_equal(inter["vp"][h], r.vp), f"pooled v head {h}"
        assert np.array_equal(sel_h[h], r.sel), f"selection head {h}"
        ma, _ = errors(inter["coarse"][h], r.c)
        assert ma < 1e-5 * max(1.0, float(np.abs(r.c).max())) + 1e-6, ("coarse", h, ma)
        ref = (oracle.round_bf16_from_f64(r.out) if w.io_dtype == "bf16"
               else r.out.astype(np.float32))
        assert_close(got[:, h, :], ref, f"out head {h}")
    return out, sel, plan


def test_qk_prep_tiny_fp32_full():
    w = WORKLOADS["tiny"]
    x = make_inputs(w)
    prep = make_qk_prep_inputs(w, x["position_ids"])
    say(f"case tiny + qk prep: {w.description}")
    prep_check(w, x, prep, w.sparsity)


PREP_LAYOUTS = [
    # name, heads, D, io, prefix, grid, sparsity, order, chunk_tiles
    ("odd_bf16_d128_h8", 8, 128, "bf16", ((TEXT, 130), (AUDIO, 64)), (9, 10, 11), 0.7, "shuffled", 0),
    ("odd_f32_d64_h3", 3, 64, "f32", ((TEXT, 70), (COND, 20), (AUDIO, 33)), (5, 6, 7), 0.5,
     "shuffled", 0),
    ("video_only_h8_ch3", 8, 128, "bf16", (), (8, 8, 16), 0.6, "raster", 3),
    ("prefix_only_h2", 2, 128, "bf16", ((TEXT, 100), (AUDIO, 77)), (0, 0, 0), 0.5, "raster", 0),
]


@pytest.mark.parametrize("name,H,D,io,prefix,grid,s,order,ch", PREP_LAYOUTS,
                         ids=[l[0] for l in PREP_LAYOUTS])
def test_qk_prep_layouts_full(name, H, D, io, prefix, grid, s, order, ch):
    w = Workload(name, H, D, io, prefix, grid, s)
    say(f"case {name} + qk prep: L={w.L} heads={H} D={D} {io} grid={grid} s={s} chunk_tiles={ch}")
    x = make_inputs(w, seed=9, video_order=order)
    prep = make_qk_prep_inputs(w, x["position_ids"], seed=9)
    prep_check(w, x, prep, s, chunk_tiles=ch)


def test_qk_prep_480p5s_selection_all_heads():
    w = WORKLOADS["480p5s"]
    say(f"case 480p5s + qk prep: {w.description}")
    x = make_inputs(w)
    prep = make_qk_prep_inputs(w, x["position_ids"])
    out, sel, plan = prep_check(w, x, prep, w.sparsity, heads=[0, 31], check_tiles=False)
    q2, k2 = oracle_prep(x, prep)
    g = oracle.geometry(x["token_tags"], x["position_ids"], w.grid)
    sel_h = sel.cpu().numpy()
    for h in range(w.heads):
        r = oracle.forward_head(q2, k2, x["v"], x["gate"], g, plan.topk, h, with_fine=False)
        assert np.array_equal(sel_h[h], r.sel), h


def test_qk_prep_768p10s_sampled():
    w = WORKLOADS["768p10s"]
    say(f"case 768p10s + qk prep: {w.description}; oracle heads 0, 41")
    x = make_inputs(w)
    prep = make_qk_prep_inputs(w, x["position_ids"])
    out, sel, plan, ws = run_qk_prep(x, prep, w.grid, w.sparsity)
    assert plan.num_chunks > 1
    g = oracle.geometry(x["token_tags"], x["position_ids"], w.grid)
    inter = intermediates(plan, ws)
    sel_all = sel.cpu().numpy()
    # every head: the prepared q/k's pooled values and the selection, bit for bit
    check_all_heads_selection(x["q"], x["k"], g, plan.topk, inter["qp"], inter["kp"], sel_all,
                              prep=prep)
    import math
    rng = np.random.default_rng(5)
    for h in (0, 41):
        # the oracle's prepared q/k for this head only (the full prep is slow)
        qh = oracle.to_f32(x["q"][:, h, :])
        kh = oracle.to_f32(x["k"][:, h, :])
        q2 = oracle.round_bf16_from_f64(oracle.qk_norm_rope(
            qh, prep["q_weight"].numpy(), prep["eps"], prep["cos"].numpy(),
            prep["sin"].numpy()).astype(np.float64)).astype(np.float32)
        k2 = oracle.round_bf16_from_f64(oracle.qk_norm_rope(
            kh, prep["k_weight"].numpy(), prep["eps"], prep["cos"].numpy(),
            prep["sin"].numpy()).astype(np.float64)).astype(np.float32)
        qp = oracle.pool_canonical(q2, g)
        kp = oracle.pool_canonical(k2, g)
        assert np.array_equal(inter["qp"][h], qp), h
        assert np.array_equal(inter["kp"][h], kp), h
        S = oracle.scores_canonical(qp, kp)
        ref_sel = oracle.select_topk(S, g, plan.topk)
        assert np.array_equal(sel_all[h], ref_sel), h
        vh = oracle.to_f32(x["v"][:, h, :]).astype(np.float64)
        gate = oracle.to_f32(x["gate"][:, h, :]).astype(np.float64)
        c = oracle.coarse(S, oracle.pool_canonical(oracle.to_f32(x["v"][:, h, :]), g),
                          1.0 / math.sqrt(w.head_dim))
        items = [0, g.P - 1, g.P, g.Nt - 1] + list(rng.choice(np.arange(g.P, g.Nt), 6,
                                                             replace=False))
        got_rows, ref_rows = [], []
        for i in sorted(set(int(t) for t in items)):
            o = oracle.fine_item(q2.astype(np.float64), k2.astype(np.float64), vh, g, ref_sel, i,
                                 1.0 / math.sqrt(w.head_dim))
            rows = g.tiles[i]
            ref_rows.append(oracle.round_bf16_from_f64(o + gate[rows] * c[i]))
            got_rows.append(out[torch.as_tensor(rows), h, :].to(torch.float64).cpu().numpy())
        assert_close(np.concatenate(got_rows), np.concatenate(ref_rows), f"out head {h}")

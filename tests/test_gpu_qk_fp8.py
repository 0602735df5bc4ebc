"""GPU parity of the forward with per-token FP8 (OCP E4M3) q and k in the fine
branch, through the C ABI, against the CPU oracle's FP8 mode.

Bar: the E4M3 key codes and per-key scales bit-exact; pooled q/k/v and the
selection bit-exact (unchanged by the mode); the output within max-abs 2e-2
and relative L2 5e-3 of the oracle's FP8 fine branch.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import (assert_close, check_all_heads_selection, errors, intermediates, key_rows,
                               oracle_prep, out_f64,
                               require_gpu, run, run_qk_prep, say)
from workloads import AUDIO, COND, TEXT, WORKLOADS, Workload, make_inputs, make_qk_prep_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _check_key_codes(plan, ws, k32, g, h, D):
    """kt8/kscale of head h against the oracle's per-row quantisation."""
    H, Nt = plan.heads, plan.num_tiles
    codes = key_rows(plan.view(ws, "kt8", torch.uint8, (H, Nt, 64 * D)).cpu(), D, 64)[h].numpy()
    scale = plan.view(ws, "kscale", torch.float32, (H, Nt, 64))[h].cpu().numpy()
    perm = g.perm()
    want_c = np.zeros((Nt, 64, D), np.uint8)
    want_s = np.zeros((Nt, 64), np.float32)
    rc, rs = oracle.quantize_rows(k32)
    for j in range(Nt):
        idx = perm[j][perm[j] >= 0]
        want_c[j, :len(idx)] = rc[idx]
        want_s[j, :len(idx)] = rs[idx]
    assert np.array_equal(codes, want_c), f"E4M3 key codes head {h}"
    assert np.array_equal(scale, want_s), f"key scales head {h}"


def fp8_check(w, x, sparsity, heads=None, chunk_tiles=0, q_in=None, k_in=None, out_sel=None):
    if out_sel is None:
        out, sel, plan, ws = run(x, w.grid, sparsity, qk_fp8=True, chunk_tiles=chunk_tiles)
    else:
        out, sel, plan, ws = out_sel
    q_in = x["q"] if q_in is None else q_in
    k_in = x["k"] if k_in is None else k_in
    g = oracle.geometry(x["token_tags"], x["position_ids"], w.grid)
    topk = oracle.topk_count(g.NV, sparsity)
    H, D = w.heads, w.head_dim
    heads = list(range(H)) if heads is None else heads
    inter = intermediates(plan, ws)
    sel_h = sel.cpu().numpy()
    got = out_f64(out)
    for h in heads:
        r = oracle.forward_head(q_in, k_in, x["v"], x["gate"], g, topk, h, qk_fp8=True)
        _check_key_codes(plan, ws, oracle.to_f32(k_in[:, h, :]), g, h, D)
        assert np.array_equal(inter["qp"][h], r.qp), f"pooled q head {h}"
        assert np.array_equal(inter["kp"][h], r.kp), f"pooled k head {h}"
        assert np.array_equal(sel_h[h], r.sel), f"selection head {h}"
        ref = (oracle.round_bf16_from_f64(r.out) if w.io_dtype == "bf16"
               else r.out.astype(np.float32))
        assert_close(got[:, h, :], ref, f"out head {h} (FP8 q/k)")
    return out, sel, plan


def test_qk_fp8_tiny_fp32_full():
    w = WORKLOADS["tiny"]
    say(f"case tiny + FP8 q/k: {w.description}")
    fp8_check(w, make_inputs(w), w.sparsity)


FP8_LAYOUTS = [
    # name, heads, D, io, prefix, grid, sparsity, order, chunk_tiles
    ("odd_bf16_d128_h8", 8, 128, "bf16", ((TEXT, 130), (AUDIO, 64)), (9, 10, 11), 0.7, "shuffled", 0),
    ("odd_f32_d64_h3", 3, 64, "f32", ((TEXT, 70), (COND, 20), (AUDIO, 33)), (5, 6, 7), 0.5,
     "shuffled", 0),
    ("video_only_h8_ch3", 8, 128, "bf16", (), (8, 8, 16), 0.6, "raster", 3),
    ("prefix_only_h2", 2, 128, "bf16", ((TEXT, 100), (AUDIO, 77)), (0, 0, 0), 0.5, "raster", 0),
    ("d64_bf16_h4_s0", 4, 64, "bf16", ((TEXT, 64),), (8, 8, 12), 0.0, "raster", 2),
]


@pytest.mark.parametrize("name,H,D,io,prefix,grid,s,order,ch", FP8_LAYOUTS,
                         ids=[l[0] for l in FP8_LAYOUTS])
def test_qk_fp8_layouts_full(name, H, D, io, prefix, grid, s, order, ch):
    w = Workload(name, H, D, io, prefix, grid, s)
    say(f"case {name} + FP8 q/k: L={w.L} heads={H} D={D} {io} grid={grid} s={s} chunk_tiles={ch}")
    fp8_check(w, make_inputs(w, seed=11, video_order=order), s, chunk_tiles=ch)


def test_qk_fp8_with_qk_prep():
    w = Workload("prep_fp8", 4, 128, "bf16", ((TEXT, 100),), (8, 12, 12), 0.6)
    say("case QK-norm + RoPE with FP8 q/k")
    x = make_inputs(w, seed=12, video_order="shuffled")
    prep = make_qk_prep_inputs(w, x["position_ids"], seed=12)
    plan_ = None
    import video_dit_block_amd as vsa
    plan_ = vsa.Plan(x["token_tags"], x["position_ids"], w.grid, w.heads, w.head_dim, w.sparsity,
                     qk_prep=True, qk_fp8=True)
    res = run_qk_prep(x, prep, w.grid, w.sparsity, plan=plan_)
    q2, k2 = oracle_prep(x, prep)
    fp8_check(w, x, w.sparsity, q_in=q2, k_in=k2, out_sel=res)


def test_qk_fp8_768p10s_sampled():
    w = WORKLOADS["768p10s"]
    say(f"case 768p10s + FP8 q/k: {w.description}; oracle heads 0, 50")
    x = make_inputs(w)
    out, sel, plan, ws = run(x, w.grid, w.sparsity, qk_fp8=True)
    assert plan.num_chunks > 1
    g = oracle.geometry(x["token_tags"], x["position_ids"], w.grid)
    topk = plan.topk
    inter = intermediates(plan, ws)
    sel_all = sel.cpu().numpy()
    # every head: pooled q/k and the selection, bit for bit (FP8 touches neither)
    check_all_heads_selection(x["q"], x["k"], g, topk, inter["qp"], inter["kp"], sel_all)
    rng = np.random.default_rng(3)
    scale = 1.0 / math.sqrt(w.head_dim)
    for h in (0, 50):
        r = oracle.forward_head(x["q"], x["k"], x["v"], x["gate"], g, topk, h, with_fine=False)
        assert np.array_equal(sel_all[h], r.sel), h
        assert np.array_equal(inter["qp"][h], r.qp), h
        kh = oracle.to_f32(x["k"][:, h, :])
        _check_key_codes(plan, ws, kh, g, h, w.head_dim)
        q8 = oracle.dequantize_rows(*oracle.quantize_rows(oracle.to_f32(x["q"][:, h, :])))
        k8 = oracle.dequantize_rows(*oracle.quantize_rows(kh))
        q64 = oracle.to_f32(x["q"][:, h, :]).astype(np.float64)
        k64 = kh.astype(np.float64)
        v64 = oracle.to_f32(x["v"][:, h, :]).astype(np.float64)
        gate = oracle.to_f32(x["gate"][:, h, :]).astype(np.float64)
        items = [0, g.P, g.Nt - 1] + list(rng.choice(np.arange(g.P, g.Nt), 6, replace=False))
        got_rows, ref_rows, full_rows = [], [], []
        for i in sorted(set(int(t) for t in items)):
            rows = g.tiles[i]
            o8 = oracle.fine_item(q8, k8, v64, g, r.sel, i, scale)
            o = oracle.fine_item(q64, k64, v64, g, r.sel, i, scale)
            ref_rows.append(oracle.round_bf16_from_f64(o8 + gate[rows] * r.c[i]))
            full_rows.append(o + gate[rows] * r.c[i])
            got_rows.append(out[torch.as_tensor(rows), h, :].to(torch.float64).cpu().numpy())
        got = np.concatenate(got_rows)
        assert_close(got, np.concatenate(ref_rows), f"out head {h} (FP8 q/k)")
        ma, rl = errors(got, np.concatenate(full_rows))
        say(f"  head {h}: FP8 q/k vs full-precision q/k: max_abs={ma:.3e} rel_l2={rl:.3e}")
        assert rl < 5e-2

"""Shared helpers of the GPU parity tests (imported by tests only)."""
from __future__ import annotations

import math
import sys

import numpy as np
import torch

import oracle
import video_dit_block_amd as vsa

# Acceptance bar for the floating-point output (bf16 I/O, fp32 accumulation):
# max-abs 2e-2 and relative L2 5e-3 against the oracle.  Coarse intermediates
# are fp32 on both sides; the pooled q/k/v and the selection are bit-exact.
MAX_ABS = 2e-2
REL_L2 = 5e-3
# fp32 I/O at ordinary logits: every product of the fine branch is formed from
# bf16 high and low parts (relative error about 2^-16 per product, fp32 sums),
# so the output carries fp32-level error, far inside the bf16 bar above.
F32_MAX_ABS = 1e-4
F32_REL_L2 = 2e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def require_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def to_dev(x, dev="cuda"):
    return {k: (v.to(dev) if k in ("q", "k", "v", "gate") else v) for k, v in x.items()}


def run(x, grid, sparsity, dev="cuda", plan=None, qk_fp8=False, chunk_tiles=0,
        tile=(4, 4, 4), ref_keep=1.0):
    """GPU forward through the C ABI.  Returns (out, sel, plan, workspace)."""
    xd = {k: x[k].to(dev) for k in ("q", "k", "v", "gate")}
    L, H, D = xd["q"].shape
    if plan is None:
        plan = vsa.Plan(x["token_tags"], x["position_ids"], grid, H, D, sparsity, tile,
                        chunk_tiles=chunk_tiles, qk_fp8=qk_fp8, ref_keep=ref_keep,
                        io_dtype=x["q"].dtype)
    out, sel = vsa.forward(xd["q"], xd["k"], xd["v"], xd["gate"], plan=plan, return_sel=True)
    torch.cuda.synchronize()
    ws = plan.workspace(xd["q"].device)
    return out, sel, plan, ws


def run_qk_prep(x, prep, grid, sparsity, dev="cuda", plan=None, chunk_tiles=0,
                tile=(4, 4, 4), ref_keep=1.0):
    """GPU forward with QK-norm + RoPE through the C ABI.  Returns (out, sel, plan, ws)."""
    xd = {k: x[k].to(dev) for k in ("q", "k", "v", "gate")}
    pd = {k: prep[k].to(dev) for k in ("q_weight", "k_weight", "cos", "sin")}
    L, H, D = xd["q"].shape
    if plan is None:
        plan = vsa.Plan(x["token_tags"], x["position_ids"], grid, H, D, sparsity, tile,
                        chunk_tiles=chunk_tiles, qk_prep=True, ref_keep=ref_keep,
                        io_dtype=x["q"].dtype)
    out, sel = vsa.forward_qk_prep(xd["q"], xd["k"], xd["v"], xd["gate"], pd["q_weight"],
                                   pd["k_weight"], prep["eps"], pd["cos"], pd["sin"], plan=plan,
                                   return_sel=True)
    torch.cuda.synchronize()
    ws = plan.workspace(xd["q"].device)
    return out, sel, plan, ws


def oracle_prep(x, prep):
    """The oracle's attention inputs q', k' (float32 numpy [L, H, D])."""
    return oracle.prep_qk(x["q"], x["k"], prep["q_weight"].numpy(), prep["k_weight"].numpy(),
                          prep["eps"], prep["cos"].numpy(), prep["sin"].numpy())


def key_rows(region: torch.Tensor, D: int, group: int) -> torch.Tensor:
    """Key blocks [H][Nb][64][D] from the Kt layout (also that of Kt_lo and the
    FP8 codes Kt8): per 64-slot block, each 32-slot half is stored as
    [D / group][32 slots][group], group elements being 64 bytes of a row (32
    bf16 channels or 64 FP8 codes).  region: the raw region as [H][Nb][64 * D]."""
    H, Nb = region.shape[0], region.shape[1]
    g = region.reshape(H, Nb, 2, D // group, 32, group)
    return g.permute(0, 1, 2, 4, 3, 5).reshape(H, Nb, 64, D)


def intermediates(plan, ws):
    """Workspace regions on the host; kt and vt are per 64-slot block (kt
    returned as rows [H][Nb][64][D])."""
    H, D, Nt, Nb = plan.heads, plan.head_dim, plan.num_tiles, plan.num_blocks
    ns = plan.layout.scores_row_stride
    return {
        "qp": plan.view(ws, "qp", torch.float32, (H, Nt, D)).cpu().numpy(),
        "kp": plan.view(ws, "kp", torch.float32, (H, Nt, D)).cpu().numpy(),
        "vp": plan.view(ws, "vp", torch.float32, (H, Nt, D)).cpu().numpy(),
        "coarse": plan.view(ws, "coarse", torch.float32, (H, Nt, D)).cpu().numpy(),
        "kt": key_rows(plan.view(ws, "kt", torch.int16, (H, Nb, 64 * D)).cpu(), D, 32),
        "vt": plan.view(ws, "vt", torch.int16, (H, Nb, 2, D, 32)).cpu(),
        "probs": plan.view(ws, "scores", torch.float32, (H, Nt, ns)).cpu().numpy()[:, :, :Nt],
    }


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = got - ref
    max_abs = float(np.max(np.abs(d))) if d.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(d) / den) if den > 0 else float(np.linalg.norm(d))
    return max_abs, rel


def assert_close(got, ref, what, max_abs=MAX_ABS, rel_l2=REL_L2):
    ma, rl = errors(got, ref)
    say(f"  {what}: max_abs={ma:.3e} rel_l2={rl:.3e}")
    assert ma <= max_abs and rl <= rel_l2, (what, ma, rl)


def out_f64(out: torch.Tensor) -> np.ndarray:
    return out.detach().to("cpu").to(torch.float64).numpy()


def check_dispatch_order(plan, ws, offsets, pvis):
    """offsets [H][NV][C+1]: listed tiles of each video query tile below each
    chunk boundary; pvis: the implicit prefix tiles of the fine list."""
    H, Nt, P, C = plan.heads, plan.num_tiles, plan.num_prefix_tiles, plan.num_chunks
    order = plan.view(ws, "order", torch.int32, (H, C, Nt)).cpu().numpy()
    for c in range(C):
        lo, hi = c * plan.chunk_tiles, min((c + 1) * plan.chunk_tiles, Nt)
        for h in range(H):
            work = np.full(Nt, hi - lo)
            work[P:] = (min(hi, pvis) - min(lo, pvis)) + offsets[h, :, c + 1] - offsets[h, :, c]
            o = order[h, c]
            assert np.array_equal(np.sort(o), np.arange(Nt)), (h, c)
            assert np.all(np.diff(work[o]) <= 0), (h, c)


def check_all_heads_selection(q_in, k_in, g, topk, qp_gpu, kp_gpu, sel_gpu, prep=None,
                              threads=8):
    """Pooled q/k and the selection of EVERY head bit-exact against the
    oracle's fixed-order pool, scores and top-k (no fine branch), spread over
    host threads (NumPy's array operations release the GIL).  q_in, k_in:
    [L, H, D] inputs (torch or float32 NumPy); prep: the QK-norm + RoPE inputs
    (CPU tensors) to apply per head first, with the R17 rounding for bf16."""
    import concurrent.futures as cf
    H = qp_gpu.shape[0]
    is_bf16 = str(getattr(q_in, "dtype", "")).endswith("bfloat16")

    def one(h):
        qh = oracle.to_f32(q_in[:, h, :])
        kh = oracle.to_f32(k_in[:, h, :])
        if prep is not None:
            def pr(x, wgt):
                r = oracle.qk_norm_rope(x, wgt.numpy(), prep["eps"], prep["cos"].numpy(),
                                        prep["sin"].numpy())
                return (oracle.round_bf16_from_f64(r.astype(np.float64)).astype(np.float32)
                        if is_bf16 else r)
            qh, kh = pr(qh, prep["q_weight"]), pr(kh, prep["k_weight"])
        qp = oracle.pool_canonical(qh, g)
        kp = oracle.pool_canonical(kh, g)
        sel = oracle.select_topk(oracle.scores_canonical(qp, kp), g, topk)
        return (h, bool(np.array_equal(qp_gpu[h], qp)), bool(np.array_equal(kp_gpu[h], kp)),
                bool(np.array_equal(sel_gpu[h], sel)))

    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        res = list(ex.map(one, range(H)))
    bad = [r for r in res if not all(r[1:])]
    say(f"  selection and pooled q/k bit-exact on {H - len(bad)} of {H} heads")
    assert not bad, bad[:4]

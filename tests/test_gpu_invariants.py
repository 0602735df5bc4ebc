"""Invariants of the HIP path that hold bit for bit, checked GPU against GPU.

- The packed order of video tokens is free (each token carries its (t, y, x)
  position): tiles, slot order and every sum are defined by positions, so a
  permuted packing gives the same selection and the same output rows, only
  permuted.
- Heads are independent: changing one head's inputs leaves every other head's
  output and selection untouched.
Both follow from the method's definition (FastH3 4-step Preview (VSA,
data-free), "Video Sparse Attention is not optional here": the geometry comes
from tags and positions; scores and selection are per head).
- Full key lists reproduce the dense path bit for bit (FastH3 NVFP4 on RTX PRO
  6000, "Block-sparse FP4 attention for VSA tiles", its correctness check):
  at sparsity 0 a video query tile lists every tile in ascending order, the
  same visits a prefix query tile makes densely, so a video tile given the
  q rows, gate rows and valid count of a prefix tile must produce that prefix
  tile's output rows exactly.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_helpers import require_gpu, run, say
from workloads import AUDIO, COND, TEXT, Workload, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


CASES = [
    Workload("inv64", 4, 128, "bf16", ((TEXT, 70), (COND, 130), (AUDIO, 33)), (9, 10, 11), 0.7),
    Workload("inv128", 4, 128, "bf16", ((TEXT, 70), (COND, 300), (AUDIO, 33)), (9, 16, 12), 0.7,
             tile=(4, 8, 4), ref_keep=0.4),
    Workload("inv64_f32", 2, 64, "f32", ((AUDIO, 50),), (5, 6, 7), 0.5),
]


@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_video_packing_order_only_permutes_output_rows(w):
    say(f"case {w.name}: packed video order shuffled")
    x = make_inputs(w, seed=21)
    npre = w.n_prefix_tokens
    g = torch.Generator().manual_seed(77)
    order = torch.cat([torch.arange(npre), npre + torch.randperm(w.L - npre, generator=g)])
    y = {n: x[n][order].contiguous() for n in ("q", "k", "v", "gate", "position_ids")}
    y["token_tags"] = x["token_tags"][order].contiguous()
    for chunk in (0, 3):
        out1, sel1, _, _ = run(x, w.grid, w.sparsity, tile=w.tile, ref_keep=w.ref_keep,
                               chunk_tiles=chunk)
        out2, sel2, _, _ = run(y, w.grid, w.sparsity, tile=w.tile, ref_keep=w.ref_keep,
                               chunk_tiles=chunk)
        assert torch.equal(sel1, sel2)
        assert torch.equal(out2, out1[order.cuda()])


@pytest.mark.parametrize("w", CASES[:2], ids=[w.name for w in CASES[:2]])
def test_heads_are_independent(w):
    say(f"case {w.name}: one head's inputs replaced")
    x = make_inputs(w, seed=22)
    out1, sel1, _, _ = run(x, w.grid, w.sparsity, tile=w.tile, ref_keep=w.ref_keep)
    y = {n: v.clone() if torch.is_tensor(v) else v for n, v in x.items()}
    rng = torch.Generator().manual_seed(5)
    for n in ("q", "k", "v", "gate"):
        y[n][:, 2] = torch.randn(y[n][:, 2].shape, generator=rng).to(y[n].dtype)
    out2, sel2, _, _ = run(y, w.grid, w.sparsity, tile=w.tile, ref_keep=w.ref_keep)
    others = [h for h in range(w.heads) if h != 2]
    assert torch.equal(out1[:, others], out2[:, others])
    assert torch.equal(sel1[others], sel2[others])
    assert not torch.equal(out1[:, 2], out2[:, 2])
    assert np.isfinite(out2.float().cpu().numpy()).all()


FULL_LIST = [
    (Workload("full64_bf16", 4, 128, "bf16", ((TEXT, 64), (AUDIO, 64)), (8, 8, 12), 0.0), 0),
    (Workload("full64_bf16_ch", 4, 128, "bf16", ((TEXT, 64), (AUDIO, 64)), (8, 8, 12), 0.0), 3),
    (Workload("full64_f32", 2, 64, "f32", ((TEXT, 64),), (8, 8, 8), 0.0), 0),
    (Workload("full128_bf16", 2, 128, "bf16", ((TEXT, 128), (COND, 128)), (8, 16, 8), 0.0,
              tile=(4, 8, 4)), 0),
]


@pytest.mark.parametrize("w,ch", FULL_LIST, ids=[c[0].name for c in FULL_LIST])
def test_full_key_list_reproduces_the_dense_path(w, ch):
    say(f"case {w.name}: sparsity 0, video tile given a prefix tile's rows, chunk_tiles={ch}")
    x = make_inputs(w, seed=31)
    g = oracle.geometry(x["token_tags"], x["position_ids"], w.grid, w.tile)
    tt = g.tile_tokens
    pre = 0                                     # a full prefix tile
    vid = g.P + 3                               # a full video tile
    assert len(g.tiles[pre]) == len(g.tiles[vid]) == tt
    src = torch.as_tensor(g.tiles[pre])
    dst = torch.as_tensor(g.tiles[vid])         # slot order of both tiles
    for n in ("q", "gate"):
        x[n][dst] = x[n][src]
    out, sel, plan, _ = run(x, w.grid, w.sparsity, chunk_tiles=ch, tile=w.tile)
    assert plan.topk == g.NV
    assert torch.equal(sel[:, vid - g.P].cpu(), torch.arange(g.P, g.Nt, dtype=torch.int32)
                       .expand(w.heads, -1))
    if ch:
        assert plan.num_chunks > 1
    assert torch.equal(out[dst], out[src])
    # and not by accident: other video tiles differ from the prefix tile
    assert not torch.equal(out[torch.as_tensor(g.tiles[vid + 1])], out[src])

"""The forward captured in a HIP graph and replayed.

A forward allocates nothing, clears nothing with hipMemset and never waits on
the host: the plan's tables go into the workspace once, before capture, and
every other workspace region is written before it is read within the same
forward.  The whole forward (gather and pooling, the coarse kernels, one fine
launch per key chunk) can therefore be captured on a stream and replayed.
Each replay must reproduce the eager forward bit for bit, with an eager
forward on other inputs, through the same workspace, run between replays.
"""
import pytest
import torch

import video_dit_block_amd as vsa
from tests.gpu_helpers import require_gpu, say
from workloads import AUDIO, COND, TEXT, WORKLOADS, Workload, make_inputs, make_qk_prep_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


CASES = [
    ("bf16_d128_chunked", Workload("g64", 3, 128, "bf16", ((TEXT, 70), (COND, 130), (AUDIO, 33)),
                                   (9, 10, 11), 0.7), dict(chunk_tiles=5)),
    ("f32_d64", WORKLOADS["tiny"], {}),
    ("omniref_fp8_chunked", WORKLOADS["omniref_small"], dict(chunk_tiles=4, qk_fp8=True)),
    ("qk_prep_chunked", Workload("gp", 2, 64, "bf16", ((TEXT, 64), (AUDIO, 20)), (8, 12, 8), 0.6),
     dict(chunk_tiles=3, qk_prep=True)),
]


@pytest.mark.parametrize("name,w,opts", CASES, ids=[c[0] for c in CASES])
def test_forward_replays_from_a_captured_graph(name, w, opts):
    say(f"case {name}: capture, then 3 replays with eager forwards between them")
    dev = torch.device("cuda", 0)
    x = make_inputs(w, seed=41)
    xd = {n: x[n].to(dev) for n in ("q", "k", "v", "gate")}
    # Other inputs of the same shapes, for the eager forwards between replays.
    yd = {n: (xd[n].float() * -1.5 + 0.25).to(xd[n].dtype) for n in xd}
    plan = vsa.Plan(x["token_tags"], x["position_ids"], w.grid, w.heads, w.head_dim, w.sparsity,
                    w.tile, ref_keep=w.ref_keep, io_dtype=w.io_dtype, **opts)
    io = vsa.VSA_BF16 if w.io_dtype == "bf16" else vsa.VSA_F32
    prep = None
    if opts.get("qk_prep"):
        p = make_qk_prep_inputs(w, x["position_ids"])
        prep = {n: p[n].to(dev) for n in ("q_weight", "k_weight", "cos", "sin")}
        eps = p["eps"]
    s = torch.cuda.Stream(dev)
    ws = plan.workspace(dev, s.cuda_stream)
    out = torch.empty_like(xd["q"])
    sel = torch.empty((w.heads, plan.num_video_tiles, plan.sel_width), dtype=torch.int32,
                      device=dev)
    torch.cuda.synchronize()

    def call(t):
        ptrs = [t[n].data_ptr() for n in ("q", "k", "v", "gate")]
        if prep is None:
            vsa.vsa_h3_forward(plan.handle, *ptrs, io, out.data_ptr(), sel.data_ptr(),
                               ws.data_ptr(), plan.workspace_bytes, s.cuda_stream)
        else:
            vsa.vsa_h3_forward_qk_prep(plan.handle, *ptrs, prep["q_weight"].data_ptr(),
                                       prep["k_weight"].data_ptr(), eps,
                                       prep["cos"].data_ptr(), prep["sin"].data_ptr(), io,
                                       out.data_ptr(), sel.data_ptr(), ws.data_ptr(),
                                       plan.workspace_bytes, s.cuda_stream)

    call(xd)
    torch.cuda.synchronize()
    out_x, sel_x = out.clone(), sel.clone()
    call(yd)
    torch.cuda.synchronize()
    out_y, sel_y = out.clone(), sel.clone()
    assert not torch.equal(out_x, out_y)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(xd)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        sel.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, out_x), f"replay {rep}: output"
        assert torch.equal(sel, sel_x), f"replay {rep}: selection"
        # Eager work between replays: a forward on other inputs through the
        # same workspace, which must still give its own eager result.
        call(yd)
        torch.cuda.synchronize()
        assert torch.equal(out, out_y) and torch.equal(sel, sel_y), f"eager after replay {rep}"
    del g

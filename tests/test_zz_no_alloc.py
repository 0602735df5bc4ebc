"""The forward that allocates nothing (vsa_h3_forward_noalloc), through the C
ABI, against the forward with a caller-provided workspace: two calls in a row
on the library's one device array, the second with a smaller input (so the
first call's contents are still there), each bit-identical to the ordinary
forward; a plan whose workspace exceeds the array is refused."""
import pytest
import torch

import video_dit_block_amd as vsa
from tests.gpu_helpers import require_gpu, say
from workloads import WORKLOADS, make_inputs, make_layout

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _both(w, seed):
    """(noalloc out, noalloc sel), (ordinary out, ordinary sel) for workload w."""
    x = make_inputs(w, seed=seed)
    dev = torch.device("cuda", 0)
    xd = {n: x[n].to(dev) for n in ("q", "k", "v", "gate")}
    plan = vsa.Plan(x["token_tags"], x["position_ids"], w.grid, w.heads, w.head_dim, w.sparsity,
                    w.tile, ref_keep=w.ref_keep, io_dtype=w.io_dtype)
    io = vsa.io_dtype_code(w.io_dtype)
    ptrs = [xd[n].data_ptr() for n in ("q", "k", "v", "gate")]
    stream = torch.cuda.current_stream(dev).cuda_stream
    outs = []
    for noalloc in (True, False):
        out = torch.full_like(xd["q"], float("nan"))
        sel = torch.full((w.heads, plan.num_video_tiles, plan.sel_width), -7, dtype=torch.int32,
                         device=dev)
        if noalloc:
            vsa.vsa_h3_forward_noalloc(plan.handle, *ptrs, io, out.data_ptr(), sel.data_ptr(),
                                       stream)
        else:
            ws = plan.workspace(dev, stream)
            vsa.vsa_h3_forward(plan.handle, *ptrs, io, out.data_ptr(), sel.data_ptr(),
                               ws.data_ptr(), plan.workspace_bytes, stream)
        torch.cuda.synchronize()
        outs.append((out, sel))
    return plan, outs[0], outs[1]


def test_noalloc_forward_matches_workspace_forward_twice():
    big = WORKLOADS["480p5s"].with_(heads=4)            # 32 MiB of the 64 MiB array
    small = WORKLOADS["tiny"]                            # 0.6 MiB, fp32 I/O
    for w, seed in ((big, 21), (small, 22)):
        plan, (o1, s1), (o2, s2) = _both(w, seed)
        say(f"case {w.name}: heads={w.heads} workspace={plan.workspace_bytes / 2**20:.1f} MiB")
        assert torch.isfinite(o1).all()
        assert torch.equal(o1, o2), w.name
        assert torch.equal(s1, s2), w.name


def test_noalloc_forward_refuses_a_workspace_beyond_the_array():
    w = WORKLOADS["480p5s"].with_(heads=8)               # 64.6 MiB > 64 MiB
    tags, pos = make_layout(w)
    plan = vsa.Plan(tags, pos, w.grid, w.heads, w.head_dim, w.sparsity)
    assert plan.workspace_bytes > 64 << 20
    fake = 1 << 40   # never dereferenced: the size check comes first
    with pytest.raises(vsa.VsaError) as e:
        vsa.vsa_h3_forward_noalloc(plan.handle, fake, fake, fake, fake, vsa.VSA_BF16, fake, None,
                                   torch.cuda.current_stream().cuda_stream)
    assert e.value.status == -5 and "at most" in str(e.value)

"""One cached plan used by forwards on two streams at once: each stream gets a
workspace of its own, so the results are bit-identical to the same forwards
run one after the other."""
import pytest
import torch

import video_dit_block_amd as vsa
from tests.gpu_helpers import require_gpu, say
from workloads import TEXT, AUDIO, Workload, make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def test_two_streams_share_one_cached_plan():
    # 8 heads over 1,088 prefix + 8x32x64 video tokens: each forward is long
    # enough that the two streams' kernels overlap on the device
    w = Workload("streams", 8, 128, "bf16", ((TEXT, 576), (AUDIO, 512)), (8, 32, 64), 0.7)
    say(f"case two streams: L={w.L} heads={w.heads}")
    xs = [make_inputs(w, seed=s) for s in (31, 32)]
    dev = torch.device("cuda", 0)
    xd = [{n: x[n].to(dev) for n in ("q", "k", "v", "gate")} for x in xs]
    tags, pos = xs[0]["token_tags"], xs[0]["position_ids"]
    for x in xs[1:]:
        assert torch.equal(torch.as_tensor(x["token_tags"]), torch.as_tensor(tags))

    def fwd(d):
        return vsa.forward(d["q"], d["k"], d["v"], d["gate"], tags, pos, w.grid, w.sparsity,
                           return_sel=True)

    # one after the other, on the current stream
    ref = [fwd(d) for d in xd]
    torch.cuda.synchronize()
    plan = vsa.get_plan(tags, pos, w.grid, w.heads, w.head_dim, w.sparsity)

    streams = [torch.cuda.Stream(dev), torch.cuda.Stream(dev)]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream(dev))
    got = [[], []]
    for rep in range(3):
        for j, s in enumerate(streams):
            with torch.cuda.stream(s):
                got[j].append(fwd(xd[j]))
    torch.cuda.synchronize()
    keys = set(plan._ws)
    for s in streams:
        assert (0, s.cuda_stream) in keys
    for j in range(2):
        for rep, (o, sel) in enumerate(got[j]):
            assert torch.equal(sel, ref[j][1]), (j, rep)
            assert torch.equal(o, ref[j][0]), (j, rep)
    say("two streams: 6 concurrent forwards bit-identical to sequential ones")

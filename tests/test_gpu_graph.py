"""The whole path captured in a HIP graph (torch.cuda.CUDAGraph over the
library's launches): the library allocates nothing, synchronizes nothing and
clears memory with kernels only, so ``Plan.run`` can be captured once and
replayed.  Every replay is checked bit for bit against the eager result,
with eager runs on other inputs in between (they reuse the same buffers)."""
import pytest
import torch

import workloads
from gpu_util import dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,opts", [("tiny", {}), ("mid", {"kmeans": (16, 3)}),
                                       ("mid", {"v_format": "mxfp4", "expcast": True}),
                                       ("mid", {"p_format": "mxfp4", "rope": True}),
                                       ("mid", {"mma": "bf16", "cube": True})])
def test_graph_replays_equal_eager(name, opts):
    import bit_attention_video_smooth_amd as vs
    w = workloads.WORKLOADS[name]
    d = dev()
    opts = dict(opts)
    if opts.pop("rope", False):
        # a 3D rotary table over an 8 x 32 x 32 token grid (S = 8192)
        opts["rope"] = workloads.rope_tables_3d(w.S, w.D, (8, 32, 32), device=d)
    if opts.pop("cube", False):
        opts["cube"] = ((8, 32, 32), (2, 8, 8))
    q, k, v = (t.to(d) for t in workloads.generate(w))
    q2, k2, v2 = (t.flip(1).contiguous() for t in (q, k, v))     # other inputs
    plan = vs.Plan((w.B, w.S, w.H, w.D), d, **opts)
    out, lse = plan.run(q, k, v)
    torch.cuda.synchronize(d)
    ref_o, ref_l = out.clone(), lse.clone()

    side = torch.cuda.Stream(device=d)
    side.wait_stream(torch.cuda.current_stream(d))
    with torch.cuda.stream(side):
        plan.run(q, k, v)                       # warm-up on the capture stream's side
    torch.cuda.current_stream(d).wait_stream(side)
    torch.cuda.synchronize(d)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan.run(q, k, v)
    torch.cuda.synchronize(d)
    for _ in range(3):
        plan.run(q2, k2, v2)                    # eager work in between, same buffers
        torch.cuda.synchronize(d)
        assert not torch.equal(plan.out, ref_o)
        g.replay()
        torch.cuda.synchronize(d)
        assert torch.equal(plan.out.view(torch.int32), ref_o.view(torch.int32))
        assert torch.equal(plan.lse2.view(torch.int32), ref_l.view(torch.int32))

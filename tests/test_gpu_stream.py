"""Every binding call with an explicit `stream=` and no workspace: the kernels
run on that stream, the workspace and default outputs are allocated on it, and
the results equal those of the same calls on the current stream bit for bit,
even while other work on the current stream allocates and overwrites memory
meanwhile (a workspace block freed while the side stream still used it would
be handed to that work)."""
import numpy as np
import pytest

import synth
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


def _bits(t):
    torch = G.torch_mod()
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.cpu().numpy().view(np.uint8)


def test_explicit_stream_without_workspace_matches_current_stream():
    torch = G.torch_mod()
    import mixture_experts_layer_expert_amd as moe
    moe.load_library()
    wl = synth.Workload("stream_case", T=1536, D=256, I=192, E=16, K=4, score=0, seed=31)
    data = synth.generate(wl)
    dev = G.DeviceInputs(data)
    w_r = G.to_dev(data["w_r"])

    def run(stream):
        logits = moe.moe_router_fwd(dev.x, w_r, stream=stream)
        route = moe.moe_route_sort(logits, wl.K, wl.score, stream=stream)
        y = moe.moe_fwd(dev.x, dev.w_gate, dev.w_up, dev.w_down, route, wl.K, wl.score,
                        stream=stream)
        g = moe.moe_bwd(dev.x, dev.w_gate, dev.w_up, dev.w_down, route, dev.dy, wl.K, wl.score,
                        stream=stream)
        dw_r = moe.moe_router_bwd(dev.x, w_r, route, g["d_topk_w"], g["dx"], wl.K, wl.score,
                                  stream=stream)
        return dict(logits=logits, y=y, dw_r=dw_r, **route, **g)

    ref = run(None)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    got = run(side)
    # meanwhile the current stream allocates and scribbles over free memory
    junk = [torch.full((1 << 22,), float(i + 1), device="cuda") for i in range(8)]
    del junk
    side.synchronize()
    torch.cuda.synchronize()
    for k in ref:
        assert np.array_equal(_bits(got[k]), _bits(ref[k])), k

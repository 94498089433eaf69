"""GPU tests of the torch.autograd wrapper (mixture_experts_layer_expert_amd.autograd)
and of graph capture of the whole chain (router, routing, forward, backward,
router backward) through the C ABI.

The wrapper's gradients are compared with the oracle's chain on the GPU's own
routing decisions (the selection is taken from the GPU logits on both
sides), to |gpu - ref| <= 1e-2 + 1e-2 |ref|; weight gradients come back in
the weights' dtype (bf16 for the expert weights), a rounding that the bar
covers (2^-9 relative).
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not G.gpu_available():
        pytest.skip("no GPU")
    import mixture_experts_layer_expert_amd as moe
    moe.load_library()


def _workload(T=520, D=192, I=128, E=16, K=4, score=0, seed=401):
    wl = synth.Workload("autograd", T=T, D=D, I=I, E=E, K=K, score=score, seed=seed)
    return wl, synth.generate(wl)


@pytest.mark.parametrize("score,K", [(0, 4), (1, 1)])
def test_autograd_gradients_match_oracle(score, K):
    from mixture_experts_layer_expert_amd import autograd as A
    import mixture_experts_layer_expert_amd as moe
    torch = G.torch_mod()
    wl, data = _workload(K=K, score=score, seed=402 + K)
    x = G.to_dev_bf16(data["x"]).requires_grad_(True)
    w_r = G.to_dev(data["w_r"]).requires_grad_(True)
    w_gate = G.to_dev_bf16(data["w_gate"]).requires_grad_(True)
    w_up = G.to_dev_bf16(data["w_up"]).requires_grad_(True)
    w_down = G.to_dev_bf16(data["w_down"]).requires_grad_(True)
    dy = G.to_dev_bf16(data["dy"])
    y = A.moe(x, w_r, w_gate, w_up, w_down, wl.K, wl.score)
    (y.float() * dy.float()).sum().backward()
    torch.cuda.synchronize()
    # the oracle chain on the GPU's routing decisions
    logits = G.host(moe.moe_router_fwd(x.detach(), w_r.detach()))
    torch.cuda.synchronize()
    idx, w = oracle.route(logits, wl.K, wl.score)
    f = synth.bf16_bits_to_f64
    L = oracle.Layer(f(data["x"]), f(data["w_gate"]), f(data["w_up"]), f(data["w_down"]), wl.K,
                     wl.score, f(data["dy"]))
    G.assert_close(G.bf16_dev_to_f64(y.detach()), oracle.forward(L, idx, w), "y")
    dx_e, drw = oracle.backward_tokens(L, idx, w)
    dwg, dwu, dwd = oracle.backward_dw(L, idx, w)
    _, dw_r, dx_r = oracle.router_backward(f(data["x"]), data["w_r"], idx, w, drw, wl.score)
    G.assert_close(G.bf16_dev_to_f64(x.grad), dx_e + dx_r, "x.grad")
    G.assert_close(G.host(w_r.grad), dw_r, "w_r.grad")
    G.assert_close(G.bf16_dev_to_f64(w_gate.grad), dwg, "w_gate.grad")
    G.assert_close(G.bf16_dev_to_f64(w_up.grad), dwu, "w_up.grad")
    G.assert_close(G.bf16_dev_to_f64(w_down.grad), dwd, "w_down.grad")
    assert w_r.grad.dtype == torch.float32 and w_gate.grad.dtype == torch.bfloat16


def test_module_trains_one_step():
    """MoELayer: parameters receive finite gradients and an SGD step changes them."""
    from mixture_experts_layer_expert_amd import autograd as A
    torch = G.torch_mod()
    gen = torch.Generator().manual_seed(7)
    layer = A.MoELayer(D=128, I=64, E=8, K=2, device="cuda", generator=gen)
    x = torch.randn((300, 128), generator=gen).to("cuda", torch.bfloat16)
    before = {n: p.detach().clone() for n, p in layer.named_parameters()}
    y = layer(x)
    y.float().square().mean().backward()
    with torch.no_grad():
        for p in layer.parameters():
            assert p.grad is not None and bool(torch.isfinite(p.grad.float()).all())
            p -= 0.1 * p.grad
    torch.cuda.synchronize()
    for n, p in layer.named_parameters():
        assert not torch.equal(p.detach(), before[n]), n


def test_graph_capture_full_chain():
    """Router projection, routing, forward, backward and router backward captured
    into one graph; three replays (with eager work and syncs in between)
    reproduce the eager results bit for bit."""
    import mixture_experts_layer_expert_amd as moe
    torch = G.torch_mod()
    wl, data = _workload(T=384, D=128, I=128, E=8, K=2, seed=403)
    dev = G.DeviceInputs(data)
    w_r = G.to_dev(data["w_r"])
    d = moe.dims(wl.T, wl.D, wl.I, wl.E, wl.K, wl.score)
    ws = {ph: torch.empty(moe.moe_workspace_bytes(d, ph), dtype=torch.uint8, device="cuda")
          for ph in range(4)}
    logits = torch.empty((wl.T, wl.E), dtype=torch.float32, device="cuda")
    y = torch.empty((wl.T, wl.D), dtype=torch.bfloat16, device="cuda")
    dw_r = torch.empty((wl.D, wl.E), dtype=torch.float32, device="cuda")

    def chain(route, grads):
        moe.moe_router_fwd(dev.x, w_r, logits=logits)
        moe.moe_route_sort(logits, wl.K, wl.score, out=route, ws=ws[0])
        moe.moe_fwd(dev.x, dev.w_gate, dev.w_up, dev.w_down, route, wl.K, wl.score, y=y, ws=ws[1])
        moe.moe_bwd(dev.x, dev.w_gate, dev.w_up, dev.w_down, route, dev.dy, wl.K, wl.score,
                    out=grads, ws=ws[2])
        moe.moe_router_bwd(dev.x, w_r, route, grads["d_topk_w"], grads["dx"], wl.K, wl.score,
                           dw_r=dw_r, ws=ws[3])

    route = moe.moe_route_sort(torch.zeros((wl.T, wl.E), dtype=torch.float32, device="cuda"),
                               wl.K, wl.score)
    grads = moe.moe_bwd(dev.x, dev.w_gate, dev.w_up, dev.w_down, route, dev.dy, wl.K, wl.score)
    chain(route, grads)
    torch.cuda.synchronize()
    ref = {"y": y.clone(), "dw_r": dw_r.clone(), "logits": logits.clone(),
           **{k: v.clone() for k, v in grads.items()}, **{"r_" + k: v.clone() for k, v in route.items()}}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the capture stream
        chain(route, grads)
    s.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        chain(route, grads)
    outs = {"y": y, "dw_r": dw_r, "logits": logits, **grads, **{"r_" + k: v for k, v in route.items()}}
    for rep in range(3):
        for t in outs.values():
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, t in outs.items():
            a, b = t, ref[k]
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b), (rep, k)

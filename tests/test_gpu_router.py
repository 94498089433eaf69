"""GPU parity of the router projection and router backward (through the C ABI)
against the CPU oracle.

Bar: floating-point outputs within |gpu - ref| <= 1e-2 + 1e-2 |ref| of the
float64 oracle, and the logits also within 1e-4 + 1e-4 |ref|: the GPU sums D
exact products of bf16 x and fp32 w_r in fp32, whose rounding error for the
unit-variance logits here stays near 1e-6, so 1e-4 still catches a
lower-precision operand (w_r rounded to bf16 moves a logit by ~1e-3).
Routing decisions are taken on the GPU's logits on both sides (same
precision), and must agree bit for bit.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_common as G

pytestmark = pytest.mark.gpu

LOGIT_TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not G.gpu_available():
        pytest.skip("no GPU")
    import mixture_experts_layer_expert_amd as moe
    moe.load_library()


CASES = {
    "tiny": dict(T=256, D=128, I=64, E=8, K=2, score=0, seed=301),
    # several token ranges for dW_r with a ragged last stage, E not a multiple of 4
    # or of the 64-expert tile, K = 3
    "ragged": dict(T=1500, D=256, I=64, E=65, K=3, score=0, seed=302),
    "sigmoid_top1": dict(T=257, D=192, I=64, E=4, K=1, score=1, seed=303),
    "k16": dict(T=96, D=128, I=64, E=64, K=16, score=0, seed=304),
    "one_token": dict(T=1, D=64, I=64, E=8, K=2, score=0, seed=305),
}


def _data(c):
    wl = synth.Workload("router", T=c["T"], D=c["D"], I=c["I"], E=c["E"], K=c["K"],
                        score=c["score"], seed=c["seed"])
    return wl, synth.generate(wl)


def _router_inputs(wl, seed):
    """Seeded router-weight gradient [T, K] (fp32) and incoming dX [T, D] (bf16)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    drw = rng.standard_normal((wl.T, wl.K), dtype=np.float32)
    dx_in = synth.f32_to_bf16_bits(rng.standard_normal((wl.T, wl.D), dtype=np.float32))
    return drw, dx_in


def _check_router(wl, data, drw_np, dx_in_np):
    """router_fwd -> route_sort -> router_bwd on the GPU against the oracle on the
    same inputs (the selection and weights the GPU produced from its logits)."""
    import mixture_experts_layer_expert_amd as moe
    x = G.to_dev_bf16(data["x"])
    w_r = G.to_dev(data["w_r"])
    logits = moe.moe_router_fwd(x, w_r)
    G.torch_mod().cuda.synchronize()
    x64 = synth.bf16_bits_to_f64(data["x"])
    ref_logits = oracle.router_logits(x64, data["w_r"])
    got_logits = G.host(logits)
    G.assert_close(got_logits, ref_logits, "logits")
    G.assert_close(got_logits, ref_logits, "logits (fp32 bound)", atol=LOGIT_TOL, rtol=LOGIT_TOL)
    route = moe.moe_route_sort(logits, wl.K, wl.score)
    G.torch_mod().cuda.synchronize()
    idx, w, _ = G.check_route_exact(route, {"logits": got_logits}, wl.K, wl.score, wl.E)
    w_gpu = G.host(route["topk_w"]).astype(np.float64)
    drw = G.to_dev(drw_np)
    dx = G.to_dev_bf16(dx_in_np)
    dw_r = moe.moe_router_bwd(x, w_r, route, drw, dx, wl.K, wl.score)
    G.torch_mod().cuda.synchronize()
    _, dw_ref, dx_r = oracle.router_backward(x64, data["w_r"], idx, w_gpu, drw_np, wl.score)
    G.assert_close(G.host(dw_r), dw_ref, "dw_r")
    G.assert_close(G.bf16_dev_to_f64(dx), synth.bf16_bits_to_f64(dx_in_np) + dx_r, "dx")
    return logits, route, dw_r, dx


@pytest.mark.parametrize("case", list(CASES))
def test_router_parity_small(case):
    wl, data = _data(CASES[case])
    drw, dx_in = _router_inputs(wl, CASES[case]["seed"] + 1000)
    _check_router(wl, data, drw, dx_in)


@pytest.mark.slow
def test_router_qwen3_30b_a3b_full_size():
    """Every element of logits, dW_r and dX at the Qwen3-30B-A3B layer shape
    (T = 8192, D = 2048, E = 128, K = 8): the oracle's router is cheap enough."""
    wl = synth.QWEN3_30B_A3B
    data = synth.generate(wl)
    drw, dx_in = _router_inputs(wl, 4242)
    _check_router(wl, data, drw, dx_in)


@pytest.mark.slow
def test_router_llama4_scout_full_size():
    """Every element of logits, dW_r and dX at the Llama-4-Scout layer shape
    (T = 8192, D = 5120, E = 16, top-1 sigmoid)."""
    wl = synth.LLAMA4_SCOUT
    data = synth.generate(wl, with_dy=False)
    drw, dx_in = _router_inputs(wl, 4343)
    _check_router(wl, data, drw, dx_in)


def test_router_in_the_layer():
    """Router + layer end to end: the GPU's dX after moe_bwd and moe_router_bwd is
    the full input gradient of the layer (expert path + router path), and dW_r is
    the router weights' gradient, both against the oracle's chain on the GPU's
    routing decisions."""
    import mixture_experts_layer_expert_amd as moe
    wl, data = _data(dict(T=640, D=192, I=128, E=16, K=4, score=0, seed=306))
    dev = G.DeviceInputs(data)
    w_r = G.to_dev(data["w_r"])
    logits = moe.moe_router_fwd(dev.x, w_r)
    route = moe.moe_route_sort(logits, wl.K, wl.score)
    grads = moe.moe_bwd(dev.x, dev.w_gate, dev.w_up, dev.w_down, route, dev.dy, wl.K, wl.score)
    dw_r = moe.moe_router_bwd(dev.x, w_r, route, grads["d_topk_w"], grads["dx"], wl.K, wl.score)
    G.torch_mod().cuda.synchronize()
    got_logits = G.host(logits)
    idx, w = oracle.route(got_logits, wl.K, wl.score)
    np.testing.assert_array_equal(G.host(route["topk_idx"]), idx)
    f = synth.bf16_bits_to_f64
    L = oracle.Layer(f(data["x"]), f(data["w_gate"]), f(data["w_up"]), f(data["w_down"]), wl.K,
                     wl.score, f(data["dy"]))
    dx_e, drw = oracle.backward_tokens(L, idx, w)
    _, dw_ref, dx_r = oracle.router_backward(f(data["x"]), data["w_r"], idx, w, drw, wl.score)
    G.assert_close(G.bf16_dev_to_f64(grads["dx"]), dx_e + dx_r, "dx (experts + router)")
    G.assert_close(G.host(dw_r), dw_ref, "dw_r")


def test_router_determinism_accumulate_and_empty():
    """Bitwise repeatable; accumulate_dwr adds exactly; T = 0 gives dW_r = 0."""
    import mixture_experts_layer_expert_amd as moe
    torch = G.torch_mod()
    wl, data = _data(dict(T=1100, D=128, I=64, E=12, K=3, score=0, seed=307))
    drw_np, dx_np = _router_inputs(wl, 77)
    x = G.to_dev_bf16(data["x"])
    w_r = G.to_dev(data["w_r"])
    logits = moe.moe_router_fwd(x, w_r)
    logits2 = torch.full_like(logits, float("nan"))
    moe.moe_router_fwd(x, w_r, logits=logits2)
    route = moe.moe_route_sort(logits, wl.K, wl.score)
    drw = G.to_dev(drw_np)
    dx1, dx2 = G.to_dev_bf16(dx_np), G.to_dev_bf16(dx_np)
    dw1 = moe.moe_router_bwd(x, w_r, route, drw, dx1, wl.K, wl.score)
    dw2 = torch.full_like(dw1, float("nan"))
    moe.moe_router_bwd(x, w_r, route, drw, dx2, wl.K, wl.score, dw_r=dw2)
    torch.cuda.synchronize()
    assert torch.equal(logits, logits2)
    assert torch.equal(dw1, dw2)
    assert torch.equal(dx1.view(torch.int16), dx2.view(torch.int16))
    moe.moe_router_bwd(x, w_r, route, drw, dx2, wl.K, wl.score, dw_r=dw2, accumulate_dwr=True)
    torch.cuda.synchronize()
    assert torch.equal(dw2, 2 * dw1)
    # empty batch
    x0 = torch.empty((0, wl.D), dtype=torch.bfloat16, device="cuda")
    lg0 = moe.moe_router_fwd(x0, w_r)
    r0 = moe.moe_route_sort(lg0, wl.K, wl.score)
    dw0 = torch.full_like(dw1, float("nan"))
    moe.moe_router_bwd(x0, w_r, r0, torch.empty((0, wl.K), dtype=torch.float32, device="cuda"),
                       x0, wl.K, wl.score, dw_r=dw0)
    torch.cuda.synchronize()
    assert lg0.shape == (0, wl.E)
    assert not dw0.any()

"""Helpers for the GPU parity tests: move synthetic inputs to the device, run
the HIP path through the C ABI, and compare with the oracle.

Tolerance for floating-point outputs (bf16 inputs, fp32 accumulation):
    |gpu - ref| <= ATOL + RTOL * |ref|   for every compared element.
"""
from __future__ import annotations

import numpy as np

import synth

ATOL = 1e-2
RTOL = 1e-2


def torch_mod():
    import torch
    return torch


def gpu_available() -> bool:
    try:
        torch = torch_mod()
        return torch.cuda.is_available()
    except Exception:
        return False


def to_dev_bf16(u16: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(u16).view(np.int16)).view(torch.bfloat16).cuda()


def to_dev(a: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_dev_to_f64(t) -> np.ndarray:
    torch = torch_mod()
    u16 = t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
    return synth.bf16_bits_to_f64(u16)


def host(t) -> np.ndarray:
    return t.detach().cpu().numpy()


def assert_close(gpu, ref, name: str, atol: float = ATOL, rtol: float = RTOL) -> float:
    """Element-wise |gpu - ref| <= atol + rtol |ref|; returns the worst ratio."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (name, gpu.shape, ref.shape)
    if gpu.size == 0:
        return 0.0
    assert np.all(np.isfinite(gpu)), f"{name}: non-finite GPU values"
    err = np.abs(gpu - ref)
    lim = atol + rtol * np.abs(ref)
    ratio = err / lim
    worst = int(np.argmax(ratio))
    w = np.unravel_index(worst, gpu.shape)
    assert ratio.flat[worst] <= 1.0, (
        f"{name}: worst element {w}: gpu={gpu[w]!r} ref={ref[w]!r} |err|={err[w]:.3e} "
        f"limit={lim[w]:.3e} (max |err| {err.max():.3e})")
    return float(ratio.flat[worst])


class DeviceInputs:
    """Device copies of one workload's inputs."""

    def __init__(self, data: dict):
        self.x = to_dev_bf16(data["x"])
        self.w_gate = to_dev_bf16(data["w_gate"])
        self.w_up = to_dev_bf16(data["w_up"])
        self.w_down = to_dev_bf16(data["w_down"])
        self.dy = None if data.get("dy") is None else to_dev_bf16(data["dy"])
        self.logits = to_dev(data["logits"].astype(np.float32))


def run_gpu(dev: DeviceInputs, K: int, score: int, backward: bool = True):
    """Route + forward (+ backward) through the C ABI; returns device tensors."""
    import mixture_experts_layer_expert_amd as moe
    route = moe.moe_route_sort(dev.logits, K, score)
    y = moe.moe_fwd(dev.x, dev.w_gate, dev.w_up, dev.w_down, route, K, score)
    grads = None
    if backward:
        grads = moe.moe_bwd(dev.x, dev.w_gate, dev.w_up, dev.w_down, route, dev.dy, K, score)
    torch_mod().cuda.synchronize()
    return route, y, grads


def oracle_layer(data: dict, K: int, score: int):
    import oracle
    f = synth.bf16_bits_to_f64
    L = oracle.Layer(f(data["x"]), f(data["w_gate"]), f(data["w_up"]), f(data["w_down"]), K, score,
                     None if data.get("dy") is None else f(data["dy"]))
    idx, w = oracle.route(data["logits"], K, score)
    return L, idx, w


def check_route_exact(route: dict, data: dict, K: int, score: int, E: int):
    """Routing indices, counts, offsets and both permutations bit-exact; weights
    within tolerance."""
    import oracle
    idx, w = oracle.route(data["logits"], K, score)
    counts, offsets, s2f, f2s = oracle.sort(idx, E)
    np.testing.assert_array_equal(host(route["topk_idx"]), idx, err_msg="topk_idx")
    np.testing.assert_array_equal(host(route["counts"]), counts, err_msg="counts")
    np.testing.assert_array_equal(host(route["offsets"]), offsets, err_msg="offsets")
    np.testing.assert_array_equal(host(route["sorted_to_flat"]), s2f, err_msg="sorted_to_flat")
    np.testing.assert_array_equal(host(route["flat_to_sorted"]), f2s, err_msg="flat_to_sorted")
    assert_close(host(route["topk_w"]), w, "topk_w", atol=1e-6, rtol=1e-5)
    return idx, w, counts

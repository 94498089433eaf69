"""Seeded synthetic inputs for the routed SwiGLU mixture-of-experts layer.

This module is shared by the tests, the oracle's callers and the benchmark.
It only draws random numbers and encodes/decodes bf16 bits; it holds none of
the layer's arithmetic (no routing, no expert MLP, no gradients).

Recipe: ``numpy.random.SeedSequence(seed).spawn(6)`` gives one stream family
per tensor, in the order below.  Each tensor is split into blocks along its
leading dimension (256 tokens for x and dy, one expert for the expert
weights) and block b draws from ``PCG64(family.spawn(n_blocks)[b])``, so the
blocks can be drawn by parallel threads and the values do not depend on the
thread count.  Every draw is ``standard_normal`` in float32, then scaled:

  x       [T, D]      scale 1            -> bf16 (round to nearest even)
  w_r     [D, E]      scale 1/sqrt(D)    -> stays float32 (router projection)
  w_gate  [E, I, D]   scale 1/sqrt(D)    -> bf16
  w_up    [E, I, D]   scale 1/sqrt(D)    -> bf16
  w_down  [E, D, I]   scale 1/sqrt(I)    -> bf16
  dy      [T, D]      scale 1            -> bf16

Expert weights are stored in the ``[out_features, in_features]`` layout of a
linear layer: gate/up of expert e map D -> I, down maps I -> D.

Router logits are the router projection of the bf16 tokens, evaluated once in
float64 from the exact bf16 / float32 values and rounded to float32; the same
logits array feeds both the GPU path and the oracle.  For the skewed token
sweep a Zipf(s=1.2) prior over experts is added before the rounding:
``logits[t, e] += ln p_e`` with ``p_e = (e+1)^-s / sum_j j^-s``, so expert 0 is
the most popular.  The projection and the prior are input synthesis (they sit
before the routing step), not part of the layer under test.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

SOFTMAX_TOPK = 0   # softmax over all experts, top-K, renormalise over the K
SIGMOID = 1        # sigmoid of the selected logit, no renormalisation


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    D: int
    I: int
    E: int
    K: int
    score: int
    seed: int
    zipf_s: float = 0.0

    @property
    def R(self) -> int:
        return self.T * self.K

    def flops_fwd(self) -> float:
        """Counted forward FLOPs: 6*D*I per routed row (gate, up, down GEMMs)."""
        return 6.0 * self.D * self.I * self.R

    def flops_bwd(self) -> float:
        """Counted backward FLOPs: 12*D*I per routed row (recompute not counted)."""
        return 12.0 * self.D * self.I * self.R


TINY = Workload("tiny", T=256, D=128, I=64, E=8, K=2, score=SOFTMAX_TOPK, seed=1)
QWEN3_30B_A3B = Workload("qwen3_30b_a3b", T=8192, D=2048, I=768, E=128, K=8,
                         score=SOFTMAX_TOPK, seed=2)
LLAMA4_SCOUT = Workload("llama4_scout", T=8192, D=5120, I=8192, E=16, K=1,
                        score=SIGMOID, seed=3)


def qwen_zipf(T: int) -> Workload:
    """Qwen3-30B-A3B layer shape with Zipf(1.2)-skewed routing at T tokens."""
    return Workload(f"qwen3_30b_a3b_zipf_T{T}", T=T, D=2048, I=768, E=128, K=8,
                    score=SOFTMAX_TOPK, seed=4, zipf_s=1.2)


ZIPF_SWEEP_T = (1024, 2048, 4096, 8192, 16384)

_CHUNK = 1 << 24


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bits.

    Inputs are finite draws, so the 32-bit add cannot wrap and no NaN
    handling is needed.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    flat_in = a.reshape(-1)
    flat_out = out.reshape(-1)
    for s in range(0, flat_in.size, _CHUNK):
        u = flat_in[s:s + _CHUNK].view(np.uint32)
        r = (u >> 16) & 1
        r += 0x7FFF
        r += u
        r >>= 16
        flat_out[s:s + _CHUNK] = r
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _draw_blocks(family: np.random.SeedSequence, shape, block_rows: int,
                 scale: float, to_bf16: bool) -> np.ndarray:
    """Draw `shape` in blocks of `block_rows` leading rows, one spawned
    PCG64 stream per block, blocks filled by a thread pool."""
    rows = shape[0]
    inner = int(np.prod(shape[1:]))
    nblk = (rows + block_rows - 1) // block_rows
    seeds = family.spawn(nblk)
    out = np.empty((rows, inner), dtype=np.uint16 if to_bf16 else np.float32)

    def fill(b: int) -> None:
        r0 = b * block_rows
        r1 = min(rows, r0 + block_rows)
        v = np.random.Generator(np.random.PCG64(seeds[b])).standard_normal(
            (r1 - r0) * inner, dtype=np.float32)
        if scale != 1.0:
            v *= np.float32(scale)
        v = v.reshape(r1 - r0, inner)
        out[r0:r1] = f32_to_bf16_bits(v) if to_bf16 else v

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(nblk)))
    return out.reshape(shape)


def zipf_log_prior(E: int, s: float) -> np.ndarray:
    """ln p_e for p_e proportional to (e+1)^-s, float64 [E]."""
    ranks = np.arange(1, E + 1, dtype=np.float64)
    logw = -s * np.log(ranks)
    return logw - math.log(np.exp(logw).sum())


def generate(wl: Workload, with_dy: bool = True) -> dict:
    """All inputs of one workload as numpy arrays (bf16 as uint16 bits)."""
    fam = np.random.SeedSequence(wl.seed).spawn(6)
    T, D, I, E = wl.T, wl.D, wl.I, wl.E
    x = _draw_blocks(fam[0], (T, D), 256, 1.0, True)
    w_r = _draw_blocks(fam[1], (D, E), D, 1.0 / math.sqrt(D), False)
    w_gate = _draw_blocks(fam[2], (E, I, D), 1, 1.0 / math.sqrt(D), True)
    w_up = _draw_blocks(fam[3], (E, I, D), 1, 1.0 / math.sqrt(D), True)
    w_down = _draw_blocks(fam[4], (E, D, I), 1, 1.0 / math.sqrt(I), True)
    dy = _draw_blocks(fam[5], (T, D), 256, 1.0, True) if with_dy else None
    logits64 = bf16_bits_to_f64(x) @ w_r.astype(np.float64)
    if wl.zipf_s:
        logits64 += zipf_log_prior(E, wl.zipf_s)[None, :]
    logits = logits64.astype(np.float32)
    return dict(x=x, w_r=w_r, logits=logits, w_gate=w_gate, w_up=w_up,
                w_down=w_down, dy=dy)


def sample_indices(n: int, count: int, seed: int, must=()) -> np.ndarray:
    """Sorted distinct sample of range(n) of about `count` entries, always
    holding the entries in `must` (first/last rows and the like)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    count = min(count, n)
    pick = set(int(v) for v in must if 0 <= v < n)
    if count > len(pick):
        pick.update(int(v) for v in rng.choice(n, size=count, replace=False))
    return np.array(sorted(pick), dtype=np.int64)

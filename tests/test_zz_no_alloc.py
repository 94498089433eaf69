"""moe_route_sort_noalloc (routing without a workspace, histograms in the
library's static device scratch) against moe_route_sort and the oracle.

Two calls in a row on one GPU, the second with fewer routed rows and fewer
experts, so the second call runs over scratch contents the first one left:
every output must equal moe_route_sort's bit for bit, and the indices,
counts, offsets and permutations must equal the oracle's."""
import numpy as np
import pytest

from tests import gpu_common as G

pytestmark = pytest.mark.gpu


def _logits(T, E, seed):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    lg[::7, :4] = 0.5  # ties toward the lower expert id
    return lg


def _outputs(torch, T, E, K):
    dev = "cuda"
    return dict(topk_idx=torch.full((T, K), -1, dtype=torch.int32, device=dev),
                topk_w=torch.full((T, K), -1.0, dtype=torch.float32, device=dev),
                counts=torch.full((E,), -1, dtype=torch.int32, device=dev),
                offsets=torch.full((E + 1,), -1, dtype=torch.int32, device=dev),
                sorted_to_flat=torch.full((T * K,), -1, dtype=torch.int32, device=dev),
                flat_to_sorted=torch.full((T * K,), -1, dtype=torch.int32, device=dev))


@pytest.mark.parametrize("cases", [
    # (T, E, K, score): the Qwen3-30B-A3B routing shape, then a smaller batch
    [(8192, 128, 8, 0), (1000, 64, 6, 0)],
    # many histogram blocks, then a ragged tail over a single block, sigmoid scores
    [(40000, 256, 4, 1), (333, 16, 1, 1)],
])
def test_noalloc_route_matches_workspace_version(cases):
    torch = G.torch_mod()
    import oracle
    import mixture_experts_layer_expert_amd as moe
    moe.load_library()
    for i, (T, E, K, score) in enumerate(cases):
        print(f"noalloc case {i}: T={T} E={E} K={K} score={score}", flush=True)
        lg = _logits(T, E, seed=100 + i)
        logits = G.to_dev(lg)
        ref = moe.moe_route_sort(logits, K, score)
        out = _outputs(torch, T, E, K)
        moe.moe_route_sort_noalloc(logits, K, score, out=out)
        torch.cuda.synchronize()
        for k in ref:
            a, b = G.host(out[k]), G.host(ref[k])
            assert a.dtype == b.dtype and a.shape == b.shape, k
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{k} differs (case {i})"
        idx, w = oracle.route(lg, K, score)
        counts, offsets, s2f, f2s = oracle.sort(idx, E)
        np.testing.assert_array_equal(G.host(out["topk_idx"]), idx)
        np.testing.assert_array_equal(G.host(out["counts"]), counts)
        np.testing.assert_array_equal(G.host(out["offsets"]), offsets)
        np.testing.assert_array_equal(G.host(out["sorted_to_flat"]), s2f)
        np.testing.assert_array_equal(G.host(out["flat_to_sorted"]), f2s)
        G.assert_close(G.host(out["topk_w"]), w, "topk_w", atol=1e-6, rtol=1e-5)


def test_noalloc_route_on_explicit_stream():
    """The same call queued on a side stream gives the same bits."""
    torch = G.torch_mod()
    import mixture_experts_layer_expert_amd as moe
    T, E, K = 2048, 128, 8
    logits = G.to_dev(_logits(T, E, seed=7))
    ref = moe.moe_route_sort(logits, K, 0)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    out = _outputs(torch, T, E, K)
    torch.cuda.synchronize()
    moe.moe_route_sort_noalloc(logits, K, 0, out=out, stream=side)
    side.synchronize()
    for k in ref:
        assert torch.equal(out[k], ref[k]), k

"""CPU checks of bench.py's host logic: its table of algorithmic work per
kernel names only kernels the library has, and prices every grouped GEMM in
matrix FLOPs and every other kernel of the step in HBM bytes."""
import bench
import synth
import mixture_experts_layer_expert_amd as moe


def _kernel_names():
    lib = moe.load_library()
    return {lib.moe_prof_kernel_name(i).decode() for i in range(lib.moe_prof_num_kernels())}


def test_work_table_names_library_kernels():
    names = _kernel_names()
    for wl in (synth.QWEN3_30B_A3B, synth.LLAMA4_SCOUT, synth.TINY):
        work = bench.kernel_work(wl)
        assert set(work) <= names, set(work) - names
        gemms = {n for n in names if n.startswith("gemm_")}
        assert gemms <= set(work)
        for n, (bound, amount) in work.items():
            assert bound in ("mfma", "mfma32", "hbm"), n
            assert amount >= 0, n
            assert (bound == "mfma") == n.startswith("gemm_"), n


def test_gemm_flops_add_up_to_the_counted_step():
    """The seven grouped GEMMs' algorithmic FLOPs are the step's counted 18 D I
    per routed row plus the recompute's 4 D I, whether gate/up + down and dA +
    the recompute run as four launches or as two chained ones."""
    wl = synth.QWEN3_30B_A3B
    work = bench.kernel_work(wl)
    separate = ["gemm_gateup_h", "gemm_down", "gemm_da", "gemm_gateup_gu", "gemm_bwd_fused"]
    chained = ["gemm_fwd_chain", "gemm_da_recompute", "gemm_bwd_fused"]
    assert sorted(n for n, (b, _) in work.items() if b == "mfma") == sorted(set(separate + chained))
    for names in (separate, chained):
        assert sum(work[n][1] for n in names) == (18 + 4) * wl.D * wl.I * wl.R
    assert wl.flops_fwd() + wl.flops_bwd() == 18 * wl.D * wl.I * wl.R


def test_step_stats_and_host_cpu():
    st = bench.step_stats([3.0, 1.0, 2.0, 4.0, 5.0])
    assert st["median"] == 3.0 and st["min"] == 1.0 and st["max"] == 5.0 and st["n"] == 5
    assert st["p10"] <= st["median"] <= st["p90"]
    h = bench.host_cpu()
    assert h["nproc"] >= 1 and h["cpus_on_host"] >= h["nproc"] and isinstance(h["cpu_model"], str)


def test_gemm_min_bytes_and_ceilings():
    """Every grouped GEMM kernel the library launches has its unavoidable bytes;
    at the Qwen3-30B-A3B shape their arithmetic intensities put gate/up and dA
    above the MFMA ridge (312 FLOP/B at 2.5 PFLOP/s and 8 TB/s) and the fused
    dXs + dW launch below it."""
    wl = synth.QWEN3_30B_A3B
    mb = bench.gemm_min_bytes(wl)
    work = bench.kernel_work(wl)
    names = _kernel_names()
    assert set(mb) == {n for n in names if n.startswith("gemm_")}
    ai = {k: work[k][1] / v for k, v in mb.items()}
    assert all(v > 0 for v in mb.values())
    assert ai["gemm_gateup_h"] > 312 and ai["gemm_da"] > 312 and ai["gemm_bwd_fused"] < 312

"""CPU-only checks of the C-ABI library: it loads without a GPU, exports
exactly the functions that include/moe.h declares, links no torch, and its
host-side validation rejects bad arguments before anything is launched."""
import ctypes
import os
import subprocess

import pytest

import mixture_experts_layer_expert_amd as moe
from mixture_experts_layer_expert_amd import binding

LIB = binding.LIB_PATH


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} not built (run python -m mixture_experts_layer_expert_amd.build)")
    return moe.load_library()


def test_exports_match_header(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = sorted(l.split()[-1] for l in out.splitlines() if " T " in l)
    assert exported == binding.header_functions()
    for name in exported:
        assert hasattr(lib, name)


def test_no_torch_dependency(lib):
    out = subprocess.run(["readelf", "-d", LIB], capture_output=True, text=True, check=True).stdout
    needed = [l for l in out.splitlines() if "NEEDED" in l]
    assert not any("torch" in l or "c10" in l for l in needed), needed


def test_version_and_status_strings(lib):
    assert lib.moe_abi_version() == 4
    for code in range(6):
        assert moe.status_string(code)


def test_workspace_bytes_host_only(lib):
    q = moe.dims(8192, 2048, 768, 128, 8)
    sizes = [moe.moe_workspace_bytes(q, ph) for ph in range(4)]
    assert all(s > 0 for s in sizes)
    # backward holds Xs, dOu, GU, dGU, Hw, dXs in bf16 + fp32 partials at least
    R = 8192 * 8
    assert sizes[2] >= R * (2048 * 2 * 3 + 768 * 2 * 5)
    assert moe.moe_workspace_bytes(moe.dims(8192, 2048, 768, 128, 8), 7) == 0
    assert moe.moe_workspace_bytes(moe.dims(16, 100, 64, 8, 2), 1) == 0          # D % 64
    assert moe.moe_workspace_bytes(moe.dims(16, 64, 64, 4, 5), 1) == 0           # K > E
    small = moe.moe_workspace_bytes(moe.dims(16, 64, 64, 4, 2), 2)
    big = moe.moe_workspace_bytes(moe.dims(32, 64, 64, 4, 2), 2)
    assert 0 < small <= big


def test_operand_size_limit(lib):
    """The GEMMs address the routed-row operands with 32-bit byte offsets: at
    the Qwen3-30B-A3B layer shape T = 65535 tokens is the largest batch (R * D * 2
    just under 2^31), T = 65536 is refused before anything is launched."""
    ok = moe.dims(65535, 2048, 768, 128, 8)
    assert all(moe.moe_workspace_bytes(ok, ph) > 0 for ph in range(4))
    over = moe.dims(65536, 2048, 768, 128, 8)
    assert all(moe.moe_workspace_bytes(over, ph) == 0 for ph in range(4))
    assert _fwd(lib, over) == 2
    # the Scout shape's bound is the 2I-wide operands: T = 65536 gives exactly 2^31 bytes
    assert moe.moe_workspace_bytes(moe.dims(65535, 5120, 8192, 16, 1, 1), 2) > 0
    assert _fwd(lib, moe.dims(65536, 5120, 8192, 16, 1, 1)) == 2


def test_backward_workspace_holds_dw_chunk_partials(lib):
    """The backward workspace grows by ceil(R / 4096) partial dW tiles of 3*I*D
    fp32 (dW_gate | dW_up, and dW_down apart, since the two dW GEMMs run in one
    launch) as the routed rows grow (the dW row chunks of hot experts)."""
    a = moe.moe_workspace_bytes(moe.dims(8192, 2048, 768, 128, 8), 2)
    b = moe.moe_workspace_bytes(moe.dims(8192 + 256, 2048, 768, 128, 8), 2)  # +2048 routed rows
    per_row = 2 * 2048 * 2 + 2 * 768 * (4 + 2 * 2 + 2 * 2) + 2048 * 4 + 4 * 4 * 3
    assert b - a >= 3 * 768 * 2048 * 4          # one more partial slot at least
    assert b - a <= 2048 * per_row + 3 * 768 * 2048 * 4 + 4096


FAKE = ctypes.c_void_p(1 << 20)      # aligned, never dereferenced: validation fails first


def _fwd(lib, d, ws_bytes=1 << 40, x=FAKE):
    return lib.moe_fwd(ctypes.byref(d), x, *([FAKE] * 8), FAKE, ctypes.c_size_t(ws_bytes), None)


@pytest.mark.parametrize("dims,code", [
    ((16, 100, 64, 8, 2, 0), 2),     # D not a multiple of 64
    ((16, 64, 96, 8, 2, 0), 2),      # I not a multiple of 64
    ((16, 64, 64, 2000, 2, 0), 2),   # E > 1024
    ((16, 64, 64, 128, 65, 0), 2),   # K > 64
    ((16, 64, 64, 4, 5, 0), 1),      # K > E
    ((16, 64, 64, 4, 0, 0), 1),      # K = 0
    ((-1, 64, 64, 4, 2, 0), 1),      # T < 0
    ((16, 64, 64, 4, 2, 3), 1),      # unknown score
    ((1 << 28, 64, 64, 16, 8, 0), 1),  # T*K >= 2^31
])
def test_bad_dims_rejected(lib, dims, code):
    d = moe.dims(*dims)
    assert _fwd(lib, d) == code
    assert lib.moe_route_sort(ctypes.byref(d), *([FAKE] * 8), ctypes.c_size_t(1 << 40), None) == code
    assert lib.moe_route_sort_noalloc(ctypes.byref(d), *([FAKE] * 7), None) == code


def test_noalloc_route_validates_before_touching_a_device(lib):
    """The allocation-free routing call checks its arguments on the host first
    (no device is needed to reject them)."""
    d = moe.dims(16, 64, 64, 4, 2)
    assert lib.moe_route_sort_noalloc(None, *([FAKE] * 7), None) == 1
    assert lib.moe_route_sort_noalloc(ctypes.byref(d), ctypes.c_void_p(0), *([FAKE] * 6),
                                      None) == 1                        # null logits
    assert lib.moe_route_sort_noalloc(ctypes.byref(d), FAKE, ctypes.c_void_p((1 << 20) + 2),
                                      *([FAKE] * 5), None) == 1         # misaligned topk_idx


def test_noalloc_route_source_allocates_nothing():
    """moe_route_sort_noalloc and its scratch lookup call no allocating routine."""
    src = open(os.path.join(os.path.dirname(moe.__file__), "csrc", "abi.hip")).read()
    start = src.index("// ---- allocation-free routing")
    end = src.index("MOE_EXPORT moe_status moe_fwd(")
    body = src[start:end]
    assert "hipGetSymbolAddress" in body and "HIP_SYMBOL(scratch)" in body
    for banned in ("hipMalloc", "hipFree", "hipHostMalloc", "hipExtMalloc", "hipMallocAsync",
                   "new ", "malloc("):
        assert banned not in body, banned
    # kernels get the looked-up device address, never the host-side name of the array
    assert "launch_route_sort(" in body and "scratch," not in body.split("launch_route_sort(")[1]


def test_bad_pointers_and_workspace(lib):
    d = moe.dims(16, 64, 64, 4, 2)
    assert _fwd(lib, d, x=ctypes.c_void_p(0)) == 1                    # null
    assert _fwd(lib, d, x=ctypes.c_void_p((1 << 20) + 8)) == 1        # bf16 matrix not 16-B aligned
    assert _fwd(lib, d, ws_bytes=16) == 3                              # workspace too small
    assert lib.moe_fwd(None, *([FAKE] * 10), ctypes.c_size_t(1 << 40), None) == 1
    bwd_args = [FAKE] * 14
    assert lib.moe_bwd(ctypes.byref(d), *bwd_args, ctypes.c_int32(2), FAKE,
                       ctypes.c_size_t(1 << 40), None) == 1           # accumulate_dw not 0/1
    assert lib.moe_bwd(ctypes.byref(d), *bwd_args, ctypes.c_int32(0), FAKE,
                       ctypes.c_size_t(8), None) == 3


def test_router_bad_args(lib):
    d = moe.dims(16, 64, 64, 4, 2)
    assert lib.moe_router_fwd(ctypes.byref(moe.dims(16, 100, 64, 4, 2)), FAKE, FAKE, FAKE,
                              None) == 2                                # D % 64
    assert lib.moe_router_fwd(ctypes.byref(d), ctypes.c_void_p(0), FAKE, FAKE, None) == 1
    assert lib.moe_router_fwd(ctypes.byref(d), FAKE, ctypes.c_void_p((1 << 20) + 4), FAKE,
                              None) == 1                                # w_r not 16-B aligned
    args = [FAKE] * 7
    assert lib.moe_router_bwd(ctypes.byref(d), *args, ctypes.c_int32(2), FAKE,
                              ctypes.c_size_t(1 << 40), None) == 1      # accumulate_dwr not 0/1
    assert lib.moe_router_bwd(ctypes.byref(d), *args, ctypes.c_int32(0), FAKE,
                              ctypes.c_size_t(8), None) == 3            # workspace too small
    assert lib.moe_router_bwd(ctypes.byref(d), *args[:6], ctypes.c_void_p(0), ctypes.c_int32(0),
                              FAKE, ctypes.c_size_t(1 << 40), None) == 1  # null dw_r
    need = moe.moe_workspace_bytes(d, moe.MOE_PHASE_ROUTER_BWD)
    assert need >= 4 * (64 * 4 + 16 * 2 + 64 * 4)    # W_r^T, dl, one partial of dW_r


def test_missing_library_fails_loudly(tmp_path):
    """No CPU fallback: a missing library is an error, not a silent substitute."""
    saved = binding._lib
    try:
        binding._lib = None
        with pytest.raises(binding.MoeError):
            binding.load_library(str(tmp_path / "libmoe.so"))
    finally:
        binding._lib = saved


def test_prof_names(lib):
    n = lib.moe_prof_num_kernels()
    names = [lib.moe_prof_kernel_name(i) for i in range(n)]
    assert all(names) and len(set(names)) == n
    assert lib.moe_prof_kernel_name(n) is None


def test_product_path_never_touches_oracle():
    """The HIP package and its binding do not import or name the CPU oracle."""
    pkg = os.path.dirname(moe.__file__)
    for root, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(root, f)).read()
                assert "import oracle" not in text and "moe_oracle" not in text, f


def test_single_hip_runtime(lib):
    """libmoe binds to the HIP runtime that torch already loaded (same soname);
    two runtimes in one process leave the second without a device."""
    maps = open("/proc/self/maps").read().splitlines()
    paths = {l.split()[-1] for l in maps if "libamdhip64" in l}
    assert len(paths) == 1, paths

"""ctypes binding of libmoe (include/moe.h).

Argument marshalling only: torch supplies device memory and the HIP stream
(the current one, or the `stream=` argument); every step of the layer runs in the library's HIP kernels.  There is
no CPU fallback: if the library is missing or a call fails, an exception is
raised.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "moe.h")

MOE_SCORE_SOFTMAX_TOPK = 0
MOE_SCORE_SIGMOID = 1
MOE_PHASE_ROUTE, MOE_PHASE_FWD, MOE_PHASE_BWD, MOE_PHASE_ROUTER_BWD = 0, 1, 2, 3
MOE_OK = 0


class MoeError(RuntimeError):
    pass


class moe_dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("D", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("K", ctypes.c_int32), ("score", ctypes.c_int32)]

    def __repr__(self):
        return (f"moe_dims(T={self.T}, D={self.D}, I={self.I}, E={self.E}, K={self.K}, "
                f"score={self.score})")


_lib = None
_vp = ctypes.c_void_p


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmoe.so (raises if it has not been built).

    torch is imported first: torch ships its own HIP runtime under the same
    soname (libamdhip64.so.7), so loading torch first makes the dynamic loader
    bind libmoe to that already-loaded runtime.  Loading libmoe first would
    bring in a second HIP runtime, which then finds no device.
    """
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (see above: one HIP runtime per process)
        if not os.path.exists(path):
            raise MoeError(f"{path} is missing: build it with "
                           "`python -m mixture_experts_layer_expert_amd.build`")
        lib = ctypes.CDLL(path)
        lib.moe_workspace_bytes.restype = ctypes.c_size_t
        lib.moe_workspace_bytes.argtypes = [ctypes.POINTER(moe_dims), ctypes.c_int32]
        lib.moe_route_sort.restype = ctypes.c_int32
        lib.moe_route_sort.argtypes = [ctypes.POINTER(moe_dims)] + [_vp] * 7 + [_vp, ctypes.c_size_t, _vp]
        lib.moe_route_sort_noalloc.restype = ctypes.c_int32
        lib.moe_route_sort_noalloc.argtypes = [ctypes.POINTER(moe_dims)] + [_vp] * 7 + [_vp]
        lib.moe_fwd.restype = ctypes.c_int32
        lib.moe_fwd.argtypes = [ctypes.POINTER(moe_dims)] + [_vp] * 9 + [_vp, ctypes.c_size_t, _vp]
        lib.moe_bwd.restype = ctypes.c_int32
        lib.moe_bwd.argtypes = ([ctypes.POINTER(moe_dims)] + [_vp] * 14 + [ctypes.c_int32] +
                                [_vp, ctypes.c_size_t, _vp])
        lib.moe_router_fwd.restype = ctypes.c_int32
        lib.moe_router_fwd.argtypes = [ctypes.POINTER(moe_dims)] + [_vp] * 3 + [_vp]
        lib.moe_router_bwd.restype = ctypes.c_int32
        lib.moe_router_bwd.argtypes = ([ctypes.POINTER(moe_dims)] + [_vp] * 7 + [ctypes.c_int32] +
                                       [_vp, ctypes.c_size_t, _vp])
        lib.moe_status_string.restype = ctypes.c_char_p
        lib.moe_status_string.argtypes = [ctypes.c_int32]
        lib.moe_abi_version.restype = ctypes.c_int32
        lib.moe_abi_version.argtypes = []
        lib.moe_last_error.restype = ctypes.c_char_p
        lib.moe_last_error.argtypes = []
        lib.moe_prof_enable.restype = ctypes.c_int32
        lib.moe_prof_enable.argtypes = [ctypes.c_int32]
        lib.moe_prof_only.restype = ctypes.c_int32
        lib.moe_prof_only.argtypes = [ctypes.c_int32]
        lib.moe_prof_num_kernels.restype = ctypes.c_int32
        lib.moe_prof_num_kernels.argtypes = []
        lib.moe_prof_kernel_name.restype = ctypes.c_char_p
        lib.moe_prof_kernel_name.argtypes = [ctypes.c_int32]
        lib.moe_prof_read.restype = ctypes.c_int32
        lib.moe_prof_read.argtypes = [_vp, _vp, ctypes.c_int32]
        _lib = lib
    return _lib


def header_functions(path: str = HEADER) -> list:
    """Names of the functions that include/moe.h declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def status_string(code: int) -> str:
    return load_library().moe_status_string(code).decode()


def _check(code: int, what: str) -> None:
    if code != MOE_OK:
        detail = load_library().moe_last_error().decode()
        raise MoeError(f"{what} failed: status {code} ({status_string(code)})"
                       + (f": {detail}" if detail else ""))


def dims(T, D, I, E, K, score=MOE_SCORE_SOFTMAX_TOPK) -> moe_dims:
    return moe_dims(int(T), int(D), int(I), int(E), int(K), int(score))


def moe_workspace_bytes(d: moe_dims, phase: int) -> int:
    return int(load_library().moe_workspace_bytes(ctypes.byref(d), int(phase)))


# ----------------------------------------------------------------------------- torch marshalling

def _torch():
    import torch
    return torch


def _ptr(t, dtype, shape, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor")
    if not t.is_cuda:
        raise MoeError(f"{name}: must be a GPU tensor")
    if t.device.index != torch.cuda.current_device():
        raise MoeError(f"{name}: on {t.device}, but the current device is "
                       f"cuda:{torch.cuda.current_device()} (the library runs there)")
    if t.dtype != dtype:
        raise MoeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise MoeError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise MoeError(f"{name}: must be contiguous")
    return _vp(t.data_ptr())


def _launch_stream(stream):
    """The stream the library's kernels go to: `stream`, else the current one."""
    torch = _torch()
    return torch.cuda.current_stream() if stream is None else stream


def _alloc_on(stream):
    """Context in which this call allocates its workspace and default outputs.

    The caching allocator ties a block to the stream that was current when it
    was allocated and hands it out again, once freed, only to later work on
    that stream.  Allocating on the launch stream keeps a workspace freed when
    the call returns from being reused by other streams while the kernels
    queued on `stream` may still use it."""
    return _torch().cuda.stream(stream)


def _workspace(d, phase, ws, device):
    torch = _torch()
    need = moe_workspace_bytes(d, phase)
    if need == 0:
        raise MoeError(f"invalid dims {d!r}")
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    return ws, need


def moe_route_sort(logits, K: int, score: int = MOE_SCORE_SOFTMAX_TOPK, *, out=None, ws=None,
                   stream=None) -> dict:
    """Routing + sort by expert.  logits: fp32 [T, E] on the GPU.

    Returns dict(topk_idx, topk_w, counts, offsets, sorted_to_flat, flat_to_sorted).
    """
    torch = _torch()
    T, E = logits.shape
    d = dims(T, 64, 64, E, K, score)
    dev = logits.device
    st = _launch_stream(stream)
    with _alloc_on(st):
        if out is None:
            out = dict(topk_idx=torch.empty((T, K), dtype=torch.int32, device=dev),
                       topk_w=torch.empty((T, K), dtype=torch.float32, device=dev),
                       counts=torch.empty(E, dtype=torch.int32, device=dev),
                       offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                       sorted_to_flat=torch.empty(T * K, dtype=torch.int32, device=dev),
                       flat_to_sorted=torch.empty(T * K, dtype=torch.int32, device=dev))
        ws, need = _workspace(d, MOE_PHASE_ROUTE, ws, dev)
    i32, f32 = torch.int32, torch.float32
    rc = load_library().moe_route_sort(
        ctypes.byref(d), _ptr(logits, f32, (T, E), "logits"),
        _ptr(out["topk_idx"], i32, (T, K), "topk_idx"), _ptr(out["topk_w"], f32, (T, K), "topk_w"),
        _ptr(out["counts"], i32, (E,), "counts"), _ptr(out["offsets"], i32, (E + 1,), "offsets"),
        _ptr(out["sorted_to_flat"], i32, (T * K,), "sorted_to_flat"),
        _ptr(out["flat_to_sorted"], i32, (T * K,), "flat_to_sorted"),
        _vp(ws.data_ptr()), ctypes.c_size_t(ws.numel() * ws.element_size()), _vp(st.cuda_stream))
    _check(rc, "moe_route_sort")
    return out


def moe_route_sort_noalloc(logits, K: int, score: int = MOE_SCORE_SOFTMAX_TOPK, *, out,
                           stream=None) -> dict:
    """moe_route_sort without a workspace: the library's static scratch holds the
    histograms.  `out` (the dict moe_route_sort returns) must be given, so that
    the call allocates nothing."""
    torch = _torch()
    T, E = logits.shape
    d = dims(T, 64, 64, E, K, score)
    st = _launch_stream(stream)
    i32, f32 = torch.int32, torch.float32
    rc = load_library().moe_route_sort_noalloc(
        ctypes.byref(d), _ptr(logits, f32, (T, E), "logits"),
        _ptr(out["topk_idx"], i32, (T, K), "topk_idx"), _ptr(out["topk_w"], f32, (T, K), "topk_w"),
        _ptr(out["counts"], i32, (E,), "counts"), _ptr(out["offsets"], i32, (E + 1,), "offsets"),
        _ptr(out["sorted_to_flat"], i32, (T * K,), "sorted_to_flat"),
        _ptr(out["flat_to_sorted"], i32, (T * K,), "flat_to_sorted"), _vp(st.cuda_stream))
    _check(rc, "moe_route_sort_noalloc")
    return out


def _layer_dims(x, w_gate, K, score):
    T, D = x.shape
    E, I, _ = w_gate.shape
    return dims(T, D, I, E, K, score)


def moe_fwd(x, w_gate, w_up, w_down, route: dict, K: int, score: int = MOE_SCORE_SOFTMAX_TOPK, *,
            y=None, ws=None, stream=None):
    """Forward.  x bf16 [T, D]; w_gate, w_up bf16 [E, I, D]; w_down bf16 [E, D, I];
    route: the dict returned by moe_route_sort.  Returns y bf16 [T, D]."""
    torch = _torch()
    d = _layer_dims(x, w_gate, K, score)
    T, D, I, E = d.T, d.D, d.I, d.E
    st = _launch_stream(stream)
    with _alloc_on(st):
        if y is None:
            y = torch.empty((T, D), dtype=torch.bfloat16, device=x.device)
        ws, need = _workspace(d, MOE_PHASE_FWD, ws, x.device)
    b, i32, f32 = torch.bfloat16, torch.int32, torch.float32
    rc = load_library().moe_fwd(
        ctypes.byref(d), _ptr(x, b, (T, D), "x"), _ptr(w_gate, b, (E, I, D), "w_gate"),
        _ptr(w_up, b, (E, I, D), "w_up"), _ptr(w_down, b, (E, D, I), "w_down"),
        _ptr(route["topk_w"], f32, (T, K), "topk_w"), _ptr(route["offsets"], i32, (E + 1,), "offsets"),
        _ptr(route["sorted_to_flat"], i32, (T * K,), "sorted_to_flat"),
        _ptr(route["flat_to_sorted"], i32, (T * K,), "flat_to_sorted"),
        _ptr(y, b, (T, D), "y"), _vp(ws.data_ptr()), ctypes.c_size_t(ws.numel() * ws.element_size()),
        _vp(st.cuda_stream))
    _check(rc, "moe_fwd")
    return y


def moe_bwd(x, w_gate, w_up, w_down, route: dict, dy, K: int, score: int = MOE_SCORE_SOFTMAX_TOPK,
            *, out=None, accumulate_dw: bool = False, ws=None, stream=None) -> dict:
    """Backward with routing held fixed.  Returns dict(dx bf16 [T,D], dw_gate fp32 [E,I,D],
    dw_up fp32 [E,I,D], dw_down fp32 [E,D,I], d_topk_w fp32 [T,K])."""
    torch = _torch()
    d = _layer_dims(x, w_gate, K, score)
    T, D, I, E = d.T, d.D, d.I, d.E
    dev = x.device
    st = _launch_stream(stream)
    with _alloc_on(st):
        if out is None:
            out = dict(dx=torch.empty((T, D), dtype=torch.bfloat16, device=dev),
                       dw_gate=torch.empty((E, I, D), dtype=torch.float32, device=dev),
                       dw_up=torch.empty((E, I, D), dtype=torch.float32, device=dev),
                       dw_down=torch.empty((E, D, I), dtype=torch.float32, device=dev),
                       d_topk_w=torch.empty((T, K), dtype=torch.float32, device=dev))
        ws, need = _workspace(d, MOE_PHASE_BWD, ws, dev)
    b, i32, f32 = torch.bfloat16, torch.int32, torch.float32
    rc = load_library().moe_bwd(
        ctypes.byref(d), _ptr(x, b, (T, D), "x"), _ptr(w_gate, b, (E, I, D), "w_gate"),
        _ptr(w_up, b, (E, I, D), "w_up"), _ptr(w_down, b, (E, D, I), "w_down"),
        _ptr(route["topk_w"], f32, (T, K), "topk_w"), _ptr(route["offsets"], i32, (E + 1,), "offsets"),
        _ptr(route["sorted_to_flat"], i32, (T * K,), "sorted_to_flat"),
        _ptr(route["flat_to_sorted"], i32, (T * K,), "flat_to_sorted"),
        _ptr(dy, b, (T, D), "dy"), _ptr(out["dx"], b, (T, D), "dx"),
        _ptr(out["dw_gate"], f32, (E, I, D), "dw_gate"), _ptr(out["dw_up"], f32, (E, I, D), "dw_up"),
        _ptr(out["dw_down"], f32, (E, D, I), "dw_down"), _ptr(out["d_topk_w"], f32, (T, K), "d_topk_w"),
        ctypes.c_int32(1 if accumulate_dw else 0),
        _vp(ws.data_ptr()), ctypes.c_size_t(ws.numel() * ws.element_size()), _vp(st.cuda_stream))
    _check(rc, "moe_bwd")
    return out


def _router_dims(x, w_r, K, score):
    T, D = x.shape
    E = w_r.shape[1]
    return dims(T, D, 64, E, K, score)


def moe_router_fwd(x, w_r, *, logits=None, stream=None):
    """Router projection.  x bf16 [T, D]; w_r fp32 [D, E].  Returns logits fp32 [T, E]."""
    torch = _torch()
    d = _router_dims(x, w_r, 1, MOE_SCORE_SOFTMAX_TOPK)
    T, D, E = d.T, d.D, d.E
    st = _launch_stream(stream)
    if logits is None:
        with _alloc_on(st):
            logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    rc = load_library().moe_router_fwd(
        ctypes.byref(d), _ptr(x, torch.bfloat16, (T, D), "x"),
        _ptr(w_r, torch.float32, (D, E), "w_r"), _ptr(logits, torch.float32, (T, E), "logits"),
        _vp(st.cuda_stream))
    _check(rc, "moe_router_fwd")
    return logits


def moe_router_bwd(x, w_r, route: dict, d_topk_w, dx, K: int,
                   score: int = MOE_SCORE_SOFTMAX_TOPK, *, dw_r=None,
                   accumulate_dwr: bool = False, ws=None, stream=None):
    """Router backward, selection fixed.  Adds the router path's input gradient
    into dx (bf16 [T, D], in place) and returns dw_r fp32 [D, E]."""
    torch = _torch()
    d = _router_dims(x, w_r, K, score)
    T, D, E = d.T, d.D, d.E
    st = _launch_stream(stream)
    with _alloc_on(st):
        if dw_r is None:
            dw_r = torch.empty((D, E), dtype=torch.float32, device=x.device)
        ws, need = _workspace(d, MOE_PHASE_ROUTER_BWD, ws, x.device)
    b, i32, f32 = torch.bfloat16, torch.int32, torch.float32
    rc = load_library().moe_router_bwd(
        ctypes.byref(d), _ptr(x, b, (T, D), "x"), _ptr(w_r, f32, (D, E), "w_r"),
        _ptr(route["topk_idx"], i32, (T, K), "topk_idx"), _ptr(route["topk_w"], f32, (T, K), "topk_w"),
        _ptr(d_topk_w, f32, (T, K), "d_topk_w"), _ptr(dx, b, (T, D), "dx"),
        _ptr(dw_r, f32, (D, E), "dw_r"), ctypes.c_int32(1 if accumulate_dwr else 0),
        _vp(ws.data_ptr()), ctypes.c_size_t(ws.numel() * ws.element_size()), _vp(st.cuda_stream))
    _check(rc, "moe_router_bwd")
    return dw_r


# ----------------------------------------------------------------------------- per-kernel timing

def moe_prof_enable(on: bool) -> None:
    """Start (True) or stop (False) per-kernel event timing; clears what was recorded."""
    load_library().moe_prof_enable(1 if on else 0)


def moe_prof_only(kernel: str | None) -> None:
    """Bracket only the named kernel (None: every kernel) while timing is enabled."""
    lib = load_library()
    kid = -1
    if kernel is not None:
        names = {lib.moe_prof_kernel_name(i).decode(): i for i in range(lib.moe_prof_num_kernels())}
        if kernel not in names:
            raise MoeError(f"unknown kernel {kernel!r}")
        kid = names[kernel]
    _check(lib.moe_prof_only(kid), "moe_prof_only")


def moe_prof_read() -> dict:
    """{kernel name: (total ms, launches)} for kernels launched since moe_prof_enable(True)."""
    lib = load_library()
    n = lib.moe_prof_num_kernels()
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int64 * n)()
    _check(lib.moe_prof_read(ctypes.cast(ms, _vp), ctypes.cast(cnt, _vp), n), "moe_prof_read")
    return {lib.moe_prof_kernel_name(i).decode(): (ms[i], cnt[i]) for i in range(n) if cnt[i]}

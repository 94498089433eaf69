"""Routed SwiGLU mixture-of-experts layer (router projection, routing + sort,
forward, backward, router backward) on AMD Instinct MI355X (gfx950):
hand-written HIP kernels behind the C ABI in include/moe.h, with a thin ctypes
binding (``binding``)."""
from .binding import (MOE_PHASE_BWD, MOE_PHASE_FWD, MOE_PHASE_ROUTE, MOE_PHASE_ROUTER_BWD,
                      MOE_SCORE_SIGMOID, MOE_SCORE_SOFTMAX_TOPK, MoeError, dims, load_library,
                      moe_bwd, moe_dims, moe_fwd, moe_prof_enable, moe_prof_only, moe_prof_read,
                      moe_route_sort, moe_route_sort_noalloc, moe_router_bwd, moe_router_fwd, moe_workspace_bytes,
                      status_string)

__all__ = ["MOE_PHASE_BWD", "MOE_PHASE_FWD", "MOE_PHASE_ROUTE", "MOE_PHASE_ROUTER_BWD",
           "MOE_SCORE_SIGMOID", "MOE_SCORE_SOFTMAX_TOPK", "MoeError", "dims", "load_library",
           "moe_bwd", "moe_dims", "moe_fwd", "moe_prof_enable", "moe_prof_only", "moe_prof_read",
           "moe_route_sort", "moe_route_sort_noalloc", "moe_router_bwd", "moe_router_fwd", "moe_workspace_bytes",
           "status_string"]

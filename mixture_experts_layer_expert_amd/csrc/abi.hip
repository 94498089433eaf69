// extern "C" entry points of libmoe: host-side validation, workspace
// carving and the launch sequences of route+sort, forward and backward.
// Nothing here reads device memory or synchronises with the host.
#include <stdio.h>

#include <algorithm>
#include <mutex>

#include "kernels.hpp"

#define MOE_EXPORT extern "C" __attribute__((visibility("default")))

namespace moe {
namespace {

constexpr size_t kAlign = 256;
constexpr int kMaxE = 1024;
static_assert(kMaxE <= kChunkMapMaxE, "the dW chunk map takes one expert per thread");
constexpr int kMaxK = 64;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// A pointer argument is acceptable if its array is empty, or if it is non-null
// and aligned to `a` bytes.
bool ptr_ok(const void* p, size_t count, size_t a) { return count == 0 || (p && aligned(p, a)); }

// Column tiles of the fused gate/up GEMM: 128 gate + 128 up rows per tile.
int64_t gateup_tiles(int64_t I) { return (I + kGemmBN / 2 - 1) / (kGemmBN / 2); }

// MOE_OK, or why the dims are rejected.
moe_status check_dims(const moe_dims* d) {
  if (!d) return MOE_ERR_BAD_ARG;
  if (d->T < 0 || d->D <= 0 || d->I <= 0 || d->E <= 0 || d->K <= 0 || d->K > d->E)
    return MOE_ERR_BAD_ARG;
  if (d->score != MOE_SCORE_SOFTMAX_TOPK && d->score != MOE_SCORE_SIGMOID) return MOE_ERR_BAD_ARG;
  if ((int64_t)d->T * d->K >= (int64_t(1) << 31)) return MOE_ERR_BAD_ARG;
  if (d->D % 64 || d->I % 64 || d->E > kMaxE || d->K > kMaxK) return MOE_ERR_UNSUPPORTED;
  // tile counts of the grouped GEMMs must fit in 32-bit grids
  const int64_t R = (int64_t)d->T * d->K;
  const int64_t mt = (R + (int64_t)d->E * (kGemmBM - 1)) / kGemmBM;
  // the chained launches (gate/up + down, dA + recompute): kNumXcd ranges of
  // at most ceil(mt / kNumXcd) + 2 kChainSlack m-tiles, each with both GEMMs'
  // column tiles (the tile indices of an XCD's range)
  const int64_t mtx = ((mt + kNumXcd - 1) / kNumXcd + 2 * kChainSlack) * kNumXcd;
  const int64_t ntd = (d->D + kGemmBN - 1) / kGemmBN, nti = (d->I + kGemmBN - 1) / kGemmBN;
  if (mtx * (gateup_tiles(d->I) + std::max(ntd, nti)) >= (int64_t(1) << 31) ||
      kNumXcd * (2 * ((mt * (gateup_tiles(d->I) + ntd) + kNumXcd - 1) / kNumXcd) + 2) >=
          (int64_t(1) << 31))
    return MOE_ERR_UNSUPPORTED;
  // the dW grids as launched (dw_grid below: the (matrix, row chunk) groups
  // rounded up to a multiple of the XCD count)
  const int64_t per_c = ((d->I + kGemmBM - 1) / kGemmBM) * ((d->D + kGemmBN - 1) / kGemmBN);
  const int64_t groups = 2 * (d->E + (R + kDwChunkRows - 1) / kDwChunkRows);
  if ((groups + kNumXcd - 1) / kNumXcd * kNumXcd * per_c >= (int64_t(1) << 31))
    return MOE_ERR_UNSUPPORTED;
  // the fused backward launch: the dXs grid and both dW grids in one
  const int64_t chunks = d->E + (R + kDwChunkRows - 1) / kDwChunkRows;
  const int64_t per_d = ((d->D + kGemmBM - 1) / kGemmBM) * ((d->I + kGemmBN - 1) / kGemmBN);
  const int64_t per_g = ((d->I + kGemmBM - 1) / kGemmBM) * ((d->D + kGemmBN - 1) / kGemmBN);
  const int64_t fused = kNumXcd * (2 * ((mt * ntd + kNumXcd - 1) / kNumXcd) + 2) + (chunks + kNumXcd) * per_d +
                        (2 * chunks + kNumXcd) * per_g;
  if (fused >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  // the GEMMs address token-major operands with 32-bit buffer offsets
  if (R * std::max<int64_t>(d->D, 2 * (int64_t)d->I) * 2 >= (int64_t(1) << 31) ||
      (int64_t)d->I * d->D * 2 >= (int64_t(1) << 31))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

struct Carve {
  char* base;
  size_t used = 0;
  template <typename T>
  T* take(size_t count) {
    T* p = reinterpret_cast<T*>(base ? base + used : nullptr);
    used += align_up(count * sizeof(T));
    return p;
  }
};

struct FwdWs {
  // chain[0]: status word of the call (nonzero: a chained launch's wait gave
  // up, or a workgroup ran on an unexpected XCD); chain[1 .. kNumXcd + 1]: the
  // XCDs' m-tile ranges; then the per-m-tile counters of the chained launch.
  // Set by the call's first kernel.
  int32_t* chain;
  int32_t* tstart;
  f16_t* h;   // SwiGLU activations H [R, I], fp16 (the down GEMM's operand)
  bf16_t* o;  // unweighted expert outputs O [R, D]
};
struct BwdWs {
  int32_t* chain;  // as FwdWs::chain
  int32_t* tstart;
  f16_t *dgu, *hw;        // fp16 operands of the gradient GEMMs (rounded values)
  f16_t *dgu_lo, *hw_lo;  // their low parts (value - rounded value), for the dW GEMMs
  uint32_t* rowoff;       // byte offset of each routed row's token row in x / dy
  int32_t *cstart, *pstart, *slist, *corder;  // dW row-chunk map
  int32_t* dw_split;      // per-expert flag: dW operand split hi + lo
  uint32_t* amax_part;    // partial maxima of |dy|
  float* gscale;          // gradient scale {s, 1/s}
  f16_t *x16, *dy16;      // fp16 x and s dy, token-major: the dW GEMMs' exact operands
  // partial dW tiles of chunks 1.. of the chunked experts: dW_gate | dW_up, and
  // dW_down apart (the two dW GEMMs run in one launch)
  float *dw_part, *dw_part_down;
  float* da;     // dA [R, I]
  f16_t* dxs;    // s dXs rows [R, D] fp16, flat slot order
  float* part;   // dRW partials
};

// dW row chunks: experts with more than kDwChunkRows rows (at most R / (chunk + 1)
// of them), the partial tiles of their chunks 1.. (fewer than R / chunk in all),
// and an upper bound on the chunk count (E + that)
int64_t dw_max_chunked(const moe_dims& d) {
  return std::min<int64_t>(d.E, (int64_t)d.T * d.K / (kDwChunkRows + 1));
}
int64_t dw_part_slots(const moe_dims& d) {
  return ((int64_t)d.T * d.K + kDwChunkRows - 1) / kDwChunkRows;
}
int64_t dw_chunks_bound(const moe_dims& d) { return d.E + dw_part_slots(d); }

// Launch table of the gate/up, recompute and down GEMMs: the lead prefetch
// policy when the experts average at least kLeadMinRows routed rows (measured:
// -1% per step at 512 rows per expert; +1.4% at 64)
int gemm_lead(const moe_dims& d) { return (int64_t)d.T * d.K >= (int64_t)kLeadMinRows * d.E; }

// router-weight-gradient partials per routed row: one per (gate/up column
// tile, wave column) of the recompute GEMM
int partials_per_row(const moe_dims& d) { return kGemmWN * (int)gateup_tiles(d.I); }

size_t route_ws(const moe_dims& d, int32_t** hist, void* base) {
  Carve c{(char*)base};
  const int R = d.T * d.K;
  const int chunk = route_chunk(R);
  const size_t nblk = (size_t)((R + chunk - 1) / chunk);
  *hist = c.take<int32_t>(std::max<size_t>(1, nblk * d.E));
  return c.used;
}

// m-tiles of the row-grouped GEMMs: at most this many over all experts
int64_t mt_bound(const moe_dims& d) {
  return ((int64_t)d.T * d.K + (int64_t)d.E * (kGemmBM - 1)) / kGemmBM;
}
int chain_grid(const moe_dims& d, int n_tiles) {
  return kNumXcd * chain_slots(mt_bound(d), n_tiles);
}
// the larger of the two chained launches' grids
int chain_grid_max(const moe_dims& d) {
  const int ntd = (d.D + kGemmBN - 1) / kGemmBN, nti = (d.I + kGemmBN - 1) / kGemmBN;
  return chain_grid(d, (int)gateup_tiles(d.I) + std::max(ntd, nti));
}
// the layout of FwdWs::chain / BwdWs::chain: status, XCD ranges, per-m-tile
// counters, (XCD, slot) claims
constexpr int kChainXcd = 1, kChainCnt = 2 + kNumXcd;
size_t chain_claim_off(const moe_dims& d) { return kChainCnt + (size_t)mt_bound(d); }
size_t chain_ints(const moe_dims& d) { return chain_claim_off(d) + (size_t)chain_grid_max(d); }
// gate/up + down and dA + recompute as chained launches (else four launches)
bool use_chain(const moe_dims& d) {
  return mt_bound(d) >= (int64_t)kNumXcd * kChainMinMtPerXcd &&
         mt_bound(d) <= (int64_t)kNumXcd * kChainMaxMtPerXcd;
}

size_t fwd_ws(const moe_dims& d, FwdWs* w, void* base) {
  Carve c{(char*)base};
  const size_t R = (size_t)d.T * d.K;
  w->chain = c.take<int32_t>(chain_ints(d));
  w->tstart = c.take<int32_t>(2 * (size_t)d.E + 2);
  w->h = c.take<f16_t>(R * d.I);
  w->o = c.take<bf16_t>(R * d.D);
  return c.used;
}

size_t bwd_ws(const moe_dims& d, BwdWs* w, void* base) {
  Carve c{(char*)base};
  const size_t R = (size_t)d.T * d.K;
  w->chain = c.take<int32_t>(chain_ints(d));
  w->tstart = c.take<int32_t>(2 * (size_t)d.E + 2);
  w->rowoff = c.take<uint32_t>(std::max<size_t>(1, R));
  w->cstart = c.take<int32_t>(d.E + 1);
  w->pstart = c.take<int32_t>(d.E);
  w->slist = c.take<int32_t>(d.E + 1);
  w->corder = c.take<int32_t>(dw_chunks_bound(d));
  w->dw_split = c.take<int32_t>(d.E);
  w->amax_part = c.take<uint32_t>(kAmaxBlocks);
  w->gscale = c.take<float>(2);
  w->x16 = c.take<f16_t>((size_t)d.T * d.D);
  w->dy16 = c.take<f16_t>((size_t)d.T * d.D);
  w->dw_part = c.take<float>(std::max<size_t>(1, (size_t)dw_part_slots(d) * 2 * d.I * d.D));
  w->dw_part_down = c.take<float>(std::max<size_t>(1, (size_t)dw_part_slots(d) * d.I * d.D));
  w->da = c.take<float>(R * d.I);
  w->dgu = c.take<f16_t>(R * 2 * d.I);
  w->hw = c.take<f16_t>(R * d.I);
  w->dgu_lo = c.take<f16_t>(R * 2 * d.I);
  w->hw_lo = c.take<f16_t>(R * d.I);
  w->dxs = c.take<f16_t>(R * d.D);
  w->part = c.take<float>(R * partials_per_row(d));
  return c.used;
}

struct RouterBwdWs {
  float *w_rt, *dl, *part;
};

size_t router_bwd_ws(const moe_dims& d, RouterBwdWs* w, void* base) {
  Carve c{(char*)base};
  int splits, tc;
  router_dwr_split(d.T, &splits, &tc);
  w->w_rt = c.take<float>((size_t)d.E * d.D);
  w->dl = c.take<float>(std::max<size_t>(1, (size_t)d.T * d.K));
  w->part = c.take<float>((size_t)splits * d.D * d.E);
  return c.used;
}

int rowgrouped_grid(const moe_dims& d, int n_tiles, bool even_split = false) {
  return kNumXcd * rowgrouped_slots(mt_bound(d), n_tiles, even_split);
}

// dW grid: (row chunk, matrix) groups of m-tiles x n-tiles, one group per XCD
// in every row of kNumXcd groups (snake order); enough workgroups per XCD for
// its share of the chunk bound
int dw_grid(int nmat, int64_t chunks, int M, int N) {
  const int64_t per_c = (int64_t)((M + kGemmBM - 1) / kGemmBM) * ((N + kGemmBN - 1) / kGemmBN);
  const int64_t groups = (int64_t)nmat * chunks;
  return (int)((groups + kNumXcd - 1) / kNumXcd * per_c * kNumXcd);
}

thread_local char last_error[256] = "";

moe_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return MOE_OK;
  snprintf(last_error, sizeof(last_error), "%s: %s (%d)", where, hipGetErrorString(e), (int)e);
  return MOE_ERR_HIP;
}

// Entry points start from a clean error state: an error left by an earlier,
// unrelated HIP call on this thread must not be reported as ours.
void clear_stale_error() {
  (void)hipGetLastError();
  last_error[0] = 0;
}

#define MOE_TRY(expr)                                            \
  do {                                                           \
    hipError_t err_ = (expr);                                    \
    if (err_ != hipSuccess) return hip_status(err_, #expr);      \
  } while (0)

}  // namespace
}  // namespace moe

using namespace moe;

MOE_EXPORT size_t moe_workspace_bytes(const moe_dims* dims, int32_t phase) {
  if (check_dims(dims) != MOE_OK) return 0;
  switch (phase) {
    case MOE_PHASE_ROUTE: {
      int32_t* h;
      return route_ws(*dims, &h, nullptr);
    }
    case MOE_PHASE_FWD: {
      FwdWs w;
      return fwd_ws(*dims, &w, nullptr);
    }
    case MOE_PHASE_BWD: {
      BwdWs w;
      return bwd_ws(*dims, &w, nullptr);
    }
    case MOE_PHASE_ROUTER_BWD: {
      RouterBwdWs w;
      return router_bwd_ws(*dims, &w, nullptr);
    }
    default:
      return 0;
  }
}

MOE_EXPORT moe_status moe_route_sort(const moe_dims* dims, const float* logits,
                                     int32_t* topk_idx, float* topk_w, int32_t* counts,
                                     int32_t* offsets, int32_t* sorted_to_flat,
                                     int32_t* flat_to_sorted, void* ws, size_t ws_bytes,
                                     void* stream) {
  moe_status s = check_dims(dims);
  if (s != MOE_OK) return s;
  const size_t R = (size_t)dims->T * dims->K;
  if (!ptr_ok(logits, (size_t)dims->T * dims->E, 4) || !ptr_ok(topk_idx, R, 4) ||
      !ptr_ok(topk_w, R, 4) || !ptr_ok(sorted_to_flat, R, 4) || !ptr_ok(flat_to_sorted, R, 4) ||
      !ptr_ok(counts, dims->E, 4) || !ptr_ok(offsets, dims->E + 1, 4) || !ptr_ok(ws, 1, 16))
    return MOE_ERR_BAD_ARG;
  int32_t* hist;
  if (ws_bytes < route_ws(*dims, &hist, ws)) return MOE_ERR_WORKSPACE;
  clear_stale_error();
  return hip_status(launch_route_sort(*dims, logits, topk_idx, topk_w, counts, offsets,
                                      sorted_to_flat, flat_to_sorted, hist, (hipStream_t)stream),
                    "route_sort");
}

// ---- allocation-free routing
//
// moe_route_sort_noalloc runs the same kernels as moe_route_sort, with the
// per-block expert histograms in `scratch` instead of a caller workspace.
// Each GPU the library runs on holds its own copy of the array until the
// process ends; host code reaches it only through the device address that
// hipGetSymbolAddress returns on that device (the array's name in host code
// is a stand-in, not a device address).  The histograms are fully written by
// the histogram kernel before the scatter kernel reads them, so nothing needs
// clearing between calls, but calls that overlap on one GPU share the array
// and race.
namespace moe {
namespace {

constexpr size_t kScratchBytes = size_t(1) << 20;  // >= E * 256 blocks * 4 for every E <= 1024
constexpr int kMaxDevices = 64;
static_assert((size_t)kMaxE * 256 * sizeof(int32_t) <= kScratchBytes,
              "the routing histograms of every accepted shape fit the scratch buffer");

static __device__ __align__(256) int32_t scratch[kScratchBytes / sizeof(int32_t)];

std::mutex scratch_mutex;
void* scratch_addr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device.
hipError_t scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    scratch_addr[dev] = p;
  }
  *out = scratch_addr[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace moe

MOE_EXPORT moe_status moe_route_sort_noalloc(const moe_dims* dims, const float* logits,
                                             int32_t* topk_idx, float* topk_w, int32_t* counts,
                                             int32_t* offsets, int32_t* sorted_to_flat,
                                             int32_t* flat_to_sorted, void* stream) {
  moe_status s = check_dims(dims);
  if (s != MOE_OK) return s;
  const size_t R = (size_t)dims->T * dims->K;
  if (!ptr_ok(logits, (size_t)dims->T * dims->E, 4) || !ptr_ok(topk_idx, R, 4) ||
      !ptr_ok(topk_w, R, 4) || !ptr_ok(sorted_to_flat, R, 4) || !ptr_ok(flat_to_sorted, R, 4) ||
      !ptr_ok(counts, dims->E, 4) || !ptr_ok(offsets, dims->E + 1, 4))
    return MOE_ERR_BAD_ARG;
  int32_t* hist;
  const size_t need = route_ws(*dims, &hist, nullptr);
  clear_stale_error();
  if (need > kScratchBytes) {
    snprintf(last_error, sizeof(last_error),
             "route_sort_noalloc: %zu bytes of histograms exceed the %zu-byte static scratch", need,
             kScratchBytes);
    return MOE_ERR_SCRATCH;
  }
  void* base = nullptr;
  MOE_TRY(scratch_ptr(&base));
  route_ws(*dims, &hist, base);
  return hip_status(launch_route_sort(*dims, logits, topk_idx, topk_w, counts, offsets,
                                      sorted_to_flat, flat_to_sorted, hist, (hipStream_t)stream),
                    "route_sort_noalloc");
}

MOE_EXPORT moe_status moe_fwd(const moe_dims* dims, const void* x, const void* w_gate,
                              const void* w_up, const void* w_down, const float* topk_w,
                              const int32_t* offsets, const int32_t* sorted_to_flat,
                              const int32_t* flat_to_sorted, void* y, void* ws, size_t ws_bytes,
                              void* stream) {
  moe_status s = check_dims(dims);
  if (s != MOE_OK) return s;
  const size_t R = (size_t)dims->T * dims->K, TD = (size_t)dims->T * dims->D;
  const size_t W = (size_t)dims->E * dims->I * dims->D;
  if (!ptr_ok(x, TD, 16) || !ptr_ok(y, TD, 16) || !ptr_ok(w_gate, W, 16) ||
      !ptr_ok(w_up, W, 16) || !ptr_ok(w_down, W, 16) || !ptr_ok(ws, 1, 16) ||
      !ptr_ok(topk_w, R, 4) || !ptr_ok(offsets, dims->E + 1, 4) ||
      !ptr_ok(sorted_to_flat, R, 4) || !ptr_ok(flat_to_sorted, R, 4))
    return MOE_ERR_BAD_ARG;
  FwdWs w;
  if (ws_bytes < fwd_ws(*dims, &w, ws)) return MOE_ERR_WORKSPACE;
  const moe_dims& d = *dims;
  if (d.T == 0) return MOE_OK;
  hipStream_t st = (hipStream_t)stream;
  clear_stale_error();

  const bool chain = use_chain(d);
  MOE_TRY(launch_tilemap(offsets, d.E, kGemmBM, w.tstart, w.chain, (int)chain_ints(d),
                         chain ? w.chain + kChainXcd : nullptr, st));

  GemmArgs g{};
  g.offsets = offsets;
  g.tstart = w.tstart;
  g.E = d.E;
  // gate/up + SwiGLU: H[R, I] = silu(Xs Wg^T) * (Xs Wu^T), the routed rows Xs
  // gathered from x inside the GEMM's operand loads
  g.A = (const bf16_t*)x;
  g.a_gather = sorted_to_flat;
  g.a_div = d.K;
  g.a_rows = d.T;
  g.lda = d.D;
  g.B0 = (const bf16_t*)w_gate;
  g.B1 = (const bf16_t*)w_up;
  g.ldb = d.D;
  g.N = d.I;
  g.K = d.D;
  g.n_tiles = (int)gateup_tiles(d.I);
  g.lead = gemm_lead(d);
  g.C0 = (bf16_t*)w.h;  // fp16 bits
  g.ldc = d.I;
  // down: O[R, D] = H Wd^T; chained, a down tile starts reading H once the
  // gate/up tiles of its m-tile have stored theirs
  GemmArgs g2 = g;
  g2.A = (const bf16_t*)w.h;  // fp16 bits
  g2.lda = d.I;
  g2.B0 = (const bf16_t*)w_down;
  g2.a_gather = nullptr;
  g2.B1 = nullptr;
  g2.ldb = d.I;
  g2.N = d.D;
  g2.K = d.I;
  g2.n_tiles = (d.D + kGemmBN - 1) / kGemmBN;
  g2.C0 = w.o;
  g2.ldc = d.D;
  if (chain) {
    g.xcd_mt = g2.xcd_mt = w.chain + kChainXcd;
    g.xcd_claim = w.chain + chain_claim_off(d);
    g.mt_signal = w.chain + kChainCnt;
    g2.mt_wait = w.chain + kChainCnt;
    g2.mt_need = g.n_tiles;
    g2.chain_err = w.chain;
    MOE_TRY(launch_gemm_chain(kGateUpH, g, kDown, g2, chain_grid(d, g.n_tiles + g2.n_tiles), st));
  } else {
    MOE_TRY(launch_gemm(kGateUpH, g, rowgrouped_grid(d, g.n_tiles), st));
    MOE_TRY(launch_gemm(kDown, g2, rowgrouped_grid(d, g2.n_tiles), st));
  }

  MOE_TRY(launch_combine(w.o, topk_w, flat_to_sorted, y, d.T, d.K, d.D, st));
  return MOE_OK;
}

MOE_EXPORT moe_status moe_bwd(const moe_dims* dims, const void* x, const void* w_gate,
                              const void* w_up, const void* w_down, const float* topk_w,
                              const int32_t* offsets, const int32_t* sorted_to_flat,
                              const int32_t* flat_to_sorted, const void* dy, void* dx,
                              float* dw_gate, float* dw_up, float* dw_down, float* d_topk_w,
                              int32_t accumulate_dw, void* ws, size_t ws_bytes, void* stream) {
  moe_status s = check_dims(dims);
  if (s != MOE_OK) return s;
  const size_t R = (size_t)dims->T * dims->K, TD = (size_t)dims->T * dims->D;
  const size_t W = (size_t)dims->E * dims->I * dims->D;
  if (!ptr_ok(x, TD, 16) || !ptr_ok(dy, TD, 16) || !ptr_ok(dx, TD, 16) ||
      !ptr_ok(w_gate, W, 16) || !ptr_ok(w_up, W, 16) || !ptr_ok(w_down, W, 16) ||
      !ptr_ok(dw_gate, W, 16) || !ptr_ok(dw_up, W, 16) || !ptr_ok(dw_down, W, 16) ||
      !ptr_ok(ws, 1, 16) || !ptr_ok(topk_w, R, 4) || !ptr_ok(offsets, dims->E + 1, 4) ||
      !ptr_ok(sorted_to_flat, R, 4) || !ptr_ok(flat_to_sorted, R, 4) || !ptr_ok(d_topk_w, R, 4))
    return MOE_ERR_BAD_ARG;
  if (accumulate_dw != 0 && accumulate_dw != 1) return MOE_ERR_BAD_ARG;
  BwdWs w;
  if (ws_bytes < bwd_ws(*dims, &w, ws)) return MOE_ERR_WORKSPACE;
  const moe_dims& d = *dims;
  hipStream_t st = (hipStream_t)stream;
  clear_stale_error();

  // max|dy|, then one set-up launch: which experts' dW operands are split
  // hi + lo (read by the recompute GEMM's epilogue and the dW GEMMs), the
  // gradient scale, the row-tile starts, the dW row-chunk map and the
  // token-row byte offsets of the routed rows (the dW GEMMs gather the rows of
  // the fp16 x and s dy through them inside their loads)
  MOE_TRY(launch_amax_bf16(dy, TD, w.amax_part, st));
  BwdSetupArgs sa{};
  sa.offsets = offsets;
  sa.s2f = sorted_to_flat;
  sa.topk_w = topk_w;
  sa.amax_part = w.amax_part;
  sa.split = w.dw_split;
  sa.gscale = w.gscale;
  sa.tstart = w.tstart;
  sa.cstart = w.cstart;
  sa.pstart = w.pstart;
  sa.slist = w.slist;
  sa.corder = w.corder;
  sa.rowoff = w.rowoff;
  const bool chain = use_chain(d);
  sa.zero = w.chain;
  sa.nzero = (int)chain_ints(d);
  sa.xcd_mt = chain ? w.chain + kChainXcd : nullptr;
  sa.dim_factor = std::max(1.0f, 3.0f * (float)d.D / (8.0f * (float)d.I));
  sa.E = d.E;
  sa.R = (int)R;
  sa.K = d.K;
  sa.row_bytes = (uint32_t)d.D * 2u;
  MOE_TRY(launch_bwd_setup(sa, st));
  MOE_TRY(launch_f16_operands(x, dy, w.gscale, w.x16, w.dy16, TD, st));
  GemmArgs g{};
  g.offsets = offsets;
  g.tstart = w.tstart;
  g.E = d.E;
  if (R > 0) {
    // dA = dOu Wd (fp32 [R, I]), dOu = the routed rows gathered from dy
    g.A = (const bf16_t*)dy;
    g.a_gather = sorted_to_flat;
    g.a_div = d.K;
    g.a_rows = d.T;
    g.lda = d.D;
    g.B0 = (const bf16_t*)w_down;
    g.ldb = d.I;
    g.N = d.I;
    g.K = d.D;
    g.n_tiles = (d.I + kGemmBN - 1) / kGemmBN;
    g.Cf = w.da;
    g.ldc = d.I;
    GemmArgs gda = g;
    // recompute G, U from the routed rows of x (gathered in the loads) and,
    // in the epilogue, the SwiGLU backward from dA: dG | dU, Hw (fp16 hi and,
    // for split experts, lo) and the router-weight partials.  Chained to dA:
    // a recompute tile's epilogue waits for the dA tiles of its m-tile.
    g = GemmArgs{};
    g.offsets = offsets;
    g.tstart = w.tstart;
    g.E = d.E;
    g.A = (const bf16_t*)x;
    g.a_gather = sorted_to_flat;
    g.a_div = d.K;
    g.a_rows = d.T;
    g.lda = d.D;
    g.B0 = (const bf16_t*)w_gate;
    g.B1 = (const bf16_t*)w_up;
    g.ldb = d.D;
    g.N = d.I;
    g.K = d.D;
    g.n_tiles = (int)gateup_tiles(d.I);
    g.lead = gemm_lead(d);
    g.C0 = w.dgu;
    g.C1 = w.dgu + d.I;
    g.C2 = w.hw;
    g.L0 = w.dgu_lo;
    g.L1 = w.dgu_lo + d.I;
    g.L2 = w.hw_lo;
    g.ldc = 2 * d.I;
    g.DA = w.da;
    g.topk_w = topk_w;
    g.s2f = sorted_to_flat;
    g.part = w.part;
    g.np = partials_per_row(d);
    g.dw_split = w.dw_split;
    g.gscale = w.gscale;
    if (chain) {
      gda.xcd_mt = g.xcd_mt = w.chain + kChainXcd;
      gda.xcd_claim = w.chain + chain_claim_off(d);
      gda.mt_signal = w.chain + kChainCnt;
      g.mt_wait = w.chain + kChainCnt;
      g.mt_need = gda.n_tiles;
      g.chain_err = w.chain;
      MOE_TRY(launch_gemm_chain(kDA, gda, kGateUpBwd, g, chain_grid(d, gda.n_tiles + g.n_tiles), st));
    } else {
      MOE_TRY(launch_gemm(kDA, gda, rowgrouped_grid(d, gda.n_tiles), st));
      MOE_TRY(launch_gemm(kGateUpBwd, g, rowgrouped_grid(d, g.n_tiles), st));
    }
  }
  // dXs = dG Wg + dU Wu   (reduction over 2I)
  GemmArgs gx{};
  gx.offsets = offsets;
  gx.tstart = w.tstart;
  gx.E = d.E;
  gx.A = w.dgu;
  gx.lda = 2 * d.I;
  gx.B0 = (const bf16_t*)w_gate;
  gx.B1 = (const bf16_t*)w_up;
  gx.ldb = d.D;
  gx.N = d.D;
  gx.K = 2 * d.I;
  gx.n_tiles = (d.D + kGemmBN - 1) / kGemmBN;
  gx.C0 = (bf16_t*)w.dxs;  // fp16 bits; rows in flat slot order (t*K + k)
  gx.ldc = d.D;
  gx.s2f = sorted_to_flat;
  gx.gscale = w.gscale;
  gx.even_split = 1;
  // dW_down[e] = dOu_e^T Hw_e   ([D, I], reduction over the expert's rows, in
  // row chunks of at most kDwChunkRows); dOu from the fp16 s dy, the result
  // times 1/s
  GemmArgs gd{};
  gd.offsets = offsets;
  gd.E = d.E;
  gd.cstart = w.cstart;
  gd.pstart = w.pstart;
  gd.corder = w.corder;
  gd.dw_part = w.dw_part_down;
  gd.dw_split = w.dw_split;
  gd.gscale = w.gscale;
  gd.A = (const bf16_t*)w.dy16;  // fp16 bits
  gd.a_rowoff = w.rowoff;
  gd.a_rows = d.T;
  gd.lda = d.D;
  gd.B0 = w.hw;
  gd.ldb = d.I;
  gd.M = d.D;
  gd.N = d.I;
  gd.nmat = 1;
  gd.B_lo = w.hw_lo;
  gd.Cf = dw_down;
  gd.accumulate = accumulate_dw;
  // dW_gate[e] = dG_e^T Xs_e, dW_up[e] = dU_e^T Xs_e   ([I, D]); Xs from the fp16 x
  GemmArgs gg = gd;
  gg.dw_part = w.dw_part;
  gg.A = w.dgu;
  gg.A2 = w.dgu + d.I;
  gg.a_rowoff = nullptr;
  gg.lda = 2 * d.I;
  gg.B0 = (const bf16_t*)w.x16;  // fp16 bits
  gg.b_rowoff = w.rowoff;
  gg.b_rows = d.T;
  gg.ldb = d.D;
  gg.M = d.I;
  gg.N = d.D;
  gg.nmat = 2;
  gg.A_lo = w.dgu_lo;
  gg.A2_lo = w.dgu_lo + d.I;
  gg.B_lo = nullptr;
  gg.Cf = dw_gate;
  gg.Cf2 = dw_up;
  // the three read only the recompute GEMM's outputs: one launch (no tail
  // between them); then the chunk partials
  MOE_TRY(launch_bwd_fused(gx, R > 0 ? rowgrouped_grid(d, gx.n_tiles, gx.even_split != 0) : 0, gd,
                           dw_grid(1, dw_chunks_bound(d), d.D, d.I), gg,
                           dw_grid(2, dw_chunks_bound(d), d.I, d.D), st));
  MOE_TRY(launch_dw_reduce(DwReduceArgs{w.dw_part_down, dw_down, nullptr, 1, d.D, d.I},
                           DwReduceArgs{w.dw_part, dw_gate, dw_up, 2, d.I, d.D}, w.slist,
                           w.pstart, w.cstart, d.E, (int)dw_max_chunked(d), st));

  if (R > 0) {
    MOE_TRY(launch_reduce_rows(w.dxs, w.gscale, dx, d.T, d.K, d.D, w.part, flat_to_sorted,
                               d_topk_w, partials_per_row(d), st));
  }
  return MOE_OK;
}

MOE_EXPORT moe_status moe_router_fwd(const moe_dims* dims, const void* x, const float* w_r,
                                     float* logits, void* stream) {
  moe_status s = check_dims(dims);
  if (s != MOE_OK) return s;
  const size_t TD = (size_t)dims->T * dims->D;
  if (!ptr_ok(x, TD, 16) || !ptr_ok(w_r, (size_t)dims->D * dims->E, 16) ||
      !ptr_ok(logits, (size_t)dims->T * dims->E, 4))
    return MOE_ERR_BAD_ARG;
  clear_stale_error();
  return hip_status(launch_router_logits(x, w_r, logits, dims->T, dims->D, dims->E,
                                         (hipStream_t)stream),
                    "router_fwd");
}

MOE_EXPORT moe_status moe_router_bwd(const moe_dims* dims, const void* x, const float* w_r,
                                     const int32_t* topk_idx, const float* topk_w,
                                     const float* d_topk_w, void* dx, float* dw_r,
                                     int32_t accumulate_dwr, void* ws, size_t ws_bytes,
                                     void* stream) {
  moe_status s = check_dims(dims);
  if (s != MOE_OK) return s;
  const size_t R = (size_t)dims->T * dims->K, TD = (size_t)dims->T * dims->D;
  const size_t DE = (size_t)dims->D * dims->E;
  if (!ptr_ok(x, TD, 16) || !ptr_ok(dx, TD, 16) || !ptr_ok(w_r, DE, 16) ||
      !ptr_ok(dw_r, DE, 16) || !ptr_ok(topk_idx, R, 4) || !ptr_ok(topk_w, R, 4) ||
      !ptr_ok(d_topk_w, R, 4) || !ptr_ok(ws, 1, 16))
    return MOE_ERR_BAD_ARG;
  if (accumulate_dwr != 0 && accumulate_dwr != 1) return MOE_ERR_BAD_ARG;
  RouterBwdWs w;
  if (ws_bytes < router_bwd_ws(*dims, &w, ws)) return MOE_ERR_WORKSPACE;
  const moe_dims& d = *dims;
  clear_stale_error();
  return hip_status(launch_router_bwd(x, w_r, topk_idx, topk_w, d_topk_w, dx, dw_r,
                                      accumulate_dwr, w.dl, w.w_rt, w.part, d.T, d.D, d.E, d.K,
                                      d.score, (hipStream_t)stream),
                    "router_bwd");
}

MOE_EXPORT const char* moe_status_string(moe_status status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_BAD_ARG: return "bad argument (null/misaligned pointer, invalid dims, K > E or T*K >= 2^31)";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape (D and I must be multiples of 64, E <= 1024, K <= 64)";
    case MOE_ERR_WORKSPACE: return "workspace smaller than moe_workspace_bytes()";
    case MOE_ERR_HIP: return "HIP launch or runtime error";
    case MOE_ERR_SCRATCH: return "shape needs more than the static scratch of the allocation-free entry point";
    default: return "unknown status";
  }
}

MOE_EXPORT int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

MOE_EXPORT const char* moe_last_error(void) { return last_error; }

MOE_EXPORT int32_t moe_prof_enable(int32_t on) { return prof::set_enabled(on); }

MOE_EXPORT int32_t moe_prof_num_kernels(void) { return kNumKernels; }

MOE_EXPORT moe_status moe_prof_only(int32_t kernel_id) {
  return prof::set_only(kernel_id) == 0 ? MOE_OK : MOE_ERR_BAD_ARG;
}

MOE_EXPORT const char* moe_prof_kernel_name(int32_t kernel_id) { return prof::name(kernel_id); }

MOE_EXPORT moe_status moe_prof_read(double* total_ms, int64_t* launches, int32_t n) {
  if (n < 0 || (n > 0 && (!total_ms || !launches))) return MOE_ERR_BAD_ARG;
  return prof::read(total_ms, launches, n) == 0 ? MOE_OK : MOE_ERR_HIP;
}

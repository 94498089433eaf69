// Optional per-kernel timing: when enabled, every kernel launch of the
// library is bracketed by two hipEvents recorded on the launch stream; the
// host later sums the elapsed times per kernel.  Off by default; when off the
// launch path reads one atomic flag and does nothing else.  A launch's two
// events are paired per host thread, so launches from several threads are
// timed correctly; launches on a stream that is being captured into a graph
// are not timed (no event records end up in the graph).
#include <atomic>
#include <mutex>
#include <vector>

#include "kernels.hpp"

namespace moe {
namespace prof {
namespace {

struct Rec {
  int kid;
  hipEvent_t start, stop;
};

std::mutex mu;  // guards recs, pool, only_kid
std::atomic<bool> enabled{false};
int only_kid = -1;  // >= 0: bracket only this kernel id
std::vector<Rec> recs;        // recorded since the last enable
std::vector<hipEvent_t> pool;  // reusable events
// the launch this host thread has begun and not yet ended
thread_local int open_kid = -1;
thread_local hipEvent_t open_start = nullptr;

bool capturing(hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  return hipStreamIsCapturing(st, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone;
}

const char* const kNames[kNumKernels] = {
    "route_topk",   "route_hist",    "route_scatter", "tilemap",
    "gemm_gateup_h", "gemm_gateup_gu", "gemm_down",    "gemm_da",
    "combine",      "reduce_rows",
    "router_logits", "router_prep",  "router_dx",
    "router_dwr",   "router_dwr_sum", "dw_reduce",   "bwd_setup",    "dy_amax",
    "f16_operands", "gemm_bwd_fused", "gemm_fwd_chain", "gemm_da_recompute"};

hipEvent_t take() {
  if (!pool.empty()) {
    hipEvent_t e = pool.back();
    pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void recycle() {
  for (const Rec& r : recs) {
    pool.push_back(r.start);
    pool.push_back(r.stop);
  }
  recs.clear();
}

}  // namespace

void begin(int kid, hipStream_t st) {
  open_kid = -1;
  if (!enabled.load(std::memory_order_acquire) || capturing(st)) return;
  std::lock_guard<std::mutex> g(mu);
  if (only_kid >= 0 && kid != only_kid) return;
  hipEvent_t e = take();
  if (!e) return;
  hipEventRecord(e, st);
  open_kid = kid;
  open_start = e;
}

void end(hipStream_t st) {
  if (open_kid < 0) return;
  std::lock_guard<std::mutex> g(mu);
  const int kid = open_kid;
  open_kid = -1;
  if (!enabled.load(std::memory_order_acquire)) {  // disabled in between: drop the pair
    pool.push_back(open_start);
    return;
  }
  hipEvent_t e = take();
  if (!e) {
    pool.push_back(open_start);
    return;
  }
  hipEventRecord(e, st);
  recs.push_back(Rec{kid, open_start, e});
}

const char* name(int kid) { return (kid >= 0 && kid < kNumKernels) ? kNames[kid] : nullptr; }

int set_enabled(int on) {
  std::lock_guard<std::mutex> g(mu);
  recycle();
  enabled.store(on != 0, std::memory_order_release);
  return 0;
}

int set_only(int kid) {
  if (kid < -1 || kid >= kNumKernels) return -1;
  std::lock_guard<std::mutex> g(mu);
  only_kid = kid;
  return 0;
}

int read(double* total_ms, int64_t* launches, int n) {
  std::lock_guard<std::mutex> g(mu);
  for (int i = 0; i < n; ++i) {
    total_ms[i] = 0.0;
    launches[i] = 0;
  }
  for (const Rec& r : recs) {
    if (hipEventSynchronize(r.stop) != hipSuccess) return -1;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return -1;
    if (r.kid < n) {
      total_ms[r.kid] += ms;
      launches[r.kid] += 1;
    }
  }
  return 0;
}

}  // namespace prof
}  // namespace moe

// Routing and sort-by-expert kernels (gfx950).
//
// Method: LigerCute README (liger-cute-kernels 0.8.3), "LigerMoE design /
// Forward pass": the routed tokens are sorted by expert before the expert
// loop; buffers are sized from the total routed capacity (overview section),
// so no per-expert capacity exists and no token is dropped.
//
// Routing rule (the page leaves it open; plainest reading): experts ranked by
// fp32 logit, larger first, equal logits toward the lower expert id; weights
// are the softmax over all experts restricted to the K selected and
// renormalised (= exp(l_k - l_0) / sum_j exp(l_j - l_0)), or the sigmoid of
// the selected logit.  Sorted order inside an expert = ascending flat slot
// f = t*K + k (a stable counting sort), so the permutation is unique.
#include "kernels.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// Top-K: a group of L lanes per token (L a power of two, K <= L; 64 / L tokens
// per wave).  Lane l of the group holds experts l, l+L, ... (NPL of them).
// K rounds of a group-wide arg-max under the (value desc, id asc) order; the
// winner's owner lane marks it taken; lane k of the group keeps round k's
// winner.
template <int NPL, int L>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int T, int E,
                                                   int K, int score, int32_t* __restrict__ idx,
                                                   float* __restrict__ w) {
  const int token = (blockIdx.x * 256 + threadIdx.x) / L;
  const int gl = threadIdx.x & (L - 1);  // lane within the token's group
  if (token >= T) return;  // uniform per group; shuffles stay inside a group
  const float* l = logits + (size_t)token * E;
  float v[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int e = gl + L * j;
    v[j] = e < E ? l[e] : 0.0f;
  }
  uint32_t taken = 0;
  int my_e = 0;
  float my_v = 0.0f, top_v = 0.0f;
  for (int k = 0; k < K; ++k) {
    float bv = 0.0f;
    int be = -1;  // -1: no candidate
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int e = gl + L * j;
      if (e < E && !((taken >> j) & 1u)) {
        if (be < 0 || v[j] > bv || (v[j] == bv && e < be)) {
          bv = v[j];
          be = e;
        }
      }
    }
#pragma unroll
    for (int off = L / 2; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oe = __shfl_xor(be, off);
      if (oe >= 0 && (be < 0 || ov > bv || (ov == bv && oe < be))) {
        bv = ov;
        be = oe;
      }
    }
    if ((be & (L - 1)) == gl) taken |= 1u << (be / L);
    if (gl == k) {
      my_e = be;
      my_v = bv;
    }
    if (k == 0) top_v = bv;
  }
  float wk;
  if (score == MOE_SCORE_SOFTMAX_TOPK) {
    const float ex = gl < K ? expf(my_v - top_v) : 0.0f;
    float s = ex;
#pragma unroll
    for (int off = L / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off);
    wk = ex / s;
  } else {
    wk = 1.0f / (1.0f + expf(-my_v));
  }
  if (gl < K) {
    idx[(size_t)token * K + gl] = my_e;
    w[(size_t)token * K + gl] = wk;
  }
}

// ---------------------------------------------------------------------------
// Per-block expert histogram of flat slots [b*chunk, (b+1)*chunk).
// hist layout [E][nblk] so that one exclusive scan in (e, b) order gives
// every block's first output row per expert.
__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ idx, int R, int E,
                                                   int chunk, int nblk, int32_t* __restrict__ hist) {
  extern __shared__ int cnt[];
  for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
  __syncthreads();
  const int f0 = blockIdx.x * chunk;
  const int f1 = min(R, f0 + chunk);
  for (int f = f0 + threadIdx.x; f < f1; f += blockDim.x) atomicAdd(&cnt[idx[f]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) hist[(size_t)e * nblk + blockIdx.x] = cnt[e];
}

// Stable scatter, one wave per block (block b owns flat slots of chunk b and
// walks them in order, 64 at a time).  The block first derives its own first
// output row per expert from the per-block histograms: base(e, b) = (rows of
// experts < e) + (rows of expert e in blocks < b); block 0 also writes counts
// and offsets.  Lanes holding the same expert are found with one ballot per
// expert-id bit; a lane's rank among them is the count of lower lanes in that
// group.  Running positions live in LDS (run[0..E)), expert totals in
// run[E..2E).
__global__ __launch_bounds__(64) void scatter_kernel(const int32_t* __restrict__ idx, int R, int E,
                                                     int chunk, int nblk,
                                                     const int32_t* __restrict__ hist,
                                                     int32_t* __restrict__ s2f,
                                                     int32_t* __restrict__ f2s,
                                                     int32_t* __restrict__ counts,
                                                     int32_t* __restrict__ offsets) {
  extern __shared__ int run[];
  int* const tot = run + E;
  const int b = blockIdx.x, lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) {
    const int32_t* h = hist + (size_t)e * nblk;
    int before = 0, all = 0;
    if ((nblk & 3) == 0) {  // 16-byte rows of 4 blocks (the table is 16-byte aligned)
      typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
      const i32x4* h4 = (const i32x4*)h;
#pragma unroll 16
      for (int j4 = 0; j4 < nblk / 4; ++j4) {
        const i32x4 c = h4[j4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          before += 4 * j4 + q < b ? c[q] : 0;
          all += c[q];
        }
      }
    } else {
#pragma unroll 8
      for (int j = 0; j < nblk; ++j) {
        const int c = h[j];
        before += j < b ? c : 0;
        all += c;
      }
    }
    run[e] = before;
    tot[e] = all;
  }
  __syncthreads();
  // exclusive scan of the expert totals (E <= 1024), 64 experts per round
  int carry = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    const int v = e < E ? tot[e] : 0;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    if (e < E) {
      const int ex = carry + incl - v;
      run[e] += ex;
      if (b == 0) {
        offsets[e] = ex;
        counts[e] = v;
      }
    }
    carry += __shfl(incl, 63);
  }
  if (b == 0 && lane == 0) offsets[E] = R;
  __syncthreads();
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  const int fbeg = b * chunk, fend = min(R, fbeg + chunk);
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int f0 = fbeg; f0 < fend; f0 += 64) {
    const int f = f0 + lane;
    const bool valid = f < fend;
    const int e = valid ? idx[f] : 0;
    uint64_t m = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool on = (e >> bit) & 1;
      const uint64_t bb = __ballot(on);
      m &= on ? bb : ~bb;
    }
    const int rank = __popcll(m & lt);
    int pos = 0;
    if (valid) pos = run[e] + rank;
    __syncthreads();  // every lane has read run[] before the group leaders advance it
    if (valid && rank == 0) run[e] = pos + __popcll(m);
    __syncthreads();
    if (valid) {
      s2f[pos] = f;
      f2s[f] = pos;
    }
  }
}

// ---------------------------------------------------------------------------
// Tile map for the row-grouped GEMMs: tstart[e] = sum_{e'<e} ceil(count/BM);
// zero[0 .. nzero) = 0 (the chained launch's status word and counters).
__global__ __launch_bounds__(1024) void tilemap_kernel(const int32_t* __restrict__ offsets, int E,
                                                       int bm, int32_t* __restrict__ tstart,
                                                       int32_t* __restrict__ zero, int nzero,
                                                       int32_t* __restrict__ xcd_mt) {
  for (int i = threadIdx.x; i < nzero; i += 1024) zero[i] = 0;
  tile_starts_block(offsets, E, bm, tstart);
  if (xcd_mt) {
    __syncthreads();
    chain_bounds_block(tstart, E, xcd_mt);
  }
}

// ---------------------------------------------------------------------------
int route_chunk(int R) {
  int per = (R + 255) / 256;
  per = (per + 63) / 64 * 64;
  return per < 1024 ? 1024 : per;
}

hipError_t launch_route_sort(const moe_dims& d, const float* logits, int32_t* idx, float* w,
                             int32_t* counts, int32_t* offsets, int32_t* s2f, int32_t* f2s,
                             int32_t* hist, hipStream_t st) {
  const int R = d.T * d.K;
  if (d.T > 0) {
    // lanes per token: the smallest of 8, 16, 32, 64 that holds the K winners
    // with at most 16 logits per lane (E <= 1024)
    int L = 8;
    while (L < 64 && (L < d.K || (d.E + L - 1) / L > 16)) L *= 2;
    const int npl = (d.E + L - 1) / L;
    const int blocks = (int)(((int64_t)d.T * L + 255) / 256);
#define MOE_TOPK(N, LL)                                                                        \
  MOE_LAUNCH(kKRouteTopk, (topk_kernel<N, LL>), dim3(blocks), dim3(256), 0, st, logits, d.T, \
             d.E, d.K, d.score, idx, w)
#define MOE_TOPK_L(LL)                  \
  do {                                  \
    if (npl <= 1) MOE_TOPK(1, LL);      \
    else if (npl <= 2) MOE_TOPK(2, LL); \
    else if (npl <= 4) MOE_TOPK(4, LL); \
    else if (npl <= 8) MOE_TOPK(8, LL); \
    else MOE_TOPK(16, LL);              \
  } while (0)
    switch (L) {
      case 8: MOE_TOPK_L(8); break;
      case 16: MOE_TOPK_L(16); break;
      case 32: MOE_TOPK_L(32); break;
      default: MOE_TOPK_L(64); break;
    }
#undef MOE_TOPK_L
#undef MOE_TOPK
  }
  const int chunk = route_chunk(R);
  const int nblk = (R + chunk - 1) / chunk;
  if (nblk > 0)
    MOE_LAUNCH(kKRouteHist, hist_kernel, dim3(nblk), dim3(256), d.E * sizeof(int), st, idx, R,
               d.E, chunk, nblk, hist);
  // with no routed rows one scatter block still writes counts = 0 and offsets = 0
  MOE_LAUNCH(kKRouteScatter, scatter_kernel, dim3(nblk > 0 ? nblk : 1), dim3(64),
             2 * d.E * sizeof(int), st, idx, R, d.E, chunk, nblk, hist, s2f, f2s, counts, offsets);
  return hipGetLastError();
}

hipError_t launch_tilemap(const int32_t* offsets, int E, int bm, int32_t* tstart, int32_t* zero,
                          int nzero, int32_t* xcd_mt, hipStream_t st) {
  if (bm != kGemmBM) return hipErrorInvalidValue;
  MOE_LAUNCH(kKTilemap, tilemap_kernel, dim3(1), dim3(1024), 0, st, offsets, E, bm, tstart, zero,
             nzero, xcd_mt);
  return hipGetLastError();
}

}  // namespace moe

// Memory-bound kernels around the expert GEMMs (gfx950): router-weighted combine, the reduction of routed gradients back onto
// tokens, and the backward's operand preparation (max|dy| for the gradient
// scale; fp16 copies of x and s dy for the weight-gradient GEMMs).  Each
// thread moves 16-byte chunks; rows are contiguous, so every wave reads and
// writes whole 16-byte-aligned row segments.
//
// Method: LigerCute README (liger-cute-kernels 0.8.3), "LigerMoE design":
//   - Forward pass: the page copies the sorted tokens into an expert-ordered
//     staging buffer before the expert loop (here the GEMMs gather the rows
//     inside their operand loads instead); a final local combine applies the
//     router weights once every expert result is there.
//   - Backward pass: routed expert-output gradients are formed first; a final
//     local step reduces the routed dX contributions back to the tokens.
#include "kernels.hpp"

namespace moe {

constexpr int kPermuteThreads = 256;

static inline int grid_for(size_t work) {
  size_t b = (work + kPermuteThreads - 1) / kPermuteThreads;
  const size_t cap = 256 * 64;  // enough resident waves to saturate HBM; the rest loop
  return (int)(b < 1 ? 1 : (b > cap ? cap : b));
}

// y[t, :] = sum_{k<K} w[t,k] * O[flat_to_sorted[t*K+k], :]   (fp32, k ascending)
// KT = K known at compile time (0: runtime K): all K row indices are read
// first and all K row loads are then in flight together.  O is read once
// (non-temporal loads).
template <int KT>
__global__ __launch_bounds__(kPermuteThreads) void combine_kernel(
    const u32x4* __restrict__ O, const float* __restrict__ w, const int32_t* __restrict__ f2s,
    u32x4* __restrict__ y, int T, int K_, int cpr) {
  const int K = KT > 0 ? KT : K_;
  const size_t total = (size_t)T * cpr;
  for (size_t c = (size_t)blockIdx.x * kPermuteThreads + threadIdx.x; c < total;
       c += (size_t)gridDim.x * kPermuteThreads) {
    const size_t t = c / cpr;
    const int j = (int)(c - t * cpr);
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    auto add = [&](float wk, u32x4 v) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += wk * bf16_lo(v[q]);
        acc[2 * q + 1] += wk * bf16_hi(v[q]);
      }
    };
    if constexpr (KT > 0) {
      int rows[KT];
      float wk[KT];
      u32x4 v[KT];
#pragma unroll
      for (int k = 0; k < KT; ++k) {
        rows[k] = f2s[t * KT + k];
        wk[k] = w[t * KT + k];
      }
#pragma unroll
      for (int k = 0; k < KT; ++k) v[k] = __builtin_nontemporal_load(O + (size_t)rows[k] * cpr + j);
#pragma unroll
      for (int k = 0; k < KT; ++k) add(wk[k], v[k]);
    } else {
      for (int k = 0; k < K; ++k)
        add(w[t * K + k], __builtin_nontemporal_load(O + (size_t)f2s[t * K + k] * cpr + j));
    }
    u32x4 out;
#pragma unroll
    for (int q = 0; q < 4; ++q) out[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
    y[c] = out;
  }
}

// dX[t, :] = (1/s) sum_{k<K} dXs[t*K + k, :]: fp16 rows of s dXs in flat slot
// order, fp32 sum, k ascending, then the power-of-two 1/s (exact) and one
// bf16 rounding.  The K rows of a token are contiguous, so the reads stream;
// they are read once (non-temporal loads).  Each thread produces 8 outputs
// from one 16-byte read per routed copy; with KT > 0 all K reads are in
// flight together.  cpr8 = D / 8.
//
// The first npart_blocks workgroups (dispatched first, so they overlap the
// streaming ones) instead reduce the router-weight gradient partials:
// d_topk_w[f] = sum_{j<np} part[flat_to_sorted[f] * np + j]   (j ascending).
template <int KT>
__global__ __launch_bounds__(kPermuteThreads) void reduce_rows_kernel(
    const u32x4* __restrict__ dXs, const float* __restrict__ gscale, u32x4* __restrict__ dx,
    int T, int K_, int cpr8, const float* __restrict__ part, const int32_t* __restrict__ f2s,
    float* __restrict__ dtw, int np, int npart_blocks) {
  const int K = KT > 0 ? KT : K_;
  if ((int)blockIdx.x < npart_blocks) {
    const int R = T * K;
    for (int f = blockIdx.x * kPermuteThreads + threadIdx.x; f < R;
         f += npart_blocks * kPermuteThreads) {
      const float* pp = part + (size_t)f2s[f] * np;
      float s = 0.0f;
      for (int j = 0; j < np; ++j) s += pp[j];
      dtw[f] = s;
    }
    return;
  }
  const float inv = gscale[1];
  const size_t total = (size_t)T * cpr8;
  const size_t nb = gridDim.x - npart_blocks;
  for (size_t c = (size_t)(blockIdx.x - npart_blocks) * kPermuteThreads + threadIdx.x; c < total;
       c += nb * kPermuteThreads) {
    const size_t t = c / cpr8;
    const int j = (int)(c - t * cpr8);
    const u32x4* rows = dXs + t * K * cpr8 + j;
    float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    auto add = [&](u32x4 v) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        a[2 * q] += f16_lo(v[q]);
        a[2 * q + 1] += f16_hi(v[q]);
      }
    };
    if constexpr (KT > 0) {
      u32x4 v[KT];
#pragma unroll
      for (int k = 0; k < KT; ++k) v[k] = __builtin_nontemporal_load(rows + (size_t)k * cpr8);
#pragma unroll
      for (int k = 0; k < KT; ++k) add(v[k]);
    } else {
      for (int k = 0; k < K; ++k) add(__builtin_nontemporal_load(rows + (size_t)k * cpr8));
    }
    u32x4 out;
#pragma unroll
    for (int q = 0; q < 4; ++q) out[q] = pack_bf16x2(a[2 * q] * inv, a[2 * q + 1] * inv);
    dx[c] = out;
  }
}

// part[b] = max over workgroup b's grid-stride share of |src| (bf16 values as
// their 15-bit magnitude patterns, which order like the values; NaN patterns
// sort above infinity).  Integer max: the result does not depend on order.
__global__ __launch_bounds__(kPermuteThreads) void amax_bf16_kernel(
    const u32x4* __restrict__ src, size_t n16, uint32_t* __restrict__ part) {
  __shared__ uint32_t wmax[kPermuteThreads / 64];
  uint32_t m = 0;
  for (size_t c = (size_t)blockIdx.x * kPermuteThreads + threadIdx.x; c < n16;
       c += (size_t)gridDim.x * kPermuteThreads) {
    const u32x4 v = __builtin_nontemporal_load(src + c);
#pragma unroll
    for (int q = 0; q < 4; ++q) m = max(m, max(v[q] & 0x7fffu, (v[q] >> 16) & 0x7fffu));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t b = 0;
    for (int w = 0; w < kPermuteThreads / 64; ++w) b = max(b, wmax[w]);
    part[blockIdx.x] = b;
  }
}

hipError_t launch_amax_bf16(const void* src, size_t n, uint32_t* part, hipStream_t st) {
  // always kAmaxBlocks workgroups, so that every maximum the reader expects is written
  MOE_LAUNCH(kKDyAmax, amax_bf16_kernel, dim3(kAmaxBlocks), dim3(kPermuteThreads), 0, st,
             (const u32x4*)src, n / 8, part);
  return hipGetLastError();
}

// x16 = fp16(x) (round to nearest: exact in fp16's normal range, infinite
// above it), dy16 = fp16(s dy) (toward zero; s |dy| < 2), 8 values per thread
// and tensor.
__global__ __launch_bounds__(kPermuteThreads) void f16_operands_kernel(
    const u32x4* __restrict__ x, const u32x4* __restrict__ dy, const float* __restrict__ gscale,
    u32x4* __restrict__ x16, u32x4* __restrict__ dy16, size_t n16) {
  const float sc = gscale[0];
  for (size_t c = (size_t)blockIdx.x * kPermuteThreads + threadIdx.x; c < n16;
       c += (size_t)gridDim.x * kPermuteThreads) {
    const u32x4 a = __builtin_nontemporal_load(x + c);
    const u32x4 b = __builtin_nontemporal_load(dy + c);
    u32x4 ao, bo;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ao[q] = pack_f16x2(bf16_lo(a[q]), bf16_hi(a[q]));  // nearest: |x| >= 65520 -> inf
      bo[q] = __builtin_bit_cast(uint32_t,
                                 __builtin_amdgcn_cvt_pkrtz(bf16_lo(b[q]) * sc, bf16_hi(b[q]) * sc));
    }
    x16[c] = ao;
    dy16[c] = bo;
  }
}

hipError_t launch_f16_operands(const void* x, const void* dy, const float* gscale, void* x16,
                               void* dy16, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  MOE_LAUNCH(kKF16Operands, f16_operands_kernel, dim3(grid_for(n / 8)), dim3(kPermuteThreads), 0,
             st, (const u32x4*)x, (const u32x4*)dy, gscale, (u32x4*)x16, (u32x4*)dy16, n / 8);
  return hipGetLastError();
}

hipError_t launch_combine(const void* O, const float* w, const int32_t* f2s, void* y, int T,
                          int K, int D, hipStream_t st) {
  const int cpr = D / 8;
  if (T == 0) return hipSuccess;
  const dim3 grid(grid_for((size_t)T * cpr)), block(kPermuteThreads);
#define MOE_COMBINE(KT)                                                                          \
  MOE_LAUNCH(kKCombine, combine_kernel<KT>, grid, block, 0, st, (const u32x4*)O, w, f2s, (u32x4*)y, \
             T, K, cpr)
  switch (K) {
    case 1: MOE_COMBINE(1); break;
    case 2: MOE_COMBINE(2); break;
    case 4: MOE_COMBINE(4); break;
    case 8: MOE_COMBINE(8); break;
    default: MOE_COMBINE(0); break;
  }
#undef MOE_COMBINE
  return hipGetLastError();
}

hipError_t launch_reduce_rows(const void* dXs, const float* gscale, void* dx, int T, int K, int D,
                              const float* part, const int32_t* f2s, float* d_topk_w, int np,
                              hipStream_t st) {
  const int cpr8 = D / 8;
  if (T == 0) return hipSuccess;
  const size_t R = (size_t)T * K;
  // one thread per routed row for the partial sums, at most 256 workgroups
  const int npart = (int)std::min<size_t>(256, (R + kPermuteThreads - 1) / kPermuteThreads);
  const dim3 grid(npart + grid_for((size_t)T * cpr8)), block(kPermuteThreads);
#define MOE_REDUCE(KT)                                                                     \
  MOE_LAUNCH(kKReduceRows, reduce_rows_kernel<KT>, grid, block, 0, st, (const u32x4*)dXs, \
             gscale, (u32x4*)dx, T, K, cpr8, part, f2s, d_topk_w, np, npart)
  switch (K) {
    case 1: MOE_REDUCE(1); break;
    case 2: MOE_REDUCE(2); break;
    case 4: MOE_REDUCE(4); break;
    case 8: MOE_REDUCE(8); break;
    default: MOE_REDUCE(0); break;
  }
#undef MOE_REDUCE
  return hipGetLastError();
}

}  // namespace moe

// Memory-bound kernels around the expert GEMMs (gfx950): gather into expert
// order, router-weighted combine, and the reduction of routed gradients back
// onto tokens.  Each thread moves 16-byte chunks; rows are contiguous, so
// every wave reads and writes whole 16-byte-aligned row segments.
//
// Method: LigerCute README (liger-cute-kernels 0.8.3), "LigerMoE design":
//   - Forward pass: the sorted tokens are copied into the expert-ordered
//     staging buffer before the expert loop; a final local combine applies the
//     router weights once every expert result is there.
//   - Backward pass: routed expert-output gradients are formed first; a final
//     local step reduces the routed dX contributions back to the tokens.
#include "kernels.hpp"

namespace moe {

constexpr int kPermuteThreads = 256;

static inline int grid_for(size_t work) {
  size_t b = (work + kPermuteThreads - 1) / kPermuteThreads;
  const size_t cap = 256 * 64;  // enough resident waves to saturate HBM; rest loop
  return (int)(b < 1 ? 1 : (b > cap ? cap : b));
}

// dst0[p, :] = src0[sorted_to_flat[p] / K, :]  (and the same for src1/dst1 if given)
__global__ __launch_bounds__(kPermuteThreads) void gather_rows_kernel(
    const u32x4* __restrict__ src0, const u32x4* __restrict__ src1, u32x4* __restrict__ dst0,
    u32x4* __restrict__ dst1, const int32_t* __restrict__ s2f, int R, int K, int cpr) {
  const size_t total = (size_t)R * cpr;
  for (size_t c = (size_t)blockIdx.x * kPermuteThreads + threadIdx.x; c < total;
       c += (size_t)gridDim.x * kPermuteThreads) {
    const size_t p = c / cpr;
    const int j = (int)(c - p * cpr);
    const size_t t = (size_t)(s2f[p] / K);
    dst0[c] = src0[t * cpr + j];
    if (src1) dst1[c] = src1[t * cpr + j];
  }
}

// y[t, :] = sum_{k<K} w[t,k] * O[flat_to_sorted[t*K+k], :]   (fp32, k ascending)
__global__ __launch_bounds__(kPermuteThreads) void combine_kernel(
    const u32x4* __restrict__ O, const float* __restrict__ w, const int32_t* __restrict__ f2s,
    u32x4* __restrict__ y, int T, int K, int cpr) {
  const size_t total = (size_t)T * cpr;
  for (size_t c = (size_t)blockIdx.x * kPermuteThreads + threadIdx.x; c < total;
       c += (size_t)gridDim.x * kPermuteThreads) {
    const size_t t = c / cpr;
    const int j = (int)(c - t * cpr);
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int k = 0; k < K; ++k) {
      const float wk = w[t * K + k];
      const u32x4 v = O[(size_t)f2s[t * K + k] * cpr + j];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += wk * bf16_lo(v[q]);
        acc[2 * q + 1] += wk * bf16_hi(v[q]);
      }
    }
    u32x4 out;
#pragma unroll
    for (int q = 0; q < 4; ++q) out[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
    y[c] = out;
  }
}

// dX[t, :] = sum_{k<K} dXs[flat_to_sorted[t*K+k], :]  (fp32 rows, fp32 sum, k ascending)
// Each thread produces 8 outputs (two 16-byte fp32 reads per routed copy).
__global__ __launch_bounds__(kPermuteThreads) void reduce_rows_kernel(
    const f32x4* __restrict__ dXs, const int32_t* __restrict__ f2s, u32x4* __restrict__ dx, int T,
    int K, int cpr) {
  const size_t total = (size_t)T * cpr;
  for (size_t c = (size_t)blockIdx.x * kPermuteThreads + threadIdx.x; c < total;
       c += (size_t)gridDim.x * kPermuteThreads) {
    const size_t t = c / cpr;
    const int j = (int)(c - t * cpr);
    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < K; ++k) {
      const f32x4* row = dXs + (size_t)f2s[t * K + k] * (2 * cpr) + 2 * j;
      a0 += row[0];
      a1 += row[1];
    }
    dx[c] = u32x4{pack_bf16x2(a0[0], a0[1]), pack_bf16x2(a0[2], a0[3]),
                  pack_bf16x2(a1[0], a1[1]), pack_bf16x2(a1[2], a1[3])};
  }
}

// d_topk_w[f] = sum_{j<np} part[flat_to_sorted[f] * np + j]   (fixed order)
__global__ __launch_bounds__(kPermuteThreads) void reduce_partials_kernel(
    const float* __restrict__ part, const int32_t* __restrict__ f2s, float* __restrict__ out,
    int R, int np) {
  for (int f = blockIdx.x * kPermuteThreads + threadIdx.x; f < R;
       f += gridDim.x * kPermuteThreads) {
    const float* p = part + (size_t)f2s[f] * np;
    float s = 0.0f;
    for (int j = 0; j < np; ++j) s += p[j];
    out[f] = s;
  }
}

hipError_t launch_gather(const void* src0, const void* src1, void* dst0, void* dst1,
                         const int32_t* s2f, int R, int K, int D, hipStream_t st) {
  const int cpr = D / 8;
  if (R == 0) return hipSuccess;
  MOE_LAUNCH(src1 ? kKGather2 : kKGather, gather_rows_kernel, dim3(grid_for((size_t)R * cpr)), dim3(kPermuteThreads),
                     0, st, (const u32x4*)src0, (const u32x4*)src1, (u32x4*)dst0, (u32x4*)dst1,
                     s2f, R, K, cpr);
  return hipGetLastError();
}

hipError_t launch_combine(const void* O, const float* w, const int32_t* f2s, void* y, int T,
                          int K, int D, hipStream_t st) {
  const int cpr = D / 8;
  if (T == 0) return hipSuccess;
  MOE_LAUNCH(kKCombine, combine_kernel, dim3(grid_for((size_t)T * cpr)), dim3(kPermuteThreads), 0,
                     st, (const u32x4*)O, w, f2s, (u32x4*)y, T, K, cpr);
  return hipGetLastError();
}

hipError_t launch_reduce_rows(const void* dXs, const int32_t* f2s, void* dx, int T, int K, int D,
                              hipStream_t st) {
  const int cpr = D / 8;
  if (T == 0) return hipSuccess;
  MOE_LAUNCH(kKReduceRows, reduce_rows_kernel, dim3(grid_for((size_t)T * cpr)), dim3(kPermuteThreads),
                     0, st, (const f32x4*)dXs, f2s, (u32x4*)dx, T, K, cpr);
  return hipGetLastError();
}

hipError_t launch_reduce_partials(const float* part, const int32_t* f2s, float* out, int R,
                                  int np, hipStream_t st) {
  if (R == 0) return hipSuccess;
  MOE_LAUNCH(kKReducePartials, reduce_partials_kernel, dim3(grid_for((size_t)R)), dim3(kPermuteThreads), 0,
                     st, part, f2s, out, R, np);
  return hipGetLastError();
}

}  // namespace moe

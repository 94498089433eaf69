// Router projection and router backward (gfx950): the input side of the
// routed layer.  The logits that the routing selects on are x W_r; with the
// top-K selection held fixed (it is piecewise constant in the logits), the
// layer's router-weight gradient dRW flows back through the weights into the
// logits (dl), the projection weights (dW_r = x^T dl) and the layer input
// (dX += dl W_r^T).
//
// Method: LigerCute README (liger-cute-kernels 0.8.3), "LigerMoE design":
// the router weights are applied to the expert outputs in the final combine
// (Forward pass); their gradient is the adjacent step on the input side.
// Router function readings: softmax over the selected K logits (softmax over
// E, top-K, renormalise), or the sigmoid of each selected logit.
//
// Kernels:
//   router_logits  dense x [T,D] (bf16) x W_r [D,E] (fp32) on the fp32 matrix
//                  cores (v_mfma_f32_16x16x4_f32), 64 x 64 tiles, LDS-staged;
//   router_prep    dl per routed slot, and W_r transposed to [E, D];
//   router_dx      dX[t] += sum_k dl[t,k] W_r[:, idx[t,k]]   (fp32, k ascending,
//                  one rounding of the sum into the bf16 dX);
//   router_dwr     dW_r = x^T dl over a fixed token range per workgroup, on the
//                  fp32 matrix cores; the sparse dl tile (K nonzeros per token)
//                  is expanded in LDS;
//   router_dwr_sum dW_r (=/+=) the sum of the token-range partials in range
//                  order (deterministic, no atomics).
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int kRTile = 64;  // tokens x experts per logits workgroup
constexpr int kRBK = 32;    // d per stage
constexpr int kAPitch = kRBK + 4;     // floats; conflict-free fragment reads
constexpr int kBPitch = kRTile + 16;  // floats

// logits[t, e] = sum_d x[t, d] w_r[d, e].  256 threads = 4 waves in 2 x 2,
// each wave 32 x 32 = 2 x 2 fragments of 16 x 16.  Fragment lanes (verified on
// gfx950): A lane l = A[l % 16][l / 16], B lane l = B[l / 16][l % 16], result
// register j of lane l = C[4 (l / 16) + j][l % 16].
__global__ __launch_bounds__(256) void router_logits_kernel(const bf16_t* __restrict__ x,
                                                            const float* __restrict__ w_r,
                                                            float* __restrict__ logits, int T,
                                                            int D, int E) {
  __shared__ float As[kRTile * kAPitch];
  __shared__ float Bs[kRBK * kBPitch];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int t0 = blockIdx.x * kRTile, e0 = blockIdx.y * kRTile;
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int d0 = 0; d0 < D; d0 += kRBK) {
    {  // A: 64 rows x 32 d bf16 -> fp32; thread = one row's 8-element chunk
      const int r = tid >> 2, c = (tid & 3) * 8;
      float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (t0 + r < T) {
        const u32x4 q = *(const u32x4*)(x + (size_t)(t0 + r) * D + d0 + c);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          v[2 * h] = bf16_lo(q[h]);
          v[2 * h + 1] = bf16_hi(q[h]);
        }
      }
#pragma unroll
      for (int h = 0; h < 8; ++h) As[r * kAPitch + c + h] = v[h];
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {  // B: 32 d-rows x 64 experts fp32, 4 per chunk
      const int ch = tid + 256 * s;
      const int k = ch >> 4, c = (ch & 15) * 4;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if ((E & 3) == 0 && e0 + c + 3 < E) {  // 16-byte aligned whole chunk
        v = *(const f32x4*)(w_r + (size_t)(d0 + k) * E + e0 + c);
      } else {
#pragma unroll
        for (int h = 0; h < 4; ++h)
          if (e0 + c + h < E) v[h] = w_r[(size_t)(d0 + k) * E + e0 + c + h];
      }
#pragma unroll
      for (int h = 0; h < 4; ++h) Bs[k * kBPitch + c + h] = v[h];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kRBK; kk += 4) {
      float a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = As[(wm * 32 + i * 16 + (lane & 15)) * kAPitch + kk + (lane >> 4)];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = Bs[(kk + (lane >> 4)) * kBPitch + wn * 32 + j * 16 + (lane & 15)];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = e0 + wn * 32 + j * 16 + (lane & 15);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = t0 + wm * 32 + i * 16 + 4 * (lane >> 4) + q;
        if (t < T && e < E) logits[(size_t)t * E + e] = acc[i][j][q];
      }
    }
}

// dl per routed slot f = t*K + k (selection fixed):
//   softmax-renormalised:  dl_k = w_k (drw_k - sum_j w_j drw_j)
//   sigmoid:               dl_k = drw_k w_k (1 - w_k)
__global__ __launch_bounds__(256) void router_dl_kernel(const float* __restrict__ topk_w,
                                                        const float* __restrict__ drw,
                                                        float* __restrict__ dl, int T, int K,
                                                        int score) {
  for (int t = blockIdx.x * 256 + threadIdx.x; t < T; t += gridDim.x * 256) {
    const float* w = topk_w + (size_t)t * K;
    const float* g = drw + (size_t)t * K;
    float* o = dl + (size_t)t * K;
    if (score == MOE_SCORE_SOFTMAX_TOPK) {
      float s = 0.0f;
      for (int k = 0; k < K; ++k) s += w[k] * g[k];
      for (int k = 0; k < K; ++k) o[k] = w[k] * (g[k] - s);
    } else {
      for (int k = 0; k < K; ++k) o[k] = g[k] * w[k] * (1.0f - w[k]);
    }
  }
}

// w_rt[e, d] = w_r[d, e]
__global__ __launch_bounds__(256) void router_transpose_kernel(const float* __restrict__ w_r,
                                                               float* __restrict__ w_rt, int D,
                                                               int E) {
  const size_t n = (size_t)D * E;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const size_t d = i / E, e = i - d * E;
    w_rt[e * D + d] = w_r[i];
  }
}

// dx[t, d..d+3] += sum_k dl[t,k] w_rt[idx[t,k], d..d+3]  (fp32 sum, k ascending,
// then one rounding with the existing bf16 value).  A workgroup per token.
__global__ __launch_bounds__(256) void router_dx_kernel(const float* __restrict__ w_rt,
                                                        const int32_t* __restrict__ idx,
                                                        const float* __restrict__ dl,
                                                        u32x2* __restrict__ dx, int T, int D,
                                                        int K) {
  const int t = blockIdx.x;
  if (t >= T) return;
  const int32_t* it = idx + (size_t)t * K;
  const float* gt = dl + (size_t)t * K;
  for (int c = threadIdx.x; c < D / 4; c += 256) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < K; ++k) s += gt[k] * *(const f32x4*)(w_rt + (size_t)it[k] * D + 4 * c);
    u32x2* p = dx + (size_t)t * (D / 4) + c;
    const u32x2 old = *p;
    *p = u32x2{pack_bf16x2(bf16_lo(old[0]) + s[0], bf16_hi(old[0]) + s[1]),
               pack_bf16x2(bf16_lo(old[1]) + s[2], bf16_hi(old[1]) + s[3])};
  }
}

// Partial dW_r over tokens [s*tc, min(T, (s+1)*tc)):
//   part[s, d, e] = sum_t x[t, d] dl_dense[t, e],  dl_dense[t, idx[t,k]] = dl[t*K+k].
// Workgroup (64 d) x (64 e) x token range; 4 waves in 2 x 2, each 32 x 32.
__global__ __launch_bounds__(256) void router_dwr_kernel(const bf16_t* __restrict__ x,
                                                         const int32_t* __restrict__ idx,
                                                         const float* __restrict__ dl,
                                                         float* __restrict__ part, int T, int D,
                                                         int E, int K, int tc) {
  __shared__ float As[kRBK * kBPitch];  // [t][d]
  __shared__ float Bs[kRBK * kBPitch];  // [t][e]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int d0 = blockIdx.x * kRTile, e0 = blockIdx.y * kRTile;
  const int ta = blockIdx.z * tc, tb = min(T, ta + tc);
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int t0 = ta; t0 < tb; t0 += kRBK) {
#pragma unroll
    for (int h = 0; h < 8; ++h) Bs[(tid >> 3) * kBPitch + (tid & 7) * 8 + h] = 0.0f;
    {  // A: 32 tokens x 64 d, bf16 -> fp32; thread = one token's 8-element chunk
      const int r = tid >> 3, c = (tid & 7) * 8;
      float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      if (t0 + r < tb) {
        const u32x4 q = *(const u32x4*)(x + (size_t)(t0 + r) * D + d0 + c);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          v[2 * h] = bf16_lo(q[h]);
          v[2 * h + 1] = bf16_hi(q[h]);
        }
      }
#pragma unroll
      for (int h = 0; h < 8; ++h) As[r * kBPitch + c + h] = v[h];
    }
    __syncthreads();
    // B: scatter the stage's routed slots that fall in this expert range
    for (int i = tid; i < kRBK * K; i += 256) {
      const int r = i / K, t = t0 + r;
      if (t < tb) {
        const int e = idx[(size_t)t * K + (i - r * K)] - e0;
        if (e >= 0 && e < kRTile) Bs[r * kBPitch + e] = dl[(size_t)t * K + (i - r * K)];
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kRBK; kk += 4) {
      float a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = As[(kk + (lane >> 4)) * kBPitch + wm * 32 + i * 16 + (lane & 15)];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        b[j] = Bs[(kk + (lane >> 4)) * kBPitch + wn * 32 + j * 16 + (lane & 15)];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }
  float* out = part + (size_t)blockIdx.z * D * E;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int e = e0 + wn * 32 + j * 16 + (lane & 15);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int d = d0 + wm * 32 + i * 16 + 4 * (lane >> 4) + q;
        if (e < E) out[(size_t)d * E + e] = acc[i][j][q];
      }
    }
}

// dw_r[i] = (accumulate ? dw_r[i] : 0) + sum_{s<S} part[s, i]   (s ascending)
__global__ __launch_bounds__(256) void router_dwr_sum_kernel(const float* __restrict__ part,
                                                             float* __restrict__ dw_r, size_t n,
                                                             int S, int accumulate) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    float a = 0.0f;
    for (int s = 0; s < S; ++s) a += part[(size_t)s * n + i];
    dw_r[i] = accumulate ? dw_r[i] + a : a;
  }
}

int blocks_for(size_t n, int cap) {
  const size_t b = (n + 255) / 256;
  return (int)(b < 1 ? 1 : (b < (size_t)cap ? b : (size_t)cap));
}

}  // namespace

hipError_t launch_router_logits(const void* x, const float* w_r, float* logits, int T, int D,
                                int E, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const dim3 grid((T + kRTile - 1) / kRTile, (E + kRTile - 1) / kRTile);
  MOE_LAUNCH(kKRouterLogits, router_logits_kernel, grid, dim3(256), 0, st, (const bf16_t*)x, w_r,
             logits, T, D, E);
  return hipGetLastError();
}

void router_dwr_split(int T, int* splits, int* tokens_per_split) {
  // at least 512 tokens per workgroup, at most 64 token ranges
  int tc = (T + 63) / 64;
  tc = (tc + kRBK - 1) / kRBK * kRBK;
  if (tc < 512) tc = 512;
  *tokens_per_split = tc;
  *splits = T > 0 ? (T + tc - 1) / tc : 1;
}

hipError_t launch_router_bwd(const void* x, const float* w_r, const int32_t* topk_idx,
                             const float* topk_w, const float* d_topk_w, void* dx, float* dw_r,
                             int accumulate, float* dl, float* w_rt, float* part, int T, int D,
                             int E, int K, int score, hipStream_t st) {
  MOE_LAUNCH(kKRouterPrep, router_transpose_kernel, dim3(blocks_for((size_t)D * E, 4096)),
             dim3(256), 0, st, w_r, w_rt, D, E);
  if (T > 0) {
    MOE_LAUNCH(kKRouterPrep, router_dl_kernel, dim3(blocks_for((size_t)T, 1024)), dim3(256), 0,
               st, topk_w, d_topk_w, dl, T, K, score);
    MOE_LAUNCH(kKRouterDx, router_dx_kernel, dim3(T), dim3(256), 0, st, w_rt, topk_idx, dl,
               (u32x2*)dx, T, D, K);
  }
  int S, tc;
  router_dwr_split(T, &S, &tc);
  const dim3 grid(D / kRTile, (E + kRTile - 1) / kRTile, S);
  MOE_LAUNCH(kKRouterDwr, router_dwr_kernel, grid, dim3(256), 0, st, (const bf16_t*)x, topk_idx,
             dl, part, T, D, E, K, tc);
  MOE_LAUNCH(kKRouterDwrSum, router_dwr_sum_kernel, dim3(blocks_for((size_t)D * E, 2048)),
             dim3(256), 0, st, part, dw_r, (size_t)D * E, S, accumulate);
  return hipGetLastError();
}

}  // namespace moe

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
//   router_logits  dense x [T,D] (bf16) x W_r [D,E] (fp32) on the bf16 matrix
//                  cores: W_r is split into three bf16 terms (exact), so the
//                  three MFMA passes accumulate exact fp32 products in fp32;
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
constexpr int kBPitch = kRTile + 16;  // floats

// logits[t, e] = sum_d x[t, d] w_r[d, e] on the bf16 matrix cores.
// Each fp32 weight is split into three bf16 terms, w = w0 + w1 + w2 with
// w0 = bf16(w), w1 = bf16(w - w0), w2 = w - w0 - w1 (round to nearest even;
// every difference is exact and w2 has at most 8 significant bits, so the
// split is exact for normal values).  x is bf16, so each product x * wi is
// exact in fp32, and the three MFMA passes accumulate the exact products of x
// and w in fp32: the precision of an fp32 product, at the bf16 rate.
// Workgroup: 64 tokens x 64 experts, 4 waves of 16 tokens x 64 experts (4
// fragments of v_mfma_f32_16x16x32_bf16 per split).  Stages of 64 d: the
// waves load the stage's W_r block (fp32, 64 d x 64 experts, coalesced along
// the experts), split it and store it in LDS as k-contiguous bf16 rows per
// expert (double-buffered); x fragments come straight from global memory.
constexpr int kLT = 64, kLE = 64, kLK = 64;
constexpr int kLPitch = kLK * 2 + 16;              // bytes per staged expert row
constexpr int kLSplit = kLE * kLPitch;             // one split's block
constexpr int kLStage = 3 * kLSplit;               // one stage (27648 bytes)
constexpr int kLDPW = kLK / 4;                     // d per wave when staging (16)

__global__ __launch_bounds__(256) void router_logits_kernel(const bf16_t* __restrict__ x,
                                                            const float* __restrict__ w_r,
                                                            float* __restrict__ logits, int T,
                                                            int D, int E) {
  __shared__ __attribute__((aligned(16))) char Bs[2 * kLStage];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * kLT, e0 = blockIdx.y * kLE;
  // staging: this thread owns expert e0 + lane and d = d0 + 16 wave .. + 15
  const int se = e0 + lane;
  float wv[kLDPW];
  auto load_w = [&](int d0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < kLDPW; ++j) {
      const int d = d0 + wave * kLDPW + j;
      wv[j] = se < E && d < D ? w_r[(size_t)d * E + se] : 0.0f;
    }
  };
  auto store_w = [&](int buf) __attribute__((always_inline)) {
    char* row = Bs + buf * kLStage + lane * kLPitch + wave * kLDPW * 2;
#pragma unroll
    for (int c = 0; c < kLDPW / 8; ++c) {
      u32x4 h0, h1, h2;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t t0b[2], t1b[2], t2b[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float w = wv[c * 8 + 2 * q + h];
          t0b[h] = f32_to_bf16(w);
          const float r1 = w - bf16_to_f32(t0b[h]);
          t1b[h] = f32_to_bf16(r1);
          t2b[h] = f32_to_bf16(r1 - bf16_to_f32(t1b[h]));
        }
        h0[q] = t0b[0] | (t0b[1] << 16);
        h1[q] = t1b[0] | (t1b[1] << 16);
        h2[q] = t2b[0] | (t2b[1] << 16);
      }
      *(u32x4*)(row + c * 16) = h0;
      *(u32x4*)(row + kLSplit + c * 16) = h1;
      *(u32x4*)(row + 2 * kLSplit + c * 16) = h2;
    }
  };
  // x fragment of k-step kk: lane l holds token row t0 + 16 wave + l % 16 and
  // d = d0 + kk + 8 (l / 16) .. + 7
  const int xt = t0 + wave * 16 + (lane & 15);
  auto load_x = [&](int d) -> bf16x8 {
    u32x4 q = {0u, 0u, 0u, 0u};  // D is a multiple of 64: a 16-byte chunk is all in or all out
    if (xt < T && d < D) q = *(const u32x4*)(x + (size_t)xt * D + d + 8 * (lane >> 4));
    return __builtin_bit_cast(bf16x8, q);
  };
  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nst = (D + kLK - 1) / kLK;  // a last partial stage reads zeros past D
  load_w(0);
  store_w(0);
  bf16x8 xa[kLK / 32], xn[kLK / 32];
#pragma unroll
  for (int s = 0; s < kLK / 32; ++s) xa[s] = load_x(s * 32);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const bool more = st + 1 < nst;
    if (more) {
      load_w((st + 1) * kLK);
#pragma unroll
      for (int s = 0; s < kLK / 32; ++s) xn[s] = load_x((st + 1) * kLK + s * 32);
    }
    const char* b = Bs + (st & 1) * kLStage;
#pragma unroll
    for (int s = 0; s < kLK / 32; ++s) {
#pragma unroll
      for (int sp = 0; sp < 3; ++sp) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // B fragment: expert column 16 j + l % 16, k = 32 s + 8 (l / 16) .. + 7
          const bf16x8 bw = *(const bf16x8*)(b + sp * kLSplit + (j * 16 + (lane & 15)) * kLPitch +
                                             (s * 32 + 8 * (lane >> 4)) * 2);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bw, xa[s], acc[j], 0, 0, 0);
        }
      }
    }
    if (more) {
      store_w((st + 1) & 1);
#pragma unroll
      for (int s = 0; s < kLK / 32; ++s) xa[s] = xn[s];
    }
    __syncthreads();
  }
  // lane l holds token row 16 wave + l % 16 and experts 16 j + 4 (l / 16) .. + 3
  const int t = t0 + wave * 16 + (lane & 15);
  if (t < T) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + j * 16 + 4 * (lane >> 4);
      float* o = logits + (size_t)t * E + e;
      if ((E & 3) == 0 && e + 3 < E) {
        *(f32x4*)o = acc[j];
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (e + q < E) o[q] = acc[j][q];
      }
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
  const dim3 grid((T + kLT - 1) / kLT, (E + kLE - 1) / kLE);
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

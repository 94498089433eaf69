// Ragged grouped bf16 GEMMs on CDNA4 matrix cores (gfx950) for the expert MLP
// and its backward.
//
// Method: LigerCute README (liger-cute-kernels 0.8.3), "LigerMoE design":
// each expert runs its MLP on its (sorted) tokens on the tensor cores
// (Forward pass); the backward recomputes the activations, computes input and
// expert-weight gradients, and accumulates the weight gradients over all token
// tiles of the expert (Backward pass).  The page's Hopper/Blackwell design
// (TMA, warp-specialised WGMMA/UMMA, TMA reduce stores) is prior art only;
// here every GEMM is one CDNA4 kernel:
//
//   - a 256-thread workgroup owns a 128 x 128 output tile; 4 waves in 2 x 2,
//     each wave 64 x 64 = 4 x 4 fragments of v_mfma_f32_16x16x32_bf16 with
//     fp32 accumulators;
//   - 64-deep K stages staged through LDS, double-buffered, with the next
//     stage's global loads in flight while the matrix cores work on the
//     current one (one barrier per stage);
//   - LDS always holds operands k-contiguous ([row][k], rows padded to 144 B,
//     so the 16 lanes of a 16-byte fragment read hit 16 distinct 4-bank
//     groups).  Operands that are k-contiguous in HBM are copied as 16-byte
//     chunks; operands that are row-contiguous (the token-major activations of
//     the weight gradients, and the weights read transposed) are loaded as 4
//     k-rows x 8 elements per thread and transposed in registers before the
//     8-byte LDS writes;
//   - the MFMA is issued with the B fragment as its first operand, so each
//     lane ends with 4 consecutive output columns of one row, written as one
//     8-byte (bf16) or 16-byte (fp32) store;
//   - precision: every product accumulates in fp32.  The forward multiplies
//     bf16 (H is stored as bf16 for the down GEMM).  The recomputed G/U (used
//     by the SwiGLU backward and the router-weight gradient) and the per-row
//     dX partials (summed over the K routed copies) stay fp32.  The gradient
//     GEMMs (dXs, dW) multiply fp16: dG/dU/Hw are rounded to fp16 (3 more
//     mantissa bits than bf16, at the same matrix-core rate) and the bf16
//     operands are converted exactly on their way into LDS.  With bf16
//     gradient operands the cancellation in the sums over an expert's tokens
//     leaves errors of several times the 1e-2 + 1e-2 |ref| bar; fp16 keeps
//     them well inside it;
//   - ragged expert segments: the tile list is built on the device from the
//     expert offsets (no host read-back, graph-capturable); rows past an
//     expert's segment are zero-filled on load and skipped on store;
//   - weight gradients: one workgroup owns one output tile and walks all of
//     its expert's rows (no atomics, deterministic); an expert with no rows
//     writes zeros;
//   - XCD-aware tile order: workgroup b runs on XCD b % 8, so each XCD takes a
//     contiguous range of the (expert, column tile, row tile) list and the
//     tiles sharing one expert's weights share that XCD's L2.
#include <type_traits>

#include "kernels.hpp"

namespace moe {

constexpr int BM = kGemmBM, BN = kGemmBN, BK = kGemmBK, NTH = 256;
constexpr int LDSR = BK + 8;       // LDS row stride, bf16 elements
constexpr int TILE = 128 * LDSR;   // one operand tile (128 rows)

static_assert(BM == 128 && BN == 128 && BK == 64, "loaders assume 128 x 64 operand tiles");

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

// K-major operand tile: 128 rows x 64 k from rows whose k-run is contiguous.
// Chunk c = tid + 256 i covers row c / 8, k-chunk c % 8 (16 B each).
template <typename RowPtr>
__device__ __forceinline__ void load_kmajor(u32x4 (&r)[4], RowPtr row_ptr, int rows_valid,
                                            int k0) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = threadIdx.x + NTH * i;
    const int row = c >> 3, kc = c & 7;
    r[i] = row < rows_valid ? *(const u32x4*)(row_ptr(row) + k0 + kc * 8) : zero4();
  }
}
__device__ __forceinline__ void store_kmajor(bf16_t* lds, const u32x4 (&r)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = threadIdx.x + NTH * i;
    const int row = c >> 3, kc = c & 7;
    *(u32x4*)(lds + row * LDSR + kc * 8) = r[i];
  }
}

// bf16 -> fp16 in place (for operands of the fp16 gradient GEMMs).
__device__ __forceinline__ void to_f16(u32x4 (&r)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int d = 0; d < 4; ++d) r[i][d] = bf16x2_to_f16x2(r[i][d]);
}

// Row-contiguous operand tile: global element (k, mn) at base[k * ld + mn].
// Thread (kq = tid % 16, mc = tid / 16) loads k-rows 4kq..4kq+3 of the 8
// columns 8mc..8mc+7; valid iff k < k_valid and the column chunk < mn_valid.
__device__ __forceinline__ void load_mnmajor(u32x4 (&r)[4], const bf16_t* base, size_t ld,
                                             int k_valid, int mn_valid) {
  const int kq = threadIdx.x & 15, mc = threadIdx.x >> 4;
  const bool col_ok = mc * 8 < mn_valid;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int k = kq * 4 + q;
    r[q] = (col_ok && k < k_valid) ? *(const u32x4*)(base + (size_t)k * ld + mc * 8) : zero4();
  }
}
// Transpose the 4 (k) x 8 (mn) block in registers and write 8 rows of 4 k.
__device__ __forceinline__ void store_mnmajor(bf16_t* lds, const u32x4 (&r)[4]) {
  const int kq = threadIdx.x & 15, mc = threadIdx.x >> 4;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int d = j >> 1;
    u32x2 v;
    if (j & 1) {
      v[0] = (r[0][d] >> 16) | (r[1][d] & 0xFFFF0000u);
      v[1] = (r[2][d] >> 16) | (r[3][d] & 0xFFFF0000u);
    } else {
      v[0] = (r[0][d] & 0xFFFFu) | (r[1][d] << 16);
      v[1] = (r[2][d] & 0xFFFFu) | (r[3][d] << 16);
    }
    *(u32x2*)(lds + (mc * 8 + j) * LDSR + kq * 4) = v;
  }
}

// LDS row of the B fragment j of wave column wn.  Gate/up tiles hold 64 gate
// rows then the 64 matching up rows; each wave takes 2 gate + the 2 matching
// up fragments so that g and u of one output land in the same lane.
template <int MODE>
__device__ __forceinline__ int b_row(int wn, int j) {
  if constexpr (MODE == kGateUpH || MODE == kGateUpGU)
    return j < 2 ? wn * 32 + j * 16 : 64 + wn * 32 + (j - 2) * 16;
  else
    return wn * 64 + j * 16;
}

template <int MODE>
__global__ __launch_bounds__(NTH) void grouped_gemm_kernel(GemmArgs p) {
  __shared__ __attribute__((aligned(16))) bf16_t lds[2][2][TILE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  constexpr bool kRowGrouped = MODE != kDW;
  constexpr bool kGateUp = MODE == kGateUpH || MODE == kGateUpGU;
  // Gradient GEMMs (dXs, dW) multiply fp16 operands: dG/dU/Hw arrive in fp16,
  // bf16 operands (weights, x, dY) are converted while staging into LDS.
  constexpr bool kF16 = MODE == kDXs || MODE == kDW;
  using frag_t = typename std::conditional<kF16, f16x8, bf16x8>::type;

  // ---------------------------------------------------------------- tile decode
  int e, m0, n0, nk, rows_valid, mat = 0, k_count = 0;
  size_t kbase = 0;
  int nt_idx = 0;
  {
    int total;
    if constexpr (kRowGrouped) {
      total = p.tstart[p.E] * p.n_tiles;
    } else {
      total = p.nmat * p.E * ceil_div(p.M, BM) * ceil_div(p.N, BN);
    }
    const int per = ceil_div(total, kNumXcd);
    const int slot = blockIdx.x / kNumXcd;
    const int tile = (blockIdx.x % kNumXcd) * per + slot;
    if (slot >= per || tile >= total) return;
    if constexpr (kRowGrouped) {
      int lo = 0, hi = p.E;  // tstart[lo]*nt <= tile < tstart[hi]*nt
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.tstart[mid] * p.n_tiles <= tile) lo = mid;
        else hi = mid;
      }
      e = lo;
      const int local = tile - p.tstart[e] * p.n_tiles;
      const int mcnt = p.tstart[e + 1] - p.tstart[e];
      nt_idx = local / mcnt;
      const int mt = local - nt_idx * mcnt;
      m0 = p.offsets[e] + mt * BM;
      rows_valid = p.offsets[e + 1] - m0;
      n0 = nt_idx * (kGateUp ? BN / 2 : BN);
      nk = p.K / BK;
    } else {
      const int tm = ceil_div(p.M, BM), tn = ceil_div(p.N, BN);
      const int per_e = tm * tn;
      mat = tile / (p.E * per_e);
      const int rem = tile - mat * p.E * per_e;
      e = rem / per_e;
      const int r2 = rem - e * per_e;
      const int mt = r2 / tn;
      nt_idx = r2 - mt * tn;
      m0 = mt * BM;
      n0 = nt_idx * BN;
      kbase = (size_t)p.offsets[e];
      k_count = p.offsets[e + 1] - p.offsets[e];
      nk = ceil_div(k_count, BK);
      rows_valid = p.M - m0;
    }
  }

  // ---------------------------------------------------------------- operand sources
  const size_t lda = p.lda, ldb = p.ldb;
  const bf16_t* a_rows = nullptr;  // row-grouped: first A row of the tile
  const bf16_t* bw0 = nullptr;     // row-grouped: expert weights
  const bf16_t* bw1 = nullptr;
  const bf16_t* a_tok = nullptr;   // kDW: A at the expert's first row, column m0
  const bf16_t* b_tok = nullptr;   // kDW: B at the expert's first row, column n0
  if constexpr (kRowGrouped) {
    a_rows = p.A + (size_t)m0 * lda;
    if constexpr (kGateUp) {
      bw0 = p.B0 + ((size_t)e * p.N + n0) * ldb;  // Wg[e] rows n0.. ([I, D])
      bw1 = p.B1 + ((size_t)e * p.N + n0) * ldb;
    } else if constexpr (MODE == kDown) {
      bw0 = p.B0 + ((size_t)e * p.N + n0) * ldb;  // Wd[e] rows n0.. ([D, I])
    } else if constexpr (MODE == kDA) {
      bw0 = p.B0 + (size_t)e * p.K * ldb + n0;    // Wd[e] as (k = d) x (n = i), ld I
    } else {                                      // kDXs: (k = i) x (n = d), ld D
      bw0 = p.B0 + (size_t)e * (p.K / 2) * ldb + n0;
      bw1 = p.B1 + (size_t)e * (p.K / 2) * ldb + n0;
    }
  } else {
    a_tok = (mat == 0 ? p.A : p.A2) + kbase * lda + m0;
    b_tok = p.B0 + kbase * ldb + n0;
  }
  const int b_rows_valid = kRowGrouped ? (kGateUp ? BN : p.N - n0) : 0;

  u32x4 ra[4], rb[4];
  auto load_stage = [&](int kt) {
    const int k0 = kt * BK;
    if constexpr (kRowGrouped) {
      load_kmajor(ra, [&](int r) { return a_rows + (size_t)r * lda; }, rows_valid, k0);
      if constexpr (kGateUp) {
        load_kmajor(
            rb, [&](int r) { return r < 64 ? bw0 + (size_t)r * ldb : bw1 + (size_t)(r - 64) * ldb; },
            b_rows_valid, k0);
      } else if constexpr (MODE == kDown) {
        load_kmajor(rb, [&](int r) { return bw0 + (size_t)r * ldb; }, b_rows_valid, k0);
      } else if constexpr (MODE == kDA) {
        load_mnmajor(rb, bw0 + (size_t)k0 * ldb, ldb, BK, b_rows_valid);
      } else {
        const int half = p.K / 2;
        const bf16_t* src = k0 < half ? bw0 + (size_t)k0 * ldb : bw1 + (size_t)(k0 - half) * ldb;
        load_mnmajor(rb, src, ldb, BK, b_rows_valid);
      }
    } else {
      const int kv = k_count - k0;
      load_mnmajor(ra, a_tok + (size_t)k0 * lda, lda, kv, p.M - m0);
      load_mnmajor(rb, b_tok + (size_t)k0 * ldb, ldb, kv, p.N - n0);
    }
  };
  auto store_stage = [&](int buf) {
    if constexpr (kF16) {
      if (p.cvt_a) to_f16(ra);
      if (p.cvt_b) to_f16(rb);
    }
    if constexpr (kRowGrouped) {
      store_kmajor(lds[buf][0], ra);
      if constexpr (MODE == kDA || MODE == kDXs) store_mnmajor(lds[buf][1], rb);
      else store_kmajor(lds[buf][1], rb);
    } else {
      store_mnmajor(lds[buf][0], ra);
      store_mnmajor(lds[buf][1], rb);
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---------------------------------------------------------------- main loop
  if (nk > 0) {
    load_stage(0);
    store_stage(0);
    __syncthreads();
  }
  const int frow = lane & 15, fk = (lane >> 4) * 8;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_stage(kt + 1);
    const bf16_t* la = lds[cur][0];
    const bf16_t* lb = lds[cur][1];
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      frag_t af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *(const frag_t*)(la + (wm * 64 + i * 16 + frow) * LDSR + kk + fk);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = *(const frag_t*)(lb + (b_row<MODE>(wn, j) + frow) * LDSR + kk + fk);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (kF16)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bfr[j], af[i], acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
        }
    }
    if (kt + 1 < nk) store_stage(cur ^ 1);
    __syncthreads();
  }

  // ---------------------------------------------------------------- epilogue
  // Lane holds, for fragment (i, j), row wm*64 + i*16 + (lane % 16) and the 4
  // consecutive columns b_row(wn, j) + 4*(lane / 16) + q of the tile.
  const int cq = 4 * (lane >> 4);
  if constexpr (MODE == kGateUpH || MODE == kGateUpGU) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 64 + i * 16 + frow;
      if (r >= rows_valid) continue;
      const size_t m = (size_t)(m0 + r);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = n0 + wn * 32 + j * 16 + cq;
        const f32x4 g = acc[i][j], u = acc[i][j + 2];
        if constexpr (MODE == kGateUpH) {
          float h[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) h[q] = g[q] * sigmoidf_(g[q]) * u[q];
          *(u32x2*)(p.C0 + m * p.ldc + col) = u32x2{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
        } else {
          // recomputed gate/up pre-activations stay fp32 for the SwiGLU backward
          *(f32x4*)(p.Cf + m * p.ldc + col) = g;
          *(f32x4*)(p.Cf2 + m * p.ldc + col) = u;
        }
      }
    }
  } else if constexpr (MODE == kDown || MODE == kDXs) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 64 + i * 16 + frow;
      if (r >= rows_valid) continue;
      const size_t m = (size_t)(m0 + r);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + wn * 64 + j * 16 + cq;
        if (col >= p.N) continue;
        const f32x4 v = acc[i][j];
        if constexpr (MODE == kDXs)  // fp32 rows: the K copies of a token are summed later
          *(f32x4*)(p.Cf + m * p.ldc + col) = v;
        else
          *(u32x2*)(p.C0 + m * p.ldc + col) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
    }
  } else if constexpr (MODE == kDA) {
    // dA = dY_routed Wd (fp32).  With g, u recomputed (fp32) and w the router
    // weight of the row:  h = silu(g) u;  partial dRW = sum dA h over the
    // wave's 64 columns;  dH = w dA;  dG = dH u silu'(g);  dU = dH silu(g);
    // Hw = w h (the weighted activations that dW_down needs).
    const int I = p.N;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 64 + i * 16 + frow;
      const bool row_ok = r < rows_valid;
      const size_t m = (size_t)(m0 + (row_ok ? r : 0));
      const float wr = row_ok ? p.topk_w[p.s2f[m]] : 0.0f;
      float dot = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + wn * 64 + j * 16 + cq;
        if (!row_ok || col >= I) continue;
        const f32x4 gv = *(const f32x4*)(p.GU + m * (2 * (size_t)I) + col);
        const f32x4 uv = *(const f32x4*)(p.GU + m * (2 * (size_t)I) + I + col);
        float dg[4], du[4], hw[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float g = gv[q];
          const float u = uv[q];
          const float da = acc[i][j][q];
          const float sg = sigmoidf_(g);
          const float h = g * sg * u;
          dot += da * h;
          const float dh = wr * da;
          dg[q] = dh * u * sg * (1.0f + g * (1.0f - sg));
          du[q] = dh * g * sg;
          hw[q] = wr * h;
        }
        // fp16 (round to nearest): operands of the fp16 gradient GEMMs
        *(u32x2*)(p.C0 + m * p.ldc + col) = u32x2{pack_f16x2(dg[0], dg[1]), pack_f16x2(dg[2], dg[3])};
        *(u32x2*)(p.C1 + m * p.ldc + col) = u32x2{pack_f16x2(du[0], du[1]), pack_f16x2(du[2], du[3])};
        *(u32x2*)(p.C2 + m * (size_t)I + col) = u32x2{pack_f16x2(hw[0], hw[1]), pack_f16x2(hw[2], hw[3])};
      }
      dot += __shfl_xor(dot, 16);
      dot += __shfl_xor(dot, 32);
      if (row_ok && lane < 16) p.part[m * p.np + nt_idx * 2 + wn] = dot;
    }
  } else {  // kDW
    float* out = (mat == 0 ? p.Cf : p.Cf2) + (size_t)e * p.M * p.N;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 64 + i * 16 + frow;
      if (m0 + r >= p.M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = n0 + wn * 64 + j * 16 + cq;
        if (col >= p.N) continue;
        f32x4* dst = (f32x4*)(out + (size_t)(m0 + r) * p.N + col);
        f32x4 v = acc[i][j];
        if (p.accumulate) v += *dst;
        *dst = v;
      }
    }
  }
}

hipError_t launch_gemm(int mode, const GemmArgs& a, int grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  const bool dw_gateup = mode == kDW && a.nmat == 2;
  switch (mode) {
    case kGateUpH:
      MOE_LAUNCH(kKGemmGateUpH, grouped_gemm_kernel<kGateUpH>, dim3(grid), dim3(NTH), 0, st, a);
      break;
    case kGateUpGU:
      MOE_LAUNCH(kKGemmGateUpGU, grouped_gemm_kernel<kGateUpGU>, dim3(grid), dim3(NTH), 0, st, a);
      break;
    case kDown:
      MOE_LAUNCH(kKGemmDown, grouped_gemm_kernel<kDown>, dim3(grid), dim3(NTH), 0, st, a);
      break;
    case kDA:
      MOE_LAUNCH(kKGemmDA, grouped_gemm_kernel<kDA>, dim3(grid), dim3(NTH), 0, st, a);
      break;
    case kDXs:
      MOE_LAUNCH(kKGemmDXs, grouped_gemm_kernel<kDXs>, dim3(grid), dim3(NTH), 0, st, a);
      break;
    case kDW:
      MOE_LAUNCH(dw_gateup ? kKGemmDWGateUp : kKGemmDWDown, grouped_gemm_kernel<kDW>, dim3(grid),
                 dim3(NTH), 0, st, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe

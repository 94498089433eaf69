// Device helpers shared by the gfx950 kernels of the MoE library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // raw bfloat16 bits
typedef uint16_t f16_t;   // raw IEEE half bits
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, workgroups dealt round-robin

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }
// the two fp16 halves of a 32-bit word as floats
__device__ __forceinline__ float f16_lo(uint32_t pair) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(pair & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t pair) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(pair >> 16));
}

// float -> bf16 bits, round to nearest, ties to even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

// float -> fp16 bits (round to nearest even), two at a time.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}

// fp16 bits of (lo - hi_lo, hi - hi_hi), rounded to nearest, where hi holds the
// two fp16 roundings of (lo, hi): the low parts of a two-term fp16 split.
__device__ __forceinline__ uint32_t f16x2_residual(float lo, float hi, uint32_t hi_bits) {
  const float r0 = lo - (float)__builtin_bit_cast(_Float16, (uint16_t)(hi_bits & 0xFFFFu));
  const float r1 = hi - (float)__builtin_bit_cast(_Float16, (uint16_t)(hi_bits >> 16));
  return pack_f16x2(r0, r1);
}

// Two bf16 (one dword) -> two fp16 (one dword).  Exact for |v| in fp16's
// normal range [2^-14, 65504]; below it the conversion truncates (absolute
// error < 2^-24) and above it saturates to 65504.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t v) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(bf16_lo(v), bf16_hi(v)));
}

// sigma(z) = 1 / (1 + e^-z) with the hardware reciprocal (v_rcp_f32, about one
// ulp) instead of an IEEE division (a ten-instruction sequence): the SwiGLU
// epilogues evaluate it once per element, and its error stays far below the
// fp16 / bf16 roundings of the values it feeds.
__device__ __forceinline__ float sigmoidf_(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

template <typename T>
__device__ __forceinline__ T ceil_div(T a, T b) { return (a + b - 1) / b; }

// Block-wide exclusive scan of one int per thread (1024 threads), returns the
// exclusive prefix; *total receives the sum.  Deterministic (integers).
__device__ inline int block_exclusive_scan_1024(int v, int* total) {
  __shared__ int wsum[16];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int before = 0, all = 0;
  for (int i = 0; i < 16; ++i) {
    if (i < wv) before += wsum[i];
    all += wsum[i];
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

// Cost of an expert's last row tile in a row-grouped GEMM, in eighths of a
// full tile, as the tiles run (every other row tile costs 8): with more than
// 192 rows the full tile's schedule (8).  With fewer, the tile loads only the
// 64-row A pieces that hold rows; when the expert has other row tiles, which
// run beside it over the same weight slices (in L2), it costs the weights'
// half of each stage plus an eighth per piece (5, 6 or 7: experts of 513-541
// rows end in a tile of at most 29 rows that costs 5).  An expert's only row
// tile streams its weight slices from memory alone and costs a full tile
// whatever its rows (measured: weighing those tiles by their rows left the
// XCD holding the coldest experts of a Zipf routing 30% behind).
__device__ __forceinline__ int last_tile_cost8(int rows, int tiles) {
  return rows > 192 || tiles < 2 ? 8 : 4 + (rows + 63) / 64;
}

// The tile map of the row-grouped GEMMs, [2 (E + 1)] ints:
//   tstart[e] = exclusive prefix over the experts of ceil(rows_e / bm), the
//     first row tile of expert e in a GEMM's tile list (tstart[E] = the
//     number of row tiles);
//   tstart[E + 1 + e] = exclusive prefix of the experts' row-tile costs
//     (8 per row tile, last_tile_cost8 for each expert's last): the cost of
//     a column tile's pass over the experts before e.
// One workgroup of 1024 threads.
__device__ inline void tile_starts_block(const int32_t* __restrict__ offsets, int E, int bm,
                                         int32_t* __restrict__ tstart) {
  int carry = 0, ccarry = 0;
  int32_t* const cpre = tstart + E + 1;
  for (int e0 = 0; e0 < E; e0 += 1024) {
    const int e = e0 + threadIdx.x;
    const int rows = e < E ? offsets[e + 1] - offsets[e] : 0;
    const int c = (rows + bm - 1) / bm;
    const int cost = c > 0 ? 8 * (c - 1) + last_tile_cost8(rows - bm * (c - 1), c) : 0;
    int total, ctotal;
    const int ex = block_exclusive_scan_1024(c, &total);
    const int cex = block_exclusive_scan_1024(cost, &ctotal);
    if (e < E) {
      tstart[e] = carry + ex;
      cpre[e] = ccarry + cex;
    }
    carry += total;
    ccarry += ctotal;
  }
  if (threadIdx.x == 0) {
    tstart[E] = carry;
    cpre[E] = ccarry;
  }
}

}  // namespace moe

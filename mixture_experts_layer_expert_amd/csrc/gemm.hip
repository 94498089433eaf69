// Ragged grouped GEMMs on CDNA4 matrix cores (gfx950) for the expert MLP and
// its backward.
//
// Method: LigerCute README (liger-cute-kernels 0.8.3), "LigerMoE design":
// each expert runs its MLP on its (sorted) tokens on the tensor cores
// (Forward pass); the backward recomputes the activations, computes input and
// expert-weight gradients, and accumulates the weight gradients over all token
// tiles of the expert (Backward pass).  The page's Hopper/Blackwell design
// (TMA, warp-specialised WGMMA/UMMA, TMA reduce stores) is prior art only;
// here every GEMM is one CDNA4 kernel:
//
//   - a 512-thread workgroup (8 waves) owns a 256 x 256 output tile; waves in
//     2 (rows) x 4 (columns), each 128 x 64 = 8 x 4 fragments of
//     v_mfma_f32_16x16x32_{bf16,f16} with fp32 accumulators (a 256 x 256 fp32
//     tile is half of a CU's register file: the largest tile one workgroup
//     can hold; with 4 waves the compiler spills above 256 accumulators);
//   - operands go HBM -> LDS directly (buffer_load ... lds: no VGPR staging),
//     64-deep K stages, double-buffered (128 KB of LDS, one workgroup per CU),
//     one barrier per stage: the next stage's loads are issued right after the
//     barrier and land while the MFMAs consume the current one.  A buffer
//     resource per operand bounds the loads, so rows past a ragged edge read
//     as zeros in hardware;
//   - LDS keeps each operand in its HBM orientation, XOR-swizzled instead of
//     padded.  k-contiguous operands ([row][k], 128-byte rows of eight 16-byte
//     chunks; chunk c of row r stored at c ^ (r/2 % 8)) are read with
//     ds_read_b128;
//     row-contiguous operands ([k][row], the token-major activations of the
//     weight gradients and the weights read transposed; chunk c of k-row k
//     stored at c ^ s(k), s(k) = 2 (k % 4) + 8 ((k/8 + k/16) % 2)) are read
//     with the gfx950 transposing ds_read_b64_tr_b16, which hands each lane 4
//     consecutive k of one row.  Both read patterns are free of bank
//     conflicts (measured: SQ_LDS_BANK_CONFLICT = 0);
//   - the MFMA takes the B fragment as its first operand, so each lane ends
//     with 4 consecutive output columns of one row (8-byte bf16 or 16-byte
//     fp32 stores);
//   - precision: every product accumulates in fp32.  The gate/up GEMM
//     multiplies bf16; H is stored as fp16 (8 times finer than bf16: with bf16
//     H the forward output of a dense top-1 layer reached 1.04 of the error
//     bar where y cancels), so the down GEMM multiplies fp16, converting its
//     bf16 weight fragments after the LDS read.  The backward runs dA =
//     dOu Wd first and stores it fp32; the recompute GEMM then holds G and U
//     in its fp32 accumulators and does the SwiGLU backward and the
//     router-weight partials in its epilogue.  The per-row dX partials s dXs
//     (summed over the K routed copies by the dX reduction, which removes s)
//     are stored fp16: that rounding (2^-12 of the row) is small against the
//     fp16 roundings of dG and dU the row already carries.  The gradient
//     GEMMs (dXs, dW) multiply fp16: dG/dU/Hw are rounded to fp16 (3 more
//     mantissa bits than bf16, at the same matrix-core rate); dXs converts
//     its bf16 weight fragments after the LDS read, and the dW GEMMs read fp16
//     copies of x and s dy written once per backward (exact for |v| in fp16's
//     normal range).  s, a power of two with s max|dy| in [1, 2), keeps the
//     gradient operands (s dy, s dG, s dU) clear of fp16's subnormal range
//     and of its overflow whatever the loss scale; the dW epilogue and the dX
//     reduction multiply their fp32 results by 1/s, so at any scale the
//     results equal those of unit-scale gradients times the scale, bit for bit.  The dW GEMMs sum over
//     all of an expert's rows, where the rounding error grows like the
//     root-sum-square of the terms while the
//     result can cancel to ~0.  Each term carries one factor of its row's
//     router weight, so for an expert whose squared router weights sum to
//     more than kDwSplitW2 (weighted up for experts with few rows and for a
//     wide D against I) the rounded operand is split in fp16 hi + lo and
//     both parts are multiplied into the same accumulators, block by block
//     (error about 2^-22 sum |terms|); the others take one pass over hi
//     (error about 2^-12 times the root-sum-square of the terms);
//   - ragged expert segments: the tile list is built on the device from the
//     expert offsets (no host read-back, graph-capturable); an expert's last
//     row tile with a padding-only 64-row piece of A loads only the pieces
//     that hold rows and multiplies only its 16-row fragments that do;
//   - weight gradients: one workgroup owns one output tile of one row chunk
//     (at most kDwChunkRows of its expert's rows); chunk 0 writes the tile,
//     later chunks write partial tiles that dw_reduce_kernel adds in chunk
//     order (no atomics, deterministic); an expert with no rows writes zeros;
//   - XCD-aware tile order: workgroup b runs on XCD b % 8, so each XCD takes a
//     contiguous range of the (expert, column tile, row tile) list and the
//     tiles sharing one expert's operands share that XCD's L2; the dW GEMMs
//     deal their (row chunk, matrix) groups of tiles to the XCDs heaviest
//     chunk first, in snake order (XCDs 0..7, then 7..0, ...);
//   - L2 prefetch: each stage also touches the lines of a later stage (one
//     4-byte DMA per lane into a scratch LDS area), either every tile its own
//     lines one stage ahead, or, for gate/up and down when the launch asks
//     for the lead policy, only the first tile of each group sharing an
//     operand slice, two stages ahead.
#include <algorithm>
#include <type_traits>

#include "kernels.hpp"

namespace moe {

constexpr int BM = kGemmBM, BN = kGemmBN, BK = kGemmBK;
constexpr int WM = kGemmWM, WN = kGemmWN;
constexpr int NW = WM * WN, NTH = NW * kWave;
constexpr int WTM = BM / WM, WTN = BN / WN;  // rows / columns per wave
constexpr int FM = WTM / 16, FN = WTN / 16;  // A / B fragments per wave
constexpr int NS = kGemmNS;                  // K stages resident in LDS
constexpr int A_BYTES = BM * BK * 2;         // BM rows x BK k, or BK k x BM rows
constexpr int B_BYTES = BN * BK * 2;
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
constexpr int LOADS_PER_STAGE = (A_BYTES + B_BYTES) / 1024 / NW;  // 1 KB loads per wave

constexpr int KROW = BK * 2;       // bytes of one k-contiguous row in LDS (128)
constexpr int KCH = BK / 8;        // 16-byte chunks per k-contiguous row (8)
constexpr int KRPI = 1024 / KROW;  // k-contiguous rows per 1 KB load instruction (8)
// The loaders, swizzles, wait counts and the L2 prefetch (one 4-byte DMA per
// lane and wave touches 64 of a stage's 512 lines) are written for this
// geometry: 256 x 256 tiles, 64-deep stages, double-buffered, 8 waves as 2 x 4.
static_assert(BM == 256 && BN == 256 && BK == 64 && NS == 2 && WM == 2 && WN == 4,
              "the one tile geometry the kernels are written for");
constexpr int PREFETCH = kGemmPrefetch;  // L2 prefetch distance in stages
static_assert(PREFETCH >= 1, "the stage waits count the prefetch touch");
static_assert(NS * STAGE_BYTES + NW * 256 <= 160 * 1024, "LDS budget");

// Weight-gradient GEMMs with a gathered operand read its k-rows (routed rows)
// through their token index.  The indices of an expert's rows pass through a
// ring of RING_SLOTS chunks of RING_ROWS indices in LDS: chunk q is loaded
// (one 4-byte-per-lane DMA per wave) 2 + (prefetch distance) stages before
// its first use, into slot q % RING_SLOTS, which no stage in flight still reads.
constexpr int RING_ROWS = NW * 64, RING_SLOTS = 3;
constexpr int RING_BYTES = RING_SLOTS * RING_ROWS * 4;
constexpr int RING_STAGES = RING_ROWS / BK;  // row blocks per chunk
static_assert(NS * STAGE_BYTES + NW * 256 + RING_BYTES <= 160 * 1024,
              "LDS budget with the index ring");

// Chained launches: polls of a wait before it gives up (each poll is a
// device-coherent load and an s_sleep: well over a second in all), and the
// hardware register that names the XCD a wave runs on.
constexpr int kChainSpinLimit = 1 << 20;
constexpr int kHwRegXccId = (3 << 11) | 20;  // bits [3:0] of HW_REG_XCC_ID

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, size_t bytes) {
  const int n = bytes > 0x7FFFFFFFull ? 0x7FFFFFFF : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// One wave-wide direct-to-LDS load: lane i's 16 bytes at voffset land at
// lds_wave_base + 16 i (lds_wave_base must be wave-uniform).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char* lds_wave_base, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LDS_PTR(void, lds_wave_base), 16, voffset, 0, 0, 0);
}

// Swizzles (see the file comment).  swz_k: 16 consecutive rows reading the
// same k-chunk land in 16 distinct 16-byte bank groups.  swz_mn: the four
// 16-lane groups of a transposing read (k-rows 8g..8g+3) split into two pairs
// that each cover all 64 banks, for either pairing of the groups.
__device__ __forceinline__ int swz_k(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int swz_mn(int k) {
  return ((k & 3) << 1) | ((((k >> 3) ^ (k >> 4)) & 1) << 3);
}

// k-contiguous tile of ROWS rows x BK k (KROW-byte rows): this wave's
// instructions j = wave + NW i each fill rows KRPI j .. KRPI j + KRPI - 1.
// off(i, row) = byte offset of the row's k = 0 element (row is the lane's row
// of instruction i).
template <int ROWS>
constexpr int kmajor_instrs() { return ROWS / KRPI / NW; }

// Issues this wave's instructions i of the tile whose piece number qbase + i
// lies in [q0, q1) (pieces let the caller spread a stage's loads over the
// MFMA sequence; with constant bounds the tests fold away).
template <int ROWS, typename RowOff>
__device__ __forceinline__ void issue_kmajor(char* tile, int wave, int lane, uint32_t k0_bytes,
                                             RowOff off, __amdgpu_buffer_rsrc_t r, int qbase,
                                             int q0, int q1) {
  constexpr int N_INSTR = kmajor_instrs<ROWS>();  // 1 KB instructions (KRPI rows) per wave
  static_assert(N_INSTR * NW * KRPI == ROWS, "the waves' instructions must cover all rows");
#pragma unroll
  for (int i = 0; i < N_INSTR; ++i) {
    if (qbase + i < q0 || qbase + i >= q1) continue;
    const int j = wave + NW * i;
    const int row = KRPI * j + lane / KCH;
    const int c = (lane % KCH) ^ swz_k(row);
    dma16(r, tile + j * 1024, off(i, row) + k0_bytes + c * 16);
  }
}

// Row-contiguous tile of BK k-rows x C columns (C = 128 or 256): instruction j
// fills k-rows j*KPI .. j*KPI + KPI - 1 (KPI = 512 / C).  Element (k, col) of
// the tile comes from byte koff(i, k) + (col0 + col) * 2 of the operand (k is
// the lane's k-row of this wave's instruction i).
template <int C>
constexpr int mnmajor_instrs() { return BK / (512 / C) / NW; }

template <int C, typename KOff>
__device__ __forceinline__ void issue_mnmajor(char* tile, int wave, int lane, int col0, KOff koff,
                                              __amdgpu_buffer_rsrc_t r, int qbase, int q0, int q1) {
  constexpr int KPI = 512 / C, LPR = C / 8;  // k-rows per instruction, lanes per k-row
  constexpr int N_INSTR = mnmajor_instrs<C>();  // 1 KB instructions per wave
  static_assert(N_INSTR * NW * KPI == BK, "the waves' instructions must cover all BK k-rows");
#pragma unroll
  for (int i = 0; i < N_INSTR; ++i) {
    if (qbase + i < q0 || qbase + i >= q1) continue;
    const int j = wave + NW * i;
    const int k = j * KPI + lane / LPR;
    const int c = (lane % LPR) ^ swz_mn(k);
    dma16(r, tile + j * 1024, koff(i, k) + (uint32_t)(col0 + c * 8) * 2u);
  }
}

// Fragment of 16 rows x 32 k starting at k = kk (a multiple of 32): lane l
// gets row r0 + l % 16, k = kk + 8 (l / 16) .. + 7.
template <typename F>
__device__ __forceinline__ F read_kmajor(const char* tile, int r0, int kk, int lane) {
  const int row = r0 + (lane & 15);
  const int c = (kk >> 3) + (lane >> 4);
  return *(const F*)(tile + row * KROW + ((c ^ swz_k(row)) << 4));
}

// Fragment of 16 "rows" (columns of the [k][col] tile) x 32 k: lane l gets
// column c0 + l % 16 and k = kk + 8 (l / 16) .. + 7, via two transposing reads.
template <int C, typename F>
__device__ __forceinline__ F read_mnmajor(const char* tile, int c0, int kk, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int col = c0 + 4 * (j & 3);
  const int k_lo = kk + 8 * g + (j >> 2);
  const int k_hi = k_lo + 4;
  const char* p_lo = tile + k_lo * (2 * C) + ((((col >> 3) ^ swz_mn(k_lo))) << 4) + ((col >> 2) & 1) * 8;
  const char* p_hi = tile + k_hi * (2 * C) + ((((col >> 3) ^ swz_mn(k_hi))) << 4) + ((col >> 2) & 1) * 8;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p_lo));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p_hi));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(F, v);
}

// bf16 fragment bits -> fp16 fragment (operands of the fp16 gradient GEMMs).
__device__ __forceinline__ f16x8 frag_to_f16(f16x8 v) {
  u32x4 u = __builtin_bit_cast(u32x4, v);
#pragma unroll
  for (int d = 0; d < 4; ++d) u[d] = bf16x2_to_f16x2(u[d]);
  return __builtin_bit_cast(f16x8, u);
}

// Epilogue staging.  A lane's accumulators hold 4 consecutive columns of 16
// different rows per fragment, so storing them directly writes 8- or 16-byte
// pieces of 16 rows per instruction.  Instead each wave stages a strip of 16
// rows x C columns (ES-byte elements) in its own LDS area (the stage buffers
// are free once the main loop is done) and writes it back as whole row
// segments, 16 bytes per lane.  Rows are padded by 16 bytes (16-byte aligned,
// spread over the banks).
template <int C, int ES>
struct Strip {
  static constexpr int ELEM = ES;
  static constexpr int ROWB = C * ES;   // bytes of one staged row
  static constexpr int SP = ROWB + 16;  // row pitch
  static constexpr int BYTES = 16 * SP;
  static constexpr int CPR = ROWB / 16;  // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;   // rows per wave-wide copy instruction
  static_assert(ROWB % 16 == 0 && 64 % CPR == 0 && 16 % RPI == 0, "strip layout");
};

// The lane's 4 values of strip row `row` from strip column `col` on.
template <class S, class V>
__device__ __forceinline__ void strip_put(char* stg, int row, int col, V v) {
  static_assert(sizeof(V) == 4 * S::ELEM, "4 elements per lane");
  *(V*)(stg + row * S::SP + col * S::ELEM) = v;
}

// Copies the staged strip out: strip row r (< nrows) goes to the byte address
// row_ptr(r, h) of its column 0, h being the copy instruction (r = h * RPI +
// lane / CPR); chunks past ncols columns are skipped.  op(dst, v) stores (or
// accumulates) one 16-byte chunk.
template <class S, class RowPtr, class Op>
__device__ __forceinline__ void strip_out(const char* stg, int lane, int nrows, int ncols,
                                          RowPtr row_ptr, Op op) {
#pragma unroll
  for (int h = 0; h < 16 / S::RPI; ++h) {
    const int r = h * S::RPI + lane / S::CPR, ch = lane % S::CPR;
    const u32x4 v = *(const u32x4*)(stg + r * S::SP + ch * 16);
    if (r < nrows && ch * (16 / S::ELEM) < ncols) op(row_ptr(r, h) + ch * 16, v);
  }
}

// LDS of one workgroup tile: NS stages, then (with L2 prefetch) 256 bytes per
// wave that the prefetch DMA writes and nothing reads, then (kDW) the ring of
// gathered row indices.
constexpr int kRingOff = NS * STAGE_BYTES + NW * 256;
template <int MODE>
constexpr int tile_lds_bytes() { return kRingOff + (MODE == kDW ? RING_BYTES : 0); }

// One workgroup tile of a grouped GEMM: the workgroup runs on XCD `xcd` and is
// that XCD's `slot`-th workgroup of this GEMM (tile decode and order); lds
// holds at least tile_lds_bytes<MODE>() bytes, 1024-byte aligned.
// LEAD: the L2 prefetch policy of the gate/up and down GEMMs (see kLead); the
// host picks it per launch from the shape (GemmArgs::lead).
template <int MODE, bool LEAD = false>
__device__ __forceinline__ void gemm_tile(const GemmArgs& p, const int xcd, const int slot,
                                          char* const lds) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  constexpr bool kRowGrouped = MODE != kDW;
  constexpr bool kGateUp = MODE == kGateUpH || MODE == kGateUpBwd;
  constexpr bool kF16 = MODE == kDown || MODE == kDXs || MODE == kDW;
  constexpr bool kBmn = MODE == kDA || MODE == kDXs || MODE == kDW;  // B row-contiguous
  using frag_t = typename std::conditional<kF16, f16x8, bf16x8>::type;
  // L2 prefetch distance of this GEMM, and whether only the first tile of each
  // group sharing an operand slice touches it
  static_assert(!LEAD || kGateUp || MODE == kDown, "the lead policy is for gate/up and down");
  constexpr bool kLead = LEAD;
  constexpr int PF = kLead ? kGemmPrefetchLead : PREFETCH;
  // the index ring is loaded RA stages ahead of its first read (the touch of
  // stage kt + 1 + PF is read at stage kt)
  constexpr int RA = 2 + PF;
  static_assert(PF <= 1 || RING_STAGES >= PF, "index chunks must span the prefetch distance");

  // ---------------------------------------------------------------- tile decode
  // The number of experts i < E with f(starts[i]) <= key, less one, for a
  // nondecreasing f(starts[]): the expert whose range holds key.  All lanes
  // read 64 starts each round (one round of loads for E <= 256) instead of a
  // binary search's chain of dependent loads.
  auto expert_of = [&](const int32_t* starts, auto f, int key) {
    int cnt = 0;
    for (int c = 0; c < p.E; c += 256) {
      int v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = c + 64 * q + lane;
        v[q] = i < p.E ? starts[i] : 0;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        cnt += (int)__popcll(__ballot(c + 64 * q + lane < p.E && f(v[q]) <= key));
    }
    return cnt - 1;
  };
  int e, m0, n0, nk, rows_valid, mat = 0, k_count = 0, nk_pass = 0, nt_idx = 0;
  int dw_chunk = 0, dw_slot = -1;  // kDW: row chunk of the expert; partial slot (chunks 1..)
  int gmt = 0, mt_first = 0;  // row-grouped: global m-tile; first of the expert's m-tiles on this XCD
  size_t kbase = 0;
  {
    if constexpr (kRowGrouped) {
      // XCD x takes a contiguous range of the tile list (expert by expert,
      // column tile by column tile, m-tile by m-tile), so an expert's tiles
      // share one L2: with xcd_mt, every column tile of a range of m-tiles
      // (both GEMMs of a chained launch then put an m-tile on the same XCD),
      // else an equal share of the tiles.
      const int nt = p.n_tiles;
      int lo, hi, key;
      if (p.xcd_mt) {
        lo = p.xcd_mt[xcd];
        hi = p.xcd_mt[xcd + 1];
        if (slot >= (hi - lo) * nt) return;
        key = lo * nt + slot;
      } else {
        // every XCD about the same tile cost (last_tile_cost8), or with even_split
        // the same tile count (column tiles of one m-tile may then sit on two
        // XCDs): XCD x starts at the tile where the list's cumulative cost
        // reaches x / kNumXcd of the total
        lo = 0;
        hi = p.tstart[p.E];
        const int32_t* const cpre = p.tstart + p.E + 1;
        const int64_t ctot = cpre[p.E];
        auto first_tile = [&](int x) -> int {
          if (x == 0) return 0;
          if (x == kNumXcd) return hi * nt;
          // the cost target in passes over the expert list, its expert, and
          // the tile within the expert's (column tile, m-tile) order
          const int64_t t = (int64_t)x * ctot / kNumXcd;
          const int ex = expert_of(cpre, [](int v) { return v; }, (int)t);
          const int c0 = cpre[ex], ce = cpre[ex + 1] - c0;
          const int t0 = p.tstart[ex], mc = p.tstart[ex + 1] - t0;
          if (ce == 0) return t0 * nt;
          const int64_t rem = (t - c0) * nt;  // eighths of a tile into the expert
          const int q = (int)(rem / ce);      // whole column tiles
          const int r = min((int)((rem - (int64_t)q * ce + 4) / 8), mc - 1);
          return t0 * nt + q * mc + r;
        };
        if (p.even_split) {
          const int per = ceil_div(hi * nt, kNumXcd);
          key = xcd * per + slot;
          if (slot >= per || key >= hi * nt) return;
        } else {
          const int k0 = first_tile(xcd), k1 = first_tile(xcd + 1);
          key = k0 + slot;
          if (key >= k1) return;
        }
      }
      auto clip = [lo, hi](int v) { return min(max(v, lo), hi); };
      e = expert_of(p.tstart, [&](int v) { return clip(v) * nt; }, key);
      const int ts0 = p.tstart[e];
      const int cs = clip(ts0), mcnt = clip(p.tstart[e + 1]) - cs;
      const int local = key - cs * nt;
      nt_idx = local / mcnt;
      const int mloc = local - nt_idx * mcnt;
      gmt = cs + mloc;
      mt_first = mloc == 0;
      const int mt = gmt - ts0;
      m0 = p.offsets[e] + mt * BM;
      rows_valid = min(BM, p.offsets[e + 1] - m0);
      n0 = nt_idx * (kGateUp ? BN / 2 : BN);  // gate/up tiles: BN/2 gate + BN/2 up rows
      nk = p.K / BK;
    } else {
      // dW: the tm x tn tiles of one (matrix, row chunk) group stay on one XCD
      // (they share the chunk's operands in L2).  The groups, heaviest chunk
      // first (corder; a chunk's matrices side by side), are dealt to the
      // XCDs in snake order (0..7, 7..0, ...), which evens out the XCDs' dW
      // work when a few hot experts hold most rows; every XCD takes one group
      // per row of 8 and starts with its heaviest.  The chunks of expert e
      // are cstart[e] .. cstart[e+1]-1.
      const int tm = ceil_div(p.M, BM), tn = ceil_div(p.N, BN);
      const int per_c = tm * tn;
      const int nchunk = p.cstart[p.E];
      const int row = slot / per_c;
      const int pos = row * kNumXcd + ((row & 1) ? kNumXcd - 1 - xcd : xcd);
      if (pos >= p.nmat * nchunk) return;
      const int rank = pos / p.nmat;
      mat = pos - rank * p.nmat;
      const int gc = p.corder[rank];
      const int r2 = slot - row * per_c;
      e = expert_of(p.cstart, [](int v) { return v; }, gc);  // cstart[e] <= gc < cstart[e+1]
      dw_chunk = gc - p.cstart[e];
      if (dw_chunk > 0) dw_slot = p.pstart[e] + dw_chunk - 1;
      const int mt = r2 / tn;
      nt_idx = r2 - mt * tn;
      m0 = mt * BM;
      n0 = nt_idx * BN;
      const int rows_e = p.offsets[e + 1] - p.offsets[e];
      kbase = (size_t)p.offsets[e] + (size_t)dw_chunk * kDwChunkRows;
      k_count = max(0, min(kDwChunkRows, rows_e - dw_chunk * kDwChunkRows));
      nk_pass = ceil_div(k_count, BK);
      // split operand: every 64-row block twice, hi stage then lo stage
      nk = ((p.A_lo || p.B_lo) && p.dw_split[e] != 0) ? 2 * nk_pass : nk_pass;
      rows_valid = p.M - m0;
    }
  }

  // Chained launches: wait until the first GEMM's tiles of this m-tile have
  // stored their results.  The producers run on this XCD and share its L2;
  // each adds to the counter there once its stores are acknowledged.  Every
  // wave observes the counter itself before it reads the results, so no
  // barrier is needed; the first read is issued here, at decode, and is
  // usually already satisfied when the wave gets to the wait.  Device-scope
  // atomic loads: a plain load could keep hitting a stale line in the CU's
  // L1.  Bounded.
  int chain_seen = 0;
  if constexpr (kRowGrouped) {
    if (p.mt_wait)
      chain_seen = __hip_atomic_load(p.mt_wait + gmt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  auto chain_wait = [&]() {
    int v = __builtin_amdgcn_readfirstlane(chain_seen);
    int n = 0;
    while (v < p.mt_need) {
      if (++n > kChainSpinLimit) {
        if (lane == 0) __hip_atomic_fetch_or(p.chain_err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
      __builtin_amdgcn_s_sleep(8);
      v = __builtin_amdgcn_readfirstlane(
          __hip_atomic_load(p.mt_wait + gmt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    }
  };

  // ---------------------------------------------------------------- operand sources
  const uint32_t lda2 = (uint32_t)p.lda * 2u, ldb2 = (uint32_t)p.ldb * 2u;
  __amdgpu_buffer_rsrc_t rA, rA2, rB, rB2;
  if constexpr (kRowGrouped) {
    rA = make_rsrc(p.A + (size_t)m0 * p.lda, (size_t)rows_valid * lda2);
    rA2 = rA;
    if constexpr (kGateUp) {  // rows n0.. of Wg[e], Wu[e] ([I, D])
      const size_t rows = (size_t)min(BN / 2, p.N - n0);
      rB = make_rsrc(p.B0 + ((size_t)e * p.N + n0) * p.ldb, rows * ldb2);
      rB2 = make_rsrc(p.B1 + ((size_t)e * p.N + n0) * p.ldb, rows * ldb2);
    } else if constexpr (MODE == kDown) {  // rows n0.. of Wd[e] ([D, I])
      const size_t rows = (size_t)min(BN, p.N - n0);
      rB = make_rsrc(p.B0 + ((size_t)e * p.N + n0) * p.ldb, rows * ldb2);
      rB2 = rB;
    } else if constexpr (MODE == kDA) {  // Wd[e] as (k = d) x (n = i), ld I
      rB = make_rsrc(p.B0 + (size_t)e * p.K * p.ldb, (size_t)p.K * ldb2);
      rB2 = rB;
    } else {  // kDXs: Wg[e] / Wu[e] as (k = i) x (n = d), ld D
      rB = make_rsrc(p.B0 + (size_t)e * (p.K / 2) * p.ldb, (size_t)(p.K / 2) * ldb2);
      rB2 = make_rsrc(p.B1 + (size_t)e * (p.K / 2) * p.ldb, (size_t)(p.K / 2) * ldb2);
    }
    if (p.a_gather) {
      rA = make_rsrc(p.A, (size_t)p.a_rows * lda2);
      rA2 = rA;
    }
  } else {
    const bf16_t* a = mat == 0 ? p.A : p.A2;
    const bf16_t* alo = mat == 0 ? p.A_lo : p.A2_lo;
    const size_t abytes = (size_t)k_count * lda2, bbytes = (size_t)k_count * ldb2;
    rA = make_rsrc(a + kbase * p.lda, abytes);
    rA2 = make_rsrc((alo ? alo : a) + kbase * p.lda, abytes);
    rB = make_rsrc(p.B0 + kbase * p.ldb, bbytes);
    rB2 = make_rsrc((p.B_lo ? p.B_lo : p.B0) + kbase * p.ldb, bbytes);
    // a gathered operand is addressed from the start of its token-major rows
    if (p.a_rowoff) rA = rA2 = make_rsrc(a, (size_t)p.a_rows * lda2);
    if (p.b_rowoff) rB = rB2 = make_rsrc(p.B0, (size_t)p.b_rows * ldb2);
  }

  // ---------------------------------------------------------------- kDW gathered operand
  // ga / gb: A / B k-rows are gathered (wave-uniform).  gofs[i]: byte offset of
  // the token row behind this lane's k-row of load instruction i of the next
  // stage; gtouch: the same for the row this lane touches for the L2 prefetch.
  const bool ga = !kRowGrouped && p.a_rowoff;
  const bool gb = !kRowGrouped && p.b_rowoff;
  constexpr int QG = mnmajor_instrs<BM>();
  uint32_t gofs[QG] = {}, gtouch = 0;
  char* const ring = lds + kRingOff;
  // kDW with a split operand: stage kt covers row block kt / 2, the hi part
  // when kt is even and the lo part when it is odd, so the exact operand's
  // lines of a block are still in L2 when its lo stage loads them again
  const bool il = !kRowGrouped && nk != nk_pass;
  auto blk = [&](int kt) { return il ? kt >> 1 : kt; };
  // index chunk of stage kt
  auto chunk_q = [&](int kt) { return blk(kt) / RING_STAGES; };
  const uint32_t* const gsrc = ga ? p.a_rowoff : gb ? p.b_rowoff : nullptr;
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(gsrc ? gsrc + kbase : nullptr,
                                              gsrc ? (size_t)k_count * 4u : 0);
  auto ring_load = [&](int q) __attribute__((always_inline)) {
    const int rb = q * RING_ROWS + wave * 64;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rS, LDS_PTR(void, ring + (q % RING_SLOTS) * (RING_ROWS * 4) + wave * 256), 4,
        (uint32_t)(rb + lane) * 4u, 0, 0, 0);
  };
  // byte offset of the token row behind k-row k of stage kt (past the rows: a
  // sentinel beyond every buffer, which reads zeros).  Branch-free, so that the
  // index reads of a stage are issued together.
  auto gtok = [&](int kt, int k) -> uint32_t {
    const int kr = blk(kt) * BK + k;
    const uint32_t v = *(const uint32_t*)(ring + (chunk_q(kt) % RING_SLOTS) * (RING_ROWS * 4) +
                                          (kr % RING_ROWS) * 4);
    return kr < k_count ? v : 0x80000000u;
  };
  auto gather_offsets = [&](int kt_load, int kt_touch) __attribute__((always_inline)) {
    constexpr int KPI = 512 / BM, LPR = BM / 8;
#pragma unroll
    for (int i = 0; i < QG; ++i) gofs[i] = gtok(kt_load, (wave + NW * i) * KPI + lane / LPR);
    gtouch = gtok(min(kt_touch, nk - 1), ((wave % (NW / 2)) * 64 + lane) / (BM / 64));
  };

  // Row-grouped A: the byte offset of each A row this lane loads (one row per
  // load instruction, fixed for the tile) and of the row it touches for the L2
  // prefetch.  Gathered rows come straight from the token-major operand; rows
  // past the expert's end get an offset beyond the buffer (they read zeros).
  constexpr int QA = kRowGrouped ? kmajor_instrs<BM>() : mnmajor_instrs<BM>();
  uint32_t aoff[QA], atouch = 0;
  if constexpr (kRowGrouped) {
    auto row_off = [&](int row) -> uint32_t {
      if (!p.a_gather) return (uint32_t)row * lda2;
      if (row >= rows_valid) return 0x80000000u;
      return (uint32_t)(p.a_gather[m0 + row] / p.a_div) * lda2;
    };
#pragma unroll
    for (int i = 0; i < QA; ++i) aoff[i] = row_off(KRPI * (wave + NW * i) + lane / KCH);
    if (wave < NW / 2) atouch = row_off(wave * 64 + lane);
  }

  // Row-grouped tiles with fewer than BM rows (an expert's last row tile):
  // the A pieces (64 rows each) from a_end on hold padding rows only and are
  // not loaded, and this wave's fragment rows from fm_valid on are padding
  // and take no fragment reads or MFMAs.  Every fragment row that is
  // multiplied lies in a loaded piece (zeros past the expert's end), so the
  // accumulators are exactly those of the zero-padded tile.  Wave-uniform.
  const int a_end = kRowGrouped ? min(QA, ceil_div(rows_valid, KRPI * NW)) : QA;
  const int fm_valid = kRowGrouped ? max(0, min(FM, ceil_div(rows_valid - wm * WTM, 16))) : FM;

  // Loads of stage kt, pieces [q0, q1) of LOADS_PER_STAGE (A first, then B);
  // A pieces only below a_end_.
  auto issue = [&](int kt, int q0, int q1, int a_end_) __attribute__((always_inline)) {
    char* sa = lds + (kt % NS) * STAGE_BYTES;
    char* sb = sa + A_BYTES;
    if constexpr (kRowGrouped) {
      const uint32_t k0b = (uint32_t)kt * BK * 2u;
      issue_kmajor<BM>(sa, wave, lane, k0b, [&](int i, int) { return aoff[i]; }, rA, 0, q0,
                       min(q1, a_end_));
      if constexpr (kGateUp) {
        // B rows 0..BN/2-1: gate rows, BN/2..BN-1: the matching up rows
        constexpr int QG = kmajor_instrs<BN / 2>();
        issue_kmajor<BN / 2>(sb, wave, lane, k0b, [&](int, int row) { return (uint32_t)row * ldb2; }, rB,
                             QA, q0, q1);
        issue_kmajor<BN / 2>(sb + (BN / 2) * BK * 2, wave, lane, k0b,
                             [&](int, int row) { return (uint32_t)row * ldb2; }, rB2, QA + QG, q0, q1);
      } else if constexpr (MODE == kDown) {
        issue_kmajor<BN>(sb, wave, lane, k0b, [&](int, int row) { return (uint32_t)row * ldb2; }, rB, QA,
                         q0, q1);
      } else if constexpr (MODE == kDA) {
        const int k0 = kt * BK;
        issue_mnmajor<BN>(sb, wave, lane, n0, [&](int, int k) { return (uint32_t)(k0 + k) * ldb2; },
                          rB, QA, q0, q1);
      } else {  // kDXs: k < I from Wg, k >= I from Wu
        const int half = p.K / 2, k0 = kt * BK;
        const bool up = k0 >= half;
        const int kr = up ? k0 - half : k0;
        issue_mnmajor<BN>(sb, wave, lane, n0, [&](int, int k) { return (uint32_t)(kr + k) * ldb2; },
                          up ? rB2 : rB, QA, q0, q1);
      }
    } else {
      // the split operand's low part against the same exact operand on odd
      // stages of a split tile
      const bool lo_pass = il && (kt & 1);
      const int k0 = blk(kt) * BK;
      issue_mnmajor<BM>(sa, wave, lane, m0, [&](int i, int k) {
        return ga ? gofs[i] : (uint32_t)(k0 + k) * lda2; }, lo_pass ? rA2 : rA, 0, q0, q1);
      issue_mnmajor<BN>(sb, wave, lane, n0, [&](int i, int k) {
        return gb ? gofs[i] : (uint32_t)(k0 + k) * ldb2; }, lo_pass ? rB2 : rB, QA, q0, q1);
    }
  };

  // L2 prefetch of stage kt: wave w touches 4 bytes of each of 64 distinct
  // 128-byte lines of the stage (waves 0 .. NW/2-1 the A lines, the rest the
  // B lines), so the stage's direct-to-LDS loads, issued PF stages
  // later, find their lines in L2.  Stages past the end re-touch stage nk - 1.
  // (Capture-free, every operand by value: selecting among captured resources
  // would make the optimiser load them through the closure at a computed
  // offset, forcing the resources out of scalar registers.)
  auto touch_stage = [](int kt, int nk_, bool il_, bool lead_, char* dst, int wave_, int lane_,
                        __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t ra2,
                        __amdgpu_buffer_rsrc_t rb, __amdgpu_buffer_rsrc_t rb2, uint32_t lda2_,
                        uint32_t ldb2_, int m0_, int n0_, int K_, uint32_t atouch_, bool ga_,
                        bool gb_, uint32_t gtouch_) __attribute__((always_inline)) {
    kt = min(kt, nk_ - 1);
    const int h = NW / 2;  // waves per operand
    const bool opa = wave_ < h;
    const int L = (opa ? wave_ : wave_ - h) * 64 + lane_;  // line within the operand
    __amdgpu_buffer_rsrc_t r;
    uint32_t off;
    if constexpr (kRowGrouped) {
      const uint32_t k0b = (uint32_t)kt * BK * 2u;
      if (opa) {
        r = ra;
        off = atouch_ + k0b;
      } else if constexpr (kGateUp) {
        const bool up = (wave_ - h) * 64 >= BN / 2;  // wave-uniform
        r = up ? rb2 : rb;
        off = (uint32_t)(up ? L - BN / 2 : L) * ldb2_ + k0b;
      } else if constexpr (MODE == kDown) {
        r = rb;
        off = (uint32_t)L * ldb2_ + k0b;
      } else {  // kDA / kDXs: B is [k][n], BN/64 lines per k-row
        constexpr int LPK = BN / 64;
        int k0 = kt * BK;
        r = rb;
        if constexpr (MODE == kDXs) {
          if (k0 >= K_ / 2) {
            k0 -= K_ / 2;
            r = rb2;
          }
        }
        off = (uint32_t)(k0 + L / LPK) * ldb2_ + (uint32_t)(n0_ + (L % LPK) * 64) * 2u;
      }
    } else {
      const bool lo_pass = il_ && (kt & 1);
      const int k0 = (il_ ? kt >> 1 : kt) * BK;
      constexpr int LPA = BM / 64, LPB = BN / 64;
      if (opa) {
        r = lo_pass ? ra2 : ra;
        off = (ga_ ? gtouch_ : (uint32_t)(k0 + L / LPA) * lda2_) + (uint32_t)(m0_ + (L % LPA) * 64) * 2u;
      } else {
        r = lo_pass ? rb2 : rb;
        off = (gb_ ? gtouch_ : (uint32_t)(k0 + L / LPB) * ldb2_) + (uint32_t)(n0_ + (L % LPB) * 64) * 2u;
      }
    }
    if (!lead_) off = 0x80000000u;  // past every buffer: no memory traffic, same count
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LDS_PTR(void, dst), 4, off, 0, 0, 0);
  };
  // The tiles that share an operand slice (an A slice: the tiles of one row
  // tile; a B slice: those of one column tile) run side by side on one XCD;
  // with kLead only the first of them touches its lines.
  const bool touch_lead = !kLead || (wave < NW / 2 ? nt_idx == 0 : mt_first != 0);
  char* const touch_dst = lds + NS * STAGE_BYTES + wave * 256;
  auto touch = [&](int kt) __attribute__((always_inline)) {
    touch_stage(kt, nk, il, touch_lead, touch_dst, wave, lane, rA, rA2, rB, rB2, lda2, ldb2, m0, n0, p.K,
                atouch, ga, gb, gtouch);
  };

  // gradient scale {s, 1/s} of the backward GEMMs (1 where unused)
  const float gsc = p.gscale ? p.gscale[0] : 1.0f;
  const float ginv = p.gscale ? p.gscale[1] : 1.0f;
  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---------------------------------------------------------------- main loop
  // The next stage's loads are spread over this stage's MFMAs: the FM * BK/32
  // rows of MFMAs are slots, and each of the first LOAD_SLOTS slots issues
  // LOADS_PER_SLOT loads before its MFMAs, so no wave holds its MFMAs back
  // behind a burst of memory instructions; the slot after them issues the
  // L2 prefetch touch.
  constexpr int SLOTS = FM * (BK / 32);
  constexpr int LOAD_SLOTS = kGemmLoadSlots;
  constexpr int LOADS_PER_SLOT = LOADS_PER_STAGE / LOAD_SLOTS;
  static_assert(LOADS_PER_SLOT * LOAD_SLOTS == LOADS_PER_STAGE && LOAD_SLOTS + 1 <= SLOTS,
                "load slots must split the stage's loads evenly and fit the MFMA rows");
  bool first_issued = false;  // stage 0's loads already issued by the gathered prologue
  if constexpr (!kRowGrouped) {
    if ((ga || gb) && nk > 0) {
      // the index chunks of stages 0 .. RA - 1; meanwhile the operand that is
      // not gathered needs no indices, so its part of stage 0 goes out at once
      // and only the index loads (issued before it) are waited for
      static_assert(QA == LOADS_PER_STAGE - QA, "gathered kDW tiles: equal A and B pieces");
      for (int s = 0; s < RA && s < nk; ++s)
        if (s == 0 || chunk_q(s) != chunk_q(s - 1)) ring_load(chunk_q(s));
      if (ga) issue(0, QA, LOADS_PER_STAGE, QA);
      else issue(0, 0, QA, QA);
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(QA) : "memory");
      __builtin_amdgcn_s_barrier();  // everyone's index chunks are in LDS
      asm volatile("" ::: "memory");
      gather_offsets(0, PF);
      if (ga) issue(0, 0, QA, QA);
      else issue(0, QA, LOADS_PER_STAGE, QA);
      first_issued = true;
    }
  }
  static_assert(NS == 2, "the prologue issues one stage");
  if constexpr (kRowGrouped) {
    // stage 0's weight pieces first: they need no row index (and, in a
    // chained down GEMM, nothing from the first GEMM), then the A pieces
    if (nk > 0) issue(0, QA, LOADS_PER_STAGE, a_end);
    if constexpr (MODE == kDown) {
      if (p.mt_wait) chain_wait();  // H rows of this m-tile stored
    }
    if (nk > 0) {
#pragma unroll
      for (int s = 1; s <= PF; ++s) touch(s);
      issue(0, 0, QA, a_end);
    }
  } else {
    if (nk > 0) {
#pragma unroll
      for (int s = 1; s <= PF; ++s) touch(s);
      if (!first_issued) issue(0, 0, LOADS_PER_STAGE, a_end);
    }
  }
  // Waves whose rows all lie past a ragged expert's end (row-grouped tiles)
  // skip the fragment reads and MFMAs; wave-uniform.
  const bool wave_rows = !kRowGrouped || wm * WTM < rows_valid;
  // One stage: wait for it, then MFMAs over it with the loads of stage
  // kt + NS - 1 interleaved (kMore: that stage exists; kPart: a row tile with
  // padding rows, see a_end and fm_valid).
  auto stage = [&](int kt, auto more_tag, auto part_tag) __attribute__((always_inline)) {
    constexpr bool kMore = decltype(more_tag)::value;
    constexpr bool kPart = decltype(part_tag)::value;
    const int a_lim = kPart ? a_end : QA;
    // stage kt has landed once only the prefetch touch issued after its loads
    // may still be in flight
    if (kt == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
    __builtin_amdgcn_s_barrier();  // every wave's part of stage kt is in LDS, and
    asm volatile("" ::: "memory");  // every wave is done reading stage kt - 1
    if constexpr (!kRowGrouped && kMore) {
      if (ga || gb) {
        // load the index chunk that stage kt + RA starts, if it starts one; read
        // the indices of the next stage's loads and of the prefetch touch
        if (kt + RA < nk && chunk_q(kt + RA) != chunk_q(kt + RA - 1)) ring_load(chunk_q(kt + RA));
        gather_offsets(kt + 1, kt + 1 + PF);
      }
    }
    if (!wave_rows) {
      // all of this wave's rows are padding: it only moves its share of the
      // next stage (and the prefetch)
      if constexpr (kMore) {
        issue(kt + NS - 1, 0, LOADS_PER_STAGE, a_lim);
        touch(kt + NS - 1 + PF);
      }
      return;
    }
    const char* sa = lds + (kt % NS) * STAGE_BYTES;
    const char* sb = sa + A_BYTES;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      frag_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if (kPart && i >= fm_valid) continue;
        if constexpr (kRowGrouped) af[i] = read_kmajor<frag_t>(sa, wm * WTM + i * 16, kk, lane);
        else af[i] = read_mnmajor<BM, frag_t>(sa, wm * WTM + i * 16, kk, lane);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if constexpr (kGateUp) {
          const int r = j < FN / 2 ? wn * (WTN / 2) + j * 16 : BN / 2 + wn * (WTN / 2) + (j - FN / 2) * 16;
          bfr[j] = read_kmajor<frag_t>(sb, r, kk, lane);
        } else if constexpr (kBmn) {
          bfr[j] = read_mnmajor<BN, frag_t>(sb, wn * WTN + j * 16, kk, lane);
        } else {
          bfr[j] = read_kmajor<frag_t>(sb, wn * WTN + j * 16, kk, lane);
        }
      }
      // down, dXs: the weights (B) are bf16; every other fp16 operand is stored as fp16
      if constexpr (MODE == kDown || MODE == kDXs) {
#pragma unroll
        for (int j = 0; j < FN; ++j) bfr[j] = frag_to_f16(bfr[j]);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int slot = (kk / 32) * FM + i;
        const bool loads_here = kMore && slot < LOAD_SLOTS;
        if (loads_here)
          issue(kt + NS - 1, slot * LOADS_PER_SLOT, (slot + 1) * LOADS_PER_SLOT, a_lim);
        if (!kPart || i < fm_valid) {
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            if constexpr (kF16)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bfr[j], af[i], acc[i][j], 0, 0, 0);
            else
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
          }
        }
        // keep the order: this slot's loads, then its row of MFMAs
        if constexpr (!kPart) {
          if (loads_here) __builtin_amdgcn_sched_group_barrier(0x020, LOADS_PER_SLOT, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, FN, 0);
        }
        // raised issue priority between MFMA rows, normal after the stage's last
        // row, so the other wave on the SIMD reads its fragments meanwhile
        // (measured: -0.6% per step)
        if (i == FM - 1) __builtin_amdgcn_s_setprio(0);
        else __builtin_amdgcn_s_setprio(1);
        if (kMore && slot == LOAD_SLOTS) {
          touch(kt + NS - 1 + PF);  // the stage's last memory instruction
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
      }
    }
  };
  // the padding-aware stages where at least one A piece is padding only (with
  // more valid rows the full tile's schedule measured faster)
  int kt = 0;
  bool part = false;
  if constexpr (kRowGrouped) part = a_end < QA;
  if (part) {
    if constexpr (kRowGrouped) {
      for (; kt + NS - 1 < nk; ++kt) stage(kt, std::true_type{}, std::true_type{});
      for (; kt < nk; ++kt) stage(kt, std::false_type{}, std::true_type{});
    }
  } else {
    for (; kt + NS - 1 < nk; ++kt) stage(kt, std::true_type{}, std::false_type{});
    for (; kt < nk; ++kt) stage(kt, std::false_type{}, std::false_type{});
  }
  // no prefetch DMA may still be writing this workgroup's LDS when it ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---------------------------------------------------------------- epilogue
  // Lane holds, for fragment (i, j), row wm*WTM + i*16 + (lane % 16) and the 4
  // consecutive columns of B fragment j starting at 4 * (lane / 16).  Results
  // leave through per-wave LDS strips (see Strip).
  const int frow = lane & 15;
  const int cq = 4 * (lane >> 4);
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();  // every wave is done reading the stage buffers
  asm volatile("" ::: "memory");
  // Results are written once and not re-read by this kernel: non-temporal
  // stores keep them from evicting lines that later kernels still read.
  auto store16 = [](char* dst, u32x4 v) { __builtin_nontemporal_store(v, (u32x4*)dst); };
  if constexpr (MODE == kGateUpH) {
    // the wave's WTN/2 gate columns and the matching up columns
    constexpr int CW = WTN / 2;
    using S = Strip<CW, 2>;
    static_assert(NW * S::BYTES <= NS * STAGE_BYTES, "staging fits the stage buffers");
    char* const stg = lds + wave * S::BYTES;
    const int col0 = n0 + wn * CW;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int rb = wm * WTM + i * 16;  // strip's first row within the tile
#pragma unroll
      for (int j = 0; j < FN / 2; ++j) {
        const int cl = j * 16 + cq;
        const f32x4 g = acc[i][j], u = acc[i][j + FN / 2];
        float h[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) h[q] = g[q] * sigmoidf_(g[q]) * u[q];
        // H is the down GEMM's fp16 operand
        strip_put<S>(stg, frow, cl, u32x2{pack_f16x2(h[0], h[1]), pack_f16x2(h[2], h[3])});
      }
      strip_out<S>(stg, lane, rows_valid - rb, p.N - col0, [&](int r, int) {
        return (char*)(p.C0 + (size_t)(m0 + rb + r) * p.ldc + col0); }, store16);
    }
  } else if constexpr (MODE == kGateUpBwd) {
    // Recomputed g, u (fp32 accumulators) and dA = dOu Wd (fp32, read back),
    // with w the router weight of the row and s the gradient scale:
    //   h = silu(g) u;   partial dRW = sum of dA h over the wave's gate columns;
    //   dH = s w dA;  dG = dH u silu'(g);  dU = dH silu(g);  Hw = w h
    // (Hw: the weighted activations that dW_down needs).  The six fp16
    // outputs (dG, dU, Hw, each as hi = round(v) and, for experts whose dW
    // operand is split, lo = round(v - hi)) leave through per-wave LDS strips
    // as whole row segments.
    constexpr int CW = WTN / 2;  // gate columns of this wave
    constexpr int FJ = FN / 2;   // gate fragments of this wave
    using S = Strip<CW, 2>;
    static_assert(NW * 6 * S::BYTES <= NS * STAGE_BYTES, "staging fits the stage buffers");
    if (p.mt_wait) chain_wait();  // chained after dA: dA rows of this m-tile stored
    char* const stg = lds + wave * 6 * S::BYTES;
    const int I = p.N;
    const int col0 = n0 + wn * CW;  // the wave's first i column
    bf16_t* const outs[6] = {p.C0, p.C1, p.C2, p.L0, p.L1, p.L2};
    const size_t ldo[6] = {(size_t)p.ldc, (size_t)p.ldc, (size_t)I,
                            (size_t)p.ldc, (size_t)p.ldc, (size_t)I};
    // the low parts are read only by the dW GEMMs of experts with a split operand
    const bool need_lo = p.dw_split[e] != 0;
    // dA and the router weight of each 16-row block are read one block ahead
    // of their use, the sort-permutation entry behind the weight two blocks
    // ahead: the compiler cannot move a block's loads above the previous
    // block's output stores (it cannot rule out aliasing), so each block would
    // otherwise wait a full memory latency.  The loads are unconditional, from
    // clamped in-bounds addresses (row m0, column 0), and padding is zeroed
    // where the values are used: a load under a branch makes the compiler's
    // wait counts assume the worst at the join.
    auto src_of = [&](int i) {
      const int r = wm * WTM + i * 16 + frow;
      return p.s2f[m0 + (r < rows_valid ? r : 0)];
    };
    int src_next = src_of(0);
    float wr_next = p.topk_w[src_next];
    if (FM > 1) src_next = src_of(1);
    // dA blocks in flight ahead of their use
    constexpr int DA_AHEAD = 4;
    constexpr int NB = DA_AHEAD + 1 < FM ? DA_AHEAD + 1 : FM;
    f32x4 dbuf[NB][FJ];
    auto load_da = [&](int i, f32x4 (&dv)[FJ]) {
      const int r = wm * WTM + i * 16 + frow;
      const size_t m = (size_t)(m0 + (r < rows_valid ? r : 0));
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        const int col = col0 + j * 16 + cq;
        dv[j] = *(const f32x4*)(p.DA + m * (size_t)I + (col < I ? col : 0));
      }
    };
#pragma unroll
    for (int a = 0; a < DA_AHEAD && a < FM; ++a) load_da(a, dbuf[a % NB]);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      // block i + DA_AHEAD's dA, block i + 1's router weight, and block
      // i + 2's source row
      const float wr_i = wr_next;
      if (i + DA_AHEAD < FM) load_da(i + DA_AHEAD, dbuf[(i + DA_AHEAD) % NB]);
      if (i + 1 < FM) {
        wr_next = p.topk_w[src_next];
        if (i + 2 < FM) src_next = src_of(i + 2);
      }
      const int rb = wm * WTM + i * 16;
      const int r = rb + frow;
      const bool row_ok = r < rows_valid;
      const float wr = row_ok ? wr_i : 0.0f;
      const float wrs = wr * gsc;  // dG, dU carry the gradient scale
      float dot = 0.0f;
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        const int cl = j * 16 + cq;  // column within the wave's CW
        const bool ok = row_ok && col0 + cl < I;
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        const f32x4 dav = ok ? dbuf[i % NB][j] : zero;
        const f32x4 gv = acc[i][j], uv = acc[i][j + FJ];
        float dg[4], du[4], hw[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float g = gv[q];
          const float u = uv[q];
          const float da = dav[q];
          const float sg = sigmoidf_(g);
          const float h = g * sg * u;
          dot += da * h;
          const float dh = wrs * da;
          dg[q] = dh * u * sg * (1.0f + g * (1.0f - sg));
          du[q] = dh * g * sg;
          hw[q] = wr * h;
        }
        // fp16 hi = round(v) and lo = round(v - hi): the dX GEMM reads hi, the
        // dW GEMMs read hi and lo
        const u32x2 hi_dg = {pack_f16x2(dg[0], dg[1]), pack_f16x2(dg[2], dg[3])};
        const u32x2 hi_du = {pack_f16x2(du[0], du[1]), pack_f16x2(du[2], du[3])};
        const u32x2 hi_hw = {pack_f16x2(hw[0], hw[1]), pack_f16x2(hw[2], hw[3])};
        strip_put<S>(stg + 0 * S::BYTES, frow, cl, hi_dg);
        strip_put<S>(stg + 1 * S::BYTES, frow, cl, hi_du);
        strip_put<S>(stg + 2 * S::BYTES, frow, cl, hi_hw);
        if (need_lo) {
          u32x2 lo_dg, lo_du, lo_hw;
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            lo_dg[h2] = f16x2_residual(dg[2 * h2], dg[2 * h2 + 1], hi_dg[h2]);
            lo_du[h2] = f16x2_residual(du[2 * h2], du[2 * h2 + 1], hi_du[h2]);
            lo_hw[h2] = f16x2_residual(hw[2 * h2], hw[2 * h2 + 1], hi_hw[h2]);
          }
          strip_put<S>(stg + 3 * S::BYTES, frow, cl, lo_dg);
          strip_put<S>(stg + 4 * S::BYTES, frow, cl, lo_du);
          strip_put<S>(stg + 5 * S::BYTES, frow, cl, lo_hw);
        }
      }
      // this wave's strips are staged (a wave's LDS accesses complete in order)
#pragma unroll
      for (int o = 0; o < 6; ++o) {
        if (o >= 3 && !need_lo) break;
        strip_out<S>(stg + o * S::BYTES, lane, rows_valid - rb, I - col0, [&](int rr, int) {
          return (char*)(outs[o] + (size_t)(m0 + rb + rr) * ldo[o] + col0); }, store16);
      }
      dot += __shfl_xor(dot, 16);
      dot += __shfl_xor(dot, 32);
      if (row_ok && lane < 16) p.part[(size_t)(m0 + r) * p.np + nt_idx * WN + wn] = dot;
    }
  } else if constexpr (MODE == kDown || MODE == kDXs || MODE == kDA) {
    // O (bf16) and s dXs (fp16) leave as 2-byte elements, dA as fp32
    using S = Strip<WTN, MODE == kDA ? 4 : 2>;
    static_assert(NW * S::BYTES <= NS * STAGE_BYTES, "staging fits the stage buffers");
    char* const stg = lds + wave * S::BYTES;
    const int col0 = n0 + wn * WTN;
    // dXs: the flat slots of the rows this lane copies out, all read before
    // the first store.  Read next to the stores, each read would wait for
    // every store issued before it (loads and stores retire in issue order
    // under one counter), a store round trip per copy instruction.
    constexpr int NH = 16 / S::RPI;
    int flat[MODE == kDXs ? FM : 1][NH];
    if constexpr (MODE == kDXs) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          const int r = wm * WTM + i * 16 + h * S::RPI + lane / S::CPR;
          flat[i][h] = p.s2f[m0 + (r < rows_valid ? r : 0)];
        }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int rb = wm * WTM + i * 16;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int cl = j * 16 + cq;
        const f32x4 v = acc[i][j];
        // dXs rows keep the gradient scale s (fp16, away from its subnormal
        // range); the dX reduction removes it after the sum
        if constexpr (MODE == kDXs)
          strip_put<S>(stg, frow, cl, u32x2{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3])});
        else if constexpr (MODE == kDA) strip_put<S>(stg, frow, cl, v);
        else strip_put<S>(stg, frow, cl, u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])});
      }
      const int nrows = rows_valid - rb, ncols = p.N - col0;
      if constexpr (MODE == kDXs) {
        // rows at their flat slot t*K + k: the K copies of a token sit
        // together for the reduction
        strip_out<S>(stg, lane, nrows, ncols, [&](int, int h) {
          return (char*)(p.C0 + (size_t)flat[i][h] * p.ldc + col0); }, store16);
      } else if constexpr (MODE == kDA) {
        strip_out<S>(stg, lane, nrows, ncols, [&](int r, int) {
          return (char*)(p.Cf + (size_t)(m0 + rb + r) * p.ldc + col0); }, store16);
      } else {
        strip_out<S>(stg, lane, nrows, ncols, [&](int r, int) {
          return (char*)(p.C0 + (size_t)(m0 + rb + r) * p.ldc + col0); }, store16);
      }
    }
  } else {  // kDW
    using S = Strip<WTN, 4>;
    static_assert(NW * S::BYTES <= NS * STAGE_BYTES, "staging fits the stage buffers");
    char* const stg = lds + wave * S::BYTES;
    // chunk 0 writes (or accumulates into) the expert's gradient; chunks 1..
    // write partial tiles that launch_dw_reduce adds in chunk order
    float* const out = dw_slot < 0 ? (mat == 0 ? p.Cf : p.Cf2) + (size_t)e * p.M * p.N
                                    : p.dw_part + ((size_t)dw_slot * p.nmat + mat) * p.M * p.N;
    const int col0 = n0 + wn * WTN;
    const bool accum = dw_slot < 0 && p.accumulate != 0;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int rb = wm * WTM + i * 16;
#pragma unroll
      for (int j = 0; j < FN; ++j) strip_put<S>(stg, frow, j * 16 + cq, acc[i][j]);
      strip_out<S>(stg, lane, rows_valid - rb, p.N - col0, [&](int r, int) {
        return (char*)(out + (size_t)(m0 + rb + r) * p.N + col0); },
        [&](char* dst, u32x4 v) {
          f32x4 x = __builtin_bit_cast(f32x4, v) * ginv;
          if (accum) x += *(const f32x4*)dst;
          __builtin_nontemporal_store(x, (f32x4*)dst);
        });
    }
  }
  // Chained launches: once every wave's results are stored (acknowledged),
  // count this tile done for its m-tile.
  if constexpr (kRowGrouped) {
    if (p.mt_signal) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (tid == 0)
        __hip_atomic_fetch_add(p.mt_signal + gmt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}


template <int MODE, bool LEAD = false>
__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(2))) void grouped_gemm_kernel(
    GemmArgs p) {
  __shared__ __attribute__((aligned(1024))) char lds[tile_lds_bytes<MODE>()];
  gemm_tile<MODE, LEAD>(p, blockIdx.x % kNumXcd, blockIdx.x / kNumXcd, lds);
}

// Two row-grouped GEMMs in one launch (see launch_gemm_chain).  A workgroup
// takes its XCD from the hardware, not from its index: workgroup b is the
// XCD's (b / kNumXcd)-th, since the dispatcher deals consecutive workgroups
// to the XCDs round-robin (starting at any XCD).  It claims that (XCD, slot)
// pair, so a dispatch that broke the pattern (two workgroups on one pair, and
// so a pair left out) is reported; then it runs the slot-th tile of its XCD:
// the first GEMM's tiles of the XCD's m-tile range, then the second's.
template <int M1, int M2, bool LEAD>
__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(2))) void gemm_chain_kernel(
    GemmArgs a1, GemmArgs a2) {
  constexpr int kLds = std::max(tile_lds_bytes<M1>(), tile_lds_bytes<M2>());
  __shared__ __attribute__((aligned(1024))) char lds[kLds];
  const int xcd = (int)(__builtin_amdgcn_s_getreg(kHwRegXccId) & 0xf) % kNumXcd;
  const int slot = blockIdx.x / kNumXcd;
  int claimed = 0;
  if (threadIdx.x == 0)
    claimed = __hip_atomic_exchange(a1.xcd_claim + (size_t)xcd * (gridDim.x / kNumXcd) + slot, 1,
                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int n1 = (a1.xcd_mt[xcd + 1] - a1.xcd_mt[xcd]) * a1.n_tiles;
  if (slot < n1) gemm_tile<M1, LEAD && M1 != kDA>(a1, xcd, slot, lds);
  else gemm_tile<M2, LEAD && M2 != kDA>(a2, xcd, slot - n1, lds);
  if (threadIdx.x == 0 && claimed != 0)
    __hip_atomic_fetch_or(a2.chain_err, 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The three backward GEMMs that read only the recompute GEMM's outputs (dXs,
// dW_down, dW_gate + dW_up) in one launch: blocks [0, g1) run the dXs grid,
// [g1, g1 + g2) the dW_down grid, the rest the dW_gate/up grid.  None reads
// another's results, so no workgroup waits for another; the GPU starts the dW
// tiles as soon as CUs come free from the dXs tiles, with no tail between
// launches.  g1 and g2 are multiples of the XCD count, so every block runs on
// the XCD its own grid's tile order intends.
__global__ __launch_bounds__(NTH) __attribute__((amdgpu_waves_per_eu(2))) void bwd_fused_kernel(
    GemmArgs dxs, GemmArgs dw_down, GemmArgs dw_gateup, int g1, int g2) {
  __shared__ __attribute__((aligned(1024))) char lds[tile_lds_bytes<kDW>()];
  static_assert(tile_lds_bytes<kDW>() >= tile_lds_bytes<kDXs>(), "one LDS size serves both");
  const int b = blockIdx.x;
  const int xcd = b % kNumXcd;  // g1, g2: multiples of kNumXcd
  if (b < g1) gemm_tile<kDXs>(dxs, xcd, b / kNumXcd, lds);
  else if (b < g1 + g2) gemm_tile<kDW>(dw_down, xcd, (b - g1) / kNumXcd, lds);
  else gemm_tile<kDW>(dw_gateup, xcd, (b - g1 - g2) / kNumXcd, lds);
}
// ---------------------------------------------------------------------------
// Backward set-up.  Everything the backward GEMMs need from the routing and
// from max|dy| comes from one launch of 1024-thread workgroups with one role
// each (they share nothing, so any order of the workgroups gives the same
// result):
//   workgroups [0, E)   expert e's dW split flag; workgroup 0 also the
//                       gradient scale;
//   workgroup E         the tile starts of the row-grouped GEMMs;
//   workgroup E + 1     the dW row-chunk map;
//   workgroups E + 2..  the token-row byte offsets of the routed rows.

// dW row chunks: nch_e = max(1, ceil(rows_e / kDwChunkRows)); cstart =
// exclusive prefix of nch (cstart[E] = total); pstart = exclusive prefix of
// (nch_e - 1) (the partial slots of chunks 1..); slist = the experts with
// nch_e > 1 in ascending order, their number in slist[E].  corder = the chunk
// ids heaviest first, the order in which the dW grids deal their (matrix,
// chunk) groups to the XCDs: every chunk of kDwChunkRows rows in chunk order,
// then each expert's one shorter chunk (rows_e mod kDwChunkRows rows, or its
// only chunk when it has no rows) by rows descending, ties by expert.
// Deterministic (integer scans and ranks); one expert per thread, so
// E <= kChunkMapMaxE.
__device__ void dw_chunkmap_block(const int32_t* __restrict__ offsets, int E,
                                  int32_t* __restrict__ cstart, int32_t* __restrict__ pstart,
                                  int32_t* __restrict__ slist, int32_t* __restrict__ corder) {
  __shared__ int key[kChunkMapMaxE];
  const int e = threadIdx.x;
  const int rows = e < E ? offsets[e + 1] - offsets[e] : 0;
  const int nch = e < E ? max(1, (rows + kDwChunkRows - 1) / kDwChunkRows) : 0;
  const int full = rows / kDwChunkRows;  // chunks of kDwChunkRows rows
  int nchunk, npart, nlist, nfull;
  const int c0 = block_exclusive_scan_1024(nch, &nchunk);
  const int p0 = block_exclusive_scan_1024(nch > 1 ? nch - 1 : 0, &npart);
  const int s0 = block_exclusive_scan_1024(nch > 1 ? 1 : 0, &nlist);
  const int f0 = block_exclusive_scan_1024(full, &nfull);
  key[e] = nch > full ? rows - full * kDwChunkRows : -1;  // the shorter chunk's rows, if any
  __syncthreads();
  if (e < E) {
    cstart[e] = c0;
    pstart[e] = p0;
    if (nch > 1) slist[s0] = e;
    for (int c = 0; c < full; ++c) corder[f0 + c] = c0 + c;
    const int k = key[e];
    if (k >= 0) {
      int rank = 0;
      for (int j = 0; j < E; ++j) {
        const int kj = key[j];
        rank += kj > k || (kj == k && j < e);
      }
      corder[nfull + rank] = c0 + full;
    }
  }
  if (e == 0) {
    cstart[E] = nchunk;
    slist[E] = nlist;
  }
}

// Expert e: S = sum of topk_w[s2f[r]]^2 over the expert's n rows r, each of
// the 1024 threads summing a fixed stride of rows (four loads in flight),
// then a fixed tree, and split[e] = S * (1 + kDwSplitRows / n) * dim_factor >
// kDwSplitW2.
// Workgroup 0 also turns the kAmaxBlocks partial maxima of |dy| into the
// gradient scale {s, 1/s}: s = 2^(1 - x) for max|dy| = m 2^x, m in [0.5, 1),
// with x clamped to [-64, 64]; s = 1 when dy is all zero or not finite.
__device__ void bwd_prep_block(int e, const int32_t* __restrict__ offsets,
                               const int32_t* __restrict__ s2f, const float* __restrict__ topk_w,
                               float dim_factor, const uint32_t* __restrict__ amax_part,
                               int32_t* __restrict__ split, float* __restrict__ gscale) {
  __shared__ float wsum[16];
  __shared__ uint32_t wmax[4];
  const int tid = threadIdx.x;
  const int r0 = offsets[e], r1 = offsets[e + 1];
  {
    float s = 0.0f;
    int r = r0 + tid;
    for (; r + 3 * 1024 < r1; r += 4 * 1024) {
      int f[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) f[i] = s2f[r + i * 1024];
      float w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = topk_w[f[i]];
#pragma unroll
      for (int i = 0; i < 4; ++i) s += w[i] * w[i];
    }
    for (; r < r1; r += 1024) {
      const float w = topk_w[s2f[r]];
      s += w * w;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if ((tid & 63) == 0) wsum[tid >> 6] = s;
  }
  if (tid < 256) {
    if (e == 0) {
      uint32_t m = 0;
      for (int b = tid; b < kAmaxBlocks; b += 256) m = max(m, amax_part[b]);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
      if ((tid & 63) == 0) wmax[tid >> 6] = m;
    }
  }
  __syncthreads();
  if (tid == 0) {
    float q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = (wsum[4 * i] + wsum[4 * i + 1]) + (wsum[4 * i + 2] + wsum[4 * i + 3]);
    const float sw2 = (q[0] + q[1]) + (q[2] + q[3]);
    const int n = r1 - r0;
    split[e] = n > 0 && sw2 * (1.0f + kDwSplitRows / (float)n) * dim_factor > kDwSplitW2 ? 1 : 0;
  }
  if (e == 0 && tid == 0) {
    const uint32_t m = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
    float sc = 1.0f;
    if (m != 0 && m < 0x7f80u) {  // finite, nonzero
      int x;
      frexpf(__uint_as_float(m << 16), &x);
      x = min(64, max(-64, x));
      sc = ldexpf(1.0f, 1 - x);
    }
    gscale[0] = sc;
    gscale[1] = 1.0f / sc;
  }
}

__global__ __launch_bounds__(1024) void bwd_setup_kernel(BwdSetupArgs a) {
  const int b = blockIdx.x;
  if (b < a.E) {
    bwd_prep_block(b, a.offsets, a.s2f, a.topk_w, a.dim_factor, a.amax_part, a.split, a.gscale);
  } else if (b == a.E) {
    for (int i = threadIdx.x; i < a.nzero; i += 1024) a.zero[i] = 0;
    tile_starts_block(a.offsets, a.E, kGemmBM, a.tstart);
    if (a.xcd_mt) {
      __syncthreads();
      chain_bounds_block(a.tstart, a.E, a.xcd_mt);
    }
  } else if (b == a.E + 1) {
    dw_chunkmap_block(a.offsets, a.E, a.cstart, a.pstart, a.slist, a.corder);
  } else {
    // rowoff[p] = (s2f[p] / K) * row_bytes
    const int nb = gridDim.x - (a.E + 2);
    for (int p = (b - a.E - 2) * 1024 + threadIdx.x; p < a.R; p += nb * 1024)
      a.rowoff[p] = (uint32_t)(a.s2f[p] / a.K) * a.row_bytes;
  }
}

hipError_t launch_bwd_setup(const BwdSetupArgs& a, hipStream_t st) {
  if (a.E <= 0 || a.R < 0) return hipErrorInvalidValue;
  const int nro = a.R > 0 ? std::min((a.R + 1023) / 1024, 256) : 0;
  MOE_LAUNCH(kKBwdSetup, bwd_setup_kernel, dim3(a.E + 2 + nro), dim3(1024), 0, st, a);
  return hipGetLastError();
}

// The chunked experts' weight gradients, both reductions in one launch:
// workgroup (stripe, z) adds, for every chunked expert e = slist[i] in turn
// and the reduction z (0: dW_down from part_down, 1: dW_gate and dW_up from
// part), out_mat[e] += sum_{c >= 1} part[pstart[e] + c - 1][mat]  (c
// ascending), striding over the expert's nmat * M * N elements, 4 per thread
// and two such groups in flight.  Partial tiles are read once (non-temporal).
constexpr int kDwReduceStripes = 512;
__global__ __launch_bounds__(256) void dw_reduce_kernel(DwReduceArgs a0, DwReduceArgs a1,
                                                        const int32_t* __restrict__ slist,
                                                        const int32_t* __restrict__ pstart,
                                                        const int32_t* __restrict__ cstart,
                                                        int E) {
  const int nlist = slist[E];
  const DwReduceArgs& a = blockIdx.y == 0 ? a0 : a1;
  const int nmat = a.nmat;
  const size_t mn = (size_t)a.M * a.N;  // a multiple of 4 (N is a multiple of 64)
  const size_t total = (size_t)nmat * mn;
  const size_t step = (size_t)gridDim.x * 256 * 4;
  auto add = [&](int e, int nch, size_t slot0, size_t q) {
    const int mat = q >= mn ? 1 : 0;
    const size_t idx = q - mat * mn;
    float* o = (mat == 0 ? a.out0 : a.out1) + (size_t)e * mn + idx;
    const f32x4 prev = *(const f32x4*)o;
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    for (int c = 1; c < nch; ++c)
      s += __builtin_nontemporal_load((const f32x4*)(a.part + ((slot0 + c - 1) * nmat + mat) * mn + idx));
    *(f32x4*)o = prev + s;
  };
  for (int i = 0; i < nlist; ++i) {
    const int e = slist[i];
    const int nch = cstart[e + 1] - cstart[e];
    const size_t slot0 = (size_t)pstart[e];
    size_t q = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    for (; q + step < total; q += 2 * step) {
      add(e, nch, slot0, q);
      add(e, nch, slot0, q + step);
    }
    if (q < total) add(e, nch, slot0, q);
  }
}

hipError_t launch_dw_reduce(const DwReduceArgs& down, const DwReduceArgs& gateup,
                            const int32_t* slist, const int32_t* pstart, const int32_t* cstart,
                            int E, int max_chunked, hipStream_t st) {
  if (max_chunked <= 0) return hipSuccess;
  MOE_LAUNCH(kKDwReduce, dw_reduce_kernel, dim3(kDwReduceStripes, 2), dim3(256), 0, st, down,
             gateup, slist, pstart, cstart, E);
  return hipGetLastError();
}

hipError_t launch_bwd_fused(const GemmArgs& dxs, int g1, const GemmArgs& dw_down, int g2,
                            const GemmArgs& dw_gateup, int g3, hipStream_t st) {
  if (g1 % kNumXcd || g2 % kNumXcd) return hipErrorInvalidValue;
  const int grid = g1 + g2 + g3;
  if (grid <= 0) return hipSuccess;
  MOE_LAUNCH(kKGemmBwdFused, bwd_fused_kernel, dim3(grid), dim3(NTH), 0, st, dxs, dw_down,
             dw_gateup, g1, g2);
  return hipGetLastError();
}

hipError_t launch_gemm(int mode, const GemmArgs& a, int grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  switch (mode) {
    case kGateUpH:
      if (a.lead)
        MOE_LAUNCH(kKGemmGateUpH, (grouped_gemm_kernel<kGateUpH, true>), dim3(grid), dim3(NTH), 0,
                   st, a);
      else
        MOE_LAUNCH(kKGemmGateUpH, grouped_gemm_kernel<kGateUpH>, dim3(grid), dim3(NTH), 0, st, a);
      break;
    case kGateUpBwd:
      if (a.lead)
        MOE_LAUNCH(kKGemmGateUpGU, (grouped_gemm_kernel<kGateUpBwd, true>), dim3(grid), dim3(NTH), 0,
                   st, a);
      else
        MOE_LAUNCH(kKGemmGateUpGU, grouped_gemm_kernel<kGateUpBwd>, dim3(grid), dim3(NTH), 0, st, a);
      break;
    case kDown:
      if (a.lead)
        MOE_LAUNCH(kKGemmDown, (grouped_gemm_kernel<kDown, true>), dim3(grid), dim3(NTH), 0, st, a);
      else
        MOE_LAUNCH(kKGemmDown, grouped_gemm_kernel<kDown>, dim3(grid), dim3(NTH), 0, st, a);
      break;
    case kDA:
      MOE_LAUNCH(kKGemmDA, grouped_gemm_kernel<kDA>, dim3(grid), dim3(NTH), 0, st, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_chain(int mode1, const GemmArgs& a1, int mode2, const GemmArgs& a2,
                             int grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  if (!a1.mt_signal || a2.mt_wait != a1.mt_signal || !a2.chain_err || a2.mt_need != a1.n_tiles ||
      a1.tstart != a2.tstart || a1.E != a2.E || !a1.xcd_mt || a2.xcd_mt != a1.xcd_mt ||
      !a1.xcd_claim || a1.mt_wait || a2.mt_signal || grid % kNumXcd)
    return hipErrorInvalidValue;
  if (mode1 == kGateUpH && mode2 == kDown) {
    if (a1.lead != a2.lead) return hipErrorInvalidValue;
    if (a1.lead)
      MOE_LAUNCH(kKGemmFwdChain, (gemm_chain_kernel<kGateUpH, kDown, true>), dim3(grid), dim3(NTH),
                 0, st, a1, a2);
    else
      MOE_LAUNCH(kKGemmFwdChain, (gemm_chain_kernel<kGateUpH, kDown, false>), dim3(grid), dim3(NTH),
                 0, st, a1, a2);
  } else if (mode1 == kDA && mode2 == kGateUpBwd) {
    if (a2.lead)
      MOE_LAUNCH(kKGemmBwdChain, (gemm_chain_kernel<kDA, kGateUpBwd, true>), dim3(grid), dim3(NTH),
                 0, st, a1, a2);
    else
      MOE_LAUNCH(kKGemmBwdChain, (gemm_chain_kernel<kDA, kGateUpBwd, false>), dim3(grid),
                 dim3(NTH), 0, st, a1, a2);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe

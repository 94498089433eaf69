// Internal declarations of the MoE library's kernels and launchers.
#pragma once

#include "moe.h"
#include "common.hpp"

namespace moe {

// ---- per-kernel timing (prof.hip)
enum KernelId : int {
  kKRouteTopk, kKRouteHist, kKRouteScatter, kKTilemap,
  kKGemmGateUpH, kKGemmGateUpGU, kKGemmDown, kKGemmDA, kKCombine, kKReduceRows, kKRouterLogits,
  kKRouterPrep, kKRouterDx, kKRouterDwr, kKRouterDwrSum, kKDwReduce, kKBwdSetup, kKDyAmax,
  kKF16Operands, kKGemmBwdFused, kKGemmFwdChain, kKGemmBwdChain, kNumKernels
};
namespace prof {
void begin(int kid, hipStream_t st);  // no-ops unless timing is enabled
void end(hipStream_t st);
const char* name(int kid);
int set_enabled(int on);
int set_only(int kid);  // -1: every kernel; else only that id (-1 returned for a bad id)
int read(double* total_ms, int64_t* launches, int n);
}  // namespace prof

// Launch `kernel` bracketed by the optional timing events.
#define MOE_LAUNCH(kid, kernel, grid, block, lds, stream, ...)              \
  do {                                                                      \
    ::moe::prof::begin((kid), (stream));                                    \
    hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);      \
    ::moe::prof::end(stream);                                               \
  } while (0)

// ---- routing / sort (route.hip)
int route_chunk(int R);
hipError_t launch_route_sort(const moe_dims& d, const float* logits, int32_t* idx, float* w,
                             int32_t* counts, int32_t* offsets, int32_t* s2f, int32_t* f2s,
                             int32_t* hist, hipStream_t st);
// tstart [E+1] (the row-grouped GEMMs' m-tile starts, bm = kGemmBM); also
// zero[0 .. nzero) = 0 and, if xcd_mt is not null, the chained launches' XCD
// ranges xcd_mt[0 .. kNumXcd] (chain_bounds_block)
hipError_t launch_tilemap(const int32_t* offsets, int E, int bm, int32_t* tstart, int32_t* zero,
                          int nzero, int32_t* xcd_mt, hipStream_t st);

// ---- permutes (permute.hip)
hipError_t launch_combine(const void* O, const float* w, const int32_t* f2s, void* y, int T,
                          int K, int D, hipStream_t st);
// dx[t] = (1/s) sum_k dXs[t*K + k] with dXs the fp16 rows of s dXs and 1/s =
// gscale[1] (fp32 sum, k ascending, one bf16 rounding); in the same launch
// d_topk_w[f] = sum_{j<np} part[f2s[f] * np + j] (j ascending).
hipError_t launch_reduce_rows(const void* dXs, const float* gscale, void* dx, int T, int K, int D,
                              const float* part, const int32_t* f2s, float* d_topk_w, int np,
                              hipStream_t st);
// Largest |v| over the n bf16 values of src (n a multiple of 8): kAmaxBlocks
// workgroup maxima (bit patterns of |v|, ordered like the values) into part.
constexpr int kAmaxBlocks = 1024;
hipError_t launch_amax_bf16(const void* src, size_t n, uint32_t* part, hipStream_t st);
// fp16 operands of the weight-gradient GEMMs from the bf16 inputs (n values
// each, a multiple of 8): x16 = x (exact in fp16's normal range, rounded to
// nearest below it, infinite from 65520 on), dy16 = s dy with s = gscale[0]
// (exact in fp16's normal range; rounded toward zero below it).
hipError_t launch_f16_operands(const void* x, const void* dy, const float* gscale, void* x16,
                               void* dy16, size_t n, hipStream_t st);

// ---- router projection and router backward (router.hip)
hipError_t launch_router_logits(const void* x, const float* w_r, float* logits, int T, int D,
                                int E, hipStream_t st);
// Token ranges of the dW_r partials: `splits` ranges of `tokens_per_split` tokens.
void router_dwr_split(int T, int* splits, int* tokens_per_split);
hipError_t launch_router_bwd(const void* x, const float* w_r, const int32_t* topk_idx,
                             const float* topk_w, const float* d_topk_w, void* dx, float* dw_r,
                             int accumulate, float* dl, float* w_rt, float* part, int T, int D,
                             int E, int K, int score, hipStream_t st);

// ---- grouped GEMMs (gemm.hip)
// Workgroup tile geometry (shared by the kernels and the host-side tile
// accounting): 256 x 256 output tiles; 8 waves as 2 (rows) x 4 (columns), each
// 128 x 64; 64-deep K stages, two resident in LDS.
constexpr int kGemmBM = 256;  // rows of a workgroup tile (routed rows or dW rows)
constexpr int kGemmBN = 256;  // columns of a tile (gate/up: BN/2 gate + BN/2 up)
constexpr int kGemmBK = 64;   // reduction depth of one LDS stage
constexpr int kGemmWM = 2;    // waves along the rows
constexpr int kGemmWN = 4;    // waves along the columns
constexpr int kGemmNS = 2;    // K stages resident in LDS
// The next stage's loads are spread over the first kGemmLoadSlots rows of
// MFMAs of the current stage.
constexpr int kGemmLoadSlots = 8;
// An expert with n rows whose router weights have squares summing to S gets
// the fp16 hi + lo split of the rounded dW operand (two MFMA passes) when
//   S * (1 + kDwSplitRows / n) * max(1, 3 D / (8 I)) > kDwSplitW2,
// the others one pass over fp16 hi.  The single-pass rounding error of a dW
// entry grows like 2^-11 times the root-sum-square of its terms, and every
// term carries one factor of the row's router weight, hence S.  Few rows
// give the per-entry sums of squares a heavier tail over the D x I entries,
// and a wide D against I makes the gate/up gradient terms larger, hence the
// two factors.
constexpr float kDwSplitW2 = 16.0f;
constexpr float kDwSplitRows = 100.0f;
// The weight-gradient GEMMs process an expert's rows in chunks of at most this
// many rows, one workgroup per (chunk, output tile), so that a hot expert's
// tiles are spread over the GPU like everyone else's.  Chunk 0 writes (or
// accumulates into) the output; chunks 1.. write partial tiles that a
// reduction then adds in chunk order.
constexpr int kDwChunkRows = 4096;
// the dW row-chunk map takes one expert per thread of a 1024-thread workgroup
constexpr int kChunkMapMaxE = 1024;
// L2 prefetch distance in stages: each stage touches the lines of the stage
// kGemmPrefetch after the one it loads.
constexpr int kGemmPrefetch = 1;
// The "lead" prefetch policy of the gate/up and down GEMMs: only the first
// tile of each group that shares an operand slice touches it, at distance
// kGemmPrefetchLead.  The launch table (abi.hip) picks it when the experts
// average at least kLeadMinRows routed rows (their tiles then run side by
// side on an XCD); with fewer rows, and in the other GEMMs, every tile
// touches its own lines at distance kGemmPrefetch, which measured faster.
constexpr int kGemmPrefetchLead = 2;
constexpr int kLeadMinRows = 256;

enum GemmMode : int {
  kGateUpH = 0,    // H  = silu(Xs Wg^T) * (Xs Wu^T)                       fp16 [R, I]
  kGateUpBwd = 1,  // recompute G = Xs Wg^T, U = Xs Wu^T; the SwiGLU backward in the
                   // epilogue from dA: dG, dU, Hw (fp16) and router-weight partials
  kDown = 2,       // O  = H Wd^T (fp16 products)                         bf16 [R, D]
  kDA = 3,         // dA = dOu Wd                                         fp32 [R, I]
  kDXs = 4,        // s dXs = s (dG Wg + dU Wu)      fp16 [R, D], row f = flat slot of the routed row
  kDW = 5,         // dW[e] = A_e^T B_e over the expert's rows              fp32
};

struct GemmArgs {
  const bf16_t* A;   // row-grouped modes: [R, lda] K-major.  kDW: token-major [R, lda]
  // Row-grouped modes: if non-null, routed row p of A is row a_gather[p] / a_div
  // of the token-major A [a_rows, lda]: the gather is folded into the loads.
  const int32_t* a_gather;
  int a_div, a_rows;
  // kDW: if non-null, k-row p of A (B) lies at byte a_rowoff[p] (b_rowoff[p]) of
  // the token-major operand [a_rows (b_rows), ld]; at most one is gathered.
  const uint32_t* a_rowoff;
  const uint32_t* b_rowoff;
  int b_rows;
  // kDW row chunks: cstart [E+1] prefix of the per-expert chunk counts
  // max(1, ceil(rows / kDwChunkRows)); pstart [E] first partial slot of an
  // expert's chunks 1..; dw_part partial tiles [slot][nmat][M][N] fp32
  const int32_t* cstart;
  const int32_t* pstart;
  const int32_t* corder;  // kDW: the chunk ids heaviest first (dw_chunkmap_block)
  float* dw_part;
  const int32_t* dw_split;  // [E] 1: the expert's dW operand is split hi + lo
  // backward gradient scale {s, 1/s} (see launch_bwd_setup), or null (s = 1):
  // kGateUpBwd scales dG and dU by s; kDW multiplies its results by 1/s (kDXs
  // keeps s in its fp16 rows; the dX reduction removes it)
  const float* gscale;
  const bf16_t* A2;  // kDW second matrix's A (dW_up), else unused
  const bf16_t* B0;  // weights (row-grouped) or token-major activations (kDW)
  const bf16_t* B1;  // up weights (kGateUp*, kDXs)
  const int32_t* offsets;  // [E+1] expert row offsets
  const int32_t* tstart;   // [2 (E+1)] the tile map (tile_starts_block; row-grouped modes)
  int E;
  int M, N, K;  // kDW: output M x N per expert.  Row-grouped: N output cols, K reduction
  int lda, ldb;
  int n_tiles;  // row-grouped: column tiles per m-tile (gate/up: ceil(I/128), else ceil(N/256))
  int nmat;     // kDW: matrices in this launch (1 or 2)
  int lead;     // gate/up, down: 1 = the lead prefetch policy (kLeadMinRows)
  const f16_t* A_lo;   // kDW: low fp16 parts of a split A (mat 0) / A2 (mat 1), or null
  const f16_t* A2_lo;
  const f16_t* B_lo;   // kDW: low fp16 part of a split B, or null
  // epilogue operands
  bf16_t* C0;
  bf16_t* C1;
  bf16_t* C2;
  f16_t* L0;  // kGateUpBwd: low fp16 parts of dG, dU, Hw
  f16_t* L1;
  f16_t* L2;
  int ldc;
  float* Cf;
  float* Cf2;
  int accumulate;
  const float* DA;   // kGateUpBwd: dA = dOu Wd, fp32 [R, I] (sorted rows)
  const float* topk_w;
  const int32_t* s2f;
  float* part;  // kGateUpBwd: router-weight-gradient partials [R, np]
  int np;
  // Two row-grouped GEMMs in one launch, the second reading the first's
  // results (launch_gemm_chain): the first GEMM's tile of m-tile g adds 1 to
  // mt_signal[g] once its results are stored; a tile of the second waits until
  // mt_wait[g] >= mt_need before it reads them.  Null when not chained.
  int32_t* mt_signal;
  const int32_t* mt_wait;
  int mt_need;
  int32_t* chain_err;  // nonzero after a wait gave up (see launch_gemm_chain)
  // Row-grouped modes: null, or the XCDs' m-tile ranges [xcd_mt[x], xcd_mt[x+1])
  // (chain_bounds_block): XCD x then takes every column tile of its m-tiles.
  // With null, XCD x takes the x-th of kNumXcd equal ranges of the tile list.
  const int32_t* xcd_mt;
  int32_t* xcd_claim;  // chained launches: one flag per (XCD, slot), zero at launch
  // Row-grouped modes without xcd_mt: 1 = the XCDs take equal tile counts, 0 =
  // equal tile costs (last_tile_cost8).  The dXs GEMM, whose last tile wave the
  // fused launch's dW tiles fill, measured faster with equal counts; the
  // others with equal costs.
  int even_split;
};

// One grouped GEMM of the row-grouped modes (kGateUpH, kGateUpBwd, kDown, kDA).
// Grid: kNumXcd * rowgrouped_slots(m-tile bound, n_tiles), with a.xcd_mt
// null; kNumXcd * chain_slots(m-tile bound, n_tiles) with the XCD ranges.
hipError_t launch_gemm(int mode, const GemmArgs& a, int grid, hipStream_t st);
// Workgroups per XCD of a row-grouped GEMM over at most mt_bound m-tiles of
// n_tiles tiles each: with equal tile counts (even_split) an equal share;
// with equal tile costs (see the tile decode) at most twice that, plus two
// (no tile costs less than 5/8 of another).
inline int rowgrouped_slots(int64_t mt_bound, int n_tiles, bool even_split = false) {
  const int64_t share = (mt_bound * n_tiles + kNumXcd - 1) / kNumXcd;
  return (int)(even_split ? share : 2 * share + 2);
}
// The chained launches' XCD ranges put an m-tile boundary near every
// kNumXcd-th of the routed rows, at most kChainSlack m-tiles away from an equal
// split of the m-tiles.  The row-grouped GEMMs are chained when the m-tile
// bound per XCD lies in [kChainMinMtPerXcd, kChainMaxMtPerXcd]: with fewer, one
// m-tile more or less unbalances the XCDs; with more, the last tile wave that
// chaining fills is a small share of the launch, while the per-tile waits and
// signals grow with the tile count (measured at the Qwen shape with
// Zipf-skewed routing over 16384 tokens, 80 m-tiles per XCD: -1.1% per step).
constexpr int kChainSlack = 3;
constexpr int kChainMinMtPerXcd = 16;
constexpr int kChainMaxMtPerXcd = 128;
inline int chain_slots(int64_t mt_bound, int n_tiles) {
  return (int)(((mt_bound + kNumXcd - 1) / kNumXcd + 2 * kChainSlack) * n_tiles);
}
// xcd_mt[0 .. kNumXcd] (see GemmArgs::xcd_mt) from the tile map (threads
// 0 .. kNumXcd of the calling block; tstart, with its cost prefix, must be
// visible to them): xcd_mt[x] is the m-tile boundary nearest to x / kNumXcd
// of the m-tiles' total cost (last_tile_cost8), clamped to within kChainSlack of
// x M / kNumXcd (M = tstart[E]), so the ranges are nondecreasing, cost about
// the same, and none holds more than ceil(M / kNumXcd) + 2 kChainSlack m-tiles.
__device__ inline void chain_bounds_block(const int32_t* __restrict__ tstart, int E,
                                          int32_t* __restrict__ xcd_mt) {
  const int x = threadIdx.x;
  if (x > kNumXcd) return;
  const int32_t* const cpre = tstart + E + 1;
  const int M = tstart[E];
  int v = x == 0 ? 0 : M;
  if (x > 0 && x < kNumXcd) {
    const int64_t t = (int64_t)x * cpre[E] / kNumXcd;
    int lo = 0, hi = E;  // cpre[lo] <= t < cpre[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (cpre[mid] <= t) lo = mid;
      else hi = mid;
    }
    // the expert's m-tiles cost 8 each but the last one
    const int mc = tstart[lo + 1] - tstart[lo];
    const int j = (int)((t - cpre[lo] + 4) / 8);
    v = tstart[lo] + min(j, mc);
    const int base = (int)((int64_t)x * M / kNumXcd);
    v = min(max(v, base - kChainSlack), base + kChainSlack);
    v = min(max(v, 0), M);
  }
  xcd_mt[x] = v;
}
// Two row-grouped GEMMs as one launch, the second reading the first's results
// (gate/up then down: a1 kGateUpH, a2 kDown; dA then the recompute: a1 kDA,
// a2 kGateUpBwd).  Each XCD takes the same range of m-tiles in both (xcd_mt,
// the same array in a1 and a2) and runs the first GEMM's tiles of its range
// before the second's; a tile of the second waits for the a1.n_tiles tiles of
// its m-tile (a2.mt_wait, filled through a1.mt_signal, which must hold zeros
// for every m-tile at launch), before its first read of A (down) or of dA (the
// recompute's epilogue).  Grid: kNumXcd * chain_slots(bound, a1.n_tiles +
// a2.n_tiles).  A workgroup takes the tiles of the XCD it runs on (read from
// the hardware), as that XCD's (b / kNumXcd)-th workgroup: the dispatcher deals
// consecutive workgroups to the XCDs round-robin, and in index order within an
// XCD, so a wait is always for a tile of the same XCD (same L2) that an
// earlier workgroup of that XCD holds.  a1.xcd_claim (grid ints, zero at
// launch) records the (XCD, slot) pairs taken: a pair taken twice sets bit 2
// of *chain_err, a wait that exceeds its spin limit bit 1 (the results are
// then not valid); every wait is bounded, so the launch always completes.
hipError_t launch_gemm_chain(int mode1, const GemmArgs& a1, int mode2, const GemmArgs& a2,
                             int grid, hipStream_t st);
// dXs (grid g1), dW_down (grid g2) and dW_gate/up (grid g3) as one launch; the
// grids are those launch_gemm would take (g1, g2 multiples of kNumXcd).
hipError_t launch_bwd_fused(const GemmArgs& dxs, int g1, const GemmArgs& dw_down, int g2,
                            const GemmArgs& dw_gateup, int g3, hipStream_t st);

// Backward set-up, one launch (its workgroups each take one role):
//   split[e] = 1 when S, the sum of the squared router weights
//     topk_w[s2f[r]]^2 over expert e's n rows r, has
//     S * (1 + kDwSplitRows / n) * dim_factor > kDwSplitW2, where the caller
//     passes dim_factor = max(1, 3 D / (8 I)) (fixed summation order, so the
//     decision repeats bit for bit): its dW operand is split hi + lo;
//   gscale = {s, 1/s}, the power of two s with s * max|dy| in [1, 2) (s = 1
//     for an all-zero or non-finite dy), from the kAmaxBlocks maxima that
//     launch_amax_bf16 left in amax_part.  The gradient GEMMs carry s * dy,
//     s * dG, s * dU in fp16, away from its subnormal range, and multiply
//     their fp32 results by 1/s (all exact);
//   tstart [E+1]: the row-tile starts of the row-grouped GEMMs (as
//     launch_tilemap);
//   the dW row-chunk map: cstart [E+1] (chunk prefix), pstart [E] (first
//     partial slot of each expert's chunks 1..), slist [E+1] (the chunked
//     experts ascending, their number in slist[E]), corder [chunk bound]
//     (the chunk ids heaviest first: the dW grids' dealing order);
//   rowoff [R]: rowoff[p] = (s2f[p] / K) * row_bytes, the byte offset of
//     routed row p's token row in x16 and dy16.
struct BwdSetupArgs {
  const int32_t* offsets;
  const int32_t* s2f;
  const float* topk_w;
  const uint32_t* amax_part;
  int32_t* split;
  float* gscale;
  int32_t* tstart;
  int32_t* cstart;
  int32_t* pstart;
  int32_t* slist;
  int32_t* corder;  // [dw chunk bound] chunk ids, heaviest first
  uint32_t* rowoff;
  int32_t* zero;  // zero[0 .. nzero) = 0: the chained launch's status word and counters
  int nzero;
  int32_t* xcd_mt;  // null, or the chained launch's XCD ranges (chain_bounds_block)
  float dim_factor;
  int E, R, K;
  uint32_t row_bytes;
};
hipError_t launch_bwd_setup(const BwdSetupArgs& a, hipStream_t st);

// Chunked experts' weight gradients: out[e] += sum over chunks 1.. of the
// partial tiles (chunk order), for the nmat (1 or 2) M x N matrices of one
// reduction; one launch takes dW_down's and dW_gate/up's.  max_chunked bounds
// the number of chunked experts.
struct DwReduceArgs {
  const float* part;
  float* out0;
  float* out1;
  int nmat, M, N;
};
hipError_t launch_dw_reduce(const DwReduceArgs& down, const DwReduceArgs& gateup,
                            const int32_t* slist, const int32_t* pstart, const int32_t* cstart,
                            int E, int max_chunked, hipStream_t st);

}  // namespace moe

// Batched LM head (bf16, more than 64 rows): the vocabulary-wide GEMM on MFMA
// with the per-slab softmax and top-k fused, logits never leave the chip.
//
// [P1] "EAGLE 推测解码为什么比 Medusa 快？（含 EAGLE-2 动态草稿树）" §4.1: the draft
// distribution is softmax(LM_Head(f-hat)) and each level keeps the top-k of
// every expanded row.  With many rows (a large batch, or every tree row at
// once) the product stops being a weight stream and becomes a dense
// contraction, so it is tiled for operand reuse:
//
//  * a workgroup owns 256 rows x 256 vocabulary columns; each of its eight
//    waves owns 128 rows x 64 columns (8 x 4 tiles of v_mfma_f32_16x16x32_bf16,
//    128 fp32 accumulators per lane), so one 64-column slab per wave;
//  * the main loop is the ping-pong MFMA core of the tiled GEMMs
//    (mfma_pingpong.h): operands straight from memory into four LDS stage
//    buffers, two wave groups offset by half a k-step so that every SIMD's
//    matrix core always has a wave feeding it;
//  * blocks are numbered so that each XCD (blocks b, b+8, ...) takes a
//    contiguous run of tiles, the row tiles of one column block adjacent, so
//    that a weight tile is fetched from memory once and re-read from that
//    XCD's L2;
//  * epilogue: a wave's 64 columns are one 64-column slab of the same record
//    layout as the other LM-head kernels (max, sum exp, top-k logits, ids),
//    one lane per row over a column-major LDS tile in the stage buffers.
#include <hip/hip_ext.h>

#include "mfma_pingpong.h"

namespace eg {

constexpr int LG_ROWS = PP_TM;   // rows per workgroup: 2 row groups of 128
constexpr int LG_COLS = PP_TN;   // columns per workgroup: 4 slabs of 64

int lmgemm_rows() { return LG_ROWS; }

// The feature rows [M][K] (row-major bf16, K a multiple of 8) in fragment
// order: block (group, s) = rows 16*group.. x k 32*s.., lane l = 16g + i's 16
// bytes (row 16*group + i, k 32*s + 8g..) at l*16.  One wave per block.
__global__ void __launch_bounds__(256) k_lg_xpack(const bf16_t* x, int M, int K, int nks, int nblocks,
                                                  bf16_t* xpk) {
  const int blk = blockIdx.x * 4 + (int)(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (blk >= nblocks) return;
  const int grp = blk / nks, s = blk - grp * nks;
  const int row = min(16 * grp + (lane & 15), M - 1), k = 32 * s + 8 * (lane >> 4);
  uint4 v = make_uint4(0u, 0u, 0u, 0u);
  if (k < K) v = ld16(x + (size_t)row * K + k);
  *(uint4*)(xpk + (size_t)blk * 512 + lane * 8) = v;
}

__global__ void __launch_bounds__(PP_THREADS) k_lmgemm(RoundArgs a, LmPlan p, int level, int per_xcd) {
  typedef bf16_t T;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;  // 128-row group, 64-column slab
  const int K = a.d;
  const int nks = K / 32;                   // a multiple of 4 (the plan checks)
  const int ngrp = (p.M + 15) / 16, ntile = (a.V + 15) / 16;
  const int ncb = (a.V + LG_COLS - 1) / LG_COLS, ntiles = ncb * p.zg;
  // block b runs on XCD b % 8; XCD x takes tiles x*per_xcd .. (row tiles of
  // a column block adjacent); the blocks past the last tile end here
  const int j = blockIdx.x >> 3, lin = (blockIdx.x & 7) * per_xcd + j;
  if (j >= per_xcd || lin >= ntiles) return;
  const int cb = lin / p.zg, rb = lin - cb * p.zg;

  // this wave's fragments 4*wave .. 4*wave+3 of every k-step: 0..15 the
  // feature groups of the row tile, 16..31 the weight tiles of the column
  // block (a group or tile past the last repeats the last)
  const T* src[PP_DMA];
#pragma unroll
  for (int u = 0; u < PP_DMA; ++u) {
    const int f = PP_DMA * wave + u;
    src[u] = f < 16 ? (const T*)a.xpk + (size_t)min(rb * 16 + f, ngrp - 1) * nks * wtile_elems<T>() + lane * 8
                    : wtile_base<T>(a.lm_head, nks, min(cb * 16 + f - 16, ntile - 1), lane);
  }
  f32x4_t acc[8][4];
  pp_main(nks, [&](int u, int s) -> const void* { return src[u] + (size_t)s * wtile_elems<T>(); }, acc);

  // ---- epilogue, two passes of 64 rows per wave: the wave's 64 x 64 block
  // goes column-major to a 16 KB tile (half of a stage buffer), row r of
  // column c at c*64 + (r ^ 4*(c%16)) (float4 stores of 16 columns spread
  // over the banks, reads of one column by 64 lanes a permutation of one
  // 64-float run); lane r then reduces row r of the pass over the 64 columns
  float* tile = pp_scratch(wave >> 1, wave & 1);
  const int c = lane & 15, g = lane >> 4;
  const int slab = cb * 4 + wn;
  const int cbase = slab * 64;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int i = pass * 4 + jj;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = 16 * q + c;
        *(float4*)(tile + col * 64 + ((16 * jj + 4 * g) ^ (4 * c))) =
            make_float4(acc[i][q][0], acc[i][q][1], acc[i][q][2], acc[i][q][3]);
      }
    }
    __builtin_amdgcn_wave_barrier();
    const int row = rb * LG_ROWS + wm * 128 + pass * 64 + lane;
    // the row's 64 logits into registers once (columns past V: -inf)
    float v[64];
#pragma unroll
    for (int col = 0; col < 64; ++col)
      v[col] = cbase + col < a.V ? tile[col * 64 + (lane ^ (4 * (col & 15)))] : -INFINITY;
    lm_slab_record(a, p, v, row, slab, cbase);
    __builtin_amdgcn_wave_barrier();  // the tile is rewritten by the next pass
  }
}

hipError_t launch_lmgemm(const RoundArgs& a, const LmPlan& p, int level, hipStream_t s, hipEvent_t e0,
                         hipEvent_t e1) {
  // the feature rows into fragment order, then the GEMM (with events, the
  // first stamps the pack's start and the second the GEMM's end)
  const int K = a.d, nks = (K + 31) / 32, nblocks = (p.M + 15) / 16 * nks;
  const bf16_t* x = level == 1 ? (const bf16_t*)a.root_feat
                               : (const bf16_t*)a.feat + (size_t)(level - 1) * a.B * a.k * K;
  const dim3 pgrid((nblocks + 3) / 4);
  if (e0)
    hipExtLaunchKernelGGL(k_lg_xpack, pgrid, dim3(256), 0u, s, e0, nullptr, 0u, x, p.M, K, nks, nblocks,
                          (bf16_t*)a.xpk);
  else
    hipLaunchKernelGGL(k_lg_xpack, pgrid, dim3(256), 0, s, x, p.M, K, nks, nblocks, (bf16_t*)a.xpk);
  const int ntiles = (a.V + LG_COLS - 1) / LG_COLS * p.zg, per_xcd = (ntiles + 7) / 8;
  const dim3 grid(per_xcd * 8), block(PP_THREADS);
  if (e1)
    hipExtLaunchKernelGGL(k_lmgemm, grid, block, 0u, s, nullptr, e1, 0u, a, p, level, per_xcd);
  else
    hipLaunchKernelGGL(k_lmgemm, grid, block, 0, s, a, p, level, per_xcd);
  return hipGetLastError();
}

}  // namespace eg

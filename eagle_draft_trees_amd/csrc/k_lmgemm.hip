// Batched LM head (bf16, more than 64 rows): the vocabulary-wide GEMM on MFMA
// with the per-slab softmax and top-k fused, logits never leave the chip.
//
// [P1] "EAGLE 推测解码为什么比 Medusa 快？（含 EAGLE-2 动态草稿树）" §4.1: the draft
// distribution is softmax(LM_Head(f-hat)) and each level keeps the top-k of
// every expanded row.  With many rows (a large batch, or every tree row at
// once) the product stops being a weight stream and becomes a dense
// contraction, so it is tiled for operand reuse:
//
//  * a workgroup owns 512 rows x 128 vocabulary columns; each of its eight
//    waves owns 128 rows x 64 columns (8 x 4 tiles of v_mfma_f32_16x16x32_bf16,
//    128 fp32 accumulators per lane), so each weight tile is read from HBM
//    once per 512 rows and each feature fragment is reused four times;
//  * per k-step of 32, the 512 feature rows (32 KB) and the 128 weight rows
//    (8 KB) are staged in LDS in MFMA-fragment order (one kilobyte per 16x32
//    fragment, lane l's 16 bytes at l*16), so every operand read is one
//    conflict-free 16-byte LDS read per lane.  The packed weight tiles are
//    already in that order, and k_lg_xpack first writes the feature rows in it
//    (k past K zeroed, rows past M repeating row M-1), so every global load of
//    either operand is one contiguous kilobyte per wave instead of 16 rows'
//    half cache lines;
//  * two LDS buffers and two register stages: the global loads of step s+2
//    are in flight while step s computes, one barrier per step;
//  * epilogue: a wave's 64 columns are one 64-column slab of the same record
//    layout as the other LM-head kernels (max, sum exp, top-k logits, ids),
//    one lane per row over a column-major LDS tile.
#include <hip/hip_ext.h>

#include "eagle_internal.h"

namespace eg {

constexpr int LG_W = 8;                 // waves per workgroup
constexpr int LG_THREADS = LG_W * WAVE;
constexpr int LG_ROWS = 512;            // rows per z-group: 4 row groups of 128
constexpr int LG_COLS = 128;            // columns per workgroup: 2 column groups of 64
constexpr int LG_XB = LG_ROWS / 16;     // feature fragments per k-step
constexpr int LG_WB = LG_COLS / 16;     // weight fragments per k-step
constexpr int LG_STAGE = (LG_XB + LG_WB) * 1024;   // bytes of one staged k-step
constexpr int LG_XP = LG_XB * WAVE / LG_THREADS;    // feature pieces per thread per step (4)
constexpr int LG_TP = 64 + 4;           // epilogue tile: padded rows per column
constexpr int LG_EPI = LG_W * 64 * LG_TP * 4;      // epilogue tile bytes (64 rows per pass)
static_assert(LG_WB * WAVE == LG_THREADS, "one weight piece per thread per step");

size_t lmgemm_lds_bytes() { return (size_t)(2 * LG_STAGE > LG_EPI ? 2 * LG_STAGE : LG_EPI); }

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

__global__ void __launch_bounds__(LG_THREADS) k_lmgemm(RoundArgs a, LmPlan p, int level) {
  typedef bf16_t T;
  constexpr int KS = El<T>::KSTEP;  // 32
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 3, wn = wave >> 2;  // 128-row group, 64-column group
  const int blk = blockIdx.x, zg = blockIdx.z;
  const int K = a.d, kk_ = a.k;
  const int nks = (K + KS - 1) / KS;
  const int ntile = (a.V + 15) / 16;
  // ---- staging sources: thread tid fills lane (tid % 64) of feature
  // fragments tid/64 + 8u (u < 4) and of weight fragment tid/64; both come
  // from fragment-ordered buffers (a group past the last reads the last)
  const int ngrp = (p.M + 15) / 16;
  const T* xsrc[LG_XP];
#pragma unroll
  for (int u = 0; u < LG_XP; ++u) {
    const int grp = min(zg * (LG_ROWS / 16) + (tid >> 6) + LG_W * u, ngrp - 1);
    xsrc[u] = (const T*)a.xpk + (size_t)grp * nks * wtile_elems<T>() + lane * El<T>::PER16;
  }
  const T* wsrc = wtile_base<T>(a.lm_head, nks, min(LG_WB * blk + (tid >> 6), ntile - 1), lane);
  typedef uint4 Stage[LG_XP + 1];
  // loads are unconditional from clamped addresses
  auto gload = [&](Stage& r, int s) __attribute__((always_inline)) {
    s = min(s, nks - 1);  // past the last step: repeats it (stored, never read)
#pragma unroll
    for (int u = 0; u < LG_XP; ++u) r[u] = ld16(xsrc[u] + (size_t)s * wtile_elems<T>());
    r[LG_XP] = ld16w(wsrc + (size_t)s * wtile_elems<T>());
  };
  auto lstore = [&](const Stage& r, int buf, int s) __attribute__((always_inline)) {
    (void)s;
    unsigned char* b = lds + buf * LG_STAGE;
#pragma unroll
    for (int u = 0; u < LG_XP; ++u) *(uint4*)(b + (size_t)((tid >> 6) + LG_W * u) * 1024 + lane * 16) = r[u];
    *(uint4*)(b + (size_t)(LG_XB + (tid >> 6)) * 1024 + lane * 16) = r[LG_XP];
  };

  f32x4_t acc[8][4];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[j][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int buf) __attribute__((always_inline)) {
    const unsigned char* b = lds + buf * LG_STAGE;
    uint4 wf[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) wf[q] = *(const uint4*)(b + (size_t)(LG_XB + wn * 4 + q) * 1024 + lane * 16);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint4 xf = *(const uint4*)(b + (size_t)(wm * 8 + j) * 1024 + lane * 16);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[j][q] = mma16(xf, wf[q], acc[j][q], T());
    }
  };

  // ---- k-steps: buffers alternate; the loads two steps ahead stay in flight
  // (straight-line body over two steps, last one or two peeled, so that the
  // compiler's wait counts stay exact)
  // (scheduling barriers keep each phase where it is written: the compiler
  // would otherwise sink the loads to the end of the body and hoist the next
  // LDS store right behind them)
  Stage ra, rb;
  gload(ra, 0);
  __builtin_amdgcn_sched_barrier(0);
  gload(rb, 1);
  __builtin_amdgcn_sched_barrier(0);
  lstore(ra, 0, 0);
  __syncthreads();
  gload(ra, 2);
  __builtin_amdgcn_sched_barrier(0);
  int s = 0;
  for (; s + 2 < nks; s += 2) {
    compute(0);
    __builtin_amdgcn_sched_barrier(0);
    lstore(rb, 1, s + 1);
    __syncthreads();
    gload(rb, s + 3);
    __builtin_amdgcn_sched_barrier(0);
    compute(1);
    __builtin_amdgcn_sched_barrier(0);
    lstore(ra, 0, s + 2);
    __syncthreads();
    gload(ra, s + 4);
    __builtin_amdgcn_sched_barrier(0);
  }
  compute(0);
  if (s + 1 < nks) {
    __builtin_amdgcn_sched_barrier(0);
    lstore(rb, 1, s + 1);
    __syncthreads();
    compute(1);
  }
  __syncthreads();  // every wave is done with the staging buffers

  // ---- epilogue, two passes of 64 rows per wave: the wave's 64 x 64 block
  // goes to its LDS tile column-major (rows padded), then lane r reduces row r
  // of the pass over the slab's 64 columns
  float* tile = (float*)lds + (size_t)wave * 64 * LG_TP;
  const int c = lane & 15, g = lane >> 4;
  const int slab = blk * 2 + wn;
  const int cbase = slab * 64;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int j = pass * 4 + jj;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = 16 * q + c;
        *(float4*)(tile + (size_t)col * LG_TP + 16 * jj + 4 * g) =
            make_float4(acc[j][q][0], acc[j][q][1], acc[j][q][2], acc[j][q][3]);
      }
    }
    __builtin_amdgcn_wave_barrier();
    const int row = zg * LG_ROWS + wm * 128 + pass * 64 + lane;
    // the row's 64 logits into registers once (columns past V: -inf)
    float v[64];
#pragma unroll
    for (int col = 0; col < 64; ++col) v[col] = cbase + col < a.V ? tile[(size_t)col * LG_TP + lane] : -INFINITY;
    float mx = -INFINITY;
#pragma unroll
    for (int col = 0; col < 64; ++col) mx = fmaxf(mx, v[col]);
    float se = 0.f;
#pragma unroll
    for (int col = 0; col < 64; ++col) se += v[col] == -INFINITY ? 0.f : expf(v[col] - mx);
    if (row < p.M && slab < p.nblk) {  // (the second half of the last block may lie past V)
      float* rec = slab_field(a.lmpart, row, slab, p);  // field f at rec[f * nblk]
      rec[0] = mx;
      rec[p.nblk] = se;
      // top-k by (logit desc, id asc): pass r takes the best column below the
      // previous pick in that order; scanning columns upward, a strictly
      // greater value wins, so the lowest column of equal values is taken
      float pv = INFINITY;
      int pc = -1;
      for (int r = 0; r < kk_; ++r) {
        float bv = -INFINITY;
        int bc = -1;
#pragma unroll
        for (int col = 0; col < 64; ++col) {
          const bool below = v[col] < pv || (v[col] == pv && col > pc);
          if (below && v[col] > bv) {
            bv = v[col];
            bc = col;
          }
        }
        rec[(2 + r) * p.nblk] = bc >= 0 ? bv : -INFINITY;
        rec[(2 + kk_ + r) * p.nblk] = __int_as_float(bc >= 0 ? cbase + bc : -1);
        pv = bc >= 0 ? bv : -INFINITY;
        pc = bc >= 0 ? bc : 64;
      }
    }
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
  const dim3 grid((a.V + LG_COLS - 1) / LG_COLS, 1, p.zg), block(LG_THREADS);
  const size_t lds = lmgemm_lds_bytes();
  if (e1)
    hipExtLaunchKernelGGL(k_lmgemm, grid, block, (uint32_t)lds, s, nullptr, e1, 0u, a, p, level);
  else
    hipLaunchKernelGGL(k_lmgemm, grid, block, lds, s, a, p, level);
  return hipGetLastError();
}

}  // namespace eg

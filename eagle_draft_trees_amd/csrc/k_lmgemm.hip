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
//    fragment, lane l's 16 bytes at l*16: the packed weight tiles are already
//    in that order), so every operand read is one conflict-free 16-byte LDS
//    read per lane;
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
  const T* xbase = (level == 1) ? (const T*)a.root_feat
                                : (const T*)a.feat + (size_t)(level - 1) * a.B * kk_ * K;

  // ---- staging sources: thread tid fills lane (tid % 64) of feature
  // fragments tid/64 + 8u (u < 4) and of weight fragment tid/64
  const int fl = lane, fg = fl >> 4, fi = fl & 15;
  const T* xsrc[LG_XP];
#pragma unroll
  for (int u = 0; u < LG_XP; ++u) {
    const int mt = (tid >> 6) + LG_W * u;
    const int row = min(zg * LG_ROWS + 16 * mt + fi, p.M - 1);  // rows past M: row M-1 (never stored)
    xsrc[u] = xbase + (size_t)row * K + 8 * fg;
  }
  const T* wsrc = wtile_base<T>(a.lm_head, nks, min(LG_WB * blk + (tid >> 6), ntile - 1), lane);
  const int klast = K - 8;
  typedef uint4 Stage[LG_XP + 1];
  // loads are unconditional from clamped addresses; feature pieces past K are
  // zeroed when stored (the wait for the data belongs there)
  auto gload = [&](Stage& r, int s) __attribute__((always_inline)) {
    s = min(s, nks - 1);  // past the last step: repeats it (stored, never read)
    const int k = s * KS + 8 * fg;
#pragma unroll
    for (int u = 0; u < LG_XP; ++u) r[u] = ld16(xsrc[u] + (min(k, klast) - 8 * fg));
    r[LG_XP] = ld16w(wsrc + (size_t)s * wtile_elems<T>());
  };
  auto lstore = [&](const Stage& r, int buf, int s) __attribute__((always_inline)) {
    unsigned char* b = lds + buf * LG_STAGE;
    const bool kin = s * KS + 8 * fg < K;
#pragma unroll
    for (int u = 0; u < LG_XP; ++u)
      *(uint4*)(b + (size_t)((tid >> 6) + LG_W * u) * 1024 + lane * 16) = mask4(r[u], kin);
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
  const dim3 grid((a.V + LG_COLS - 1) / LG_COLS, 1, p.zg), block(LG_THREADS);
  const size_t lds = lmgemm_lds_bytes();
  if (e0 || e1)
    hipExtLaunchKernelGGL(k_lmgemm, grid, block, (uint32_t)lds, s, e0, e1, 0u, a, p, level);
  else
    hipLaunchKernelGGL(k_lmgemm, grid, block, lds, s, a, p, level);
  return hipGetLastError();
}

}  // namespace eg

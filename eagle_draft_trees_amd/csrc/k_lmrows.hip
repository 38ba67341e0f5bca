// LM head for 17..64 rows (bf16): the vocabulary-wide product on the
// 64-row streaming core, softmax and top-k fused, logits never leave the chip.
//
// [P1] "EAGLE 推测解码为什么比 Medusa 快？（含 EAGLE-2 动态草稿树）" §4.1: the draft
// distribution is softmax(LM_Head(f-hat)), and each level keeps the top-k
// tokens of every expanded node; a frontier of 17..64 rows (for instance 16
// sequences x top-4, or a batch of 64 chains) puts that many rows through
// the LM head at once.
//
//  * a workgroup streams 128*NQ vocabulary columns (8*NQ weight tiles of 16)
//    against the 64 rows (mfma_stream.h: weights and features loaded straight
//    into LDS several k-steps ahead), NQ chosen so that the workgroups number
//    about one per compute unit: each weight byte is read once, and the
//    features (read from L2 by every workgroup) are a fraction 4 / (8 NQ) of
//    the weight bytes;
//  * the feature rows: at levels 2 and up, the level's down epilogue has
//    also written them in 16-row blocks (one kilobyte per 16 rows x 32 k,
//    row-major inside a block), so a fragment is one contiguous kilobyte; at level 1 (the caller's root
//    features) they are read in place, lane l of an X fragment reading 16
//    bytes of row l%16, rows past M repeating row M-1 (a packing launch of its
//    own would cost more than it saves there);
//  * XCD x (blocks x, x+8, ...) takes a contiguous run of column blocks;
//  * epilogue: the 64 x 128*NQ logits go column-major to LDS (64-column
//    slabs, row r of column c at c*64 + (r XOR 4*(c%16)): the float4 stores of
//    16 columns spread over the banks, a column's read by 64 lanes is a
//    permutation of one run), then wave j reduces slab j, one lane per row, to
//    the same slab records as the other LM-head kernels (k_lmmerge merges
//    them).
#include <hip/hip_ext.h>

#include "mfma_stream.h"

namespace eg {

template <int NQ>
__global__ void __launch_bounds__(PS_THREADS) k_lmrows(RoundArgs a, LmPlan p, int level) {
  typedef bf16_t T;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = a.d, nks = K / 32;  // a multiple of ps_unroll<NQ>() (the plan checks)
  const int ntile = (a.V + 15) / 16;
  // column block of this workgroup: XCD x (blocks x, x+8, ...) takes a
  // contiguous run of column blocks
  const int nblk = (ntile + 8 * NQ - 1) / (8 * NQ), per = (nblk + 7) / 8;
  const int cbk = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (cbk >= nblk) return;
  const int t0 = cbk * 8 * NQ;  // the block's first 16-column tile
  // X fragment (wave % 4): row 16*(wave%4) + l%16, k 8*(l/16) of the step.
  // Packed (levels whose down epilogue wrote xpk in this call): one kilobyte
  // per 16 rows x 32 k, row-major inside it (xpk_index), the groups past the
  // last repeat it (rows past M within a group hold other data, and only give
  // rows that are never recorded).  In place: rows past M repeat row M-1.  The wave's weight tiles
  // NQ*wave + q (a tile past the last repeats the last).
  const T* xsrc;
  size_t xstep = 32;
  if (level >= 2 && a.lm_px) {
    xsrc = (const T*)a.xpk + (size_t)min(wave & 3, (p.M - 1) >> 4) * nks * 512 + (lane & 15) * 32 + 8 * (lane >> 4);
    xstep = 512;
  } else {
    const T* xbase = (level == 1) ? (const T*)a.root_feat
                                  : (const T*)a.feat + (size_t)(level - 1) * a.B * a.k * K;
    xsrc = xbase + (size_t)min(16 * (wave & 3) + (lane & 15), p.M - 1) * K + 8 * (lane >> 4);
  }
  const T* wsrc[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) wsrc[q] = wtile_base<T>(a.lm_head, nks, min(t0 + NQ * wave + q, ntile - 1), lane);
  f32x4_t acc[4][NQ];
  ps_main<NQ>(
      nks, [&](int s) -> const void* { return xsrc + xstep * s; },
      [&](int q, int s) -> const void* { return wsrc[q] + (size_t)s * wtile_elems<T>(); }, acc);

  // logits into the slab tiles
  const int c = lane & 15, g = lane >> 4;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int col = 16 * (NQ * wave + q) + c;  // column within the block
    float* tile = ps_slab<NQ>(col >> 6);
    const int cc = col & 63;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
      *(float4*)(tile + cc * 64 + ((16 * mt + 4 * g) ^ (4 * c))) =
          make_float4(acc[mt][q][0], acc[mt][q][1], acc[mt][q][2], acc[mt][q][3]);
  }
  __syncthreads();
  // slab j of the block: wave j, lane = row
  if (wave < 2 * NQ) {
    const int slab = cbk * 2 * NQ + wave, cbase = slab * 64;
    const float* tile = ps_slab<NQ>(wave);
    float v[64];
#pragma unroll
    for (int col = 0; col < 64; ++col)
      v[col] = cbase + col < a.V ? tile[col * 64 + (lane ^ (4 * (col & 15)))] : -INFINITY;
    lm_slab_record(a, p, v, lane, slab, cbase);
  }
}

hipError_t launch_lmrows(const RoundArgs& a, const LmPlan& p, int level, hipStream_t s, hipEvent_t e0,
                         hipEvent_t e1) {
  if (a.dtype != EAGLE_BF16 || a.d % (32 * (p.nq == 1 ? 8 : 4)) || p.M > 64 || p.M < 1) return hipErrorInvalidValue;
  const int ntile = (a.V + 15) / 16;
  const int nblk = (ntile + 8 * p.nq - 1) / (8 * p.nq);
  const dim3 grid((nblk + 7) / 8 * 8), block(PS_THREADS);
  auto go = [&](auto kern) {
    if (e0 || e1)
      hipExtLaunchKernelGGL(kern, grid, block, 0u, s, e0, e1, 0u, a, p, level);
    else
      hipLaunchKernelGGL(kern, grid, block, 0, s, a, p, level);
  };
  switch (p.nq) {
    case 1: go(k_lmrows<1>); break;
    case 2: go(k_lmrows<2>); break;
    case 3: go(k_lmrows<3>); break;
    case 4: go(k_lmrows<4>); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace eg

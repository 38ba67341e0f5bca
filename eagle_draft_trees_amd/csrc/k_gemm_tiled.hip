// Layer GEMMs of many rows (bf16, more than 64 rows: the extend of a large
// batch, or a wide frontier) on the tiled MFMA core.
//
// [P3] zdszero.github.io spec_medusa_eagle, "在 SGLang 里": the draft extend
// runs the draft layer over every accepted position of every sequence; with
// hundreds of rows its GEMMs stop being weight streams and become dense
// contractions.  The skinny layer GEMMs (k_gemm) hold 64 rows per workgroup
// and would read each weight matrix once per 64 rows; here a workgroup holds
// a 256 x 256 output tile (mfma_pingpong.h: operands straight into LDS, two
// wave groups offset by half a k-step), so a weight tile is read once per 256
// rows.
//
//  * X first goes into MFMA fragment order (k_gt_xpack): the FC's gathered
//    parent / true feature rows, x0 for q/k/v as its high and low bf16 parts
//    (two k-ranges: X_hi W^T + X_lo W^T, the same split as the skinny path),
//    the attention output for O, y*gain for gate/up.  The down projection's X
//    (the SwiGLU activations) is already stored in 16-row blocks; each lane's
//    DMA address picks its piece of a block.
//  * gate/up: a tile is 128 output columns, its gate tiles in the first half
//    of the weight fragments and the matching up tiles in the second.
//  * When the tiles alone would leave compute units idle, K is split across
//    workgroups (k-step ranges, multiples of four steps).
//  * Tiles write fp32 partials in the split layout of the skinny GEMMs, and
//    k_gemm_fin sums them in split order (deterministic) and runs the op's
//    fused epilogue (bias and token projection, RoPE and the K/V write,
//    residual and the RMSNorm partials, residual and the next feature), so
//    those epilogues are the same code as on the skinny path.  Unsplit
//    gate/up runs its SwiGLU epilogue in the tile instead: its partials would
//    be the largest (two matrices of rows x ffn) and the epilogue is local.
//  * Blocks are numbered so that XCD x (blocks x, x+8, ...) takes a
//    contiguous run of tiles, the row tiles of one (column block, split)
//    adjacent: they read the same weight slice, once from memory.
#include "mfma_pingpong.h"

namespace eg {

// The rows of a layer GEMM's X in fragment order: block (group, step) of 512
// elements at (group * nsx + step) * 512, lane l's 8 at l * 8 holding row
// 16*group + l%16, k 32*step + 8*(l/16) (rows past M repeat row M-1).  One
// wave per block.
template <int OP>
__global__ void __launch_bounds__(256) k_gt_xpack(RoundArgs a, GemmPlan p) {
  typedef bf16_t T;
  const int nks = p.K / 32, nsx = p.hl ? 2 * nks : nks;
  const int ngrp = (p.M + 15) / 16;
  const int blk = blockIdx.x * 4 + (int)(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (blk >= ngrp * nsx) return;
  const int grp = blk / nsx, s = blk - grp * nsx;
  const int row = min(16 * grp + (lane & 15), p.M - 1);
  const bool lo = p.hl && s >= nks;  // q/k/v: x0's low part
  const int k = 32 * (lo ? s - nks : s) + 8 * (lane >> 4);
  const T* src;
  if (OP == OP_FC) {
    if (a.mode == MODE_LEVEL) {
      const int b = row / a.k, j = row - b * a.k;
      const eagle_frontier_node& nd = a.frontier[((size_t)a.depth * a.B + b) * a.k + j];
      src = a.depth == 1 ? (const T*)a.root_feat + (size_t)b * a.d
                         : (const T*)a.feat + (((size_t)(a.depth - 1) * a.B + b) * a.k + clamp_slot(nd.pslot, a.k)) * a.d;
    } else {
      int tok;
      ext_row_src<T>(a, row, src, tok);
    }
  } else if (OP == OP_QKV) {
    src = (const T*)(lo ? a.x0l : a.x0b) + (size_t)row * p.K;
  } else if (OP == OP_O) {
    src = (const T*)a.attn + (size_t)row * p.K;
  } else {  // gate/up
    src = (const T*)a.yg + (size_t)row * p.K;
  }
  *(uint4*)((T*)a.xpk + (size_t)blk * 512 + lane * 8) = ld16(src + k);
}

// gate/up of an unsplit tile: act = silu(g / rms) * (u / rms) for the tile's
// 256 rows x 128 columns.  1/rms of each row comes from the O launch's
// per-block sums of squares (two threads per row, in block order, then their
// two sums); the up waves (wn 2, 3) hand their blocks to the gate waves of
// the same columns (wn 0, 1) through a stage buffer each, in MFMA lane order,
// so each gate lane finds its own elements' up values at its own offsets.
// The activations are stored in 16-row blocks, as the down projection reads
// them.
__device__ __forceinline__ void gateup_epilogue(const RoundArgs& a, const GemmPlan& p, const f32x4_t (&acc)[8][4],
                                                int rb, int cb) {
  typedef bf16_t T;
  __shared__ float s_ss[PP_TM][2];
  __shared__ float s_rstd[PP_TM];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  {
    const int r = tid >> 1, h = tid & 1, row = min(rb * PP_TM + r, p.M - 1);
    float sacc = 0.f;
    for (int q = h; q < p.nps; q += 2) sacc += a.ssq[(size_t)q * a.rows + row];
    s_ss[r][h] = sacc;
  }
  if (wn >= 2) {
    uint4* buf = wm == 0 ? (wn == 2 ? pp_s0 : pp_s1) : (wn == 2 ? pp_s2 : pp_s3);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) buf[(i * 4 + q) * WAVE + lane] = __builtin_bit_cast(uint4, acc[i][q]);
  }
  __syncthreads();
  if (tid < PP_TM) s_rstd[tid] = 1.0f / sqrtf((s_ss[tid][0] + s_ss[tid][1]) / (float)a.d + a.eps);
  __syncthreads();
  if (wn >= 2) return;
  const uint4* ubuf = wm == 0 ? (wn == 0 ? pp_s0 : pp_s1) : (wn == 0 ? pp_s2 : pp_s3);
  const int c = lane & 15, g = lane >> 4;
  const int nksf = (a.F + 31) / 32;  // the activations' k-steps (the down projection's K is F)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4_t u = __builtin_bit_cast(f32x4_t, ubuf[(i * 4 + q) * WAVE + lane]);
      const int col = cb * 128 + 64 * wn + 16 * q + c;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int lr = 128 * wm + 16 * i + 4 * g + r, row = rb * PP_TM + lr;
        if (row < p.M && col < p.N) {
          const float rs = s_rstd[lr];
          const float gv = acc[i][q][r] * rs, uv = u[r] * rs;
          El<T>::st((T*)a.act, xpk_index<T>(row, col, nksf), gv / (1.0f + expf(-gv)) * uv);
        }
      }
    }
  }
}

template <int OP>
__global__ void __launch_bounds__(PP_THREADS) k_gemm_tiled(RoundArgs a, GemmPlan p, int per_xcd) {
  typedef bf16_t T;
  constexpr int NW = OP == OP_GATEUP ? 2 : 1;
  constexpr int COLW = PP_TN / NW;  // output columns per tile
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int nks = p.K / 32;                  // weight k-steps (a multiple of 4)
  const int nsx = p.hl ? 2 * nks : nks;      // X k-steps
  const int ngrp = (p.M + 15) / 16, ntile = (p.N + 15) / 16;
  const int ncb = (p.N + COLW - 1) / COLW, nrb = (p.M + PP_TM - 1) / PP_TM;
  const int j = blockIdx.x >> 3, lin = (blockIdx.x & 7) * per_xcd + j;
  if (j >= per_xcd || lin >= ncb * nrb * p.S) return;
  const int rb = lin % nrb, rest = lin / nrb, split = rest % p.S, cb = rest / p.S;
  // down, extend: the sequence state advances here (the prefix grows by the
  // accepted length, the bonus token becomes the next root); nothing in this
  // launch or its finishing launch reads either field
  if (OP == OP_DOWN && a.mode == MODE_EXTEND && lin == 0) ext_advance_state(a, tid, PP_THREADS);
  const int s0 = split * p.tks, ns = min(nsx - s0, p.tks);  // this split's X steps (a multiple of 4)

  // this wave's four fragments of a step: u = 0, 1 the row tile's X group
  // 2*wave + u, u = 2, 3 the column block's weight tile 2*wave + u - 2
  // (gate/up: tiles 0..7 gate, 8..15 the same columns' up tiles); a group or
  // tile past the last repeats the last
  const T* base[PP_DMA];
#pragma unroll
  for (int u = 0; u < PP_DMA; ++u) {
    const int f = 2 * wave + (u & 1);
    if (u < 2) {
      const int grp = min(rb * 16 + f, ngrp - 1);
      base[u] = OP == OP_DOWN ? (const T*)a.act + (size_t)grp * nks * 512 + (lane & 15) * 32 + (lane >> 4) * 8
                              : (const T*)a.xpk + (size_t)grp * nsx * 512 + lane * 8;
    } else {
      const int t = NW == 2 ? cb * 8 + (f & 7) : cb * 16 + f;
      const int tt = min(t, ntile - 1);
      if (OP == OP_FC) base[u] = wtile_base<T>(a.fc_w, nks, tt, lane);
      if (OP == OP_QKV) base[u] = qkv_tile<T>(a, tt, nks, lane);
      if (OP == OP_O) base[u] = wtile_base<T>(a.wo, nks, tt, lane);
      if (OP == OP_GATEUP) base[u] = wtile_base<T>(f < 8 ? a.w_gate : a.w_up, nks, tt, lane);
      if (OP == OP_DOWN) base[u] = wtile_base<T>(a.w_down, nks, tt, lane);
    }
  }
  auto src = [&](int u, int s) __attribute__((always_inline)) -> const void* {
    int st = s0 + s;
    if (u >= 2 && st >= nks) st -= nks;  // q/k/v: the low part's steps reuse the weights
    return base[u] + (size_t)st * 512;
  };
  f32x4_t acc[8][4];
  pp_main<true>(ns, src, acc);

  if constexpr (OP == OP_GATEUP) {
    if (p.S == 1) {  // unsplit: the SwiGLU epilogue here, no partials
      gateup_epilogue(a, p, acc, rb, cb);
      return;
    }
  }

  // partials in the skinny GEMMs' split layout: (64-row group zg, 64-column
  // block blk, split, 16-column tile q) -> (w, 16-row tile mt, lane) x 4
  const int w = NW == 2 ? wn >> 1 : 0;
  const int blk = NW == 2 ? cb * 2 + (wn & 1) : cb * 4 + wn;
  if (blk < p.nblk) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int zg = rb * 4 + 2 * wm + (i >> 2), mt = i & 3;
      if (zg < p.zg) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float* part = a.gpart + ((((size_t)zg * p.nblk + blk) * p.S + split) * 4 + q) * (NW * 4) * 64 * 4;
          *(f32x4_t*)(part + ((size_t)(w * 4 + mt) * 64 + lane) * 4) = acc[i][q];
        }
      }
    }
  }
}

template <int OP>
static hipError_t launch_tiled_op(const RoundArgs& a, const GemmPlan& p, hipStream_t s) {
  const int nks = p.K / 32, nsx = p.hl ? 2 * nks : nks;
  if (p.K % 128 || p.mt != 4 || p.ct != 4 || p.S < 1 || p.tks % 4 || p.tks < 4) return hipErrorInvalidValue;
  if (OP != OP_DOWN) {
    const int nblocks = (p.M + 15) / 16 * nsx;
    hipLaunchKernelGGL(k_gt_xpack<OP>, dim3((nblocks + 3) / 4), dim3(256), 0, s, a, p);
  }
  constexpr int COLW = PP_TN / (OP == OP_GATEUP ? 2 : 1);
  const int tiles = (p.N + COLW - 1) / COLW * ((p.M + PP_TM - 1) / PP_TM) * p.S, per_xcd = (tiles + 7) / 8;
  hipLaunchKernelGGL(k_gemm_tiled<OP>, dim3(per_xcd * 8), dim3(PP_THREADS), 0, s, a, p, per_xcd);
  return hipGetLastError();
}

hipError_t launch_gemm_tiled(int op, const RoundArgs& a, const GemmPlan& p, hipStream_t s) {
  if (a.dtype != EAGLE_BF16) return hipErrorInvalidValue;
  switch (op) {
    case OP_FC: return launch_tiled_op<OP_FC>(a, p, s);
    case OP_QKV: return launch_tiled_op<OP_QKV>(a, p, s);
    case OP_O: return launch_tiled_op<OP_O>(a, p, s);
    case OP_GATEUP: return launch_tiled_op<OP_GATEUP>(a, p, s);
    default: return launch_tiled_op<OP_DOWN>(a, p, s);
  }
}

}  // namespace eg

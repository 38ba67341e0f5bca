// FC, O and down projections of 17..64 bf16 rows (a frontier such as 16
// sequences x top-4 or 64 chains, a short extend) on the 64-row streaming
// core.
//
// [P1] "EAGLE 推测解码为什么比 Medusa 快？（含 EAGLE-2 动态草稿树）" §4.1 and [P3]
// zdszero.github.io spec_medusa_eagle, "在 SGLang 里": every level runs the FC
// and the draft decoder layer over the frontier's rows.  At 17..64 rows each
// weight matrix is still read once per pass and the product is bound by that
// stream; the skinny GEMMs (k_gemm) reach 2.5-4.5 TB/s there because every
// workgroup stages all the rows' X (64 rows x its K range) through registers
// and LDS for only 64 columns, and these three need K split to fill the
// machine.  Here (mfma_stream.h) a workgroup streams 128*NQ columns with the
// weights and the rows' X fragments loaded straight into LDS several k-steps
// ahead:
//  * X is read in place: lane l of a fragment reads 16 bytes of row l%16 of
//    the op's activation rows (the FC's gathered parent / true feature rows,
//    the attention output for O, the packed SwiGLU activations for down);
//    rows past M repeat row M-1;
//  * K is split across workgroups (ranges of whole loop iterations, as even
//    as whole iterations allow) where the column blocks alone would leave
//    compute units idle;
//  * the workgroups write fp32 partials in the split layout of the skinny
//    GEMMs, and k_gemm_fin sums them in split order (deterministic) and runs
//    the op's fused epilogue, the same code as on the skinny path.
#include "mfma_stream.h"

namespace eg {

template <int OP, int NQ>
__global__ void __launch_bounds__(PS_THREADS) k_gemm_rows(RoundArgs a, GemmPlan p) {
  typedef bf16_t T;
  static_assert(OP == OP_FC || OP == OP_O || OP == OP_DOWN, "FC, O and down");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = p.K, nks = K / 32;
  const int ntile = (p.N + 15) / 16;
  const int split = blockIdx.x % p.S, cb = blockIdx.x / p.S;
  // this split's k-steps: the K range in units of the loop's unroll, dealt
  // as evenly as whole units allow (the first units % S splits one more)
  constexpr int U = ps_unroll<NQ>();
  const int units = nks / U, uq = units / p.S, ur = units - uq * p.S;
  const int s0 = (split * uq + min(split, ur)) * U, ns = (uq + (split < ur ? 1 : 0)) * U;
  // down, extend: the sequence state advances here (the prefix grows by the
  // accepted length, the bonus token becomes the next root); nothing in this
  // launch or its finishing launch reads either field
  if (OP == OP_DOWN && a.mode == MODE_EXTEND && blockIdx.x == 0) ext_advance_state(a, tid, PS_THREADS);

  // this lane's X row and k offset within a step
  const int r = min(16 * (wave & 3) + (lane & 15), p.M - 1), kq = 8 * (lane >> 4);
  const T* xs;
  size_t xstep = 32;  // elements per k-step
  if (OP == OP_FC) {
    if (a.mode == MODE_LEVEL) {
      const int b = r / a.k, j = r - b * a.k;
      const eagle_frontier_node& nd = a.frontier[((size_t)a.depth * a.B + b) * a.k + j];
      xs = a.depth == 1 ? (const T*)a.root_feat + (size_t)b * a.d
                        : (const T*)a.feat + (((size_t)(a.depth - 1) * a.B + b) * a.k + clamp_slot(nd.pslot, a.k)) * a.d;
    } else {
      int tok;
      ext_row_src<T>(a, r, xs, tok);
    }
    xs += kq;
  } else if (OP == OP_O) {
    xs = (const T*)a.attn + (size_t)r * K + kq;
  } else {  // down: 16-row blocks of the packed activations
    xs = (const T*)a.act + (size_t)(r >> 4) * nks * 512 + (r & 15) * 32 + kq;
    xstep = 512;
  }
  // the wave's weight tiles; a tile past the last repeats the last
  int tl[NQ];
  const T* ws[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    tl[q] = cb * 8 * NQ + NQ * wave + q;
    const int tt = min(tl[q], ntile - 1);
    if (OP == OP_FC) ws[q] = wtile_base<T>(a.fc_w, nks, tt, lane);
    if (OP == OP_O) ws[q] = wtile_base<T>(a.wo, nks, tt, lane);
    if (OP == OP_DOWN) ws[q] = wtile_base<T>(a.w_down, nks, tt, lane);
  }
  f32x4_t acc[4][NQ];
  ps_main<NQ>(
      ns, [&](int s) -> const void* { return xs + (size_t)(s0 + s) * xstep; },
      [&](int q, int s) -> const void* { return ws[q] + (size_t)(s0 + s) * wtile_elems<T>(); }, acc);

  // partials: (64-row group 0, 64-column block t/4, split, tile t%4) ->
  // (16-row tile mt < p.mt, lane) x 4
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    if (tl[q] < ntile) {
      const int blk = tl[q] >> 2, ct = tl[q] & 3;
      float* part = a.gpart + ((((size_t)blk * p.S + split) * 4 + ct) * p.mt) * 64 * 4;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        if (mt < p.mt) *(f32x4_t*)(part + ((size_t)mt * 64 + lane) * 4) = acc[mt][q];
    }
  }
}

template <int OP>
static hipError_t launch_rows_op(const RoundArgs& a, const GemmPlan& p, hipStream_t s) {
  const int ntile = (p.N + 15) / 16;
  const dim3 grid((ntile + 8 * p.nq - 1) / (8 * p.nq) * p.S), block(PS_THREADS);
  switch (p.nq) {
    case 1: hipLaunchKernelGGL((k_gemm_rows<OP, 1>), grid, block, 0, s, a, p); break;
    case 2: hipLaunchKernelGGL((k_gemm_rows<OP, 2>), grid, block, 0, s, a, p); break;
    case 4: hipLaunchKernelGGL((k_gemm_rows<OP, 4>), grid, block, 0, s, a, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_rows(int op, const RoundArgs& a, const GemmPlan& p, hipStream_t s) {
  if (a.dtype != EAGLE_BF16 || p.M < 1 || p.M > 64 || p.zg != 1 || p.K % 256 || p.S < 1 ||
      p.S > p.K / (32 * (p.nq == 1 ? 8 : 4)))
    return hipErrorInvalidValue;
  switch (op) {
    case OP_FC: return launch_rows_op<OP_FC>(a, p, s);
    case OP_O: return launch_rows_op<OP_O>(a, p, s);
    case OP_DOWN: return launch_rows_op<OP_DOWN>(a, p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace eg

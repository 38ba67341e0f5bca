// Frozen LM head + softmax + top-k, per vocabulary slab.
//
// [P1] "EAGLE 推测解码为什么比 Medusa 快？（含 EAGLE-2 动态草稿树）" §4.1: the draft
// distribution is softmax(LM_Head(f-hat)), and each level keeps the top-k
// tokens of every expanded node.  The slab records written here are merged
// into the rows' log-sum-exp and top-k by k_lmmerge.
//
// k_lmhead (one launch over the vocabulary): four waves per workgroup each
// stream 16 LM-head rows against the M feature rows (MFMA, A operand from
// LDS, X staged in K chunks with the next chunk's loads in flight during the
// current chunk, the next weight loads issued before the current MFMAs); the
// 64-column logit tile goes to LDS and each row's slab is reduced to (max,
// sum exp) and its top-k (logit desc, id asc).  Logits never leave the chip.
#include <hip/hip_ext.h>
#include <float.h>

#include <type_traits>

#include "skinny_core.h"

namespace eg {

template <typename T, int MT>
__global__ void __launch_bounds__(BLOCK) k_lmhead(RoundArgs a, LmPlan p, int level) {
  constexpr int KS = El<T>::KSTEP;
  constexpr int PER = El<T>::PER16;
  constexpr int ES = (int)sizeof(T);
  constexpr int ROWS = MT * 16;
  constexpr int U = MT == 1 ? 8 : 4;  // weight k-steps in flight (more m-tiles: more MFMA per load)
  constexpr int XRB = (4096 / MT) & ~15;
  constexpr int XST = XRB + 16;
  constexpr int KCH = (XRB / ES) / (2 * U * KS) * (2 * U * KS);  // elements per staged X chunk
  static_assert(KCH > 0, "chunk");
  static_assert(ROWS * 65 * 4 <= ROWS * XST, "logit tile aliases the X tile");
  __shared__ __attribute__((aligned(16))) unsigned char xs[ROWS * XST];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // workgroup -> (slab, row group): XCD x (blocks x, x+8, ...) takes a
  // contiguous run, the row groups of one slab adjacent
  const int nbz = p.nblk * p.zg, bpx = (nbz + 7) / 8;
  const int lb = (int)(blockIdx.x & 7) * bpx + (int)(blockIdx.x >> 3);
  if (lb >= nbz) return;
  const int zg = lb % p.zg, blk = lb / p.zg;
  const int K = a.d, kk_ = a.k;
  const int cl = wave * 16 + (lane & 15);
  const int n = blk * 64 + cl;
  const bool nv = n < a.V;
  const int nkt = (K + KS - 1) / KS;
  const int ntl = (a.V + 15) / 16;
  const T* wr = wtile_base<T>(a.lm_head, nkt, min(blk * 4 + wave, ntl - 1), lane);  // packed tile
  const T* xbase = (level == 1) ? (const T*)a.root_feat
                                : (const T*)a.feat + (size_t)(level - 1) * a.B * kk_ * K;
  const int rows_here = min(ROWS, p.M - zg * 64);
  const int kq = (lane >> 4) * PER;
  const unsigned char* xl = xs + (lane & 15) * XST + (lane >> 4) * 16;

  f32x4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nit = (K + U * KS - 1) / (U * KS);
  // X staging: a chunk is CPR 16-byte pieces per row, SB per thread, all
  // loaded before any is stored so that their latencies overlap.  Loads are
  // unconditional (a piece beyond K or the rows reads a valid piece of row 0
  // and is masked to zero) so that no load is left in flight on any path.
  constexpr int CPR = KCH / PER;
  constexpr int SB = ROWS * CPR / BLOCK;
  static_assert(SB * BLOCK == ROWS * CPR, "staging covers a chunk exactly");
  uint4 xv[SB];
  auto stage_load = [&](int kc) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const int idx = tid + u * BLOCK;
      const int r = idx / CPR, c = idx % CPR, k = kc + c * PER;
      const bool ok = k < K && r < rows_here;  // else: row 0's piece (valid), stored as zeros
      xv[u] = mask4(ld16(xbase + (size_t)(zg * 64 + (r < rows_here ? r : 0)) * K + min(k, K - PER)), ok);
    }
  };
  auto stage_store = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const int idx = tid + u * BLOCK;
      *(uint4*)(xs + (idx / CPR) * XST + (idx % CPR) * 16) = xv[u];
    }
  };
  // Weight loads are unconditional from a clamped in-row address (a product
  // beyond K is masked to zero at use), and two register buffers alternate, so
  // the loads of iteration it+1 stay in flight while iteration it runs (see the
  // layer GEMMs for the same structure).
  const int klast = K - PER;
  auto wload = [&](uint4 (&buf)[U], int it) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) buf[u] = ld16w(wr + (size_t)min(it * U + u, nkt - 1) * wtile_elems<T>());
  };
  auto compute = [&](const uint4 (&buf)[U], int it, int kc) __attribute__((always_inline)) {
    const int kb = it * U * KS;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = kb + u * KS;
      const bool kin = k + kq < K;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint4 xf = mask4(*(const uint4*)(xl + mt * 16 * XST + (k - kc) * ES), kin);
        acc[mt] = mma16(xf, buf[u], acc[mt], T());
      }
    }
  };
  uint4 wa[U], wb[U];
  stage_load(0);  // the first chunk's X and the first weights are in flight together
  wload(wa, 0);
  stage_store();
  __syncthreads();
  int it = 0;
  for (int kc = 0; kc < K; kc += KCH) {
    if (kc > 0) {  // this chunk's X, loaded during the previous chunk, into LDS
      __syncthreads();
      stage_store();
      __syncthreads();
    }
    // the next chunk's X in flight during this chunk's MFMAs (older than the
    // weight loads issued meanwhile, so storing it waits for it alone)
    if (kc + KCH < K) stage_load(kc + KCH);
    const int itend = min(nit, (kc + KCH) / (U * KS));
    for (; it + 1 < itend; it += 2) {
      wload(wb, it + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(wa, it, kc);
      wload(wa, it + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute(wb, it + 1, kc);
    }
    if (it < itend) {  // odd count: last chunk only
      compute(wa, it, kc);
      ++it;
    }
  }

  __syncthreads();
  float* tile = (float*)xs;  // [ROWS][65] logits
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      tile[(mt * 16 + (lane >> 4) * 4 + r) * 65 + cl] = nv ? acc[mt][r] : -INFINITY;
  __syncthreads();

  // per-row slab partials: (max, sum exp, top-k logits, top-k ids).  Each lane
  // ranks its column against the row's 64 columns in LDS (value desc, id asc:
  // ranks are unique); the lanes ranked below k write the slab's sorted list.
  for (int mr = wave; mr < rows_here; mr += 4) {
    const int row = zg * 64 + mr;
    const float* trow = tile + mr * 65;
    const float x = trow[lane];
    int rank = 0;
#pragma unroll
    for (int j = 0; j < 64; ++j) {
      const float y = trow[j];
      rank += (y > x || (y == x && j < lane)) ? 1 : 0;
    }
    const float mx = wave_max_dpp(x);
    const float s = wave_sum_dpp(x == -INFINITY ? 0.f : expf(x - mx));
    float* rec = slab_field(a.lmpart, row, blk, p);  // field f at rec[f * nblk]
    if (lane == 0) { rec[0] = mx; rec[p.nblk] = s; }
    if (rank < kk_) {
      rec[(2 + rank) * p.nblk] = x;
      rec[(2 + kk_ + rank) * p.nblk] = __int_as_float(x == -INFINITY ? -1 : blk * 64 + lane);
    }
  }
}

// LM head for at most 16 rows (drafting levels and level 1): the level GEMMs'
// streaming core over 16-column tiles of the vocabulary.  A workgroup holds CT
// tiles (one slab of CT*16 columns) and splits K over KSW waves per tile; X
// (the rows' features) is staged in LDS when it fits.  The slab's logits meet
// in LDS and one wave per row reduces them to the slab record (max, sum exp,
// top-k by (logit desc, id asc) from a wave top-k over 64-bit keys).
template <typename T, bool XL>
__global__ void __launch_bounds__(SK_MAXW * WAVE) k_lmskinny(RoundArgs a, LmPlan p, int level) {
  constexpr int KS = El<T>::KSTEP;
  constexpr int BU = 4;
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nwv = (int)(blockDim.x >> 6);
  // slab: XCD x (blocks x, x+8, ...) takes a contiguous run
  const int bpx = (p.nblk + 7) / 8;  // blocks per XCD
  const int bk = (int)(blockIdx.x & 7) * bpx + (int)(blockIdx.x >> 3);
  if (bk >= p.nblk) return;
  const int ct = wave % p.CT, ks = wave / p.CT;
  const int t = bk * p.CT + ct;
  const int c = lane & 15, g = lane >> 4;
  const int K = a.d, kk_ = a.k;
  const int n = t * 16 + c;
  const bool nv = n < a.V;
  const int nks = (K + KS - 1) / KS;
  // the packed tile (a tile past the last reads tile 0, discarded)
  const T* const wr[1] = {wtile_base<T>(a.lm_head, nks, t < (a.V + 15) / 16 ? t : 0, lane)};
  const T* xbase = (level == 1) ? (const T*)a.root_feat
                                : (const T*)a.feat + (size_t)(level - 1) * a.B * kk_ * K;
  const T* x0 = xbase + (size_t)(c < p.M ? c : 0) * K;  // rows past M repeat row 0 (discarded)
  const int s0k = (int)((long)ks * nks / p.KSW), s1k = (int)((long)(ks + 1) * nks / p.KSW);
  f32x4_t acc[1];
  const int nbu = ((nks + p.KSW - 1) / p.KSW + BU - 1) / BU;
  sk_stream<T, 1, BU, XL>(wr, x0, x0, K, K, s0k, s1k, nbu, dyn, acc, xbase, p.M);

  // K slices meet in LDS (over the X tile, once every wave is done with it),
  // then the slab's logits [16 rows][CT*16 columns]
  if (XL) __syncthreads();
  f32x4_t* red = (f32x4_t*)dyn;
  float* lg = (float*)(dyn + (size_t)nwv * WAVE * sizeof(f32x4_t));
  const int ncol = p.CT * 16, LW = ncol + 1;
  red[wave * WAVE + lane] = acc[0];
  __syncthreads();
  if (ks == 0) {
    f32x4_t v = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < p.KSW; ++s) v += red[(s * p.CT + ct) * WAVE + lane];
#pragma unroll
    for (int r = 0; r < 4; ++r) lg[(4 * g + r) * LW + ct * 16 + c] = nv ? v[r] : -INFINITY;
  }
  __syncthreads();

  // one wave per row: up to four columns per lane
  __shared__ __attribute__((aligned(16))) unsigned long long s_tk[SK_MAXW][2 * WAVE];  // wave_topk scratch
  const int col0 = bk * ncol;
  // (NC = columns per lane: two for slabs of up to 128 columns, else four)
  auto epi = [&](auto ncl) __attribute__((always_inline)) {
    constexpr int NC = decltype(ncl)::value;
    for (int row = wave; row < p.M; row += nwv) {
      float x[NC];
      unsigned long long key[NC];
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < NC; ++u) {
        const int j = lane + 64 * u;
        x[u] = j < ncol ? lg[row * LW + j] : -INFINITY;
        key[u] = x[u] == -INFINITY ? 0ull : argkey(x[u], col0 + j);
        mx = fmaxf(mx, x[u]);
      }
      mx = wave_max_dpp(mx);
      float se = 0.f;
#pragma unroll
      for (int u = 0; u < NC; ++u) se += x[u] == -INFINITY ? 0.f : expf(x[u] - mx);
      se = wave_sum_dpp(se);
      float* rec = slab_field(a.lmpart, row, bk, p);  // field f at rec[f * nblk]
      if (lane == 0) {
        rec[0] = mx;
        rec[p.nblk] = se;
      }
      const unsigned long long mine = wave_topk<NC>(key, kk_, s_tk[wave]);  // lane r: the r-th entry
      if (lane < kk_) {
        rec[(2 + lane) * p.nblk] = mine ? argkey_value(mine) : -INFINITY;
        rec[(2 + kk_ + lane) * p.nblk] = __int_as_float(mine ? argkey_id(mine) : -1);
      }
    }
  };
  if (ncol <= 128)
    epi(std::integral_constant<int, 2>());
  else
    epi(std::integral_constant<int, 4>());
}

// Launch through hipExtLaunchKernel when events are given (they then mark the
// kernel's own start and end), through the plain launch otherwise.
template <typename... A>
static void lm_launch(void (*k)(A...), dim3 g, dim3 b, size_t sh, hipStream_t s, hipEvent_t e0,
                      hipEvent_t e1, A... args) {
  if (e0 || e1)
    hipExtLaunchKernelGGL(k, g, b, (uint32_t)sh, s, e0, e1, 0u, args...);
  else
    hipLaunchKernelGGL(k, g, b, sh, s, args...);
}

template <typename T>
static hipError_t launch_lm_t(const RoundArgs& a, const LmPlan& p, int level, hipStream_t s,
                              hipEvent_t e0, hipEvent_t e1) {
  const int nbz = p.nblk * p.zg;
  const dim3 grid((nbz + 7) / 8 * 8), block(BLOCK);
  switch (p.mt) {
    case 1: lm_launch(k_lmhead<T, 1>, grid, block, 0, s, e0, e1, a, p, level); break;
    case 2: lm_launch(k_lmhead<T, 2>, grid, block, 0, s, e0, e1, a, p, level); break;
    case 3: lm_launch(k_lmhead<T, 3>, grid, block, 0, s, e0, e1, a, p, level); break;
    default: lm_launch(k_lmhead<T, 4>, grid, block, 0, s, e0, e1, a, p, level); break;
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_lmsk_t(const RoundArgs& a, const LmPlan& p, int level, hipStream_t s,
                                hipEvent_t e0, hipEvent_t e1) {
  const int nwv = p.CT * p.KSW;
  const size_t epi = (size_t)nwv * WAVE * sizeof(f32x4_t) + (size_t)16 * (p.CT * 16 + 1) * sizeof(float);
  const dim3 grid((p.nblk + 7) / 8 * 8), block(nwv * WAVE);
  if (p.xlds) {
    const size_t xb = sk_xtile_bytes(a.d, (int)sizeof(T));
    lm_launch(k_lmskinny<T, true>, grid, block, xb > epi ? xb : epi, s, e0, e1, a, p, level);
  } else {
    lm_launch(k_lmskinny<T, false>, grid, block, epi, s, e0, e1, a, p, level);
  }
  return hipGetLastError();
}

hipError_t launch_lmhead(const RoundArgs& a, const LmPlan& p, int level, hipStream_t s,
                         hipEvent_t e0, hipEvent_t e1) {
  if (p.big) return launch_lmgemm(a, p, level, s, e0, e1);
  if (p.nq) return launch_lmrows(a, p, level, s, e0, e1);
  if (p.sk)
    return a.dtype == EAGLE_BF16 ? launch_lmsk_t<bf16_t>(a, p, level, s, e0, e1)
                                 : launch_lmsk_t<float>(a, p, level, s, e0, e1);
  return a.dtype == EAGLE_BF16 ? launch_lm_t<bf16_t>(a, p, level, s, e0, e1)
                               : launch_lm_t<float>(a, p, level, s, e0, e1);
}

}  // namespace eg

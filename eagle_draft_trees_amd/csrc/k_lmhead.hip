// Frozen LM head + softmax + top-k + EAGLE-2 expansion, in one launch.
//
// [P1] "EAGLE 推测解码为什么比 Medusa 快？（含 EAGLE-2 动态草稿树）" §4.1: the draft
// distribution is softmax(LM_Head(f-hat)); §10.3: a node's value is the product
// of confidences on its root path, each level expands the best k nodes.
// [P3] zdszero.github.io spec_medusa_eagle, "在 SGLang 里": select_top_k_tokens
// multiplies the running score by this level's top-k probabilities and keeps
// the best topk of topk^2.  Scores are kept as sums of log-probabilities.
//
// Phase 1 (every workgroup): four waves each stream 16 vocabulary rows of the
// LM head (the same MFMA weight-streaming loop as the draft GEMMs) against the
// M feature rows; the 64-column logit tile goes to LDS.  Per row, one wave
// reduces its 64 columns to (max, sum exp) and the slab's top-k (logit desc,
// id asc).  Logits never leave the chip.
// Phase 2 (the grid's last workgroup): per row, combine the slabs' (max, sum)
// into log-sum-exp and merge the sorted slab lists by a tournament; log p =
// logit - lse.  Then per sequence: level 1 puts the root's k children into the
// pool and frontier; level L >= 2 scores the k*k children (parent score +
// log p), appends all of them to the pool in (frontier slot, rank) order and
// keeps the best k by (score desc, pool index asc) as the next frontier.
#include <float.h>

#include "eagle_internal.h"

namespace eg {

constexpr int LM_MAXBLK = 4096;  // vocab <= 262144

template <typename T, int MT>
__global__ void __launch_bounds__(BLOCK) k_lmhead(RoundArgs a, LmPlan p, int level) {
  constexpr int KS = El<T>::KSTEP;
  constexpr int PER = El<T>::PER16;
  constexpr int ROWS = MT * 16;
  __shared__ float tile[ROWS][65];
  __shared__ unsigned char heads[4][LM_MAXBLK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int blk = blockIdx.x, zg = blockIdx.z;
  const int K = a.d, kk_ = a.k;
  const int cl = wave * 16 + (lane & 15);
  const int n = blk * 64 + cl;
  const bool nv = n < a.V;
  const T* wr = (const T*)a.lm_head + (size_t)(nv ? n : 0) * K;

  const T* xr[MT];
  bool rv[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int row = zg * 64 + mt * 16 + (lane & 15);
    rv[mt] = row < p.M;
    const int r = rv[mt] ? row : 0;
    xr[mt] = (level == 1) ? (const T*)a.root_feat + (size_t)r * K
                          : (const T*)a.feat + ((size_t)(level - 1) * a.B * kk_ + r) * K;
  }

  f32x4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int kq = (lane >> 4) * PER;
  const uint4 zero = make_uint4(0, 0, 0, 0);
  constexpr int U = 4;
  int k = 0;
  for (; k + U * KS <= K; k += U * KS) {
    uint4 wf[U];
#pragma unroll
    for (int u = 0; u < U; ++u) wf[u] = nv ? ld16(wr + k + u * KS + kq) : zero;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint4 xf = rv[mt] ? ld16(xr[mt] + k + u * KS + kq) : zero;
        acc[mt] = mma16(xf, wf[u], acc[mt], T());
      }
  }
  for (; k < K; k += KS) {
    const int kk = k + kq;
    const bool kin = kk < K;
    const uint4 wf = (nv && kin) ? ld16(wr + kk) : zero;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint4 xf = (rv[mt] && kin) ? ld16(xr[mt] + kk) : zero;
      acc[mt] = mma16(xf, wf, acc[mt], T());
    }
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) tile[mt * 16 + (lane >> 4) * 4 + r][cl] = nv ? acc[mt][r] : -INFINITY;
  __syncthreads();

  // ---- per-row slab partials: (max, sum exp, top-k logits, top-k ids)
  const int rows_here = min(ROWS, p.M - zg * 64);
  for (int mr = wave; mr < rows_here; mr += 4) {
    const int row = zg * 64 + mr;
    float x = tile[mr][lane];
    const int id0 = blk * 64 + lane;
    const float mx = wave_max(x);
    const float s = wave_sum(x == -INFINITY ? 0.f : expf(x - mx));
    float* rec = a.lmpart + ((size_t)row * p.nblk + blk) * p.rec;
    if (lane == 0) { rec[0] = mx; rec[1] = s; }
    for (int r = 0; r < kk_; ++r) {
      float v = x;
      int id = (x == -INFINITY) ? INT_MAX : id0;
      wave_argmax(v, id);
      if (lane == 0) {
        rec[2 + r] = v;
        rec[2 + kk_ + r] = __int_as_float(id == INT_MAX ? -1 : id);
      }
      if (id == id0) x = -INFINITY;
    }
  }

  if (!arrive_last(a.cnt + GRID_CNT, p.nblk * p.zg)) return;

  // ---- phase 2a: per row, log-sum-exp and the global top-k
  for (int row = wave; row < p.M; row += 4) {
    const float* base = a.lmpart + (size_t)row * p.nblk * p.rec;
    float M = -INFINITY, S = 0.f;
    for (int bb = lane; bb < p.nblk; bb += 64) {
      const float mb = base[(size_t)bb * p.rec], sb = base[(size_t)bb * p.rec + 1];
      if (mb == -INFINITY) continue;
      const float nm = fmaxf(M, mb);
      S = (M == -INFINITY ? 0.f : S * expf(M - nm)) + sb * expf(mb - nm);
      M = nm;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float oM = __shfl_xor(M, o), oS = __shfl_xor(S, o);
      const float nm = fmaxf(M, oM);
      if (nm != -INFINITY) {
        S = (M == -INFINITY ? 0.f : S * expf(M - nm)) + (oM == -INFINITY ? 0.f : oS * expf(oM - nm));
        M = nm;
      }
    }
    M = __shfl(M, 0);
    S = __shfl(S, 0);
    const float lse = M + logf(S);

    for (int bb = lane; bb < p.nblk; bb += 64) heads[wave][bb] = 0;
    float* res = a.lmres + (size_t)row * 2 * kk_;
    for (int r = 0; r < kk_; ++r) {
      float v = -INFINITY;
      int id = INT_MAX;
      for (int bb = lane; bb < p.nblk; bb += 64) {
        const int h = heads[wave][bb];
        if (h >= kk_) continue;
        const float cv = base[(size_t)bb * p.rec + 2 + h];
        const int ci = __float_as_int(base[(size_t)bb * p.rec + 2 + kk_ + h]);
        if (ci < 0) continue;
        if (cv > v || (cv == v && ci < id)) { v = cv; id = ci; }
      }
      wave_argmax(v, id);
      if (id != INT_MAX && ((id >> 6) & 63) == lane) heads[wave][id >> 6]++;
      if (lane == 0) {
        res[r] = __int_as_float(id == INT_MAX ? 0 : id);
        res[kk_ + r] = v - lse;
      }
    }
  }
  __syncthreads();

  // ---- phase 2b: expansion and select per sequence
  const int pn = a.pool_n;
  for (int b = wave; b < a.B; b += 4) {
    eagle_pool_entry* pool = a.pool + (size_t)b * pn;
    eagle_frontier_node* fnew = a.frontier + ((size_t)level * a.B + b) * kk_;
    if (level == 1) {
      const float* res = a.lmres + (size_t)b * 2 * kk_;
      if (lane < kk_) {
        const int id = __float_as_int(res[lane]);
        const float lp = res[kk_ + lane];
        pool[lane] = eagle_pool_entry{lp, lp, id, -1, 1, -1};
        eagle_frontier_node nd;
        nd.token = id;
        nd.score = lp;
        nd.pool_idx = lane;
        nd.pslot = -1;
        for (int i = 0; i < EAGLE_MAX_DEPTH; ++i) nd.anc[i] = 0;
        nd.anc[0] = lane;
        fnew[lane] = nd;
      }
      continue;
    }
    const eagle_frontier_node* fprev = a.frontier + ((size_t)(level - 1) * a.B + b) * kk_;
    const int base = kk_ + (level - 2) * kk_ * kk_;
    const int nc = kk_ * kk_;
    float sc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int c = lane + 64 * t;
      sc[t] = -INFINITY;
      if (c < nc) {
        const int j = c / kk_, r = c % kk_;
        const float* res = a.lmres + ((size_t)b * kk_ + j) * 2 * kk_;
        const int id = __float_as_int(res[r]);
        const float lp = res[kk_ + r];
        const float s = fprev[j].score + lp;
        sc[t] = s;
        pool[base + c] = eagle_pool_entry{s, lp, id, fprev[j].pool_idx, level, j};
      }
    }
    for (int jn = 0; jn < kk_; ++jn) {
      float v = -INFINITY;
      int id = INT_MAX;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int c = lane + 64 * t;
        if (c < nc && (sc[t] > v || (sc[t] == v && c < id))) { v = sc[t]; id = c; }
      }
      wave_argmax(v, id);
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (lane + 64 * t == id) sc[t] = -INFINITY;
      if (id == INT_MAX) continue;  // fewer than k candidates (cannot happen with k*k >= k)
      const int j = id / kk_;
      const eagle_frontier_node& par = fprev[j];
      // the winner's pool record was written by this wave above
      const float* res = a.lmres + ((size_t)b * kk_ + j) * 2 * kk_;
      const int tok = __float_as_int(res[id % kk_]);
      if (lane < EAGLE_MAX_DEPTH) {
        int av = (lane < level - 1) ? par.anc[lane] : 0;
        if (lane == level - 1) av = jn;
        fnew[jn].anc[lane] = av;
      }
      if (lane == 0) {
        fnew[jn].token = tok;
        fnew[jn].score = v;
        fnew[jn].pool_idx = base + id;
        fnew[jn].pslot = j;
      }
    }
  }
}

template <typename T>
static hipError_t launch_lm_t(const RoundArgs& a, const LmPlan& p, int level, hipStream_t s) {
  const dim3 grid(p.nblk, 1, p.zg), block(BLOCK);
  switch (p.mt) {
    case 1: hipLaunchKernelGGL((k_lmhead<T, 1>), grid, block, 0, s, a, p, level); break;
    case 2: hipLaunchKernelGGL((k_lmhead<T, 2>), grid, block, 0, s, a, p, level); break;
    case 3: hipLaunchKernelGGL((k_lmhead<T, 3>), grid, block, 0, s, a, p, level); break;
    default: hipLaunchKernelGGL((k_lmhead<T, 4>), grid, block, 0, s, a, p, level); break;
  }
  return hipGetLastError();
}

hipError_t launch_lmhead(const RoundArgs& a, const LmPlan& p, int level, hipStream_t s) {
  return a.dtype == EAGLE_BF16 ? launch_lm_t<bf16_t>(a, p, level, s)
                               : launch_lm_t<float>(a, p, level, s);
}

}  // namespace eg

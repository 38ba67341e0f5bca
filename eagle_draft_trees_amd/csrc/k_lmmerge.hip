// Merge of the LM head's slab records into each row's softmax and top-k,
// then the EAGLE-2 expansion of one drafting level.
//
// [P1] "EAGLE 推测解码为什么比 Medusa 快？（含 EAGLE-2 动态草稿树）" §4.1: the draft
// distribution is softmax(LM_Head(f-hat)); §10.3: a node's value is the product
// of confidences on its root path, each level expands the best k nodes.
// [P3] zdszero.github.io spec_medusa_eagle, "在 SGLang 里": select_top_k_tokens
// multiplies the running score by this level's top-k probabilities and keeps
// the best topk of topk^2.  Scores are kept as sums of log-probabilities.
//
// k_lmmerge (one workgroup per sequence, one wave per row): combines the
// slabs' (max, sum) into a log-sum-exp, takes the row's top-k from the k slabs
// with the best heads and writes (id, log p = logit - lse).  Then level 1 puts
// the root's k children into the pool and frontier; for level L >= 2 the
// workgroup scores the k*k children (parent score + log p), appends all of
// them to the pool in (frontier slot, rank) order and keeps the best k by
// (score desc, pool index asc) as the next frontier; on a static tree the
// next frontier's slots are instead the template's (parent slot, rank) picks.
#include <float.h>
#include <limits.h>

#include <algorithm>

#include "eagle_internal.h"

namespace eg {

// Merge of the slab records, one workgroup per sequence and one wave per row.
// Each slab's list is sorted, so the row's top-k lies in the k slabs whose
// heads are the k largest (any other slab has k heads above all its entries):
// k argmax rounds over the slab heads pick those slabs, k more over their k*k
// entries give the row's top-k.  All rows of a sequence meet in the same
// workgroup, so the expansion that follows needs no cross-workgroup election.
// NH > 0: each lane keeps its (at most NH) slab heads in registers; NH == 0:
// in LDS (long vocabularies).
constexpr int MG_LDS = 64 * 1024;  // slab head keys of the rows in flight (NH == 0)

template <int NH>
__global__ void __launch_bounds__(SK_MAXW * WAVE) k_lmmerge(RoundArgs a, LmPlan p, int level) {
  extern __shared__ unsigned long long hk[];                  // NH == 0: [waves][nblk] slab head keys
  __shared__ float sres[EAGLE_MAX_TOPK * 2 * EAGLE_MAX_TOPK];  // per row: k id bits, k log p
  __shared__ int sanc[EAGLE_MAX_TOPK * EAGLE_MAX_DEPTH];
  __shared__ float psc[EAGLE_MAX_TOPK];
  __shared__ int ppi[EAGLE_MAX_TOPK];
  constexpr int NL = NH > 0 ? NH : 4;  // slabs per lane per load batch

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nwv = (int)(blockDim.x >> 6);
  const int b = blockIdx.x, kk_ = a.k, nblk = p.nblk, rec = p.rec;
  const int swidth = p.sk ? p.CT * 16 : 64;  // vocabulary columns per slab
  const int rows = level == 1 ? 1 : kk_;
  const int row0 = level == 1 ? b : b * kk_;

  // the parent frontier, needed by the expansion, is loaded first by wave 0
  // and stored to LDS once its rows are merged
  const eagle_frontier_node* fprev = a.frontier + ((size_t)(level - 1) * a.B + b) * kk_;
  const int nanc = kk_ * EAGLE_MAX_DEPTH;
  int ra[4] = {0, 0, 0, 0}, rpi = 0;
  float rsc = 0.f;
  if (level >= 2 && wave == 0) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int idx = lane + 64 * t;
      if (idx < nanc) ra[t] = fprev[idx / EAGLE_MAX_DEPTH].anc[idx % EAGLE_MAX_DEPTH];
    }
    if (lane < kk_) {
      rsc = fprev[lane].score;
      rpi = fprev[lane].pool_idx;
    }
  }

  unsigned long long* hkw = hk + (size_t)wave * nblk;
  for (int r = wave; r < rows; r += nwv) {
    const int row = row0 + r;
    const float* base = a.lmpart + (size_t)row * nblk * rec;
    // log-sum-exp over the slabs and the slab head keys; NL slabs per lane are
    // loaded before any is used
    float M = -INFINITY, S = 0.f;
    unsigned long long hkey[NH > 0 ? NH : 1];
    unsigned long long best = 0ull;
    for (int bb0 = 0; bb0 < nblk; bb0 += NL * WAVE) {
      float mv[NL], sv[NL], hv[NL];
      int hi[NL];
#pragma unroll
      for (int u = 0; u < NL; ++u) {
        const float* rc = base + min(bb0 + lane + WAVE * u, nblk - 1);  // field f at rc[f * nblk]
        mv[u] = rc[0];
        sv[u] = rc[nblk];
        hv[u] = rc[2 * nblk];
        hi[u] = __float_as_int(rc[(2 + kk_) * nblk]);
      }
#pragma unroll
      for (int u = 0; u < NL; ++u) {
        const int bb = bb0 + lane + WAVE * u;
        const bool in = bb < nblk;
        if (in && mv[u] != -INFINITY) {
          const float nm = fmaxf(M, mv[u]);
          S = (M == -INFINITY ? 0.f : S * expf(M - nm)) + sv[u] * expf(mv[u] - nm);
          M = nm;
        }
        const unsigned long long key = (in && hi[u] >= 0) ? argkey(hv[u], hi[u]) : 0ull;
        if (NH > 0) {
          hkey[u] = key;
        } else if (in) {
          hkw[bb] = key;
        }
        best = key > best ? key : best;
      }
      if (NH > 0) break;  // NH * WAVE >= nblk
    }
    const float Mw = wave_max_dpp(M);
    const float Sw = wave_sum_dpp(M == -INFINITY ? 0.f : S * expf(M - Mw));
    const float lse = Mw + logf(Sw);

    // the k slabs with the largest heads (a head's slab follows from its
    // token id): lane j ends up holding the j-th
    int mysel = 0, nsel = 0;
    for (; nsel < kk_; ++nsel) {
      const unsigned long long win = wave_max_key(best);
      if (win == 0ull) break;
      if (lane == nsel) mysel = argkey_id(win) / swidth;
      if (NH > 0) {
        best = 0ull;
#pragma unroll
        for (int u = 0; u < (NH > 0 ? NH : 1); ++u) {
          hkey[u] = hkey[u] == win ? 0ull : hkey[u];  // keys are unique: one owner
          best = hkey[u] > best ? hkey[u] : best;
        }
      } else if (best == win) {  // the owner's next head: the best of its slabs below win
        best = 0ull;
        for (int bb = lane; bb < nblk; bb += WAVE) {
          const unsigned long long kv = hkw[bb];
          best = (kv < win && kv > best) ? kv : best;
        }
      }
    }
    // their k*k entries, at most four per lane
    unsigned long long key[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int c = lane + WAVE * t, j = c / kk_, e = c - j * kk_;
      const int sl = __shfl(mysel, j < WAVE ? j : 0);
      const float* rc = base + sl;
      key[t] = 0ull;
      if (c < nsel * kk_) {
        const int id = __float_as_int(rc[(2 + kk_ + e) * nblk]);
        key[t] = id < 0 ? 0ull : argkey(rc[(2 + e) * nblk], id);
      }
    }
    unsigned long long mine = 0ull;  // lane q: the row's q-th entry
    for (int q = 0; q < kk_; ++q) {
      unsigned long long bk = 0ull;
#pragma unroll
      for (int t = 0; t < 4; ++t) bk = key[t] > bk ? key[t] : bk;
      const unsigned long long win = wave_max_key(bk);
#pragma unroll
      for (int t = 0; t < 4; ++t) key[t] = key[t] == win ? 0ull : key[t];
      if (lane == q) mine = win;
    }
    const int myid = mine ? argkey_id(mine) : 0;
    const float lp = (mine ? argkey_value(mine) : -INFINITY) - lse;
    if (lane < kk_) {
      float* res = a.lmres + (size_t)row * 2 * kk_;
      res[lane] = __int_as_float(myid);
      res[kk_ + lane] = lp;
      sres[r * 2 * kk_ + lane] = __int_as_float(myid);
      sres[r * 2 * kk_ + kk_ + lane] = lp;
    }
    if (level == 1 && lane < kk_) {  // the root's k children: pool and frontier
      eagle_pool_entry* pool = a.pool + (size_t)b * a.pool_n;
      eagle_frontier_node* fnew = a.frontier + ((size_t)1 * a.B + b) * kk_;
      pool[lane] = eagle_pool_entry{lp, lp, myid, -1, 1, -1};
      eagle_frontier_node nd;
      nd.token = myid;
      nd.score = lp;
      nd.pool_idx = lane;
      nd.pslot = -1;
      for (int i = 0; i < EAGLE_MAX_DEPTH; ++i) nd.anc[i] = 0;
      nd.anc[0] = lane;
      fnew[lane] = nd;
    }
  }
  if (level == 1) return;

  // ---- expansion and select (levels >= 2): wave 0 scores the k*k children
  // (parent score + log p), appends all of them to the pool in (frontier
  // slot, rank) order and keeps the best k by (score desc, pool index asc)
  if (wave == 0) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int idx = lane + 64 * t;
      if (idx < nanc) sanc[idx] = ra[t];
    }
    if (lane < kk_) {
      psc[lane] = rsc;
      ppi[lane] = rpi;
    }
  }
  __syncthreads();
  if (wave != 0) return;
  eagle_pool_entry* pool = a.pool + (size_t)b * a.pool_n;
  eagle_frontier_node* fnew = a.frontier + ((size_t)level * a.B + b) * kk_;
  const int pbase = kk_ + (level - 2) * kk_ * kk_;
  const int nc = kk_ * kk_;
  unsigned long long key[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int c = lane + 64 * t;
    key[t] = 0ull;
    if (c < nc) {
      const int j = c / kk_, r = c % kk_;
      const float* rr = sres + j * 2 * kk_;
      const int id = __float_as_int(rr[r]);
      const float lp = rr[kk_ + r];
      const float s = psc[j] + lp;
      key[t] = s == -INFINITY ? 0ull : argkey(s, c);
      pool[pbase + c] = eagle_pool_entry{s, lp, id, ppi[j], level, j};
    }
  }
  // lane jn: the jn-th kept child (candidate index cw = parent slot * k +
  // rank, score csc); -1 for a slot left as it was (fewer than k candidates,
  // impossible as k*k >= k)
  int cw = -1;
  float csc = 0.f;
  if (a.tmpl) {
    // static tree ([P1] §10.1): slot jn is the child of rank tmpl[.][jn][1]
    // of slot tmpl[.][jn][0], whatever its score (entries clamped into range)
    if (lane < kk_) {
      const int* tp = a.tmpl + ((size_t)(level - 1) * kk_ + lane) * 2;
      const int pj = clamp_slot(tp[0], kk_), rk = clamp_slot(tp[1], kk_);
      cw = pj * kk_ + rk;
      csc = psc[pj] + sres[pj * 2 * kk_ + kk_ + rk];  // the same sum as the candidate's key
    }
  } else {
    unsigned long long mine = 0ull;
    for (int jn = 0; jn < kk_; ++jn) {
      unsigned long long bk = 0ull;
#pragma unroll
      for (int t = 0; t < 4; ++t) bk = key[t] > bk ? key[t] : bk;
      const unsigned long long win = wave_max_key(bk);
#pragma unroll
      for (int t = 0; t < 4; ++t) key[t] = key[t] == win ? 0ull : key[t];
      if (lane == jn) mine = win;
    }
    cw = mine ? argkey_id(mine) : -1;
    csc = mine ? argkey_value(mine) : 0.f;
  }
  if (lane < kk_ && cw >= 0) {
    const int j = cw / kk_;
    fnew[lane].token = __float_as_int(sres[j * 2 * kk_ + (cw - j * kk_)]);
    fnew[lane].score = csc;
    fnew[lane].pool_idx = pbase + cw;
    fnew[lane].pslot = j;
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int idx = lane + 64 * t, jn = idx / EAGLE_MAX_DEPTH, i = idx % EAGLE_MAX_DEPTH;
    const int c = __shfl(cw, jn < WAVE ? jn : 0);
    if (idx < nanc && c >= 0) {
      const int j = c / kk_;
      fnew[jn].anc[i] = i < level - 1 ? sanc[j * EAGLE_MAX_DEPTH + i] : (i == level - 1 ? jn : 0);
    }
  }
}

hipError_t launch_lmmerge(const RoundArgs& a, const LmPlan& p, int level, hipStream_t s) {
  const int rows = level == 1 ? 1 : a.k;
  const int nseq = level == 1 ? p.M : p.M / a.k;
  if (p.nblk <= 4 * WAVE) {
    hipLaunchKernelGGL(k_lmmerge<4>, dim3(nseq), dim3(rows * WAVE), 0, s, a, p, level);
  } else if (p.nblk <= 8 * WAVE) {
    hipLaunchKernelGGL(k_lmmerge<8>, dim3(nseq), dim3(rows * WAVE), 0, s, a, p, level);
  } else {
    const int fit = MG_LDS / (p.nblk * (int)sizeof(unsigned long long));
    const int nwv = std::max(1, std::min(rows, fit));
    hipLaunchKernelGGL(k_lmmerge<0>, dim3(nseq), dim3(nwv * WAVE), (size_t)nwv * p.nblk * sizeof(unsigned long long),
                       s, a, p, level);
  }
  return hipGetLastError();
}

}  // namespace eg

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

#include "skinny_core.h"

namespace eg {

// Merge of the slab records, one workgroup per sequence and one wave per row.
// Each slab's list is sorted, so the row's top-k lies in the k slabs whose
// heads are the k largest (any other slab has k heads above all its entries):
// a wave top-k over the slab heads picks those slabs (k argmax rounds when
// the heads do not fit four per lane), another over their k*k entries gives
// the row's top-k.  All rows of a sequence meet in the same
// workgroup, so the expansion that follows needs no cross-workgroup election.
// NH > 0: each lane keeps its (at most NH) slab heads in registers; NH == 0:
// in LDS (long vocabularies).
constexpr int MG_LDS = 64 * 1024;  // slab head keys of the rows in flight (NH == 0)

// Publication of the next level's rows to the FC hand-over workgroups of the
// same launch: one 64-bit mailbox entry per next-level row, (parent row + 1)
// in the high word and (token + 1) in the low word, so that 0 means "not yet
// written".  Each entry is a single agent-scope atomic store (it is written
// through to where the hand-over workgroups, possibly on other XCDs, read it
// with agent-scope atomic loads), and it carries everything they need: the
// pool and frontier records are for the next launches, which the kernel
// boundary orders.  The entry goes out as soon as the row's child is chosen.
__device__ __forceinline__ unsigned long long* mailbox(const RoundArgs& a) {
  return (unsigned long long*)(a.cnt + CNT_MBOX);
}
__device__ __forceinline__ void post_row(const RoundArgs& a, int row, int prow, int tok) {
  const unsigned long long e = ((unsigned long long)(uint32_t)(prow + 1) << 32) | (uint32_t)(tok + 1);
  __hip_atomic_store(mailbox(a) + row, e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// mwv: waves that take rows (the block may hold more, which only pass the
// barriers); pub: publish for FC hand-over workgroups when done
template <int NH>
__device__ __forceinline__ void merge_body(const RoundArgs& a, const LmPlan& p, int level, int b, int mwv,
                                           unsigned long long* hk, bool pub) {
  __shared__ float sres[EAGLE_MAX_TOPK * 2 * EAGLE_MAX_TOPK];  // per row: k id bits, k log p
  __shared__ int sanc[EAGLE_MAX_TOPK * EAGLE_MAX_DEPTH];
  __shared__ float psc[EAGLE_MAX_TOPK];
  __shared__ int ppi[EAGLE_MAX_TOPK];
  __shared__ __attribute__((aligned(16))) unsigned long long s_tk[SK_MAXW][2 * WAVE];  // wave_topk scratch
  constexpr int NL = NH > 0 ? NH : 4;  // slabs per lane per load batch

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nwv = mwv;
  const int kk_ = a.k, nblk = p.nblk, rec = p.rec;
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
  for (int r = wave; r < rows && wave < nwv; r += nwv) {
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
    if constexpr (NH == 4) {
      const unsigned long long w = wave_topk<4>(hkey, kk_, s_tk[wave]);
      nsel = __popcll(__ballot(w != 0ull));
      mysel = w ? argkey_id(w) / swidth : 0;
    } else {
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
    const unsigned long long mine = wave_topk<4>(key, kk_, s_tk[wave]);  // lane q: the row's q-th entry
    const int myid = mine ? argkey_id(mine) : 0;
    const float lp = (mine ? argkey_value(mine) : -INFINITY) - lse;
    if (lane < kk_) {
      float* res = a.lmres + (size_t)row * 2 * kk_;
      res[lane] = __int_as_float(myid);
      res[kk_ + lane] = lp;
      sres[r * 2 * kk_ + lane] = __int_as_float(myid);
      sres[r * 2 * kk_ + kk_ + lane] = lp;
    }
    if (level == 1 && pub && lane < kk_) post_row(a, b * kk_ + lane, b, myid);
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
  if (level == 1) return;  // one row per sequence: its wave wrote the pool and frontier

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
    const unsigned long long mine = wave_topk<4>(key, kk_, s_tk[0]);
    cw = mine ? argkey_id(mine) : -1;
    csc = mine ? argkey_value(mine) : 0.f;
  }
  if (pub && lane < kk_) {  // (cw < 0 cannot happen: k*k >= k candidates)
    const int j = cw >= 0 ? cw / kk_ : 0;
    post_row(a, b * kk_ + lane, b * kk_ + j, cw >= 0 ? __float_as_int(sres[j * 2 * kk_ + (cw - j * kk_)]) : 0);
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

// FC hand-over ([P1] §4.1 input equation: the next level's row is [feature of
// the parent || embedding of the node's token]).  While the merge workgroups
// of the launch pick the next frontier (latency-bound: one workgroup per
// sequence), these workgroups stream the feature half of W_fc over all of this
// level's rows -- every one of them can be a parent -- and keep the products
// on chip.  Once every merge has published, each forms the next rows' x0 =
// W_fc[:, :d] h(parent) + tok_proj[token] + fc_b for its columns, so the next
// level starts at q/k/v.  The wait is bounded: a workgroup that gives up
// flags ERR_SYNC and proceeds (it never hangs).  The merge workgroups have
// the lowest block indices, so they are dispatched before any of these.
constexpr int HANDOVER_SPINS = 1 << 17;
template <typename T>
__device__ __forceinline__ void fc_handover(const RoundArgs& a, const SkPlan& fp, int level, int nseq, int wg,
                                            unsigned char* dyn) {
  constexpr int KS = El<T>::KSTEP;
  constexpr int BU = 4;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nwv = (int)(blockDim.x >> 6);  // == fp.CT * fp.KSW
  const int ct = wave % fp.CT, ks = wave / fp.CT;
  const int t = wg * fp.CT + ct;
  const int c = lane & 15, g = lane >> 4;
  const int K = a.d, nks = (K + KS - 1) / KS;
  const T* const wr[1] = {wtile_base<T>(a.fc_w, nks, t < fp.ntile ? t : 0, lane)};
  // this level's rows: the root features (level 1) or the level's features
  const T* xs = level == 1 ? (const T*)a.root_feat : (const T*)a.feat + (size_t)(level - 1) * a.B * a.k * K;
  const T* x0 = xs + (size_t)(c < fp.M ? c : 0) * K;  // rows past M repeat row 0 (unused)
  const int s0k = (int)((long)ks * nks / fp.KSW), s1k = (int)((long)(ks + 1) * nks / fp.KSW);
  const int nbu = ((nks + fp.KSW - 1) / fp.KSW + BU - 1) / BU;
  f32x4_t acc[1];
  sk_stream<T, 1, BU, false>(wr, x0, x0, K, K, s0k, s1k, nbu, dyn, acc);

  // K slices meet in LDS; the products [tile][row][column] stay there
  f32x4_t* red = (f32x4_t*)dyn;
  float* fs = (float*)(dyn + (size_t)nwv * WAVE * sizeof(f32x4_t));
  red[wave * WAVE + lane] = acc[0];
  __syncthreads();
  if (ks == 0) {
    f32x4_t v = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < fp.KSW; ++s) v += red[(s * fp.CT + ct) * WAVE + lane];
#pragma unroll
    for (int r = 0; r < 4; ++r) fs[(ct * 16 + 4 * g + r) * 16 + c] = v[r];
  }

  // wait until the mailbox holds every next-level row (wave 0: lane r polls
  // entry r), then take the rows' parent and token from it
  __shared__ int s_tok[16], s_prow[16];
  const int R = a.B * a.k;  // the next level's rows (at most 16)
  if (wave == 0) {
    unsigned long long e = 0ull;
    for (int spins = 0;; ++spins) {
      if (lane < R) e = __hip_atomic_load(mailbox(a) + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (__ballot(lane < R && e == 0ull) == 0ull) break;
      if (spins > HANDOVER_SPINS) {
        if (lane == 0) atomicOr(a.err, ERR_SYNC);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    if (lane < R) {
      const int b = lane / a.k;
      const int prow = (int)(uint32_t)(e >> 32) - 1, tok = (int)(uint32_t)e - 1;
      s_tok[lane] = clamp_tok(tok, a.V, a.err);
      s_prow[lane] = level == 1 ? b : b * a.k + clamp_slot(prow - b * a.k, a.k);
    }
  }
  __syncthreads();
  // every hand-over workgroup has read the mailbox once `seen` counts them
  // all: the last one clears the entries and the count for the next launch
  if (tid == 0) {
    const int prev = __hip_atomic_fetch_add(a.cnt + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == fp.nwg - 1) {
      for (int r = 0; r < R; ++r) __hip_atomic_store(mailbox(a) + r, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.cnt + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  const int W = fp.CT * 16;
  for (int idx = tid; idx < R * W; idx += (int)blockDim.x) {
    const int row = idx / W, cc = idx - row * W, tl = cc >> 4, col = cc & 15;
    const int n = (wg * fp.CT + tl) * 16 + col;
    if (n >= a.d) continue;
    const float x = fs[(tl * 16 + s_prow[row]) * 16 + col] + a.tok_proj[(size_t)s_tok[row] * a.d + n] +
                    El<T>::ld((const T*)a.fc_b, n);
    st_x0<T>(a, (size_t)row * a.d + n, x);
  }
}

// merge workgroups (blocks 0..nseq-1) and, with FUSE, the FC hand-over
// workgroups of the next level after them
template <int NH, typename T, bool FUSE>
__global__ void __launch_bounds__(SK_MAXW * WAVE) k_lmmerge(RoundArgs a, LmPlan p, SkPlan fp, int level, int nseq,
                                                           int mwv) {
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];
  const int blk = blockIdx.x;
  if (!FUSE || blk < nseq) {
    merge_body<NH>(a, p, level, blk, mwv, (unsigned long long*)dyn, FUSE);
    return;
  }
  fc_handover<T>(a, fp, level, nseq, blk - nseq, dyn);
}

// The merge's launch.  fp.nwg > 0: the FC hand-over of the next level rides
// along (fp is the FC plan over this level's rows with CT * KSW waves, the
// block size of the launch).
template <int NH, typename T>
static void launch_merge_t(const RoundArgs& a, const LmPlan& p, const SkPlan& fp, int level, int nseq, int mwv,
                           size_t lds, hipStream_t s) {
  const int rows = level == 1 ? 1 : a.k;
  if (fp.nwg > 0) {
    const int nwv = fp.CT * fp.KSW;
    const size_t fl = (size_t)nwv * WAVE * sizeof(f32x4_t) + (size_t)fp.CT * 256 * sizeof(float);
    hipLaunchKernelGGL((k_lmmerge<NH, T, true>), dim3(nseq + fp.nwg), dim3(nwv * WAVE), lds > fl ? lds : fl, s, a,
                       p, fp, level, nseq, NH == 0 ? mwv : nwv);
  } else {
    const int nwv = NH == 0 ? mwv : rows;
    hipLaunchKernelGGL((k_lmmerge<NH, T, false>), dim3(nseq), dim3(nwv * WAVE), lds, s, a, p, fp, level, nseq, nwv);
  }
}

template <typename T>
static hipError_t launch_merge_dt(const RoundArgs& a, const LmPlan& p, const SkPlan& fp, int level, hipStream_t s) {
  const int rows = level == 1 ? 1 : a.k;
  const int nseq = level == 1 ? p.M : p.M / a.k;
  if (p.nblk <= 4 * WAVE) {
    launch_merge_t<4, T>(a, p, fp, level, nseq, rows, 0, s);
  } else if (p.nblk <= 8 * WAVE) {
    launch_merge_t<8, T>(a, p, fp, level, nseq, rows, 0, s);
  } else {
    const int fit = MG_LDS / (p.nblk * (int)sizeof(unsigned long long));
    const int nwv = std::max(1, std::min(rows, fit));
    launch_merge_t<0, T>(a, p, fp, level, nseq, nwv, (size_t)nwv * p.nblk * sizeof(unsigned long long), s);
  }
  return hipGetLastError();
}

hipError_t launch_lmmerge(const RoundArgs& a, const LmPlan& p, int level, hipStream_t s, const SkPlan* handover) {
  SkPlan none{};
  const SkPlan& fp = handover ? *handover : none;
  return a.dtype == EAGLE_BF16 ? launch_merge_dt<bf16_t>(a, p, fp, level, s) : launch_merge_dt<float>(a, p, fp, level, s);
}

}  // namespace eg

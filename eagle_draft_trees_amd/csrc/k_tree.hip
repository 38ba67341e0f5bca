// Rerank + tree build, greedy verify walk, workspace zero fill.
#include "eagle_internal.h"

namespace eg {

constexpr int MAX_POOL = EAGLE_MAX_TOPK + (EAGLE_MAX_DEPTH - 1) * EAGLE_MAX_TOPK * EAGLE_MAX_TOPK;
constexpr int MAX_POOL_P2 = 4096;  // next power of two
static_assert(MAX_POOL <= MAX_POOL_P2, "pool");

// Rerank and build, one workgroup per sequence.
// [P1] "EAGLE 推测解码为什么比 Medusa 快？（含 EAGLE-2 动态草稿树）" §10.3: after the
// last level, the m best nodes by value over all nodes are flattened for
// verification; ties prefer the shallower node.  [P3] zdszero.github.io
// spec_medusa_eagle, "在 SGLang 里": organize_draft_results keeps the best
// num_draft_tokens-1, build_tree_kernel_efficient adds the root and builds the
// tree and mask.  [P4] "投机解码：从eagle1到dflash" EAGLE-2 diagram: flat order
// x1, x2, x3, x1a, x1b, ... ; 0/1 ancestor mask; per-level positions.
//
// Selection: one 64-bit key per pool entry = (score desc, depth asc, index asc)
// as an unsigned integer; a bitonic sort in LDS orders them and the first m-1
// are kept.  Flattening: depth by depth, each kept node's rank among its depth
// by (parent's flat index, pool index).
__global__ void __launch_bounds__(BLOCK) k_rerank(RoundArgs a, int32_t* tokens, int32_t* parents,
                                                  int32_t* depth, int32_t* positions, uint8_t* mask,
                                                  float* logscore) {
  __shared__ unsigned long long key[MAX_POOL_P2];
  __shared__ short flat_of[MAX_POOL];
  __shared__ int sel[EAGLE_MAX_TREE];
  __shared__ unsigned sk2[EAGLE_MAX_TREE];
  __shared__ int sdep[EAGLE_MAX_TREE];
  __shared__ int fpar[EAGLE_MAX_TREE], fdep[EAGLE_MAX_TREE];
  __shared__ unsigned long long fanc[EAGLE_MAX_TREE];

  const int tid = threadIdx.x, b = blockIdx.x;
  const int n = a.pool_n, m = a.m, ns = m - 1;
  const eagle_pool_entry* pool = a.pool + (size_t)b * n;
  int np = 1;
  while (np < n) np <<= 1;  // <= MAX_POOL_P2

  for (int e = tid; e < np; e += BLOCK) {
    unsigned long long kv = 0ull;  // padding sorts last
    if (e < n) {
      const eagle_pool_entry pe = pool[e];
      uint32_t u = __float_as_uint(pe.score);
      u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // order-preserving for floats
      kv = ((unsigned long long)u << 32) | ((unsigned long long)(255 - (pe.depth & 255)) << 24) |
           (unsigned long long)(0xFFFFFF - e);
      flat_of[e] = -1;
    }
    key[e] = kv;
  }
  if (tid < EAGLE_MAX_TREE) sk2[tid] = 0xFFFFFFFFu;
  __syncthreads();
  // bitonic sort, best key first
  for (int size = 2; size <= np; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < (np >> 1); i += BLOCK) {
        const int lo = 2 * stride * (i / stride) + (i % stride), hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const unsigned long long x = key[lo], y = key[hi];
        if ((x < y) == desc) { key[lo] = y; key[hi] = x; }
      }
      __syncthreads();
    }
  }
  if (tid < ns) sel[tid] = 0xFFFFFF - (int)(key[tid] & 0xFFFFFFull);
  __syncthreads();

  // pool records are device data: keep depth in 1..D and parents inside the pool
  int e = -1, dep = 0, par = -1;
  if (tid < ns) {
    e = sel[tid];
    dep = min(max(pool[e].depth, 1), a.D);
    par = pool[e].parent;
    if (par < 0 || par >= n) par = -1;
    sdep[tid] = dep;
  }
  if (tid < EAGLE_MAX_TREE) {
    fpar[tid] = 0;
    fdep[tid] = 0;
    if (tid >= ns) sdep[tid] = 0;
  }
  __syncthreads();
  // flatten depth by depth: rank among the same depth by (parent's flat index, pool index)
  int base = 1;
  for (int dd = 1; dd <= a.D; ++dd) {
    const bool mine = tid < ns && dep == dd;
    unsigned k2 = 0xFFFFFFFFu;
    if (mine) {
      k2 = ((unsigned)(par < 0 ? 0 : (int)flat_of[par] & 0xFFFF) << 16) | (unsigned)e;
      sk2[tid] = k2;
    }
    __syncthreads();
    int cnt = 0, rank = 0;
#pragma unroll
    for (int j = 0; j < EAGLE_MAX_TREE; ++j) {
      cnt += sdep[j] == dd ? 1 : 0;
      rank += sk2[j] < k2 ? 1 : 0;
    }
    if (mine) flat_of[e] = (short)(base + rank);
    base += cnt;
    __syncthreads();
    if (mine) sk2[tid] = 0xFFFFFFFFu;
  }
  __syncthreads();

  int P = clamp_prefix(a.prefix_len[b], a);
  int32_t* tk = tokens + (size_t)b * m;
  int32_t* pa = parents + (size_t)b * m;
  if (tid == 0) {
    tk[0] = clamp_tok(a.root_token[b], a.V, a.err);
    pa[0] = -1;
    if (depth) depth[(size_t)b * m] = 0;
    if (positions) positions[(size_t)b * m] = P - 1;
    if (logscore) logscore[(size_t)b * m] = 0.f;
    fpar[0] = -1;
    fdep[0] = 0;
    fanc[0] = 1ull;
  }
  if (tid < ns && flat_of[e] >= 1 && flat_of[e] < m) {
    const int f = flat_of[e];
    const int pf = (par < 0 || flat_of[par] < 0) ? 0 : flat_of[par];
    tk[f] = pool[e].token;
    pa[f] = pf;
    if (depth) depth[(size_t)b * m + f] = dep;
    if (positions) positions[(size_t)b * m + f] = P - 1 + dep;
    if (logscore) logscore[(size_t)b * m + f] = pool[e].score;
    fpar[f] = pf;
    fdep[f] = dep;
  }
  __syncthreads();
  for (int dd = 1; dd <= a.D; ++dd) {
    if (tid < m && tid > 0 && fdep[tid] == dd && fpar[tid] < tid)
      fanc[tid] = fanc[fpar[tid]] | (1ull << tid);
    __syncthreads();
  }
  if (mask) {
    uint8_t* mk = mask + (size_t)b * m * m;
    for (int idx = tid; idx < m * m; idx += BLOCK) mk[idx] = (uint8_t)((fanc[idx / m] >> (idx % m)) & 1ull);
  }
}

// The kk-th largest of the wave's unique 64-bit keys (N per lane, 0 = empty;
// 1 <= kk <= their number): exactly kk keys are >= the result.  Found bit by
// bit, most significant first: the high word is the largest h with at least
// kk high words >= h, each step counting N ballots on the scalar unit; the low
// word only matters under ties of the high word, and is then the smallest low
// word among the tied keys (all of them taken) or found the same way.
template <int N>
__device__ __forceinline__ unsigned long long wave_kth_key(const unsigned long long (&key)[N], int kk) {
  uint32_t hi[N], lo[N];
#pragma unroll
  for (int j = 0; j < N; ++j) {
    hi[j] = (uint32_t)(key[j] >> 32);
    lo[j] = (uint32_t)key[j];
  }
  uint32_t hp = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t t = hp | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < N; ++j) cnt += __popcll(__ballot(hi[j] >= t));
    if (cnt >= kk) hp = t;
  }
  int cgt = 0, ceq = 0;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    cgt += __popcll(__ballot(hi[j] > hp));
    ceq += __popcll(__ballot(hi[j] == hp && key[j] != 0ull));
  }
  const int need = kk - cgt;  // 1..ceq of the keys with high word hp
  uint32_t lp = 0u;
  if (need == ceq) {
    lp = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < N; ++j) lp = min(lp, (hi[j] == hp && key[j] != 0ull) ? lo[j] : 0xFFFFFFFFu);
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) lp = min(lp, (uint32_t)__shfl_xor((int)lp, o));
  } else {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t t = lp | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int j = 0; j < N; ++j) cnt += __popcll(__ballot(hi[j] == hp && lo[j] >= t));
      if (cnt >= need) lp = t;
    }
  }
  return ((unsigned long long)hp << 32) | lp;
}

// The same rerank and build in one wave per sequence, for pools of at most
// 64*KPL entries: the pool is copied to LDS once, the (m-1)-th largest key is
// found by a bitwise search over the keys in registers (wave_kth_key), the
// keys at or above it are the kept nodes (their order does not matter: the
// flatten orders them), and one lane per kept node does the flatten (depth by
// depth, its rank among the kept nodes of its depth by (parent's flat index,
// pool index)) and its mask row.  Results are those of k_rerank.
template <int KPL>
__global__ void __launch_bounds__(WAVE) k_rerank_wave(RoundArgs a, int32_t* tokens, int32_t* parents,
                                                      int32_t* depth, int32_t* positions, uint8_t* mask,
                                                      float* logscore) {
  constexpr int NMAX = 64 * KPL;
  constexpr int QPL = NMAX * 3 / 64;  // 8-byte pieces of the pool per lane (3 per entry)
  __shared__ eagle_pool_entry sp[NMAX];
  __shared__ short flat_of[NMAX];
  __shared__ int sel[EAGLE_MAX_TREE];
  __shared__ __attribute__((aligned(16))) unsigned sk2[WAVE];
  __shared__ int fpar[EAGLE_MAX_TREE], fdep[EAGLE_MAX_TREE];
  __shared__ unsigned long long fanc[EAGLE_MAX_TREE];

  const int lane = threadIdx.x, b = blockIdx.x;
  const int n = a.pool_n, m = a.m, ns = m - 1;
  {  // the pool into LDS, every load issued before any store
    const unsigned long long* src = (const unsigned long long*)(a.pool + (size_t)b * n);
    unsigned long long* dst = (unsigned long long*)sp;
    const int nq = n * 3;
    unsigned long long v[QPL];
#pragma unroll
    for (int u = 0; u < QPL; ++u) v[u] = src[min(lane + WAVE * u, nq - 1)];
#pragma unroll
    for (int u = 0; u < QPL; ++u)
      if (lane + WAVE * u < nq) dst[lane + WAVE * u] = v[u];
    for (int e = lane; e < n; e += WAVE) flat_of[e] = -1;
  }
  __syncthreads();

  // keys (score desc, depth asc, index asc) as unsigned integers; padding is 0
  unsigned long long key[KPL];
  {
    float sc[KPL];
    int dp[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) {  // every LDS read in flight before any is used
      const int e = min(lane * KPL + j, n - 1);
      sc[j] = sp[e].score;
      dp[j] = sp[e].depth;
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int e = lane * KPL + j;
      uint32_t u = __float_as_uint(sc[j]);
      u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
      key[j] = e < n ? ((unsigned long long)u << 32) | ((unsigned long long)(255 - (dp[j] & 255)) << 24) |
                           (unsigned long long)(0xFFFFFF - e)
                     : 0ull;
    }
  }
  {  // the kept set: the ns largest keys (ns <= n), packed into sel[] in any order
    const unsigned long long tau = wave_kth_key<KPL>(key, ns);
    const unsigned long long below = (1ull << lane) - 1ull;
    int base = 0;
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const bool in = key[j] != 0ull && key[j] >= tau;
      const unsigned long long msk = __ballot(in);
      const int pos = base + __popcll(msk & below);
      if (in && pos < ns) sel[pos] = 0xFFFFFF - (int)(key[j] & 0xFFFFFFull);  // (keys are unique: pos < ns)
      base += __popcll(msk);
    }
  }
  __syncthreads();

  // pool records are device data: keep depth in 1..D and parents inside the pool
  const bool act = lane < ns;
  int e = 0, dep = 0, par = -1;
  if (act) {
    e = sel[lane];
    dep = min(max(sp[e].depth, 1), a.D);
    par = sp[e].parent;
    if (par < 0 || par >= n) par = -1;
  }
  int base = 1;
  for (int dd = 1; dd <= a.D; ++dd) {
    const bool mine = act && dep == dd;
    const unsigned k2 =
        mine ? (((unsigned)(par < 0 ? 0 : (int)flat_of[par] & 0xFFFF) << 16) | (unsigned)e) : 0xFFFFFFFFu;
    sk2[lane] = k2;
    __syncthreads();
    int rank = 0;
    uint4 qv[WAVE / 4];  // all sixteen broadcast reads in flight before any is used
#pragma unroll
    for (int u = 0; u < WAVE / 4; ++u) qv[u] = *(const uint4*)&sk2[4 * u];
    asm volatile("" ::: "memory");
#pragma unroll
    for (int u = 0; u < WAVE / 4; ++u)
      rank += (qv[u].x < k2 ? 1 : 0) + (qv[u].y < k2 ? 1 : 0) + (qv[u].z < k2 ? 1 : 0) + (qv[u].w < k2 ? 1 : 0);
    if (mine) flat_of[e] = (short)(base + rank);
    base += __popcll(__ballot(mine));
    __syncthreads();
  }

  const int P = clamp_prefix(a.prefix_len[b], a);
  int32_t* tk = tokens + (size_t)b * m;
  int32_t* pa = parents + (size_t)b * m;
  fpar[lane] = lane == 0 ? -1 : 0;
  fdep[lane] = 0;
  if (lane == 0) {
    tk[0] = clamp_tok(a.root_token[b], a.V, a.err);
    pa[0] = -1;
    if (depth) depth[(size_t)b * m] = 0;
    if (positions) positions[(size_t)b * m] = P - 1;
    if (logscore) logscore[(size_t)b * m] = 0.f;
  }
  __syncthreads();
  if (act && flat_of[e] >= 1 && flat_of[e] < m) {
    const int f = flat_of[e];
    const int pf = (par < 0 || flat_of[par] < 0) ? 0 : flat_of[par];
    tk[f] = sp[e].token;
    pa[f] = pf;
    if (depth) depth[(size_t)b * m + f] = dep;
    if (positions) positions[(size_t)b * m + f] = P - 1 + dep;
    if (logscore) logscore[(size_t)b * m + f] = sp[e].score;
    fpar[f] = pf;
    fdep[f] = dep;
  }
  // ancestor bitmasks, depth by depth (a parent precedes its children); lane f
  // holds flat node f's
  unsigned long long anc = lane == 0 ? 1ull : 0ull;
  fanc[lane] = anc;
  __syncthreads();
  const int myd = fdep[lane], myp = fpar[lane];
  for (int dd = 1; dd <= a.D; ++dd) {
    if (lane > 0 && lane < m && myd == dd && myp < lane) {
      anc = fanc[myp] | (1ull << lane);
      fanc[lane] = anc;
    }
    __syncthreads();
  }
  if (mask && lane < m) {  // lane f writes mask row f
    uint8_t* row = mask + ((size_t)b * m + lane) * m;
    if ((m & 3) == 0 && ((uintptr_t)mask & 3) == 0) {
      for (int c = 0; c < m; c += 4) {
        const unsigned x = (unsigned)(anc >> c) & 0xFu;
        ((unsigned*)row)[c >> 2] = (x & 1u) | ((x & 2u) << 7) | ((x & 4u) << 14) | ((x & 8u) << 21);
      }
    } else {
      for (int c = 0; c < m; ++c) row[c] = (uint8_t)((anc >> c) & 1ull);
    }
  }
}

// inclusive prefix sum over the wave's lanes (a fixed order)
__device__ __forceinline__ float wave_incl_scan(float v, int lane) {
#pragma unroll
  for (int o = 1; o < WAVE; o <<= 1) {
    const float t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Static tree build ([P1] §10.1: EAGLE-1 and Medusa draft on a tree of fixed
// shape): the tree is every template node, read straight from the frontier
// records the levels wrote.  Node (depth L, slot j) has flat index
// 1 + (L-1)*k + j; its parent is the root (L = 1) or slot pslot of depth L-1,
// and its ancestors are the slots its record lists for depths 1..L.  One wave
// per sequence, lane f builds flat node f (the first m nodes).
__global__ void __launch_bounds__(WAVE) k_static_build(RoundArgs a, int32_t* tokens, int32_t* parents,
                                                       int32_t* depth, int32_t* positions, uint8_t* mask,
                                                       float* logscore) {
  const int b = blockIdx.x, f = threadIdx.x, k = a.k, m = a.m;
  if (f >= m) return;
  const int P = clamp_prefix(a.prefix_len[b], a);
  int tok, par, dep;
  float sc;
  unsigned long long anc = 1ull;  // the root
  if (f == 0) {
    tok = clamp_tok(a.root_token[b], a.V, a.err);
    par = -1;
    dep = 0;
    sc = 0.f;
  } else {
    dep = 1 + (f - 1) / k;
    const int j = (f - 1) - (dep - 1) * k;
    const eagle_frontier_node& nd = a.frontier[((size_t)dep * a.B + b) * k + j];
    tok = nd.token;
    sc = nd.score;
    par = dep == 1 ? 0 : 1 + (dep - 2) * k + clamp_slot(nd.pslot, k);
    for (int e = 1; e <= dep; ++e) {  // ancestors at depths 1..dep, then self
      const int af = 1 + (e - 1) * k + clamp_slot(nd.anc[e - 1], k);
      if (af < m) anc |= 1ull << af;
    }
    anc |= 1ull << f;
  }
  tokens[(size_t)b * m + f] = tok;
  parents[(size_t)b * m + f] = par;
  if (depth) depth[(size_t)b * m + f] = dep;
  if (positions) positions[(size_t)b * m + f] = P - 1 + dep;
  if (logscore) logscore[(size_t)b * m + f] = sc;
  if (mask) {
    uint8_t* row = mask + ((size_t)b * m + f) * m;
    for (int c = 0; c < m; ++c) row[c] = (uint8_t)((anc >> c) & 1ull);
  }
}

hipError_t launch_static_build(const RoundArgs& a, int32_t* tokens, int32_t* parents, int32_t* depth,
                               int32_t* positions, uint8_t* mask, float* logscore, hipStream_t s) {
  hipLaunchKernelGGL(k_static_build, dim3(a.B), dim3(WAVE), 0, s, a, tokens, parents, depth, positions, mask,
                     logscore);
  return hipGetLastError();
}

// Greedy verify, one workgroup (16 waves) per sequence.  [P4] EAGLE-2 diagram:
// accept the longest consistent path from the root and back off to the last
// accepted node; the target's choice there is the bonus token.
__global__ void __launch_bounds__(1024) k_verify(int m, int D, int V, const float* tl,
                                                 const int32_t* tokens, const int32_t* parents,
                                                 int32_t* alen, int32_t* apath, int32_t* bonus) {
  __shared__ float wv[16];
  __shared__ int wi[16];
  __shared__ int s_best, s_child;
  __shared__ int path[EAGLE_MAX_DEPTH + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, b = blockIdx.x;
  int node = 0, len = 1;
  if (tid == 0) path[0] = 0;
  for (int step = 0; step <= D; ++step) {
    const float* row = tl + ((size_t)b * m + node) * V;
    float v = -INFINITY;
    int id = INT_MAX;
    for (int i0 = tid; i0 < V; i0 += 1024 * 8) {
      float x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i0 + u * 1024;
        x[u] = i < V ? row[i] : -INFINITY;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)  // this thread's indices increase: the first max wins
        if (x[u] > v) { v = x[u]; id = i0 + u * 1024; }
    }
    wave_argmax(v, id);
    if (lane == 0) { wv[wave] = v; wi[wave] = id; }
    if (tid == 0) s_child = -1;
    __syncthreads();
    if (tid == 0) {
      float bv = wv[0];
      int bi = wi[0];
      for (int w = 1; w < 16; ++w)
        if (wv[w] > bv || (wv[w] == bv && wi[w] < bi)) { bv = wv[w]; bi = wi[w]; }
      s_best = bi == INT_MAX ? 0 : bi;
    }
    __syncthreads();
    const int best = s_best;
    if (tid < m && parents[(size_t)b * m + tid] == node && tid != node &&
        tokens[(size_t)b * m + tid] == best)
      s_child = tid;
    __syncthreads();
    const int c = s_child;
    if (c < 0 || len > D) {
      if (tid == 0) {
        alen[b] = len;
        bonus[b] = best;
      }
      break;
    }
    if (tid == 0) path[len] = c;
    node = c;
    ++len;
    __syncthreads();
  }
  __syncthreads();
  if (tid <= D) apath[(size_t)b * (D + 1) + tid] = tid < len ? path[tid] : -1;
}

// Relaxed acceptance walk ([P2] closing notes on SGLang's verification: the
// target's probabilities and a probability threshold decide acceptance, and
// one rejection-sampling draw at the level where every candidate fails gives
// the bonus).  At node x, p = softmax(logits[x] / T); x's children are tried
// in flat order and the walk descends to the first with p(c) >= threshold.
// At the stop, the bonus is drawn by inverse CDF (smallest id whose
// cumulative residual mass exceeds u * total) from p with x's children
// removed; from p itself if they held all of its mass.
//
// Two launches.  k_relaxed_stats spreads the softmax statistics of every
// tree row over the chip: workgroup (segment s, row) reduces ids
// [s*SEGV, (s+1)*SEGV) of the row to (max, sum of exp(z - max)), z = l / T,
// reading 256 consecutive ids per wave instruction pair.  k_verify_relaxed
// (one workgroup per sequence) then walks: a visited node's statistics are
// its 16 segment pairs combined in segment order, and the children (flat
// slots 0..m-1, i.e. wave 0) are tested with one ballot.  At the stop, each
// segment's residual mass is its mass minus the removed children that fall
// in it; the segment holding u * total is found in segment order and only
// that segment (about V/16 ids) is scanned in id order: contiguous chunks
// per thread, a wave-wide scan, the waves chained in order, every bound the
// same sum wherever it is formed.
constexpr int RS_SEG = 16;     // segments per row
constexpr int RS_T = 256;      // threads of a statistics workgroup
constexpr int RS_U = 8;        // loads in flight per thread
constexpr int RV_T = 1024;
constexpr int RV_W = RV_T / WAVE;

// blockIdx.z picks the array: 0 = (tl, stats), 1 = (tl2, stats2)
__global__ void __launch_bounds__(RS_T) k_relaxed_stats(int V, const float* tl, float2* stats, const float* tl2,
                                                        float2* stats2, float temperature) {
#pragma clang fp contract(off)
  __shared__ float s_m[RS_T / WAVE], s_s[RS_T / WAVE];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sg = blockIdx.x, row = blockIdx.y;
  const int SEGV = (V + RS_SEG - 1) / RS_SEG;
  const int a0 = min(V, sg * SEGV), a1 = min(V, a0 + SEGV);
  const float* r = (blockIdx.z == 0 ? tl : tl2) + (size_t)row * V;
  float2* out = blockIdx.z == 0 ? stats : stats2;
  const float invT = 1.0f / temperature;
  float mx = -INFINITY, sm = 0.f;
  for (int x0 = a0 + tid; x0 < a1; x0 += RS_T * RS_U) {
    float z[RS_U];
#pragma unroll
    for (int q = 0; q < RS_U; ++q) {  // unconditional loads from clamped ids: all in flight at once
      const int x = x0 + q * RS_T;
      const float l = r[min(x, a1 - 1)];
      z[q] = x < a1 ? l * invT : -INFINITY;
    }
    float bm = mx;
#pragma unroll
    for (int q = 0; q < RS_U; ++q) bm = z[q] > bm ? z[q] : bm;  // -inf and NaN never win
    if (bm > mx) {
      sm = mx == -INFINITY ? 0.f : sm * expf(mx - bm);
      mx = bm;
    }
#pragma unroll
    for (int q = 0; q < RS_U; ++q)
      if (z[q] > -INFINITY) sm += expf(z[q] - mx);
  }
  const float wm = wave_max_dpp(mx);
  const float ws = wave_sum_dpp(mx == -INFINITY ? 0.f : sm * expf(mx - wm));
  if (lane == 0) {
    s_m[wave] = wm;
    s_s[wave] = ws;
  }
  __syncthreads();
  if (tid == 0) {
    float M = s_m[0];
    for (int w = 1; w < RS_T / WAVE; ++w) M = fmaxf(M, s_m[w]);
    float S = 0.f;
    for (int w = 0; w < RS_T / WAVE; ++w) S += s_m[w] == -INFINITY ? 0.f : s_s[w] * expf(s_m[w] - M);
    out[(size_t)row * RS_SEG + sg] = make_float2(M, S);
  }
}

// TOPK: strict rejection sampling of deterministic candidates (the draft's
// top-k children are a fixed list, not draws from q): each child is a
// point-mass proposal, accepted iff u_c * (mass left) <= p(t_c), i.e. u_c <=
// the residual's probability of t_c; a rejected token leaves the residual
// (removed and renormalised).  The bonus is the same residual draw as the
// relaxed walk's.  uniforms [B][m+1]: u[c] decides flat node c, u[m] draws.
__device__ __forceinline__ float clamp_u(float u) { return u >= 0.f ? (u < 1.f ? u : 0.99999994f) : 0.f; }

template <bool TOPK>
__global__ void __launch_bounds__(RV_T) k_verify_relaxed(int m, int D, int V, const float* tl,
                                                         const int32_t* tokens, const int32_t* parents,
                                                         float temperature, float thr, const float* uniforms,
                                                         const float2* stats, int32_t* alen, int32_t* apath,
                                                         int32_t* bonus) {
  // no fused multiply-adds: z = l / T and each exp(z - M) are formed the same
  // way here as in the statistics kernel
#pragma clang fp contract(off)
  __shared__ float s_seg[RS_SEG], s_res[RS_SEG];
  __shared__ float s_ws[RV_W];
  __shared__ float s_M, s_local;
  __shared__ int s_kid[EAGLE_MAX_TREE], s_kseg[EAGLE_MAX_TREE];
  __shared__ float s_ke[EAGLE_MAX_TREE];
  __shared__ int s_nk, s_len, s_node, s_pick, s_seg_pick, s_excl, s_last;
  __shared__ int path[EAGLE_MAX_DEPTH + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, b = blockIdx.x;
  const int SEGV = (V + RS_SEG - 1) / RS_SEG;
  const float invT = 1.0f / temperature;
  const float u = clamp_u(TOPK ? uniforms[(size_t)b * (m + 1) + m] : uniforms[b]);  // into [0, 1); NaN -> 0

  // ---- the walk, in wave 0 alone: lane j holds flat slot j (m <= 64).  Per
  // visited node one round trip: lanes 0..15 load its segment statistics and
  // every child lane loads its token's logit, together; M and S are wave
  // reductions in a fixed order; one ballot gives the first passing child.
  if (wave == 0) {
    const bool inm = lane < m;
    const int par = inm ? parents[(size_t)b * m + lane] : -2;
    const int tok = inm ? tokens[(size_t)b * m + lane] : -1;
    const bool inr = tok >= 0 && tok < V;
    const float uk = (TOPK && inm) ? clamp_u(uniforms[(size_t)b * (m + 1) + lane]) : 0.f;
    int node = 0, len = 1;
    if (lane == 0) path[0] = 0;
    for (;;) {
      const float* row = tl + ((size_t)b * m + node) * V;
      const bool kid = inm && lane != node && par == node;
      const float2 sp = stats[((size_t)b * m + node) * RS_SEG + (lane & (RS_SEG - 1))];
      const float l = row[(kid && inr) ? tok : 0];
      const float sm_ = lane < RS_SEG ? sp.x : -INFINITY;
      const float M = wave_max_dpp(sm_);
      const float seg = (lane < RS_SEG && sp.x > -INFINITY) ? sp.y * expf(sp.x - M) : 0.f;
      const float S = wave_sum_dpp(seg);
      const float z = (kid && inr) ? l * invT : -INFINITY;
      const float e = z > -INFINITY ? expf(z - M) : 0.f;
      const unsigned long long kb = __ballot(kid);
      // a token that an earlier child already carries is removed once: its
      // mass leaves the residual only with the first
      bool dup = false;
      for (unsigned long long rest = kb; rest; rest &= rest - 1ull) {  // the children, in flat order
        const int j = __ffsll((long long)rest) - 1;
        dup = dup || (j < lane && __builtin_amdgcn_readlane(tok, j) == tok);
      }
      bool pass;
      if (TOPK) {
        // the mass left when this child is tried: S less the earlier children's
        // (distinct) tokens; accept iff u_c * left <= e_c (> 0)
        const float ee = (kid && inr && !dup) ? e : 0.f;
        const float incl = wave_incl_scan(ee, lane);
        const float excl = __shfl_up(incl, 1);
        const float left = S - (lane > 0 ? excl : 0.f);
        pass = kid && ee > 0.f && uk * (left > 0.f ? left : 0.f) <= ee && len <= D;
      } else {
        pass = kid && inr && e / S >= thr && len <= D;
      }
      const unsigned long long pb = __ballot(pass);
      if (!pb) {  // the stop: what the residual draw needs
        if (lane < RS_SEG) s_seg[lane] = seg;
        if (kid) {
          const int slot = __popcll(kb & ((1ull << lane) - 1ull));
          s_kid[slot] = inr ? tok : -1;
          s_kseg[slot] = inr ? tok / SEGV : -1;
          s_ke[slot] = dup ? 0.f : e;
        }
        if (lane == 0) {
          s_M = M;
          s_nk = __popcll(kb);
          s_len = len;
          s_node = node;
        }
        break;
      }
      const int c = __ffsll((long long)pb) - 1;
      if (lane == 0) path[len] = c;
      node = c;
      ++len;
    }
  }
  __syncthreads();

  // ---- the bonus: residual draw at the stop node.  Segment masses less the
  // removed children (flat order), the segment holding u * total, then an
  // id-order scan of that segment alone.
  const int node = s_node, len = s_len;
  const float* row = tl + ((size_t)b * m + node) * V;
  const float M = s_M;
  const int nk = s_nk;
  if (tid < RS_SEG) {  // segment tid's mass less its removed children, in flat order
    float r = s_seg[tid];
    for (int k = 0; k < nk; ++k)
      if (s_kseg[k] == tid) r -= s_ke[k];
    s_res[tid] = r > 0.f ? r : 0.f;
  }
  __syncthreads();
  if (tid == 0) {
    float res[RS_SEG];
    float tot = 0.f;
    for (int sg = 0; sg < RS_SEG; ++sg) {
      res[sg] = s_res[sg];
      tot += res[sg];
    }
    int excl = 1;
    if (!(tot > 0.f)) {  // the children held all the mass: draw from p
      excl = 0;
      tot = 0.f;
      for (int sg = 0; sg < RS_SEG; ++sg) {
        res[sg] = s_seg[sg];
        tot += res[sg];
      }
    }
    float target = u * tot;
    if (!(target < tot)) target = nextafterf(tot, 0.f);
    int pick = -1, last = -1;
    float cum = 0.f;
    for (int sg = 0; sg < RS_SEG; ++sg) {
      if (res[sg] > 0.f) {
        if (pick < 0 && target < cum + res[sg]) {
          pick = sg;
          s_local = target - cum;
        }
        last = sg;
      }
      cum += res[sg];
    }
    if (pick < 0) {  // rounding at the very top: the last segment with mass, at its end
      pick = last;
      s_local = last >= 0 ? nextafterf(res[last], 0.f) : 0.f;
    }
    s_seg_pick = pick;
    s_excl = excl;
    s_pick = -1;
    s_last = -1;
  }
  __syncthreads();
  const int sg = s_seg_pick;
  if (sg >= 0) {
    const bool excl = s_excl != 0;
    const float local = s_local;
    const int a0 = min(V, sg * SEGV), a1 = min(V, a0 + SEGV);
    const int CH = (a1 - a0 + RV_T - 1) / RV_T;  // ids per thread, contiguous
    const int x0 = min(a1, a0 + tid * CH), x1 = min(a1, x0 + CH);
    auto mass = [&](int x, float l) {
      const float z = l * invT;
      bool out = !(z > -INFINITY);
      if (excl)
        for (int k = 0; k < nk; ++k) out = out || s_kid[k] == x;
      return out ? 0.f : expf(z - M);
    };
    // the chunk's logits, four unconditional loads from clamped ids at a time
    constexpr int CB = 4;
    float w = 0.f;
    for (int xb = x0; xb < x1; xb += CB) {
      float lv[CB];
#pragma unroll
      for (int q = 0; q < CB; ++q) lv[q] = row[min(xb + q, x1 - 1)];
#pragma unroll
      for (int q = 0; q < CB; ++q)
        if (xb + q < x1) w += mass(xb + q, lv[q]);
    }
    // chunk bounds: lo = (earlier waves) + (earlier lanes), hi = lo + own,
    // each formed as the same sum as the neighbouring chunk's bound
    const float wi = wave_incl_scan(w, lane);
    const float wprev = __shfl_up(wi, 1);
    if (lane == WAVE - 1) s_ws[wave] = wi;
    __syncthreads();
    float base = 0.f, tot = 0.f;
    for (int v = 0; v < RV_W; ++v) {
      if (v == wave) base = tot;
      tot = tot + s_ws[v];
    }
    const float lo = base + (lane > 0 ? wprev : 0.f), hi = base + wi;
    if (w > 0.f) {
      atomicMax(&s_last, tid);
      if (lo <= local && local < hi) {
        const float rem = local - lo;
        float acc = 0.f;
        int pick = -1, lastx = -1;
        for (int xb = x0; xb < x1 && pick < 0; xb += CB) {
          float lv[CB];
#pragma unroll
          for (int q = 0; q < CB; ++q) lv[q] = row[min(xb + q, x1 - 1)];
#pragma unroll
          for (int q = 0; q < CB; ++q) {
            if (xb + q >= x1 || pick >= 0) continue;
            const float e = mass(xb + q, lv[q]);
            if (e > 0.f) lastx = xb + q;
            if (e > 0.f && rem < acc + e) pick = xb + q;
            else acc += e;
          }
        }
        s_pick = pick >= 0 ? pick : lastx;
      }
    }
    __syncthreads();
    if (s_pick < 0 && tid == s_last) {  // the segment's scan came out below the target: its last id with mass
      int lastx = -1;
      for (int x = x0; x < x1; ++x)
        if (mass(x, row[x]) > 0.f) lastx = x;
      s_pick = lastx;
    }
    __syncthreads();
  }
  if (tid == 0) {
    alen[b] = len;
    bonus[b] = s_pick >= 0 ? s_pick : 0;
  }
  if (tid <= D) apath[(size_t)b * (D + 1) + tid] = tid < len ? path[tid] : -1;
}

__global__ void k_zero(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_rerank(const RoundArgs& a, int32_t* tokens, int32_t* parents, int32_t* depth,
                         int32_t* positions, uint8_t* mask, float* logscore, hipStream_t s) {
  int np = 1;
  while (np < a.pool_n) np <<= 1;
  if (np <= 64 * 8)
    hipLaunchKernelGGL(k_rerank_wave<8>, dim3(a.B), dim3(WAVE), 0, s, a, tokens, parents, depth, positions,
                       mask, logscore);
  else if (np <= 64 * 16)
    hipLaunchKernelGGL(k_rerank_wave<16>, dim3(a.B), dim3(WAVE), 0, s, a, tokens, parents, depth, positions,
                       mask, logscore);
  else
    hipLaunchKernelGGL(k_rerank, dim3(a.B), dim3(BLOCK), 0, s, a, tokens, parents, depth, positions,
                       mask, logscore);
  return hipGetLastError();
}

hipError_t launch_verify(int B, int m, int D, int V, const float* tl, const int32_t* tokens,
                         const int32_t* parents, int32_t* alen, int32_t* apath, int32_t* bonus,
                         hipStream_t s) {
  hipLaunchKernelGGL(k_verify, dim3(B), dim3(1024), 0, s, m, D, V, tl, tokens, parents, alen, apath,
                     bonus);
  return hipGetLastError();
}

hipError_t launch_verify_relaxed(int B, int m, int D, int V, const float* tl, const int32_t* tokens,
                                 const int32_t* parents, float temperature, float threshold,
                                 const float* uniforms, void* scratch, int32_t* alen, int32_t* apath,
                                 int32_t* bonus, hipStream_t s, bool topk) {
  float2* st = (float2*)scratch;
  hipLaunchKernelGGL(k_relaxed_stats, dim3(RS_SEG, B * m, 1), dim3(RS_T), 0, s, V, tl, st, tl, st, temperature);
  if (topk)
    hipLaunchKernelGGL(k_verify_relaxed<true>, dim3(B), dim3(RV_T), 0, s, m, D, V, tl, tokens, parents, temperature,
                       threshold, uniforms, (const float2*)st, alen, apath, bonus);
  else
    hipLaunchKernelGGL(k_verify_relaxed<false>, dim3(B), dim3(RV_T), 0, s, m, D, V, tl, tokens, parents,
                       temperature, threshold, uniforms, (const float2*)st, alen, apath, bonus);
  return hipGetLastError();
}

size_t verify_relaxed_scratch_bytes(int B, int m) { return (size_t)B * m * RS_SEG * sizeof(float2); }

// Strict verification by recursive rejection sampling ([P1] §6.2: accept a
// drafted token t iff u <= min(1, p(t)/q(t)), otherwise resample from
// norm(max(0, p - q)), node by node).  p and q are the target's and the
// draft's softmax(logits / T) at the current node.  Children are tried in
// flat order, child c accepted iff u_c * q(t_c) <= p(t_c); after a rejection
// p becomes norm(max(0, p - q)) (kept when that has no mass); when every
// child is rejected the bonus is drawn from the current p by inverse CDF
// with the sequence's last uniform.
//
// The residual after any number of rejections at a node has a closed form.
// Start from c = 0, N = 1; on a rejection set c' = c + N and
// N' = sum_x max(0, p(x) - c' q(x)); if N' > 0 then (c, N) = (c', N').  The
// current p is then max(0, p - c q) / N: by induction, since q >= 0,
// max(0, max(0, p - c q)/N - q) = max(0, p - (c + N) q) / N, whose mass is
// N'/N.  So a rejection costs one pass over the two rows and writes nothing.
//
// Two launches.  k_relaxed_stats (grid z = 2: the target's rows and the
// draft's) reduces every row to per-segment (max, sum) over the chip.
// k_verify_rejection (one workgroup per sequence) walks: wave 0 holds the
// tree (lane = flat slot), combines the node's segment statistics and forms
// p and q at each child's token with one load per lane; the workgroup tries
// the children in flat order, each rejection one pass over both rows
// (strided, eight clamped loads per row in flight per thread, summed in a
// fixed order).  The draw scans contiguous id chunks per thread in id order,
// every chunk bound the same sum wherever it is formed.
constexpr int RJ_T = 1024;
constexpr int RJ_W = RJ_T / WAVE;
constexpr int RJ_U = 8;

// block-wide sum in a fixed order (waves, then their partials in wave order);
// every thread gets it
__device__ __forceinline__ float rj_block_sum(float v, float* sbuf, int tid) {
  const float w = wave_sum_dpp(v);
  __syncthreads();
  if ((tid & 63) == 0) sbuf[tid >> 6] = w;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < RJ_W; ++i) t += sbuf[i];
  return t;
}

__global__ void __launch_bounds__(RJ_T) k_verify_rejection(int m, int D, int V, const float* tl, const float* dl,
                                                           const int32_t* tokens, const int32_t* parents,
                                                           float temperature, const float* uniforms,
                                                           const float2* stp, const float2* stq, int32_t* alen,
                                                           int32_t* apath, int32_t* bonus) {
  // no fused multiply-adds: p - c q and each exp(z - M) are formed the same
  // way wherever they appear
#pragma clang fp contract(off)
  __shared__ float s_red[RJ_W];
  __shared__ float s_stat[4];  // Mp, Sp, Mq, Sq of the current node
  __shared__ int s_kid[EAGLE_MAX_TREE], s_kok[EAGLE_MAX_TREE];
  __shared__ float s_kp[EAGLE_MAX_TREE], s_kq[EAGLE_MAX_TREE], s_ku[EAGLE_MAX_TREE];
  __shared__ int s_nk, s_pick, s_last;
  __shared__ int path[EAGLE_MAX_DEPTH + 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, b = blockIdx.x;
  const float invT = 1.0f / temperature;
  const float* ub = uniforms + (size_t)b * (m + 1);
  const bool inm = wave == 0 && lane < m;
  const int par = inm ? parents[(size_t)b * m + lane] : -2;
  const int tok = inm ? tokens[(size_t)b * m + lane] : -1;
  const float uk = inm ? ub[lane] : 1.f;  // the lane's node's uniform, used if it is tried
  const bool inr = tok >= 0 && tok < V;
  int node = 0, len = 1;
  if (tid == 0) path[0] = 0;
  // p(x) = exp(z - Mp) * (1 / Sp): one reciprocal per node instead of a
  // division per id in every pass
  float Mp = 0.f, rSp = 1.f, Mq = 0.f, rSq = 1.f, c = 0.f, N = 1.f;
  auto pv = [&](float l) -> float {
    const float z = l * invT;
    return z > -INFINITY ? expf(z - Mp) * rSp : 0.f;
  };
  auto qv = [&](float l) -> float {
    const float z = l * invT;
    return z > -INFINITY ? expf(z - Mq) * rSq : 0.f;
  };
  const float* rp = tl;
  const float* rq = dl;
  for (;;) {
    rp = tl + ((size_t)b * m + node) * V;
    rq = dl + ((size_t)b * m + node) * V;
    if (wave == 0) {
      const bool kid = inm && lane != node && par == node;
      const size_t si = ((size_t)b * m + node) * RS_SEG + (lane & (RS_SEG - 1));
      const float2 sp = stp[si], sq = stq[si];
      const float lp = rp[(kid && inr) ? tok : 0], lq = rq[(kid && inr) ? tok : 0];
      const float MP = wave_max_dpp(lane < RS_SEG ? sp.x : -INFINITY);
      const float MQ = wave_max_dpp(lane < RS_SEG ? sq.x : -INFINITY);
      const float SP = wave_sum_dpp((lane < RS_SEG && sp.x > -INFINITY) ? sp.y * expf(sp.x - MP) : 0.f);
      const float SQ = wave_sum_dpp((lane < RS_SEG && sq.x > -INFINITY) ? sq.y * expf(sq.x - MQ) : 0.f);
      const unsigned long long kb = __ballot(kid);
      if (kid) {
        const int slot = __popcll(kb & ((1ull << lane) - 1ull));
        const float zp = lp * invT, zq = lq * invT;
        s_kid[slot] = lane;
        s_kok[slot] = inr;
        s_ku[slot] = uk;
        s_kp[slot] = (inr && zp > -INFINITY) ? expf(zp - MP) * (1.0f / SP) : 0.f;
        s_kq[slot] = (inr && zq > -INFINITY) ? expf(zq - MQ) * (1.0f / SQ) : 0.f;
      }
      if (lane == 0) {
        s_nk = len <= D ? __popcll(kb) : 0;  // a path of depth+1 nodes is not extended
        s_stat[0] = MP;
        s_stat[1] = SP;
        s_stat[2] = MQ;
        s_stat[3] = SQ;
      }
    }
    __syncthreads();
    Mp = s_stat[0];
    rSp = 1.0f / s_stat[1];
    Mq = s_stat[2];
    rSq = 1.0f / s_stat[3];
    c = 0.f;
    N = 1.f;
    const int nk = s_nk;
    int next = -1;
    for (int j = 0; j < nk; ++j) {  // uniform loop: every thread takes the same decisions
      const float pc = s_kp[j], qc = s_kq[j];
      const float dc = pc - c * qc;
      const float rc = (dc > 0.f ? dc : 0.f) / N;
      // a token the residual gives no mass is never accepted (also when q
      // underflows to 0 at a low temperature: 0 <= 0 would pass)
      if (s_kok[j] && rc > 0.f && s_ku[j] * qc <= rc) {
        next = s_kid[j];
        break;
      }
      // rejected: the mass of max(0, p - (c + N) q)
      const float cn = c + N;
      float part = 0.f;
      for (int x0 = tid; x0 < V; x0 += RJ_T * RJ_U) {
        float lp[RJ_U], lq[RJ_U];
#pragma unroll
        for (int u = 0; u < RJ_U; ++u) {  // unconditional loads from clamped ids: all in flight at once
          const int x = min(x0 + u * RJ_T, V - 1);
          lp[u] = rp[x];
          lq[u] = rq[x];
        }
#pragma unroll
        for (int u = 0; u < RJ_U; ++u) {
          const float r = pv(lp[u]) - cn * qv(lq[u]);
          part += (x0 + u * RJ_T < V && r > 0.f) ? r : 0.f;
        }
      }
      const float Nn = rj_block_sum(part, s_red, tid);
      if (Nn > 0.f) {
        c = cn;
        N = Nn;
      }
    }
    if (next < 0) break;
    if (tid == 0) path[len] = next;
    node = next;
    ++len;
    __syncthreads();  // s_kid, s_kp, s_kq, s_stat are rewritten for the next node
  }

  // ---- the bonus: inverse CDF of the current p, contiguous id chunks in order
  const float ubonus = ub[m] >= 0.f ? (ub[m] < 1.f ? ub[m] : 0.99999994f) : 0.f;
  const int CH = (V + RJ_T - 1) / RJ_T;
  const int x0 = min(V, tid * CH), x1 = min(V, x0 + CH);
  const bool useq = c > 0.f;  // uniform
  auto weight = [&](float lp, float lq) -> float {  // mass of an id, up to the factor 1/N
    const float d = pv(lp) - (useq ? c * qv(lq) : 0.f);
    return d > 0.f ? d : 0.f;
  };
  float w = 0.f;
  for (int xa = x0; xa < x1; xa += RJ_U) {
    float lp[RJ_U], lq[RJ_U];
#pragma unroll
    for (int u = 0; u < RJ_U; ++u) {
      const int x = min(xa + u, V - 1);
      lp[u] = rp[x];
      lq[u] = useq ? rq[x] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < RJ_U; ++u)
      if (xa + u < x1) w += weight(lp[u], lq[u]);
  }
  const float wi = wave_incl_scan(w, lane);
  const float wprev = __shfl_up(wi, 1);
  __syncthreads();
  if (lane == WAVE - 1) s_red[wave] = wi;
  if (tid == 0) {
    s_pick = -1;
    s_last = -1;
  }
  __syncthreads();
  float base = 0.f, tot = 0.f;
  for (int v = 0; v < RJ_W; ++v) {
    if (v == wave) base = tot;
    tot = tot + s_red[v];
  }
  const float lo = base + (lane > 0 ? wprev : 0.f), hi = base + wi;
  float target = ubonus * tot;
  if (!(target < tot)) target = nextafterf(tot, 0.f);
  if (w > 0.f) {
    atomicMax(&s_last, tid);
    if (lo <= target && target < hi) {
      // the chunk again, in the same order and the same sums, eight loads in
      // flight; acc and lastx stop at the pick
      const float rem = target - lo;
      float acc = 0.f;
      int pick = -1, lastx = -1;
      for (int xa = x0; xa < x1 && pick < 0; xa += RJ_U) {
        float lp[RJ_U], lq[RJ_U];
#pragma unroll
        for (int u = 0; u < RJ_U; ++u) {
          const int x = min(xa + u, V - 1);
          lp[u] = rp[x];
          lq[u] = useq ? rq[x] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < RJ_U; ++u) {
          if (xa + u < x1 && pick < 0) {
            const float e = weight(lp[u], lq[u]);
            if (e > 0.f) lastx = xa + u;
            if (e > 0.f && rem < acc + e) pick = xa + u;
            else acc += e;
          }
        }
      }
      s_pick = pick >= 0 ? pick : lastx;
    }
  }
  __syncthreads();
  if (s_pick < 0 && tid == s_last) {  // the chunk's scan came out below the target: its last id with mass
    int lastx = -1;
    for (int xa = x0; xa < x1; xa += RJ_U) {
      float lp[RJ_U], lq[RJ_U];
#pragma unroll
      for (int u = 0; u < RJ_U; ++u) {
        const int x = min(xa + u, V - 1);
        lp[u] = rp[x];
        lq[u] = useq ? rq[x] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < RJ_U; ++u)
        if (xa + u < x1 && weight(lp[u], lq[u]) > 0.f) lastx = xa + u;
    }
    s_pick = lastx;
  }
  __syncthreads();
  if (tid == 0) {
    alen[b] = len;
    bonus[b] = s_pick >= 0 ? s_pick : 0;
  }
  if (tid <= D) apath[(size_t)b * (D + 1) + tid] = tid < len ? path[tid] : -1;
}

hipError_t launch_verify_rejection(int B, int m, int D, int V, const float* tl, const float* dl,
                                   const int32_t* tokens, const int32_t* parents, float temperature,
                                   const float* uniforms, void* scratch, int32_t* alen, int32_t* apath,
                                   int32_t* bonus, hipStream_t s) {
  float2* stp = (float2*)scratch;
  float2* stq = stp + (size_t)B * m * RS_SEG;
  hipLaunchKernelGGL(k_relaxed_stats, dim3(RS_SEG, B * m, 2), dim3(RS_T), 0, s, V, tl, stp, dl, stq, temperature);
  hipLaunchKernelGGL(k_verify_rejection, dim3(B), dim3(RJ_T), 0, s, m, D, V, tl, dl, tokens, parents, temperature,
                     uniforms, (const float2*)stp, (const float2*)stq, alen, apath, bonus);
  return hipGetLastError();
}

size_t verify_rejection_scratch_bytes(int B, int m) { return 2 * (size_t)B * m * RS_SEG * sizeof(float2); }

// RoPE frequencies theta^(-2i/hd), i < hd/2, in fp64 ([P1] §12 item 5 positions;
// reading R8: theta and rotate-half pairs), once per workspace
__global__ void k_rope_table(double* t, int half, double theta, int hd) {
  const int i = (int)threadIdx.x;
  if (i < half) t[i] = pow(theta, -2.0 * (double)i / (double)hd);
}

hipError_t launch_rope_table(double* t, int hd, float theta, hipStream_t s) {
  hipLaunchKernelGGL(k_rope_table, dim3(1), dim3(WAVE * 2), 0, s, t, hd / 2, (double)theta, hd);
  return hipGetLastError();
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  const int blocks = (int)(n16 / BLOCK + 1 < 4096 ? n16 / BLOCK + 1 : 4096);
  hipLaunchKernelGGL(k_zero, dim3(blocks), dim3(BLOCK), 0, s, (uint4*)p, n16);
  return hipGetLastError();
}

}  // namespace eg

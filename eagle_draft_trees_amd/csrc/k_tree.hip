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

__global__ void k_zero(uint4* p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_rerank(const RoundArgs& a, int32_t* tokens, int32_t* parents, int32_t* depth,
                         int32_t* positions, uint8_t* mask, float* logscore, hipStream_t s) {
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

hipError_t launch_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  const int blocks = (int)(n16 / BLOCK + 1 < 4096 ? n16 / BLOCK + 1 : 4096);
  hipLaunchKernelGGL(k_zero, dim3(blocks), dim3(BLOCK), 0, s, (uint4*)p, n16);
  return hipGetLastError();
}

}  // namespace eg

// Internal declarations of the gfx950 EAGLE-2 draft-round library: element
// types, MFMA wrappers, wave reductions, the workspace layout and launch plans.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "eagle_mi355x.h"

namespace eg {

typedef uint16_t bf16_t;  // bf16 bit pattern
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;
constexpr int BLOCK = 256;       // four waves
constexpr int NCNT = 1 << 16;    // last-block counters in the workspace
constexpr int GRID_CNT = NCNT - 1;
// FC hand-over: counter 1 counts the workgroups that have read the mailbox,
// whose 16 64-bit entries sit at counters CNT_MBOX..CNT_MBOX+31
constexpr int CNT_MBOX = 128;
constexpr int GEMM_MAXS = 64;    // split-K ways at most
constexpr int GW_KSW = 4;                   // layer GEMM workgroup: 4 column tiles x GW_KSW K slices
constexpr int GW_THREADS = 4 * GW_KSW * 64;
// k-steps per wave per X chunk: four with one weight stream, two with two or
// with X in two parts (hl: the bf16 q/k/v projection's x0 = hi + lo, whose two
// chunks share the LDS)
__host__ __device__ constexpr int gw_bu(int nw, bool hl = false) { return (nw == 2 || hl) ? 2 : 4; }
constexpr int GW_FIN_THREADS = 1024;        // split-sum workgroup: one (column tile, m-tile, lane) per thread

enum Op { OP_FC = 0, OP_QKV = 1, OP_O = 2, OP_GATEUP = 3, OP_DOWN = 4 };
enum Mode { MODE_LEVEL = 0, MODE_EXTEND = 1, MODE_VERIFY = 2 };  // verify: target-side tree attention
enum ErrBits { ERR_TOKEN = 1, ERR_PREFIX = 2, ERR_SYNC = 4 };

// ------------------------------------------------------------------ elements

__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }
// round to nearest, ties to even (finite inputs)
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

template <typename T> struct El;
template <> struct El<float> {
  static constexpr int KSTEP = 16;  // k covered by one 16-byte-per-lane fragment across a wave
  static constexpr int PER16 = 4;   // elements per 16 bytes
  __device__ static __forceinline__ float ld(const float* p, size_t i) { return p[i]; }
  __device__ static __forceinline__ void st(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct El<bf16_t> {
  static constexpr int KSTEP = 32;
  static constexpr int PER16 = 8;
  __device__ static __forceinline__ float ld(const bf16_t* p, size_t i) { return bf2f(p[i]); }
  __device__ static __forceinline__ void st(bf16_t* p, size_t i, float v) { p[i] = (bf16_t)f2bf(v); }
};

// 16x16 output tile, 16 bytes of A (rows) and 16 bytes of B (columns) per lane.
// Lane l supplies A[l%16][kslot(l/16)] and B[kslot(l/16)][l%16]; it receives
// D[4*(l/16)+r][l%16], r = 0..3.  Both operands use the same k permutation,
// so any assignment of k to (lane group, element) contracts correctly.
__device__ __forceinline__ f32x4_t mma16(uint4 a, uint4 b, f32x4_t c, bf16_t) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mma16(uint4 a, uint4 b, f32x4_t c, float) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  return c;
}

// ------------------------------------------------------------------ wave reductions

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
// butterfly sum; every lane takes lane 0's total so all lanes agree bit for bit
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return __shfl(v, 0);
}
// ------------------------------------------------------------------ DPP reductions
// Cross-lane steps on the DPP path (a VALU operand modifier, no LDS round trip):
// xor 1 and xor 2 within quads, then half-row and row mirrors; after those every
// lane of a 16-lane row holds the row's result, and the four rows are combined
// with row broadcasts into lane 63 (see wave_max_u32).  The step order is
// fixed, so float results are deterministic.

__device__ __forceinline__ unsigned dpp_u32(unsigned x, int ctrl_sel) {
  switch (ctrl_sel) {
    case 0: return (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false);   // quad xor 1
    case 1: return (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false);   // quad xor 2
    case 2: return (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x141, 0xF, 0xF, false);  // half-row mirror
    default: return (unsigned)__builtin_amdgcn_update_dpp(0, (int)x, 0x140, 0xF, 0xF, false); // row mirror
  }
}

// Order-preserving 64-bit key of (value desc, id asc): larger key = better.
__device__ __forceinline__ unsigned long long argkey(float v, int id) {
  uint32_t u = __float_as_uint(v);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)u << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)id);
}
__device__ __forceinline__ float argkey_value(unsigned long long k) {
  uint32_t u = (uint32_t)(k >> 32);
  u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(u);
}
__device__ __forceinline__ int argkey_id(unsigned long long k) {
  return (int)(0xFFFFFFFFu - (uint32_t)k);
}


// maximum over the wave of unsigned 32-bit values (0 is the identity); every lane gets it
// Cross-row finish of a DPP reduction with the GFX9 row broadcasts: after the
// four intra-row steps every lane of a 16-lane row holds the row's result;
// row_bcast:15 folds row 0 into row 1 and row 2 into row 3, row_bcast:31 folds
// lane 31 into rows 2 and 3, so lane 63 holds the wave's result and one
// readlane broadcasts it (no scalar-unit work per row).
__device__ __forceinline__ unsigned dpp_bcast15(unsigned x, unsigned id) {
  return (unsigned)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x142, 0xA, 0xF, false);
}
__device__ __forceinline__ unsigned dpp_bcast31(unsigned x, unsigned id) {
  return (unsigned)__builtin_amdgcn_update_dpp((int)id, (int)x, 0x143, 0xC, 0xF, false);
}
__device__ __forceinline__ unsigned wave_max_u32(unsigned v) {
#pragma unroll
  for (int s = 0; s < 4; ++s) v = max(v, dpp_u32(v, s));
  v = max(v, dpp_bcast15(v, 0u));
  v = max(v, dpp_bcast31(v, 0u));
  return (unsigned)__builtin_amdgcn_readlane(v, 63);
}
// maximum 64-bit key over the wave (every lane gets it): the highest high
// word by a 32-bit reduction; when one lane holds it (the usual case for
// keys led by a float value) its low word is read from that lane, otherwise
// a second reduction takes the highest low word among the lanes that tie
__device__ __forceinline__ unsigned long long wave_max_key(unsigned long long k) {
  const unsigned hi = (unsigned)(k >> 32);
  const unsigned mh = wave_max_u32(hi);
  const unsigned long long tie = __ballot(hi == mh);
  unsigned ml;
  if (__popcll(tie) == 1)
    ml = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)k, __ffsll((long long)tie) - 1);
  else
    ml = wave_max_u32(hi == mh ? (unsigned)k : 0u);
  return ((unsigned long long)mh << 32) | ml;
}

// The k largest of the wave's 64-bit keys (N per lane, unique, 0 = empty),
// sorted: lane j < k receives the j-th largest, 0 past the number of keys.
// k <= 16.  Instead of k dependent rounds of a wave argmax:
//  1. threshold: each lane's largest key; the k-th largest of those 64 lane
//     maxima (ranked by counting against all of them, read back from LDS) is
//     a key with at least k - 1 keys above it, so every key of the top k is
//     at or above it (with fewer than k non-empty lanes, every key counts);
//  2. the keys at or above the threshold -- at most k*N, from the lanes whose
//     maximum ranked below k -- are packed into LDS;
//  3. each packed key is ranked by counting the packed keys above it, and the
//     first k are placed at their rank.
// `sh`: 128 words of LDS owned by the wave.
__device__ __forceinline__ unsigned lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}
template <int N>
__device__ __forceinline__ unsigned long long wave_topk(const unsigned long long (&key)[N], int k,
                                                        unsigned long long* sh) {
  static_assert(N <= 4, "at most 4 keys per lane (k*N <= 64 packed keys)");
  const int lane = (int)lane_id();
  unsigned long long lm = key[0];
#pragma unroll
  for (int e = 1; e < N; ++e) lm = key[e] > lm ? key[e] : lm;
  sh[lane] = lm;
  __builtin_amdgcn_wave_barrier();
  int r = 0;  // rank of this lane's maximum among the lane maxima
#pragma unroll
  for (int i = 0; i < WAVE; i += 8) {  // four 16-byte broadcast reads in flight at a time
    ulonglong2 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = *(const ulonglong2*)(sh + i + 2 * j);
#pragma unroll
    for (int j = 0; j < 4; ++j) r += (v[j].x > lm ? 1 : 0) + (v[j].y > lm ? 1 : 0);
    asm volatile("" : "+v"(r)::"memory");  // this batch is used before the next is read
  }
  const unsigned long long nzl = __ballot(lm != 0ull);
  const int nl = __popcll(nzl);
  unsigned long long tau = 1ull;  // fewer than k non-empty lanes: every key
  if (nl >= k) {
    const unsigned long long at = __ballot(lm != 0ull && r == k - 1);
    const int l = __ffsll((long long)at) - 1;
    tau = ((unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)(lm >> 32), l) << 32) |
          (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)lm, l);
  }
  // pack the keys >= tau into sh[64..64+nc)
  int nc = 0;
  unsigned long long* pk = sh + WAVE;
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const bool in = key[e] != 0ull && key[e] >= tau;
    const unsigned long long m = __ballot(in);
    if (in) pk[nc + __popcll(m & ((1ull << lane) - 1ull))] = key[e];
    nc += __popcll(m);
  }
  __builtin_amdgcn_wave_barrier();
  // rank the packed keys (nc <= 64): lane l holds packed key l
  const unsigned long long c = lane < nc ? pk[lane] : 0ull;
  int rk = 0;
  for (int i = 0; i < nc; i += 8) {  // pk[nc..i+7] (within pk[0..63]) may be stale: masked
    ulonglong2 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = *(const ulonglong2*)(pk + i + 2 * j);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      rk += ((i + 2 * j < nc && v[j].x > c) ? 1 : 0) + ((i + 2 * j + 1 < nc && v[j].y > c) ? 1 : 0);
    asm volatile("" : "+v"(rk)::"memory");
  }
  __builtin_amdgcn_wave_barrier();
  if (lane < nc && rk < k) sh[rk] = c;
  __builtin_amdgcn_wave_barrier();
  const unsigned long long out = lane < min(k, nc) ? sh[lane] : 0ull;
  __builtin_amdgcn_wave_barrier();
  return out;
}

__device__ __forceinline__ float wave_sum_dpp(float v) {
#pragma unroll
  for (int s = 0; s < 4; ++s) v += __uint_as_float(dpp_u32(__float_as_uint(v), s));
  v += __uint_as_float(dpp_bcast15(__float_as_uint(v), 0u));
  v += __uint_as_float(dpp_bcast31(__float_as_uint(v), 0u));
  return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 63));
}

__device__ __forceinline__ float wave_max_dpp(float v) {
  const unsigned ninf = __float_as_uint(-INFINITY);
#pragma unroll
  for (int s = 0; s < 4; ++s) v = fmaxf(v, __uint_as_float(dpp_u32(__float_as_uint(v), s)));
  v = fmaxf(v, __uint_as_float(dpp_bcast15(__float_as_uint(v), ninf)));
  v = fmaxf(v, __uint_as_float(dpp_bcast31(__float_as_uint(v), ninf)));
  return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), 63));
}

// (value desc, id asc) winner across the wave; every lane gets the result
__device__ __forceinline__ void wave_argmax(float& v, int& id) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(v, o);
    int oi = __shfl_xor(id, o);
    if (ov > v || (ov == v && oi < id)) { v = ov; id = oi; }
  }
}

// ------------------------------------------------------------------ workspace

struct WsLayout {
  size_t err, cnt, pool, frontier, feat, tk, tv, ext_h;
  size_t x0f, x0b, x0l, q, attn, yf, yg, rstd, ssq, act;
  size_t gpart, lmpart, lmres, apart, xpk, rope;
  size_t total;
  int rows_max, pool_n;
};

struct GemmPlan {
  int M, N, K, nw, mt, zg, nblk, S, Kc;
  int hl;              // X in two bf16 parts (the bf16 q/k/v projection)
  int ct;              // column tiles per workgroup (3 or 4; 4 whenever K is split)
  int nps;             // gate/up: RMSNorm partial sums per row written by the O launch
  size_t part_floats;  // split-K partial floats (0 when S == 1 on the skinny path)
  int tiled;           // bf16, more than 64 rows, K a multiple of 128: k_gemm_tiled, then k_gemm_fin
  int tks;             // tiled / rows: k-steps per split (a multiple of the main loop's unroll)
  int rows;            // bf16, 17..64 rows, K a multiple of 256: k_gemm_rows, then k_gemm_fin
  int nq;              // rows: 16-column weight tiles per wave
};
// K elements of one X chunk of a layer GEMM (the GW_KSW slices' k-steps)
inline int gemm_kc(int nw, int es, bool hl = false) { return GW_KSW * gw_bu(nw, hl) * (es == 2 ? 32 : 16); }
// dynamic LDS of a layer GEMM workgroup: two X chunks, then the K-slice
// partials, then the output tile and the RMSNorm partials
inline size_t gemm_lds_bytes(const GemmPlan& p, int es) {
  const size_t rows = (size_t)p.mt * 16;
  const size_t xt = (p.hl ? 4 : 2) * rows * ((size_t)gemm_kc(p.nw, es, p.hl) * es + 16);
  const size_t red = (size_t)(GW_KSW - 1) * 4 * p.nw * p.mt * 64 * 16;
  const size_t tile = (size_t)p.nw * rows * 65 * 4 + rows * 16 * 4;
  return xt > red ? (xt > tile ? xt : tile) : (red > tile ? red : tile);
}

// Level GEMM with at most 16 rows: CT column tiles of 16 per workgroup, K split
// over KSW waves per tile (CT * KSW <= SK_MAXW waves), nwg workgroups.
constexpr int SK_MAXW = 16;
constexpr int SK_QKVW = 12;  // waves of a q/k/v projection workgroup at most
struct SkPlan {
  int M, N, K, ntile, CT, KSW, nwg;
  int nps;   // gate/up: RMSNorm partial sums per row written by the O launch
  int xlds;  // X staged in LDS (its 16 rows fit)
};

struct LmPlan {
  int M, mt, zg, nblk, rec;  // rec = floats per (row, slab) partial; nblk = slabs
  int sk, CT, KSW, xlds;     // sk: streaming-core kernel (M <= 16), CT tiles x KSW waves
  int big;                   // bf16, more than 64 rows, d a multiple of 128: the tiled GEMM (k_lmgemm), zg row tiles
  int nq;                    // bf16, 17..64 rows, d a multiple of 128: k_lmrows with nq 16-column tiles per wave
  size_t part_floats;
};

struct AttnPlan {
  int RS, g, nq, nqt;  // rows per sequence, GQA group, queries per KV head, 16-query tiles
  int nsplit;          // key splits per tile (partials merged by a second kernel when > 1)
  int waves;           // waves per workgroup: 4 (three workgroups per CU) or 8 (one)
  size_t part_floats;  // split partials
};

GemmPlan plan_gemm(int op, int M, const eagle_dims& d);
SkPlan plan_skinny(int op, int M, const eagle_dims& d);
LmPlan plan_lm(int M, const eagle_dims& d, int topk);
AttnPlan plan_attn(int mode, int RS, const eagle_dims& d, const eagle_tree_cfg& c, int nseq);
WsLayout plan_ws(const eagle_dims& d, const eagle_tree_cfg& c);
size_t elem_size(const eagle_dims& d);

// ------------------------------------------------------------------ kernel argument blocks

struct RoundArgs {
  // shapes
  int dtype;  // eagle_dtype
  int B, d, H, Hkv, hd, F, V, D, k, m, max_prefix;
  float eps, theta;
  int mode, depth;  // depth = depth of the rows being forwarded (level - 1)
  int rows, RS;     // total rows, rows per sequence
  // weights
  const void *fc_w, *fc_b, *wq, *wk, *wv, *wo, *post_norm, *w_gate, *w_up, *w_down, *embed, *lm_head;
  const float* tok_proj;  // [V][d]: the token half of the FC per vocabulary entry
  // state
  void *k_cache, *v_cache;
  int* prefix_len;
  void* root_feat;
  int* root_token;
  // extend inputs
  const void* true_feat;
  const int *tokens, *accept_len, *accept_path, *bonus;
  // workspace
  int* err;
  int* cnt;
  eagle_pool_entry* pool;
  eagle_frontier_node* frontier;  // [D+1][B][k]
  void *feat, *tk, *tv, *ext_h;
  float* x0f;
  void* x0b;
  void* x0l;  // bf16: the low part of x0, bf16(x0 - bf16(x0))
  float* q;
  void* attn;
  const uint8_t* vmask;  // tree verify: the [B][m][m] ancestor-or-self mask
  const int32_t* tmpl;   // static tree: [D][k] (parent slot, child rank) per slot; null = dynamic
  float* yf;
  void* yg;
  float *rstd, *ssq;
  void* act;
  float *gpart, *lmpart, *lmres, *apart;
  const double* rope;  // [hd/2]: theta^(-2i/hd) in fp64, written at workspace init
  void* xpk;  // batched LM head: its input rows in MFMA fragment order
  int pool_n;
  // levels (bf16, 17..64 rows): the down epilogue also writes the level's
  // features into xpk in 16-row blocks (xpk_index, d/32 k-steps) for the
  // streaming LM head that follows in the same call
  int lm_px;
};

// ------------------------------------------------------------------ device helpers

// v if keep, else all-zero bits (a bitwise mask, never a select between
// memory locations).
__device__ __forceinline__ uint4 mask4(uint4 v, bool keep) {
  const unsigned m = keep ? 0xFFFFFFFFu : 0u;
  return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m);
}

// ------------------------------------------------------------------ packed weights
// A streamed matrix W [N][K] is stored as tiles of 16 output rows x KSTEP
// inputs (one kilobyte, the B operand of one 16x16 MFMA step) in the order a
// wave loads them: lane l's 16 bytes at l * PER16 elements; tile (t, s) at
// (t * nks + s) * 16 * KSTEP, nks = ceil(K / KSTEP).  Rows and K are padded
// with zeros to whole tiles.

// elements of one tile
template <typename T> __host__ __device__ constexpr int wtile_elems() { return 16 * El<T>::KSTEP; }

// lane `lane`'s piece of tile (t, 0); k-step s adds s * wtile_elems<T>()
template <typename T>
__device__ __forceinline__ const T* wtile_base(const void* w, int nks, int t, int lane) {
  return (const T*)w + (size_t)t * nks * wtile_elems<T>() + lane * El<T>::PER16;
}

// The SwiGLU activations (the down projection's X) are stored in blocks of
// 16 rows x one k-step (one contiguous kilobyte), row-major inside a block:
// element (r, k) of the [rows][K] matrix at ((r/16) * nks + k/KSTEP) * 16 *
// KSTEP + (r%16) * KSTEP + k%KSTEP.  A lane's A-operand piece (row i, 16
// bytes) is one aligned 16-byte load, and the rows of a block that lie past
// the real rows fill whole cache lines at its end, which a reader that
// points those lanes at the last real row never fetches.
template <typename T>
__host__ __device__ __forceinline__ size_t xpk_index(int r, int k, int nks) {
  constexpr int KS = El<T>::KSTEP;
  const int s = k / KS;
  return (((size_t)(r >> 4) * nks + s) * 16 + (r & 15)) * KS + (k - s * KS);
}

// q/k/v tiles are numbered over the heads in the order [q heads | k heads |
// v heads], hd/16 tiles per head; tile j of a head holds its rows 8j..8j+7
// and hd/2+8j..hd/2+8j+7 (8 rotation pairs)
template <typename T>
__device__ __forceinline__ const T* qkv_tile(const RoundArgs& a, int t, int nks, int lane) {
  const int per = a.hd / 16, head = t / per;
  if (head < a.H) return wtile_base<T>(a.wq, nks, t, lane);
  if (head < a.H + a.Hkv) return wtile_base<T>(a.wk, nks, t - a.H * per, lane);
  return wtile_base<T>(a.wv, nks, t - (a.H + a.Hkv) * per, lane);
}

__device__ __forceinline__ int clamp_tok(int t, int V, int* err) {
  if (t < 0 || t >= V) {
    atomicOr(err, ERR_TOKEN);
    t = t < 0 ? 0 : V - 1;
  }
  return t;
}

__device__ __forceinline__ int clamp_prefix(int P, const RoundArgs& a) {
  const int hi = a.max_prefix - a.m;
  if (P < 1 || P > hi) {
    atomicOr(a.err, ERR_PREFIX);
    P = P < 1 ? 1 : hi;
  }
  return P;
}

__device__ __forceinline__ int clamp_slot(int s, int k) { return s < 0 ? 0 : (s >= k ? k - 1 : s); }

// Rows per sequence of the extend: an accepted path holds the root and at
// most one node per level, and no more nodes than the tree, so min(m, D+1)
// rows cover every accepted length.
__host__ __device__ inline int ext_rows(int m, int D) { return m < D + 1 ? m : D + 1; }

// accept_len of sequence b, clamped to 1..(extend rows per sequence)
__device__ __forceinline__ int ext_alen(const RoundArgs& a, int b) {
  const int l = a.accept_len[b];
  return l < 1 ? 1 : (l > a.RS ? a.RS : l);
}

// Sources of extend row `row` (sequence row / RS, row i within it): the
// target's feature at path node min(i, alen-1) and the token of path node
// i+1, or the bonus for row alen-1 (rows past it repeat that row's feature
// and carry the next path entry's token or the bonus; they are computed and
// ignored).  Flat tree indices are clamped into the tree.
template <typename T>
__device__ __forceinline__ void ext_row_src(const RoundArgs& a, int row, const T*& feat, int& tok) {
  const int b = row / a.RS, i = row - b * a.RS;
  const int last = ext_alen(a, b) - 1, ii = i < last ? i : last;
  const int* path = a.accept_path + (size_t)b * (a.D + 1);
  const int pi = clamp_slot(path[ii], a.m);
  feat = (const T*)a.true_feat + ((size_t)b * a.m + pi) * a.d;
  tok = i < last ? a.tokens[(size_t)b * a.m + clamp_slot(path[i + 1], a.m)] : a.bonus[b];
}

// Token of FC row `row` (a frontier node's own token at a level; the next
// path token or the bonus in the extend), clamped into the vocabulary: the
// row's token half of the FC is tok_proj[token].
template <typename T>
__device__ __forceinline__ int fc_row_token(const RoundArgs& a, int row) {
  int tok;
  if (a.mode == MODE_LEVEL) {
    const int b = row / a.k, j = row - b * a.k;
    tok = a.frontier[((size_t)a.depth * a.B + b) * a.k + j].token;
  } else {
    const T* f;
    ext_row_src<T>(a, row, f, tok);
  }
  return clamp_tok(tok, a.V, a.err);
}

// Extend: the sequence state advances (the prefix grows by the accepted
// length, the bonus becomes the next root token).  Called by one workgroup
// of a launch that reads neither field.
__device__ __forceinline__ void ext_advance_state(const RoundArgs& a, int tid, int nthreads) {
  for (int b = tid; b < a.B; b += nthreads) {
    a.prefix_len[b] = clamp_prefix(a.prefix_len[b], a) + ext_alen(a, b);
    a.root_token[b] = clamp_tok(a.bonus[b], a.V, a.err);
  }
}

// Sine and cosine of the RoPE angle pos * inv (inv = theta^(-2i/hd) from the
// workspace's fp64 table): the angle in fp64, reduced to [-pi, pi] in fp64,
// then its sine and cosine in fp32 (the rotation itself is applied in fp32)
__device__ __forceinline__ void rope_sincos(int pos, double inv, float& sn, float& cs) {
  const double ang = (double)pos * inv;
  const double red = ang - 6.283185307179586 * rint(ang * 0.15915494309189535);
  sincosf((float)red, &sn, &cs);
}

__device__ __forceinline__ uint4 ld16(const void* p) { return *(const uint4*)p; }

// x0 element idx of the layer's rows: fp32 (the residual), the dtype copy and,
// for bf16, the low part that the q/k/v projection adds back
template <typename T>
__device__ __forceinline__ void st_x0(const RoundArgs& a, size_t idx, float x) {
  a.x0f[idx] = x;
  El<T>::st((T*)a.x0b, idx, x);
  if constexpr (sizeof(T) == 2) {
    const uint32_t h = f2bf(x);
    ((bf16_t*)a.x0l)[idx] = (bf16_t)f2bf(x - bf2f(h));
  }
}
// 16-byte load from a pointer known to be global memory (for pointers that
// were themselves read from LDS, whose address space the compiler cannot infer)
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16g(const void* p) {
  const u32x4_t v = *(const __attribute__((address_space(1))) u32x4_t*)(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
// 16-byte load of a packed weight piece, non-temporal: the weight stream is
// read once per pass and should not evict what the next kernels reuse (the
// KV cache, activations, partial records)
__device__ __forceinline__ uint4 ld16w(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4_t*)(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Last-block election across workgroups (possibly on different XCDs, whose L2s
// are not coherent with each other).  Every thread waits until its own global
// stores are complete (a workgroup-scope fence does not wait for them), the
// block synchronises, and one thread alone releases at agent scope (one L2
// write-back per block instead of one per wave) and bumps the counter.  The
// block that arrives last acquires at agent scope (one L2 invalidate) and
// resets the counter.  Returns true in that block only.
__device__ __forceinline__ bool arrive_last(int* cnt, int total) {
  __shared__ int s_last;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const int prev = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == total - 1);
    if (s_last) {
      __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
  }
  __syncthreads();
  return s_last != 0;
}

// block-wide (value desc, id asc) argmax of 256 threads; result in every thread
__device__ __forceinline__ void block_argmax(float& v, int& id, float* sv, int* si) {
  wave_argmax(v, id);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) { sv[wave] = v; si[wave] = id; }
  __syncthreads();
  v = sv[0];
  id = si[0];
#pragma unroll
  for (int w = 1; w < BLOCK / WAVE; ++w)
    if (sv[w] > v || (sv[w] == v && si[w] < id)) { v = sv[w]; id = si[w]; }
}

// launchers (return a hipError_t)
hipError_t launch_gemm(int op, const RoundArgs& a, const GemmPlan& p, hipStream_t s);
hipError_t launch_skinny(int op, const RoundArgs& a, const SkPlan& p, hipStream_t s);
int lmgemm_rows();  // rows per k_lmgemm tile
hipError_t launch_gemm_rows(int op, const RoundArgs& a, const GemmPlan& p, hipStream_t s);
hipError_t launch_gemm_tiled(int op, const RoundArgs& a, const GemmPlan& p, hipStream_t s);
hipError_t launch_lmrows(const RoundArgs& a, const LmPlan& p, int level, hipStream_t s, hipEvent_t e0,
                         hipEvent_t e1);
hipError_t launch_lmgemm(const RoundArgs& a, const LmPlan& p, int level, hipStream_t s, hipEvent_t e0,
                         hipEvent_t e1);
// e0/e1 (may be null): events stamped at the LM-head kernel's own start and end
// Slab records of the LM head, field-major per row: field f (0 max, 1 sum of
// exp, 2..k+1 the slab's top-k logits, k+2..2k+1 their token ids) of slab blk
// of row `row` at lmpart[(row * rec + f) * nblk + blk], so a pass over one
// field of every slab is contiguous.  Returns the address of field 0.
__device__ __forceinline__ float* slab_field(float* lmpart, int row, int blk, const LmPlan& p) {
  return lmpart + (size_t)row * p.rec * p.nblk + blk;
}
// One row's record of one 64-column slab, from the row's 64 logits in
// registers (columns past the vocabulary at -inf): max, sum of exp(v - max),
// and the top-k by (logit desc, id asc).  Pass r takes the best column below
// the previous pick in that order; scanning columns upward, a strictly
// greater value wins, so the lowest column of equal values is taken.
__device__ __forceinline__ void lm_slab_record(const RoundArgs& a, const LmPlan& p, const float (&v)[64], int row,
                                               int slab, int cbase) {
  const int kk_ = a.k;
  float mx = -INFINITY;
#pragma unroll
  for (int col = 0; col < 64; ++col) mx = fmaxf(mx, v[col]);
  float se = 0.f;
#pragma unroll
  for (int col = 0; col < 64; ++col) se += v[col] == -INFINITY ? 0.f : expf(v[col] - mx);
  if (row < p.M && slab < p.nblk) {
    float* rec = slab_field(a.lmpart, row, slab, p);  // field f at rec[f * nblk]
    rec[0] = mx;
    rec[p.nblk] = se;
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
}
hipError_t launch_lmhead(const RoundArgs& a, const LmPlan& p, int level, hipStream_t s,
                         hipEvent_t e0 = nullptr, hipEvent_t e1 = nullptr);
// handover (may be null): the FC hand-over of the next level rides along in
// the merge's launch (the FC plan over this level's rows; its CT * KSW waves
// are the launch's block size)
hipError_t launch_lmmerge(const RoundArgs& a, const LmPlan& p, int level, hipStream_t s,
                          const SkPlan* handover = nullptr);
hipError_t launch_attn(const RoundArgs& a, const AttnPlan& p, hipStream_t s);
hipError_t launch_rope_table(double* t, int hd, float theta, hipStream_t s);
hipError_t launch_rerank(const RoundArgs& a, int32_t* tokens, int32_t* parents, int32_t* depth,
                         int32_t* positions, uint8_t* mask, float* logscore, hipStream_t s);
hipError_t launch_verify(int B, int m, int D, int V, const float* tl, const int32_t* tokens,
                         const int32_t* parents, int32_t* alen, int32_t* apath, int32_t* bonus,
                         hipStream_t s);
// topk: the deterministic-candidate rejection walk (uniforms [B][m+1], no threshold)
hipError_t launch_verify_relaxed(int B, int m, int D, int V, const float* tl, const int32_t* tokens,
                                 const int32_t* parents, float temperature, float threshold,
                                 const float* uniforms, void* scratch, int32_t* alen, int32_t* apath,
                                 int32_t* bonus, hipStream_t s, bool topk = false);
size_t verify_relaxed_scratch_bytes(int B, int m);
hipError_t launch_verify_rejection(int B, int m, int D, int V, const float* tl, const float* dl,
                                   const int32_t* tokens, const int32_t* parents, float temperature,
                                   const float* uniforms, void* scratch, int32_t* alen, int32_t* apath,
                                   int32_t* bonus, hipStream_t s);
size_t verify_rejection_scratch_bytes(int B, int m);
hipError_t launch_static_build(const RoundArgs& a, int32_t* tokens, int32_t* parents, int32_t* depth,
                               int32_t* positions, uint8_t* mask, float* logscore, hipStream_t s);
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);
// one matrix W [N][K] (row-major, rows ld elements apart) into the packed
// tile layout; pair_hd > 0: q/k/v row grouping of rotation pairs for head_dim pair_hd
hipError_t launch_pack(const void* src, void* dst, int N, int K, int ld, int es, int pair_hd, hipStream_t s);
// token-projection table: tp[v][n] = sum_k embed[v][k] * fc_w[n][d + k] (fp32),
// from the row-major embed [V][d] and fc_w [d][2d]
hipError_t launch_tokproj(const void* embed, const void* fc_w, float* tp, int V, int d, int es, hipStream_t s);

}  // namespace eg

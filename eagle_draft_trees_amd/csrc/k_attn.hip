// Tree-masked attention of the draft decoder layer.
//
// Levels: a frontier row at depth L sits at position P-1+L and sees every
// prefix row plus the in-tree K/V of its ancestors and itself, never a sibling
// or cousin ([P1] "EAGLE 推测解码为什么比 Medusa 快？（含 EAGLE-2 动态草稿树）"
// §12 item 5: the mask looks only at ancestors; [P4] "投机解码：从eagle1到dflash"
// EAGLE-2 diagram: tree causal mask).  Extend: row i sees the prefix and
// extend rows 0..i, which the QKV epilogue has already appended to the cache
// ([P3] zdszero.github.io spec_medusa_eagle, "在 SGLang 里").  Tree verify (the
// target model's attention over the flattened tree, [P1] §6.2: one target
// forward with tree attention scores every node; [P4] EAGLE-2 diagram, stage
// two: a node sees only its ancestors and itself): the tree rows sit in the
// cache right after the prefix, and query i sees every prefix row plus tree
// row j iff mask[i][j] is set.
//
// One workgroup per (sequence, KV head, tile of 16 queries); the queries of a
// tile are (row, head of the GQA group) pairs.  Its waves split the keys in
// chunks of 16: the prefix rows first, then (levels) every in-tree slot of
// depths 1..L as extra keys, masked per query to that query's ancestors and
// itself.  Per chunk a wave
//   * computes the 16x16 score tile S^T = K Q^T on MFMA (bf16: q split into a
//     high and a low bf16 part, so the scores keep about 16 mantissa bits;
//     fp32: the fp32 MFMA), lane (g, q) holding keys 4g..4g+3 of query q;
//   * updates each query's running max and sum (online softmax);
//   * accumulates P V: bf16 on MFMA (16x16x16, keys as the contraction),
//     with the probabilities split into a high and a low bf16 part; fp32 on
//     the vector ALUs, each lane owning hd/64 output dimensions.
// The next chunk's K and V loads are in flight while a chunk computes.  The
// waves' partial (max, sum, output) meet in LDS and are combined in wave order
// (deterministic); there is no cross-workgroup step.  Scores 1/sqrt(hd) q.k.
//
// A workgroup has four or eight waves.  Every wave uses the same query operand,
// which sits in LDS and is read there at each chunk: held in registers it
// would take 32 per lane (bf16 hd 128) and leave room for only one workgroup
// per compute unit.  Four waves then fit three workgroups per compute unit,
// which pays when the launch has a few hundred workgroups (they all run at
// once instead of in rounds); eight waves keep more keys in flight per
// workgroup where the launch has one workgroup per compute unit or fewer, or
// many rounds of them.
#include "eagle_internal.h"

namespace eg {

constexpr int AT_MW = 4;      // waves per workgroup of the split merge
constexpr int AT_Q = 16;      // queries per workgroup (one MFMA tile)
constexpr int AT_C = 16;      // keys per chunk
constexpr int AT_MAXS = 8;    // key splits of one query tile at most

// What a lane loads of a chunk's 16 V rows: N loads, load u from key row
// key(u, g) at column col(lane).
//  * bf16 (P V on MFMA): lane (g, i) loads keys 4g..4g+3, each at the NT = hd/16
//    consecutive columns NT*i .. NT*i+NT-1.  Tile t of the product then takes
//    hd column NT*i + t as its row i, so element t of the four loads is the
//    lane's A operand for tile t, and the result row 4g+r of tile t is hd
//    column NT*(4g+r) + t: each lane ends with NT*4 consecutive columns.
//  * fp32 (P V on the vector ALUs): lane loads every key row at its hd/64
//    columns DPL*lane ...
template <typename T, int HD> struct AtV;
template <> struct AtV<bf16_t, 128> {
  static constexpr int N = 4;
  typedef uint4 raw;
  __device__ static int key(int u, int g) { return 4 * g + u; }
  __device__ static int col(int lane) { return 8 * (lane & 15); }
  __device__ static raw ld(const bf16_t* p) { return *(const uint4*)p; }
  __device__ static uint32_t el(raw v, int t) {  // 16-bit element t (t compile-time)
    const uint32_t d = (t >> 1) == 0 ? v.x : (t >> 1) == 1 ? v.y : (t >> 1) == 2 ? v.z : v.w;
    return (t & 1) ? d >> 16 : d & 0xFFFFu;
  }
};
template <> struct AtV<bf16_t, 64> {
  static constexpr int N = 4;
  typedef uint2 raw;
  __device__ static int key(int u, int g) { return 4 * g + u; }
  __device__ static int col(int lane) { return 4 * (lane & 15); }
  __device__ static raw ld(const bf16_t* p) { return *(const uint2*)p; }
  __device__ static uint32_t el(raw v, int t) {
    const uint32_t d = (t >> 1) == 0 ? v.x : v.y;
    return (t & 1) ? d >> 16 : d & 0xFFFFu;
  }
};
template <> struct AtV<float, 128> {
  static constexpr int N = AT_C;
  typedef float2 raw;
  __device__ static int key(int u, int) { return u; }
  __device__ static int col(int lane) { return 2 * lane; }
  __device__ static raw ld(const float* p) { return *(const float2*)p; }
  __device__ static void cvt(raw r, float* v) { v[0] = r.x; v[1] = r.y; }
};
template <> struct AtV<float, 64> {
  static constexpr int N = AT_C;
  typedef float raw;
  __device__ static int key(int u, int) { return u; }
  __device__ static int col(int lane) { return lane; }
  __device__ static raw ld(const float* p) { return *p; }
  __device__ static void cvt(raw r, float* v) { v[0] = r; }
};

// 16x16x16 bf16 product: lane (g, i) supplies A[i][4g..4g+3] and
// B[4g..4g+3][i] (four bf16 in two words), receives D[4g+r][i].
__device__ __forceinline__ f32x4_t mma16k16(uint2 a, uint2 b, f32x4_t c) {
  typedef short s16x4_t __attribute__((ext_vector_type(4)));
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                   __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
}

template <typename T, int HD, int W>
__global__ void __launch_bounds__(W * WAVE, W == 4 ? 3 : 2) k_attn(RoundArgs a, AttnPlan p) {
  constexpr int KS = El<T>::KSTEP;
  constexpr int PER = El<T>::PER16;
  constexpr int NKS = HD / KS;   // MFMA k-steps over the head dimension
  constexpr int DPL = HD / 64;   // output dimensions per lane in the fp32 P.V step
  constexpr bool MFPV = sizeof(T) == 2;  // P.V on MFMA
  constexpr int NT = HD / 16;    // MFMA tiles over the head dimension
  constexpr int OP = HD + 4;     // padded LDS row of a wave's partial output
  typedef AtV<T, HD> VV;
  constexpr int NV = VV::N;
  __shared__ __attribute__((aligned(16))) float sP[W][AT_Q][AT_C];  // fp32: this chunk's probabilities, per wave
  __shared__ float sAl[W][AT_Q];            // fp32: this chunk's rescale of the running output
  __shared__ float sM[W][AT_Q], sL[W][AT_Q];
  __shared__ __attribute__((aligned(16))) float sO[W][AT_Q][OP];
  __shared__ int sLim[AT_Q];
  __shared__ int sAnc[AT_Q][EAGLE_MAX_DEPTH];
  __shared__ uint8_t sMb[AT_Q][EAGLE_MAX_TREE];  // tree verify: the queries' mask rows
  // the query operand (its high and low parts) of every lane, the same for
  // every wave: read from LDS at each use instead of held in registers
  __shared__ __attribute__((aligned(16))) uint4 sQ[2][NKS][WAVE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int q = lane & 15, g = lane >> 4;
  // Block order.  Group gi = (sequence, KV head, split), split-major:
  // consecutive groups (which land on different XCDs) take the splits of one
  // KV head, so each XCD reads whole cache rows (every head of a row range)
  // instead of one head's 256-byte slice of rows.  Block b runs on XCD b % 8;
  // the query tiles of one group (GQA: several query heads share a KV head)
  // are blocks b, b+8, ... on that one XCD, so they read its K/V through that
  // XCD's L2 instead of once per XCD.  Blocks past the last group end here.
  const int xcd = blockIdx.x & 7, jx = blockIdx.x >> 3;
  const int gi = (jx / p.nqt) * 8 + xcd, qt = jx % p.nqt;
  if (gi >= a.B * a.Hkv * p.nsplit) return;
  const int split = gi % p.nsplit, bk = gi / p.nsplit, kvh = bk % a.Hkv, b = bk / a.Hkv;
  const int wg = bk * p.nqt + qt;
  const int q0 = qt * AT_Q;
  const int P = clamp_prefix(a.prefix_len[b], a);
  const bool level = a.mode == MODE_LEVEL, verify = a.mode == MODE_VERIFY;
  const int HDq = a.H * HD;

  // ---- per-query visibility: prefix limit and (levels) ancestor slots
  if (tid < AT_Q) {
    const int gq = q0 + tid;
    const int row = min(gq, p.nq - 1) / p.g;
    sLim[tid] = gq >= p.nq ? 0 : ((level || verify) ? P : P + row + 1);
    if (level) {  // the record's 16 ancestor slots in four 16-byte loads (all in flight together)
      const eagle_frontier_node& nd = a.frontier[((size_t)a.depth * a.B + b) * a.k + row];
      uint4 an[EAGLE_MAX_DEPTH / 4];
#pragma unroll
      for (int u = 0; u < EAGLE_MAX_DEPTH / 4; ++u) an[u] = ld16(&nd.anc[4 * u]);
#pragma unroll
      for (int dd = 0; dd < EAGLE_MAX_DEPTH; ++dd) {
        const uint4 v = an[dd / 4];
        const int s_ = (int)((dd & 3) == 0 ? v.x : (dd & 3) == 1 ? v.y : (dd & 3) == 2 ? v.z : v.w);
        sAnc[tid][dd] = (gq < p.nq && dd < a.depth) ? clamp_slot(s_, a.k) : -1;
      }
    }
  }
  // keys: Pv prefix rows (the widest limit in the tile), then ntree in-tree slots
  // (all wave-uniform; said so explicitly so that chunk indices and branches stay scalar)
  const int lastrow = (min(q0 + AT_Q, p.nq) - 1) / p.g;
  const int Pv = __builtin_amdgcn_readfirstlane(
      level ? P : verify ? min(P + a.m, a.max_prefix) : min(P + lastrow + 1, a.max_prefix));
  const int ntree = __builtin_amdgcn_readfirstlane(level ? a.depth * a.k : 0);
  const int cp = (Pv + AT_C - 1) / AT_C;
  const int nch = cp + (ntree + AT_C - 1) / AT_C;
  // this split's chunks [c0, c1) (splits of one tile merge in k_attn_merge)
  const int cps = (nch + p.nsplit - 1) / p.nsplit;
  const int c0 = split * cps, c1 = min(nch, c0 + cps);
  const size_t rs = (size_t)a.Hkv * HD;  // stride between key rows of the cache
  const T* Kp = (const T*)a.k_cache + ((size_t)b * a.max_prefix * a.Hkv + kvh) * HD;
  const T* Vp = (const T*)a.v_cache + ((size_t)b * a.max_prefix * a.Hkv + kvh) * HD;
  const T* Kt = (const T*)a.tk;
  const T* Vt = (const T*)a.tv;
  // row of key i of chunk c (clamped to a valid row; masked later)
  auto krow = [&](const T* prefix, const T* tree, int c, int i) __attribute__((always_inline)) -> const T* {
    if (c < cp) return prefix + (size_t)min(c * AT_C + i, Pv - 1) * rs;
    int t = (c - cp) * AT_C + i;
    t = t < ntree ? t : 0;
    const int dep = t / a.k + 1, slot = t - (dep - 1) * a.k;
    return tree + ((((size_t)b * a.D + dep) * a.k + slot) * a.Hkv + kvh) * HD;
  };

  // the first chunk's K/V loads go out now, ahead of the query setup
  typedef typename VV::raw vraw;
  const int cl = sizeof(T) == 2 ? min(c1, cp) : c1;  // end of the ping-pong range
  const int vcol = VV::col(lane);
  auto load = [&](uint4 (&kr)[NKS], vraw (&vr)[NV], int c) __attribute__((always_inline)) {
    c = min(c, cl - 1);  // past the range's last chunk: repeat it (unused)
    if (sizeof(T) == 2 || c < cp) {  // consecutive prefix rows; the last chunk's tail repeats row Pv-1
      const int r0 = c * AT_C, rmax = Pv - 1 - r0;
      const T* kp = Kp + (size_t)(r0 + min(q, rmax)) * rs;
#pragma unroll
      for (int s = 0; s < NKS; ++s) kr[s] = ld16(kp + s * KS + g * PER);
#pragma unroll
      for (int u = 0; u < NV; ++u) vr[u] = VV::ld(Vp + (size_t)(r0 + min(VV::key(u, g), rmax)) * rs + vcol);
    } else {
      const T* kp = krow(Kp, Kt, c, q);
#pragma unroll
      for (int s = 0; s < NKS; ++s) kr[s] = ld16(kp + s * KS + g * PER);
#pragma unroll
      for (int u = 0; u < NV; ++u) vr[u] = VV::ld(krow(Vp, Vt, c, VV::key(u, g)) + vcol);
    }
  };

  // this wave's chunks: c0+w, c0+w+W, ... below cl (a wave-uniform count);
  // the first is in flight before the query setup.  bf16: cl ends the prefix
  // chunks, and the wave's in-tree chunks (same stride) follow one by one.
  uint4 ka[NKS], kb[NKS];
  vraw va[NV], vb[NV];
  const int nmine = __builtin_amdgcn_readfirstlane(c0 + w < cl ? (cl - 1 - c0 - w) / W + 1 : 0);
  if (nmine >= 1) load(ka, va, c0 + w);

  // ---- this lane's query operand (query q0+q, dims of k-step s for lane group g),
  // pre-scaled by 1/sqrt(hd); bf16 keeps a high and a low part
  const float scale = rsqrtf((float)HD);
  if (w == 0) {
    const int gq = min(q0 + q, p.nq - 1);
    const bool qv = q0 + q < p.nq;
    const int row = b * p.RS + gq / p.g, head = kvh * p.g + gq % p.g;
    const float* qp = a.q + ((size_t)row * a.H + head) * HD;
    const float qs = qv ? scale : 0.f;  // padding queries: zero (their rows are never written)
    float4 qx[NKS][PER / 4];
#pragma unroll
    for (int s = 0; s < NKS; ++s)
#pragma unroll
      for (int u = 0; u < PER / 4; ++u) qx[s][u] = *(const float4*)(qp + s * KS + g * PER + 4 * u);
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      float x[PER];
#pragma unroll
      for (int u = 0; u < PER / 4; ++u) {
        x[4 * u] = qx[s][u].x * qs;
        x[4 * u + 1] = qx[s][u].y * qs;
        x[4 * u + 2] = qx[s][u].z * qs;
        x[4 * u + 3] = qx[s][u].w * qs;
      }
      if constexpr (sizeof(T) == 2) {
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t h0 = f2bf(x[2 * e]), h1 = f2bf(x[2 * e + 1]);
          const uint32_t l0 = f2bf(x[2 * e] - bf2f(h0)), l1 = f2bf(x[2 * e + 1] - bf2f(h1));
          hw[e] = h0 | (h1 << 16);
          lw[e] = l0 | (l1 << 16);
        }
        sQ[0][s][lane] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        sQ[1][s][lane] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      } else {
        sQ[0][s][lane] = make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                           __float_as_uint(x[3]));
        sQ[1][s][lane] = make_uint4(0, 0, 0, 0);
      }
    }
  }
  // tree verify: the tile's mask rows, one byte per thread (padding queries
  // see no tree row)
  if (verify) {
    for (int idx = tid; idx < AT_Q * a.m; idx += W * WAVE) {
      const int qq = idx / a.m, j = idx - qq * a.m, gq = q0 + qq;
      const int row = min(gq, p.nq - 1) / p.g;
      sMb[qq][j] = gq < p.nq ? a.vmask[((size_t)b * a.m + row) * a.m + j] : (uint8_t)0;
    }
  }
  __syncthreads();

  // running softmax state of query q (replicated over the lane groups) and
  // this lane's output dimensions for all 16 queries
  float m = -INFINITY, l = 0.f;
  // bf16: query q's output at columns NT*(4g+r)+t in accm[t][r];
  // fp32: this lane's DPL columns of every query in acc
  f32x4_t accm[MFPV ? NT : 1];
  float acc[MFPV ? 1 : AT_Q][DPL];
#pragma unroll
  for (int t = 0; t < (MFPV ? NT : 1); ++t) accm[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < (MFPV ? 1 : AT_Q); ++i)
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[i][e] = 0.f;

  // masking and the online-softmax update of one chunk's scores: lane (g, q)
  // holds S^T[4g + r][q]; returns this chunk's rescale of the running output
  // and the lane's four probabilities
  auto smax = [&](const f32x4_t& st, int c, float& al, float (&pr4)[4]) __attribute__((always_inline)) {
    float sc[4];
    float cmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * g + r;
      bool vis;
      if (c < cp) {
        const int key = c * AT_C + i;
        vis = key < sLim[q];
        if (verify) {  // a tree row: its entry in the query's mask row
          const unsigned j = (unsigned)(key - P);
          vis = vis || (j < (unsigned)a.m && sMb[q][j] != 0);
        }
      } else {
        const int t = (c - cp) * AT_C + i;
        const int dep = min(t / a.k + 1, EAGLE_MAX_DEPTH), slot = t - (dep - 1) * a.k;
        vis = t < ntree && q0 + q < p.nq && sAnc[q][dep - 1] == slot;
      }
      sc[r] = vis ? st[r] : -INFINITY;
      cmax = fmaxf(cmax, sc[r]);
    }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    const float mnew = fmaxf(m, cmax);
    al = (m == -INFINITY) ? 0.f : expf(m - mnew);
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr4[r] = sc[r] == -INFINITY ? 0.f : expf(sc[r] - mnew);
      ps += pr4[r];
    }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    l = l * al + ps;
    m = mnew;
  };
  // lane (g, q) holds query q's probabilities of keys 4g..4g+3: the B operand
  // of the 16x16x16 P.V product as it stands; a high and a low bf16 part keep
  // about 16 bits of each probability
  auto psplit = [&](const float (&pr4)[4], uint2& bh, uint2& bl) __attribute__((always_inline)) {
    uint32_t h[4], lo[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      h[r] = f2bf(pr4[r]);
      lo[r] = f2bf(pr4[r] - bf2f(h[r]));
    }
    bh = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    bl = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
  };

  // the query operand in LDS, read through a lane index the compiler must
  // treat as new at every chunk (so that it reads LDS there rather than keep
  // the operand in registers across the loop)
  auto qlane = [&]() __attribute__((always_inline)) {
    int ql = lane;
    asm volatile("" : "+v"(ql));
    return ql;
  };
  auto chunk = [&](const uint4 (&kr)[NKS], const vraw (&vr)[NV], int c) __attribute__((always_inline)) {
    const int ql = qlane();
    // scores: lane (g, q) gets S^T[4g + r][q], r = 0..3
    f32x4_t st = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      st = mma16(kr[s], sQ[0][s][ql], st, T());
      if constexpr (sizeof(T) == 2) st = mma16(kr[s], sQ[1][s][ql], st, T());
    }
    float al, pr4[4];
    smax(st, c, al, pr4);
    if constexpr (MFPV) {
      // V is exact in bf16
      uint2 bh, bl;
      psplit(pr4, bh, bl);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const uint2 av = make_uint2(VV::el(vr[0], t) | (VV::el(vr[1], t) << 16),
                                    VV::el(vr[2], t) | (VV::el(vr[3], t) << 16));
        f32x4_t o = accm[t] * al;
        o = mma16k16(av, bh, o);
        accm[t] = mma16k16(av, bl, o);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) sP[w][q][4 * g + r] = pr4[r];
      if (g == 0) sAl[w][q] = al;
      __builtin_amdgcn_wave_barrier();  // the wave's LDS writes before its reads
      // P.V: this lane's output dimensions, every query of the tile
      float v[AT_C][DPL];
#pragma unroll
      for (int j = 0; j < AT_C; ++j) VV::cvt(vr[j], v[j]);
#pragma unroll
      for (int i = 0; i < AT_Q; ++i) {
        const float ai = sAl[w][i];
        float pr[AT_C];  // the query's 16 probabilities: four aligned 16-byte broadcast reads
#pragma unroll
        for (int u = 0; u < AT_C / 4; ++u) {
          const float4 f = *(const float4*)&sP[w][i][4 * u];
          pr[4 * u] = f.x;
          pr[4 * u + 1] = f.y;
          pr[4 * u + 2] = f.z;
          pr[4 * u + 3] = f.w;
        }
        float o[DPL];
#pragma unroll
        for (int e = 0; e < DPL; ++e) o[e] = acc[i][e] * ai;
#pragma unroll
        for (int j = 0; j < AT_C; ++j)
#pragma unroll
          for (int e = 0; e < DPL; ++e) o[e] += pr[j] * v[j][e];
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[i][e] = o[e];
      }
      __builtin_amdgcn_wave_barrier();  // reads done before the next chunk's writes
    }
  };

  // bf16: an in-tree chunk.  The in-tree K/V are fp32; each is split into a
  // high and a low bf16 part, and the products keep the three significant
  // terms (hi.hi, hi.lo, lo.hi) of both the scores and P.V.
  auto tchunk = [&](int c) __attribute__((always_inline)) {
    const int ql = qlane();
    const float* KtF = (const float*)a.tk;
    const float* VtF = (const float*)a.tv;
    auto trow = [&](const float* tree, int i) __attribute__((always_inline)) -> const float* {
      int t = (c - cp) * AT_C + i;
      t = t < ntree ? t : 0;
      const int dep = t / a.k + 1, slot = t - (dep - 1) * a.k;
      return tree + ((((size_t)b * a.D + dep) * a.k + slot) * a.Hkv + kvh) * HD;
    };
    auto split8 = [&](const float4& x0, const float4& x1, uint4& hi, uint4& lo) __attribute__((always_inline)) {
      const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t h0 = f2bf(x[2 * e]), h1 = f2bf(x[2 * e + 1]);
        hw[e] = h0 | (h1 << 16);
        lw[e] = f2bf(x[2 * e] - bf2f(h0)) | (f2bf(x[2 * e + 1] - bf2f(h1)) << 16);
      }
      hi = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      lo = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    };
    // loads first: the key row of lane column q, and V rows 4g..4g+3 at the lane's NT columns
    const float* kp = trow(KtF, q);
    float4 kx[NKS][2];
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      kx[s][0] = *(const float4*)(kp + s * KS + g * PER);
      kx[s][1] = *(const float4*)(kp + s * KS + g * PER + 4);
    }
    float vx[4][NT];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float* vp = trow(VtF, 4 * g + u) + vcol;
#pragma unroll
      for (int t = 0; t < NT; t += 4) {
        const float4 f = *(const float4*)(vp + t);
        vx[u][t] = f.x;
        vx[u][t + 1] = f.y;
        vx[u][t + 2] = f.z;
        vx[u][t + 3] = f.w;
      }
    }
    f32x4_t st = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      uint4 kh, kl;
      split8(kx[s][0], kx[s][1], kh, kl);
      const uint4 qhs = sQ[0][s][ql], qls = sQ[1][s][ql];
      st = mma16(kh, qhs, st, T());
      st = mma16(kh, qls, st, T());
      st = mma16(kl, qhs, st, T());
    }
    float al, pr4[4];
    smax(st, c, al, pr4);
    uint2 bh, bl;
    psplit(pr4, bh, bl);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      uint32_t vh[4], vl[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        vh[u] = f2bf(vx[u][t]);
        vl[u] = f2bf(vx[u][t] - bf2f(vh[u]));
      }
      const uint2 ah = make_uint2(vh[0] | (vh[1] << 16), vh[2] | (vh[3] << 16));
      const uint2 alo = make_uint2(vl[0] | (vl[1] << 16), vl[2] | (vl[3] << 16));
      f32x4_t o = accm[t] * al;
      o = mma16k16(ah, bh, o);
      o = mma16k16(ah, bl, o);
      accm[t] = mma16k16(alo, bh, o);
    }
  };

  // two chunks in flight (ping-pong register sets).  The loop body is
  // branch-free with a wave-uniform trip count, so that the wait for a set's
  // loads sits at its first use (an exit between the halves made the compiler
  // wait for the other set before issuing the next loads).  A load past the
  // wave's last chunk repeats the range's last chunk: unused, or taken by the
  // odd chunk after the loop.
  if constexpr (sizeof(T) == 2) {
    int c = c0 + w;
    const int npair = nmine >> 1;
    for (int i = 0; i < npair; ++i, c += 2 * W) {
      load(kb, vb, c + W);
      __builtin_amdgcn_sched_barrier(0);
      chunk(ka, va, c);
      load(ka, va, c + 2 * W);
      __builtin_amdgcn_sched_barrier(0);
      chunk(kb, vb, c + W);
    }
    if (nmine & 1) chunk(ka, va, c);
  } else if (nmine == 1) {
    // fp32 (sixteen V rows per chunk in registers): with the loop above the
    // compiler spills, so the halves keep their own exits here
    chunk(ka, va, c0 + w);
  } else if (nmine > 1) {
    for (int c = c0 + w;; c += 2 * W) {
      load(kb, vb, c + W);
      __builtin_amdgcn_sched_barrier(0);
      chunk(ka, va, c);
      if (c + W >= cl) break;
      load(ka, va, c + 2 * W);
      __builtin_amdgcn_sched_barrier(0);
      chunk(kb, vb, c + W);
      if (c + 2 * W >= cl) break;
    }
  }
  if constexpr (sizeof(T) == 2) {  // this wave's in-tree chunks, c ≡ c0 + w (mod W)
    const int f = max(c0, cp);
    for (int c = f + ((c0 + w - f) % W + W) % W; c < c1; c += W) tchunk(c);
  }

  // ---- combine the waves' partial results in wave order
  if (g == 0) {
    sM[w][q] = m;
    sL[w][q] = l;
  }
  if constexpr (MFPV) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {  // NT consecutive columns per r
      float* dst = &sO[w][q][NT * (4 * g + r)];
#pragma unroll
      for (int t = 0; t < NT; t += 4)
        *(float4*)(dst + t) = make_float4(accm[t][r], accm[t + 1][r], accm[t + 2][r], accm[t + 3][r]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < AT_Q; ++i)
#pragma unroll
      for (int e = 0; e < DPL; ++e) sO[w][i][lane * DPL + e] = acc[i][e];
  }
  __syncthreads();
  {
    // W*WAVE/AT_Q threads per query: each weighs the waves itself (max over waves that
    // saw a key, then exp(m_w - M)) and sums its DPT columns in wave order
    constexpr int TPQ = W * WAVE / AT_Q;
    constexpr int DPT = HD / TPQ;
    const int i = tid / TPQ, d0 = (tid % TPQ) * DPT, gq = q0 + i;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < W; ++ww)
      if (sL[ww][i] > 0.f) M = fmaxf(M, sM[ww][i]);
    float L = 0.f, O[DPT];
#pragma unroll
    for (int e = 0; e < DPT; ++e) O[e] = 0.f;
#pragma unroll
    for (int ww = 0; ww < W; ++ww) {
      const float lw = sL[ww][i];
      const float wt = lw > 0.f ? expf(sM[ww][i] - M) : 0.f;
      L += lw * wt;
#pragma unroll
      for (int e = 0; e < DPT; ++e) O[e] += wt * sO[ww][i][d0 + e];
    }
    if (p.nsplit == 1) {
      if (gq < p.nq) {
        const float inv = L > 0.f ? 1.0f / L : 0.f;
        const int row = b * p.RS + gq / p.g, head = kvh * p.g + gq % p.g;
        const size_t o = (size_t)row * HDq + head * HD + d0;
#pragma unroll
        for (int e = 0; e < DPT; ++e) El<T>::st((T*)a.attn, o + e, O[e] * inv);
      }
    } else {
      // partial of this split, per query: unnormalised output, then max and sum
      float* part = a.apart + (((size_t)wg * p.nsplit + split) * AT_Q + i) * (HD + 4);
#pragma unroll
      for (int e = 0; e < DPT; ++e) part[d0 + e] = O[e];
      if (tid % TPQ == 0) {
        part[HD] = M;
        part[HD + 1] = L;
      }
    }
  }
}

// Combine the key splits of each (sequence, KV head, query tile) in split
// order: softmax-weighted sum of the splits' unnormalised outputs.  Every load
// is issued up front (clamped, masked), so the kernel waits once.
template <typename T, int HD>
__global__ void __launch_bounds__(AT_MW * WAVE) k_attn_merge(RoundArgs a, AttnPlan p) {
  constexpr int PT = AT_Q * HD / (AT_MW * WAVE);  // outputs per thread
  __shared__ float sW[AT_MAXS][AT_Q], sInv[AT_Q];
  const int tid = threadIdx.x, wg = blockIdx.x;
  const int qt = wg % p.nqt, bk = wg / p.nqt, kvh = bk % a.Hkv, b = bk / a.Hkv;
  const int q0 = qt * AT_Q;
  const int ns = p.nsplit;
  const float* part = a.apart + (size_t)wg * ns * AT_Q * (HD + 4);
  float ov[PT][AT_MAXS];
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int idx = tid + u * AT_MW * WAVE, i = idx / HD, dd = idx - i * HD;
#pragma unroll
    for (int s = 0; s < AT_MAXS; ++s)
      ov[u][s] = part[((size_t)min(s, ns - 1) * AT_Q + i) * (HD + 4) + dd];
  }
  if (tid < AT_Q) {
    float mm[AT_MAXS], ll[AT_MAXS];
#pragma unroll
    for (int s = 0; s < AT_MAXS; ++s) {
      const float* ps = part + ((size_t)min(s, ns - 1) * AT_Q + tid) * (HD + 4);
      mm[s] = ps[HD];
      ll[s] = s < ns ? ps[HD + 1] : 0.f;
    }
    float M = -INFINITY;
#pragma unroll
    for (int s = 0; s < AT_MAXS; ++s)
      if (ll[s] > 0.f) M = fmaxf(M, mm[s]);
    float L = 0.f;
#pragma unroll
    for (int s = 0; s < AT_MAXS; ++s) {
      const float wt = ll[s] > 0.f ? expf(mm[s] - M) : 0.f;
      sW[s][tid] = wt;
      L += ll[s] * wt;
    }
    sInv[tid] = L > 0.f ? 1.0f / L : 0.f;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < PT; ++u) {
    const int idx = tid + u * AT_MW * WAVE, i = idx / HD, dd = idx - i * HD, gq = q0 + i;
    float O = 0.f;
#pragma unroll
    for (int s = 0; s < AT_MAXS; ++s) O += sW[s][i] * ov[u][s];  // weight 0 past ns
    if (gq >= p.nq) continue;
    const int row = b * p.RS + gq / p.g, head = kvh * p.g + gq % p.g;
    El<T>::st((T*)a.attn, (size_t)row * (a.H * HD) + head * HD + dd, O * sInv[i]);
  }
}

template <typename T, int HD>
static hipError_t launch_attn_t(const RoundArgs& a, const AttnPlan& p, hipStream_t s) {
  const int tiles = a.B * a.Hkv * p.nqt, groups = a.B * a.Hkv * p.nsplit;
  const dim3 grid((groups + 7) / 8 * 8 * p.nqt);
  if (p.waves == 4)
    hipLaunchKernelGGL((k_attn<T, HD, 4>), grid, dim3(4 * WAVE), 0, s, a, p);
  else if (p.waves == 8)
    hipLaunchKernelGGL((k_attn<T, HD, 8>), grid, dim3(8 * WAVE), 0, s, a, p);
  else
    return hipErrorInvalidValue;
  if (p.nsplit > 1) hipLaunchKernelGGL((k_attn_merge<T, HD>), dim3(tiles), dim3(AT_MW * WAVE), 0, s, a, p);
  return hipGetLastError();
}

hipError_t launch_attn(const RoundArgs& a, const AttnPlan& p, hipStream_t s) {
  if (a.dtype == EAGLE_BF16) return a.hd == 128 ? launch_attn_t<bf16_t, 128>(a, p, s) : launch_attn_t<bf16_t, 64>(a, p, s);
  return a.hd == 128 ? launch_attn_t<float, 128>(a, p, s) : launch_attn_t<float, 64>(a, p, s);
}

}  // namespace eg

// Host side of the C ABI: argument validation (before any launch), workspace
// layout, launch plans and the round's entry points.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "skinny_core.h"

namespace eg {

static thread_local char g_err[512] = "";

static int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
static inline int cdiv(int a, int b) { return (a + b - 1) / b; }

size_t elem_size(const eagle_dims& d) { return d.dtype == EAGLE_BF16 ? 2 : 4; }

static constexpr size_t SK_XLDS_MAX = 140 * 1024;  // LDS for a staged X tile (of 160 KB per CU)

// Layer GEMMs at more than 16 rows (the extend, wide frontiers): 64 output
// columns per workgroup over its whole K range (X streamed through LDS in
// chunks); K is split across workgroups only to cover the compute units.
GemmPlan plan_gemm(int op, int M, const eagle_dims& d) {
  GemmPlan p{};
  p.M = M;
  p.nw = 1;
  switch (op) {
    case OP_FC: p.N = d.d; p.K = d.d; break;  // the feature half (the token half is tabulated)
    case OP_QKV: p.N = (d.n_heads + 2 * d.n_kv_heads) * d.head_dim; p.K = d.d; break;
    case OP_O: p.N = d.d; p.K = d.n_heads * d.head_dim; break;
    case OP_GATEUP: p.N = d.ffn; p.K = d.d; p.nw = 2; break;
    default: p.N = d.d; p.K = d.ffn; break;
  }
  p.mt = std::min(4, cdiv(std::min(M, 64), 16));
  p.zg = cdiv(M, 64);
  p.ct = 4;
  p.nblk = cdiv(p.N, 64);
  p.hl = op == OP_QKV && d.dtype == EAGLE_BF16;
  const int kc = gemm_kc(p.nw, (int)elem_size(d), p.hl);
  // K is split across workgroups only when the column blocks alone leave
  // more than half of the compute units idle; a split keeps two chunks or more
  const int base = p.nblk * p.zg;
  int S = 1;
  if (base < 128) {
    S = std::max(1, std::min(cdiv(256, base), cdiv(p.K, 2 * kc)));
  } else if (op != OP_O) {
    // unsplit: three column tiles per workgroup when that leaves fewer of the
    // 256 compute units idle in the launch's last round of workgroups (the O
    // launch keeps four: its blocks define the RMSNorm partials gate/up reads)
    auto idle = [](int wgs) { return cdiv(wgs, 256) * 256 - wgs; };
    const int n3 = cdiv(cdiv(p.N, 16), 3);
    if (cdiv(n3 * p.zg, 256) <= cdiv(base, 256) && idle(n3 * p.zg) < idle(base)) {
      p.ct = 3;
      p.nblk = n3;
    }
  }
  p.Kc = cdiv(cdiv(p.K, S), kc) * kc;
  p.S = cdiv(p.K, p.Kc);
  p.nps = op == OP_GATEUP ? cdiv(d.d, 64) : 0;
  p.part_floats = p.S > 1 ? (size_t)p.nblk * p.zg * p.S * 4 * p.nw * p.mt * 256 : 0;
  // Many rows (bf16): 256 x 256 MFMA tiles (gate/up: 128 output columns of
  // gate and up), K split into ranges of whole 4-step groups until the tiles
  // about fill the 256 compute units; the partials always go through
  // k_gemm_fin, which runs the epilogue.  Taken unless the split ranges
  // would be short (under 32 k-steps): their fp32 partials then cost more
  // than the skinny path's weight re-reads (o and fc at 512 rows x d 4096).
  if (d.dtype == EAGLE_BF16 && M > 64 && p.K % 128 == 0) {
    const int nsx = (p.hl ? 2 : 1) * p.K / 32;
    const int tiles = cdiv(p.N, op == OP_GATEUP ? 128 : 256) * cdiv(M, 256);
    const int S = std::max(1, std::min({256 / tiles, nsx / 16, GEMM_MAXS}));
    const int tks = cdiv(cdiv(nsx, S), 4) * 4;
    if (S == 1 || tks >= 32) {
      p.tiled = 1;
      p.tks = tks;
      p.S = cdiv(nsx, tks);
      p.Kc = tks * 32;
      p.mt = 4;
      p.zg = cdiv(M, 64);
      p.ct = 4;
      p.nblk = cdiv(p.N, 64);
      p.part_floats = (size_t)p.nblk * p.zg * p.S * 4 * p.nw * p.mt * 256;
    }
  }
  // 17..64 rows (bf16), O and down, and FC where k_gemm would split K: the
  // streaming kernel, 128*nq columns per workgroup, nq the smallest that
  // keeps the column blocks to about one workgroup per compute unit; when they
  // number under 128, K split so that the workgroups about fill the compute
  // units.  Partials go through k_gemm_fin, which runs the epilogue.  q/k/v,
  // gate/up and an unsplit FC stay on k_gemm: there they need no finishing
  // launch, and at one weight tile per wave the streaming kernel's
  // row-gathered X loads cost about what its split saves (measured at 40 and
  // 64 rows, d 4096-8192).
  if (!p.tiled && d.dtype == EAGLE_BF16 && M >= 17 && M <= 64 && p.K % 256 == 0 &&
      (op == OP_O || op == OP_DOWN || (op == OP_FC && p.S > 1))) {
    const int ntile = cdiv(p.N, 16), nks = p.K / 32;
    const int nwg1 = cdiv(ntile, 8);
    int nq = 1, S = 1;
    if (nwg1 >= 128) {
      nq = std::min(4, cdiv(nwg1, 256));
      if (nq == 3) nq = 4;
    } else {
      S = std::max(1, std::min({256 / nwg1, nks / 16, GEMM_MAXS}));
    }
    const int U = nq == 1 ? 8 : 4;  // k-steps per loop iteration
    p.rows = 1;
    p.nq = nq;
    // the kernel deals the K range's nks/U iterations over the S splits as
    // evenly as whole iterations allow
    p.S = std::min(S, nks / U);
    p.tks = cdiv(nks / U, p.S) * U;  // the longest split
    p.Kc = p.tks * 32;
    p.mt = cdiv(M, 16);
    p.zg = 1;
    p.ct = 4;
    p.nblk = cdiv(p.N, 64);
    p.part_floats = (size_t)p.nblk * p.S * 4 * p.mt * 256;
  }
  return p;
}

// Level GEMMs (at most 16 rows): about one workgroup per compute unit, each
// with up to 16 waves that split K; column tiles per workgroup grow with N.
SkPlan plan_skinny(int op, int M, const eagle_dims& d) {
  SkPlan p{};
  const GemmPlan g = plan_gemm(op, M, d);
  p.M = M;
  p.N = g.N;
  p.K = g.K;
  p.ntile = cdiv(p.N, 16);
  p.CT = std::max(1, std::min(SK_MAXW, cdiv(p.ntile, 256)));
  const int nks = cdiv(p.K, d.dtype == EAGLE_BF16 ? 32 : 16);
  const int nw = op == OP_GATEUP ? 2 : 1;
  // one column tile per workgroup: all 16 waves split K (every CU busy);
  // several tiles: fewer, longer K slices (at least 32 k-steps; gate/up, two
  // weight streams per wave, at least 25) stream better.  Measured at the
  // 7B shape's gate/up (3 tiles, 128 k-steps): 5 slices 33.4 us, 4 slices
  // 34.3; its q/k/v with 5 slices (15 waves) took 25.6 us against 22.0.
  const int maxw = op == OP_QKV ? SK_QKVW : SK_MAXW;
  p.CT = std::min(p.CT, maxw);
  p.KSW = p.CT == 1 ? std::max(1, std::min(maxw, nks / 8))
                    : std::max(1, std::min(maxw / p.CT, nks / (op == OP_GATEUP ? 25 : 32)));
  p.nwg = cdiv(p.ntile, p.CT);
  p.nps = 0;
  // the X tile is staged in LDS when it fits and is shared by at least two
  // weight streams (with one, staging costs as much as it saves)
  // (not the FC, whose X rows are gathered from two sources)
  // (not the down projection either: its X, the SwiGLU activations, is stored
  // packed, one contiguous kilobyte per k-step, and is read from L2 directly)
  // (the bf16 q/k/v projection stages both parts of x0, in two K phases)
  const size_t xt = op == OP_QKV && d.dtype == EAGLE_BF16 ? sk_hl_tile_bytes(p.K, 2)
                                                          : sk_xtile_bytes(p.K, (int)elem_size(d));
  p.xlds = op != OP_FC && op != OP_DOWN && p.CT * nw >= 2 && xt <= SK_XLDS_MAX;
  return p;
}

static inline bool use_skinny(int mode, int rows) {
  return (mode == MODE_LEVEL || mode == MODE_EXTEND) && rows <= 16;
}

// compute units of the current device (cached per device ordinal; 256 when
// the query fails)
static int device_cus() {
  static std::mutex mu;
  static int cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lk(mu);
  if (!cus[dev]) {
    int n = 0;
    cus[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : 256;
  }
  return cus[dev];
}

// FC hand-over (levels of at most 16 rows): level L's merge launch computes
// the FC of level L+1.  Returns false when the configuration keeps the FC in
// each level's own call.  *fp: the FC plan over the M rows of level L (B at
// level 1, B*k after), its waves raised to cover the merge's.  Its workgroups
// wait for the merges, so all of them and the merges must be resident at
// once: one workgroup per compute unit at most (a workgroup of that many
// waves fills one), more column tiles per workgroup where needed.
static bool handover_plan(const eagle_dims& d, const eagle_tree_cfg& c, int level, SkPlan* fp) {
  const int R = c.batch * c.topk;
  if (R > 16) return false;
  const int M = level == 1 ? c.batch : R;
  SkPlan p = plan_skinny(OP_FC, M, d);
  const int nseq = c.batch, ncu = device_cus();
  if (nseq + p.nwg > ncu) {
    while (p.CT < SK_MAXW && nseq + cdiv(p.ntile, p.CT) > ncu) ++p.CT;
    p.KSW = SK_MAXW / p.CT;  // every wave the compute unit holds: the K slices stay short
    p.nwg = cdiv(p.ntile, p.CT);
    if (nseq + p.nwg > ncu) return false;
  }
  const int mwaves = level == 1 ? 1 : c.topk;  // merge waves of the launch
  const int ksw = std::max(p.KSW, cdiv(mwaves, p.CT));
  if (p.CT * ksw > SK_MAXW) return false;
  p.KSW = ksw;
  if (fp) *fp = p;
  return true;
}

LmPlan plan_lm(int M, const eagle_dims& d, int topk) {
  LmPlan p{};
  p.M = M;
  p.mt = std::min(4, cdiv(std::min(M, 64), 16));
  p.zg = cdiv(M, 64);
  p.sk = M <= 16;
  if (p.sk) {  // slabs of CT*16 columns, about one workgroup per compute unit
    const int ntile = cdiv(d.vocab, 16);
    const int nks = cdiv(d.d, d.dtype == EAGLE_BF16 ? 32 : 16);
    p.CT = std::max(1, std::min(SK_MAXW, cdiv(ntile, 256)));
    p.KSW = std::max(1, std::min(SK_MAXW / p.CT, nks / 32));
    p.nblk = cdiv(ntile, p.CT);
    p.xlds = p.CT >= 2 && sk_xtile_bytes(d.d, (int)elem_size(d)) <= SK_XLDS_MAX;
  } else {
    p.nblk = cdiv(d.vocab, 64);
    p.big = d.dtype == EAGLE_BF16 && M > 64 && d.d % 128 == 0;
    if (p.big) p.zg = cdiv(M, lmgemm_rows());
    // 17..64 rows: the streaming kernel, 128 * nq columns per workgroup with
    // nq the smallest that keeps the workgroups to about one per compute unit
    // (k-steps a multiple of the loop's unroll).  With one weight tile per wave
    // (vocabularies up to 32768) only above 48 rows: there every one of the
    // four 16-row MFMA tiles is in use and it beat k_lmhead (13B shape, 64 rows
    // x d 5120, X packed by the down epilogue: 82 vs 93 us); at 40 rows x d
    // 8192 it measured slower (146-152 vs 106 us).
    if (d.dtype == EAGLE_BF16 && M <= 64 && d.d % 128 == 0) {
      const int nq = std::min(4, cdiv(cdiv(d.vocab, 16), 8 * 256));
      if ((nq >= 2 || M > 48) && d.d % (32 * (nq == 1 ? 8 : 4)) == 0) p.nq = nq;
    }
  }
  p.rec = 2 + 2 * topk;
  p.part_floats = (size_t)M * p.nblk * p.rec;
  return p;
}

// Attention: one workgroup per (sequence, KV head, 16-query tile); when those
// are fewer than about 256 the keys are split further (at least 4 chunks of 16
// keys per split) so that every compute unit streams part of the KV.
AttnPlan plan_attn(int mode, int RS, const eagle_dims& d, const eagle_tree_cfg& c, int nseq) {
  AttnPlan p{};
  p.RS = RS;
  p.g = d.n_heads / d.n_kv_heads;
  p.nq = RS * p.g;
  p.nqt = cdiv(p.nq, 16);
  const int tiles = nseq * d.n_kv_heads * p.nqt;
  const int keys = c.max_prefix + (mode == MODE_LEVEL ? c.depth * c.topk : 0);
  const int chunks = cdiv(keys, 16);
  p.nsplit = std::max(1, std::min({8, cdiv(256, tiles), std::max(1, chunks / 4)}));
  p.part_floats = p.nsplit > 1 ? (size_t)tiles * p.nsplit * 16 * (d.head_dim + 4) : 0;
  // four-wave workgroups (three per compute unit) when the launch fits in one
  // such round but not in one of eight-wave workgroups
  const int wgs = tiles * p.nsplit;
  p.waves = wgs > 256 && wgs <= 768 ? 4 : 8;
  return p;
}

WsLayout plan_ws(const eagle_dims& d, const eagle_tree_cfg& c) {
  WsLayout L{};
  const size_t es = elem_size(d);
  const int B = c.batch, k = c.topk, D = c.depth, m = c.m;
  const int re = ext_rows(m, D), rows_lv = B * k, rows_ex = B * re;
  L.rows_max = std::max(std::max(rows_lv, rows_ex), B);
  L.pool_n = k + (D - 1) * k * k;
  const size_t R = L.rows_max, HD = (size_t)d.n_heads * d.head_dim;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  };
  L.err = take(16);
  L.cnt = take((size_t)NCNT * 4);
  L.pool = take((size_t)B * L.pool_n * sizeof(eagle_pool_entry));
  L.frontier = take((size_t)(D + 1) * B * k * sizeof(eagle_frontier_node));
  L.feat = take((size_t)D * B * k * d.d * es);
  // in-tree K/V in fp32: their scores reach the thousands at deep levels,
  // where a bf16 rounding of a key moves the softmax
  const size_t kvt = (size_t)B * D * k * d.n_kv_heads * d.head_dim * 4;
  L.tk = take(kvt);
  L.tv = take(kvt);
  L.ext_h = take((size_t)rows_ex * d.d * es);
  L.x0f = take(R * d.d * 4);
  L.x0b = take(R * d.d * es);
  L.x0l = take(R * d.d * es);
  L.q = take(R * HD * 4);
  L.attn = take(R * HD * es);
  L.yf = take(R * d.d * 4);
  L.yg = take(R * d.d * es);
  L.rstd = take(R * 4);
  L.ssq = take((size_t)cdiv(d.d, 16) * R * 4);
  L.act = take((size_t)cdiv((int)R, 16) * 16 * cdiv(d.ffn, es == 2 ? 32 : 16) * (es == 2 ? 32 : 16) * es);  // packed
  size_t gp = 0;
  for (int op = OP_FC; op <= OP_DOWN; ++op)
    for (int M : {rows_lv, rows_ex}) gp = std::max(gp, plan_gemm(op, M, d).part_floats);
  L.gpart = take(gp * 4);
  const size_t lp = std::max(plan_lm(B, d, k).part_floats, plan_lm(rows_lv, d, k).part_floats);
  L.lmpart = take(lp * 4);
  L.lmres = take((size_t)std::max(B, rows_lv) * 2 * k * 4);
  // the batched LM head's input rows in fragment order (16 rows x 32 k per KB)
  // and the tiled layer GEMMs' X (q/k/v: x0's two parts, 2d)
  L.xpk = take(d.dtype == EAGLE_BF16 ? (size_t)cdiv(std::max(B, (int)R), 16) * 16 * cdiv(2 * d.d, 32) * 32 * 2 : 0);
  // (tree verify: m rows per sequence)
  const size_t ap = std::max({plan_attn(MODE_LEVEL, k, d, c, B).part_floats,
                              plan_attn(MODE_EXTEND, re, d, c, B).part_floats,
                              plan_attn(MODE_EXTEND, m, d, c, B).part_floats});
  L.apart = take(ap * 4);
  L.rope = take((size_t)d.head_dim / 2 * sizeof(double));
  L.total = off;
  return L;
}

// ------------------------------------------------------------------ validation

static int check_dims(const eagle_dims* d) {
  if (!d) return fail(EAGLE_ERR_ARG, "dims is NULL");
  if (d->dtype != EAGLE_F32 && d->dtype != EAGLE_BF16) return fail(EAGLE_ERR_ARG, "dtype %d", d->dtype);
  if (d->d <= 0 || d->n_heads <= 0 || d->n_kv_heads <= 0 || d->head_dim <= 0 || d->ffn <= 0 || d->vocab <= 0)
    return fail(EAGLE_ERR_SHAPE, "non-positive dimension");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(EAGLE_ERR_UNSUPPORTED, "head_dim %d (64 or 128)", d->head_dim);
  if (d->d != d->n_heads * d->head_dim)
    return fail(EAGLE_ERR_SHAPE, "d %d != n_heads %d * head_dim %d", d->d, d->n_heads, d->head_dim);
  if (d->n_heads % d->n_kv_heads) return fail(EAGLE_ERR_SHAPE, "n_heads %% n_kv_heads != 0");
  if (d->ffn % 8) return fail(EAGLE_ERR_UNSUPPORTED, "ffn %d not a multiple of 8", d->ffn);
  if (d->vocab > 64 * 4096) return fail(EAGLE_ERR_UNSUPPORTED, "vocab %d > 262144", d->vocab);
  if (!(d->rms_eps >= 0.f) || !(d->rope_theta > 0.f)) return fail(EAGLE_ERR_ARG, "rms_eps / rope_theta");
  return EAGLE_OK;
}

static int check_cfg(const eagle_dims* d, const eagle_tree_cfg* c) {
  if (!c) return fail(EAGLE_ERR_ARG, "cfg is NULL");
  if (c->batch < 1) return fail(EAGLE_ERR_SHAPE, "batch %d", c->batch);
  if (c->depth < 2 || c->depth > EAGLE_MAX_DEPTH) return fail(EAGLE_ERR_UNSUPPORTED, "depth %d (2..16)", c->depth);
  if (c->topk < 1 || c->topk > EAGLE_MAX_TOPK) return fail(EAGLE_ERR_UNSUPPORTED, "topk %d (1..16)", c->topk);
  if (d && c->topk > d->vocab) return fail(EAGLE_ERR_SHAPE, "topk %d > vocab %d", c->topk, d->vocab);
  if (c->m < 2 || c->m > EAGLE_MAX_TREE) return fail(EAGLE_ERR_UNSUPPORTED, "m %d (2..64)", c->m);
  const long pool = (long)c->topk + (long)(c->depth - 1) * c->topk * c->topk;
  if (c->m - 1 > pool) return fail(EAGLE_ERR_SHAPE, "m-1 = %d > pool %ld", c->m - 1, pool);
  if (c->max_prefix < c->m + 1) return fail(EAGLE_ERR_SHAPE, "max_prefix %d < m+1", c->max_prefix);
  if (d) {
    const AttnPlan pa = plan_attn(MODE_EXTEND, c->m, *d, *c, c->batch);
    const long wg = (long)c->batch * d->n_kv_heads * pa.nqt;
    if (wg > (1L << 30)) return fail(EAGLE_ERR_UNSUPPORTED, "attention grid %ld too large", wg);
    const int rows_ex = c->batch * ext_rows(c->m, c->depth);
    for (int op = OP_FC; op <= OP_DOWN; ++op)
      for (int M : {c->batch * c->topk, rows_ex})
        if (plan_gemm(op, M, *d).S > GEMM_MAXS)
          return fail(EAGLE_ERR_UNSUPPORTED, "K too long for %d split-K ways", GEMM_MAXS);
    long blocks = 0;
    for (int op = OP_FC; op <= OP_DOWN; ++op)
      blocks = std::max(blocks, (long)plan_gemm(op, rows_ex, *d).nblk * cdiv(rows_ex, 64));
    if (blocks >= GRID_CNT || (long)c->batch * c->m > 4096)
      return fail(EAGLE_ERR_UNSUPPORTED, "batch*m %d too large", c->batch * c->m);
  }
  return EAGLE_OK;
}

static int check_ws(const eagle_dims* d, const eagle_tree_cfg* c, const void* ws, size_t ws_bytes) {
  if (!ws) return fail(EAGLE_ERR_ARG, "workspace is NULL");
  if ((uintptr_t)ws % 256) return fail(EAGLE_ERR_ARG, "workspace not 256-byte aligned");
  const size_t need = plan_ws(*d, *c).total;
  if (ws_bytes < need) return fail(EAGLE_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_bytes, need);
  return EAGLE_OK;
}

// the nine streamed matrices: rows N, inputs K (source rows ld apart), q/k/v
// pair grouping.  Only the feature half of fc_w (its first d columns) is
// streamed; its token half enters through the token-projection table.
struct PackMat {
  const void* eagle_weights::*field;
  const char* name;
  int N, K, ld, pair_hd;
};
static void pack_mats(const eagle_dims& d, PackMat (&m)[9]) {
  const int hq = d.n_heads * d.head_dim, hk = d.n_kv_heads * d.head_dim;
  m[0] = {&eagle_weights::fc_w, "fc_w", d.d, d.d, 2 * d.d, 0};
  m[1] = {&eagle_weights::wq, "wq", hq, d.d, d.d, d.head_dim};
  m[2] = {&eagle_weights::wk, "wk", hk, d.d, d.d, d.head_dim};
  m[3] = {&eagle_weights::wv, "wv", hk, d.d, d.d, d.head_dim};
  m[4] = {&eagle_weights::wo, "wo", d.d, hq, hq, 0};
  m[5] = {&eagle_weights::w_gate, "w_gate", d.ffn, d.d, d.d, 0};
  m[6] = {&eagle_weights::w_up, "w_up", d.ffn, d.d, d.d, 0};
  m[7] = {&eagle_weights::w_down, "w_down", d.d, d.ffn, d.ffn, 0};
  m[8] = {&eagle_weights::lm_head, "lm_head", d.vocab, d.d, d.d, 0};
}
static size_t tokproj_bytes(const eagle_dims& d) { return (size_t)d.vocab * d.d * 4; }
static size_t packed_mat_bytes(int N, int K, int es) {
  const int ks = es == 2 ? 32 : 16;
  return (size_t)cdiv(N, 16) * 16 * ((size_t)cdiv(K, ks) * ks) * es;
}

static int check_weights(const eagle_weights* w, bool tail_only) {
  if (!w) return fail(EAGLE_ERR_ARG, "weights is NULL");
  if (w->packed != EAGLE_PACKED_WEIGHTS)
    return fail(EAGLE_ERR_ARG, "weights are not packed (pack them once with eagle_pack_weights)");
  if (!w->lm_head) return fail(EAGLE_ERR_ARG, "weight lm_head is NULL");
  if (tail_only) return EAGLE_OK;
  const void* need[] = {w->fc_w, w->fc_b, w->wq, w->wk, w->wv, w->wo, w->post_norm,
                        w->w_gate, w->w_up, w->w_down, w->embed, w->tok_proj};
  const char* names[] = {"fc_w", "fc_b", "wq", "wk", "wv", "wo", "post_norm",
                         "w_gate", "w_up", "w_down", "embed", "tok_proj"};
  for (int i = 0; i < 12; ++i)
    if (!need[i]) return fail(EAGLE_ERR_ARG, "weight %s is NULL", names[i]);
  return EAGLE_OK;
}

static int check_state(const eagle_seq_state* s) {
  if (!s) return fail(EAGLE_ERR_ARG, "state is NULL");
  if (!s->k_cache || !s->v_cache || !s->prefix_len || !s->root_feat || !s->root_token)
    return fail(EAGLE_ERR_ARG, "state has a NULL pointer");
  return EAGLE_OK;
}

static RoundArgs make_args(const eagle_dims& d, const eagle_tree_cfg& c, const eagle_weights* w,
                           const eagle_seq_state* st, void* ws) {
  RoundArgs a{};
  a.dtype = d.dtype;
  a.B = c.batch; a.d = d.d; a.H = d.n_heads; a.Hkv = d.n_kv_heads; a.hd = d.head_dim;
  a.F = d.ffn; a.V = d.vocab; a.D = c.depth; a.k = c.topk; a.m = c.m; a.max_prefix = c.max_prefix;
  a.eps = d.rms_eps; a.theta = d.rope_theta;
  if (w) {
    a.fc_w = w->fc_w; a.fc_b = w->fc_b; a.wq = w->wq; a.wk = w->wk; a.wv = w->wv; a.wo = w->wo;
    a.post_norm = w->post_norm; a.w_gate = w->w_gate; a.w_up = w->w_up; a.w_down = w->w_down;
    a.embed = w->embed; a.lm_head = w->lm_head; a.tok_proj = (const float*)w->tok_proj;
  }
  if (st) {
    a.k_cache = st->k_cache; a.v_cache = st->v_cache; a.prefix_len = st->prefix_len;
    a.root_feat = st->root_feat; a.root_token = st->root_token;
  }
  const WsLayout L = plan_ws(d, c);
  char* base = (char*)ws;
  a.err = (int*)(base + L.err);
  a.cnt = (int*)(base + L.cnt);
  a.pool = (eagle_pool_entry*)(base + L.pool);
  a.frontier = (eagle_frontier_node*)(base + L.frontier);
  a.feat = base + L.feat; a.tk = base + L.tk; a.tv = base + L.tv; a.ext_h = base + L.ext_h;
  a.x0f = (float*)(base + L.x0f); a.x0b = base + L.x0b; a.x0l = base + L.x0l; a.q = (float*)(base + L.q);
  a.attn = base + L.attn; a.yf = (float*)(base + L.yf); a.yg = base + L.yg;
  a.rstd = (float*)(base + L.rstd); a.ssq = (float*)(base + L.ssq); a.act = base + L.act;
  a.gpart = (float*)(base + L.gpart); a.lmpart = (float*)(base + L.lmpart);
  a.lmres = (float*)(base + L.lmres); a.apart = (float*)(base + L.apart); a.xpk = base + L.xpk;
  a.rope = (const double*)(base + L.rope);
  a.pool_n = L.pool_n;
  return a;
}

static int hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(EAGLE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return EAGLE_OK;
}

// draft layer over `rows` rows (frontier or extend): FC, QKV+RoPE+KV, attention,
// O+residual+norm stats, gate/up+SwiGLU, down+residual.  skip_fc: x0 is
// already in the workspace (the previous level's FC hand-over).
static int run_layer(RoundArgs a, const eagle_dims& d, const eagle_tree_cfg& c, hipStream_t s,
                     bool skip_fc = false) {
  static const char* names[] = {"fc", "qkv", "o", "gateup", "down"};
  for (int op = skip_fc ? OP_QKV : OP_FC; op <= OP_DOWN; ++op) {
    if (op == OP_O) {
      const AttnPlan pa = plan_attn(a.mode, a.RS, d, c, a.B);
      int r = hip_ok(launch_attn(a, pa, s), "attention launch");
      if (r) return r;
    }
    int r;
    if (use_skinny(a.mode, a.rows)) {
      SkPlan p = plan_skinny(op, a.rows, d);
      if (op == OP_GATEUP) p.nps = plan_skinny(OP_O, a.rows, d).nwg;
      r = hip_ok(launch_skinny(op, a, p, s), names[op]);
    } else {
      r = hip_ok(launch_gemm(op, a, plan_gemm(op, a.rows, d), s), names[op]);
    }
    if (r) return r;
  }
  return EAGLE_OK;
}

}  // namespace eg

using namespace eg;

extern "C" {

const char* eagle_status_str(int status) {
  switch (status) {
    case EAGLE_OK: return "ok";
    case EAGLE_ERR_ARG: return "invalid argument";
    case EAGLE_ERR_SHAPE: return "inconsistent shape";
    case EAGLE_ERR_UNSUPPORTED: return "unsupported configuration";
    case EAGLE_ERR_WORKSPACE: return "workspace too small";
    case EAGLE_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* eagle_last_error(void) { return g_err; }

size_t eagle_workspace_bytes(const eagle_dims* dims, const eagle_tree_cfg* cfg) {
  if (check_dims(dims) || check_cfg(dims, cfg)) return 0;
  return plan_ws(*dims, *cfg).total;
}

size_t eagle_packed_weights_bytes(const eagle_dims* dims) {
  if (check_dims(dims)) return 0;
  PackMat m[9];
  pack_mats(*dims, m);
  size_t total = 0;
  for (const PackMat& x : m) total += align256(packed_mat_bytes(x.N, x.K, (int)elem_size(*dims)));
  return total + align256(tokproj_bytes(*dims));
}

int eagle_pack_weights(const eagle_dims* dims, const eagle_weights* src, void* dst, size_t dst_bytes,
                       eagle_weights* out, void* stream) {
  int r;
  if ((r = check_dims(dims))) return r;
  if (!src || !dst || !out) return fail(EAGLE_ERR_ARG, "src, dst or out is NULL");
  if (src->packed) return fail(EAGLE_ERR_ARG, "src is already packed");
  if ((uintptr_t)dst % 256) return fail(EAGLE_ERR_ARG, "dst not 256-byte aligned");
  const size_t need = eagle_packed_weights_bytes(dims);
  if (dst_bytes < need) return fail(EAGLE_ERR_WORKSPACE, "dst %zu < %zu bytes", dst_bytes, need);
  PackMat m[9];
  pack_mats(*dims, m);
  for (const PackMat& x : m) {
    const void* p = src->*(x.field);
    if (!p) return fail(EAGLE_ERR_ARG, "weight %s is NULL", x.name);
    if ((uintptr_t)p % 16) return fail(EAGLE_ERR_ARG, "weight %s not 16-byte aligned", x.name);
  }
  if (!src->fc_b || !src->post_norm || !src->embed) return fail(EAGLE_ERR_ARG, "fc_b, post_norm or embed is NULL");
  if ((uintptr_t)src->embed % 16) return fail(EAGLE_ERR_ARG, "embed not 16-byte aligned");
  const int es = (int)elem_size(*dims);
  eagle_weights o = *src;
  size_t off = 0;
  for (const PackMat& x : m) {
    unsigned char* d = (unsigned char*)dst + off;
    if ((r = hip_ok(launch_pack(src->*(x.field), d, x.N, x.K, x.ld, es, x.pair_hd, (hipStream_t)stream), "pack")))
      return r;
    o.*(x.field) = d;
    off += align256(packed_mat_bytes(x.N, x.K, es));
  }
  float* tp = (float*)((unsigned char*)dst + off);
  if ((r = hip_ok(launch_tokproj(src->embed, src->fc_w, tp, dims->vocab, dims->d, es, (hipStream_t)stream),
                  "token projection")))
    return r;
  o.tok_proj = tp;
  o.packed = EAGLE_PACKED_WEIGHTS;
  *out = o;
  return EAGLE_OK;
}

int eagle_workspace_init(const eagle_dims* dims, const eagle_tree_cfg* cfg, void* ws, size_t ws_bytes,
                         void* stream) {
  int r;
  if ((r = check_dims(dims)) || (r = check_cfg(dims, cfg)) || (r = check_ws(dims, cfg, ws, ws_bytes)))
    return r;
  const WsLayout L = plan_ws(*dims, *cfg);
  if ((r = hip_ok(launch_zero(ws, L.total, (hipStream_t)stream), "zero fill"))) return r;
  return hip_ok(launch_rope_table((double*)((char*)ws + L.rope), dims->head_dim, dims->rope_theta,
                                  (hipStream_t)stream), "rope table");
}

static int draft_level(const eagle_dims* dims, const eagle_weights* w, const eagle_tree_cfg* cfg,
                       const eagle_seq_state* state, int32_t level, int32_t flags, void* ws,
                       size_t ws_bytes, hipEvent_t e0, hipEvent_t e1, void* stream,
                       const int32_t* tmpl = nullptr) {
  int r;
  if ((r = check_dims(dims)) || (r = check_cfg(dims, cfg)) || (r = check_ws(dims, cfg, ws, ws_bytes)))
    return r;
  if (flags != EAGLE_LEVEL_FULL && flags != EAGLE_LEVEL_TAIL_ONLY && flags != EAGLE_LEVEL_LMHEAD_ONLY &&
      flags != EAGLE_LEVEL_FULL_FC)
    return fail(EAGLE_ERR_ARG, "flags %d", flags);
  if (level < 1 || level > cfg->depth) return fail(EAGLE_ERR_ARG, "level %d (1..%d)", level, cfg->depth);
  const bool lm_only = flags == EAGLE_LEVEL_LMHEAD_ONLY;
  const bool full = flags == EAGLE_LEVEL_FULL || flags == EAGLE_LEVEL_FULL_FC;
  const bool tail_only = level == 1 || !full;
  // the merge of this call also forms the next level's FC input (hand-over)
  SkPlan fp{};
  const bool handover = level < cfg->depth && handover_plan(*dims, *cfg, level, &fp);
  if ((r = check_weights(w, tail_only && !handover)) || (r = check_state(state))) return r;
  const hipStream_t s = (hipStream_t)stream;
  RoundArgs a = make_args(*dims, *cfg, w, state, ws);
  a.tmpl = tmpl;
  if (level == 1) {
    a.rows = cfg->batch;
    const LmPlan pl = plan_lm(cfg->batch, *dims, cfg->topk);
    if ((r = hip_ok(launch_lmhead(a, pl, 1, s, e0, e1), "lm head"))) return r;
    if (lm_only) return EAGLE_OK;
    return hip_ok(launch_lmmerge(a, pl, 1, s, handover ? &fp : nullptr), "lm merge");
  }
  a.mode = MODE_LEVEL;
  a.depth = level - 1;
  a.rows = cfg->batch * cfg->topk;
  a.RS = cfg->topk;
  // x0 of this level was formed by the previous level's hand-over, unless the
  // caller asks for it here
  const bool have_x0 = flags == EAGLE_LEVEL_FULL && handover_plan(*dims, *cfg, level - 1, nullptr);
  const LmPlan pl = plan_lm(a.rows, *dims, cfg->topk);
  a.lm_px = !tail_only && pl.nq > 0;  // the layer runs here: its down epilogue packs the LM head's X
  if (!tail_only && (r = run_layer(a, *dims, *cfg, s, have_x0))) return r;
  if ((r = hip_ok(launch_lmhead(a, pl, level, s, e0, e1), "lm head"))) return r;
  if (lm_only) return EAGLE_OK;
  return hip_ok(launch_lmmerge(a, pl, level, s, handover ? &fp : nullptr), "lm merge");
}

int eagle_draft_level(const eagle_dims* dims, const eagle_weights* w, const eagle_tree_cfg* cfg,
                      const eagle_seq_state* state, int32_t level, int32_t flags, void* ws,
                      size_t ws_bytes, void* stream) {
  return draft_level(dims, w, cfg, state, level, flags, ws, ws_bytes, nullptr, nullptr, stream);
}

int eagle_draft_level_timed(const eagle_dims* dims, const eagle_weights* w,
                            const eagle_tree_cfg* cfg, const eagle_seq_state* state, int32_t level,
                            int32_t flags, void* ws, size_t ws_bytes, void* start_event,
                            void* stop_event, void* stream) {
  return draft_level(dims, w, cfg, state, level, flags, ws, ws_bytes, (hipEvent_t)start_event,
                     (hipEvent_t)stop_event, stream);
}

int eagle_draft_level_static(const eagle_dims* dims, const eagle_weights* w, const eagle_tree_cfg* cfg,
                             const eagle_seq_state* state, int32_t level, int32_t flags,
                             const int32_t* tmpl, void* ws, size_t ws_bytes, void* stream) {
  if (!tmpl) return fail(EAGLE_ERR_ARG, "template is NULL");
  return draft_level(dims, w, cfg, state, level, flags, ws, ws_bytes, nullptr, nullptr, stream, tmpl);
}

int eagle_build_static_tree(const eagle_dims* dims, const eagle_tree_cfg* cfg,
                            const eagle_seq_state* state, void* ws, size_t ws_bytes, int32_t* tokens,
                            int32_t* parents, int32_t* depth, int32_t* positions, uint8_t* mask,
                            float* node_logscore, void* stream) {
  int r;
  if ((r = check_dims(dims)) || (r = check_cfg(dims, cfg)) || (r = check_ws(dims, cfg, ws, ws_bytes)))
    return r;
  if ((r = check_state(state))) return r;
  if (!tokens || !parents) return fail(EAGLE_ERR_ARG, "tokens/parents is NULL");
  if (cfg->m > 1 + cfg->depth * cfg->topk)
    return fail(EAGLE_ERR_SHAPE, "m %d > 1 + depth*topk = %d (the static tree's size)", cfg->m,
                1 + cfg->depth * cfg->topk);
  RoundArgs a = make_args(*dims, *cfg, nullptr, state, ws);
  return hip_ok(launch_static_build(a, tokens, parents, depth, positions, mask, node_logscore,
                                    (hipStream_t)stream),
                "static build");
}

int eagle_tree_verify_attention(const eagle_dims* dims, const eagle_tree_cfg* cfg, const float* q,
                                const void* k_cache, const void* v_cache, const int32_t* prefix_len,
                                const uint8_t* mask, void* out, void* ws, size_t ws_bytes, void* stream) {
  int r;
  if ((r = check_dims(dims)) || (r = check_cfg(dims, cfg)) || (r = check_ws(dims, cfg, ws, ws_bytes)))
    return r;
  if (!q || !k_cache || !v_cache || !prefix_len || !mask || !out)
    return fail(EAGLE_ERR_ARG, "q, k_cache, v_cache, prefix_len, mask or out is NULL");
  RoundArgs a = make_args(*dims, *cfg, nullptr, nullptr, ws);
  a.mode = MODE_VERIFY;
  a.RS = cfg->m;
  a.rows = cfg->batch * cfg->m;
  a.q = (float*)q;
  a.k_cache = (void*)k_cache;
  a.v_cache = (void*)v_cache;
  a.prefix_len = (int32_t*)prefix_len;
  a.vmask = mask;
  a.attn = out;
  const AttnPlan pa = plan_attn(MODE_EXTEND, cfg->m, *dims, *cfg, cfg->batch);
  return hip_ok(launch_attn(a, pa, (hipStream_t)stream), "tree verify attention");
}

int eagle_rerank_build_tree(const eagle_dims* dims, const eagle_tree_cfg* cfg,
                            const eagle_seq_state* state, void* ws, size_t ws_bytes, int32_t* tokens,
                            int32_t* parents, int32_t* depth, int32_t* positions, uint8_t* mask,
                            float* node_logscore, void* stream) {
  int r;
  if ((r = check_dims(dims)) || (r = check_cfg(dims, cfg)) || (r = check_ws(dims, cfg, ws, ws_bytes)))
    return r;
  if ((r = check_state(state))) return r;
  if (!tokens || !parents) return fail(EAGLE_ERR_ARG, "tokens/parents is NULL");
  RoundArgs a = make_args(*dims, *cfg, nullptr, state, ws);
  return hip_ok(launch_rerank(a, tokens, parents, depth, positions, mask, node_logscore,
                              (hipStream_t)stream),
                "rerank");
}

int eagle_verify_greedy(const eagle_tree_cfg* cfg, int32_t vocab, const float* target_logits,
                        const int32_t* tokens, const int32_t* parents, int32_t* accept_len,
                        int32_t* accept_path, int32_t* bonus, void* stream) {
  int r;
  if ((r = check_cfg(nullptr, cfg))) return r;
  if (vocab < 1) return fail(EAGLE_ERR_SHAPE, "vocab %d", vocab);
  if (!target_logits || !tokens || !parents || !accept_len || !accept_path || !bonus)
    return fail(EAGLE_ERR_ARG, "verify: NULL pointer");
  return hip_ok(launch_verify(cfg->batch, cfg->m, cfg->depth, vocab, target_logits, tokens, parents,
                              accept_len, accept_path, bonus, (hipStream_t)stream),
                "verify");
}

size_t eagle_verify_rejection_scratch_bytes(const eagle_tree_cfg* cfg, int32_t vocab) {
  if (check_cfg(nullptr, cfg) || vocab < 1) return 0;
  return verify_rejection_scratch_bytes(cfg->batch, cfg->m);
}

int eagle_verify_rejection(const eagle_tree_cfg* cfg, int32_t vocab, const float* target_logits,
                           const float* draft_logits, const int32_t* tokens, const int32_t* parents,
                           float temperature, const float* uniforms, int32_t* accept_len,
                           int32_t* accept_path, int32_t* bonus, void* scratch, size_t scratch_bytes,
                           void* stream) {
  int r;
  if ((r = check_cfg(nullptr, cfg))) return r;
  if (vocab < 1) return fail(EAGLE_ERR_SHAPE, "vocab %d", vocab);
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(EAGLE_ERR_ARG, "temperature %g (positive, finite)", (double)temperature);
  if (!target_logits || !draft_logits || !tokens || !parents || !uniforms || !accept_len || !accept_path ||
      !bonus || !scratch)
    return fail(EAGLE_ERR_ARG, "verify_rejection: NULL pointer");
  if ((uintptr_t)scratch % 8) return fail(EAGLE_ERR_ARG, "scratch not 8-byte aligned");
  const size_t need = verify_rejection_scratch_bytes(cfg->batch, cfg->m);
  if (scratch_bytes < need) return fail(EAGLE_ERR_WORKSPACE, "scratch %zu < %zu bytes", scratch_bytes, need);
  if ((long)cfg->batch * cfg->m > 65535) return fail(EAGLE_ERR_UNSUPPORTED, "batch*m %d too large", cfg->batch * cfg->m);
  return hip_ok(launch_verify_rejection(cfg->batch, cfg->m, cfg->depth, vocab, target_logits, draft_logits,
                                        tokens, parents, temperature, uniforms, scratch, accept_len,
                                        accept_path, bonus, (hipStream_t)stream),
                "verify_rejection");
}

int eagle_verify_rejection_topk(const eagle_tree_cfg* cfg, int32_t vocab, const float* target_logits,
                                const int32_t* tokens, const int32_t* parents, float temperature,
                                const float* uniforms, int32_t* accept_len, int32_t* accept_path, int32_t* bonus,
                                void* scratch, size_t scratch_bytes, void* stream) {
  int r;
  if ((r = check_cfg(nullptr, cfg))) return r;
  if (vocab < 1) return fail(EAGLE_ERR_SHAPE, "vocab %d", vocab);
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(EAGLE_ERR_ARG, "temperature %g (positive, finite)", (double)temperature);
  if (!target_logits || !tokens || !parents || !uniforms || !accept_len || !accept_path || !bonus || !scratch)
    return fail(EAGLE_ERR_ARG, "verify_rejection_topk: NULL pointer");
  if ((uintptr_t)scratch % 8) return fail(EAGLE_ERR_ARG, "scratch not 8-byte aligned");
  const size_t need = verify_relaxed_scratch_bytes(cfg->batch, cfg->m);
  if (scratch_bytes < need) return fail(EAGLE_ERR_WORKSPACE, "scratch %zu < %zu bytes", scratch_bytes, need);
  if ((long)cfg->batch * cfg->m > 65535) return fail(EAGLE_ERR_UNSUPPORTED, "batch*m %d too large", cfg->batch * cfg->m);
  return hip_ok(launch_verify_relaxed(cfg->batch, cfg->m, cfg->depth, vocab, target_logits, tokens, parents,
                                      temperature, 0.f, uniforms, scratch, accept_len, accept_path, bonus,
                                      (hipStream_t)stream, true),
                "verify_rejection_topk");
}

// ---- eagle_verify_rejection_topk_noalloc: the scratch lives in a file-scope
// device array (each device holds its own copy for the life of the process).
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is taken once per device with hipGetSymbolAddress and only
// that address is passed to kernels.
#define NOALLOC_SCRATCH_BYTES ((size_t)EAGLE_NOALLOC_MAX_ROWS * 16 * 8)
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];
static std::mutex g_noalloc_mu;
static void* g_noalloc_ptr[64];  // per device ordinal

// the current device's address of `scratch` (null on failure, with the message set)
static void* noalloc_scratch() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    fail(EAGLE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= 64) {
    fail(EAGLE_ERR_UNSUPPORTED, "device ordinal %d (0..63)", dev);
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_noalloc_mu);
  if (!g_noalloc_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      fail(EAGLE_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      return nullptr;
    }
    g_noalloc_ptr[dev] = ptr;
  }
  return g_noalloc_ptr[dev];
}

int eagle_verify_rejection_topk_noalloc(const eagle_tree_cfg* cfg, int32_t vocab, const float* target_logits,
                                        const int32_t* tokens, const int32_t* parents, float temperature,
                                        const float* uniforms, int32_t* accept_len, int32_t* accept_path,
                                        int32_t* bonus, void* stream) {
  int r;
  if ((r = check_cfg(nullptr, cfg))) return r;
  if ((long)cfg->batch * cfg->m > EAGLE_NOALLOC_MAX_ROWS)
    return fail(EAGLE_ERR_UNSUPPORTED, "batch*m %d above the no-allocation limit %d", cfg->batch * cfg->m,
                EAGLE_NOALLOC_MAX_ROWS);
  const size_t need = verify_relaxed_scratch_bytes(cfg->batch, cfg->m);
  if (need > NOALLOC_SCRATCH_BYTES)
    return fail(EAGLE_ERR_UNSUPPORTED, "scratch %zu above %zu bytes", need, NOALLOC_SCRATCH_BYTES);
  void* ptr = noalloc_scratch();
  if (!ptr) return EAGLE_ERR_HIP;
  return eagle_verify_rejection_topk(cfg, vocab, target_logits, tokens, parents, temperature, uniforms, accept_len,
                                     accept_path, bonus, ptr, NOALLOC_SCRATCH_BYTES, stream);
}

size_t eagle_verify_relaxed_scratch_bytes(const eagle_tree_cfg* cfg) {
  if (check_cfg(nullptr, cfg)) return 0;
  return verify_relaxed_scratch_bytes(cfg->batch, cfg->m);
}

int eagle_verify_relaxed(const eagle_tree_cfg* cfg, int32_t vocab, const float* target_logits,
                         const int32_t* tokens, const int32_t* parents, float temperature,
                         float threshold, const float* uniforms, int32_t* accept_len,
                         int32_t* accept_path, int32_t* bonus, void* scratch, size_t scratch_bytes,
                         void* stream) {
  int r;
  if ((r = check_cfg(nullptr, cfg))) return r;
  if (vocab < 1) return fail(EAGLE_ERR_SHAPE, "vocab %d", vocab);
  if (!(temperature > 0.f) || !std::isfinite(temperature))
    return fail(EAGLE_ERR_ARG, "temperature %g (positive, finite)", (double)temperature);
  if (!std::isfinite(threshold)) return fail(EAGLE_ERR_ARG, "threshold is not finite");
  if (!target_logits || !tokens || !parents || !uniforms || !accept_len || !accept_path || !bonus ||
      !scratch)
    return fail(EAGLE_ERR_ARG, "verify_relaxed: NULL pointer");
  if ((uintptr_t)scratch % 8) return fail(EAGLE_ERR_ARG, "scratch not 8-byte aligned");
  const size_t need = verify_relaxed_scratch_bytes(cfg->batch, cfg->m);
  if (scratch_bytes < need) return fail(EAGLE_ERR_WORKSPACE, "scratch %zu < %zu bytes", scratch_bytes, need);
  if ((long)cfg->batch * cfg->m > 65535) return fail(EAGLE_ERR_UNSUPPORTED, "batch*m %d too large", cfg->batch * cfg->m);
  return hip_ok(launch_verify_relaxed(cfg->batch, cfg->m, cfg->depth, vocab, target_logits, tokens, parents,
                                      temperature, threshold, uniforms, scratch, accept_len, accept_path,
                                      bonus, (hipStream_t)stream),
                "verify_relaxed");
}

int eagle_draft_extend(const eagle_dims* dims, const eagle_weights* w, const eagle_tree_cfg* cfg,
                       const eagle_seq_state* state, const void* true_feat, const int32_t* tokens,
                       const int32_t* accept_len, const int32_t* accept_path, const int32_t* bonus,
                       void* ws, size_t ws_bytes, void* stream) {
  int r;
  if ((r = check_dims(dims)) || (r = check_cfg(dims, cfg)) || (r = check_ws(dims, cfg, ws, ws_bytes)))
    return r;
  if ((r = check_weights(w, false)) || (r = check_state(state))) return r;
  if (!true_feat || !tokens || !accept_len || !accept_path || !bonus)
    return fail(EAGLE_ERR_ARG, "extend: NULL pointer");
  RoundArgs a = make_args(*dims, *cfg, w, state, ws);
  a.mode = MODE_EXTEND;
  a.depth = 0;
  a.RS = ext_rows(cfg->m, cfg->depth);  // an accepted path's longest length
  a.rows = cfg->batch * a.RS;
  a.true_feat = true_feat;
  a.tokens = tokens;
  a.accept_len = accept_len;
  a.accept_path = accept_path;
  a.bonus = bonus;
  return run_layer(a, *dims, *cfg, (hipStream_t)stream);
}

int eagle_ws_view(const eagle_dims* dims, const eagle_tree_cfg* cfg, const void* ws, int32_t what,
                  void** ptr, size_t* bytes) {
  int r;
  if ((r = check_dims(dims)) || (r = check_cfg(dims, cfg))) return r;
  if (!ws || !ptr || !bytes) return fail(EAGLE_ERR_ARG, "ws_view: NULL pointer");
  const WsLayout L = plan_ws(*dims, *cfg);
  const size_t es = elem_size(*dims);
  const size_t B = cfg->batch, k = cfg->topk, D = cfg->depth, m = cfg->m;
  size_t off, n;
  switch (what) {
    case EAGLE_WS_ERROR: off = L.err; n = 16; break;
    case EAGLE_WS_POOL: off = L.pool; n = B * L.pool_n * sizeof(eagle_pool_entry); break;
    case EAGLE_WS_FRONTIER: off = L.frontier; n = (D + 1) * B * k * sizeof(eagle_frontier_node); break;
    case EAGLE_WS_FEAT: off = L.feat; n = D * B * k * dims->d * es; break;
    case EAGLE_WS_TREE_K: off = L.tk; n = B * D * k * dims->n_kv_heads * dims->head_dim * 4; break;
    case EAGLE_WS_TREE_V: off = L.tv; n = B * D * k * dims->n_kv_heads * dims->head_dim * 4; break;
    case EAGLE_WS_EXT_H: off = L.ext_h; n = B * ext_rows((int)m, (int)D) * dims->d * es; break;
    case EAGLE_WS_X0: off = L.x0f; n = (size_t)L.rows_max * dims->d * 4; break;
    case EAGLE_WS_ATTN: off = L.attn; n = (size_t)L.rows_max * dims->n_heads * dims->head_dim * es; break;
    case EAGLE_WS_Y: off = L.yf; n = (size_t)L.rows_max * dims->d * 4; break;
    default: return fail(EAGLE_ERR_ARG, "ws_view: region %d", what);
  }
  *ptr = (char*)ws + off;
  *bytes = n;
  return EAGLE_OK;
}

}  // extern "C"

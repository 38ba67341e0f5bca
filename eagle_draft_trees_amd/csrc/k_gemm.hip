// Skinny weight-streaming GEMMs of the draft layer on MFMA, with the layer's
// elementwise work fused into the loaders and epilogues.
//
//   Y[M][N] = X[M][K] * W[N][K]^T,  M = frontier rows (B*k) or extend rows (B*min(m, D+1))
//
// At drafting shapes M is 1..64 while W is megabytes, so every kernel here is
// bound by streaming W from HBM once.  A workgroup holds CTW adjacent 16-column
// tiles (four, or three where that leaves fewer compute units idle) times four
// K slices, one wave each, over one K range.  It stages the X rows of that K
// range in LDS chunk by chunk (shared by its waves), so the only global loads
// in the main loop are W's: one 16-byte load per lane per k-step (one
// contiguous kilobyte of the packed tile per wave instruction), each fed to a
// 16x16 MFMA per m-tile (bf16: v_mfma_f32_16x16x32_bf16; fp32: four 16x16x4
// steps) with its A operand read from LDS.  When the column blocks would leave
// most compute units idle, K is split across workgroups (four-tile blocks
// only); each split writes fp32 partials and k_gemm_fin sums them in split
// order -- deterministic, no float atomics -- and runs the epilogue.
//
// Fused steps (draft head of [P1] "EAGLE 推测解码为什么比 Medusa 快？" §4.1 and
// [P3] zdszero.github.io spec_medusa_eagle, "在 SGLang 里"):
//   FC      X = the parent (level) or true (extend) feature, gathered on the
//           fly, against the feature half of W_fc; epilogue + the row token's
//           token-projection entry + bias -> x0 (fp32 residual, dtype copy)
//   QKV     x0 taken as two bf16 parts (bf16); epilogue applies RoPE at the
//           row's tree position to q and k ([P1] §12 item 5: positions shared
//           per level) and writes k, v straight into the in-tree slot (levels,
//           fp32) or the prefix cache (extend)
//   O       epilogue adds the residual x0, keeps y, emits y*gain for the MLP
//           and per-block sums of squares (each gate/up workgroup sums them
//           into the RMSNorm 1/rms of its rows)
//   GATEUP  two weight streams per wave (gate and up rows of the same 16
//           columns); epilogue silu(g/rms) * (u/rms)
//   DOWN    epilogue adds the residual y -> predicted feature (no final norm);
//           the extend also writes the next root feature, and its first
//           workgroup advances the sequence state
#include "eagle_internal.h"

namespace eg {


// gate/up: the RMSNorm statistic of a row is the sum of the O launch's
// per-workgroup row partials; tpr = blockDim / rows (at most 16) threads per
// row each sum every tpr-th partial (loads issued here, the sums used after
// the GEMM)
__device__ __forceinline__ float ssq_prefetch(const RoundArgs& a, const GemmPlan& p, int zg, int tid, int rows) {
  const int tpr = min(16, (int)blockDim.x / rows);
  float s = 0.f;
  const int r = tid / tpr, j = tid - r * tpr, row = zg * 64 + r;
  if (r < rows && row < p.M) {
    for (int q0 = j; q0 < p.nps; q0 += 4 * tpr) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int q = q0 + tpr * u;
        v[u] = q < p.nps ? a.ssq[(size_t)q * a.rows + row] : 0.f;
      }
      s += (v[0] + v[1]) + (v[2] + v[3]);
    }
  }
  return s;
}
// 1 / rms per row from the tpr partial sums of ssq_prefetch (sq: ROWS*16 floats of LDS)
template <int ROWS>
__device__ __forceinline__ void rstd_finish(const RoundArgs& a, float* sq, float ssq_part, float* s_rstd, int tid) {
  const int tpr = min(16, (int)blockDim.x / ROWS);
  if (tid < ROWS * tpr) sq[tid] = ssq_part;
  __syncthreads();
  if (tid < ROWS) {
    float sacc = 0.f;
    for (int j = 0; j < tpr; ++j) sacc += sq[tid * tpr + j];
    s_rstd[tid] = 1.0f / sqrtf(sacc / (float)a.d + a.eps);
  }
}

// The ops' epilogues on one 64-column block of one z-group; tile[NW][ROWS][65]
// in LDS holds the block's sums (all threads of the workgroup call this).
template <typename T, int OP, int MT, int CTW>
__device__ __forceinline__ void gemm_epilogue(const RoundArgs& a, const GemmPlan& p, float* tile,
                                              const float* s_rstd, int blk, int zg, int tid) {
  constexpr int NW = (OP == OP_GATEUP) ? 2 : 1;
  constexpr int ROWS = MT * 16;
  constexpr int BW = CTW * 16;  // columns of the block
  static_assert(OP != OP_O || CTW == 4, "the O launch keeps 64-column blocks");
#define TILE(w, r, c) tile[((w) * ROWS + (r)) * 65 + (c)]
  const int rows_here = min(ROWS, p.M - zg * 64);
  if (OP == OP_FC) {  // + the token half: the row's token-projection table entry
    __shared__ int s_tok[ROWS];
    if (tid < rows_here) s_tok[tid] = fc_row_token<T>(a, zg * 64 + tid);
    __syncthreads();
    for (int idx = tid; idx < rows_here * BW; idx += (int)blockDim.x) {
      const int mr = idx / BW, c = idx % BW, nn = blk * BW + c, row = zg * 64 + mr;
      if (nn >= p.N) continue;
      const float v = TILE(0, mr, c) + a.tok_proj[(size_t)s_tok[mr] * a.d + nn] + El<T>::ld((const T*)a.fc_b, nn);
      st_x0<T>(a, (size_t)row * a.d + nn, v);
    }
  } else if (OP == OP_QKV) {
    // the block's tiles are tiles CTW*blk .. CTW*blk+CTW-1 (hd/16 tiles per
    // head); tile j of a head holds the rotation pairs (8j+e, hd/2+8j+e),
    // e < 8, in its columns e and 8+e
    const int per = a.hd / 16, half = a.hd / 2, ntile = (p.N + 15) / 16;
    const int hq = a.H, hk = a.Hkv;
    for (int idx = tid; idx < rows_here * CTW * 8; idx += (int)blockDim.x) {
      const int mr = idx / (CTW * 8), pr = idx % (CTW * 8), ct = pr >> 3, e = pr & 7, row = zg * 64 + mr;
      const int t = CTW * blk + ct;
      if (t >= ntile) continue;
      const int head = t / per;
      const int fi = 8 * (t % per) + e;  // frequency index within the half
      float lo = TILE(0, mr, ct * 16 + e), hi = TILE(0, mr, ct * 16 + 8 + e);
      int b, slot, pos;
      if (a.mode == MODE_LEVEL) {
        b = row / a.k;
        slot = row % a.k;
        pos = clamp_prefix(a.prefix_len[b], a) - 1 + a.depth;
      } else {
        b = row / a.RS;
        slot = row % a.RS;
        pos = clamp_prefix(a.prefix_len[b], a) + slot;
      }
      if (head < hq + hk) {  // q or k: rotate the (fi, fi+half) pair
        float sn, cs;
        rope_sincos(pos, a.rope[fi], sn, cs);
        const float nlo = lo * cs - hi * sn, nhi = hi * cs + lo * sn;
        lo = nlo;
        hi = nhi;
      }
      if (head < hq) {
        float* qr = a.q + (size_t)row * (a.H * a.hd) + head * a.hd;
        qr[fi] = lo;
        qr[fi + half] = hi;
      } else {
        const bool isk = head < hq + hk;
        const int kvh = isk ? head - hq : head - hq - hk;
        if (a.mode == MODE_LEVEL) {  // in-tree K/V are kept in fp32 (workspace)
          float* dst = (float*)(isk ? a.tk : a.tv) + ((((size_t)b * a.D + a.depth) * a.k + slot) * a.Hkv + kvh) * a.hd;
          dst[fi] = lo;
          dst[fi + half] = hi;
        } else {
          T* base = (T*)(isk ? a.k_cache : a.v_cache);
          const int P = clamp_prefix(a.prefix_len[b], a);
          T* dst = base + (((size_t)b * a.max_prefix + P + slot) * a.Hkv + kvh) * a.hd;
          El<T>::st(dst, fi, lo);
          El<T>::st(dst, fi + half, hi);
        }
      }
    }
  } else if (OP == OP_O) {
    for (int idx = tid; idx < rows_here * 64; idx += (int)blockDim.x) {
      const int mr = idx >> 6, c = idx & 63, nn = blk * 64 + c, row = zg * 64 + mr;
      if (nn >= p.N) { TILE(0, mr, c) = 0.f; continue; }
      const float y = TILE(0, mr, c) + a.x0f[(size_t)row * a.d + nn];
      TILE(0, mr, c) = y;
      a.yf[(size_t)row * a.d + nn] = y;
      El<T>::st((T*)a.yg, (size_t)row * a.d + nn, y * El<T>::ld((const T*)a.post_norm, nn));
    }
    __syncthreads();
    if (tid < rows_here) {  // this workgroup's share of each row's sum of squares
      float s = 0.f;
      for (int c = 0; c < 64; ++c) s += TILE(0, tid, c) * TILE(0, tid, c);
      a.ssq[(size_t)blk * a.rows + zg * 64 + tid] = s;
    }
  } else if (OP == OP_GATEUP) {
    for (int idx = tid; idx < rows_here * BW; idx += (int)blockDim.x) {
      const int mr = idx / BW, c = idx % BW, nn = blk * BW + c, row = zg * 64 + mr;
      if (nn >= p.N) continue;
      const float r = s_rstd[mr];
      const float g = TILE(0, mr, c) * r, u = TILE(NW - 1, mr, c) * r;
      El<T>::st((T*)a.act, xpk_index<T>(row, nn, (a.F + El<T>::KSTEP - 1) / El<T>::KSTEP), g / (1.0f + expf(-g)) * u);
    }
  } else {  // OP_DOWN
    for (int idx = tid; idx < rows_here * BW; idx += (int)blockDim.x) {
      const int mr = idx / BW, c = idx % BW, nn = blk * BW + c, row = zg * 64 + mr;
      if (nn >= p.N) continue;
      const float h = TILE(0, mr, c) + a.yf[(size_t)row * a.d + nn];
      if (a.mode == MODE_LEVEL) {
        El<T>::st((T*)a.feat, ((size_t)a.depth * a.B * a.k + row) * a.d + nn, h);
        if (a.lm_px) El<T>::st((T*)a.xpk, xpk_index<T>(row, nn, a.d / El<T>::KSTEP), h);
      } else {
        El<T>::st((T*)a.ext_h, (size_t)row * a.d + nn, h);
        const int b = row / a.RS, i = row % a.RS;
        if (i == ext_alen(a, b) - 1) El<T>::st((T*)a.root_feat, (size_t)b * a.d + nn, h);
      }
    }
  }
#undef TILE
}

template <typename T, int OP, int MT, int CTW>
__global__ void __launch_bounds__(CTW * GW_KSW * 64) k_gemm(RoundArgs a, GemmPlan p) {
  constexpr int THREADS = CTW * GW_KSW * 64;  // CTW column tiles x GW_KSW K slices
  constexpr int NW = (OP == OP_GATEUP) ? 2 : 1;
  constexpr int KS = El<T>::KSTEP;
  constexpr int PER = El<T>::PER16;
  constexpr int ES = (int)sizeof(T);
  constexpr int ROWS = MT * 16;
  constexpr bool HL = OP == OP_QKV && sizeof(T) == 2;  // x0 as two bf16 parts, two chunks per buffer
  constexpr int NPART = HL ? 2 : 1;
  constexpr int BU = gw_bu(NW, HL);          // k-steps per wave per chunk
  constexpr int KC = GW_KSW * BU * KS;       // chunk of K: every slice's k-steps
  constexpr int XST = KC * ES + 16;          // LDS row stride: an m-tile's 16 rows on different banks
  constexpr int XBUF = ROWS * XST;           // one X chunk
  constexpr int NPC = KC / PER;              // 16-byte pieces per row of a chunk
  constexpr int XP = (ROWS * NPC + THREADS - 1) / THREADS;  // pieces per thread
  // two X chunks [ROWS][KC] (double buffer); then the K-slice partials; then
  // the output tile
  extern __shared__ __attribute__((aligned(16))) unsigned char xs[];
  __shared__ const T* rsrc[ROWS];  // FC: the source row of each row
  __shared__ float s_rstd[ROWS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ct = wave % CTW, ks = wave / CTW;  // column tile, K slice (of GW_KSW)
  const int c = lane & 15, g = lane >> 4;
  // workgroup -> (column block, split, row group): XCD x (blocks x, x+8,
  // ...) takes a contiguous run, the row groups (which read the same
  // weights) and the splits of one column block adjacent
  const int nbz = p.nblk * p.S * p.zg, bpx = (nbz + 7) / 8;
  const int lb = (int)(blockIdx.x & 7) * bpx + (int)(blockIdx.x >> 3);
  if (lb >= nbz) return;
  const int zg = lb % p.zg, split = (lb / p.zg) % p.S, blk = lb / (p.zg * p.S);
  const int cl = ct * 16 + c;
  const int K = p.K;

  // ---- this lane's packed weight tile, CTW*blk + ct (a tile past the last
  // reads tile 0, discarded; rows past N within a tile are zero)
  const int nks = (K + KS - 1) / KS;
  const T* wr[NW];
  {
    const int t = CTW * blk + ct, tt = t < (p.N + 15) / 16 ? t : 0;
    if (OP == OP_QKV) wr[0] = qkv_tile<T>(a, tt, nks, lane);
    if (OP == OP_FC) wr[0] = wtile_base<T>(a.fc_w, nks, tt, lane);
    if (OP == OP_O) wr[0] = wtile_base<T>(a.wo, nks, tt, lane);
    if (OP == OP_GATEUP) {
      wr[0] = wtile_base<T>(a.w_gate, nks, tt, lane);
      wr[NW - 1] = wtile_base<T>(a.w_up, nks, tt, lane);
    }
    if (OP == OP_DOWN) wr[0] = wtile_base<T>(a.w_down, nks, tt, lane);
  }

  // gate/up: the RMSNorm statistic of this z-group's rows (loads issued now)
  const float ssq_part = OP == OP_GATEUP && p.S == 1 ? ssq_prefetch(a, p, zg, tid, ROWS) : 0.f;
  // down, extend: the sequence state advances here (the prefix grows by the
  // accepted length, the bonus token becomes the next root).  Nothing in this
  // launch reads either field, so one workgroup does it without an election.
  if (OP == OP_DOWN && a.mode == MODE_EXTEND && blk == 0 && split == 0 && zg == 0)
    ext_advance_state(a, tid, THREADS);

  // ---- FC rows: the parent (level) or true (extend) feature, gathered on the
  // fly; rows past M take row 0's source
  if (OP == OP_FC && tid < ROWS) {
    const int row0 = zg * 64 + tid;
    const bool ok = row0 < p.M;
    const int row = ok ? row0 : zg * 64;  // row 0 of the group always exists
    const T* s0;
    if (a.mode == MODE_LEVEL) {
      const int b = row / a.k, j = row % a.k;
      const eagle_frontier_node& nd = a.frontier[((size_t)a.depth * a.B + b) * a.k + j];
      if (a.depth == 1) s0 = (const T*)a.root_feat + (size_t)b * a.d;
      else s0 = (const T*)a.feat + (((size_t)(a.depth - 1) * a.B + b) * a.k + clamp_slot(nd.pslot, a.k)) * a.d;
    } else {
      int tok;
      ext_row_src<T>(a, row, s0, tok);
    }
    rsrc[tid] = s0;
  }
  const int k0 = split * p.Kc;
  const int kn = min(K, k0 + p.Kc) - k0;  // this split's K range [k0, k0 + kn)
  const int nb = (kn + KC - 1) / KC;      // its chunks
  const int klast = K - PER;
  __syncthreads();

  f32x4_t acc[NW][MT];
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[w][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Weights of chunk b: this wave's BU k-steps of its slice.  Loads are
  // unconditional from clamped in-row addresses (k past the split is masked
  // at use), so that the compiler keeps an exact count of loads in flight.
  auto wload = [&](uint4 (&buf)[BU][NW], int b) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < BU; ++u)
#pragma unroll
      for (int w = 0; w < NW; ++w)
        buf[u][w] = ld16w(wr[w] + (size_t)min((k0 + b * KC) / KS + ks * BU + u, nks - 1) * wtile_elems<T>());
  };
  // X chunk b: XP 16-byte pieces per thread into registers, then into LDS.
  // Non-FC rows are rows of one activation matrix; the FC's row pointers come
  // from LDS.  Rows past M read row 0 of the group and k past K reads the
  // row's last piece: every MFMA output row depends on its own X row only,
  // products past the split are masked, and the epilogues store rows below M.
  const T* xsrc = OP == OP_QKV ? (const T*)a.x0b : OP == OP_O ? (const T*)a.attn : (const T*)a.yg;
  // The down projection's X (the SwiGLU activations) is stored packed: its
  // pieces are walked in packed order (16-row group, k-step, lane), so that
  // consecutive threads read consecutive 16 bytes; a row group past M reads
  // the group's first row group instead (its rows are never stored).
  auto xpiece = [&](int q, int& r, int& pc) __attribute__((always_inline)) {
    const int i = min(tid + q * THREADS, ROWS * NPC - 1);
    if (OP == OP_DOWN) {
      constexpr int SPC = KC / KS;  // k-steps per chunk
      const int z = i / (SPC * 64), rem = i - z * (SPC * 64), sl = rem >> 6, l = rem & 63;
      r = 16 * z + (l & 15);
      pc = sl * (KS / PER) + (l >> 4);
    } else {
      r = i / NPC;
      pc = i % NPC;
    }
  };
  // (HL: part 1 is x0's low part, its pieces at the same places of the
  // buffer's second chunk)
  auto xload = [&](uint4 (&xr)[NPART][XP], int b) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < XP; ++q) {
      int r, pc;
      xpiece(q, r, pc);
      const int k = min(k0 + b * KC + pc * PER, klast);
      const T* src;
      if (OP == OP_FC) {
        src = rsrc[r] + k;
      } else if (OP == OP_DOWN) {
        const int row = zg * 64 + r;
        src = (const T*)a.act + xpk_index<T>(row < ((p.M + 15) & ~15) ? row : zg * 64 + (r & 15), k, nks);
      } else {
        const int row = zg * 64 + r;
        src = xsrc + (size_t)(row < p.M ? row : zg * 64) * K + k;
      }
      xr[0][q] = ld16g(src);
      if constexpr (HL) xr[NPART - 1][q] = ld16g((const T*)a.x0l + (src - xsrc));
    }
  };
  // unconditional stores: a slot past the chunk repeats the last piece (same
  // value, same place), so no load is sunk into a branch of its own
  auto xstore = [&](const uint4 (&xr)[NPART][XP], int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < XP; ++q) {
      int r, pc;
      xpiece(q, r, pc);
#pragma unroll
      for (int h = 0; h < NPART; ++h) *(uint4*)(xs + (buf * NPART + h) * XBUF + r * XST + pc * 16) = xr[h][q];
    }
  };
  auto comp = [&](const uint4 (&wbuf)[BU][NW], int b, int buf) __attribute__((always_inline)) {
    const unsigned char* xrow = xs + buf * NPART * XBUF + c * XST;
#pragma unroll
    for (int u = 0; u < BU; ++u) {
      const int kc = (ks * BU + u) * KS + g * PER;  // offset in the chunk
      const bool kin = b * KC + kc < kn;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int h = 0; h < NPART; ++h) {
          const uint4 xf = mask4(*(const uint4*)(xrow + h * XBUF + mt * 16 * XST + kc * ES), kin);
#pragma unroll
          for (int w = 0; w < NW; ++w) acc[w][mt] = mma16(xf, wbuf[u][w], acc[w][mt], T());
        }
      }
    }
  };

  // ---- pipeline over the split's chunks: chunk b is computed from X buffer
  // b % 2 and weight buffer b % 2 while chunk b+1's X (registers, then the
  // other LDS buffer) and weights are in flight; chunk b+2's loads are issued
  // after chunk b's MFMAs, and one barrier per chunk hands the X buffers over.
  // Loads past the last chunk read clamped in-range addresses and are unused.
  uint4 xr[NPART][XP];
  uint4 wa[BU][NW], wb[BU][NW];
  // (scheduling barriers keep the prologue's loads in the loop's order: X
  // chunk, then that chunk's weights)
  xload(xr, 0);
  __builtin_amdgcn_sched_barrier(0);
  wload(wa, 0);
  __builtin_amdgcn_sched_barrier(0);
  xstore(xr, 0);
  xload(xr, 1);
  __builtin_amdgcn_sched_barrier(0);
  wload(wb, 1);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  // the loop body is one straight block (two chunks) and the last one or two
  // chunks are peeled, so that every entry sees the same loads in flight and
  // the compiler's wait counts stay exact
  int b = 0;
  for (; b + 2 < nb; b += 2) {
    comp(wa, b, 0);
    xstore(xr, 1);
    xload(xr, b + 2);
    __builtin_amdgcn_sched_barrier(0);
    wload(wa, b + 2);
    __syncthreads();
    comp(wb, b + 1, 1);
    xstore(xr, 0);
    xload(xr, b + 3);
    __builtin_amdgcn_sched_barrier(0);
    wload(wb, b + 3);
    __syncthreads();
  }
  if (b < nb) comp(wa, b, 0);
  if (b + 1 < nb) {
    xstore(xr, 1);
    __syncthreads();
    comp(wb, b + 1, 1);
  }
  __syncthreads();  // every wave is done with the X buffers

  // ---- the K slices meet in LDS (over the X buffers); slice 0's waves sum
  // them in slice order
  f32x4_t* red = (f32x4_t*)xs;  // [slice 1..GW_KSW-1][column tile][NW * MT][64]
  if (ks != 0) {
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        red[(((ks - 1) * CTW + ct) * (NW * MT) + w * MT + mt) * WAVE + lane] = acc[w][mt];
  }
  __syncthreads();
  const bool fin = ks == 0;
  if (fin) {
#pragma unroll
    for (int s = 0; s < GW_KSW - 1; ++s)
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[w][mt] += red[((s * CTW + ct) * (NW * MT) + w * MT + mt) * WAVE + lane];
  }

  // ---- split K: the partials go to the workspace and k_gemm_fin sums them
  if (p.S > 1) {
    if (fin) {
      float* part = a.gpart + (((((size_t)zg * p.nblk + blk) * p.S + split) * CTW + ct) * (NW * MT) * 64) * 4;
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          *(f32x4_t*)(part + ((size_t)(w * MT + mt) * 64 + lane) * 4) = acc[w][mt];
    }
    return;
  }
  __syncthreads();  // the output tile is over the slice partials
  float* tile = (float*)xs;  // [NW][ROWS][65]
  if (fin) {
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) tile[(w * ROWS + mt * 16 + g * 4 + r) * 65 + cl] = acc[w][mt][r];
  }
  if (OP == OP_GATEUP) rstd_finish<ROWS>(a, tile + NW * ROWS * 65, ssq_part, s_rstd, tid);
  __syncthreads();
  gemm_epilogue<T, OP, MT, CTW>(a, p, tile, s_rstd, blk, zg, tid);
}

// Sum of a split GEMM's partials for one 64-column block of one z-group, in
// split order (one (column tile, m-tile, lane) per thread, every split's
// loads in flight together), then the op's epilogue.
template <typename T, int OP, int MT>
__global__ void __launch_bounds__(GW_FIN_THREADS) k_gemm_fin(RoundArgs a, GemmPlan p) {
  constexpr int NW = (OP == OP_GATEUP) ? 2 : 1;
  constexpr int ROWS = MT * 16;
  __shared__ float tile[NW * ROWS * 65 + ROWS * 16];
  __shared__ float s_rstd[ROWS];
  const int tid = threadIdx.x, lane = tid & 63, c = lane & 15, g = lane >> 4;
  const int blk = blockIdx.x, zg = blockIdx.z;
  const float ssq_part = OP == OP_GATEUP ? ssq_prefetch(a, p, zg, tid, ROWS) : 0.f;
  if (tid < 4 * MT * WAVE) {
    const int ct = tid / (MT * WAVE), mt = (tid / WAVE) % MT;
    const float* base = a.gpart + ((size_t)zg * p.nblk + blk) * p.S * 4 * (NW * MT) * 64 * 4;
    f32x4_t sum[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) sum[w] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < p.S; s0 += 8) {
      f32x4_t v[8][NW];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float* ps = base + (((size_t)min(s0 + u, p.S - 1) * 4 + ct) * (NW * MT) * 64) * 4;
#pragma unroll
        for (int w = 0; w < NW; ++w) v[u][w] = *(const f32x4_t*)(ps + ((size_t)(w * MT + mt) * 64 + lane) * 4);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int w = 0; w < NW; ++w)
          if (s0 + u < p.S) sum[w] += v[u][w];
    }
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int r = 0; r < 4; ++r) tile[(w * ROWS + mt * 16 + g * 4 + r) * 65 + ct * 16 + c] = sum[w][r];
  }
  if (OP == OP_GATEUP) rstd_finish<ROWS>(a, tile + NW * ROWS * 65, ssq_part, s_rstd, tid);
  __syncthreads();
  gemm_epilogue<T, OP, MT, 4>(a, p, tile, s_rstd, blk, zg, tid);
}

template <typename T, int OP, int CTW>
static void launch_main(const RoundArgs& a, const GemmPlan& p, hipStream_t s) {
  const int nbz = p.nblk * p.S * p.zg;
  const dim3 grid((nbz + 7) / 8 * 8), block(CTW * GW_KSW * 64);
  const size_t lds = gemm_lds_bytes(p, (int)sizeof(T));
  switch (p.mt) {
    case 1: hipLaunchKernelGGL((k_gemm<T, OP, 1, CTW>), grid, block, lds, s, a, p); break;
    case 2: hipLaunchKernelGGL((k_gemm<T, OP, 2, CTW>), grid, block, lds, s, a, p); break;
    case 3: hipLaunchKernelGGL((k_gemm<T, OP, 3, CTW>), grid, block, lds, s, a, p); break;
    default: hipLaunchKernelGGL((k_gemm<T, OP, 4, CTW>), grid, block, lds, s, a, p); break;
  }
}

template <typename T, int OP>
static hipError_t launch_op(const RoundArgs& a, const GemmPlan& p, hipStream_t s) {
  if (p.rows) {  // 17..64 rows: the streaming GEMM writes partials, k_gemm_fin finishes
    if (sizeof(T) != 2) return hipErrorInvalidValue;
    const hipError_t e = launch_gemm_rows(OP, a, p, s);
    if (e != hipSuccess) return e;
    switch (p.mt) {
      case 1: hipLaunchKernelGGL((k_gemm_fin<T, OP, 1>), dim3(p.nblk), dim3(GW_FIN_THREADS), 0, s, a, p); break;
      case 2: hipLaunchKernelGGL((k_gemm_fin<T, OP, 2>), dim3(p.nblk), dim3(GW_FIN_THREADS), 0, s, a, p); break;
      case 3: hipLaunchKernelGGL((k_gemm_fin<T, OP, 3>), dim3(p.nblk), dim3(GW_FIN_THREADS), 0, s, a, p); break;
      default: hipLaunchKernelGGL((k_gemm_fin<T, OP, 4>), dim3(p.nblk), dim3(GW_FIN_THREADS), 0, s, a, p); break;
    }
    return hipGetLastError();
  }
  if (p.tiled) {  // many rows: the tiled MFMA GEMM writes partials, k_gemm_fin finishes
    if (sizeof(T) != 2 || p.mt != 4) return hipErrorInvalidValue;
    const hipError_t e = launch_gemm_tiled(OP, a, p, s);
    if (e != hipSuccess) return e;
    if (OP == OP_GATEUP && p.S == 1) return hipSuccess;  // epilogue in the tiled launch
    hipLaunchKernelGGL((k_gemm_fin<T, OP, 4>), dim3(p.nblk, 1, p.zg), dim3(GW_FIN_THREADS), 0, s, a, p);
    return hipGetLastError();
  }
  if constexpr (OP != OP_O) {
    if (p.ct == 3) {
      if (p.S != 1) return hipErrorInvalidValue;  // three-tile blocks are never split
      launch_main<T, OP, 3>(a, p, s);
      return hipGetLastError();
    }
  }
  if (p.ct != 4) return hipErrorInvalidValue;
  launch_main<T, OP, 4>(a, p, s);
  if (p.S > 1) {
    const dim3 fgrid(p.nblk, 1, p.zg);
    switch (p.mt) {
      case 1: hipLaunchKernelGGL((k_gemm_fin<T, OP, 1>), fgrid, dim3(GW_FIN_THREADS), 0, s, a, p); break;
      case 2: hipLaunchKernelGGL((k_gemm_fin<T, OP, 2>), fgrid, dim3(GW_FIN_THREADS), 0, s, a, p); break;
      case 3: hipLaunchKernelGGL((k_gemm_fin<T, OP, 3>), fgrid, dim3(GW_FIN_THREADS), 0, s, a, p); break;
      default: hipLaunchKernelGGL((k_gemm_fin<T, OP, 4>), fgrid, dim3(GW_FIN_THREADS), 0, s, a, p); break;
    }
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_t(int op, const RoundArgs& a, const GemmPlan& p, hipStream_t s) {
  switch (op) {
    case OP_FC: return launch_op<T, OP_FC>(a, p, s);
    case OP_QKV: return launch_op<T, OP_QKV>(a, p, s);
    case OP_O: return launch_op<T, OP_O>(a, p, s);
    case OP_GATEUP: return launch_op<T, OP_GATEUP>(a, p, s);
    default: return launch_op<T, OP_DOWN>(a, p, s);
  }
}

hipError_t launch_gemm(int op, const RoundArgs& a, const GemmPlan& p, hipStream_t s) {
  return a.dtype == EAGLE_BF16 ? launch_t<bf16_t>(op, a, p, s) : launch_t<float>(op, a, p, s);
}

}  // namespace eg

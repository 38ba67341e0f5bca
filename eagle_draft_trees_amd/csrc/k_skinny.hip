// Weight-streaming GEMMs of the draft layer where at most 16 rows are
// forwarded (a drafting level's frontier, or the extend's accepted paths):
//
//   Y[M][N] = X[M][K] * W[N][K]^T,  M <= 16
//
// At this shape every byte of W is used once, so the kernel is bound by
// streaming W from HBM; what limits a simple design is latency, not
// arithmetic: a few serialized memory round trips per workgroup (staging,
// cross-workgroup split-K hand-off) cost more than the streaming itself.  So:
//
//  * one workgroup holds CT column tiles of 16 columns and splits K over KSW
//    waves per tile (CT * KSW <= 16 waves); the K partial sums meet in LDS
//    and one wave per tile finishes them in slice order (deterministic), so
//    there is no cross-workgroup hand-off at all;
//  * each lane loads its 16 bytes of W (16 columns x 64 bytes per wave
//    instruction) straight into registers, BU k-steps per batch, two batches
//    in flight (ping-pong buffers); loads are unconditional from clamped
//    in-bounds addresses, and products past the slice are masked to zero;
//  * X comes from an LDS copy of its 16 rows staged once per workgroup when
//    that fits (K <= 4096 bf16); otherwise each lane also loads its 16 bytes
//    of X (an L2 hit) per k-step.  X loads share the memory queue with the
//    weight loads and cost about a quarter of the streaming rate, so the LDS
//    copy is preferred;
//  * the layer's elementwise work is fused into the epilogue (bias, RoPE and
//    the in-tree KV write, residuals, the SwiGLU), and the RMSNorm statistic
//    is finished where it is consumed: the O epilogue writes per-workgroup
//    row sums of squares, and every gate/up workgroup reduces them itself.
//
// Draft layer of [P1] "EAGLE 推测解码为什么比 Medusa 快？" §4.1 and [P3]
// zdszero.github.io spec_medusa_eagle, "在 SGLang 里"; tree positions of the
// RoPE step per [P1] §12 item 5 (positions shared per level).
#include "skinny_core.h"

namespace eg {

// column of lane column c (0..15) of tile t; a q/k/v tile holds 8 rotation
// pairs (i, i + hd/2) of one head so that the RoPE epilogue is lane-local
__device__ __forceinline__ int sk_col(int op, int t, int c, int hd) {
  if (op == OP_QKV) {
    const int per = hd / 16, head = t / per, j = t - head * per;
    return head * hd + (c < 8 ? 8 * j + c : hd / 2 + 8 * j + (c - 8));
  }
  return t * 16 + c;
}

// XL: X staged once in LDS (when its 16 rows fit) instead of loaded from L2
// at every k-step; the weight loop then issues only weight loads.
// (the q/k/v projection runs at most SK_QKVW waves: its two-part X staging
// needs the registers)
template <typename T, int OP, bool XL>
__global__ void __launch_bounds__((OP == OP_QKV ? SK_QKVW : SK_MAXW) * WAVE) k_skinny(RoundArgs a, SkPlan p) {
  constexpr int NW = (OP == OP_GATEUP) ? 2 : 1;  // weight streams per wave (gate and up)
  constexpr int KS = El<T>::KSTEP;
  constexpr int BU = (NW == 2) ? (XL ? 3 : 2) : 4;  // k-steps per load batch (registers permitting)
  // dynamic LDS: the X tile [16][K] (row stride K*ES + 16 bytes, so the 16
  // rows of one read fall in different banks), then reused for the K-slice
  // partial sums [wave][NW][64] once every wave is done with X
  extern __shared__ __attribute__((aligned(16))) unsigned char dyn[];
  f32x4_t* red = (f32x4_t*)dyn;
  __shared__ __attribute__((aligned(16))) float s_ssq[SK_MAXW][16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // column block: XCD x (blocks x, x+8, ...) takes a contiguous run
  const int bpx = (p.nwg + 7) / 8;  // blocks per XCD
  const int bk = (int)(blockIdx.x & 7) * bpx + (int)(blockIdx.x >> 3);
  if (bk >= p.nwg) return;
  const int ct = wave % p.CT, ks = wave / p.CT;
  const int t = bk * p.CT + ct;
  const int c = lane & 15, g = lane >> 4;
  const bool tv = t < p.ntile;
  const int n = sk_col(OP, tv ? t : 0, c, a.hd);
  const bool nv = tv && n < p.N;
  const int K = p.K;

  // ---- this lane's packed weight tile (a tile past the last reads tile 0,
  // discarded; rows past N within a tile are zero)
  const int nks = (K + KS - 1) / KS;
  const T* wr[NW];
  {
    const int tt = tv ? t : 0;
    if (OP == OP_QKV) wr[0] = qkv_tile<T>(a, tt, nks, lane);
    if (OP == OP_FC) wr[0] = wtile_base<T>(a.fc_w, nks, tt, lane);
    if (OP == OP_O) wr[0] = wtile_base<T>(a.wo, nks, tt, lane);
    if (OP == OP_GATEUP) {
      wr[0] = wtile_base<T>(a.w_gate, nks, tt, lane);
      wr[NW - 1] = wtile_base<T>(a.w_up, nks, tt, lane);
    }
    if (OP == OP_DOWN) wr[0] = wtile_base<T>(a.w_down, nks, tt, lane);
  }

  // ---- this lane's X row: row c (rows past M repeat row 0; discarded).  The
  // FC streams the feature half of W_fc over the gathered parent (level) or
  // true (extend) feature; the token half is the row's token-projection
  // table entry, added in the epilogue.
  const int xr = c < p.M ? c : 0;
  const T* x0;
  const T* x1;
  const int kswitch = K;
  __shared__ int s_tok[16];
  if (OP == OP_FC) {
    int tok;
    if (a.mode == MODE_LEVEL) {
      const int b = xr / a.k, j = xr - b * a.k;
      const eagle_frontier_node& nd = a.frontier[((size_t)a.depth * a.B + b) * a.k + j];
      tok = nd.token;
      if (a.depth == 1) x0 = (const T*)a.root_feat + (size_t)b * a.d;
      else x0 = (const T*)a.feat + (((size_t)(a.depth - 1) * a.B + b) * a.k + clamp_slot(nd.pslot, a.k)) * a.d;
    } else {  // extend: the true feature of the path node and the next token
      ext_row_src<T>(a, xr, x0, tok);
    }
    x1 = x0;
    if (tid < 16) s_tok[tid] = clamp_tok(tok, a.V, a.err);  // wave 0, lane = row c
  } else if (OP == OP_DOWN) {  // packed activations: this lane's piece of k-step 0 (row c;
    // rows past M read row 0, so the block's padding lines are never fetched)
    x0 = (const T*)a.act + (size_t)xr * KS + g * El<T>::PER16;
    x1 = x0;
  } else {
    const T* xb = (OP == OP_QKV) ? (const T*)a.x0b : (OP == OP_O) ? (const T*)a.attn : (const T*)a.yg;
    x0 = xb + (size_t)xr * K;
    x1 = x0;
  }

  // ---- gate/up: prefetch this thread's share of the O epilogue's RMSNorm
  // partials (row tid%16, partials tid/16 + j*QJ); they are summed after the
  // main loop, so their latency hides behind the weight stream
  constexpr int SQ = 8;
  float sqv[SQ];
  const int qrow = tid & 15, qj = tid >> 4, QJ = (int)(blockDim.x >> 4);
  if (OP == OP_GATEUP) {
#pragma unroll
    for (int u = 0; u < SQ; ++u)
      sqv[u] = a.ssq[(size_t)min(qj + u * QJ, p.nps - 1) * a.rows + min(qrow, p.M - 1)];
  }

  // ---- the epilogue's own inputs, loaded now so that their latency hides
  // behind the weight stream: O the residual x0 and the norm gain, down the
  // residual y, q/k/v the prefix length of each row's sequence (for RoPE)
  float pre[4] = {0.f, 0.f, 0.f, 0.f};
  float gain = 0.f;
  int pre_p[4] = {0, 0, 0, 0};
  if (OP == OP_O || OP == OP_DOWN) {
    const float* res = OP == OP_O ? a.x0f : a.yf;
    const int nn = nv ? n : 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) pre[r] = res[(size_t)min(4 * g + r, p.M - 1) * a.d + nn];
    if (OP == OP_O) gain = El<T>::ld((const T*)a.post_norm, nn);
  }
  double inv = 0.0;  // q/k/v: this lane's RoPE frequency
  if (OP == OP_QKV) {
#pragma unroll
    for (int r = 0; r < 4; ++r) pre_p[r] = a.prefix_len[min(4 * g + r, p.M - 1) / a.RS];
    const int tt = tv ? t : 0, per = a.hd / 16, j = tt - (tt / per) * per;
    inv = a.rope[8 * j + (c < 8 ? c : c - 8)];
  }

  // ---- this wave's K slice: k-steps [s0k, s1k)
  const int s0k = (int)((long)ks * nks / p.KSW), s1k = (int)((long)(ks + 1) * nks / p.KSW);
  f32x4_t acc[NW];
  const int nbu = ((nks + p.KSW - 1) / p.KSW + BU - 1) / BU;
  if constexpr (OP == OP_QKV && sizeof(T) == 2) {  // x0 as its two bf16 parts
    sk_stream_hl<T, BU, XL>(wr[0], (const T*)a.x0b, (const T*)a.x0l, K, ks, p.KSW, dyn, acc[0], p.M);
  } else {
    sk_stream<T, NW, BU, XL, OP == OP_DOWN>(wr, x0, x1, kswitch, K, s0k, s1k, nbu, dyn, acc, x0 - (size_t)xr * K,
                                            p.M);
  }

  // ---- K slices meet in LDS; wave (ct, slice 0) sums them in slice order
  if (XL) __syncthreads();  // every wave is done reading the X tile it overwrites
#pragma unroll
  for (int w = 0; w < NW; ++w) red[(wave * NW + w) * WAVE + lane] = acc[w];
  if (OP == OP_GATEUP) {  // RMSNorm sums: this thread's partials, then the wave's 4 per row
    float s = 0.f;
#pragma unroll
    for (int u = 0; u < SQ; ++u)
      if (qj + u * QJ < p.nps) s += sqv[u];
    for (int q = qj + SQ * QJ; q < p.nps; q += QJ) s += a.ssq[(size_t)q * a.rows + min(qrow, p.M - 1)];
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    if (lane < 16) s_ssq[wave][lane] = s;
  }
  __syncthreads();
  // the epilogue is spread over the tile's first waves: wave ks (< 4) finishes
  // the rows 4g+r with r % KSW == ks of every lane group (all four when KSW is 1)
  const bool fin = ks < 4;
  auto mine = [&](int r) __attribute__((always_inline)) { return r % p.KSW == ks; };
  f32x4_t v[NW];
#pragma unroll
  for (int w = 0; w < NW; ++w) v[w] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (fin) {  // the first MS slices' reads in flight together (a slot past KSW repeats the last, unused)
    constexpr int MS = NW == 2 ? 8 : (OP == OP_QKV ? SK_QKVW : SK_MAXW);
    f32x4_t rv[MS][NW];
#pragma unroll
    for (int s = 0; s < MS; ++s)
#pragma unroll
      for (int w = 0; w < NW; ++w) rv[s][w] = red[((min(s, p.KSW - 1) * p.CT + ct) * NW + w) * WAVE + lane];
#pragma unroll
    for (int s = 0; s < MS; ++s)
#pragma unroll
      for (int w = 0; w < NW; ++w)
        if (s < p.KSW) v[w] += rv[s][w];  // slice order
    for (int s = MS; s < p.KSW; ++s)
#pragma unroll
      for (int w = 0; w < NW; ++w) v[w] += red[((s * p.CT + ct) * NW + w) * WAVE + lane];
  }

  // ---- epilogues; lane holds rows 4g..4g+3 of column n
  if (OP == OP_FC) {
    if (fin && nv) {
      const float bias = El<T>::ld((const T*)a.fc_b, n);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * g + r;
        if (!mine(r) || row >= p.M) continue;
        const float x = v[0][r] + a.tok_proj[(size_t)s_tok[row] * a.d + n] + bias;
        st_x0<T>(a, (size_t)row * a.d + n, x);
      }
    }
  } else if (OP == OP_QKV) {
    if (fin) {
      const int per = a.hd / 16, head = t / per, j = t - head * per, half = a.hd / 2;
      const bool low = c < 8;
      const int fi = 8 * j + (low ? c : c - 8);  // frequency index within the half
      const bool rot = head < a.H + a.Hkv;
      int lastpos = INT_MIN;  // rows of one position (a level's rows of one sequence) share the angle
      float sn = 0.f, cs = 1.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (!mine(r)) continue;  // wave-uniform
        const float own = v[0][r];
        const float other = __shfl_xor(own, 8);
        const int row = 4 * g + r;
        if (!tv || row >= p.M) continue;
        float lo = low ? own : other, hi = low ? other : own;
        // levels: a frontier slot at tree position P-1+depth; extend: row i of
        // the sequence at position P+i, appended to the prefix cache
        const bool lv = a.mode == MODE_LEVEL;
        const int bb = row / a.RS, slot = row - bb * a.RS;
        const int P = clamp_prefix(pre_p[r], a);
        if (rot) {
          const int pos = lv ? P - 1 + a.depth : P + slot;
          if (pos != lastpos) {
            rope_sincos(pos, inv, sn, cs);
            lastpos = pos;
          }
          const float nlo = lo * cs - hi * sn, nhi = hi * cs + lo * sn;
          lo = nlo;
          hi = nhi;
        }
        const float val = low ? lo : hi;
        const int idx = low ? fi : fi + half;
        if (head < a.H) {
          a.q[(size_t)row * (a.H * a.hd) + head * a.hd + idx] = val;
        } else {
          const bool isk = head < a.H + a.Hkv;
          const int kvh = isk ? head - a.H : head - a.H - a.Hkv;
          if (lv)  // in-tree K/V are kept in fp32 (workspace)
            ((float*)(isk ? a.tk : a.tv))[((((size_t)bb * a.D + a.depth) * a.k + slot) * a.Hkv + kvh) * a.hd + idx] = val;
          else
            El<T>::st((T*)(isk ? a.k_cache : a.v_cache), (((size_t)bb * a.max_prefix + P + slot) * a.Hkv + kvh) * a.hd + idx, val);
        }
      }
    }
  } else if (OP == OP_O) {
    float sq[4] = {0.f, 0.f, 0.f, 0.f};
    if (fin) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * g + r;
        if (!mine(r) || !nv || row >= p.M) continue;
        const float y = v[0][r] + pre[r];
        a.yf[(size_t)row * a.d + n] = y;
        El<T>::st((T*)a.yg, (size_t)row * a.d + n, y * gain);
        sq[r] = y * y;
      }
      // sum over the tile's 16 columns (the 16 lanes of one DPP row)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (!mine(r)) continue;  // wave-uniform
#pragma unroll
        for (int st = 0; st < 4; ++st) sq[r] += __uint_as_float(dpp_u32(__float_as_uint(sq[r]), st));
        if (c == 0) s_ssq[ct][4 * g + r] = sq[r];
      }
    }
    __syncthreads();
    if (tid < p.M) {
      float s = 0.f;
      for (int q = 0; q < p.CT; ++q) s += s_ssq[q][tid];
      a.ssq[(size_t)bk * a.rows + tid] = s;
    }
  } else if (OP == OP_GATEUP) {
    if (fin && nv) {
      // the rows' sums of squares: every wave's four (rows 4g..4g+3) read together,
      // then added in wave order
      const int nwv = (int)(blockDim.x >> 6);
      float4 sw[SK_MAXW];
#pragma unroll
      for (int w = 0; w < SK_MAXW; ++w) sw[w] = *(const float4*)&s_ssq[min(w, nwv - 1)][4 * g];
      asm volatile("" ::: "memory");
      float ssr[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < SK_MAXW; ++w)
        if (w < nwv) {
          ssr[0] += sw[w].x;
          ssr[1] += sw[w].y;
          ssr[2] += sw[w].z;
          ssr[3] += sw[w].w;
        }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * g + r;
        if (!mine(r) || row >= p.M) continue;
        const float ss = ssr[r];
        const float rs = 1.0f / sqrtf(ss / (float)a.d + a.eps);
        const float gg = v[0][r] * rs, uu = v[NW - 1][r] * rs;
        El<T>::st((T*)a.act, xpk_index<T>(row, n, (a.F + KS - 1) / KS), gg / (1.0f + expf(-gg)) * uu);
      }
    }
  } else {  // OP_DOWN: predicted feature of the level or extend row (no final norm)
    if (fin && nv) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * g + r;
        if (!mine(r) || row >= p.M) continue;
        const float h = v[0][r] + pre[r];
        if (a.mode == MODE_LEVEL) {
          El<T>::st((T*)a.feat, ((size_t)a.depth * a.B * a.k + row) * a.d + n, h);
        } else {  // extend: row alen-1 of a sequence is its next root feature
          El<T>::st((T*)a.ext_h, (size_t)row * a.d + n, h);
          const int bb = row / a.RS, i = row - bb * a.RS;
          if (i == ext_alen(a, bb) - 1) El<T>::st((T*)a.root_feat, (size_t)bb * a.d + n, h);
        }
      }
    }
    // nothing in this launch reads prefix_len or root_token
    if (a.mode == MODE_EXTEND && bk == 0) ext_advance_state(a, tid, (int)blockDim.x);
  }
}

template <typename T, int OP>
static void launch_sk_op(const RoundArgs& a, const SkPlan& p, hipStream_t s) {
  constexpr int NW = (OP == OP_GATEUP) ? 2 : 1;
  const dim3 grid((p.nwg + 7) / 8 * 8), block(WAVE * p.CT * p.KSW);
  const size_t red = (size_t)WAVE * p.CT * p.KSW * NW * sizeof(f32x4_t);
  if (p.xlds && OP != OP_DOWN) {  // the down projection's X is packed, never staged
    const size_t xb = OP == OP_QKV && sizeof(T) == 2 ? sk_hl_tile_bytes(p.K, 2) : sk_xtile_bytes(p.K, (int)sizeof(T));
    hipLaunchKernelGGL((k_skinny<T, OP, OP != OP_DOWN>), grid, block, xb > red ? xb : red, s, a, p);
  } else {
    hipLaunchKernelGGL((k_skinny<T, OP, false>), grid, block, red, s, a, p);
  }
}

template <typename T>
static hipError_t launch_sk_t(int op, const RoundArgs& a, const SkPlan& p, hipStream_t s) {
  switch (op) {
    case OP_FC: launch_sk_op<T, OP_FC>(a, p, s); break;
    case OP_QKV: launch_sk_op<T, OP_QKV>(a, p, s); break;
    case OP_O: launch_sk_op<T, OP_O>(a, p, s); break;
    case OP_GATEUP: launch_sk_op<T, OP_GATEUP>(a, p, s); break;
    default: launch_sk_op<T, OP_DOWN>(a, p, s); break;
  }
  return hipGetLastError();
}

hipError_t launch_skinny(int op, const RoundArgs& a, const SkPlan& p, hipStream_t s) {
  return a.dtype == EAGLE_BF16 ? launch_sk_t<bf16_t>(op, a, p, s) : launch_sk_t<float>(op, a, p, s);
}

}  // namespace eg

// Skinny weight-streaming GEMMs of the draft layer on MFMA, with the layer's
// elementwise work fused into the loaders and epilogues.
//
//   Y[M][N] = X[M][K] * W[N][K]^T,  M = frontier rows (B*k) or extend rows (B*m)
//
// At drafting shapes M is 1..64 while W is megabytes, so every kernel here is
// bound by streaming W from HBM once.  A workgroup is four waves = 64 adjacent
// output columns over one K range.  It stages the X rows of that K range in
// LDS chunk by chunk (shared by the four waves), so the only global loads in
// the main loop are W's: one 16-byte load per lane per k-step (16 rows x 64
// contiguous bytes per wave instruction), eight k-steps in flight, each fed to
// a 16x16 MFMA (bf16: v_mfma_f32_16x16x32_bf16; fp32: four 16x16x4 steps)
// with its A operand read from LDS.  When the grid would be too small to keep
// HBM busy, K is split across workgroups; each split writes fp32 partials and
// the last workgroup to arrive (counter in the workspace) sums them in split
// order -- deterministic, no float atomics -- and runs the epilogue.
//
// Fused steps (draft head of [P1] "EAGLE 推测解码为什么比 Medusa 快？" §4.1 and
// [P3] zdszero.github.io spec_medusa_eagle, "在 SGLang 里"):
//   FC      X = [parent feature || embed[token]] gathered on the fly (no
//           concatenated copy); epilogue + bias -> x0 (fp32 residual, dtype copy)
//   QKV     epilogue applies RoPE at the row's tree position to q and k
//           ([P1] §12 item 5: positions shared per level) and writes k, v
//           straight into the in-tree slot (levels) or the prefix cache (extend)
//   O       epilogue adds the residual x0, keeps y, emits y*gain for the MLP
//           and per-block sums of squares; the grid's last block turns them
//           into the RMSNorm 1/rms per row
//   GATEUP  two weight streams per wave (gate and up rows of the same 16
//           columns); epilogue silu(g/rms) * (u/rms)
//   DOWN    epilogue adds the residual y -> predicted feature (no final norm);
//           the extend also writes the next root feature and advances the
//           sequence state in the grid's last block
#include "eagle_internal.h"

namespace eg {

__device__ __forceinline__ int qkv_col(int blk, int c, int hd) {
  const int per = hd / 64, head = blk / per, j = blk % per, half = hd / 2;
  const int off = (c < 32) ? (32 * j + c) : (half + 32 * j + (c - 32));
  return head * hd + off;
}

template <typename T, int OP, int MT>
__global__ void __launch_bounds__(BLOCK) k_gemm(RoundArgs a, GemmPlan p) {
  constexpr int NW = (OP == OP_GATEUP) ? 2 : 1;
  constexpr int KS = El<T>::KSTEP;
  constexpr int PER = El<T>::PER16;
  constexpr int ES = (int)sizeof(T);
  constexpr int ROWS = MT * 16;
  constexpr int XRB = (4096 / MT) & ~15;  // bytes of X per row in LDS per staged chunk
  constexpr int XST = XRB + 16;   // LDS row stride: 16 rows of one m-tile hit disjoint banks
  static_assert(NW * ROWS * 65 * 4 <= ROWS * XST, "epilogue tile aliases the X tile");
  __shared__ __attribute__((aligned(16))) unsigned char xs[ROWS * XST];
  __shared__ const T* rsrc[2][ROWS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int blk = blockIdx.x, split = blockIdx.y, zg = blockIdx.z;
  const int cl = wave * 16 + (lane & 15);
  const int K = p.K;

  // ---- this lane's output column and weight rows
  int n;
  bool nv;
  const T* wr[NW];
  if (OP == OP_QKV) {
    n = qkv_col(blk, cl, a.hd);
    nv = true;
    const int hq = a.H * a.hd, hk = a.Hkv * a.hd;
    if (n < hq) wr[0] = (const T*)a.wq + (size_t)n * K;
    else if (n < hq + hk) wr[0] = (const T*)a.wk + (size_t)(n - hq) * K;
    else wr[0] = (const T*)a.wv + (size_t)(n - hq - hk) * K;
  } else {
    n = blk * 64 + cl;
    nv = n < p.N;
    const size_t off = (size_t)(nv ? n : 0) * K;
    if (OP == OP_FC) wr[0] = (const T*)a.fc_w + off;
    if (OP == OP_O) wr[0] = (const T*)a.wo + off;
    if (OP == OP_GATEUP) { wr[0] = (const T*)a.w_gate + off; wr[NW - 1] = (const T*)a.w_up + off; }
    if (OP == OP_DOWN) wr[0] = (const T*)a.w_down + off;
  }

  // ---- X rows of this z-group; the FC gathers [parent feature || embed[token]]
  if (tid < ROWS) {
    const int row = zg * 64 + tid;
    const T* s0 = nullptr;
    const T* s1 = (const T*)a.embed;
    if (row < p.M) {
      if (OP == OP_FC) {
        int tok;
        if (a.mode == MODE_LEVEL) {
          const int b = row / a.k, j = row % a.k;
          const eagle_frontier_node& nd = a.frontier[((size_t)a.depth * a.B + b) * a.k + j];
          tok = nd.token;
          if (a.depth == 1) s0 = (const T*)a.root_feat + (size_t)b * a.d;
          else s0 = (const T*)a.feat + (((size_t)(a.depth - 1) * a.B + b) * a.k + clamp_slot(nd.pslot, a.k)) * a.d;
        } else {
          const int b = row / a.m, i = row % a.m;
          int alen = a.accept_len[b];
          alen = alen < 1 ? 1 : (alen > a.D + 1 ? a.D + 1 : alen);
          const int last = alen - 1, ii = i < last ? i : last;
          const int* path = a.accept_path + (size_t)b * (a.D + 1);
          int pi = path[ii];
          pi = pi < 0 ? 0 : (pi >= a.m ? a.m - 1 : pi);
          s0 = (const T*)a.true_feat + ((size_t)b * a.m + pi) * a.d;
          if (i < last) {
            int pn = path[i + 1];
            pn = pn < 0 ? 0 : (pn >= a.m ? a.m - 1 : pn);
            tok = a.tokens[(size_t)b * a.m + pn];
          } else {
            tok = a.bonus[b];
          }
        }
        tok = clamp_tok(tok, a.V, a.err);
        s1 = (const T*)a.embed + (size_t)tok * a.d;  // read with k - d
      } else if (OP == OP_QKV) {
        s0 = (const T*)a.x0b + (size_t)row * K;
      } else if (OP == OP_O) {
        s0 = (const T*)a.attn + (size_t)row * K;
      } else if (OP == OP_GATEUP) {
        s0 = (const T*)a.yg + (size_t)row * K;
      } else {
        s0 = (const T*)a.act + (size_t)row * K;
      }
    }
    rsrc[0][tid] = s0;
    rsrc[1][tid] = s1;
  }
  const int kswitch = (OP == OP_FC) ? a.d : K;
  const int k0 = split * p.Kc;
  const int k1 = min(K, k0 + p.Kc);
  const int kn = k1 - k0;
  __syncthreads();

  f32x4_t acc[NW][MT];
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[w][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int kq = (lane >> 4) * PER;          // this lane group's k offset in a k-step
  const unsigned char* xl = xs + (lane & 15) * XST + (lane >> 4) * 16;
  // software pipeline: the next U k-steps' weights are in flight while the
  // current U k-steps run on the MFMA units.  X is staged in LDS one chunk of
  // KCH elements at a time (shared by the four waves).
  constexpr int U = (MT * NW > 4) ? 4 : 8;
  constexpr int KCH = (XRB / ES) / (2 * U * KS) * (2 * U * KS);
  static_assert(KCH > 0, "X chunk");
  const int nit = (kn + U * KS - 1) / (U * KS);
  // X staging: a chunk is at most CPR 16-byte pieces per row, SB per thread,
  // loaded SBB at a time (all of a batch before any is stored, so that their
  // latencies overlap; smaller batches where registers are scarce).  Every
  // slot loads and stores unconditionally: when the split needs fewer pieces
  // than there are slots, the extra slots repeat real pieces (same address,
  // same value, same LDS location), and rows past M read row 0 and store
  // zeros, so no load is left in flight on any path.
  constexpr int CPR = KCH / PER;
  constexpr int SB = ROWS * CPR / BLOCK;
  static_assert(SB * BLOCK == ROWS * CPR, "staging covers a chunk exactly");
  constexpr int SBB = (MT * NW >= 3 && SB > 8) ? SB / 2 : SB;
  static_assert(SB % SBB == 0, "staging batches");
  uint4 xv[SBB];
  int xo[SBB];
  auto stage_load = [&](int kc, int b0) __attribute__((always_inline)) {
    const int nch = max(min(KCH, kn - kc), PER) / PER, tot = ROWS * nch;
#pragma unroll
    for (int u = 0; u < SBB; ++u) {
      const int idx = (tid + (b0 + u) * BLOCK) % tot;
      const int r = idx / nch, c = idx - r * nch;
      const int k = min(k0 + kc + c * PER, K - PER);
      const T* s0 = rsrc[0][r];
      const bool ok = s0 != nullptr && kc + c * PER < kn;
      const int rr = s0 != nullptr ? r : 0;  // row 0 of the group always exists
      const T* base = k < kswitch ? rsrc[0][rr] : rsrc[1][rr];
      xv[u] = mask4(ld16g(base + (k < kswitch ? k : k - kswitch)), ok);
      xo[u] = r * XST + c * 16;
    }
  };
  auto stage_store = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < SBB; ++u) *(uint4*)(xs + xo[u]) = xv[u];
  };
  // Weight loads are unconditional from a clamped in-row address (k beyond
  // this split reads valid memory whose product is masked to zero at use), so
  // that the compiler can keep a precise count of loads in flight.  Two
  // register buffers alternate (ping-pong): the loads of iteration it+1 are in
  // flight while iteration it runs, and no register copy at the loop edge
  // forces them to complete early.
  const int klast = K - PER;
  auto wload = [&](uint4 (&buf)[U][NW], int it) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int w = 0; w < NW; ++w)
        buf[u][w] = ld16(wr[w] + min(k0 + it * U * KS + u * KS + kq, klast));
  };
  auto compute = [&](const uint4 (&buf)[U][NW], int it, int kc) __attribute__((always_inline)) {
    const int kb = it * U * KS;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = kb + u * KS;
      const bool kin = k + kq < kn;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint4 xf = mask4(*(const uint4*)(xl + mt * 16 * XST + (k - kc) * ES), kin);
#pragma unroll
        for (int w = 0; w < NW; ++w) acc[w][mt] = mma16(xf, buf[u][w], acc[w][mt], T());
      }
    }
  };
  uint4 wa[U][NW], wb[U][NW];
  // first chunk's X loads go out before the first weight loads; both are in
  // flight together
  stage_load(0, 0);
  wload(wa, 0);
  stage_store();
#pragma unroll
  for (int b0 = SBB; b0 < SB; b0 += SBB) {
    stage_load(0, b0);
    stage_store();
  }
  __syncthreads();
  // Chunks hold an even number of iterations (KCH is a multiple of 2*U*KS),
  // so each chunk starts on buffer wa.  The loads of the iteration after the
  // last may be issued too (clamped, in bounds, unused).
  int it = 0;
  for (int kc = 0; kc < kn; kc += KCH) {
    if (kc > 0) {  // all of this split's X for the chunk; drains the pipeline once per chunk
      __syncthreads();
#pragma unroll
      for (int b0 = 0; b0 < SB; b0 += SBB) {
        stage_load(kc, b0);
        stage_store();
      }
      __syncthreads();
    }
    const int itend = min(nit, (kc + KCH) / (U * KS));
    // The scheduling barriers keep each batch of loads ahead of the MFMAs on
    // the other buffer (the compiler would otherwise sink them and wait early);
    // the loop body is one straight block so that its wait counts stay exact.
    for (; it + 1 < itend; it += 2) {
      wload(wb, it + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(wa, it, kc);
      wload(wa, it + 2);
      __builtin_amdgcn_sched_barrier(0);
      compute(wb, it + 1, kc);
    }
    if (it < itend) {  // odd count: last chunk only
      compute(wa, it, kc);
      ++it;
    }
  }

  // ---- split-K: partials, last block reduces in split order
  const int bid = zg * p.nblk + blk;
  if (p.S > 1) {
    float* part = a.gpart + ((((size_t)bid * p.S + split) * 4 + wave) * (NW * MT) * 64) * 4;
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        *(f32x4_t*)(part + ((size_t)(w * MT + mt) * 64 + lane) * 4) = acc[w][mt];
    if (!arrive_last(a.cnt + bid, p.S)) return;
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[w][mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // splits' loads issued eight at a time, summed in split order
    for (int s0 = 0; s0 < p.S; s0 += 8) {
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          f32x4_t v[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const float* ps =
                a.gpart + ((((size_t)bid * p.S + s0 + u) * 4 + wave) * (NW * MT) * 64) * 4;
            v[u] = s0 + u < p.S ? *(const f32x4_t*)(ps + ((size_t)(w * MT + mt) * 64 + lane) * 4)
                                : f32x4_t{0.f, 0.f, 0.f, 0.f};
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) acc[w][mt] += v[u];
        }
    }
  }
  // the epilogue tile reuses the X tile's LDS
  __syncthreads();
  float* tile = (float*)xs;  // [NW][ROWS][65]
#define TILE(w, r, c) tile[((w) * ROWS + (r)) * 65 + (c)]
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) TILE(w, mt * 16 + (lane >> 4) * 4 + r, cl) = acc[w][mt][r];
  __syncthreads();

  // ---- epilogues
  const int rows_here = min(ROWS, p.M - zg * 64);
  if (OP == OP_FC) {
    for (int idx = tid; idx < rows_here * 64; idx += BLOCK) {
      const int mr = idx >> 6, c = idx & 63, nn = blk * 64 + c, row = zg * 64 + mr;
      if (nn >= p.N) continue;
      const float v = TILE(0, mr, c) + El<T>::ld((const T*)a.fc_b, nn);
      a.x0f[(size_t)row * a.d + nn] = v;
      El<T>::st((T*)a.x0b, (size_t)row * a.d + nn, v);
    }
  } else if (OP == OP_QKV) {
    const int per = a.hd / 64, head = blk / per, jj = blk % per, half = a.hd / 2;
    const int hq = a.H, hk = a.Hkv;
    for (int idx = tid; idx < rows_here * 32; idx += BLOCK) {
      const int mr = idx >> 5, c = idx & 31, row = zg * 64 + mr;
      const int fi = 32 * jj + c;  // frequency index within the half
      float lo = TILE(0, mr, c), hi = TILE(0, mr, c + 32);
      int b, slot, pos;
      if (a.mode == MODE_LEVEL) {
        b = row / a.k;
        slot = row % a.k;
        pos = clamp_prefix(a.prefix_len[b], a) - 1 + a.depth;
      } else {
        b = row / a.m;
        slot = row % a.m;
        pos = clamp_prefix(a.prefix_len[b], a) + slot;
      }
      if (head < hq + hk) {  // q or k: rotate the (fi, fi+half) pair
        const double inv = pow((double)a.theta, -2.0 * (double)fi / (double)a.hd);
        double sd, cd;
        sincos((double)pos * inv, &sd, &cd);
        const float cs = (float)cd, sn = (float)sd;
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
        T* dst;
        if (a.mode == MODE_LEVEL) {
          T* base = (T*)(isk ? a.tk : a.tv);
          dst = base + ((((size_t)b * a.D + a.depth) * a.k + slot) * a.Hkv + kvh) * a.hd;
        } else {
          T* base = (T*)(isk ? a.k_cache : a.v_cache);
          const int P = clamp_prefix(a.prefix_len[b], a);
          dst = base + (((size_t)b * a.max_prefix + P + slot) * a.Hkv + kvh) * a.hd;
        }
        El<T>::st(dst, fi, lo);
        El<T>::st(dst, fi + half, hi);
      }
    }
  } else if (OP == OP_O) {
    for (int idx = tid; idx < rows_here * 64; idx += BLOCK) {
      const int mr = idx >> 6, c = idx & 63, nn = blk * 64 + c, row = zg * 64 + mr;
      if (nn >= p.N) { TILE(0, mr, c) = 0.f; continue; }
      const float y = TILE(0, mr, c) + a.x0f[(size_t)row * a.d + nn];
      TILE(0, mr, c) = y;
      a.yf[(size_t)row * a.d + nn] = y;
      El<T>::st((T*)a.yg, (size_t)row * a.d + nn, y * El<T>::ld((const T*)a.post_norm, nn));
    }
    __syncthreads();
    if (tid < rows_here) {
      float s = 0.f;
      for (int c = 0; c < 64; ++c) s += TILE(0, tid, c) * TILE(0, tid, c);
      a.ssq[(size_t)blk * a.rows + zg * 64 + tid] = s;
    }
    if (arrive_last(a.cnt + GRID_CNT, p.nblk * p.zg)) {
      for (int row = tid; row < p.M; row += BLOCK) {
        float s = 0.f;
        for (int b0 = 0; b0 < p.nblk; b0 += 16) {
          float v[16];
#pragma unroll
          for (int u = 0; u < 16; ++u)
            v[u] = b0 + u < p.nblk ? a.ssq[(size_t)(b0 + u) * a.rows + row] : 0.f;
#pragma unroll
          for (int u = 0; u < 16; ++u) s += v[u];
        }
        a.rstd[row] = 1.0f / sqrtf(s / (float)a.d + a.eps);
      }
    }
  } else if (OP == OP_GATEUP) {
    for (int idx = tid; idx < rows_here * 64; idx += BLOCK) {
      const int mr = idx >> 6, c = idx & 63, nn = blk * 64 + c, row = zg * 64 + mr;
      if (nn >= p.N) continue;
      const float r = a.rstd[row];
      const float g = TILE(0, mr, c) * r, u = TILE(NW - 1, mr, c) * r;
      El<T>::st((T*)a.act, (size_t)row * a.F + nn, g / (1.0f + expf(-g)) * u);
    }
  } else {  // OP_DOWN
    for (int idx = tid; idx < rows_here * 64; idx += BLOCK) {
      const int mr = idx >> 6, c = idx & 63, nn = blk * 64 + c, row = zg * 64 + mr;
      if (nn >= p.N) continue;
      const float h = TILE(0, mr, c) + a.yf[(size_t)row * a.d + nn];
      if (a.mode == MODE_LEVEL) {
        El<T>::st((T*)a.feat, ((size_t)a.depth * a.B * a.k + row) * a.d + nn, h);
      } else {
        El<T>::st((T*)a.ext_h, (size_t)row * a.d + nn, h);
        const int b = row / a.m, i = row % a.m;
        int alen = a.accept_len[b];
        alen = alen < 1 ? 1 : (alen > a.D + 1 ? a.D + 1 : alen);
        if (i == alen - 1) El<T>::st((T*)a.root_feat, (size_t)b * a.d + nn, h);
      }
    }
    if (a.mode == MODE_EXTEND && arrive_last(a.cnt + GRID_CNT, p.nblk * p.zg)) {
      for (int b = tid; b < a.B; b += BLOCK) {
        int alen = a.accept_len[b];
        alen = alen < 1 ? 1 : (alen > a.D + 1 ? a.D + 1 : alen);
        a.prefix_len[b] = clamp_prefix(a.prefix_len[b], a) + alen;
        a.root_token[b] = clamp_tok(a.bonus[b], a.V, a.err);
      }
    }
  }
#undef TILE
}

template <typename T, int OP>
static hipError_t launch_op(const RoundArgs& a, const GemmPlan& p, hipStream_t s) {
  const dim3 grid(p.nblk, p.S, p.zg), block(BLOCK);
  switch (p.mt) {
    case 1: hipLaunchKernelGGL((k_gemm<T, OP, 1>), grid, block, 0, s, a, p); break;
    case 2: hipLaunchKernelGGL((k_gemm<T, OP, 2>), grid, block, 0, s, a, p); break;
    case 3: hipLaunchKernelGGL((k_gemm<T, OP, 3>), grid, block, 0, s, a, p); break;
    default: hipLaunchKernelGGL((k_gemm<T, OP, 4>), grid, block, 0, s, a, p); break;
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

// Weight-streaming core shared by the level GEMMs (k_skinny.hip) and the
// LM head (k_lmhead.hip) at drafting shapes, where at most 16 rows of X meet
// a weight matrix that is read exactly once.
//
// One wave streams NW packed weight tiles (16 output columns each, one
// contiguous kilobyte per k-step and wave load instruction) over its K slice,
// k-steps [s0k, s1k), into 16x16 MFMA accumulators.  BU k-steps form a load
// batch and two batches are in flight (ping-pong register sets).  Loads are
// unconditional from clamped in-bounds addresses (products past the slice are
// masked to zero), the steady-state loop body is one straight block, and the
// last one or two batches are peeled: all so that the compiler's wait counts
// stay exact and no load waits behind a needless drain.
//
// X is either staged once in LDS (XL: its rows, row stride K*ES + 16 so that
// the rows of one read fall in different banks; staged while the first two
// weight batches are in flight) or loaded per k-step from L2.  X loads share the
// memory queue with the weight loads and cost a quarter to a third of the
// streaming rate, so the LDS copy is used wherever it fits and is shared.
#pragma once
#include "eagle_internal.h"

namespace eg {

// wr[w]: this lane's piece of k-step 0 of its packed tile (wtile_base).
// XP: X is stored packed (16 rows x one k-step per kilobyte, xpk_index) and
// x0 is this lane's piece of k-step 0; otherwise X is row-major:
// Row c of X (c = lane % 16) is x0[k] for k < kswitch and x1[k - kswitch]
// beyond (the FC's gathered [feature || embedding] input); callers with one
// source pass x1 = x0 and kswitch = K.  nbu is the number of BU-k-step
// batches of the longest slice in the block, the same for every wave (a wave
// with a shorter slice runs masked batches), since the loop holds barriers.  With XL, X must be M contiguous rows
// of stride K starting at xs (only those rows are staged: LDS rows past M
// keep stale values, which reach only the discarded output rows past M), and
// every thread of the block must call this (it stages X and synchronises).
template <typename T, int NW, int BU, bool XL, bool XP = false>
__device__ __forceinline__ void sk_stream(const T* const (&wr)[NW], const T* x0, const T* x1, int kswitch,
                                          int K, int s0k, int s1k, int nbu, unsigned char* dyn,
                                          f32x4_t (&acc)[NW], const T* xs = nullptr, int M = 16) {
  constexpr int KS = El<T>::KSTEP;
  constexpr int PER = El<T>::PER16;
  constexpr int ES = (int)sizeof(T);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int kend = min(K, s1k * KS);
  const int nb = nbu;  // the same in every wave of the block (the loop's barriers)
  const int klast = K - PER;
  const int XST = K * ES + 16;
  const unsigned char* xrow = dyn + c * XST;
#pragma unroll
  for (int w = 0; w < NW; ++w) acc[w] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nkt = (K + KS - 1) / KS;  // k-step tiles of a packed row block
  // loads past the slice repeat its last k-step (the bytes this lane has just
  // loaded) rather than read the next slice's, which another wave streams:
  // with the non-temporal policy those would be fetched from HBM twice
  const int stmax = min(max(s1k - 1, 0), nkt - 1);
  auto load = [&](uint4 (&wb)[BU][NW], uint4 (&xb)[BU], int b) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < BU; ++u) {
      const int st = min(s0k + b * BU + u, stmax);
      const int kc = min(st * KS + g * PER, klast);
#pragma unroll
      for (int w = 0; w < NW; ++w) wb[u][w] = ld16w(wr[w] + (size_t)st * wtile_elems<T>());
      if (!XL) xb[u] = XP ? ld16(x0 + (size_t)st * wtile_elems<T>()) : ld16(kc < kswitch ? x0 + kc : x1 + (kc - kswitch));
    }
  };
  auto comp = [&](const uint4 (&wb)[BU][NW], const uint4 (&xb)[BU], int b) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < BU; ++u) {
      const int k = (s0k + b * BU + u) * KS + g * PER;
      const uint4 xv = XL ? *(const uint4*)(xrow + min(k, klast) * ES) : xb[u];
      const uint4 xf = mask4(xv, k < kend);
#pragma unroll
      for (int w = 0; w < NW; ++w) acc[w] = mma16(xf, wb[u][w], acc[w], T());
    }
  };

  uint4 wa[BU][NW], xa[BU], wbf[BU][NW], xbf[BU];
  if (XL) {
    // The M real rows, piece by piece over all threads.  A thread's first SPT
    // pieces are loaded first, then both weight batches, then the pieces are
    // stored: the stores wait for X alone and the weights stay in flight
    // across the barrier.  Stores are unconditional (a slot past the end
    // repeats the last piece: same value, same place), so no load is sunk
    // into a branch of its own.
    constexpr int SPT = NW == 2 ? 6 : 9;  // with two weight streams, registers are scarcer
    const int npc = K / PER, tot = M * npc, nt = (int)blockDim.x;
    uint4 v[SPT];
    auto xload = [&](int i0) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < SPT; ++u) {
        const int i = min(i0 + u * nt, tot - 1);
        v[u] = ld16(xs + (size_t)(i / npc) * K + (i % npc) * PER);
      }
    };
    auto xstore = [&](int i0) __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < SPT; ++u) {
        const int i = min(i0 + u * nt, tot - 1);
        *(uint4*)(dyn + (i / npc) * XST + (i % npc) * 16) = v[u];
      }
    };
    xload((int)threadIdx.x);
    __builtin_amdgcn_sched_barrier(0);
    load(wa, xa, 0);
    __builtin_amdgcn_sched_barrier(0);
    load(wbf, xbf, 1);
    __builtin_amdgcn_sched_barrier(0);
    xstore((int)threadIdx.x);
    for (int i0 = (int)threadIdx.x + nt * SPT; i0 < tot; i0 += nt * SPT) {  // rows longer than one pass
      xload(i0);
      xstore(i0);
    }
    __syncthreads();
  } else {
    load(wa, xa, 0);
    __builtin_amdgcn_sched_barrier(0);
    load(wbf, xbf, 1);
    __builtin_amdgcn_sched_barrier(0);
  }
  // Both buffers stay in flight: each batch's MFMAs are followed by the load
  // two batches ahead into the same buffer (loads past the slice repeat its
  // last k-step and are unused); the last one or two batches are peeled.
  int b = 0;
  for (; b + 2 < nb; b += 2) {
    comp(wa, xa, b);
    load(wa, xa, b + 2);
    __builtin_amdgcn_sched_barrier(0);
    comp(wbf, xbf, b + 1);
    load(wbf, xbf, b + 3);
    __builtin_amdgcn_sched_barrier(0);
    // keep the waves of the block in step: the memory system serves older
    // waves first, and waves that finish early leave the compute unit with
    // fewer loads in flight for the rest of the stream
    __builtin_amdgcn_s_barrier();
  }
  if (b < nb) comp(wa, xa, b);
  if (b + 1 < nb) comp(wbf, xbf, b + 1);
}

// Bytes of X tile staged by sk_stream<XL = true>.
__host__ __device__ inline size_t sk_xtile_bytes(int K, int es) { return (size_t)16 * ((size_t)K * es + 16); }

// The q/k/v projection's input x0 carried as two bf16 parts, x0 = hi + lo
// (hi = bf16(x0), lo = bf16(x0 - hi): about 16 mantissa bits), the A operand
// taken twice per weight fragment.  At the tree's deeper levels the scores
// q.k of a row's own and ancestor keys reach the thousands (the residual
// stream grows level by level at these weights), and one bf16 rounding of x0
// there moves the output by more than bf16 activations elsewhere do; the
// second MFMA per fragment costs nothing at a weight-streaming shape.
//
// XL: the M rows of both parts are staged in LDS in two K phases (the hi rows
// at tile rows 0..15, the lo rows at 16..31, each phase's k-steps H0 = the
// larger half, row stride H0*KS*ES + 16 bytes): phase p covers k-steps
// [p*H0, p*H0 + Hp), split over the KSW waves of a column tile like the whole
// range is in sk_stream.  At the phase boundary the block restages the tile.
// Otherwise each lane loads its
// two 16-byte X pieces per k-step from L2.  K must be a whole number of
// k-steps.  Every thread of the block calls this.
__host__ __device__ inline int sk_hl_half(int K, int ks) { return ((K / ks) + 1) / 2; }
__host__ __device__ inline size_t sk_hl_tile_bytes(int K, int es) {
  const int KS = es == 2 ? 32 : 16;
  return (size_t)32 * ((size_t)sk_hl_half(K, KS) * KS * es + 16);
}

// xh, xl: row 0 of the two parts ([M][K] row-major each).
template <typename T, int BU, bool XL>
__device__ __forceinline__ void sk_stream_hl(const T* wr, const T* xh, const T* xl, int K, int ks, int KSW,
                                             unsigned char* dyn, f32x4_t& acc, int M) {
  constexpr int KS = El<T>::KSTEP;
  constexpr int PER = El<T>::PER16;
  constexpr int ES = (int)sizeof(T);
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, g = lane >> 4;
  const size_t xro = (size_t)(c < M ? c : 0) * K;  // this lane's row (rows past M read row 0, discarded)
  const int nks = K / KS;
  const int H0 = sk_hl_half(K, KS), H1 = nks - H0;
  const int XST = H0 * KS * ES + 16;
  // this wave's k-steps in each phase
  const int a0 = ks * H0 / KSW, e0 = (ks + 1) * H0 / KSW;
  const int a1 = H0 + ks * H1 / KSW, e1 = H0 + (ks + 1) * H1 / KSW;
  // batches per phase, the same in every wave; even and at least two, so that
  // the phase boundary falls between two loop iterations
  const int nbh = max(2, (((H0 + KSW - 1) / KSW + BU - 1) / BU + 1) & ~1);
  const int nb = 2 * nbh;
  acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // k-step of batch b, element u, and whether it is in the wave's range
  auto kstep = [&](int b, int u, bool& in) __attribute__((always_inline)) {
    const int ph = b >= nbh, s = (ph ? a1 : a0) + (b - ph * nbh) * BU + u;
    in = s < (ph ? e1 : e0);
    return s;
  };
  auto load = [&](uint4 (&wb)[BU], uint4 (&xb)[BU][2], int b) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < BU; ++u) {
      bool in;
      const int st = min(kstep(b, u, in), nks - 1);
      wb[u] = ld16w(wr + (size_t)st * wtile_elems<T>());
      if (!XL) {
        const size_t o = xro + (size_t)st * KS + g * PER;
        xb[u][0] = ld16(xh + o);
        xb[u][1] = ld16(xl + o);
      }
    }
  };
  auto comp = [&](const uint4 (&wb)[BU], const uint4 (&xb)[BU][2], int b) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < BU; ++u) {
      bool in;
      const int s = kstep(b, u, in);
      uint4 vh, vl;
      if (XL) {
        const int ph = b >= nbh;
        const int sl = min(max(s - ph * H0, 0), H0 - 1);  // a slot outside the phase: clamped, masked below
        const int off = sl * KS * ES + g * 16;
        vh = *(const uint4*)(dyn + c * XST + off);
        vl = *(const uint4*)(dyn + (16 + c) * XST + off);
      } else {
        vh = xb[u][0];
        vl = xb[u][1];
      }
      acc = mma16(mask4(vh, in), wb[u], acc, T());
      acc = mma16(mask4(vl, in), wb[u], acc, T());
    }
  };
  // phase p of both parts into LDS: M rows x Hp k-steps, 16-byte pieces, in
  // passes of SPT pieces per thread (one pass at the 7B shape).  Keeping the
  // next phase's pieces in registers across the phase was measured slower than
  // restaging at the boundary, so the restage is synchronous.
  constexpr int SPT = 7;
  const int nt = (int)blockDim.x;
  auto stage = [&](int ph) __attribute__((always_inline)) {
    const int npc = (ph ? H1 : H0) * KS / PER, tot = 2 * M * npc;
    for (int i0 = (int)threadIdx.x; i0 < tot; i0 += nt * SPT) {
      uint4 v[SPT];
      int dst[SPT];
#pragma unroll
      for (int u = 0; u < SPT; ++u) {  // a slot past the end repeats the last piece (same value, same place)
        const int i = min(i0 + u * nt, tot - 1), q = i / npc, pc = i - q * npc;
        const int part = q >= M, r = q - part * M;
        v[u] = ld16((part ? xl : xh) + (size_t)r * K + (size_t)ph * H0 * KS + pc * PER);
        dst[u] = (part * 16 + r) * XST + pc * 16;
      }
#pragma unroll
      for (int u = 0; u < SPT; ++u) *(uint4*)(dyn + dst[u]) = v[u];
    }
  };
  uint4 wa[BU], wbf[BU], xa[BU][2], xbf[BU][2];
  load(wa, xa, 0);
  __builtin_amdgcn_sched_barrier(0);
  load(wbf, xbf, 1);
  __builtin_amdgcn_sched_barrier(0);
  if (XL) {
    stage(0);
    __syncthreads();
  }
  // phase 0, then the restage (every wave done with phase 0's tile), then phase 1
  int b = 0;
  for (; b + 2 <= nbh; b += 2) {
    comp(wa, xa, b);
    load(wa, xa, b + 2);
    __builtin_amdgcn_sched_barrier(0);
    comp(wbf, xbf, b + 1);
    load(wbf, xbf, b + 3);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
  }
  if (XL) {
    __syncthreads();
    stage(1);
    __syncthreads();
  }
  for (; b + 2 < nb; b += 2) {
    comp(wa, xa, b);
    load(wa, xa, b + 2);
    __builtin_amdgcn_sched_barrier(0);
    comp(wbf, xbf, b + 1);
    load(wbf, xbf, b + 3);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
  }
  if (b < nb) comp(wa, xa, b);
  if (b + 1 < nb) comp(wbf, xbf, b + 1);
}

}  // namespace eg

// The main loop of the 64-row weight-streaming GEMMs (bf16): a workgroup of
// eight waves computes 64 rows x 128*NQ columns of X[M][K] W[N][K]^T on
// v_mfma_f32_16x16x32_bf16, each wave 64 rows x 16*NQ columns.
//
// At 17..64 rows a layer's weights are read once and reused across only four
// 16-row MFMA tiles, so the loop is bound by the weight stream.  Its design
// keeps that stream going and the features off the critical path:
//  * operands move from memory straight into LDS (global_load_lds_dwordx4:
//    lane l's 16 bytes land at l*16, one kilobyte MFMA fragment per wave
//    instruction), the weights non-temporal.  A k-step of 32 is 4 + 8*NQ fragments: the rows' four X
//    fragments and the workgroup's 8*NQ weight tiles;
//  * four stage buffers of 36 KB, a step's loads issued three steps ahead.
//    Each wave loads its own NQ weight fragments, and waves 0..3 the four X
//    fragments; waves 4..7 load their last weight fragment a second time
//    (same bytes, same place: one contiguous kilobyte, where an X fragment is
//    sixteen rows' pieces), so every wave issues NQ+1 loads per step and
//    waits for a fixed count;
//  * with one weight tile per wave (NQ = 1) a stage holds two k-steps (8 X
//    and 16 weight fragments, 24 KB: three loads per wave, no repeats), so a
//    barrier covers two k-steps and the loads run six k-steps ahead;
//  * each stage t: wait for its loads and the previous stage's LDS reads,
//    one workgroup barrier, issue the loads of stage t+3 into the buffer
//    stage t-1 used, read the X fragments and the wave's weight fragments,
//    the MFMAs.
//  * The loop body is one branch-free step per buffer (the compiler then
//    keeps the loads in flight across the LDS reads of other buffers), so the
//    k-step count is a multiple of four (of eight with NQ = 1).
#pragma once

#include "eagle_internal.h"

namespace eg {

constexpr int PS_W = 8;                  // waves per workgroup
// cache policy of the weight loads: non-temporal (each weight byte is read
// once per pass; without the hint the stream evicts the prefix K/V and the
// activations that the next launches re-read)
constexpr int PS_WNT = 2;
constexpr int PS_THREADS = PS_W * WAVE;
constexpr int PS_MAXQ = 4;               // weight tiles per wave at most
constexpr int PS_STAGE = (4 + 8 * PS_MAXQ) * 64;  // uint4 per stage buffer (36 KB)

static __shared__ __attribute__((aligned(1024))) uint4 ps_s0[PS_STAGE];
static __shared__ __attribute__((aligned(1024))) uint4 ps_s1[PS_STAGE];
static __shared__ __attribute__((aligned(1024))) uint4 ps_s2[PS_STAGE];
static __shared__ __attribute__((aligned(1024))) uint4 ps_s3[PS_STAGE];
constexpr int PS_STAGE1 = 24 * 64;  // uint4 per stage buffer with NQ = 1 (two k-steps, 24 KB)
static __shared__ __attribute__((aligned(1024))) uint4 ps_t0[PS_STAGE1];
static __shared__ __attribute__((aligned(1024))) uint4 ps_t1[PS_STAGE1];
static __shared__ __attribute__((aligned(1024))) uint4 ps_t2[PS_STAGE1];
static __shared__ __attribute__((aligned(1024))) uint4 ps_t3[PS_STAGE1];

// k-steps per unrolled loop body (four stage buffers)
template <int NQ> constexpr int ps_unroll() { return NQ == 1 ? 8 : 4; }

// s_waitcnt immediate (gfx9 layout: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8) of vmcnt(n) with lgkmcnt(0)
__host__ __device__ constexpr int ps_wait_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// nsteps k-steps (a multiple of ps_unroll<NQ>()) into acc: lane (g, c) of
// acc[mt][q] holds rows 16*mt + 4g..4g+3 and column 16*(NQ*wave + q) + c of
// the tile.  srcx(s): this lane's 16 bytes of X fragment (wave % 4) at k-step s;
// srcw(q, s): this lane's 16 bytes of the wave's weight tile q at step s.
// Every wave of the workgroup must call it; it ends with the loads drained
// and a workgroup barrier, the stage buffers free for the caller.
template <int NQ, typename SrcX, typename SrcW>
__device__ __forceinline__ void ps_main(int nsteps, const SrcX& srcx, const SrcW& srcw, f32x4_t (&acc)[4][NQ]) {
  static_assert(NQ >= 1 && NQ <= PS_MAXQ, "weight tiles per wave");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  auto lds = [](uint4* p) __attribute__((always_inline)) { return (__attribute__((address_space(3))) void*)p; };
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int q = 0; q < NQ; ++q) acc[mt][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // stage t: its loads and the previous stage's reads complete, barrier
  // (every wave's loads of stage t have landed and every wave is done with
  // the buffer of stage t-1), stage t+3's loads into that buffer, reads and
  // MFMAs; two later stages stay in flight
#define PS_STEP(BUF, NEXT, t)                 \
  __builtin_amdgcn_sched_barrier(0);          \
  __builtin_amdgcn_s_waitcnt(WAIT);           \
  __builtin_amdgcn_s_barrier();               \
  __builtin_amdgcn_sched_barrier(0);          \
  dma(NEXT, (t) + 3);                         \
  __builtin_amdgcn_sched_barrier(0);          \
  step(BUF);
  if constexpr (NQ == 1) {
    // a stage is k-steps 2t, 2t+1: X fragment (wave % 4) of k-step 2t + wave/4
    // at slot `wave`, the wave's weight tile of k-step 2t + kk at slot
    // 8 + 8 kk + wave
    constexpr int WAIT = ps_wait_vm_lgkm0(2 * 3);
    const int nst = nsteps / 2;
    auto dma = [&](uint4* buf, int t) __attribute__((always_inline)) {
      t = min(t, nst - 1);  // past the last stage: repeats it into a buffer not read again
      __builtin_amdgcn_global_load_lds(srcx(2 * t + (wave >> 2)), lds(buf + wave * WAVE), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(srcw(0, 2 * t), lds(buf + (8 + wave) * WAVE), 16, 0, PS_WNT);
      __builtin_amdgcn_global_load_lds(srcw(0, 2 * t + 1), lds(buf + (16 + wave) * WAVE), 16, 0, PS_WNT);
    };
    auto step = [&](const uint4* buf) __attribute__((always_inline)) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        uint4 xa[4];
        const uint4 wb = buf[(8 + 8 * kk + wave) * WAVE + lane];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) xa[mt] = buf[(4 * kk + mt) * WAVE + lane];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt][0] = mma16(xa[mt], wb, acc[mt][0], bf16_t());
      }
    };
    dma(ps_t0, 0);
    dma(ps_t1, 1);
    dma(ps_t2, 2);
    for (int t = 0; t < nst; t += 4) {
      PS_STEP(ps_t0, ps_t3, t)
      PS_STEP(ps_t1, ps_t0, t + 1)
      PS_STEP(ps_t2, ps_t1, t + 2)
      PS_STEP(ps_t3, ps_t2, t + 3)
    }
  } else {
    constexpr int WAIT = ps_wait_vm_lgkm0(2 * (NQ + 1));
    auto dma = [&](uint4* buf, int s) __attribute__((always_inline)) {
      s = min(s, nsteps - 1);  // past the last step: repeats it into a buffer not read again
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        __builtin_amdgcn_global_load_lds(srcw(q, s), lds(buf + (4 + NQ * wave + q) * WAVE), 16, 0, PS_WNT);
      // waves 0..3: X fragment `wave`; waves 4..7 repeat their last weight
      // fragment (a wave-uniform select, no branch)
      const bool xw = wave < 4;
      __builtin_amdgcn_global_load_lds(xw ? srcx(s) : srcw(NQ - 1, s),
                                       lds(buf + (xw ? wave : 4 + NQ * wave + NQ - 1) * WAVE), 16, 0, 0);
    };
    auto step = [&](const uint4* buf) __attribute__((always_inline)) {
      uint4 xa[4], wb[NQ];
#pragma unroll
      for (int q = 0; q < NQ; ++q) wb[q] = buf[(4 + NQ * wave + q) * WAVE + lane];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) xa[mt] = buf[mt * WAVE + lane];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int q = 0; q < NQ; ++q) acc[mt][q] = mma16(xa[mt], wb[q], acc[mt][q], bf16_t());
    };
    dma(ps_s0, 0);
    dma(ps_s1, 1);
    dma(ps_s2, 2);
    for (int t = 0; t < nsteps; t += 4) {
      PS_STEP(ps_s0, ps_s3, t)
      PS_STEP(ps_s1, ps_s0, t + 1)
      PS_STEP(ps_s2, ps_s1, t + 2)
      PS_STEP(ps_s3, ps_s2, t + 3)
    }
  }
#undef PS_STEP
  __builtin_amdgcn_s_waitcnt(0);  // the repeated loads past the last step, the last reads
  __syncthreads();
}

// A 64-row x 64-column float tile for the epilogues, slab j < 2 * NQ: with
// NQ = 1 stage buffer j, else half (j & 1) of stage buffer j >> 1
template <int NQ>
__device__ __forceinline__ float* ps_slab(int j) {
  if constexpr (NQ == 1) return (float*)(j == 0 ? ps_t0 : ps_t1);
  uint4* base = (j >> 1) == 0 ? ps_s0 : (j >> 1) == 1 ? ps_s1 : (j >> 1) == 2 ? ps_s2 : ps_s3;
  return (float*)base + (j & 1) * 64 * 64;
}

}  // namespace eg

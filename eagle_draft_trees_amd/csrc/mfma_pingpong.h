// The main loop of the tiled bf16 GEMMs (the batched LM head and the layer
// GEMMs of many rows): a workgroup of eight waves computes a 256 x 256 tile of
// X[M][K] W[N][K]^T on v_mfma_f32_16x16x32_bf16, each wave a 128 x 64 block.
//
//  * Operands move from memory straight into LDS (global_load_lds_dwordx4:
//    lane l's 16 bytes land at l*16).  A k-step of 32 is 32 one-kilobyte MFMA
//    fragments: 16 of X (16 rows each, fragment order: lane l holds row l%16,
//    k 8*(l/16)..+7) and 16 of W.  The caller names, per wave, the global
//    address of each lane's 16 bytes of its four fragments of a step, so any
//    source layout whose fragments are gatherable by lane works.
//  * Four stage buffers of one k-step (32 KB each); a step's loads are issued
//    three steps ahead, four fragments by each wave (with MIX two of X and two
//    of W, the weight loads non-temporal).  Loads past the last step
//    repeat it into buffers that are not read again, so every wave waits for a
//    fixed count (vmcnt(8): the two later steps stay in flight).
//  * The waves run as two groups of four (one wave of each group per SIMD),
//    offset by half a step: while one group reads its twelve fragments from
//    LDS and issues its next loads, the other runs its 32 MFMAs on operands
//    already in registers, so each SIMD's matrix core always has a wave
//    feeding it.  Each half step ends in a workgroup barrier.
//  * The loop body is four branch-free steps: the compiler tells the four
//    buffers apart (separate __shared__ objects) and then adds no waits of its
//    own between a buffer's loads and another buffer's reads, but it loses
//    that at control-flow merges.  So the step count is a multiple of four.
#pragma once

#include "eagle_internal.h"

namespace eg {

constexpr int PP_W = 8;                 // waves per workgroup
constexpr int PP_THREADS = PP_W * WAVE;
constexpr int PP_TM = 256, PP_TN = 256;  // tile rows, columns
constexpr int PP_DMA = 4;               // fragments each wave loads per k-step

static __shared__ __attribute__((aligned(1024))) uint4 pp_s0[2048];
static __shared__ __attribute__((aligned(1024))) uint4 pp_s1[2048];
static __shared__ __attribute__((aligned(1024))) uint4 pp_s2[2048];
static __shared__ __attribute__((aligned(1024))) uint4 pp_s3[2048];

// s_waitcnt immediates (gfx9 layout: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8): vmcnt(8) alone, and vmcnt(8) with lgkmcnt(0)
constexpr int PP_WAIT_VM8 = 8 | (7 << 4) | (15 << 8);
constexpr int PP_WAIT_VM8_LGKM0 = 8 | (7 << 4);

// nsteps k-steps (a multiple of 4, at least 4) into acc (wave (wm, wn) =
// (wave & 1, wave >> 1): rows 128*wm + 16*i, columns 64*wn + 16*q of the
// tile; lane (g, c) of acc[i][q] holds rows 4g..4g+3 and column c).
// src(u, s) is the address of this lane's 16 bytes of this wave's fragment u
// at step s < nsteps.  MIX: u = 0, 1 the step's X fragment 2*wave + u (of
// 0..15), u = 2, 3 its W fragment 2*wave + u - 2 (of 0..15; slot 16 + that in
// the stage buffer); otherwise fragment 4*wave + u of the step (0..15 X,
// 16..31 W).
// Every wave of the workgroup must call it; it ends with the loads drained
// and a workgroup barrier, the stage buffers free for the caller.
template <bool MIX = false, typename Src>
__device__ __forceinline__ void pp_main(int nsteps, const Src& src, f32x4_t (&acc)[8][4]) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool first = wave < 4;              // group that runs half a step ahead
  const int wm = wave & 1, wn = wave >> 1;
  // MIX: this wave's fragments u = 0, 1 are X fragments 2*wave + u and
  // u = 2, 3 W fragments 16 + 2*wave + u - 2, the weight loads non-temporal
  // (read once per pass); else fragments 4*wave + u (waves 0..3 X, 4..7 W)
  auto dma = [&](uint4* buf, int s) __attribute__((always_inline)) {
    s = min(s, nsteps - 1);
    auto at = [&](int f) __attribute__((always_inline)) {
      return (__attribute__((address_space(3))) void*)(buf + f * WAVE);
    };
    if constexpr (MIX) {
      __builtin_amdgcn_global_load_lds(src(0, s), at(2 * wave), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(src(1, s), at(2 * wave + 1), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(src(2, s), at(16 + 2 * wave), 16, 0, 2);
      __builtin_amdgcn_global_load_lds(src(3, s), at(17 + 2 * wave), 16, 0, 2);
    } else {
#pragma unroll
      for (int u = 0; u < PP_DMA; ++u) __builtin_amdgcn_global_load_lds(src(u, s), at(PP_DMA * wave + u), 16, 0, 0);
    }
  };
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[i][q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint4 xa[8], wb[4];
  auto rd = [&](const uint4* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) wb[q] = buf[(16 + 4 * wn + q) * WAVE + lane];
#pragma unroll
    for (int i = 0; i < 8; ++i) xa[i] = buf[(8 * wm + i) * WAVE + lane];
  };
  auto comp = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[i][q] = mma16(xa[i], wb[q], acc[i][q], bf16_t());
    __builtin_amdgcn_s_setprio(0);
  };
  // Step t: read buffer t%4 and issue step t+3's loads into buffer (t+3)%4
  // (last read at step t-1, by the second group, before the barrier that
  // precedes this half step), wait for step t+1's loads and the reads,
  // barrier, MFMAs, barrier.  The first group reads step t while the second
  // computes step t-1 and vice versa.
#define PP_STEP(BUF, NEXT, t)                       \
  __builtin_amdgcn_sched_barrier(0);                \
  rd(BUF);                                          \
  __builtin_amdgcn_sched_barrier(0);                \
  dma(NEXT, (t) + 3);                               \
  __builtin_amdgcn_s_waitcnt(PP_WAIT_VM8_LGKM0);    \
  __builtin_amdgcn_sched_barrier(0);                \
  __builtin_amdgcn_s_barrier();                     \
  __builtin_amdgcn_sched_barrier(0);                \
  comp();                                           \
  __builtin_amdgcn_sched_barrier(0);                \
  __builtin_amdgcn_s_waitcnt(PP_WAIT_VM8);          \
  __builtin_amdgcn_s_barrier();

  dma(pp_s0, 0);
  dma(pp_s1, 1);
  dma(pp_s2, 2);
  __builtin_amdgcn_s_waitcnt(PP_WAIT_VM8);
  __builtin_amdgcn_s_barrier();
  if (!first) __builtin_amdgcn_s_barrier();  // the second group starts half a step later
  for (int t = 0; t < nsteps; t += 4) {
    PP_STEP(pp_s0, pp_s3, t)
    PP_STEP(pp_s1, pp_s0, t + 1)
    PP_STEP(pp_s2, pp_s1, t + 2)
    PP_STEP(pp_s3, pp_s2, t + 3)
  }
#undef PP_STEP
  if (first) __builtin_amdgcn_s_barrier();   // (the same barrier count in both groups)
  __builtin_amdgcn_s_waitcnt(0);             // the repeated loads past the last step
  __syncthreads();
}

// Half (h) of stage buffer b as a 16 KB float scratch for the epilogues
__device__ __forceinline__ float* pp_scratch(int b, int h) {
  uint4* base = b == 0 ? pp_s0 : b == 1 ? pp_s1 : b == 2 ? pp_s2 : pp_s3;
  return (float*)base + h * 64 * 64;
}

}  // namespace eg

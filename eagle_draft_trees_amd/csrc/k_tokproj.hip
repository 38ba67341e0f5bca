// Token-projection table (one-time set-up, next to the weight packing).
//
// The draft head's FC takes the row [f || e(t)] ([P1] "EAGLE 推测解码为什么比
// Medusa 快？" §4.1 input equation; [P2] Core Idea), so its output is
//   W_fc [f || e(t)] + b = W_fc[:, :d] f + W_fc[:, d:2d] e(t) + b,
// and the second term depends on the token alone.  It is tabulated once per
// vocabulary entry,
//   tp[v][n] = sum_k embed[v][k] * fc_w[n][d + k]      (fp32 sums, [V][d]),
// which at the 7B shape is 0.5 GB of HBM: the drafting calls then read one
// 16 KB table row per FC row instead of streaming the 33.5 MB token half of
// fc_w in every layer pass.
//
// k_tokproj: one workgroup per 64 x 64 output tile, each wave a 32 x 32 part
// as 2 x 2 MFMA tiles.  The operands are read straight from the row-major
// sources (each lane 16 bytes of a row per k-step; rows of a tile are reused
// from L2 by the neighbouring workgroups): a set-up kernel, measured in
// milliseconds, not on the drafting path.
#include <algorithm>

#include "eagle_internal.h"

namespace eg {

template <typename T>
__global__ void __launch_bounds__(256) k_tokproj(const T* embed, const T* fc_w, float* tp, int V, int d) {
  constexpr int KS = El<T>::KSTEP;
  constexpr int PER = El<T>::PER16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int n0 = blockIdx.x * 64 + (wave & 1) * 32;  // d is a multiple of 64
  const int v0 = blockIdx.y * 64 + (wave >> 1) * 32;
  const T* ar[2];
  const T* br[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int v = min(v0 + 16 * i + c, V - 1);  // rows past V repeat the last; not stored
    ar[i] = embed + (size_t)v * d + g * PER;
    br[i] = fc_w + (size_t)(n0 + 16 * i + c) * (2 * d) + d + g * PER;
  }
  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < d; k += KS) {  // d is a multiple of KS
    uint4 a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      a[i] = ld16(ar[i] + k);
      b[i] = ld16(br[i] + k);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = mma16(a[i], b[j], acc[i][j], T());
  }
  // lane (c, g) holds rows 4g..4g+3 (token) of column c (output n) of each tile
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int v = v0 + 16 * i + 4 * g + r;
      if (v >= V) continue;
#pragma unroll
      for (int j = 0; j < 2; ++j) tp[(size_t)v * d + n0 + 16 * j + c] = acc[i][j][r];
    }
}

hipError_t launch_tokproj(const void* embed, const void* fc_w, float* tp, int V, int d, int es, hipStream_t s) {
  const dim3 grid(d / 64, (V + 63) / 64), block(256);
  if (es == 2)
    hipLaunchKernelGGL(k_tokproj<bf16_t>, grid, block, 0, s, (const bf16_t*)embed, (const bf16_t*)fc_w, tp, V, d);
  else
    hipLaunchKernelGGL(k_tokproj<float>, grid, block, 0, s, (const float*)embed, (const float*)fc_w, tp, V, d);
  return hipGetLastError();
}

}  // namespace eg

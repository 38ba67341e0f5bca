// Weight packing (one-time set-up): a row-major matrix W [N][K] into tiles of
// 16 output rows x KSTEP inputs, each tile one kilobyte in the order a wave's
// 64 lanes load it, so that every weight load of the drafting kernels is one
// contiguous kilobyte.  q/k/v matrices group their rows by RoPE pairs (tile j
// of a head: rows 8j..8j+7 and hd/2+8j..hd/2+8j+7) so that the rotation in
// the QKV epilogues pairs columns within a lane's tile.  Rows and K past the
// matrix are zero.  The source rows are `ld` elements apart (ld >= K: the
// FC's feature half is the first d columns of the [d][2d] fc_w).
#include <algorithm>

#include "eagle_internal.h"

namespace eg {

template <int ES>
__global__ void __launch_bounds__(256) k_pack(const unsigned char* src, unsigned char* dst, int N, int K,
                                              int ld, int pair_hd, long total) {
  constexpr int KS = ES == 2 ? 32 : 16, PER = 16 / ES;
  const int nks = (K + KS - 1) / KS;
  for (long p = (long)blockIdx.x * blockDim.x + threadIdx.x; p < total; p += (long)gridDim.x * blockDim.x) {
    const long tile = p >> 6;
    const int lane = (int)(p & 63), c = lane & 15, g = lane >> 4;
    const int t = (int)(tile / nks), s = (int)(tile - (long)t * nks);
    int r;
    if (pair_hd > 0) {
      const int per = pair_hd / 16, head = t / per, j = t - head * per;
      r = head * pair_hd + (c < 8 ? 8 * j + c : pair_hd / 2 + 8 * j + (c - 8));
    } else {
      r = 16 * t + c;
    }
    const int k = s * KS + g * PER;  // K is a multiple of 8: a piece is wholly in or out
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r < N && k < K) v = *(const uint4*)(src + ((size_t)r * ld + k) * ES);
    *(uint4*)(dst + (size_t)p * 16) = v;
  }
}

hipError_t launch_pack(const void* src, void* dst, int N, int K, int ld, int es, int pair_hd, hipStream_t s) {
  const int ks = es == 2 ? 32 : 16;
  const long total = (long)((N + 15) / 16) * ((K + ks - 1) / ks) * 64;
  const int blocks = (int)std::min<long>((total + 255) / 256, 8192);
  if (es == 2)
    hipLaunchKernelGGL(k_pack<2>, dim3(blocks), dim3(256), 0, s, (const unsigned char*)src, (unsigned char*)dst, N, K,
                       ld, pair_hd, total);
  else
    hipLaunchKernelGGL(k_pack<4>, dim3(blocks), dim3(256), 0, s, (const unsigned char*)src, (unsigned char*)dst, N, K,
                       ld, pair_hd, total);
  return hipGetLastError();
}

}  // namespace eg

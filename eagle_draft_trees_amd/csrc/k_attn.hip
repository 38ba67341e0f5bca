// Tree-masked attention of the draft decoder layer.
//
// Levels: a frontier row at depth L sits at position P-1+L and sees every
// prefix row plus the in-tree K/V of its ancestors and itself, never a sibling
// or cousin ([P1] "EAGLE 推测解码为什么比 Medusa 快？（含 EAGLE-2 动态草稿树）"
// §12 item 5: the mask looks only at ancestors; [P4] "投机解码：从eagle1到dflash"
// EAGLE-2 diagram: tree causal mask).  Extend: row i sees the prefix and
// extend rows 0..i, which the QKV epilogue has already appended to the cache
// ([P3] zdszero.github.io spec_medusa_eagle, "在 SGLang 里").
//
// All rows of a sequence share its prefix, so one workgroup takes one
// (sequence, KV head, query tile) and one slice of the prefix: the K/V tiles of
// that slice are staged in LDS once and used by every query row and every
// query head of the GQA group.  Each slice writes (max, sum, unnormalised
// output) partials; a separate slice handles the per-row in-tree keys; the
// last workgroup to finish a (sequence, KV head, query tile) merges the slices
// in slice order (deterministic).  Scores 1/sqrt(hd) * q.k in fp32.
#include "eagle_internal.h"

namespace eg {

constexpr int AT_QT = 32;  // queries per workgroup
constexpr int AT_KT = 32;  // keys per LDS tile
constexpr int AT_MAXSPLIT = 128;  // merge weights and maxima reuse the K/V tiles' LDS

template <typename T, int HDIM>
__global__ void __launch_bounds__(BLOCK) k_attn(RoundArgs a, AttnPlan p) {
  __shared__ float sQ[AT_QT][129];
  __shared__ float sK[AT_KT][129];
  __shared__ float sV[AT_KT][128];
  __shared__ float sS[AT_QT][AT_KT + 1];
  __shared__ float sM[AT_QT], sL[AT_QT], sScale[AT_QT];
  __shared__ int sLim[AT_QT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wg = blockIdx.x, split = blockIdx.y;
  const int qt = wg % p.nqt, bk = wg / p.nqt, kvh = bk % a.Hkv, b = bk / a.Hkv;
  constexpr int hd = HDIM;
  const int g = p.g;
  const int q0 = qt * AT_QT;
  const int nq = min(AT_QT, p.nq - q0);
  const int P = clamp_prefix(a.prefix_len[b], a);
  const float scale = rsqrtf((float)hd);
  const int HD = a.H * hd;

  // queries: qi -> (row within sequence, head)
  for (int idx = tid; idx < nq * hd; idx += BLOCK) {
    const int qi = idx / hd, dd = idx % hd, gq = q0 + qi;
    const int row = b * p.RS + gq / g, head = kvh * g + gq % g;
    sQ[qi][dd] = a.q[(size_t)row * HD + head * hd + dd] * scale;
  }
  if (tid < AT_QT) {
    const int gq = q0 + tid;
    sLim[tid] = (a.mode == MODE_LEVEL) ? P : P + gq / g + 1;
    sM[tid] = -INFINITY;
    sL[tid] = 0.f;
  }
  __syncthreads();

  const size_t prec = (size_t)hd + 2;
  float* part = a.apart + ((size_t)wg * p.nsplit + split) * AT_QT * prec;
  constexpr int qg_pv = BLOCK / hd;  // query groups in the P.V step
  const int dpv = tid % hd, qpv = tid / hd;
  float acc[AT_QT / 2];
#pragma unroll
  for (int i = 0; i < AT_QT / 2; ++i) acc[i] = 0.f;

  if (split < p.nps) {
    int maxlim = 0;
    for (int qi = 0; qi < nq; ++qi) maxlim = max(maxlim, sLim[qi]);
    const int klo = split * p.KCH;
    const int khi = min(maxlim, klo + p.KCH);
    const T* Kb = (const T*)a.k_cache + ((size_t)b * a.max_prefix * a.Hkv + kvh) * hd;
    const T* Vb = (const T*)a.v_cache + ((size_t)b * a.max_prefix * a.Hkv + kvh) * hd;
    const size_t rstride = (size_t)a.Hkv * hd;
    for (int kt0 = klo; kt0 < khi; kt0 += AT_KT) {
      const int nk = min(AT_KT, khi - kt0);
      {
        // 16-byte loads: PER elements of one key row per thread and chunk
        constexpr int PER = El<T>::PER16;
        const int cpr = hd / PER;  // chunks per key row
        for (int idx = tid; idx < AT_KT * cpr; idx += BLOCK) {
          const int kr = idx / cpr, d0 = (idx % cpr) * PER;
          uint4 kv = make_uint4(0, 0, 0, 0), vv = kv;
          if (kr < nk) {
            kv = ld16(Kb + (size_t)(kt0 + kr) * rstride + d0);
            vv = ld16(Vb + (size_t)(kt0 + kr) * rstride + d0);
          }
          const T* ke = (const T*)&kv;
          const T* ve = (const T*)&vv;
#pragma unroll
          for (int e = 0; e < PER; ++e) {
            sK[kr][d0 + e] = El<T>::ld(ke, e);
            sV[kr][d0 + e] = El<T>::ld(ve, e);
          }
        }
      }
      __syncthreads();
      {
        const int kr = tid % AT_KT;
        for (int qi = tid / AT_KT; qi < nq; qi += BLOCK / AT_KT) {
          float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
          for (int dd = 0; dd < hd; dd += 4) {
            s0 += sQ[qi][dd] * sK[kr][dd];
            s1 += sQ[qi][dd + 1] * sK[kr][dd + 1];
            s2 += sQ[qi][dd + 2] * sK[kr][dd + 2];
            s3 += sQ[qi][dd + 3] * sK[kr][dd + 3];
          }
          const float s = (s0 + s1) + (s2 + s3);
          sS[qi][kr] = (kr < nk && kt0 + kr < sLim[qi]) ? s : -INFINITY;
        }
      }
      __syncthreads();
      {
        const int half = lane >> 5, kr = lane & 31;
        for (int qi = wave * 2 + half; qi < nq; qi += 8) {
          const float x = sS[qi][kr];
          float t = x;
#pragma unroll
          for (int o = 16; o > 0; o >>= 1) t = fmaxf(t, __shfl_xor(t, o));
          const float mold = sM[qi];
          const float mnew = fmaxf(mold, t);
          const float pr = (mnew == -INFINITY || x == -INFINITY) ? 0.f : expf(x - mnew);
          float ps = pr;
#pragma unroll
          for (int o = 16; o > 0; o >>= 1) ps += __shfl_xor(ps, o);
          ps = __shfl(ps, half * 32);
          sS[qi][kr] = pr;
          if (kr == 0) {
            const float sc = (mold == -INFINITY) ? (mnew == -INFINITY ? 1.f : 0.f) : expf(mold - mnew);
            sScale[qi] = sc;
            sL[qi] = sL[qi] * sc + ps;
            sM[qi] = mnew;
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < AT_QT / 2; ++i) {
        const int qi = qpv + i * qg_pv;
        if (qi < nq) {
          float s0 = 0.f, s1 = 0.f;
#pragma unroll
          for (int kr = 0; kr < AT_KT; kr += 2) {  // keys >= nk have weight 0 and value 0
            s0 += sS[qi][kr] * sV[kr][dpv];
            s1 += sS[qi][kr + 1] * sV[kr + 1][dpv];
          }
          acc[i] = acc[i] * sScale[qi] + (s0 + s1);
        }
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < AT_QT / 2; ++i) {
      const int qi = qpv + i * qg_pv;
      if (qi < nq) part[qi * prec + 2 + dpv] = acc[i];
    }
    if (tid < nq) {
      part[tid * prec] = sM[tid];
      part[tid * prec + 1] = sL[tid];
    }
  } else {
    // in-tree keys of a level row: its ancestors' slots and its own
    for (int qi = wave; qi < nq; qi += 4) {
      const int gq = q0 + qi, j = gq / g;
      const eagle_frontier_node& nd = a.frontier[((size_t)a.depth * a.B + b) * a.k + j];
      float m = -INFINITY, l = 0.f, o0 = 0.f, o1 = 0.f;
      const float qa = sQ[qi][lane], qb = (lane + 64 < hd) ? sQ[qi][lane + 64] : 0.f;
      // every ancestor's K/V is loaded up front so the loads overlap
      float ka[EAGLE_MAX_DEPTH], kb[EAGLE_MAX_DEPTH], va[EAGLE_MAX_DEPTH], vb[EAGLE_MAX_DEPTH];
#pragma unroll
      for (int dep = 1; dep <= EAGLE_MAX_DEPTH; ++dep) {
        ka[dep - 1] = kb[dep - 1] = va[dep - 1] = vb[dep - 1] = 0.f;
        if (dep <= a.depth) {
          const size_t off =
              ((((size_t)b * a.D + dep) * a.k + clamp_slot(nd.anc[dep - 1], a.k)) * a.Hkv + kvh) * hd;
          const T* kp = (const T*)a.tk + off;
          const T* vp = (const T*)a.tv + off;
          ka[dep - 1] = El<T>::ld(kp, lane);
          va[dep - 1] = El<T>::ld(vp, lane);
          if (lane + 64 < hd) {
            kb[dep - 1] = El<T>::ld(kp, lane + 64);
            vb[dep - 1] = El<T>::ld(vp, lane + 64);
          }
        }
      }
#pragma unroll
      for (int dep = 1; dep <= EAGLE_MAX_DEPTH; ++dep) {
        if (dep <= a.depth) {
          const float s = wave_sum(qa * ka[dep - 1] + qb * kb[dep - 1]);
          const float mnew = fmaxf(m, s);
          const float sc = (m == -INFINITY) ? 0.f : expf(m - mnew);
          const float pr = expf(s - mnew);
          l = l * sc + pr;
          o0 = o0 * sc + pr * va[dep - 1];
          o1 = o1 * sc + pr * vb[dep - 1];
          m = mnew;
        }
      }
      part[qi * prec + 2 + lane] = o0;
      if (lane + 64 < hd) part[qi * prec + 2 + lane + 64] = o1;
      if (lane == 0) {
        part[qi * prec] = m;
        part[qi * prec + 1] = l;
      }
    }
  }

  if (!arrive_last(a.cnt + wg, p.nsplit)) return;

  // merge the slices in slice order: per-query weights first (LDS), then the
  // weighted sum of each slice's unnormalised output
  float* sw = &sK[0][0];  // [nq][nsplit] slice sums, then weights; nq * nsplit <= 32 * 128
  float* smx = &sV[0][0];  // [nq][nsplit] slice maxima
  const float* wbase = a.apart + (size_t)wg * p.nsplit * AT_QT * prec;
  for (int idx = tid; idx < nq * p.nsplit; idx += BLOCK) {
    const int qi = idx / p.nsplit, s = idx % p.nsplit;
    const float* ps = wbase + ((size_t)s * AT_QT + qi) * prec;
    smx[idx] = ps[0];
    sw[idx] = ps[1];
  }
  __syncthreads();
  if (tid < nq) {
    float M = -INFINITY;
    for (int s = 0; s < p.nsplit; ++s)
      if (sw[tid * p.nsplit + s] > 0.f) M = fmaxf(M, smx[tid * p.nsplit + s]);
    float L = 0.f;
    for (int s = 0; s < p.nsplit; ++s) {
      const float ls = sw[tid * p.nsplit + s];
      const float w = ls > 0.f ? expf(smx[tid * p.nsplit + s] - M) : 0.f;
      sw[tid * p.nsplit + s] = w;
      L += ls * w;
    }
    sScale[tid] = 1.0f / L;
  }
  __syncthreads();
  for (int idx = tid; idx < nq * hd; idx += BLOCK) {
    const int qi = idx / hd, dd = idx % hd, gq = q0 + qi;
    float O = 0.f;
#pragma unroll 8
    for (int s = 0; s < p.nsplit; ++s)
      O += sw[qi * p.nsplit + s] * wbase[((size_t)s * AT_QT + qi) * prec + 2 + dd];
    const int row = b * p.RS + gq / g, head = kvh * g + gq % g;
    El<T>::st((T*)a.attn, (size_t)row * HD + head * hd + dd, O * sScale[qi]);
  }
}

hipError_t launch_attn(const RoundArgs& a, const AttnPlan& p, hipStream_t s) {
  const dim3 grid(a.B * a.Hkv * p.nqt, p.nsplit), block(BLOCK);
  if (a.dtype == EAGLE_BF16) {
    if (a.hd == 128) hipLaunchKernelGGL((k_attn<bf16_t, 128>), grid, block, 0, s, a, p);
    else hipLaunchKernelGGL((k_attn<bf16_t, 64>), grid, block, 0, s, a, p);
  } else {
    if (a.hd == 128) hipLaunchKernelGGL((k_attn<float, 128>), grid, block, 0, s, a, p);
    else hipLaunchKernelGGL((k_attn<float, 64>), grid, block, 0, s, a, p);
  }
  return hipGetLastError();
}

}  // namespace eg

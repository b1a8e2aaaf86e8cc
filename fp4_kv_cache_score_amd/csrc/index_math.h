// Indexer score arithmetic shared by the scan kernel and the fused score ->
// Top-K kernel, so that both produce the same float for every entry, bit for
// bit.  A pool entry's 512-byte E4M3 key row is held by 32 lanes, 16 bytes
// each: lane (sub = lane & 31) owns bytes [16 sub, 16 sub + 16), i.e. indexer
// head sub / 4 and 16 of its 64 dims; the two halves of a wave hold two
// entries.  Reading of the pages (they give no formula, only that Full /
// Reindex layers score the context with an indexer, "DeepSeek V4.1-Flash
// Cuts KV Cache by 437x", paragraph on the three operating modes):
//   s_j = sum_h w_h * ReLU(sum_i qI[h][i] * kI[j][h][i]),  8 heads x 64 E4M3.
#ifndef CSA2_INDEX_MATH_H
#define CSA2_INDEX_MATH_H

#include "csa2_internal.h"

namespace csa2 {

// This lane's 16 query values (E4M3 -> fp32, exact).
__device__ __forceinline__ void load_q_slice(const uint8_t* qsrc, float (&qf)[16]) {
  const u32x4 qv = *reinterpret_cast<const u32x4*>(qsrc);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)qv[d], false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)qv[d], true);
    qf[4 * d + 0] = lo.x;
    qf[4 * d + 1] = lo.y;
    qf[4 * d + 2] = hi.x;
    qf[4 * d + 3] = hi.y;
  }
}

__device__ __forceinline__ float bfly_add(float v, int m) { return v + __shfl_xor(v, m, 64); }

// The score of the entry whose 16 key bytes this lane holds in v (wh: the
// weight of this lane's head).  The FP8 x FP8 products are exact in fp32;
// each lane accumulates its 16 with fmaf, a 4-lane butterfly completes the
// head dot, then ReLU, the head weight and an 8-head butterfly give the
// score in every lane of the half-wave.  Every lane must take part.
__device__ __forceinline__ float entry_score(const u32x4& v, const float (&qf)[16], float wh) {
  float acc = 0.f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[d], false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[d], true);
    acc = fmaf(lo.x, qf[4 * d + 0], acc);
    acc = fmaf(lo.y, qf[4 * d + 1], acc);
    acc = fmaf(hi.x, qf[4 * d + 2], acc);
    acc = fmaf(hi.y, qf[4 * d + 3], acc);
  }
  acc = bfly_add(acc, 1);
  acc = bfly_add(acc, 2);
  float r = acc > 0.f ? acc * wh : 0.f;
  r = bfly_add(r, 4);
  r = bfly_add(r, 8);
  r = bfly_add(r, 16);
  return r;
}

}  // namespace csa2

#endif  // CSA2_INDEX_MATH_H

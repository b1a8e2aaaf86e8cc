// Decode attention over the selected FP4 global entries and the FP8 window.
//
// The global entries are FP4 E2M1 with one E8M0 scale per 32 elements and are
// restored to real values right before use; the sliding-window rows are FP8
// ("DeepSeek V4.1-Flash Cuts KV Cache by 437x", paragraphs on FP4 quantisation
// and sliding window attention; "DeepSeek V4.1 Flash Architecture Breakdown",
// section "How are cache precision and storage arranged?").  Keys and values
// are the same 512-wide latent row (shared K/V); all 16 heads share each
// gathered row, so each row is read from HBM once per query row.
//
// k_attn_partial: one work-group per (query row, split of 32 keys).  A split
// is either 32 gathered FP4 entries or 32 FP8 window rows (never mixed).
//   1. stage q (16 x 512 bf16) and the split's keys in LDS.  FP4 rows are
//      dequantised with gfx950's scaled FP4->bf16 convert (exact: an E2M1
//      value times a power of two has at most two significant bits), FP8 rows
//      with the FP8->f32 convert truncated to bf16 (exact for E4M3).
//   2. logits with v_dot2_f32_bf16 (bf16 products are exact in fp32); each
//      wave takes a quarter of the 512 dims and the quarters are summed in a
//      fixed order.
//   3. per-head max and exp (fp32), written as (max, sum) partials.
//   4. P x V in fp32 FMA (p is never rounded to bf16).
// k_attn_combine merges the splits (and optionally an incoming (o, lse)) by
// log-sum-exp weights in a fixed order: the result equals one softmax over
// the union of the key sets.  All arithmetic is fp32 VALU; decode keeps the
// matrix cores for the multi-query prefill contraction.
#include "csa2_internal.h"

namespace csa2 {
namespace {

constexpr int kThreads = 256;
constexpr int KS = kKeysPerSplit;            // 32 keys per split
constexpr int kCsStrideU = kD / 2 + 8;       // staged key row stride in u32 (bf16 pairs + pad)
constexpr int kQU = kD / 2;                  // q row stride in u32

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

__global__ __launch_bounds__(kThreads, 2)
void k_attn_partial(AttnArgs a, int32_t Sg) {
  __shared__ __attribute__((aligned(16))) uint32_t qs[kH * kQU];          // 16 KiB
  __shared__ __attribute__((aligned(16))) uint32_t cs[KS * kCsStrideU];   // 33 KiB
  __shared__ __attribute__((aligned(16))) float zp[4][kH][KS];            // 8 KiB
  __shared__ __attribute__((aligned(16))) float ps[KS][kH];               // 2 KiB
  __shared__ int valid_s[KS];

  const int row = blockIdx.y;
  const int split = blockIdx.x;
  const int S = gridDim.x;
  const int b = row / a.Q;
  const int t = row - b * a.Q;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  {  // q -> LDS
    const u32x4* qg = reinterpret_cast<const u32x4*>(a.q + (size_t)row * kH * kD);
    u32x4* qd = reinterpret_cast<u32x4*>(qs);
    for (int i = tid; i < kH * kD / 8; i += kThreads) qd[i] = qg[i];
  }

  if (split < Sg) {
    // FP4 gather: (key j, 32-element block) pairs; 16 code bytes + 1 scale each.
    for (int pr = tid; pr < KS * kScaleRow; pr += kThreads) {
      const int j = pr / kScaleRow;
      const int blk = pr - j * kScaleRow;
      const int kpos = split * KS + j;
      const int32_t e = kpos < a.K ? a.idx[(size_t)row * a.K + kpos] : -1;
      u32x4 o0 = {0u, 0u, 0u, 0u}, o1 = o0, o2 = o0, o3 = o0;
      if (e >= 0) {
        const size_t er = (size_t)b * (size_t)a.M + (size_t)e;
        const u32x4 codes = *reinterpret_cast<const u32x4*>(a.latent + er * kLatRow + blk * 16);
        const uint32_t sc = a.scale[er * kScaleRow + blk];
        const float scale = __uint_as_float(sc ? (sc << 23) : 0x00400000u);
        uint32_t w[16];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          w[4 * d + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes[d], scale, 0));
          w[4 * d + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes[d], scale, 1));
          w[4 * d + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes[d], scale, 2));
          w[4 * d + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes[d], scale, 3));
        }
        o0 = u32x4{w[0], w[1], w[2], w[3]};
        o1 = u32x4{w[4], w[5], w[6], w[7]};
        o2 = u32x4{w[8], w[9], w[10], w[11]};
        o3 = u32x4{w[12], w[13], w[14], w[15]};
      }
      u32x4* dst = reinterpret_cast<u32x4*>(cs + j * kCsStrideU + blk * 16);
      dst[0] = o0;
      dst[1] = o1;
      dst[2] = o2;
      dst[3] = o3;
      if (blk == 0) valid_s[j] = e >= 0;
    }
  } else {
    // FP8 window rows: (row j, 16-byte segment) pairs.
    const int ws = split - Sg;
    for (int pr = tid; pr < KS * (kD / 16); pr += kThreads) {
      const int j = pr / (kD / 16);
      const int seg = pr - j * (kD / 16);
      const int wr = ws * KS + j;
      const bool ok = wr < a.W;
      u32x4 o0 = {0u, 0u, 0u, 0u}, o1 = o0;
      if (ok) {
        const uint8_t* src = a.swa + ((size_t)b * a.swa_rows + t + wr) * kD + seg * 16;
        const u32x4 v = *reinterpret_cast<const u32x4*>(src);
        uint32_t w[8];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[d], false);
          const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[d], true);
          w[2 * d + 0] = (__float_as_uint(lo.x) >> 16) | (__float_as_uint(lo.y) & 0xFFFF0000u);
          w[2 * d + 1] = (__float_as_uint(hi.x) >> 16) | (__float_as_uint(hi.y) & 0xFFFF0000u);
        }
        o0 = u32x4{w[0], w[1], w[2], w[3]};
        o1 = u32x4{w[4], w[5], w[6], w[7]};
      }
      u32x4* dst = reinterpret_cast<u32x4*>(cs + j * kCsStrideU + seg * 8);
      dst[0] = o0;
      dst[1] = o1;
      if (seg == 0) valid_s[j] = ok;
    }
  }
  __syncthreads();

  {  // logits: wave = quarter of the dims; lane = 4 heads x 2 keys
    const int hg = lane >> 4;
    const int kg = lane & 15;
    const int u0 = wave * (kD / 8);          // first u32 of this wave's 128 dims
    float acc[4][2];
#pragma unroll
    for (int h = 0; h < 4; ++h) acc[h][0] = acc[h][1] = 0.f;
#pragma unroll 4
    for (int du = 0; du < kD / 8; du += 4) {
      u32x4 qv[4], cv[2];
#pragma unroll
      for (int h = 0; h < 4; ++h)
        qv[h] = *reinterpret_cast<const u32x4*>(qs + (4 * hg + h) * kQU + u0 + du);
#pragma unroll
      for (int k = 0; k < 2; ++k)
        cv[k] = *reinterpret_cast<const u32x4*>(cs + (kg + 16 * k) * kCsStrideU + u0 + du);
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
          for (int w = 0; w < 4; ++w)
            acc[h][k] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qv[h][w]), as_bf16x2(cv[k][w]),
                                                        acc[h][k], false);
    }
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      zp[wave][4 * hg + h][kg] = acc[h][0];
      zp[wave][4 * hg + h][kg + 16] = acc[h][1];
    }
  }
  __syncthreads();

  {  // softmax statistics: thread = (head, 2 keys)
    const int h = tid >> 4;
    const int j0 = tid & 15;
    float z[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int j = j0 + 16 * k;
      const float s = ((zp[0][h][j] + zp[1][h][j]) + zp[2][h][j]) + zp[3][h][j];
      z[k] = valid_s[j] ? s : -INFINITY;
    }
    float m = fmaxf(z[0], z[1]);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    float p0 = 0.f, p1 = 0.f;
    if (m != -INFINITY) {
      p0 = __expf(z[0] - m);
      p1 = __expf(z[1] - m);
    }
    float l = p0 + p1;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) l += __shfl_xor(l, o, 64);
    ps[j0][h] = p0;
    ps[j0 + 16][h] = p1;
    if (j0 == 0) {
      float* mlp = a.ml + (((size_t)row * S + split) * kH + h) * 2;
      mlp[0] = m;
      mlp[1] = l;
    }
  }
  __syncthreads();

  {  // P x V: wave = 4 heads, lane = 8 dims
    const int h0 = wave * 4;
    const int d0 = lane * 8;
    float acc[4][8];
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[h][i] = 0.f;
#pragma unroll 4
    for (int j = 0; j < KS; ++j) {
      const float4 p = *reinterpret_cast<const float4*>(&ps[j][h0]);
      const u32x4 c = *reinterpret_cast<const u32x4*>(cs + j * kCsStrideU + d0 / 2);
      float cf[8];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        cf[2 * w + 0] = __uint_as_float(c[w] << 16);
        cf[2 * w + 1] = __uint_as_float(c[w] & 0xFFFF0000u);
      }
      const float pv[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[h][i] = fmaf(pv[h], cf[i], acc[h][i]);
    }
    float* op = a.opart + (((size_t)row * S + split) * kH + h0) * kD + d0;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float4* dst = reinterpret_cast<float4*>(op + (size_t)h * kD);
      dst[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
      dst[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
    }
  }
}

// One work-group (64 lanes x 8 dims) per (head, query row).
__global__ __launch_bounds__(64)
void k_attn_combine(const float* __restrict__ opart, const float* __restrict__ ml,
                    int32_t S, const float* o_in, const float* lse_in, float* o,
                    float* lse) {
  const int h = blockIdx.x;
  const int row = blockIdx.y;
  const int d0 = threadIdx.x * 8;
  const float* mlr = ml + (size_t)row * S * kH * 2;
  float mx = -INFINITY;
  for (int s = 0; s < S; ++s) mx = fmaxf(mx, mlr[((size_t)s * kH + h) * 2]);
  float lin = -INFINITY;
  if (lse_in) {
    lin = lse_in[(size_t)row * kH + h];
    mx = fmaxf(mx, lin);
  }
  float L = 0.f;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  if (mx != -INFINITY) {
    for (int s = 0; s < S; ++s) {
      const float ms = mlr[((size_t)s * kH + h) * 2];
      const float ls = mlr[((size_t)s * kH + h) * 2 + 1];
      if (ls > 0.f) {
        const float wgt = __expf(ms - mx);
        L += ls * wgt;
        const float4* src = reinterpret_cast<const float4*>(opart + (((size_t)row * S + s) * kH + h) * kD + d0);
        const float4 x0 = src[0], x1 = src[1];
        acc[0] = fmaf(wgt, x0.x, acc[0]); acc[1] = fmaf(wgt, x0.y, acc[1]);
        acc[2] = fmaf(wgt, x0.z, acc[2]); acc[3] = fmaf(wgt, x0.w, acc[3]);
        acc[4] = fmaf(wgt, x1.x, acc[4]); acc[5] = fmaf(wgt, x1.y, acc[5]);
        acc[6] = fmaf(wgt, x1.z, acc[6]); acc[7] = fmaf(wgt, x1.w, acc[7]);
      }
    }
    if (lse_in && lin != -INFINITY) {
      const float wgt = __expf(lin - mx);
      L += wgt;
      const float4* src = reinterpret_cast<const float4*>(o_in + ((size_t)row * kH + h) * kD + d0);
      const float4 x0 = src[0], x1 = src[1];
      acc[0] = fmaf(wgt, x0.x, acc[0]); acc[1] = fmaf(wgt, x0.y, acc[1]);
      acc[2] = fmaf(wgt, x0.z, acc[2]); acc[3] = fmaf(wgt, x0.w, acc[3]);
      acc[4] = fmaf(wgt, x1.x, acc[4]); acc[5] = fmaf(wgt, x1.y, acc[5]);
      acc[6] = fmaf(wgt, x1.z, acc[6]); acc[7] = fmaf(wgt, x1.w, acc[7]);
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float4* dst = reinterpret_cast<float4*>(o + ((size_t)row * kH + h) * kD + d0);
  dst[0] = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  dst[1] = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
  if (threadIdx.x == 0) lse[(size_t)row * kH + h] = L > 0.f ? mx + logf(L) : -INFINITY;
}

}  // namespace

int32_t attn_splits_global(int32_t K) { return K > 0 ? (K + KS - 1) / KS : 0; }
int32_t attn_splits_window(int32_t W) { return W > 0 ? (W + KS - 1) / KS : 0; }

hipError_t launch_attn_partial(const AttnArgs& a, hipStream_t s) {
  const int32_t Sg = attn_splits_global(a.K);
  const int32_t Sw = attn_splits_window(a.W);
  if (Sg + Sw == 0) return hipSuccess;
  k_attn_partial<<<dim3((unsigned)(Sg + Sw), (unsigned)a.rows), dim3(kThreads), 0, s>>>(a, Sg);
  return hipGetLastError();
}

hipError_t launch_attn_combine(const float* opart, const float* ml, int32_t rows,
                               int32_t splits, const float* o_in, const float* lse_in,
                               float* o, float* lse, hipStream_t s) {
  k_attn_combine<<<dim3((unsigned)kH, (unsigned)rows), dim3(64), 0, s>>>(opart, ml, splits, o_in,
                                                                           lse_in, o, lse);
  return hipGetLastError();
}

}  // namespace csa2

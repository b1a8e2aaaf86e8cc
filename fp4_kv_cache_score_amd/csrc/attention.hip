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
// k_attn_partial: one work-group per (query row, split).  A row's keys are cut
// into chunks of 32 (the selected global entries first, then the window rows)
// and a split is a run of consecutive chunks, processed with an online
// softmax.  Per work-group:
//   prologue  q (16 x 512 bf16) and the split's entry numbers go to LDS, the
//             first chunk's codes are loaded into registers;
//   per chunk 1. dequantise the registers into an LDS tile of bf16 rows: FP4
//                with gfx950's scaled FP4->bf16 convert (exact: an E2M1 value
//                times a power of two has at most two significant bits), FP8
//                with the FP8->f32 convert truncated to bf16 (exact for E4M3);
//             2. issue the next chunk's loads, so that they are in flight
//                while this chunk is computed;
//             3. logits with v_dot2_f32_bf16 (the bf16 products are exact in
//                fp32): each wave takes a quarter of the 512 dims and the
//                quarters are summed in a fixed order;
//             4. running max / sum per head (fp32), rescale factor, exp;
//             5. P x V in fp32 FMA (p is never rounded to bf16).
// With one split per row the work-group normalises and writes o and lse;
// otherwise it writes (unnormalised o, max, sum) partials and k_attn_combine
// merges them (and optionally an incoming (o, lse)) by log-sum-exp weights in
// a fixed order, so that the result equals one softmax over the union of the
// key sets.  All arithmetic is fp32 VALU; decode keeps the matrix cores for
// the multi-query prefill contraction.
#include "csa2_internal.h"

namespace csa2 {
namespace {

constexpr int kThreads = 256;
constexpr int KS = kKeysPerSplit;            // 32 keys per chunk
constexpr int kCsStrideU = kD / 2 + 4;       // staged key row stride in u32: 16 rows hit 16 bank groups
constexpr int kQU = kD / 2 + 4;              // q row stride in u32 (padded like the key rows)
constexpr int kZS = KS + 4;                  // logit row stride (4 heads of a wave in 4 bank groups)
constexpr int kMaxChunksPerSplit = 32;       // entry numbers staged per work-group: 1024
constexpr int kGroupsPerRound = 256;         // work-groups that run at once, one per compute unit

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

struct ChunkRegs {
  u32x4 v[4];       // global: 2 x 16 code bytes; window: 4 x 16 E4M3 bytes
  uint32_t sc[2];   // global: E8M0 scale codes
  int32_t e[2];     // global: entry numbers (-1: none)
  bool ok[4];       // window: row present
};

__device__ __forceinline__ void load_chunk(const AttnArgs& a, int chunk, int Cg, int b, int t,
                                           const int32_t* idx_s, int key0, ChunkRegs& r) {
  const int tid = threadIdx.x;
  if (chunk < Cg) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int pr = tid + i * kThreads;        // (key j, 32-element block) pair
      const int j = pr >> 4;
      const int blk = pr & 15;
      const int kpos = chunk * KS + j;
      const int32_t e = kpos < a.K ? idx_s[kpos - key0] : -1;
      r.e[i] = e;
      if (e >= 0) {
        const size_t er = (size_t)b * (size_t)a.M + (size_t)e;
        r.v[i] = *reinterpret_cast<const u32x4*>(a.latent + er * kLatRow + blk * 16);
        r.sc[i] = a.scale[er * kScaleRow + blk];
      }
    }
  } else {
    const int wc = chunk - Cg;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pr = tid + i * kThreads;        // (row j, 16-byte segment) pair
      const int j = pr >> 5;
      const int seg = pr & 31;
      const int wr = wc * KS + j;
      r.ok[i] = wr < a.W;
      if (r.ok[i]) {
        const uint8_t* src = a.swa + ((size_t)b * a.swa_rows + t + wr) * kD + seg * 16;
        r.v[i] = *reinterpret_cast<const u32x4*>(src);
      }
    }
  }
}

__device__ __forceinline__ void stage_chunk(int chunk, int Cg, const ChunkRegs& r, uint32_t* cs,
                                            int* valid_s) {
  const int tid = threadIdx.x;
  if (chunk < Cg) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int pr = tid + i * kThreads;
      const int j = pr >> 4;
      const int blk = pr & 15;
      u32x4 o0 = {0u, 0u, 0u, 0u}, o1 = o0, o2 = o0, o3 = o0;
      if (r.e[i] >= 0) {
        const uint32_t sc = r.sc[i];
        const float scale = __uint_as_float(sc ? (sc << 23) : 0x00400000u);   // 2^(sc-127)
        uint32_t w[16];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          w[4 * d + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(r.v[i][d], scale, 0));
          w[4 * d + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(r.v[i][d], scale, 1));
          w[4 * d + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(r.v[i][d], scale, 2));
          w[4 * d + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(r.v[i][d], scale, 3));
        }
        o0 = u32x4{w[0], w[1], w[2], w[3]};
        o1 = u32x4{w[4], w[5], w[6], w[7]};
        o2 = u32x4{w[8], w[9], w[10], w[11]};
        o3 = u32x4{w[12], w[13], w[14], w[15]};
      }
      // The 16 lanes of a key write its 1 KiB row; lane blk writes its four
      // 16-byte pieces in the order rotated by blk/4, so that each store
      // instruction covers 16 distinct bank groups.
      u32x4* dst = reinterpret_cast<u32x4*>(cs + j * kCsStrideU + blk * 16);
      const int rot = blk >> 2;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int c = (q4 + rot) & 3;
        const u32x4 x = c == 0 ? o0 : (c == 1 ? o1 : (c == 2 ? o2 : o3));
        dst[c] = x;
      }
      if (blk == 0) valid_s[j] = r.e[i] >= 0;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pr = tid + i * kThreads;
      const int j = pr >> 5;
      const int seg = pr & 31;
      u32x4 o0 = {0u, 0u, 0u, 0u}, o1 = o0;
      if (r.ok[i]) {
        uint32_t w[8];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)r.v[i][d], false);
          const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)r.v[i][d], true);
          w[2 * d + 0] = (__float_as_uint(lo.x) >> 16) | (__float_as_uint(lo.y) & 0xFFFF0000u);
          w[2 * d + 1] = (__float_as_uint(hi.x) >> 16) | (__float_as_uint(hi.y) & 0xFFFF0000u);
        }
        o0 = u32x4{w[0], w[1], w[2], w[3]};
        o1 = u32x4{w[4], w[5], w[6], w[7]};
      }
      // lanes seg and seg + 8 store their two pieces in opposite order
      u32x4* dst = reinterpret_cast<u32x4*>(cs + j * kCsStrideU + seg * 8);
      const int rot = (seg >> 3) & 1;
      dst[rot] = rot ? o1 : o0;
      dst[rot ^ 1] = rot ? o0 : o1;
      if (seg == 0) valid_s[j] = r.ok[i];
    }
  }
}

// G heads per work-group (16 or 8): grid (splits, rows, 16 / G).
template <int G>
__global__ __launch_bounds__(kThreads, 2)
void k_attn_partial(AttnArgs a, int32_t Cg, int32_t C, int32_t cps, int32_t final_out) {
  static_assert(G == 16 || G == 8, "heads per work-group");
  constexpr int NHG = G / 4;               // groups of 4 heads
  constexpr int KG = 64 / NHG;             // logits: key lanes per head group
  constexpr int NK = 32 / KG;              // logits: keys per lane
  constexpr int SPH = kThreads / G;        // softmax: threads per head
  constexpr int SK = KS / SPH;             // softmax: keys per thread
  constexpr int DP = 4 / NHG;              // P x V: dim parts
  constexpr int LD = kD / DP / 64;         // P x V: dims per lane
  __shared__ __attribute__((aligned(16))) uint32_t qs[G * kQU];
  __shared__ __attribute__((aligned(16))) uint32_t cs[KS * kCsStrideU];   // 33 KiB
  __shared__ __attribute__((aligned(16))) float zp[4][G][kZS];
  __shared__ __attribute__((aligned(16))) float ps[KS][G];
  __shared__ int32_t idx_s[kMaxChunksPerSplit * KS];                      // 4 KiB
  __shared__ int valid_s[KS];
  __shared__ float mh[G], lh[G];
  __shared__ __attribute__((aligned(16))) float ah[G];

  const int row = blockIdx.y;
  const int split = blockIdx.x;
  const int S = gridDim.x;
  const int hb = blockIdx.z * G;           // first head of this work-group
  const int b = row / a.Q;
  const int t = row - b * a.Q;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int c0 = split * cps;
  const int c1 = (c0 + cps < C) ? c0 + cps : C;

  {  // q of the G heads -> LDS
    const u32x4* qg = reinterpret_cast<const u32x4*>(a.q + ((size_t)row * kH + hb) * kD);
    for (int i = tid; i < G * kD / 8; i += kThreads)   // 64 16-byte pieces per head row
      *reinterpret_cast<u32x4*>(qs + (i >> 6) * kQU + (i & 63) * 4) = qg[i];
  }
  // entry numbers of this split's global keys -> LDS
  const int key0 = c0 * KS;
  const int gend = (c1 < Cg ? c1 : Cg) * KS;
  const int key1 = gend < a.K ? gend : a.K;
  for (int k = key0 + tid; k < key1; k += kThreads) idx_s[k - key0] = a.idx[(size_t)row * a.K + k];
  if (tid < G) {
    mh[tid] = -INFINITY;
    lh[tid] = 0.f;
  }
  __syncthreads();

  ChunkRegs r;
  load_chunk(a, c0, Cg, b, t, idx_s, key0, r);

  // P x V accumulators: wave = (4 heads, 1/DP of the dims), lane = LD dims
  const int h0 = 4 * (wave % NHG);
  const int d0 = (wave / NHG) * (kD / DP) + lane * LD;
  float acc[4][LD];
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int i = 0; i < LD; ++i) acc[h][i] = 0.f;

  for (int c = c0; c < c1; ++c) {
    stage_chunk(c, Cg, r, cs, valid_s);
    __syncthreads();
    if (c + 1 < c1) load_chunk(a, c + 1, Cg, b, t, idx_s, key0, r);

    {  // logits: wave = quarter of the dims; lane = 4 heads x NK keys
      const int hg = lane / KG;
      const int kg = lane % KG;
      const int u0 = wave * (kD / 8);          // first u32 of this wave's 128 dims
      float z[4][NK];
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int k = 0; k < NK; ++k) z[h][k] = 0.f;
#pragma unroll 4
      for (int du = 0; du < kD / 8; du += 4) {
        u32x4 qv[4], cv[NK];
#pragma unroll
        for (int h = 0; h < 4; ++h)
          qv[h] = *reinterpret_cast<const u32x4*>(qs + (4 * hg + h) * kQU + u0 + du);
#pragma unroll
        for (int k = 0; k < NK; ++k)
          cv[k] = *reinterpret_cast<const u32x4*>(cs + (kg + KG * k) * kCsStrideU + u0 + du);
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
          for (int k = 0; k < NK; ++k)
#pragma unroll
            for (int w = 0; w < 4; ++w)
              z[h][k] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qv[h][w]), as_bf16x2(cv[k][w]),
                                                        z[h][k], false);
      }
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int k = 0; k < NK; ++k) zp[wave][4 * hg + h][kg + KG * k] = z[h][k];
    }
    __syncthreads();

    {  // online softmax statistics: thread = (head, SK keys)
      const int h = tid / SPH;
      const int j0 = tid % SPH;
      float z[SK];
#pragma unroll
      for (int k = 0; k < SK; ++k) {
        const int j = j0 + SPH * k;
        const float s = ((zp[0][h][j] + zp[1][h][j]) + zp[2][h][j]) + zp[3][h][j];
        z[k] = valid_s[j] ? s : -INFINITY;
      }
      float m = z[0];
#pragma unroll
      for (int k = 1; k < SK; ++k) m = fmaxf(m, z[k]);
#pragma unroll
      for (int o = 1; o < SPH; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      const float m_old = mh[h];
      const float m_new = fmaxf(m_old, m);
      float p[SK];
      float alpha = 1.f;
#pragma unroll
      for (int k = 0; k < SK; ++k) p[k] = 0.f;
      if (m_new != -INFINITY) {
#pragma unroll
        for (int k = 0; k < SK; ++k) p[k] = __expf(z[k] - m_new);
        alpha = __expf(m_old - m_new);
      }
      float l = p[0];
#pragma unroll
      for (int k = 1; k < SK; ++k) l += p[k];
#pragma unroll
      for (int o = 1; o < SPH; o <<= 1) l += __shfl_xor(l, o, 64);
#pragma unroll
      for (int k = 0; k < SK; ++k) ps[j0 + SPH * k][h] = p[k];
      if (j0 == 0) {
        mh[h] = m_new;
        lh[h] = lh[h] * alpha + l;
        ah[h] = alpha;
      }
    }
    __syncthreads();

    {  // P x V
      const float4 al = *reinterpret_cast<const float4*>(&ah[h0]);
      const float alv[4] = {al.x, al.y, al.z, al.w};
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int i = 0; i < LD; ++i) acc[h][i] *= alv[h];
#pragma unroll 4
      for (int j = 0; j < KS; ++j) {
        const float4 p = *reinterpret_cast<const float4*>(&ps[j][h0]);
        uint32_t cw[LD / 2];
        if constexpr (LD == 8) {
          const u32x4 cv = *reinterpret_cast<const u32x4*>(cs + j * kCsStrideU + d0 / 2);
          cw[0] = cv[0]; cw[1] = cv[1]; cw[2] = cv[2]; cw[3] = cv[3];
        } else {
          const uint2 cv = *reinterpret_cast<const uint2*>(cs + j * kCsStrideU + d0 / 2);
          cw[0] = cv.x; cw[1] = cv.y;
        }
        float cf[LD];
#pragma unroll
        for (int w = 0; w < LD / 2; ++w) {
          cf[2 * w + 0] = __uint_as_float(cw[w] << 16);
          cf[2 * w + 1] = __uint_as_float(cw[w] & 0xFFFF0000u);
        }
        const float pv[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
          for (int i = 0; i < LD; ++i) acc[h][i] = fmaf(pv[h], cf[i], acc[h][i]);
      }
    }
    __syncthreads();
  }

  if (final_out && S == 1) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float L = lh[h0 + h];
      const float inv = L > 0.f ? 1.f / L : 0.f;
      float* dst = a.o + ((size_t)row * kH + hb + h0 + h) * kD + d0;
#pragma unroll
      for (int i = 0; i < LD; i += 4)
        *reinterpret_cast<float4*>(dst + i) =
            make_float4(acc[h][i] * inv, acc[h][i + 1] * inv, acc[h][i + 2] * inv, acc[h][i + 3] * inv);
    }
    if (tid < G) {
      const float L = lh[tid];
      a.lse[(size_t)row * kH + hb + tid] = L > 0.f ? mh[tid] + logf(L) : -INFINITY;
    }
  } else {
    float* op = a.opart + (((size_t)row * S + split) * kH + hb + h0) * kD + d0;
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int i = 0; i < LD; i += 4)
        *reinterpret_cast<float4*>(op + (size_t)h * kD + i) =
            make_float4(acc[h][i], acc[h][i + 1], acc[h][i + 2], acc[h][i + 3]);
    if (tid < G) {
      float* mlp = a.ml + (((size_t)row * S + split) * kH + hb + tid) * 2;
      mlp[0] = mh[tid];
      mlp[1] = lh[tid];
    }
  }
}

// One work-group (128 lanes x 4 dims) per (head, query row).  Every split's
// (max, sum) pair is loaded at once, then the partial rows in unrolled groups
// of independent loads.
constexpr int kCombThreads = 128;
constexpr int kCombMaxS = 63;            // splits per row (lane kCombMaxS holds an incoming result)

__global__ __launch_bounds__(kCombThreads)
void k_attn_combine(const float* __restrict__ opart, const float* __restrict__ ml,
                    int32_t S, const float* o_in, const float* lse_in, float* o,
                    float* lse) {
  __shared__ float wgt_s[kCombMaxS + 1];
  __shared__ float L_s;
  const int h = blockIdx.x;
  const int row = blockIdx.y;
  const int tid = threadIdx.x;
  const float* mlr = ml + (size_t)row * S * kH * 2;
  if (tid < 64) {
    // lanes 0..S-1 hold one split each (S <= 63), lane S the incoming result
    float m = -INFINITY, l = 0.f;
    if (tid < S) {
      m = mlr[((size_t)tid * kH + h) * 2];
      l = mlr[((size_t)tid * kH + h) * 2 + 1];
    } else if (tid == S && lse_in) {
      const float li = lse_in[(size_t)row * kH + h];
      if (li != -INFINITY) {
        m = li;
        l = 1.f;
      }
    }
    if (!(l > 0.f)) m = -INFINITY;
    float mx = m;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    const float w = (mx != -INFINITY && l > 0.f) ? __expf(m - mx) : 0.f;
    // fixed-order sum of the weighted split sums (lane order)
    float Lsum = w * l;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) Lsum += __shfl_xor(Lsum, off, 64);
    if (tid <= S && tid <= kCombMaxS) wgt_s[tid] = w;
    if (tid == 0) L_s = Lsum > 0.f ? Lsum : 0.f;
    if (tid == 0) lse[(size_t)row * kH + h] = Lsum > 0.f ? mx + logf(Lsum) : -INFINITY;
  }
  __syncthreads();
  const float L = L_s;
  const int d0 = tid * 4;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const float* src = opart + ((size_t)row * S * kH + h) * kD + d0;
  int s = 0;
  for (; s + 4 <= S; s += 4) {
    float4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = *reinterpret_cast<const float4*>(src + (size_t)(s + u) * kH * kD);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float w = wgt_s[s + u];
      acc.x = fmaf(w, x[u].x, acc.x);
      acc.y = fmaf(w, x[u].y, acc.y);
      acc.z = fmaf(w, x[u].z, acc.z);
      acc.w = fmaf(w, x[u].w, acc.w);
    }
  }
  for (; s < S; ++s) {
    const float4 x = *reinterpret_cast<const float4*>(src + (size_t)s * kH * kD);
    const float w = wgt_s[s];
    acc.x = fmaf(w, x.x, acc.x);
    acc.y = fmaf(w, x.y, acc.y);
    acc.z = fmaf(w, x.z, acc.z);
    acc.w = fmaf(w, x.w, acc.w);
  }
  if (lse_in) {
    const float w = wgt_s[S];
    if (w > 0.f) {
      const float4 x = *reinterpret_cast<const float4*>(o_in + ((size_t)row * kH + h) * kD + d0);
      acc.x = fmaf(w, x.x, acc.x);
      acc.y = fmaf(w, x.y, acc.y);
      acc.z = fmaf(w, x.z, acc.z);
      acc.w = fmaf(w, x.w, acc.w);
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  *reinterpret_cast<float4*>(o + ((size_t)row * kH + h) * kD + d0) =
      make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

}  // namespace

int32_t attn_chunks(int32_t K, int32_t W) {
  return (K > 0 ? (K + KS - 1) / KS : 0) + (W > 0 ? (W + KS - 1) / KS : 0);
}

AttnPlan attn_plan(int64_t rows, int32_t chunks) {
  // Pick heads per work-group G (16 or 8) and splits S so that the launch
  // fills the chip without giving some compute units two work-groups while
  // others idle: estimated time = rounds of kGroupsPerRound work-groups x
  // (chunks per work-group x G/16 + a fixed prologue), plus a merge launch
  // when S > 1.
  AttnPlan best{16, 1, 0.0};
  if (chunks <= 0) return AttnPlan{16, 0, 0.0};
  double best_cost = 1e30;
  for (int G = 16; G >= 8; G /= 2) {
    const int64_t lo = (chunks + kMaxChunksPerSplit - 1) / kMaxChunksPerSplit;
    for (int64_t S = lo; S <= chunks && S <= kCombMaxS; ++S) {
      const int64_t cps = (chunks + S - 1) / S;
      const int64_t Se = (chunks + cps - 1) / cps;
      if (Se != S) continue;
      const int64_t groups = rows * (16 / G) * S;
      const int64_t rounds = (groups + kGroupsPerRound - 1) / kGroupsPerRound;
      const double cost = (double)rounds * ((double)cps * G / 16.0 + 0.5) + (S > 1 ? 1.0 : 0.0);
      if (cost < best_cost - 1e-9) {
        best_cost = cost;
        best = AttnPlan{G, (int32_t)S, cost};
      }
    }
  }
  return best;
}

hipError_t launch_attn_partial(const AttnArgs& a, const AttnPlan& plan, bool final_out, hipStream_t s) {
  const int32_t Cg = a.K > 0 && a.latent ? (a.K + KS - 1) / KS : 0;
  const int32_t C = Cg + (a.W > 0 ? (a.W + KS - 1) / KS : 0);
  const int32_t splits = plan.splits;
  if (C == 0 || splits <= 0) return hipSuccess;
  const int32_t cps = (C + splits - 1) / splits;
  if (cps > kMaxChunksPerSplit || (C + cps - 1) / cps != splits) return hipErrorInvalidValue;
  const dim3 block(kThreads);
  if (plan.G == 8)
    k_attn_partial<8><<<dim3((unsigned)splits, (unsigned)a.rows, 2), block, 0, s>>>(
        a, Cg, C, cps, final_out ? 1 : 0);
  else
    k_attn_partial<16><<<dim3((unsigned)splits, (unsigned)a.rows, 1), block, 0, s>>>(
        a, Cg, C, cps, final_out ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_attn_combine(const float* opart, const float* ml, int32_t rows,
                               int32_t splits, const float* o_in, const float* lse_in,
                               float* o, float* lse, hipStream_t s) {
  if (splits > kCombMaxS) return hipErrorInvalidValue;
  k_attn_combine<<<dim3((unsigned)kH, (unsigned)rows), dim3(kCombThreads), 0, s>>>(
      opart, ml, splits, o_in, lse_in, o, lse);
  return hipGetLastError();
}

}  // namespace csa2

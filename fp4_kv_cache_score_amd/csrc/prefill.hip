// Chunked-prefill kernels: the indexer score and the sparse attention of many
// query tokens at once, as matrix-core (MFMA) contractions.
//
// A prefill chunk runs the same CSA2 steps as decode for Q query tokens at a
// time: score the pool with the indexer, select Top-K per token, attend over
// the selected FP4 entries and the FP8 window ("DeepSeek V4.1-Flash Cuts KV
// Cache by 437x", paragraphs on prefill cost, the three operating modes and
// sliding window attention).  With Q tokens the score is a dense contraction
// per indexer head ([Q x 64] . [64 x M] in E4M3), and the attention of one
// token is a contraction over its gathered keys with the 16 heads as rows.
//
// k_prefill_score: one work-group per 128 queries x 128 pool entries.  For
//   each of the 8 indexer heads the E4M3 query and key slices (64 values per
//   row) are staged in LDS as bf16 (exact: an E4M3 value has 4 significant
//   bits and an exponent inside bf16's range), double-buffered so that the
//   next head's loads are in flight during this head's math; each wave
//   computes a 64 x 64 block with v_mfma_f32_32x32x16_bf16 (the products are
//   exact in fp32), and the fp32 head result is folded into the score as
//   w_h * ReLU(.).  Entries a query cannot see yet are written as -inf.
//   The FP8 matrix instruction is not used: measured on gfx950, its
//   accumulation error reaches ~450 x 2^-24 of the sum of |products| (about
//   2^-15 relative), against ~0.4 x 2^-24 for the bf16 instruction and for
//   sequential fp32 FMA, and the score feeds an exact Top-K.
//
// k_prefill_attn: one work-group per query row.  The row's keys (selected
//   global entries, then its window rows) are taken 64 at a time, dequantised
//   exactly into a bf16 LDS tile (as in decode), and
//     S = q . C^T   with v_mfma_f32_16x16x32_bf16 (16 heads x 16 keys per wave)
//     online softmax per head in fp32,
//     O += P . C    with the same MFMA, P split into bf16 hi + lo parts so that
//                   the rounding of P stays below 2^-16 relative.
//   The P . C operand needs 8 consecutive keys of one dim per lane; it is read
//   as 32-bit pairs of dims from the key-major tile and repacked with
//   v_perm_b32, two dims feeding two output tiles.
#include "csa2_internal.h"

namespace csa2 {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Indexer score (FP8 MFMA)
// ---------------------------------------------------------------------------

constexpr int kSQ = 128;                 // queries per work-group tile
constexpr int kSE = 128;                 // pool entries per work-group tile
constexpr int kSThreads = 256;
constexpr int kSRow = 128 + 16;          // LDS bytes per staged row (64 bf16 of one head + pad)

__device__ __forceinline__ int64_t visible(int64_t pos0, int32_t t, int32_t ratio, int64_t M) {
  if (pos0 < 0) return M;
  const int64_t v = (pos0 + t + 1) / ratio;
  return v < M ? v : M;
}

// Scores of entries 0 .. N-1 (N <= M; also the score row length) for every
// query; n_valid (optional, [B][Q]) receives each query's visible count.
__global__ __launch_bounds__(kSThreads, 2)
void k_prefill_score(const uint8_t* __restrict__ key, int64_t M, int32_t N,
                     const uint8_t* __restrict__ q_idx, const float* __restrict__ w_idx,
                     int32_t Q, int64_t pos0, int32_t ratio, float* __restrict__ scores,
                     int32_t* __restrict__ n_valid) {
  __shared__ __attribute__((aligned(16))) uint8_t qs[2][kSQ * kSRow];
  __shared__ __attribute__((aligned(16))) uint8_t ks[2][kSE * kSRow];
  __shared__ __attribute__((aligned(16))) float ws[kHI][kSQ];   // head weights, rows contiguous
  __shared__ int32_t vis_s[kSQ];          // entries visible to each query row of the tile

  const int b = blockIdx.z;
  const int q0 = blockIdx.y * kSQ;
  const int64_t e0 = (int64_t)blockIdx.x * kSE;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wq = wave & 1;                // 64-query half of the tile
  const int we = wave >> 1;               // 64-entry half of the tile
  const uint8_t* qb = q_idx + (size_t)b * Q * kKeyRow;
  const uint8_t* kb = key + (size_t)b * (size_t)M * kKeyRow;
  float* sb = scores + (size_t)b * Q * (size_t)N;
  if (n_valid && blockIdx.x == 0 && tid < kSQ && q0 + tid < Q)
    n_valid[(size_t)b * Q + q0 + tid] = (int32_t)visible(pos0, q0 + tid, ratio, M);

  const int qlast = (q0 + kSQ < Q ? q0 + kSQ : Q) - 1;
  if (e0 >= visible(pos0, qlast, ratio, M)) {   // no query of the tile sees these entries
    for (int i = tid; i < kSQ * kSE; i += kSThreads) {
      const int r = i / kSE, c = i - r * kSE;
      if (q0 + r < Q && e0 + c < N) sb[(size_t)(q0 + r) * N + e0 + c] = -INFINITY;
    }
    return;
  }

  for (int i = tid; i < kSQ * kHI; i += kSThreads) {
    const int r = i / kHI, h = i - r * kHI;
    ws[h][r] = q0 + r < Q ? w_idx[((size_t)b * Q + q0 + r) * kHI + h] : 0.f;
  }
  if (tid < kSQ) vis_s[tid] = (int32_t)visible(pos0, q0 + tid, ratio, M);   // one division per row

  // staging: thread -> two (row, 16-byte part) pieces of each of Q and K.
  // Rows past Q or N load the last row instead (never written out), so the
  // loads are unconditional.
  u32x4 rq[2], rk[2];
  const uint8_t* qrow[2];
  const uint8_t* krow[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + i * kSThreads;
    const int row = c >> 2, part = c & 3;
    const int t = q0 + row < Q ? q0 + row : Q - 1;
    const int64_t e = e0 + row < N ? e0 + row : N - 1;
    qrow[i] = qb + (size_t)t * kKeyRow + part * 16;
    krow[i] = kb + (size_t)e * kKeyRow + part * 16;
  }
  auto load = [&](int h) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      rq[i] = *reinterpret_cast<const u32x4*>(qrow[i] + h * kDI);
      rk[i] = *reinterpret_cast<const u32x4*>(krow[i] + h * kDI);
    }
  };
  // 16 E4M3 values -> 16 bf16 (two 16-byte pieces), exact
  auto widen = [](const u32x4& x, u32x4& lo, u32x4& hi) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t w0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x[d], 1.0f, false));
      const uint32_t w1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x[d], 1.0f, true));
      if (d < 2) {
        lo[2 * d] = w0;
        lo[2 * d + 1] = w1;
      } else {
        hi[2 * d - 4] = w0;
        hi[2 * d - 3] = w1;
      }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = tid + i * kSThreads;
      const int row = c >> 2, part = c & 3;
      u32x4 lo, hi;
      widen(rq[i], lo, hi);
      *reinterpret_cast<u32x4*>(&qs[buf][row * kSRow + part * 32]) = lo;
      *reinterpret_cast<u32x4*>(&qs[buf][row * kSRow + part * 32 + 16]) = hi;
      widen(rk[i], lo, hi);
      *reinterpret_cast<u32x4*>(&ks[buf][row * kSRow + part * 32]) = lo;
      *reinterpret_cast<u32x4*>(&ks[buf][row * kSRow + part * 32 + 16]) = hi;
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[r][c][v] = 0.f;

  // Per head: MFMA on the staged buffer, then the next head is staged from
  // the registers (loaded one head's compute earlier) and the head after it
  // is loaded into them.
  load(0);
  store(0);
  load(1);
  __syncthreads();
  const int g = lane >> 5;       // which 32-value half of the head slice
  const int lr = lane & 31;
#pragma unroll 1
  for (int h = 0; h < kHI; ++h) {
    const int buf = h & 1;
    // operands: lane holds 32 bf16 (4 k-steps of 8) of its row's half g
    bf16x8 A[2][4], Bv[2][4];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const uint8_t* src = &qs[buf][(64 * wq + 32 * r + lr) * kSRow + 64 * g];
#pragma unroll
      for (int k = 0; k < 4; ++k) A[r][k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(src + 16 * k));
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint8_t* src = &ks[buf][(64 * we + 32 * c + lr) * kSRow + 64 * g];
#pragma unroll
      for (int k = 0; k < 4; ++k) Bv[c][k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(src + 16 * k));
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      // head weights of the 16 query rows this lane holds in each block
      float wv[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 w4 = *reinterpret_cast<const float4*>(&ws[h][64 * wq + 32 * r + 8 * j + 4 * g]);
        wv[4 * j] = w4.x;
        wv[4 * j + 1] = w4.y;
        wv[4 * j + 2] = w4.z;
        wv[4 * j + 3] = w4.w;
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        f32x16 s = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < 4; ++k) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[r][k], Bv[c][k], s, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          // ReLU on the bit pattern: a signed max with 0 maps negatives and -0 to +0
          const float rl = __int_as_float(max(__float_as_int(s[v]), 0));
          acc[r][c][v] = fmaf(rl, wv[v], acc[r][c][v]);
        }
      }
    }
    if (h + 1 < kHI) store(buf ^ 1);
    load(h + 2 < kHI ? h + 2 : kHI - 1);   // past the end: a harmless reload
    __syncthreads();
  }

  // write: value v of block (r, c) is query row 8*(v/4) + 4*g + v%4, entry lr
  const int32_t ea = (int32_t)e0 + 64 * we + lr;     // entries of blocks c = 0, 1
  const int32_t eb = ea + 32;
  const bool oka = ea < N, okb = eb < N;
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int tr = 64 * wq + 32 * r + 8 * (v >> 2) + 4 * g + (v & 3);
      if (q0 + tr >= Q) continue;
      const int32_t vis = vis_s[tr];
      float* srow = sb + (size_t)(q0 + tr) * N;
      if (oka) srow[ea] = ea < vis ? acc[r][0][v] : -INFINITY;
      if (okb) srow[eb] = eb < vis ? acc[r][1][v] : -INFINITY;
    }
}

// ---------------------------------------------------------------------------
// Sparse attention (bf16 MFMA)
// ---------------------------------------------------------------------------

constexpr int kAThreads = 256;
constexpr int kAC = 64;                      // keys per chunk
constexpr int kARowU = kD / 2 + 4;           // key row stride in u32 (1040 B)
constexpr int kAPRow = kAC + 8;              // P row stride in bf16 (144 B)
constexpr int kAIdx = 1024;                  // entry numbers staged in LDS

struct PfRegs {
  u32x4 v[8];        // global: 4 x 16 code bytes; window: 8 x 16 E4M3 bytes
  uint32_t sc[4];    // global: E8M0 scale codes, 0xFFFFFFFF for "no entry"
};

__global__ __launch_bounds__(kAThreads, 2)
void k_prefill_attn(AttnArgs a, int32_t Cg, int32_t C, const float* __restrict__ o_in,
                    const float* __restrict__ lse_in) {
  __shared__ __attribute__((aligned(16))) uint32_t cs[kAC * kARowU];        // 65 KiB
  __shared__ __attribute__((aligned(16))) uint16_t ph[kH * kAPRow];         // P hi
  __shared__ __attribute__((aligned(16))) uint16_t pl[kH * kAPRow];         // P lo
  __shared__ int32_t idx_s[kAIdx];
  __shared__ int valid_s[kAC];
  __shared__ float red[4][kH];

  const int row = blockIdx.x;
  const int b = row / a.Q;
  const int t = row - b * a.Q;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ln = lane & 15;        // MFMA column / A row
  const int lg = lane >> 4;        // MFMA k-group / output row group
  // window rows t + wr with wr < wfirst are positions before the context's
  // first token (a first chunk): never read, never keys
  const int64_t wgap = a.pos0 >= 0 ? (int64_t)(a.W - 1) - (a.pos0 + t) : 0;
  const int32_t wfirst = wgap > 0 ? (int32_t)wgap : 0;

  // q as A operands: head ln, dims 32 s + 8 lg .. +7, for k-steps s = 0..15
  bf16x8 qa[16];
  {
    const uint16_t* qr = a.q + ((size_t)row * kH + ln) * kD + 8 * lg;
#pragma unroll
    for (int s = 0; s < 16; ++s)
      qa[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qr + 32 * s));
  }
  const int nst = a.K < kAIdx ? a.K : kAIdx;
  for (int k = tid; k < nst; k += kAThreads) idx_s[k] = a.idx[(size_t)row * a.K + k];
  __syncthreads();

  auto entry = [&](int kpos) -> int32_t {
    if (kpos >= a.K) return -1;
    return kpos < kAIdx ? idx_s[kpos] : a.idx[(size_t)row * a.K + kpos];
  };
  PfRegs r;
  auto load = [&](int chunk) {
    if (chunk < Cg) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pr = tid + i * kAThreads;      // (key j, 32-element block)
        const int j = pr >> 4, blk = pr & 15;
        const int32_t e = entry(chunk * kAC + j);
        r.sc[i] = 0xFFFFFFFFu;
        if (e >= 0) {
          const size_t er = (size_t)b * (size_t)a.M + (size_t)e;
          r.v[i] = *reinterpret_cast<const u32x4*>(a.latent + er * kLatRow + blk * 16);
          r.sc[i] = a.scale[er * kScaleRow + blk];
        }
      }
    } else {
      const int wc = chunk - Cg;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int pr = tid + i * kAThreads;      // (row j, 16-byte segment)
        const int j = pr >> 5, seg = pr & 31;
        const int wr = wc * kAC + j;
        if (wr < a.W && wr >= wfirst)
          r.v[i] = *reinterpret_cast<const u32x4*>(a.swa + ((size_t)b * a.swa_rows + t + wr) * kD + seg * 16);
      }
    }
  };
  auto stage = [&](int chunk) {
    if (chunk < Cg) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int pr = tid + i * kAThreads;
        const int j = pr >> 4, blk = pr & 15;
        u32x4 o[4] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
        const bool present = r.sc[i] != 0xFFFFFFFFu;
        if (present) {
          const uint32_t sc = r.sc[i];
          const float scale = __uint_as_float(sc ? (sc << 23) : 0x00400000u);   // 2^(sc-127)
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            o[d][0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(r.v[i][d], scale, 0));
            o[d][1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(r.v[i][d], scale, 1));
            o[d][2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(r.v[i][d], scale, 2));
            o[d][3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(r.v[i][d], scale, 3));
          }
        }
        u32x4* dst = reinterpret_cast<u32x4*>(cs + j * kARowU + blk * 16);
        const int rot = blk >> 2;   // 16 lanes of a key row store to 16 bank groups
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int c = (q4 + rot) & 3;
          dst[c] = c == 0 ? o[0] : (c == 1 ? o[1] : (c == 2 ? o[2] : o[3]));
        }
        if (blk == 0) valid_s[j] = present;
      }
    } else {
      const int wc = chunk - Cg;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int pr = tid + i * kAThreads;
        const int j = pr >> 5, seg = pr & 31;
        const int wr = wc * kAC + j;
        const bool ok = wr < a.W && wr >= wfirst;
        u32x4 o0 = {0u, 0u, 0u, 0u}, o1 = o0;
        if (ok) {
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
        u32x4* dst = reinterpret_cast<u32x4*>(cs + j * kARowU + seg * 8);
        const int rot = (seg >> 3) & 1;
        dst[rot] = rot ? o1 : o0;
        dst[rot ^ 1] = rot ? o0 : o1;
        if (seg == 0) valid_s[j] = ok;
      }
    }
  };

  // Output accumulators: wave owns dims 128 wave .. +127 as 4 tile pairs;
  // tile 2u column n <-> dim 128 wave + 32 u + 2 n, tile 2u+1 <-> that + 1.
  f32x4 O[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) O[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[4], l_run[4];   // heads 4 lg + i
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.f;
  }

  if (C > 0) load(0);
#pragma unroll 1
  for (int c = 0; c < C; ++c) {
    stage(c);
    __syncthreads();
    if (c + 1 < C) load(c + 1);

    // S = q . C^T for keys 16 wave .. +15 of the chunk
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    {
      const uint32_t* kr = cs + (16 * wave + ln) * kARowU + 4 * lg;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const bf16x8 bk = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(kr + 16 * k));
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[k], bk, s, 0, 0, 0);
        if ((k & 3) == 3) __builtin_amdgcn_sched_barrier(0);   // at most 4 key operands in flight
      }
    }
    const bool kv = valid_s[16 * wave + ln] != 0;
    float cm[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = kv ? s[i] : -INFINITY;
      s[i] = x;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
      cm[i] = x;
    }
    if (ln == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][4 * lg + i] = cm[i];
    }
    __syncthreads();
    float alpha[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int hh = 4 * lg + i;
      const float mx = fmaxf(fmaxf(red[0][hh], red[1][hh]), fmaxf(red[2][hh], red[3][hh]));
      const float m_new = fmaxf(m_run[i], mx);
      float p = 0.f;
      alpha[i] = 1.f;
      if (m_new != -INFINITY) {
        p = __expf(s[i] - m_new);
        alpha[i] = __expf(m_run[i] - m_new);
      }
      m_run[i] = m_new;
      float ps = p;
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) ps += __shfl_xor(ps, o, 64);
      l_run[i] = l_run[i] * alpha[i] + ps;
      // P split into bf16 hi + lo (p - hi is exact in fp32)
      const uint32_t pu = __float_as_uint(p);
      const uint32_t hi = (pu + 0x7FFFu + ((pu >> 16) & 1u)) & 0xFFFF0000u;
      const float lo = p - __uint_as_float(hi);
      const uint32_t lu = __float_as_uint(lo);
      const uint32_t lo16 = (lu + 0x7FFFu + ((lu >> 16) & 1u)) >> 16;
      ph[hh * kAPRow + 16 * wave + ln] = (uint16_t)(hi >> 16);
      pl[hh * kAPRow + 16 * wave + ln] = (uint16_t)lo16;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) O[u][i] *= alpha[i];
    __syncthreads();

    // O += P . C: A = P[head ln][keys 32 ks + 8 lg ..], B = C[those keys][dim]
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 ahi = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&ph[ln * kAPRow + 32 * ks + 8 * lg]));
      const bf16x8 alo = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&pl[ln * kAPRow + 32 * ks + 8 * lg]));
      const uint32_t* kr = cs + (32 * ks + 8 * lg) * kARowU + 64 * wave + ln;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        uint32_t x[8];
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) x[rr] = kr[rr * kARowU + 16 * u];
        u32x4 be, bo;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          be[i] = __builtin_amdgcn_perm(x[2 * i + 1], x[2 * i], 0x05040100u);
          bo[i] = __builtin_amdgcn_perm(x[2 * i + 1], x[2 * i], 0x07060302u);
        }
        const bf16x8 bev = __builtin_bit_cast(bf16x8, be);
        const bf16x8 bov = __builtin_bit_cast(bf16x8, bo);
        O[2 * u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bev, O[2 * u], 0, 0, 0);
        O[2 * u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bev, O[2 * u], 0, 0, 0);
        O[2 * u + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bov, O[2 * u + 1], 0, 0, 0);
        O[2 * u + 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bov, O[2 * u + 1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);   // one tile pair's operands live at a time
      }
    }
    __syncthreads();
  }

  // total sum per head over the 4 waves' keys
  float lin[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) lin[i] = lse_in ? lse_in[(size_t)row * kH + 4 * lg + i] : -INFINITY;
  if (ln == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][4 * lg + i] = l_run[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int hh = 4 * lg + i;
    const float L = ((red[0][hh] + red[1][hh]) + red[2][hh]) + red[3][hh];
    float lse = L > 0.f ? m_run[i] + logf(L) : -INFINITY;
    float wself = L > 0.f ? 1.f / L : 0.f;
    float win = 0.f;
    if (lse_in) {   // merge with an incoming (o, lse) as one softmax over both key sets
      const float li = lin[i];   // read before the barrier above: lse may alias lse_in
      const float mx = fmaxf(li, lse);
      if (mx != -INFINITY) {
        const float ea = li == -INFINITY ? 0.f : __expf(li - mx);
        const float eb = lse == -INFINITY ? 0.f : __expf(lse - mx);
        const float tot = ea + eb;
        win = ea / tot;
        wself *= eb / tot;
        lse = mx + logf(tot);
      }
    }
    float* orow = a.o + ((size_t)row * kH + hh) * kD + 128 * wave + 2 * ln;
    const float* irow = lse_in ? o_in + ((size_t)row * kH + hh) * kD + 128 * wave + 2 * ln : nullptr;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float2 v = make_float2(O[2 * u][i] * wself, O[2 * u + 1][i] * wself);
      if (irow) {
        const float2 x = *reinterpret_cast<const float2*>(irow + 32 * u);
        v.x = fmaf(win, x.x, v.x);
        v.y = fmaf(win, x.y, v.y);
      }
      *reinterpret_cast<float2*>(orow + 32 * u) = v;
    }
    if (ln == 0 && wave == 0) a.lse[(size_t)row * kH + hh] = lse;
  }
}

}  // namespace

hipError_t launch_prefill_score(const uint8_t* key, int32_t B, int64_t M, int32_t N,
                                const uint8_t* q_idx, const float* w_idx, int32_t Q, int64_t pos0,
                                int32_t ratio, float* scores, int32_t* n_valid, hipStream_t s) {
  if (N <= 0 || N > M || Q <= 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((N + kSE - 1) / kSE), (unsigned)((Q + kSQ - 1) / kSQ), (unsigned)B);
  k_prefill_score<<<grid, dim3(kSThreads), 0, s>>>(key, M, N, q_idx, w_idx, Q, pos0, ratio, scores,
                                                   n_valid);
  return hipGetLastError();
}

hipError_t launch_prefill_attn(const AttnArgs& a, const float* o_in, const float* lse_in,
                               hipStream_t s) {
  const int32_t Cg = a.K > 0 && a.latent ? (a.K + kAC - 1) / kAC : 0;
  const int32_t C = Cg + (a.W > 0 ? (a.W + kAC - 1) / kAC : 0);
  k_prefill_attn<<<dim3((unsigned)a.rows), dim3(kAThreads), 0, s>>>(a, Cg, C, o_in, lse_in);
  return hipGetLastError();
}

}  // namespace csa2

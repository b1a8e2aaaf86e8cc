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
// k_prefill_attn: one work-group of two waves per query row; wave h owns
//   output dims 256 h .. 256 h + 255.  The row's keys (selected global entries,
//   then its window rows) are taken 32 per step.  Each lane loads 2 blocks of
//   32 dims of one key (this wave's half), dequantises them exactly to bf16
//   straight into the key operand of
//     S^T = C . q^T   (v_mfma_f32_16x16x32_bf16, 16 keys x 16 heads, the dims
//                      of the contraction taken in the order the lanes hold
//                      them, q permuted to match),
//   and stages the same bf16 rows in LDS.  The two waves' partial S^T (one per
//   dim half) are exchanged through LDS and added in a fixed order, so both run
//   the same online softmax per head in fp32.  S^T leaves each lane with P for
//   4 keys of one head, which is the A-operand layout of
//     O += P . C      (same MFMA; P split into bf16 hi + lo parts so that the
//                      rounding of P stays below 2^-16 relative),
//   whose B operand (8 keys of one dim per lane) comes from the staged rows with
//   gfx950's transposing LDS read (ds_read_b64_tr_b16).  The softmax reference
//   moves only when a logit exceeds it by more than 8 (natural log), outside the
//   inner loop, so O stays in the matrix accumulators.  One barrier per step.
#include "csa2_internal.h"

#include <type_traits>

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

// Entries query t sees: the first M (the sequence's length), within the causal limit.
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
                     int32_t* __restrict__ n_valid, const int32_t* __restrict__ len, PoolMap map) {
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
  float* sb = scores + (size_t)b * Q * (size_t)N;
  const int64_t Ms = len ? (int64_t)len[b] : M;           // this sequence's entries
  if (n_valid && blockIdx.x == 0 && tid < kSQ && q0 + tid < Q)
    n_valid[(size_t)b * Q + q0 + tid] = (int32_t)visible(pos0, q0 + tid, ratio, Ms);

  const int qlast = (q0 + kSQ < Q ? q0 + kSQ : Q) - 1;
  if (e0 >= visible(pos0, qlast, ratio, Ms)) {   // no query of the tile sees these entries
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
  if (tid < kSQ) vis_s[tid] = (int32_t)visible(pos0, q0 + tid, ratio, Ms);   // one division per row

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
    krow[i] = key + (size_t)pool_row(map, b, e, M) * kKeyRow + part * 16;
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
  // A tile inside the chunk and the scanned entries, all of whose entries its
  // first (least-seeing) query sees: every value is stored, no test per value;
  // 32-bit offsets from the sequence's score base.
  if (q0 + kSQ <= Q && e0 + kSE <= N && e0 + kSE <= (int64_t)vis_s[0] &&
      (uint64_t)Q * (uint64_t)N < (1ull << 31)) {
    const uint32_t o0 = (uint32_t)(q0 + 64 * wq + 4 * g) * (uint32_t)N + (uint32_t)ea;
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const uint32_t off = o0 + (uint32_t)(32 * r + 8 * (v >> 2) + (v & 3)) * (uint32_t)N;
        sb[off] = acc[r][0][v];
        sb[off + 32] = acc[r][1][v];
      }
    return;
  }
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

constexpr int kWK = 32;                        // keys per step (two MFMA sets of 16)
constexpr int kHalf = kD / 2;                  // output dims per wave
constexpr int kTRow = kHalf * 2;               // staged key row of one wave: 256 bf16 (512 B)
constexpr float kPfLazy = 8.f;                 // softmax reference slack (natural log units)

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef i16x4 __attribute__((address_space(3))) lds_i16x4;

// Max and sum over the four 16-lane rows (gfx950 permlane swaps).
__device__ __forceinline__ float pf_rows_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float pf_rows_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Byte offset of (key row r, byte c) in a wave's staged tile: 32-byte units
// XOR-swizzled by the row's low 3 bits, 16-byte halves swapped by its bit 3.
// The 8 rows that half a wave's transposed read touches then fall on 8
// different 32-byte bank groups, and the 16 rows of a staging store on 16
// different 16-byte ones.
__device__ __forceinline__ int tile_off(int r, int c) {
  return r * kTRow + ((((c >> 5) ^ (r & 7)) << 5) | ((c & 31) ^ (((r >> 3) & 1) << 4)));
}

template <bool kPaged>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_prefill_attn(AttnArgs a, int32_t Cg, int32_t Cw, const float* o_in, const float* lse_in) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[2][kWK * kTRow];   // 32 KiB
  __shared__ __attribute__((aligned(16))) float xs[2][2][64 * 8];         // partial S, by step parity

  // rows of one XCD are consecutive tokens (their window rows overlap in L2)
  int row;
  {
    const int bid = blockIdx.x, R = a.rows;
    const int q8 = R >> 3, r8 = R & 7, x = bid & 7, k = bid >> 3;
    row = x * q8 + (x < r8 ? x : r8) + k;
  }
  const int b = row / a.Q;
  const int t = row - b * a.Q;
  const int hw = threadIdx.x >> 6;           // this wave's half of the dims
  const int lane = threadIdx.x & 63;
  const int ln = lane & 15;
  const int lg = lane >> 4;
  const int64_t wgap = a.pos0 >= 0 ? (int64_t)(a.W - 1) - (a.pos0 + t) : 0;
  const int32_t wfirst = wgap > 0 ? (int32_t)wgap : 0;

  // q (this half) as the B operand of S^T = C . q^T: lane (head ln, group lg)
  // holds, for k-step s, dims 256 hw + 32 (4 (s / 4) + lg) + 8 (s % 4) .. +7,
  // the order in which the key operand below holds them
  bf16x8 qv[8];
  {
    const uint16_t* qr = a.q + ((size_t)row * kH + ln) * kD + kHalf * hw;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      qv[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                             qr + 32 * (4 * (s >> 2) + lg) + 8 * (s & 3)));
  }
  // the last position holding an entry (-1 entries select nothing); the
  // entry numbers are read 512 at a time, all loads in flight together
  const int32_t* irow = a.idx ? a.idx + (size_t)row * a.K : nullptr;
  int last = -1;
  if (Cg > 0) {
    for (int k0 = 0; k0 < a.K; k0 += 512) {
      int32_t e[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) e[u] = irow[min(k0 + 64 * u + lane, a.K - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (e[u] >= 0 && k0 + 64 * u + lane < a.K) last = max(last, k0 + 64 * u + lane);
    }
  }
  for (int o = 32; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o, 64));
  const int cg = __builtin_amdgcn_readfirstlane(Cg > 0 ? (last + kWK) / kWK : 0);
  const int ws0 = __builtin_amdgcn_readfirstlane(wfirst / kWK);   // window steps before position 0
  const int n_it = cg + (Cw > ws0 ? Cw - ws0 : 0);

  const uint8_t* lat_b = a.latent ? a.latent + 128 * hw : nullptr;   // indexed by pool row
  const uint8_t* sc_b = a.scale;
  const uint8_t* swa_b = a.swa ? a.swa + ((size_t)b * a.swa_rows + t) * kD + kHalf * hw : nullptr;
  // a readable stand-in for loads past the last step (this row's q: 16 KiB)
  const uint8_t* spare = reinterpret_cast<const uint8_t*>(a.q + (size_t)row * kH * kD);
  const int kmax = a.K > 0 ? a.K - 1 : 0;

  // entry number for step `it` (an unconditional load at a clamped position)
  const int32_t* irow_s = irow ? irow : reinterpret_cast<const int32_t*>(spare);
  auto entry = [&](int it, int u) __attribute__((always_inline)) -> int32_t {
    return irow_s[min(it * kWK + 16 * u + ln, kmax)];
  };
  // step `it`, set u: key 16 u + ln; lane group lg loads blocks lg and 4 + lg
  // of this half.  Global: v0, v1 = 16 E2M1 bytes each, v2 = v3 = the entry's
  // scale bytes.  Window: (v0, v1), (v2, v3) = 32 E4M3 bytes each.  All four
  // loads are issued unconditionally from selected, valid addresses.
  auto load = [&](int it, int u, int32_t e, u32x4& v0, u32x4& v1, u32x4& v2, u32x4& v3)
      __attribute__((always_inline)) -> bool {
    const bool g = it < cg;
    const int kpos = it * kWK + 16 * u + ln;
    const bool okg = kpos < a.K && e >= 0;
    const int wr = (it - cg + ws0) * kWK + 16 * u + ln;
    const bool okw = wr < a.W && wr >= wfirst;
    const uint8_t *p0, *p1, *p2, *p3;
    if (g) {
      const int32_t ec = okg ? e : 0;                         // entry 0 exists
      // the paged kind has its own kernel, so the contiguous loop holds no table load
      const int64_t pr = kPaged ? pool_row(a.map, b, ec, a.M) : (int64_t)b * a.M + ec;
      const uint8_t* gl = lat_b + (size_t)pr * kLatRow;
      p0 = gl + 16 * lg;
      p1 = gl + 16 * (4 + lg);
      p2 = p3 = sc_b + (size_t)pr * kScaleRow;
    } else {
      const uint8_t* wp = a.W > 0 ? swa_b + (size_t)(okw ? wr : a.W - 1) * kD : spare;
      p0 = wp + 32 * lg;
      p1 = p0 + 16;
      p2 = wp + 32 * (4 + lg);
      p3 = p2 + 16;
    }
    v0 = *reinterpret_cast<const u32x4*>(p0);
    v1 = *reinterpret_cast<const u32x4*>(p1);
    v2 = *reinterpret_cast<const u32x4*>(p2);
    v3 = *reinterpret_cast<const u32x4*>(p3);
    return g ? okg : okw;
  };

  uint8_t* my = tile[hw];
  // dequantise set u (k-steps 4 i + d from block 4 i + lg of this half),
  // accumulate the partial S^T and stage the bf16 rows for P . C
  auto score_set = [&](auto gtag, int u, const u32x4& v0, const u32x4& v1, const u32x4& v2,
                       const u32x4& v3, f32x4& s0, f32x4& s1) __attribute__((always_inline)) {
    constexpr bool kGlobal = decltype(gtag)::value;
    const int r = 16 * u + ln;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int blk = 4 * i + lg;
      u32x4 w[4];
      if (kGlobal) {
        const u32x4& c = i ? v1 : v0;
        const uint32_t sw = hw ? v2[2 + i] : v2[i];          // scale bytes of blocks 8 hw + 4 i ..
        const uint32_t scb = (sw >> (8 * lg)) & 0xFFu;
        const float scale = __uint_as_float(scb ? (scb << 23) : 0x00400000u);   // 2^(scb-127)
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          w[d][0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[d], scale, 0));
          w[d][1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[d], scale, 1));
          w[d][2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[d], scale, 2));
          w[d][3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c[d], scale, 3));
        }
      } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const u32x4& c = i ? (d < 2 ? v2 : v3) : (d < 2 ? v0 : v1);
          const uint32_t x0 = c[2 * (d & 1)], x1 = c[2 * (d & 1) + 1];
          w[d][0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x0, 1.0f, false));
          w[d][1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x0, 1.0f, true));
          w[d][2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x1, 1.0f, false));
          w[d][3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)x1, 1.0f, true));
        }
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const bf16x8 kv = __builtin_bit_cast(bf16x8, w[d]);
        if (d & 1) s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qv[4 * i + d], s1, 0, 0, 0);
        else       s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qv[4 * i + d], s0, 0, 0, 0);
        *reinterpret_cast<u32x4*>(my + tile_off(r, 64 * blk + 16 * d)) = w[d];
      }
    }
  };

  // O[j][i]: head 4 lg + i, dim 256 hw + 16 j + ln
  f32x4 O[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) O[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;   // softmax reference of head ln
  float l_run = 0.f;         // this lane's share of head ln's sum

  u32x4 a0, a1, a2, a3, b0, b1, b2, b3;
  int32_t ea = -1, eb = -1;
  bool oka = false, okb = false;
  if (n_it > 0) {
    oka = load(0, 0, entry(0, 0), a0, a1, a2, a3);
    okb = load(0, 1, entry(0, 1), b0, b1, b2, b3);
    ea = entry(1, 0);
    eb = entry(1, 1);
  }
  // transposed-read rows: key 4 lg + ln / 4 (+ 16 for set 1), dims + 4 (ln % 4)
  const int tr0 = 4 * lg + (ln >> 2), tr1 = tr0 + 16;

  // one step's scores: dequantise and score both sets (the next step's loads
  // issued as each set's registers free up), exchange the halves' partial
  // sums; x0 / x1 = full logits of keys 4 lg + e (+16), head ln, -inf when absent
  auto step_scores = [&](int it, f32x4& x0, f32x4& x1) __attribute__((always_inline)) -> float {
    f32x4 sa0 = {0.f, 0.f, 0.f, 0.f}, sa1 = sa0, sb0 = sa0, sb1 = sa0;
    const uint64_t va = __ballot(oka), vb = __ballot(okb);
    const bool global = it < cg;
    __asm__ volatile("" ::: "memory");       // this step's staging after the last step's reads
    if (global) score_set(std::true_type{}, 0, a0, a1, a2, a3, sa0, sa1);
    else        score_set(std::false_type{}, 0, a0, a1, a2, a3, sa0, sa1);
    oka = load(it + 1, 0, ea, a0, a1, a2, a3);
    ea = entry(it + 2, 0);
    if (global) score_set(std::true_type{}, 1, b0, b1, b2, b3, sb0, sb1);
    else        score_set(std::false_type{}, 1, b0, b1, b2, b3, sb0, sb1);
    okb = load(it + 1, 1, eb, b0, b1, b2, b3);
    eb = entry(it + 2, 1);
    {  // the two halves' partial sums, added in a fixed order by both waves
      float* xw = &xs[it & 1][hw][lane * 8];
      *reinterpret_cast<f32x4*>(xw) = sa0 + sa1;
      *reinterpret_cast<f32x4*>(xw + 4) = sb0 + sb1;
    }
    __syncthreads();
    const float* x0p = &xs[it & 1][0][lane * 8];
    const float* x1p = &xs[it & 1][1][lane * 8];
    x0 = *reinterpret_cast<const f32x4*>(x0p) + *reinterpret_cast<const f32x4*>(x1p);
    x1 = *reinterpret_cast<const f32x4*>(x0p + 4) + *reinterpret_cast<const f32x4*>(x1p + 4);
    float mc = -INFINITY;
    const uint32_t ba = (uint32_t)(va >> (4 * lg)), bb = (uint32_t)(vb >> (4 * lg));   // keys 4 lg ..
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x0[e] = (ba >> e) & 1u ? x0[e] : -INFINITY;
      x1[e] = (bb >> e) & 1u ? x1[e] : -INFINITY;
      mc = fmaxf(mc, fmaxf(x0[e], x1[e]));
    }
    return pf_rows_max(mc);
  };
  // one step's P . C on this half's dims, with the current reference
  auto step_pv = [&](const f32x4& x0, const f32x4& x1) __attribute__((always_inline)) {
    // absent keys are -inf: exp gives 0 (a reference of -inf only occurs while
    // every key so far is absent, and then 0 stands in for it)
    const float mr = m_run == -INFINITY ? 0.f : m_run;
    float p[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p[e] = __expf(x0[e] - mr);
      p[4 + e] = __expf(x1[e] - mr);
    }
    // A operand: keys 4 lg + e of set 0, then of set 1 (the B reads below take
    // the same keys); P = hi + lo in bf16
    u32x4 ph, pl;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      l_run += p[2 * e] + p[2 * e + 1];
      const bf16x2 hv = __builtin_convertvector((f32x2){p[2 * e], p[2 * e + 1]}, bf16x2);
      const f32x2 hf = __builtin_convertvector(hv, f32x2);
      const bf16x2 lv = __builtin_convertvector((f32x2){p[2 * e] - hf[0], p[2 * e + 1] - hf[1]}, bf16x2);
      ph[e] = __builtin_bit_cast(uint32_t, hv);
      pl[e] = __builtin_bit_cast(uint32_t, lv);
    }
    const bf16x8 ahi = __builtin_bit_cast(bf16x8, ph);
    const bf16x8 alo = __builtin_bit_cast(bf16x8, pl);
    __asm__ volatile("" ::: "memory");       // staging stores before the transposed reads
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int c = 32 * j + 8 * (ln & 3);
      const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(my + tile_off(tr0, c)));
      const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(my + tile_off(tr1, c)));
      const u32x2 c0 = __builtin_bit_cast(u32x2, r0), c1 = __builtin_bit_cast(u32x2, r1);
      const bf16x8 bv = __builtin_bit_cast(bf16x8, u32x4{c0[0], c0[1], c1[0], c1[1]});
      O[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bv, O[j], 0, 0, 0);
      O[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bv, O[j], 0, 0, 0);
    }
  };

  // Steps run in an inner loop that touches O only with matrix instructions;
  // a step whose logits exceed the reference by more than kPfLazy leaves the
  // loop, and O is rescaled before that step's P . C.
  int it = 0;
  while (it < n_it) {
    f32x4 x0, x1;
    float mc = -INFINITY;
    bool raise = false;
#pragma unroll 1
    for (; it < n_it; ++it) {
      mc = step_scores(it, x0, x1);
      raise = mc > m_run + kPfLazy;
      if (__ballot(raise) != 0) break;
      step_pv(x0, x1);
    }
    if (it >= n_it) break;
    const float m_new = raise ? mc : m_run;
    const float alpha = m_run == -INFINITY ? 0.f : __expf(m_run - m_new);
    l_run *= alpha;
    m_run = m_new;
    float al[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * lg + i, 64);
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) O[j][i] *= al[i];
    step_pv(x0, x1);
    ++it;
  }

  // per head: total sum, lse, merge with an incoming result; lane (ln, lg)
  // writes dims 256 hw + 16 j + ln of heads 4 lg + i
  const float L = pf_rows_sum(l_run);
  const float lse_h = L > 0.f ? m_run + logf(L) : -INFINITY;   // head ln
  float wself[4], win[4], lse4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float Li = __shfl(L, 4 * lg + i, 64);
    float lse = __shfl(lse_h, 4 * lg + i, 64);
    wself[i] = Li > 0.f ? 1.f / Li : 0.f;
    win[i] = 0.f;
    if (lse_in) {   // one softmax over both key sets
      const float li = lse_in[(size_t)row * kH + 4 * lg + i];
      const float mx = fmaxf(li, lse);
      if (mx != -INFINITY) {
        const float e1 = li == -INFINITY ? 0.f : __expf(li - mx);
        const float e2 = lse == -INFINITY ? 0.f : __expf(lse - mx);
        const float tot = e1 + e2;
        win[i] = e1 / tot;
        wself[i] *= e2 / tot;
        lse = mx + logf(tot);
      }
    }
    lse4[i] = lse;
  }
  // the incoming lse is read by both waves before wave 0 overwrites it
  if (lse_in) __syncthreads();
  float* orow = a.o + (size_t)row * kH * kD + kHalf * hw;
  if (lse_in) {
    // the incoming rows may be the output rows: every value this lane merges
    // is read before any is written (one round trip, not one per value)
    const float* inrow = o_in + (size_t)row * kH * kD + kHalf * hw;
    f32x4 X[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) X[j][i] = inrow[(size_t)(4 * lg + i) * kD + 16 * j + ln];
    __asm__ volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        orow[(size_t)(4 * lg + i) * kD + 16 * j + ln] = fmaf(win[i], X[j][i], O[j][i] * wself[i]);
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) orow[(size_t)(4 * lg + i) * kD + 16 * j + ln] = O[j][i] * wself[i];
  }
  if (hw == 0 && ln < 4)
    a.lse[(size_t)row * kH + 4 * lg + ln] = ln == 0 ? lse4[0] : (ln == 1 ? lse4[1] : (ln == 2 ? lse4[2] : lse4[3]));
}

}  // namespace

hipError_t launch_prefill_score(const uint8_t* key, int32_t B, int64_t M, int32_t N,
                                const uint8_t* q_idx, const float* w_idx, int32_t Q, int64_t pos0,
                                int32_t ratio, float* scores, int32_t* n_valid, const int32_t* len,
                                const PoolMap& map, hipStream_t s) {
  if (N <= 0 || N > M || Q <= 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((N + kSE - 1) / kSE), (unsigned)((Q + kSQ - 1) / kSQ), (unsigned)B);
  k_prefill_score<<<grid, dim3(kSThreads), 0, s>>>(key, M, N, q_idx, w_idx, Q, pos0, ratio, scores,
                                                   n_valid, len, map);
  return hipGetLastError();
}

hipError_t launch_prefill_attn(const AttnArgs& a, const float* o_in, const float* lse_in,
                               hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  const int32_t Cg = a.K > 0 && a.latent ? (a.K + kWK - 1) / kWK : 0;
  const int32_t Cw = a.W > 0 ? (a.W + kWK - 1) / kWK : 0;
  if (a.map.pages)
    k_prefill_attn<true><<<dim3((unsigned)a.rows), dim3(128), 0, s>>>(a, Cg, Cw, o_in, lse_in);
  else
    k_prefill_attn<false><<<dim3((unsigned)a.rows), dim3(128), 0, s>>>(a, Cg, Cw, o_in, lse_in);
  return hipGetLastError();
}

}  // namespace csa2

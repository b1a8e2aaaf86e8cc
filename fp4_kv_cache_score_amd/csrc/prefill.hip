// Chunked-prefill indexer score: the scores of many query tokens at once, as
// a matrix-core (MFMA) contraction.
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
//   next head's loads are in flight during this head's math; each of the
//   8 waves computes 32 queries x 64 entries as two 32 x 32 products with
//   v_mfma_f32_32x32x16_bf16 that share the query operand and the head
//   weights (the products are exact in fp32; at most 128 VGPRs, so two
//   work-groups give a SIMD four waves, whose stores and loads overlap the
//   others' math), and the fp32 head result is folded into the score as
//   w_h * ReLU(.).  Entries a query cannot see yet are written as -inf.
//   The scores are stored non-temporally: they stream to memory instead of
//   displacing the keys and queries the other tiles still read from the
//   caches (measured: the chunk's score and select together 30 us faster).
//   When asked, the kernel also writes the largest visible score of every
//   run of 16 entries of each query: a run is one 16-lane row of the
//   product's layout, reduced by a DPP reduce-scatter.
//   The FP8 matrix instruction is not used: measured on gfx950, its
//   accumulation error reaches ~450 x 2^-24 of the sum of |products| (about
//   2^-15 relative), against ~0.4 x 2^-24 for the bf16 instruction and for
//   sequential fp32 FMA, and the score feeds an exact Top-K.
//
// The attention of the chunk's tokens runs in attention.hip (one work-group
// per token on the matrix cores).
#include "csa2_internal.h"


namespace csa2 {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Indexer score (bf16 MFMA on exactly widened E4M3 operands)
// ---------------------------------------------------------------------------

constexpr int kSQ = 128;                 // queries per work-group tile
constexpr int kSE = 128;                 // pool entries per work-group tile
constexpr int kSThreads = 512;             // 8 waves: 2 (query halves) x 4 (entry quarters)
constexpr int kSRow = 128 + 16;          // LDS bytes per staged row (64 bf16 of one head + pad)

// Entries query t sees: the first M (the sequence's length), within the causal limit.
__device__ __forceinline__ int64_t visible(int64_t pos0, int32_t t, int32_t ratio, int64_t M) {
  if (pos0 < 0) return M;
  const int64_t v = (pos0 + t + 1) / ratio;
  return v < M ? v : M;
}

// Signed-integer image of a float that orders as the floats do (-0 just
// below +0); the map is its own inverse.
__device__ __forceinline__ int32_t ord_i32(int32_t u) { return u ^ ((u >> 31) & 0x7FFFFFFF); }

// Sixteen values per lane, the maximum of each over the 16 lanes of a DPP row
// (lanes 16 j .. 16 j + 15); lane i of the row receives value i's.  A
// reduce-scatter: at each of four exchanges a lane keeps half of its values
// and takes the partner's copies of them, the partners being the lanes across
// bit 3 (rotation by 8), across bits 0-2 (mirror in each half-row), across
// bit 1 and across bit 0 (quad swaps); the kept half follows the lane's own
// bit 3, 2, 1, 0, and the four partner sets together span the row.  15
// exchanges in place of 64.
__device__ __forceinline__ int32_t row16_max_scatter(const int32_t (&m)[16]) {
  const int l = threadIdx.x & 15;
  const bool b3 = l & 8, b2 = l & 4, b1 = l & 2, b0 = l & 1;
  int32_t y[8], z[4], w[2];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int32_t send = b3 ? m[k] : m[k + 8], keep = b3 ? m[k + 8] : m[k];
    y[k] = max(keep, __builtin_amdgcn_mov_dpp(send, 0x128, 0xF, 0xF, true));   // row_ror:8
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int32_t send = b2 ? y[k] : y[k + 4], keep = b2 ? y[k + 4] : y[k];
    z[k] = max(keep, __builtin_amdgcn_mov_dpp(send, 0x141, 0xF, 0xF, true));   // row_half_mirror
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int32_t send = b1 ? z[k] : z[k + 2], keep = b1 ? z[k + 2] : z[k];
    w[k] = max(keep, __builtin_amdgcn_mov_dpp(send, 0x4E, 0xF, 0xF, true));    // quad_perm [2,3,0,1]
  }
  const int32_t send = b0 ? w[0] : w[1], keep = b0 ? w[1] : w[0];
  return max(keep, __builtin_amdgcn_mov_dpp(send, 0xB1, 0xF, 0xF, true));      // quad_perm [1,0,3,2]
}

// Scores of entries 0 .. N-1 (N <= M; also the score row length) for every
// query; n_valid (optional, [B][Q]) receives each query's visible count.
// gmax (optional, [ceil(N / 128)][B * Q][8]): at [t][b Q + q][j] the largest
// visible score of entries 128 t + 16 j .. + 15 of query q of sequence b
// (-inf when it sees none); each work-group writes its tile's runs as whole
// 128-byte lines.
__global__ __launch_bounds__(kSThreads, 4)   // 4 waves per SIMD: two work-groups per CU
void k_prefill_score(const uint8_t* __restrict__ key, int64_t M, int32_t N,
                     const uint8_t* __restrict__ q_idx, const float* __restrict__ w_idx,
                     int32_t Q, int64_t pos0, int32_t ratio, float* __restrict__ scores,
                     int32_t* __restrict__ n_valid, const int32_t* __restrict__ len, PoolMap map,
                     float* __restrict__ gmax) {
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
  const int wq = wave & 3;                // 32-query quarter of the tile
  const int we = wave >> 2;               // 64-entry half of the tile
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
    if (gmax)
      for (int i = tid; i < kSQ * (kSE / 16); i += kSThreads) {
        const int r = i / (kSE / 16), j = i - r * (kSE / 16);
        if (q0 + r < Q)
          gmax[(((size_t)(e0 >> 7) * gridDim.z + b) * Q + q0 + r) * (kSE / 16) + j] = -INFINITY;
      }
    return;
  }

  for (int i = tid; i < kSQ * kHI; i += kSThreads) {
    const int r = i / kHI, h = i - r * kHI;
    ws[h][r] = q0 + r < Q ? w_idx[((size_t)b * Q + q0 + r) * kHI + h] : 0.f;
  }
  if (tid < kSQ) vis_s[tid] = (int32_t)visible(pos0, q0 + tid, ratio, Ms);   // one division per row

  // staging: thread -> one (row, 16-byte part) piece of each of Q and K.
  // Rows past Q or N load the last row instead (never written out), so the
  // loads are unconditional.
  static_assert(kSQ * 4 == kSThreads && kSE * 4 == kSThreads, "one piece of Q and of K per thread");
  u32x4 rq, rk;
  const uint8_t* qrow;
  const uint8_t* krow;
  {
    const int row = tid >> 2, part = tid & 3;
    const int t = q0 + row < Q ? q0 + row : Q - 1;
    const int64_t e = e0 + row < N ? e0 + row : N - 1;
    qrow = qb + (size_t)t * kKeyRow + part * 16;
    krow = key + (size_t)pool_row(map, b, e, M) * kKeyRow + part * 16;
  }
  auto load = [&](int h) {
    rq = *reinterpret_cast<const u32x4*>(qrow + h * kDI);
    rk = *reinterpret_cast<const u32x4*>(krow + h * kDI);
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
    const int row = tid >> 2, part = tid & 3;
    u32x4 lo, hi;
    widen(rq, lo, hi);
    *reinterpret_cast<u32x4*>(&qs[buf][row * kSRow + part * 32]) = lo;
    *reinterpret_cast<u32x4*>(&qs[buf][row * kSRow + part * 32 + 16]) = hi;
    widen(rk, lo, hi);
    *reinterpret_cast<u32x4*>(&ks[buf][row * kSRow + part * 32]) = lo;
    *reinterpret_cast<u32x4*>(&ks[buf][row * kSRow + part * 32 + 16]) = hi;
  };

  // acc[c]: this wave's 32 queries, entries 32 c .. of its 64
  f32x16 acc[2];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[c][v] = 0.f;

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
    bf16x8 A[4], Bv[2][4];
    {
      const uint8_t* src = &qs[buf][(32 * wq + lr) * kSRow + 64 * g];
#pragma unroll
      for (int k = 0; k < 4; ++k) A[k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(src + 16 * k));
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint8_t* src = &ks[buf][(64 * we + 32 * c + lr) * kSRow + 64 * g];
#pragma unroll
      for (int k = 0; k < 4; ++k) Bv[c][k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(src + 16 * k));
    }
    // head weights of the 16 query rows this lane holds (the same in both blocks)
    float wv[16];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 w4 = *reinterpret_cast<const float4*>(&ws[h][32 * wq + 8 * j + 4 * g]);
      wv[4 * j] = w4.x;
      wv[4 * j + 1] = w4.y;
      wv[4 * j + 2] = w4.z;
      wv[4 * j + 3] = w4.w;
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      f32x16 t = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < 4; ++k) t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A[k], Bv[c][k], t, 0, 0, 0);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        // ReLU on the bit pattern: a signed max with 0 maps negatives and -0 to +0
        const float rl = __int_as_float(max(__float_as_int(t[v]), 0));
        acc[c][v] = fmaf(rl, wv[v], acc[c][v]);
      }
    }
    if (h + 1 < kHI) store(buf ^ 1);
    load(h + 2 < kHI ? h + 2 : kHI - 1);   // past the end: a harmless reload
    __syncthreads();
  }

  // write: value v of block c is query row 8*(v/4) + 4*g + v%4 of the wave's
  // 32, entry 32 c + lr of its 64
  const int32_t ea = (int32_t)e0 + 64 * we + lr;
  const bool full = q0 + kSQ <= Q && e0 + kSE <= N && e0 + kSE <= (int64_t)vis_s[0];
  // A tile inside the chunk and the scanned entries, all of whose entries its
  // first (least-seeing) query sees: every value is stored, no test per value.
  // A store's row is the same for the whole wave but for the half-wave's
  // offset of 4 g rows, so its address is a wave-uniform row base plus one
  // per-lane 32-bit byte offset.
  if (full && N < (1 << 26)) {
    const int ws_ = __builtin_amdgcn_readfirstlane(wave);   // the wave, as a scalar
    const float* base0 = sb + (size_t)(q0 + 32 * (ws_ & 3)) * N + e0 + 64 * (ws_ >> 2);
    const uint32_t loff = ((uint32_t)(4 * g) * (uint32_t)N + (uint32_t)lr) * 4u;
#pragma unroll
    for (int v = 0; v < 16; ++v)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const float* rb = base0 + (size_t)(8 * (v >> 2) + (v & 3)) * N + 32 * c;
        __builtin_nontemporal_store(acc[c][v], (float*)((const char*)rb + loff));
      }
  } else {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int32_t ec = ea + 32 * c;
      if (ec >= N) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int tr = 32 * wq + 8 * (v >> 2) + 4 * g + (v & 3);
        if (q0 + tr >= Q) continue;
        __builtin_nontemporal_store(ec < vis_s[tr] ? acc[c][v] : -INFINITY, &sb[(size_t)(q0 + tr) * N + ec]);
      }
    }
  }
  // the run maxima after the score stores are issued (their traffic drains
  // meanwhile)
  if (gmax) {
    // the head weights are no longer read: their LDS holds the tile's run
    // maxima, [query][run] (128 x 8)
    float* gm_s = &ws[0][0];
    static_assert(kHI * kSQ == kSQ * (kSE / 16), "the run maxima fit the head weights' LDS");
    // run maxima: block c holds 32 of the wave's entries (one per lane of a
    // half-wave) for 16 query rows; each 16-lane row of the wave is one run of
    // one query row per value, and after the reduction lane i of a row holds
    // value i's
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      int32_t m[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float x = acc[c][v];
        if (!full) {
          const int tr = 32 * wq + 8 * (v >> 2) + 4 * g + (v & 3);
          x = ea + 32 * c < N && ea + 32 * c < vis_s[tr] ? x : -INFINITY;
        }
        m[v] = ord_i32(__float_as_int(x));
      }
      const int32_t o = row16_max_scatter(m);
      const int i = lane & 15;
      const int ql = 32 * wq + 8 * (i >> 2) + 4 * g + (i & 3);
      const int rl = 4 * we + 2 * c + ((lane >> 4) & 1);   // run of the tile (0 .. 7)
      gm_s[ql * (kSE / 16) + rl] = __int_as_float(ord_i32(o));
    }
    // a barrier ordering LDS only: the score stores stay in flight
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    // a query's 8 runs of the tile go out as two 16-byte pieces, the tile's
    // queries contiguous (runs past N hold -inf)
    if (tid < 2 * kSQ) {
      const int ql = tid >> 1, hh = tid & 1;
      if (q0 + ql < Q)
        *reinterpret_cast<float4*>(gmax + (((size_t)(e0 >> 7) * gridDim.z + b) * Q + q0 + ql) * (kSE / 16) + 4 * hh) =
            *reinterpret_cast<const float4*>(&gm_s[ql * (kSE / 16) + 4 * hh]);
    }
  }
}

}  // namespace

hipError_t launch_prefill_score(const uint8_t* key, int32_t B, int64_t M, int32_t N,
                                const uint8_t* q_idx, const float* w_idx, int32_t Q, int64_t pos0,
                                int32_t ratio, float* scores, int32_t* n_valid, const int32_t* len,
                                const PoolMap& map, hipStream_t s, float* gmax) {
  if (N <= 0 || N > M || Q <= 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((N + kSE - 1) / kSE), (unsigned)((Q + kSQ - 1) / kSQ), (unsigned)B);
  k_prefill_score<<<grid, dim3(kSThreads), 0, s>>>(key, M, N, q_idx, w_idx, Q, pos0, ratio, scores,
                                                   n_valid, len, map, gmax);
  return hipGetLastError();
}

}  // namespace csa2

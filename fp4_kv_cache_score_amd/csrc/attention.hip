// Sparse attention over the selected FP4 global entries and the FP8 window,
// on the matrix cores, for decode (one query token per sequence) and chunked
// prefill (many tokens).
//
// The global entries are FP4 E2M1 with one E8M0 scale per 32 elements and are
// restored to real values right before use; the sliding-window rows are FP8
// ("DeepSeek V4.1-Flash Cuts KV Cache by 437x", paragraphs on FP4 quantisation
// and sliding window attention; "DeepSeek V4.1 Flash Architecture Breakdown",
// section "How are cache precision and storage arranged?").  Keys and values
// are the same 512-wide latent row (shared K/V), and all 16 heads of a query
// token attend over the same gathered rows, so one token's attention is two
// dense contractions with the heads as rows:
//   S^T = C . q^T   (keys x heads, over the 512 dims)
//   O   = P . C     (heads x dims, over the keys)
// at 16 x 512 x 2 MACs per gathered 272-byte row: matrix-core work, not a
// memory stream.
//
// k_attn: two waves per work-group; wave h owns output dims 256 h .. 256 h +
//   255.  The row's keys (selected global entries, then its window rows) are
//   taken 32 per step.  Each lane loads 2 blocks of 32 dims of one key (this
//   wave's half), dequantises them exactly to bf16 (E2M1 x 2^(scale - 127) and
//   E4M3 have at most 4 significant bits and an exponent inside bf16's range)
//   straight into the key operand of S^T (v_mfma_f32_16x16x32_bf16, 16 keys x
//   16 heads, the dims of the contraction taken in the order the lanes hold
//   them, q permuted to match), and stages the same bf16 rows in LDS.  The two
//   waves' partial S^T (one per dim half) are exchanged through LDS and added
//   in a fixed order, so both run the same online softmax per head in fp32.
//   S^T leaves each lane with P for 4 keys of one head, which is the A-operand
//   layout of O += P . C (same instruction; P split into bf16 hi + lo parts so
//   that its rounding stays below 2^-16 relative), whose B operand (8 keys of
//   one dim per lane) comes from the staged rows with gfx950's transposing LDS
//   read (ds_read_b64_tr_b16).  The softmax reference moves only when a logit
//   exceeds it by more than 8 (natural log), outside the inner loop, so O stays
//   in the matrix accumulators.  One barrier per step.
//   Two launch shapes:
//   - one work-group per query row over all its keys (prefill: the many rows
//     fill the chip); rows of one XCD are consecutive tokens, whose window
//     rows overlap in its L2;
//   - split (decode: B rows are too few for the chip): work-group (row, s)
//     takes a contiguous run of the row's steps and writes its unnormalised
//     O, its softmax reference and its sum per head; k_attn_combine merges
//     the splits of a row in a fixed order.  A work-group mostly waits on
//     memory (its q, its entry numbers, then the gathered rows) and one
//     compute unit serves only a few tens of GB/s, so small work-groups spread
//     over every compute unit beat fewer, larger ones (measured: four key
//     streams per work-group, merged in LDS, were slower for decode and for
//     prefill).  The splits of a row land on one XCD when the row count is a
//     multiple of 8 (they read the same q).
// Either way the result equals one softmax over the union of the selected
// entries and the window rows, merged with an incoming (o, lse) when given.
#include "csa2_internal.h"

#include <type_traits>

namespace csa2 {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef i16x4 __attribute__((address_space(3))) lds_i16x4;

constexpr int kWK = kAttnStepKeys;             // keys per step (two MFMA sets of 16)
constexpr int kHalf = kD / 2;                  // output dims per wave of k_attn
constexpr int kQuarter = kD / 4;               // output dims per wave of k_attn_dec
constexpr float kLazy = 8.f;                   // softmax reference slack (natural log units)

// Max and sum over the four 16-lane rows (gfx950 permlane swaps; every lane
// combines the same two values in the same order, so all get the same result).
__device__ __forceinline__ float rows_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// A wave owns kDims consecutive output dims (part p: dims kDims p ..); each
// lane dequantises NB = kDims / 128 blocks of 32 dims of one key per set.
// Byte offset of (key row r, byte c) in a wave's staged tile of kDims bf16
// per row: 32-byte units XOR-swizzled by the row's low 3 bits, 16-byte halves
// swapped by its bit 3.  The 8 rows that half a wave's transposed read
// touches then fall on 8 different 32-byte bank groups, and the 16 rows of a
// staging store on 16 different 16-byte ones (rows are a multiple of 256
// bytes long, so the bank of a byte depends only on its place in the row).
template <int kDims>
__device__ __forceinline__ int tile_off(int r, int c) {
  return r * (2 * kDims) + ((((c >> 5) ^ (r & 7)) << 5) | ((c & 31) ^ (((r >> 3) & 1) << 4)));
}

// q (this wave's part) as the B operand of S^T = C . q^T: lane (head ln,
// group lg) holds, for k-step s, dims kDims p + 32 (4 (s / 4) + lg) + 8 (s % 4)
// .. +7, the order in which score_set holds the keys' dims.
template <int kDims>
__device__ __forceinline__ void load_q(const uint16_t* q, int row, int p, int ln, int lg,
                                       bf16x8 (&qv)[kDims / 32]) {
  const uint16_t* qr = q + ((size_t)row * kH + ln) * kD + kDims * p;
#pragma unroll
  for (int s = 0; s < kDims / 32; ++s)
    qv[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                           qr + 32 * (4 * (s >> 2) + lg) + 8 * (s & 3)));
}

// Set u of a step (keys 16 u .. 16 u + 15; this lane: key 16 u + ln, blocks
// 4 i + lg, i < NB, of this wave's part): dequantise exactly to bf16, add the
// partial S^T (s0: k-steps of even d, s1: odd d) and stage the bf16 rows in
// this wave's tile for P . C.  Global keys: c0 (, c1) = the 16 E2M1 bytes of
// the block(s), c2 = the key's 16 scale bytes (words NB p .. NB p + NB - 1:
// this part's).  Window rows: (c0, c1) (, (c2, c3)) = the 32 E4M3 bytes of
// the block(s).
template <bool kGlobal, int kDims>
__device__ __forceinline__ void score_set(uint8_t* my, const bf16x8 (&qv)[kDims / 32], int p,
                                          int ln, int lg, int u, const u32x4& c0,
                                          const u32x4& c1, const u32x4& c2, const u32x4& c3,
                                          f32x4& s0, f32x4& s1) {
  constexpr int NB = kDims / 128;
  const int r = 16 * u + ln;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int blk = 4 * i + lg;
    u32x4 w[4];
    if (kGlobal) {
      const u32x4& c = i ? c1 : c0;
      const uint32_t sw = c2[NB * p + i];                    // scale bytes of blocks 4 (NB p + i) ..
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
        const u32x4& c = i ? (d < 2 ? c2 : c3) : (d < 2 ? c0 : c1);
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
      *reinterpret_cast<u32x4*>(my + tile_off<kDims>(r, 64 * blk + 16 * d)) = w[d];
    }
  }
}

// The NW parts' partial S^T (sa: set 0, sb: set 1) added in a fixed order by
// every wave through xsb (this step's parity buffer; one barrier).  x0 / x1 =
// logits of keys 4 lg + e (+16), head ln, -inf where the ballots va / vb (bit
// = key) say absent; returns the step's largest logit of head ln.
template <int NW>
__device__ __forceinline__ float exchange_logits(float (*xsb)[64 * 8], int p, int lane, int lg,
                                                 const f32x4& sa, const f32x4& sb, uint64_t va,
                                                 uint64_t vb, f32x4& x0, f32x4& x1) {
  float* xw = &xsb[p][lane * 8];
  *reinterpret_cast<f32x4*>(xw) = sa;
  *reinterpret_cast<f32x4*>(xw + 4) = sb;
  __syncthreads();
  x0 = *reinterpret_cast<const f32x4*>(&xsb[0][lane * 8]);
  x1 = *reinterpret_cast<const f32x4*>(&xsb[0][lane * 8 + 4]);
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    x0 += *reinterpret_cast<const f32x4*>(&xsb[w][lane * 8]);
    x1 += *reinterpret_cast<const f32x4*>(&xsb[w][lane * 8 + 4]);
  }
  float mc = -INFINITY;
  const uint32_t ba = (uint32_t)(va >> (4 * lg)), bb = (uint32_t)(vb >> (4 * lg));   // keys 4 lg ..
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x0[e] = (ba >> e) & 1u ? x0[e] : -INFINITY;
    x1[e] = (bb >> e) & 1u ? x1[e] : -INFINITY;
    mc = fmaxf(mc, fmaxf(x0[e], x1[e]));
  }
  return rows_max(mc);
}

// One step's P . C on this wave's part of the dims, with the current
// reference (absent keys are -inf: exp gives 0; a reference of -inf only
// occurs while every key so far is absent, and then 0 stands in for it).
// O[j][i]: head 4 lg + i, dim kDims p + 16 j + ln.
template <int kDims>
__device__ __forceinline__ void pv_step(const uint8_t* my, int tr0, int tr1, int ln,
                                        const f32x4& x0, const f32x4& x1, float m_run,
                                        float& l_run, f32x4 (&O)[kDims / 16]) {
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
  for (int j = 0; j < kDims / 16; ++j) {
    const int c = 32 * j + 8 * (ln & 3);
    const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(my + tile_off<kDims>(tr0, c)));
    const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(my + tile_off<kDims>(tr1, c)));
    const u32x2 c0 = __builtin_bit_cast(u32x2, r0), c1 = __builtin_bit_cast(u32x2, r1);
    const bf16x8 bv = __builtin_bit_cast(bf16x8, u32x4{c0[0], c0[1], c1[0], c1[1]});
    O[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bv, O[j], 0, 0, 0);
    O[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bv, O[j], 0, 0, 0);
  }
}

// Move head ln's softmax reference to the step's largest logit mc (when
// `raise`) and rescale O and this lane's sum to it.  The kernels run their
// steps in an inner loop that touches O only with matrix instructions; a
// step whose logits exceed the reference by more than kLazy leaves that loop
// and comes here before its P . C.
template <int NJ>
__device__ __forceinline__ void raise_reference(bool raise, float mc, int lg, f32x4 (&O)[NJ],
                                                float& m_run, float& l_run) {
  const float m_new = raise ? mc : m_run;
  const float alpha = m_run == -INFINITY ? 0.f : __expf(m_run - m_new);
  l_run *= alpha;
  m_run = m_new;
  float al[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * lg + i, 64);
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) O[j][i] *= al[i];
}

// A split's partial of a row: O unnormalised (relative to the reference of
// its head), the reference and the sum per head.
template <int kDims>
__device__ __forceinline__ void store_partial(const AttnArgs& a, int row, int split, int splits,
                                              int p, int ln, int lg,
                                              const f32x4 (&O)[kDims / 16], float m_run,
                                              float L) {
  const size_t ps = (size_t)row * splits + split;
  float* op = a.opart + ps * kH * kD + kDims * p;
#pragma unroll
  for (int j = 0; j < kDims / 16; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) op[(size_t)(4 * lg + i) * kD + 16 * j + ln] = O[j][i];
  if (p == 0 && lg == 0) {
    a.ml[(ps * kH + ln) * 2] = m_run;
    a.ml[(ps * kH + ln) * 2 + 1] = L;
  }
}

// A row's result: o normalised and lse per head, merged with an incoming
// (o_in, lse_in) into one softmax over both key sets when given (o_in may be
// a.o itself).  Called by every thread of the work-group.
template <int kDims>
__device__ __forceinline__ void store_final(const AttnArgs& a, int row, int p, int ln, int lg,
                                            const f32x4 (&O)[kDims / 16], float m_run, float L,
                                            const float* o_in, const float* lse_in) {
  // per head: lse, merge with an incoming result; lane (ln, lg) writes dims
  // kDims p + 16 j + ln of heads 4 lg + i
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
  // the incoming lse is read by every wave before wave 0 overwrites it
  if (lse_in) __syncthreads();
  float* orow = a.o + (size_t)row * kH * kD + kDims * p;
  if (lse_in) {
    // the incoming rows may be the output rows: every value this lane merges
    // is read before any is written (one round trip, not one per value)
    const float* inrow = o_in + (size_t)row * kH * kD + kDims * p;
    f32x4 X[kDims / 16];
#pragma unroll
    for (int j = 0; j < kDims / 16; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) X[j][i] = inrow[(size_t)(4 * lg + i) * kD + 16 * j + ln];
    __asm__ volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < kDims / 16; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        orow[(size_t)(4 * lg + i) * kD + 16 * j + ln] = fmaf(win[i], X[j][i], O[j][i] * wself[i]);
  } else {
#pragma unroll
    for (int j = 0; j < kDims / 16; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) orow[(size_t)(4 * lg + i) * kD + 16 * j + ln] = O[j][i] * wself[i];
  }
  if (p == 0 && ln < 4)
    a.lse[(size_t)row * kH + 4 * lg + ln] = ln == 0 ? lse4[0] : (ln == 1 ? lse4[1] : (ln == 2 ? lse4[2] : lse4[3]));
}

// One work-group per query row over all its keys (many rows: prefill, or a
// decode batch large enough to fill the chip).  Each step's rows are loaded
// into registers one step ahead.
template <bool kPaged>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_attn(AttnArgs a, int32_t Cg, int32_t Cw) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[2][kWK * 2 * kHalf];   // 32 KiB
  __shared__ __attribute__((aligned(16))) float xs[2][2][64 * 8];             // partial S, by step parity

  // rows of one XCD are consecutive tokens (their window rows overlap in L2)
  const int R = a.rows;
  const int q8 = R >> 3, r8 = R & 7, xcd = blockIdx.x & 7, kk = blockIdx.x >> 3;
  const int row = xcd * q8 + (xcd < r8 ? xcd : r8) + kk;
  const int b = row / a.Q;
  const int t = row - b * a.Q;
  const int hw = threadIdx.x >> 6;           // this wave's half of the dims
  const int lane = threadIdx.x & 63;
  const int ln = lane & 15;
  const int lg = lane >> 4;
  const int64_t wgap = a.pos0 >= 0 ? (int64_t)(a.W - 1) - (a.pos0 + t) : 0;
  const int32_t wfirst = wgap > 0 ? (int32_t)wgap : 0;

  bf16x8 qv[8];
  load_q<kHalf>(a.q, row, hw, ln, lg, qv);
  const int32_t* irow = a.idx ? a.idx + (size_t)row * a.K : nullptr;
  // the last position holding an entry (-1 entries select nothing); the
  // entry numbers are read 512 at a time, all loads in flight together
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
  const int st_end = cg + (Cw > ws0 ? Cw - ws0 : 0);

  const uint8_t* lat_b = a.latent ? a.latent + 128 * hw : nullptr;   // indexed by pool row
  const uint8_t* sc_b = a.scale;
  const uint8_t* swa_b = a.swa ? a.swa + ((size_t)b * a.swa_rows + t) * kD + kHalf * hw : nullptr;
  // a readable stand-in for loads past the last step (this row's q: 16 KiB)
  const uint8_t* spare = reinterpret_cast<const uint8_t*>(a.q + (size_t)row * kH * kD);
  const int kmax = a.K > 0 ? a.K - 1 : 0;

  // entry number for step `st` (an unconditional load at a clamped position)
  const int32_t* irow_s = irow ? irow : reinterpret_cast<const int32_t*>(spare);
  auto entry = [&](int st, int u) __attribute__((always_inline)) -> int32_t {
    return irow_s[min(st * kWK + 16 * u + ln, kmax)];
  };
  // step `st`, set u: key 16 u + ln; lane group lg loads blocks lg and 4 + lg
  // of this half.  Global: v0, v1 = 16 E2M1 bytes each, v2 = v3 = the entry's
  // scale bytes.  Window: (v0, v1), (v2, v3) = 32 E4M3 bytes each.  All four
  // loads are issued unconditionally from selected, valid addresses.
  auto load = [&](int st, int u, int32_t e, u32x4& v0, u32x4& v1, u32x4& v2, u32x4& v3)
      __attribute__((always_inline)) -> bool {
    const bool g = st < cg;
    const int kpos = st * kWK + 16 * u + ln;
    const bool okg = kpos < a.K && e >= 0;
    const int wr = (st - cg + ws0) * kWK + 16 * u + ln;
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
  f32x4 O[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) O[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;   // softmax reference of head ln
  float l_run = 0.f;         // this lane's share of head ln's sum

  u32x4 a0, a1, a2, a3, b0, b1, b2, b3;
  int32_t ea = -1, eb = -1;
  bool oka = false, okb = false;
  if (st_end > 0) {
    oka = load(0, 0, entry(0, 0), a0, a1, a2, a3);
    okb = load(0, 1, entry(0, 1), b0, b1, b2, b3);
    ea = entry(1, 0);
    eb = entry(1, 1);
  }
  // one step's logits: dequantise and score both sets (the next step's loads
  // issued as each set's registers free up), then exchange the halves' sums
  auto step_scores = [&](int st, f32x4& x0, f32x4& x1) __attribute__((always_inline)) -> float {
    f32x4 sa0 = {0.f, 0.f, 0.f, 0.f}, sa1 = sa0, sb0 = sa0, sb1 = sa0;
    const uint64_t va = __ballot(oka), vb = __ballot(okb);
    const bool global = st < cg;
    __asm__ volatile("" ::: "memory");       // this step's staging after the last step's reads
    if (global) score_set<true, kHalf>(my, qv, hw, ln, lg, 0, a0, a1, a2, a3, sa0, sa1);
    else        score_set<false, kHalf>(my, qv, hw, ln, lg, 0, a0, a1, a2, a3, sa0, sa1);
    oka = load(st + 1, 0, ea, a0, a1, a2, a3);
    ea = entry(st + 2, 0);
    if (global) score_set<true, kHalf>(my, qv, hw, ln, lg, 1, b0, b1, b2, b3, sb0, sb1);
    else        score_set<false, kHalf>(my, qv, hw, ln, lg, 1, b0, b1, b2, b3, sb0, sb1);
    okb = load(st + 1, 1, eb, b0, b1, b2, b3);
    eb = entry(st + 2, 1);
    return exchange_logits<2>(xs[st & 1], hw, lane, lg, sa0 + sa1, sb0 + sb1, va, vb, x0, x1);
  };
  // transposed-read rows: key 4 lg + ln / 4 (+ 16 for set 1), dims + 4 (ln % 4)
  const int tr0 = 4 * lg + (ln >> 2), tr1 = tr0 + 16;
  for (int it = 0; it < st_end;) {
    f32x4 x0, x1;
    float mc = -INFINITY;
    bool raise = false;
#pragma unroll 1
    for (; it < st_end; ++it) {
      mc = step_scores(it, x0, x1);
      raise = mc > m_run + kLazy;
      if (__ballot(raise) != 0) break;
      pv_step<kHalf>(my, tr0, tr1, ln, x0, x1, m_run, l_run, O);
    }
    if (it >= st_end) break;
    raise_reference<16>(raise, mc, lg, O, m_run, l_run);
    pv_step<kHalf>(my, tr0, tr1, ln, x0, x1, m_run, l_run, O);
    ++it;
  }
  store_final<kHalf>(a, row, hw, ln, lg, O, m_run, rows_sum(l_run), a.o_in, a.lse_in);
}

// Decode (one query row per sequence, B rows too few for the chip): grid
// (rows, splits); work-group (row, s) runs steps s * cps .. s * cps + cps - 1
// of its row (global steps first, Cg of them, then Cw window steps).  A
// decode launch has fewer work-groups than the chip has compute units, so a
// work-group's steps run back to back on one compute unit: four waves, one
// per SIMD, each owning a quarter of the dims (its own dequantisation, S^T
// partial and P . C; the partial logits summed through LDS), which halves
// the serial chain of matrix instructions and LDS round trips per step
// against two waves on halves.  Each wave first issues the transfers of up
// to kDecDepth steps at once, direct global-to-LDS, into a ring of per-step
// slots (its own quarter of every row), so a work-group waits on memory once
// per kDecDepth steps (entry numbers, then rows) rather than once per step.
// Slot layout, 16-byte chunks XOR-swizzled so that the 16 rows a set reads
// fall on different banks: global step, chunk c of key k (the quarter's 64
// E2M1 bytes) at 64 k + 16 (c ^ (k / 4 % 4)) and the key's 16 scale bytes at
// kScaleOff + 16 k; window step, chunk c of row r (the quarter's 128 E4M3
// bytes) at 128 r + 16 (c ^ (r % 8)).  kSplit: a partial per work-group,
// merged by k_attn_combine; otherwise one work-group per row writes o and
// lse.
constexpr int kDecWaves = kD / kQuarter;       // 4
constexpr int kDecDepth = 5;                   // steps in flight per wave
constexpr int kSlot = kWK * kQuarter;          // 4 KiB: a window step of one wave
constexpr int kScaleOff = kWK * kQuarter / 2;  // a global step's scales (after 32 x 64 bytes)

__device__ __forceinline__ void dma16(const void* src, uint8_t* lds_dst) {
  // 16 bytes per lane; lane l's bytes land at lds_dst + 16 l (lds_dst uniform)
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_dst, 16, 0, 0);
}

template <bool kPaged, bool kSplit>
__global__ __launch_bounds__(64 * kDecWaves) __attribute__((amdgpu_waves_per_eu(1, 2)))
void k_attn_dec(AttnArgs a, int32_t Cg, int32_t Cw, int32_t cps) {
  __shared__ __attribute__((aligned(16))) uint8_t ring[kDecWaves][kDecDepth][kSlot];   // 80 KiB
  __shared__ __attribute__((aligned(16))) uint8_t tile[kDecWaves][kWK * 2 * kQuarter]; // 32 KiB
  __shared__ __attribute__((aligned(16))) float xs[2][kDecWaves][64 * 8];             // 16 KiB
  __shared__ int32_t ents[kDecWaves][kDecDepth * kWK];

  const int row = blockIdx.x, split = blockIdx.y;
  const int b = row;                         // one query row per sequence
  const int p = threadIdx.x >> 6;            // this wave's quarter of the dims
  const int lane = threadIdx.x & 63;
  const int ln = lane & 15;
  const int lg = lane >> 4;
  const int st0 = split * cps;
  const int st_end = min(st0 + cps, Cg + Cw);

  bf16x8 qv[kQuarter / 32];
  load_q<kQuarter>(a.q, row, p, ln, lg, qv);
  const int32_t* irow = a.idx ? a.idx + (size_t)row * a.K : nullptr;
  const uint8_t* lat_b = a.latent ? a.latent + (kQuarter / 2) * p : nullptr;
  const uint8_t* swa_b = a.swa ? a.swa + (size_t)b * a.swa_rows * kD + kQuarter * p : nullptr;
  uint8_t* my = tile[p];
  uint8_t (*rg)[kSlot] = ring[p];
  int32_t* en = ents[p];

  f32x4 O[kQuarter / 16];
#pragma unroll
  for (int j = 0; j < kQuarter / 16; ++j) O[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;
  float l_run = 0.f;
  // transposed-read rows: key 4 lg + ln / 4 (+ 16 for set 1), dims + 4 (ln % 4)
  const int tr0 = 4 * lg + (ln >> 2), tr1 = tr0 + 16;

  for (int bs = st0; bs < st_end; bs += kDecDepth) {
    const int nb = min(kDecDepth, st_end - bs);
    const int ng = max(0, min(bs + nb, Cg) - bs);   // global steps of the batch
    // the batch's entry numbers (-1 past K), this wave's copy
    int32_t ev[(kDecDepth * kWK + 63) / 64];
#pragma unroll
    for (int m = 0; m < (kDecDepth * kWK + 63) / 64; ++m) {
      const int t = lane + 64 * m;
      const int kpos = bs * kWK + t;
      ev[m] = t < ng * kWK && kpos < a.K ? irow[kpos] : -1;
    }
#pragma unroll
    for (int m = 0; m < (kDecDepth * kWK + 63) / 64; ++m)
      if (lane + 64 * m < kDecDepth * kWK) en[lane + 64 * m] = ev[m];
    for (int s = 0; s < ng; ++s) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int k = 16 * j + (lane >> 2);
        const int c = (lane & 3) ^ ((k >> 2) & 3);
        const int32_t e = en[s * kWK + k];
        const int32_t ec = e >= 0 ? e : 0;                     // entry 0 exists
        const int64_t pr = kPaged ? pool_row(a.map, b, ec, a.M) : (int64_t)b * a.M + ec;
        dma16(lat_b + (size_t)pr * kLatRow + 16 * c, &rg[s][1024 * j]);
      }
      const int k = lane & 31;
      const int32_t e = en[s * kWK + k];
      const int32_t ec = e >= 0 ? e : 0;
      const int64_t pr = kPaged ? pool_row(a.map, b, ec, a.M) : (int64_t)b * a.M + ec;
      dma16(a.scale + (size_t)pr * kScaleRow, &rg[s][kScaleOff]);
    }
    // the window rows (issued after the entry numbers were waited for: a
    // wait for a load counts every transfer issued before it)
    for (int s = ng; s < nb; ++s) {
      const int wr0 = (bs + s - Cg) * kWK;
#pragma unroll
      for (int j = 0; j < kSlot / 1024; ++j) {
        const int r = 8 * j + (lane >> 3);
        const int c = (lane & 7) ^ (r & 7);
        const int wr = min(wr0 + r, a.W - 1);
        dma16(swa_b + (size_t)wr * kD + 16 * c, &rg[s][1024 * j]);
      }
    }
    // every transfer of the batch (and q) has landed
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)

    auto step_scores = [&](int it, f32x4& x0, f32x4& x1) __attribute__((always_inline)) -> float {
      const uint8_t* sl = rg[it - bs];
      f32x4 sa0 = {0.f, 0.f, 0.f, 0.f}, sa1 = sa0, sb0 = sa0, sb1 = sa0;
      bool oka, okb;
      __asm__ volatile("" ::: "memory");     // this step's staging after the last step's reads
      if (it < Cg) {
        const int s = it - bs;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int k = 16 * u + ln;
          const u32x4 c0 = *reinterpret_cast<const u32x4*>(sl + 64 * k + ((lg ^ ((k >> 2) & 3)) << 4));
          const u32x4 sc = *reinterpret_cast<const u32x4*>(sl + kScaleOff + 16 * k);
          const bool ok = en[s * kWK + k] >= 0;
          if (u == 0) {
            oka = ok;
            score_set<true, kQuarter>(my, qv, p, ln, lg, 0, c0, c0, sc, sc, sa0, sa1);
          } else {
            okb = ok;
            score_set<true, kQuarter>(my, qv, p, ln, lg, 1, c0, c0, sc, sc, sb0, sb1);
          }
        }
      } else {
        const int wr0 = (it - Cg) * kWK;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int r = 16 * u + ln, x = r & 7;
          const uint8_t* rp = sl + 128 * r;
          const u32x4 c0 = *reinterpret_cast<const u32x4*>(rp + (((2 * lg) ^ x) << 4));
          const u32x4 c1 = *reinterpret_cast<const u32x4*>(rp + (((2 * lg + 1) ^ x) << 4));
          const bool ok = wr0 + r < a.W;
          if (u == 0) {
            oka = ok;
            score_set<false, kQuarter>(my, qv, p, ln, lg, 0, c0, c1, c0, c1, sa0, sa1);
          } else {
            okb = ok;
            score_set<false, kQuarter>(my, qv, p, ln, lg, 1, c0, c1, c0, c1, sb0, sb1);
          }
        }
      }
      return exchange_logits<kDecWaves>(xs[it & 1], p, lane, lg, sa0 + sa1, sb0 + sb1,
                                        __ballot(oka), __ballot(okb), x0, x1);
    };
    for (int it = bs; it < bs + nb;) {
      f32x4 x0, x1;
      float mc = -INFINITY;
      bool raise = false;
#pragma unroll 1
      for (; it < bs + nb; ++it) {
        mc = step_scores(it, x0, x1);
        raise = mc > m_run + kLazy;
        if (__ballot(raise) != 0) break;
        pv_step<kQuarter>(my, tr0, tr1, ln, x0, x1, m_run, l_run, O);
      }
      if (it >= bs + nb) break;
      raise_reference<kQuarter / 16>(raise, mc, lg, O, m_run, l_run);
      pv_step<kQuarter>(my, tr0, tr1, ln, x0, x1, m_run, l_run, O);
      ++it;
    }
  }

  const float L = rows_sum(l_run);   // head ln's sum (relative to m_run)
  if (kSplit) store_partial<kQuarter>(a, row, split, gridDim.y, p, ln, lg, O, m_run, L);
  else        store_final<kQuarter>(a, row, p, ln, lg, O, m_run, L, a.o_in, a.lse_in);
}

// One work-group (128 lanes x 4 dims) per (query row, head), the row index
// fastest: with a row count that is a multiple of 8, a row's merges then run
// on the XCD whose work-groups wrote its partials, and read them from that
// L2 (measured: 0.5 us less per layer than head-first).  The partial
// rows of up to kCombBatch splits are loaded together with every split's
// (reference, sum) pair, so that the merge waits on one round trip to memory;
// the weights are formed in LDS by the first wave, and the rows are summed in
// split order, then the incoming result.
constexpr int kCombThreads = 128;
constexpr int kCombBatch = 8;            // partial rows in flight per lane

__global__ __launch_bounds__(kCombThreads)
void k_attn_combine(const float* __restrict__ opart, const float* __restrict__ ml,
                    int32_t S, const float* o_in, const float* lse_in, float* o,
                    float* lse) {
  __shared__ float wgt_s[kAttnMaxSplits + 1];
  __shared__ float L_s;
  const int row = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int d0 = tid * 4;
  const float* src = opart + ((size_t)row * S * kH + h) * kD + d0;
  float4 x[kCombBatch];
#pragma unroll
  for (int u = 0; u < kCombBatch; ++u)
    if (u < S) x[u] = *reinterpret_cast<const float4*>(src + (size_t)u * kH * kD);
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
    if (tid <= S && tid <= kAttnMaxSplits) wgt_s[tid] = w;
    if (tid == 0) L_s = Lsum > 0.f ? Lsum : 0.f;
    if (tid == 0) lse[(size_t)row * kH + h] = Lsum > 0.f ? mx + logf(Lsum) : -INFINITY;
  }
  __syncthreads();
  const float L = L_s;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int u = 0; u < kCombBatch; ++u) {
    if (u < S) {
      const float w = wgt_s[u];
      acc.x = fmaf(w, x[u].x, acc.x);
      acc.y = fmaf(w, x[u].y, acc.y);
      acc.z = fmaf(w, x[u].z, acc.z);
      acc.w = fmaf(w, x[u].w, acc.w);
    }
  }
  for (int s = kCombBatch; s < S; ++s) {
    const float4 y = *reinterpret_cast<const float4*>(src + (size_t)s * kH * kD);
    const float w = wgt_s[s];
    acc.x = fmaf(w, y.x, acc.x);
    acc.y = fmaf(w, y.y, acc.y);
    acc.z = fmaf(w, y.z, acc.z);
    acc.w = fmaf(w, y.w, acc.w);
  }
  if (lse_in) {
    const float w = wgt_s[S];
    if (w > 0.f) {
      const float4 y = *reinterpret_cast<const float4*>(o_in + ((size_t)row * kH + h) * kD + d0);
      acc.x = fmaf(w, y.x, acc.x);
      acc.y = fmaf(w, y.y, acc.y);
      acc.z = fmaf(w, y.z, acc.z);
      acc.w = fmaf(w, y.w, acc.w);
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  *reinterpret_cast<float4*>(o + ((size_t)row * kH + h) * kD + d0) =
      make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
}

}  // namespace

int32_t attn_steps(int32_t K, int32_t W) {
  return (K > 0 ? (K + kWK - 1) / kWK : 0) + (W > 0 ? (W + kWK - 1) / kWK : 0);
}

int32_t attn_max_splits(int64_t rows, int32_t steps) {
  // more splits than it takes to give every compute unit a few work-groups
  // only add partial traffic
  int64_t s = (kAttnFillGroups + rows - 1) / (rows > 0 ? rows : 1);
  if (s > steps) s = steps;
  if (s > kAttnMaxSplits) s = kAttnMaxSplits;
  return (int32_t)(s > 0 ? s : 1);
}

AttnPlan attn_plan(int64_t rows, int32_t steps) {
  // Many rows fill the chip with one work-group per row (k_attn).  Fewer rows
  // (decode) cut each row into S runs of cps steps, one k_attn_dec
  // work-group each (one per compute unit: its LDS), then merge the partials.
  // A work-group waits for its entry numbers, then for its gathered rows
  // (once per kDecDepth steps), then computes its steps (about 1.3 us each,
  // a chain of LDS round trips, matrix instructions and a barrier); each
  // split adds a 32 KiB partial to write and merge.  The estimate
  // (microseconds, fitted to timestamps taken inside decode launches) picks S.
  if (steps <= 0 || rows >= kAttnSplitRows) return AttnPlan{1, 0};
  const int32_t smax = attn_max_splits(rows, steps);
  AttnPlan best{1, steps};
  double best_cost = 1e30;
  for (int32_t S = 1; S <= smax; ++S) {
    const int32_t cps = (steps + S - 1) / S;
    if ((S - 1) * cps >= steps) continue;          // every split holds a step
    const double groups = (double)(rows * S);
    const double rounds = (double)(((int64_t)groups + 255) / 256);
    const double batches = (double)((cps + kDecDepth - 1) / kDecDepth);
    const double cost = rounds * (2.0 + 0.8 * batches + 1.35 * cps) +
                        (S > 1 ? 3.0 + groups * 0.004 : 0.0);
    if (cost < best_cost - 1e-9) {
      best_cost = cost;
      best = AttnPlan{S, cps};
    }
  }
  return best;
}

hipError_t launch_attn(const AttnArgs& a, const AttnPlan& plan, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  const int32_t Cg = a.K > 0 && a.latent ? (a.K + kWK - 1) / kWK : 0;
  const int32_t Cw = a.W > 0 ? (a.W + kWK - 1) / kWK : 0;
  const int32_t S = plan.splits;
  if (plan.cps > 0) {
    // decode: whole steps per split, one query row per sequence
    if (S < 1 || S > kAttnMaxSplits || (Cg + Cw + plan.cps - 1) / plan.cps != S ||
        (S - 1) * plan.cps >= Cg + Cw || a.Q != 1 || a.pos0 >= 0 ||
        (S > 1 && (!a.opart || !a.ml)))
      return hipErrorInvalidValue;
    const dim3 grid((unsigned)a.rows, (unsigned)S);
    if (S > 1) {
      if (a.map.pages) k_attn_dec<true, true><<<grid, dim3(64 * kDecWaves), 0, s>>>(a, Cg, Cw, plan.cps);
      else             k_attn_dec<false, true><<<grid, dim3(64 * kDecWaves), 0, s>>>(a, Cg, Cw, plan.cps);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      k_attn_combine<<<dim3((unsigned)a.rows, (unsigned)kH), dim3(kCombThreads), 0, s>>>(
          a.opart, a.ml, S, a.o_in, a.lse_in, a.o, a.lse);
    } else {
      if (a.map.pages) k_attn_dec<true, false><<<grid, dim3(64 * kDecWaves), 0, s>>>(a, Cg, Cw, plan.cps);
      else             k_attn_dec<false, false><<<grid, dim3(64 * kDecWaves), 0, s>>>(a, Cg, Cw, plan.cps);
    }
    return hipGetLastError();
  }
  if (S != 1) return hipErrorInvalidValue;
  if (a.map.pages)
    k_attn<true><<<dim3((unsigned)a.rows), dim3(128), 0, s>>>(a, Cg, Cw);
  else
    k_attn<false><<<dim3((unsigned)a.rows), dim3(128), 0, s>>>(a, Cg, Cw);
  return hipGetLastError();
}

}  // namespace csa2

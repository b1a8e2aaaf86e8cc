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
// k_attn_partial: one work-group of 8 waves per (query row, split).  A row's
// keys are cut into chunks of 32 (the selected global entries first, then the
// window rows) and a split is a run of consecutive chunks.  Wave w takes the
// 4 heads 4(w%4).. and key stream w/4: keys 16(w/4)..16(w/4)+15 of every
// chunk, with its own online-softmax state; the two streams are merged at the
// end.  Per chunk (double-buffered, one barrier per chunk), after computing
// on the current buffer the next chunk is staged into the other one:
//   stage   the chunk's codes (loaded one compute phase ahead) are
//           restored and written to LDS twice: as bf16 rows of dim pairs
//           with the true scale (for q . c; FP4 with gfx950's scaled
//           FP4->bf16 convert, FP8 with the FP8->bf16 convert, both exact),
//           and as fp16 key pairs per dim (for P x V): an FP4 value enters
//           as E2M1 x 2^(sc - ref), ref being the largest scale code of its
//           32-dim block among the split's entries staged so far (a running
//           maximum, kept in LDS per staged chunk), exact while
//           sc >= ref - 23; an FP8 value is exact;
//   logits  q sits in registers (each lane: 4 heads x 32 dims); a lane forms
//           4 heads x 4 keys over its 32 dims with v_dot2_f32_bf16 (exact
//           bf16 products, fp32 sums), and the 16 lanes of a row sum their
//           parts with 15 DPP adds: heads and keys are laid out in a
//           lane-rotated order so that every step adds the same registers;
//   softmax per head over the stream's 16 keys (fp32): running max, rescale
//           factor, p = exp(z - max), running sum;
//   P x V   each lane owns 8 dims of the 4 heads; p is rounded to fp16
//           (relative error at most 2^-11) and every v_dot2_f32_f16 adds two
//           keys of one dim, so the key pairs are used as staged.  The sums
//           over global keys are in units of 2^(ref - 127) per block: they
//           are rescaled by 2^(old - new) when a chunk raises ref, and
//           brought to units of 1 before the first window chunk or at the
//           end (exact powers of two).
// With one split per row the work-group merges an incoming (o, lse) when
// given, normalises and writes o and lse; otherwise it writes (unnormalised
// o, max, sum) partials and k_attn_combine, launched right after it, merges
// them (and the incoming result) by log-sum-exp weights in a fixed order, so
// that the result equals one softmax over the union of the key sets.  All
// arithmetic runs on the VALU with fp32 accumulation; decode keeps the matrix
// cores for the multi-query prefill contraction.
#include "csa2_internal.h"

namespace csa2 {
namespace {

constexpr int kThreads = 512;                   // 8 waves: 4 head groups x 2 key streams
constexpr int KS = kKeysPerSplit;               // 32 keys per chunk, 16 per stream
constexpr int kRowU = kD / 2;                   // staged key row: 256 u32 of dim pairs
constexpr int kPairU = kD + 4;                  // staged key pair: 512 u32 (+ pad) of key pairs
constexpr int kRowBufU = KS * kRowU;            // 32 KiB
constexpr int kPairBufU = (KS / 2) * kPairU;    // 32.25 KiB
constexpr int kMaxChunksPerSplit = 32;          // entry numbers staged per work-group: 1024
constexpr int kGroupsPerRound = 256;            // work-groups that run at once, one per compute unit

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2, u); }

__device__ __forceinline__ float fdot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(a), as_bf16x2(b), c, false);
}

// fp16 pair dot product with fp32 accumulation (v_dot2_f32_f16)
__device__ __forceinline__ float hdot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
}

// Value of x in the lane named by the DPP control word (within a row of 16).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppXor7 = 0x141;       // row_half_mirror
constexpr int kDppXor15 = 0x140;      // row_mirror
constexpr int kDppRor4 = 0x124;       // row_ror:4 (lane i reads lane i - 4 of its row)
constexpr int kDppRor8 = 0x128;       // row_ror:8
constexpr int kDppRor12 = 0x12C;      // row_ror:12 (lane i reads lane i + 4 of its row)
constexpr float kLazyMax = 8.f;       // softmax reference slack (natural log units)

// Max and sum over the four rows of 16 lanes: gfx950's permlane swaps
// exchange rows 0<->1, 2<->3 and halves 0-31<->32-63 in a VALU operation
// (both operands the same value); each lane combines the same two values
// in the same order, so every lane gets the same result.
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

// Staging unit of a thread: key pair kp (keys 2kp, 2kp+1 of the chunk) and a
// 16-dim segment seg.  The bit assignment keeps both LDS layouts' stores to
// at most two lanes per bank group.
__device__ __forceinline__ int unit_kp(int tid) { return (tid & 1) | ((tid >> 2) & 0xE); }
__device__ __forceinline__ int unit_seg(int tid) { return ((tid >> 1) & 3) | ((tid >> 4) & 0x1C); }

struct ChunkRegs {
  u32x4 v[2];       // per key: 16 bytes (global: 32 E2M1 codes, half of them used; window: 16 E4M3)
  uint32_t sc[2];   // global: E8M0 scale codes
  bool ok[2];       // key present
};

// Per-sequence bases of the inputs a work-group reads.
struct RowBase {
  const uint8_t* lat;     // latent of pool row 0
  const uint8_t* sc;      // scales of pool row 0
  const uint8_t* win;     // window row 0 of the query row
};

// One 16-byte load per key from a selected address, with no branch: an
// absent key reads entry 0 or row 0 of the sequence and is masked by ok, so
// that no register merge has to wait for the loads.  Every address read is
// inside the inputs.
__device__ __forceinline__ void load_chunk(const AttnArgs& a, const RowBase& rb, int chunk, int Cg,
                                           const int32_t* idx_s, int key0, ChunkRegs& r) {
  const int tid = threadIdx.x;
  const int kp = unit_kp(tid);
  const int seg = unit_seg(tid);
  const bool glob = chunk < Cg;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int kpos = chunk * KS + 2 * kp + i;                 // global key position
    const int wr = (chunk - Cg) * KS + 2 * kp + i;            // window row
    const int32_t e = idx_s[(kpos - key0) & (kMaxChunksPerSplit * KS - 1)];
    const bool ok = glob ? (kpos < a.K && e >= 0) : (wr < a.W);
    r.ok[i] = ok;
    const size_t er = (size_t)(glob && ok ? e : 0);
    const uint8_t* gsrc = rb.lat + er * kLatRow + (seg >> 1) * 16;
    const uint8_t* wsrc = rb.win + (size_t)(!glob && ok ? wr : 0) * kD + seg * 16;
    r.v[i] = *reinterpret_cast<const u32x4*>(glob ? gsrc : wsrc);
    // window chunks read a byte of q instead (the pool may be absent)
    const uint8_t* sp = glob ? rb.sc + er * kScaleRow + (seg >> 1) : reinterpret_cast<const uint8_t*>(a.q);
    r.sc[i] = *sp;
  }
}

// Largest of x over the 16 lanes that share lane bits 1 and 2 (the 16 key
// pairs of one staging segment): lane bits 0, 3, 4, 5.
__device__ __forceinline__ uint32_t kp_max(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kDppXor1, 0xF, 0xF, false));
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kDppRor8, 0xF, 0xF, false));
  auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = max(a[0], a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return max(b[0], b[1]);
}

// ref: this thread's block's running reference (the largest scale code of
// the split's keys staged so far), updated here for a global chunk and
// published in refb[block] for the compute phase.
__device__ __forceinline__ void stage_chunk(int chunk, int Cg, const ChunkRegs& r, uint32_t* rowb,
                                            uint32_t* pairb, int32_t* valid_s, uint32_t& ref,
                                            uint32_t* refb) {
  const int tid = threadIdx.x;
  const int kp = unit_kp(tid);
  const int seg = unit_seg(tid);
  // Absent keys are converted like the others (their codes are finite data
  // of entry 0 or row 0): their logits are masked and their p is 0.
  uint32_t w[2][8];   // per key: 16 bf16 of dims seg*16 .. seg*16+15 as 8 dim pairs
  uint32_t f[2][8];   // the same dims in fp16, in units of 2^(ref-127) for global keys
  if (chunk < Cg) {
    const bool hi = seg & 1;             // the 8 code bytes are the upper half of the 16 loaded
    ref = max(ref, kp_max(max(r.ok[0] ? r.sc[0] : 0u, r.ok[1] ? r.sc[1] : 0u)));
    if (kp == 0 && !hi) refb[seg >> 1] = ref;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t sc = r.sc[i];
      const float scale = __uint_as_float(sc ? (sc << 23) : 0x00400000u);   // 2^(sc-127)
      // 2^(sc-ref) <= 1 for a present key; an absent key (entry 0's codes,
      // whose scale may exceed ref) stages zeros, so that 0 x p stays 0
      const float rel = r.ok[i] ? __builtin_amdgcn_ldexpf(1.0f, (int)sc - (int)ref) : 0.f;
      const uint32_t x0 = hi ? r.v[i][2] : r.v[i][0];
      const uint32_t x1 = hi ? r.v[i][3] : r.v[i][1];
#define CSA2_CVT_FP4(M)                                                                          \
      w[i][M] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x0, scale, M));     \
      w[i][4 + M] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(x1, scale, M)); \
      f[i][M] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x0, rel, M));        \
      f[i][4 + M] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(x1, rel, M));
      CSA2_CVT_FP4(0)
      CSA2_CVT_FP4(1)
      CSA2_CVT_FP4(2)
      CSA2_CVT_FP4(3)
#undef CSA2_CVT_FP4
    }
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        w[i][2 * d] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)r.v[i][d], 1.0f, false));
        w[i][2 * d + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)r.v[i][d], 1.0f, true));
        f[i][2 * d] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)r.v[i][d], 1.0f, false));
        f[i][2 * d + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)r.v[i][d], 1.0f, true));
      }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    uint32_t* dst = rowb + (2 * kp + i) * kRowU + seg * 8;
    *reinterpret_cast<u32x4*>(dst) = u32x4{w[i][0], w[i][1], w[i][2], w[i][3]};
    *reinterpret_cast<u32x4*>(dst + 4) = u32x4{w[i][4], w[i][5], w[i][6], w[i][7]};
  }
  uint32_t pr[16];    // dim seg*16 + j: (key 2kp, key 2kp+1)
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    pr[2 * m] = __builtin_amdgcn_perm(f[1][m], f[0][m], 0x05040100u);
    pr[2 * m + 1] = __builtin_amdgcn_perm(f[1][m], f[0][m], 0x07060302u);
  }
  uint32_t* pd = pairb + kp * kPairU + seg * 16;
#pragma unroll
  for (int p4 = 0; p4 < 4; ++p4)
    *reinterpret_cast<u32x4*>(pd + 4 * p4) = u32x4{pr[4 * p4], pr[4 * p4 + 1], pr[4 * p4 + 2], pr[4 * p4 + 3]};
  if (seg == 0) {
    valid_s[2 * kp] = r.ok[0];
    valid_s[2 * kp + 1] = r.ok[1];
  }
}

// grid (splits, rows), kThreads
__global__ __launch_bounds__(kThreads, 1)
void k_attn_partial(AttnArgs a, int32_t Cg, int32_t C, int32_t cps) {
  __shared__ __attribute__((aligned(16))) uint32_t rowb[2][kRowBufU];
  __shared__ __attribute__((aligned(16))) uint32_t pairb[2][kPairBufU];
  __shared__ __attribute__((aligned(16))) uint32_t ps[8][8][4];   // [wave][key pair][head]: fp16 p pair
  __shared__ uint32_t refb[2][kScaleRow];   // per staged chunk and 32-dim block: the running reference
  __shared__ int32_t idx_s[kMaxChunksPerSplit * KS];
  __shared__ int32_t valid_s[2][KS];
  __shared__ float mls[4][4][2];

  const int row = blockIdx.y;
  const int split = blockIdx.x;
  const int S = gridDim.x;
  const int b = row / a.Q;
  const int t = row - b * a.Q;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hg = wave & 3;                 // heads 4hg .. 4hg+3
  const int st = wave >> 2;                // key stream
  const int c0 = split * cps;
  const int c1 = (c0 + cps < C) ? c0 + cps : C;

  // entry numbers of this split's global keys -> LDS
  const int key0 = c0 * KS;
  const int gend = (c1 < Cg ? c1 : Cg) * KS;
  const int key1 = gend < a.K ? gend : a.K;
  for (int k = key0 + tid; k < key1; k += kThreads) {   // entry -> pool row (-1 stays)
    const int32_t e = a.idx[(size_t)row * a.K + k];
    idx_s[k - key0] = e >= 0 ? (int32_t)pool_row(a.map, b, e, a.M) : -1;
  }

  // logits lane: key group kb (4 keys), dim part dp (dims 8dp + 128j .. +7, j < 4).
  // Head slot s holds head 4hg + (s ^ hx) and key slot s key 4kb + (s ^ kx).
  const int kb = lane >> 4;
  const int dp = lane & 15;
  const int hx = dp & 3;
  const int kx = (dp >> 2) & 3;
  u32x4 qr[4][4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint16_t* qh = a.q + ((size_t)row * kH + 4 * hg + (s ^ hx)) * kD + 8 * dp;
#pragma unroll
    for (int j = 0; j < 4; ++j) qr[s][j] = *reinterpret_cast<const u32x4*>(qh + 128 * j);
  }
  __syncthreads();

  RowBase rbase;
  rbase.lat = a.latent;   // idx_s holds pool rows
  rbase.sc = a.scale;
  rbase.win = a.swa + ((size_t)b * a.swa_rows + t) * kD;
  ChunkRegs r;
  load_chunk(a, rbase, c0, Cg, idx_s, key0, r);
  uint32_t sref = 0;   // running reference of the block this thread stages
  stage_chunk(c0, Cg, r, rowb[0], pairb[0], valid_s[0], sref, refb[0]);
  load_chunk(a, rbase, c0 + 1 < c1 ? c0 + 1 : c0, Cg, idx_s, key0, r);
  __syncthreads();

  float acc[4][8];                         // P x V: heads 4hg.. x dims 4l..4l+3, 256+4l..
#pragma unroll
  for (int h = 0; h < 4; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[h][i] = 0.f;
  float m_run = -INFINITY;                 // softmax state of head 4hg + hx in this stream
  float l_run = 0.f;
  uint32_t r_lo = 0, r_hi = 0;             // references of the blocks of dims 4l.. and 256+4l..

  for (int c = c0; c < c1; ++c) {
    const int cur = (c - c0) & 1;

    float zs;
    {  // logits of 4 heads x 4 keys over 32 dims, then summed over the row's 16 lanes
      const uint32_t* rb = rowb[cur] + (16 * st + 4 * kb) * kRowU + 4 * dp;
      float z[4][4];
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int k = 0; k < 4; ++k) z[h][k] = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t* kr = rb + (k ^ kx) * kRowU;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 cv = *reinterpret_cast<const u32x4*>(kr + 64 * j);
#pragma unroll
          for (int h = 0; h < 4; ++h)
#pragma unroll
            for (int w = 0; w < 4; ++w) z[h][k] = fdot2(qr[h][j][w], cv[w], z[h][k]);
        }
      }
      // The partner in each step flips the lane bits that select the slot
      // order, so the element in my slot (h, k) sits in its slot (h ^ x, k ^ y).
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int k = 0; k < 2; ++k) z[h][k] += dpp<kDppXor15>(z[h ^ 3][k ^ 3]);
#pragma unroll
      for (int h = 0; h < 4; ++h) z[h][0] += dpp<kDppXor7>(z[h ^ 3][1]);
#pragma unroll
      for (int h = 0; h < 2; ++h) z[h][0] += dpp<kDppXor2>(z[h ^ 2][0]);
      z[0][0] += dpp<kDppXor1>(z[1][0]);
      zs = z[0][0];                        // head 4hg + hx, key 4kb + kx of the stream
    }

    float alpha;
    {  // online softmax of head 4hg + hx over the stream's 16 keys
      const int kk = 4 * kb + kx;
      const float zv = valid_s[cur][16 * st + kk] ? zs : -INFINITY;
      float mc = fmaxf(zv, dpp<kDppRor4>(zv));
      mc = rows_max(fmaxf(mc, dpp<kDppRor8>(mc)));
      // The reference m_run moves only when the chunk's max passes it by
      // more than kLazyMax, so that p <= e^kLazyMax and most chunks need no
      // rescaling; o / l and m + log l are the same for any reference.
      const float m_new = mc > m_run + kLazyMax ? mc : m_run;
      float p = 0.f;
      alpha = 1.f;
      if (m_new != -INFINITY) {
        p = __expf(zv - m_new);
        alpha = __expf(m_run - m_new);
      }
      float ls = p + dpp<kDppRor4>(p);
      ls = rows_sum(ls + dpp<kDppRor8>(ls));
      l_run = l_run * alpha + ls;
      m_run = m_new;
      // key pairs (kk, kk + 1) for kk even: the odd key is in lane dp + 4;
      // p in fp16 (round to nearest even, relative error below 2^-11;
      // p <= e^kLazyMax stays far below the fp16 maximum)
      const float po = dpp<kDppRor12>(p);
      const uint32_t pu = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){p, po}, f16x2));
      if (!(dp & 4)) ps[wave][kk >> 1][hx] = pu;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    {  // P x V
      // unit changes of the sums: a global chunk that raised a block's
      // reference (2^(old - new)), or the first window chunk after global
      // ones (to units of 1)
      float glo = 1.f, ghi = 1.f;
      if (c < Cg) {
        const uint32_t n_lo = refb[cur][lane >> 3];
        const uint32_t n_hi = refb[cur][8 + (lane >> 3)];
        glo = __builtin_amdgcn_ldexpf(1.0f, (int)r_lo - (int)n_lo);
        ghi = __builtin_amdgcn_ldexpf(1.0f, (int)r_hi - (int)n_hi);
        r_lo = n_lo;
        r_hi = n_hi;
      } else if (c == Cg && c0 < Cg) {
        glo = __builtin_amdgcn_ldexpf(1.0f, (int)r_lo - 127);
        ghi = __builtin_amdgcn_ldexpf(1.0f, (int)r_hi - 127);
      }
      float al[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) al[h] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), h));
      if (al[0] != 1.f || al[1] != 1.f || al[2] != 1.f || al[3] != 1.f || glo != 1.f || ghi != 1.f) {
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[h][i] *= al[h] * glo;
            acc[h][4 + i] *= al[h] * ghi;
          }
      }
      const uint32_t* pb = pairb[cur] + (8 * st) * kPairU + 4 * lane;
      const uint32_t* pw = &ps[wave][0][0];
      // two register sets, each loaded one step before use; the scheduling
      // barriers keep the compiler from sinking the loads to their uses
      u32x4 A[3], Bx[3];
      auto load_pair = [&](u32x4* x, int kp) {
        x[0] = *reinterpret_cast<const u32x4*>(pw + kp * 4);
        x[1] = *reinterpret_cast<const u32x4*>(pb + kp * kPairU);
        x[2] = *reinterpret_cast<const u32x4*>(pb + kp * kPairU + 256);
      };
      auto pv_pair = [&](const u32x4* x) {
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            acc[h][i] = hdot2(x[0][h], x[1][i], acc[h][i]);
            acc[h][4 + i] = hdot2(x[0][h], x[2][i], acc[h][4 + i]);
          }
      };
      load_pair(A, 0);
#pragma unroll 1
      for (int kp = 0; kp < 8; kp += 2) {
        load_pair(Bx, kp + 1);
        __builtin_amdgcn_sched_barrier(0);
        pv_pair(A);
        __builtin_amdgcn_sched_barrier(0);
        load_pair(A, (kp + 2) & 7);      // the last step reloads pair 0, unused
        __builtin_amdgcn_sched_barrier(0);
        pv_pair(Bx);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // the next chunk's codes (loaded one compute phase ago) go to the other buffer
    if (c + 1 < c1) stage_chunk(c + 1, Cg, r, rowb[cur ^ 1], pairb[cur ^ 1], valid_s[cur ^ 1], sref, refb[cur ^ 1]);
    load_chunk(a, rbase, c + 2 < c1 ? c + 2 : c1 - 1, Cg, idx_s, key0, r);   // past the end: a harmless reload
    __syncthreads();
  }

  if (c1 <= Cg) {   // the split holds global keys only: to units of 1
    const float unit_lo = __builtin_amdgcn_ldexpf(1.0f, (int)r_lo - 127);
    const float unit_hi = __builtin_amdgcn_ldexpf(1.0f, (int)r_hi - 127);
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[h][i] *= unit_lo;
        acc[h][4 + i] *= unit_hi;
      }
  }
  // stream 1 hands its (o, max, sum) to stream 0 through LDS
  float* xa = reinterpret_cast<float*>(rowb[0]) + hg * 32 * 64 + lane;
  if (st == 1) {
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i) xa[(h * 8 + i) * 64] = acc[h][i];
    if (lane < 4) {
      mls[hg][lane][0] = m_run;
      mls[hg][lane][1] = l_run;
    }
  }
  __syncthreads();

  float Mh[4], Lh[4];
  if (st == 0) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float m0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m_run), h));
      const float l0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l_run), h));
      const float m1 = mls[hg][h][0];
      const float l1 = mls[hg][h][1];
      const float M = fmaxf(m0, m1);
      const float w0 = m0 == -INFINITY ? 0.f : __expf(m0 - M);
      const float w1 = m1 == -INFINITY ? 0.f : __expf(m1 - M);
      Mh[h] = M;
      Lh[h] = l0 * w0 + l1 * w1;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[h][i] = acc[h][i] * w0 + xa[(h * 8 + i) * 64] * w1;
    }
  }

  if (S == 1) {   // the whole row is here: merge an incoming result, normalise, write
    if (st == 0) {
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const size_t hr = (size_t)row * kH + 4 * hg + h;
        float M = Mh[h], L = Lh[h];
        if (a.lse_in) {     // (o, lse) in/out may alias: each lane reads its own elements first
          const float li = a.lse_in[hr];
          const float M2 = fmaxf(M, li);
          const float w1 = M == -INFINITY ? 0.f : __expf(M - M2);
          const float w2 = li == -INFINITY ? 0.f : __expf(li - M2);
          const float4 x0 = *reinterpret_cast<const float4*>(a.o_in + hr * kD + 4 * lane);
          const float4 x1 = *reinterpret_cast<const float4*>(a.o_in + hr * kD + 256 + 4 * lane);
          const float xi[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[h][i] = acc[h][i] * w1 + xi[i] * w2;
          L = L * w1 + w2;
          M = M2;
        }
        const float inv = L > 0.f ? 1.f / L : 0.f;
        float* dst = a.o + hr * kD + 4 * lane;
        *reinterpret_cast<float4*>(dst) = make_float4(acc[h][0] * inv, acc[h][1] * inv, acc[h][2] * inv, acc[h][3] * inv);
        *reinterpret_cast<float4*>(dst + 256) = make_float4(acc[h][4] * inv, acc[h][5] * inv, acc[h][6] * inv, acc[h][7] * inv);
        if (lane == 0) a.lse[hr] = L > 0.f ? M + logf(L) : -INFINITY;
      }
    }
    return;
  }

  if (st == 0) {   // this split's partial: unnormalised o, max, sum
    float* op = a.opart + (((size_t)row * S + split) * kH + 4 * hg) * kD + 4 * lane;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      *reinterpret_cast<float4*>(op + (size_t)h * kD) = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
      *reinterpret_cast<float4*>(op + (size_t)h * kD + 256) = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
    }
    if (lane < 4) {
      const float L = lane == 0 ? Lh[0] : lane == 1 ? Lh[1] : lane == 2 ? Lh[2] : Lh[3];
      const float M = lane == 0 ? Mh[0] : lane == 1 ? Mh[1] : lane == 2 ? Mh[2] : Mh[3];
      float* mlp = a.ml + (((size_t)row * S + split) * kH + 4 * hg + lane) * 2;
      mlp[0] = M;
      mlp[1] = L;
    }
  }
}

// One work-group (128 lanes x 4 dims) per (head, query row).  The partial
// rows of up to kCombBatch splits are loaded together with every split's
// (max, sum) pair, so that the merge waits on one round trip to memory; the
// weights are formed in LDS by the first wave, and the rows are summed in
// split order, then the incoming result.
constexpr int kCombThreads = 128;
constexpr int kCombMaxS = 63;            // splits per row (lane kCombMaxS holds an incoming result)
constexpr int kCombBatch = 8;            // partial rows in flight per lane

__global__ __launch_bounds__(kCombThreads)
void k_attn_combine(const float* __restrict__ opart, const float* __restrict__ ml,
                    int32_t S, const float* o_in, const float* lse_in, float* o,
                    float* lse) {
  __shared__ float wgt_s[kCombMaxS + 1];
  __shared__ float L_s;
  const int h = blockIdx.x;
  const int row = blockIdx.y;
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
    if (tid <= S && tid <= kCombMaxS) wgt_s[tid] = w;
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

int32_t attn_chunks(int32_t K, int32_t W) {
  return (K > 0 ? (K + KS - 1) / KS : 0) + (W > 0 ? (W + KS - 1) / KS : 0);
}

AttnPlan attn_plan(int64_t rows, int32_t chunks) {
  // Splits S per row so that the launch fills the chip without giving some
  // compute units two work-groups while others idle (a work-group's LDS
  // takes a compute unit): estimated time = rounds of kGroupsPerRound
  // work-groups x (chunks per work-group + a fixed prologue), plus a merge
  // launch when S > 1.
  if (chunks <= 0) return AttnPlan{16, 0, 0.0};
  AttnPlan best{16, 1, 1e30};
  const int64_t lo = (chunks + kMaxChunksPerSplit - 1) / kMaxChunksPerSplit;
  for (int64_t S = lo; S <= chunks && S <= kCombMaxS; ++S) {
    const int64_t cps = (chunks + S - 1) / S;
    if ((chunks + cps - 1) / cps != S) continue;
    const int64_t rounds = (rows * S + kGroupsPerRound - 1) / kGroupsPerRound;
    const double cost = (double)rounds * ((double)cps + 0.5) + (S > 1 ? 1.0 : 0.0);
    if (cost < best.cost - 1e-9) best = AttnPlan{16, (int32_t)S, cost};
  }
  return best;
}

hipError_t launch_attn_partial(const AttnArgs& a, const AttnPlan& plan, hipStream_t s) {
  const int32_t Cg = a.K > 0 && a.latent ? (a.K + KS - 1) / KS : 0;
  const int32_t C = Cg + (a.W > 0 ? (a.W + KS - 1) / KS : 0);
  const int32_t splits = plan.splits;
  if (C == 0 || splits <= 0) return hipSuccess;
  const int32_t cps = (C + splits - 1) / splits;
  if (cps > kMaxChunksPerSplit || (C + cps - 1) / cps != splits || splits > kCombMaxS)
    return hipErrorInvalidValue;
  k_attn_partial<<<dim3((unsigned)splits, (unsigned)a.rows), dim3(kThreads), 0, s>>>(a, Cg, C, cps);
  if (splits == 1) return hipGetLastError();
  k_attn_combine<<<dim3((unsigned)kH, (unsigned)a.rows), dim3(kCombThreads), 0, s>>>(
      a.opart, a.ml, splits, a.o_in, a.lse_in, a.o, a.lse);
  return hipGetLastError();
}

}  // namespace csa2

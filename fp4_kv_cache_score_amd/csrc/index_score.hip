// Indexer score kernel: streams E4M3 index keys from HBM, one pass per query row.
//
// Reading of the pages (they give no formula, only that Full / Reindex layers
// score the context with an indexer, "DeepSeek V4.1-Flash Cuts KV Cache by
// 437x", paragraph on the three operating modes):
//   s_j = sum_h w_h * ReLU(sum_i qI[h][i] * kI[j][h][i]),  8 heads x 64 E4M3.
//
// Work split (the arithmetic is in index_math.h): a pool entry's 512-byte
// key row is read by 32 lanes with one 16-byte load each (two entries per
// wave64 load), so every wave load is a fully coalesced 1 KiB; each lane
// issues them in batches of 4, the next batch in flight while the current one
// is computed.  Every lane holds the full query slice it needs in registers,
// so HBM sees each key byte exactly once.
// Optionally the kernel adds the scores' top-12-bit order keys into a
// per-row histogram (the first radix digit of the Top-K select), built in
// LDS per work-group and flushed with one atomic per non-empty bin.
#include "csa2_internal.h"
#include "index_math.h"

namespace csa2 {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;                        // 16-byte loads per lane and batch (two batches in flight)

// EPW pool entries per wave, 4 waves per work-group.  With a candidate list
// the work-group first copies its EPW * 4 entry numbers to LDS (one round
// trip), so that every key load of the streaming loop is independent.
template <int EPW, bool kCand, bool kHist>
__global__ __launch_bounds__(kThreads)
void k_index_score(const uint8_t* __restrict__ key, int64_t M,
                   const uint8_t* __restrict__ q_idx,
                   const float* __restrict__ w_idx, int32_t Q, int64_t pos0,
                   int32_t ratio, const int32_t* __restrict__ cand, int32_t N,
                   float* __restrict__ scores, uint32_t* __restrict__ hist,
                   const int32_t* __restrict__ len, PoolMap map, ZeroSpans zs) {
  constexpr int kEntriesPerWG = EPW * (kThreads / 64);
  {  // the spans to clear on the side: 16 bytes per thread of the first work-groups
    const int64_t t = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * kThreads + threadIdx.x;
    const int64_t q0 = zs.n[0] / 4, q1 = q0 + zs.n[1] / 4, q2 = q1 + zs.n[2] / 4;
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    if (t < q0) reinterpret_cast<uint4*>(zs.p[0])[t] = z;
    else if (t < q1) reinterpret_cast<uint4*>(zs.p[1])[t - q0] = z;
    else if (t < q2) reinterpret_cast<uint4*>(zs.p[2])[t - q1] = z;
  }
  constexpr int kIters = EPW / (2 * kUnroll);
  static_assert(EPW % (2 * kUnroll) == 0, "EPW must be a multiple of 16");
  __shared__ uint32_t lh[kHist ? kHistBins : 1];
  __shared__ int32_t ce[kCand ? kEntriesPerWG : 1];
  const int row = blockIdx.y;
  const int b = row / Q;
  const int t = row - b * Q;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int sub = lane & 31;
  const int head = sub >> 2;

  // Entries visible to this query: the sequence's length (M, or len[b] for a
  // ragged batch), within the causal limit when there is one.
  int64_t vis = len ? (int64_t)len[b] : M;
  if (pos0 >= 0) {
    const int64_t v = (pos0 + t + 1) / ratio;
    vis = v < vis ? v : vis;
  }

  const int64_t g0 = (int64_t)blockIdx.x * kEntriesPerWG;
  if (kCand) {   // candidates -> pool rows (-1: absent or not visible to this query)
    const int32_t* cb = cand + (size_t)b * N;
    for (int i = threadIdx.x; i < kEntriesPerWG; i += kThreads) {
      const int64_t p = g0 + i;
      const int32_t c = p < N ? cb[p] : -1;
      ce[i] = (c >= 0 && c < vis) ? (int32_t)pool_row(map, b, c, M) : -1;
    }
  }
  float qf[16];
  const uint8_t* qsrc = q_idx + (size_t)row * kKeyRow + sub * 16;
  load_q_slice(qsrc, qf);
  const float wh = w_idx[(size_t)row * kHI + head];

  if (kHist)
    for (int i = threadIdx.x; i < kHistBins; i += kThreads) lh[i] = 0u;
  if (kHist || kCand) __syncthreads();

  float* srow = scores + (size_t)row * N;
  const int wofs = wave * EPW;
  // the wave's EPW consecutive entries lie in one page (pages hold >= 64
  // entries and a wave starts at a multiple of EPW): one lookup per wave
  const int64_t w0 = g0 + wofs;
  const int64_t roff = kCand ? 0 : (w0 < M ? pool_row(map, b, w0, M) : 0) - w0;   // row - entry
  const uint8_t* kb = key + sub * 16;

  // Batches of kUnroll loads per lane, software-pipelined: the next batch is
  // issued before this one is consumed, so a wave keeps loads in flight while
  // it computes.
  u32x4 v[2][kUnroll];
  bool ok[2][kUnroll];
  auto issue = [&](int it, int bi) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int lp = wofs + it * (2 * kUnroll) + 2 * u + half;   // position within the work-group
      const int64_t p = g0 + lp;
      int64_t e = p;                       // flat: the entry; kb is offset so that e indexes it
      bool valid = p < N && e < vis;
      if (kCand) {
        e = ce[lp];                        // candidate: its pool row
        valid = e >= 0;
      }
      ok[bi][u] = valid;
      // every lane loads (an absent entry reads the query row instead, its
      // score is -inf whatever it holds): a load under a branch would make
      // the compiler wait for each one before issuing the next
      const uint8_t* src = valid ? kb + (roff + e) * kKeyRow : qsrc;
      v[bi][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
    }
  };
  issue(0, 0);
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int cb = it & 1;
    if (it + 1 < kIters) issue(it + 1, cb ^ 1);
    __builtin_amdgcn_sched_barrier(0);     // the next batch issues before this one is used
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float r = entry_score(v[cb][u], qf, wh);
      const int64_t p = g0 + wofs + it * (2 * kUnroll) + 2 * u + half;
      if (sub == 0 && p < N) {
        srow[p] = ok[cb][u] ? r : -INFINITY;
        if (kHist && ok[cb][u]) atomicAdd(&lh[score_key(r) >> (32 - kHistBits)], 1u);
      }
    }
  }

  if (kHist) {
    __syncthreads();
    uint32_t* hrow = hist + (size_t)row * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += kThreads) {
      const uint32_t c = lh[i];
      if (c) atomicAdd(&hrow[i], c);
    }
  }
}

template <int EPW>
hipError_t launch_epw(const uint8_t* key, int32_t B, int64_t M, const uint8_t* q_idx,
                      const float* w_idx, int32_t Q, int64_t pos0, int32_t ratio,
                      const int32_t* cand, int32_t N, float* scores, uint32_t* hist,
                      const int32_t* len, const PoolMap& map, hipStream_t s,
                      const ZeroSpans* zero) {
  const dim3 grid((unsigned)((N + EPW * 4 - 1) / (EPW * 4)), (unsigned)(B * Q));
  const dim3 block(kThreads);
  ZeroSpans zs{{nullptr, nullptr, nullptr}, {0, 0, 0}};
  if (zero) {
    // spans the grid cannot take 16 bytes per thread go to fill launches
    const int64_t threads = (int64_t)grid.x * grid.y * kThreads;
    int64_t words = 0;
    bool side = true;
    for (int i = 0; i < 3; ++i) {
      if (zero->n[i] < 0) return hipErrorInvalidValue;
      side = side && !(zero->n[i] & 3) && !(zero->n[i] && ((uintptr_t)zero->p[i] & 15));
      words += zero->n[i];
    }
    if (side && words / 4 <= threads) {
      zs = *zero;
    } else {
      for (int i = 0; i < 3; ++i) {
        if (!zero->n[i]) continue;
        const hipError_t e = launch_fill_zero(zero->p[i], zero->n[i], s);
        if (e != hipSuccess) return e;
      }
    }
  }
  if (cand) {
    if (hist)
      k_index_score<EPW, true, true><<<grid, block, 0, s>>>(key, M, q_idx, w_idx, Q, pos0, ratio, cand, N, scores, hist, len, map, zs);
    else
      k_index_score<EPW, true, false><<<grid, block, 0, s>>>(key, M, q_idx, w_idx, Q, pos0, ratio, cand, N, scores, hist, len, map, zs);
  } else {
    if (hist)
      k_index_score<EPW, false, true><<<grid, block, 0, s>>>(key, M, q_idx, w_idx, Q, pos0, ratio, cand, N, scores, hist, len, map, zs);
    else
      k_index_score<EPW, false, false><<<grid, block, 0, s>>>(key, M, q_idx, w_idx, Q, pos0, ratio, cand, N, scores, hist, len, map, zs);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_index_score(const uint8_t* key, int32_t B, int64_t M,
                              const uint8_t* q_idx, const float* w_idx,
                              int32_t Q, int64_t pos0, int32_t ratio,
                              const int32_t* cand, int32_t N, float* scores,
                              uint32_t* hist, const int32_t* len, const PoolMap& map,
                              hipStream_t s, const ZeroSpans* zero) {
  // 64 entries per wave (256 per work-group) keep enough loads in flight on
  // long rows; short rows (candidate pools) take 32 so that the launch still
  // has >= 1024 work-groups.
  const int64_t rows = (int64_t)B * Q;
  if (rows * ((N + 255) / 256) >= 1024)
    return launch_epw<64>(key, B, M, q_idx, w_idx, Q, pos0, ratio, cand, N, scores, hist, len, map, s,
                          zero);
  return launch_epw<32>(key, B, M, q_idx, w_idx, Q, pos0, ratio, cand, N, scores, hist, len, map, s,
                        zero);
}

}  // namespace csa2

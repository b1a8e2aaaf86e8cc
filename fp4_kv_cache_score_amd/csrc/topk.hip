// Top-K select with the lower-index tie-break, ascending output.
//
// The pages say only that Full and Reindex layers select Top-K entries from
// the indexer scores ("DeepSeek V4.1-Flash Cuts KV Cache by 437x", paragraph
// on the three operating modes); equal scores going to the lower pool index
// and the ascending output order are this library's fixed conventions.
//
// Every (score, position) pair maps to a unique 62-bit composite order key
//   key32(score) : (n - 1 - position)
// (key32 is the order-preserving uint32 image of the float), so the K largest
// composites are exactly the wanted set, and a radix select over the
// composite finds them.
//
// Rows of up to 2^18 positions (every decode and prefill shape here) use
// k_topk_row, one 1024-thread work-group per row:
//  1. a histogram of the top 12 key bits (taken from the score kernel, which
//     builds it while it writes the scores, or built here) gives the digit
//     that holds the K-th largest key;
//  2. while that digit holds more positions than the LDS candidate slots,
//     one more streaming pass refines the prefix by 12 bits;
//  3. one pass marks every position strictly above the prefix in an LDS
//     bitmap and copies the prefix's members to LDS;
//  4. 12-bit radix passes over the LDS candidates resolve the rest (ties
//     are broken by the position bits), and the chosen ones are marked;
//  5. a block prefix sum over the bitmap's popcounts writes the positions in
//     ascending order.
// Long rows on few rows (and rows over 2^18) use the multi-work-group path:
// k_topk_hist (unless the score kernel built the histogram) -> k_topk_collect
// (positions above the threshold bin and that bin's members, appended with
// one atomic per work-group) -> k_topk_finish (radix passes over the members
// and an ordered extraction through bitmap segments; it leaves the row's
// counters, and optionally its histogram, zeroed for the next select).
// Ties, -0 vs +0, rows with fewer than K valid positions are handled exactly;
// the result is deterministic.
#include "csa2_internal.h"
#include "index_math.h"

namespace csa2 {
namespace {

constexpr int kSelThreads = 256;
constexpr int kChunk = 4096;              // positions per collect / hist work-group
constexpr int kFinThreads = 1024;
constexpr int kSegBits = 18;              // bitmap segment of 2^18 positions (32 KiB)
constexpr int kSeg = 1 << kSegBits;
constexpr int kSegWords = kSeg / 32;      // 8192
constexpr int kCompBits = 50;             // 20 low key bits + 30 position bits
constexpr int kDigit = 10;                // multi-work-group finish: 10-bit digits
constexpr int kRowDigit = 12;             // one-work-group select: 12-bit digits

__device__ __forceinline__ int32_t row_count(const int32_t* n_valid, int32_t n_all,
                                             int row, int32_t N) {
  int32_t n = n_valid ? n_valid[row] : n_all;
  return n < 0 ? 0 : (n > N ? N : n);
}

// Inclusive prefix sum over the 64 lanes of a wave: a scan inside each row
// of 16 lanes with DPP row shifts, then the row totals added with readlane.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);   // row_shr:8
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row > 0 ? r0 : 0u) + (row > 1 ? r1 : 0u) + (row > 2 ? r2 : 0u);
}

// The calling wave's exclusive prefix over the block's per-wave totals
// slot[k * stride] (k < NW <= 16) and their sum: lane k reads total k, a DPP
// scan runs within the first row of 16 lanes, and two single-lane reads give
// the results (a few instructions per wave instead of NW reads and adds).
template <int NW>
__device__ __forceinline__ void wave_prefix(const uint32_t* slot, int stride, uint32_t* before,
                                            uint32_t* all) {
  static_assert(NW >= 1 && NW <= 16, "one DPP row of totals");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t r = slot[(lane < NW ? lane : 0) * stride];
  uint32_t t = lane < NW ? r : 0u;
  t += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)t, 0x111, 0xF, 0xF, true);   // row_shr:1
  t += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)t, 0x112, 0xF, 0xF, true);   // row_shr:2
  t += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)t, 0x114, 0xF, 0xF, true);   // row_shr:4
  t += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)t, 0x118, 0xF, 0xF, true);   // row_shr:8
  *all = (uint32_t)__builtin_amdgcn_readlane((int)t, NW - 1);
  const uint32_t prev = (uint32_t)__builtin_amdgcn_readlane((int)t, wave > 0 ? wave - 1 : 0);
  *before = wave > 0 ? prev : 0u;
}

// Exclusive prefix sum over the NT threads of a block; *total receives the sum.
// lds must hold NT/64 words and is free again on return.  Each wave scans
// with DPP, publishes its total, and every wave then adds the totals of the
// waves before it.
template <int NT>
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t* lds, uint32_t* total) {
  constexpr int NW = NT / 64;
  const int wave = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan(v);
  lds[wave] = (uint32_t)__builtin_amdgcn_readlane((int)x, 63);   // every lane: no branch
  __syncthreads();
  uint32_t before, all;
  wave_prefix<NW>(lds, 1, &before, &all);
  *total = all;
  __syncthreads();
  return before + x - v;
}

// Bins of the K0-th and K1-th largest keys in a 4096-bin histogram (bins
// ordered by key), from one read of the histogram and one block scan.
// above[s] = number of keys in bins above bin[s]; above < K <= above + h[bin].
// bin[s] is -1 if the histogram holds fewer than K_s keys (K1 = 0: unused).
// lds: NT/64 + 5 words.  h is 16-byte aligned.
// This thread's PER bins of a 4096-bin histogram, highest first: thread 0
// owns the highest bins, c[i] = h[4096 - PER tid - 1 - i].  h 16-byte aligned.
template <int PER>
__device__ __forceinline__ void hist_slice(const uint32_t* h, uint32_t (&c)[PER]) {
  const int lo = kHistBins - (int)(threadIdx.x + 1) * PER;
#pragma unroll
  for (int j = 0; j < PER / 4; ++j) {
    const uint4 v = *reinterpret_cast<const uint4*>(h + lo + 4 * j);
    c[PER - 1 - 4 * j] = v.x;
    c[PER - 2 - 4 * j] = v.y;
    c[PER - 3 - 4 * j] = v.z;
    c[PER - 4 - 4 * j] = v.w;
  }
}

template <int NT>
__device__ void threshold_bins_c(const uint32_t (&c)[kHistBins / NT], uint32_t K0, uint32_t K1,
                                 uint32_t* lds, int* bin, uint32_t* above);

template <int NT>
__device__ void threshold_bins(const uint32_t* h, uint32_t K0, uint32_t K1, uint32_t* lds,
                               int* bin, uint32_t* above) {
  uint32_t c[kHistBins / NT];
  hist_slice(h, c);
  threshold_bins_c<NT>(c, K0, K1, lds, bin, above);
}

// threshold_bins on counts already in registers (hist_slice's layout)
template <int NT>
__device__ void threshold_bins_c(const uint32_t (&c)[kHistBins / NT], uint32_t K0, uint32_t K1,
                                 uint32_t* lds, int* bin, uint32_t* above) {
  constexpr int PER = kHistBins / NT;          // a multiple of 4
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) s += c[i];
  // every thread stores the same defaults (a store behind a branch costs far
  // more than the redundant writes in these once-per-block phases)
  lds[NT / 64 + 1] = 0xFFFFFFFFu;
  lds[NT / 64 + 2] = 0u;
  lds[NT / 64 + 3] = 0xFFFFFFFFu;
  lds[NT / 64 + 4] = 0u;
  uint32_t tot;
  const uint32_t ex = block_excl_scan<NT>(s, lds, &tot);
  const int top = kHistBins - 1 - (int)threadIdx.x * PER;
  const uint32_t Ks[2] = {K0, K1};
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint32_t K = Ks[t];
    // the bin where the running count first reaches K (selects, no branch)
    uint32_t acc = ex, fb = 0u, fa = 0u;
    bool hit = false;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const bool hi = K > 0 && acc < K && K <= acc + c[i];
      fb = hi ? (uint32_t)(top - i) : fb;
      fa = hi ? acc : fa;
      hit = hit || hi;
      acc += c[i];
    }
    if (hit) {
      lds[NT / 64 + 1 + 2 * t] = fb;
      lds[NT / 64 + 2 + 2 * t] = fa;
    }
  }
  __syncthreads();
  bin[0] = (int)lds[NT / 64 + 1];
  above[0] = lds[NT / 64 + 2];
  bin[1] = (int)lds[NT / 64 + 3];
  above[1] = lds[NT / 64 + 4];
  __syncthreads();
}

__global__ __launch_bounds__(kSelThreads)
void k_topk_hist(const float* __restrict__ scores, int32_t N,
                 const int32_t* __restrict__ n_valid, int32_t n_all,
                 uint32_t* __restrict__ hist) {
  __shared__ uint32_t lh[kHistBins];
  const int row = blockIdx.y;
  const int32_t n = row_count(n_valid, n_all, row, N);
  const int64_t c0 = (int64_t)blockIdx.x * kChunk;
  if (c0 >= n) return;
  for (int i = threadIdx.x; i < kHistBins; i += kSelThreads) lh[i] = 0u;
  __syncthreads();
  const float* sr = scores + (size_t)row * N;
  for (int i = 0; i < kChunk / kSelThreads; ++i) {
    const int64_t p = c0 + i * kSelThreads + threadIdx.x;
    if (p < n) atomicAdd(&lh[score_key(sr[p]) >> (32 - kHistBits)], 1u);
  }
  __syncthreads();
  uint32_t* hr = hist + (size_t)row * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += kSelThreads) {
    const uint32_t c = lh[i];
    if (c) atomicAdd(&hr[i], c);
  }
}

// Positions of one work-group's chunk above select t's threshold bin go to
// t.sel, the bin's members (key, position) to t.candk / t.candp, each list
// with one atomic per work-group; slots in any order (the finish step orders
// the output through a bitmap).  Work-group 0 of the row also records the
// bin and the count above it in counters [2] and [3] for the finish step.
template <int PER>
__device__ void collect_one(const uint32_t (&key)[PER], int64_t c0, int32_t n, int row,
                            int bstar, uint32_t above, const SelectSet& t, uint32_t* lds,
                            uint32_t* base_s) {
  uint32_t* cnt = t.counters + (size_t)row * kCounterWords;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    cnt[2] = (uint32_t)bstar;
    cnt[3] = above;
  }
  uint32_t ngt = 0, neq = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int64_t p = c0 + i * kSelThreads + threadIdx.x;
    const int bin = (int)(key[i] >> (32 - kHistBits));
    ngt += (p < n && bin > bstar) ? 1u : 0u;
    neq += (p < n && bin == bstar) ? 1u : 0u;
  }
  uint32_t tot;
  const uint32_t ex = block_excl_scan<kSelThreads>((ngt << 16) | neq, lds, &tot);
  if (threadIdx.x == 0) {
    base_s[0] = (tot >> 16) ? atomicAdd(&cnt[0], tot >> 16) : 0u;
    base_s[1] = (tot & 0xFFFFu) ? atomicAdd(&cnt[1], tot & 0xFFFFu) : 0u;
  }
  __syncthreads();
  uint32_t rg = base_s[0] + (ex >> 16);
  uint32_t re = base_s[1] + (ex & 0xFFFFu);
  int32_t* srow = t.sel + (size_t)row * t.K;
  uint32_t* ckr = t.candk + (size_t)row * t.cap;
  int32_t* cpr = t.candp + (size_t)row * t.cap;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int64_t p = c0 + i * kSelThreads + threadIdx.x;
    if (p >= n) continue;
    const int bin = (int)(key[i] >> (32 - kHistBits));
    if (bin > bstar) {
      if (rg < (uint32_t)t.K) srow[rg] = (int32_t)p;
      ++rg;
    } else if (bin == bstar) {
      if (re < (uint32_t)t.cap) {
        ckr[re] = key[i];
        cpr[re] = (int32_t)p;
      }
      ++re;
    }
  }
}

// One pass over the scores for up to two selects (t1.K == 0: one) that
// share the row's top-12-bit histogram.
__global__ __launch_bounds__(kSelThreads)
void k_topk_collect(const float* __restrict__ scores, int32_t N,
                    const int32_t* __restrict__ n_valid, int32_t n_all,
                    const uint32_t* __restrict__ hist, SelectSet t0, SelectSet t1) {
  constexpr int PER = kChunk / kSelThreads;   // 16 positions per thread
  __shared__ uint32_t lds[kSelThreads / 64 + 5];
  __shared__ uint32_t base_s[2];
  const int row = blockIdx.y;
  const int32_t n = row_count(n_valid, n_all, row, N);
  const bool go0 = n > t0.K;
  const bool go1 = t1.K > 0 && n > t1.K;
  if (!go0 && !go1) return;
  const int64_t c0 = (int64_t)blockIdx.x * kChunk;
  if (c0 >= n) return;
  const float* sr = scores + (size_t)row * N;
  // Issue every load of this work-group's chunk before the threshold search.
  uint32_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int64_t p = c0 + i * kSelThreads + threadIdx.x;
    key[i] = p < n ? score_key(sr[p]) : 0u;
  }
  int bstar[2];
  uint32_t above[2];
  threshold_bins<kSelThreads>(hist + (size_t)row * kHistBins, go0 ? (uint32_t)t0.K : 0u,
                              go1 ? (uint32_t)t1.K : 0u, lds, bstar, above);
  if (go0) collect_one<PER>(key, c0, n, row, bstar[0], above[0], t0, lds, base_s);
  if (go1) collect_one<PER>(key, c0, n, row, bstar[1], above[1], t1, lds, base_s);
}

// Visit every member of the threshold bin: from the candidate list, or (after
// an overflow) from the score row positions [lo, hi).
template <typename F>
__device__ __forceinline__ void visit_bin(bool overflow, uint32_t C, const uint32_t* ck,
                                          const int32_t* cp, const float* sr, int bstar,
                                          int64_t lo, int64_t hi, F&& f) {
  if (!overflow) {
    for (uint32_t i = threadIdx.x; i < C; i += kFinThreads) {
      const int32_t p = cp[i];
      if (p >= lo && p < hi) f(ck[i], p);
    }
  } else {
    for (int64_t p = lo + threadIdx.x; p < hi; p += kFinThreads) {
      const uint32_t key = score_key(sr[p]);
      if ((int)(key >> (32 - kHistBits)) == bstar) f(key, (int32_t)p);
    }
  }
}

// grid (rows, selects): select blockIdx.y of t0 / t1 on its row.
__global__ __launch_bounds__(kFinThreads)
void k_topk_finish(const float* __restrict__ scores, int32_t N,
                   const int32_t* __restrict__ n_valid, int32_t n_all,
                   uint32_t* hist, int32_t zero_hist, SelectSet t0, SelectSet t1) {
  __shared__ uint32_t lds[kFinThreads / 64 + 8];
  __shared__ uint32_t rh[1 << kDigit];
  __shared__ uint32_t bitmap[kSegWords];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const SelectSet& t = blockIdx.y ? t1 : t0;
  const int32_t K = t.K;
  uint32_t* counters = t.counters;
  const int32_t cap = t.cap;
  const int32_t n = row_count(n_valid, n_all, row, N);
  int32_t* orow = t.out + (size_t)row * K;
  const int32_t* mrow = t.cand_map ? t.cand_map + (size_t)row * N : nullptr;
  // Leave this row's counters (and, when asked, its histogram: select 0's
  // work-group, as no finish reads it) zeroed for the next select.  The
  // counters are read and cleared through the same pointers, and every read
  // happens before the barrier that precedes the clearing.
  auto clean = [&]() {
    if (tid < kCounterWords) counters[(size_t)row * kCounterWords + tid] = 0u;
    if (zero_hist && blockIdx.y == 0)
      for (int i = tid; i < kHistBins; i += kFinThreads) hist[(size_t)row * kHistBins + i] = 0u;
  };
  if (n <= K) {
    for (int i = tid; i < K; i += kFinThreads) orow[i] = i < n ? (mrow ? mrow[i] : i) : -1;
    clean();
    return;
  }
  // the threshold bin and the count above it, as the collect step found them
  const int bstar = (int)counters[(size_t)row * kCounterWords + 2];
  const uint32_t above = counters[(size_t)row * kCounterWords + 3];
  const uint32_t ccount = counters[(size_t)row * kCounterWords + 1];
  __syncthreads();   // every thread has read the counters
  clean();
  if (bstar < 0) {  // inconsistent histogram: cannot happen for valid inputs
    for (int i = tid; i < K; i += kFinThreads) orow[i] = -1;
    return;
  }
  const bool overflow = ccount > (uint32_t)cap;
  const uint32_t C = overflow ? 0u : ccount;
  const uint32_t* ck = t.candk + (size_t)row * cap;
  const int32_t* cp = t.candp + (size_t)row * cap;
  const float* sr = scores + (size_t)row * N;
  const uint64_t nm1 = (uint64_t)(n - 1);
  auto comp_of = [&](uint32_t key, int32_t p) -> uint64_t {
    return ((uint64_t)(key & 0xFFFFFu) << 30) | (nm1 - (uint64_t)p);
  };

  // Radix select the remaining need = K - above composites inside bin b*.
  uint32_t need = (uint32_t)K - above;
  uint64_t prefix = 0;
  int sh = kCompBits;
  bool done = false;
  while (!done && sh > 0) {
    sh -= kDigit;
    for (int i = tid; i < (1 << kDigit); i += kFinThreads) rh[i] = 0u;
    __syncthreads();
    visit_bin(overflow, C, ck, cp, sr, bstar, 0, n, [&](uint32_t key, int32_t p) {
      const uint64_t c = comp_of(key, p);
      if ((c >> (sh + kDigit)) == prefix) atomicAdd(&rh[(c >> sh) & ((1u << kDigit) - 1)], 1u);
    });
    __syncthreads();
    const uint32_t hv = rh[(1 << kDigit) - 1 - tid];   // thread 0 owns the highest digit
    if (tid == 0) {
      lds[kFinThreads / 64 + 1] = 0u;
      lds[kFinThreads / 64 + 2] = 0u;
      lds[kFinThreads / 64 + 3] = 0u;
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan<kFinThreads>(hv, lds, &tot);
    if (ex < need && need <= ex + hv) {
      lds[kFinThreads / 64 + 1] = (uint32_t)((1 << kDigit) - 1 - tid);
      lds[kFinThreads / 64 + 2] = ex;
      lds[kFinThreads / 64 + 3] = hv;
    }
    __syncthreads();
    const uint32_t dig = lds[kFinThreads / 64 + 1];
    const uint32_t exs = lds[kFinThreads / 64 + 2];
    const uint32_t hvs = lds[kFinThreads / 64 + 3];
    __syncthreads();
    need -= exs;
    prefix = (prefix << kDigit) | dig;
    done = (hvs == need);
  }
  const uint64_t thr = prefix << sh;   // chosen bin members: composite >= thr

  // Ordered extraction, one bitmap segment at a time.
  const int32_t* srow = t.sel + (size_t)row * K;
  const uint32_t nsel = above < (uint32_t)K ? above : (uint32_t)K;
  uint32_t written = 0;
  for (int64_t s0 = 0; s0 < n; s0 += kSeg) {
    const int64_t s1 = (s0 + kSeg < n) ? s0 + kSeg : n;
    for (int i = tid; i < kSegWords; i += kFinThreads) bitmap[i] = 0u;
    __syncthreads();
    for (uint32_t i = tid; i < nsel; i += kFinThreads) {
      const int64_t p = srow[i];
      if (p >= s0 && p < s1) atomicOr(&bitmap[(p - s0) >> 5], 1u << ((p - s0) & 31));
    }
    visit_bin(overflow, C, ck, cp, sr, bstar, s0, s1, [&](uint32_t key, int32_t p) {
      if (comp_of(key, p) >= thr) atomicOr(&bitmap[(p - s0) >> 5], 1u << ((p - s0) & 31));
    });
    __syncthreads();
    constexpr int WPT = kSegWords / kFinThreads;   // 8 words per thread
    uint32_t wv[WPT];
    uint32_t cnt = 0;
#pragma unroll
    for (int w = 0; w < WPT; ++w) {
      wv[w] = bitmap[tid * WPT + w];
      cnt += __popc(wv[w]);
    }
    uint32_t tot;
    uint32_t pos = written + block_excl_scan<kFinThreads>(cnt, lds, &tot);
    if (!mrow) {   // stores only: no load in this loop (see k_topk_row)
#pragma unroll
      for (int w = 0; w < WPT; ++w) {
        uint32_t m = wv[w];
        while (m) {
          const int bit = __ffs(m) - 1;
          m &= m - 1;
          const int64_t p = s0 + (int64_t)(tid * WPT + w) * 32 + bit;
          if (pos < (uint32_t)K) orow[pos] = (int32_t)p;
          ++pos;
        }
      }
    } else {
#pragma unroll
      for (int w = 0; w < WPT; ++w) {
        uint32_t m = wv[w];
        while (m) {
          const int bit = __ffs(m) - 1;
          m &= m - 1;
          const int64_t p = s0 + (int64_t)(tid * WPT + w) * 32 + bit;
          if (pos < (uint32_t)K) orow[pos] = mrow[p];
          ++pos;
        }
      }
    }
    written += tot;
    __syncthreads();
  }
  for (uint32_t i = written + tid; i < (uint32_t)K; i += kFinThreads) orow[i] = -1;
}

// ---------------------------------------------------------------------------
// One work-group per row (rows of at most kRowMaxN positions).
// ---------------------------------------------------------------------------

constexpr int kRowThreads = 1024;
constexpr int kRowWords = kRowMaxN / 32;   // bitmap words (8192 = 32 KiB)
constexpr int kRowCap = 1536;              // LDS candidate slots
constexpr int kRowUnroll = 8;              // loads in flight per thread while streaming
constexpr int kPreF4 = 8;                  // prefetched 16-byte pieces per thread (rows up to 32768)

struct RowLds {
  uint32_t hist[kHistBins];
  uint32_t bitmap[kRowWords];
  uint32_t ckey[kRowCap];
  int32_t cpos[kRowCap];
  uint32_t scan[kRowThreads / 64 + 8];
  uint32_t ccount;
};

__device__ __forceinline__ uint64_t composite(uint32_t key, int32_t p, uint32_t nm1) {
  return ((uint64_t)key << 30) | (uint64_t)(nm1 - (uint32_t)p);
}

// f(key, position) for every position p < n of the row.  16-byte loads, 8 in
// flight per thread, when the row is 16-byte aligned; otherwise 4-byte loads.
template <typename F>
__device__ __forceinline__ void stream_row(const float* __restrict__ sr, int32_t n, F&& f) {
  int32_t done = 0;
  if (((uintptr_t)sr & 15u) == 0) {
    const float4* s4 = reinterpret_cast<const float4*>(sr);
    const int32_t n4 = n >> 2;
    for (int32_t base = 0; base < n4; base += kRowThreads * kRowUnroll) {
      float4 v[kRowUnroll];
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) {
        const int32_t i = base + u * kRowThreads + (int32_t)threadIdx.x;
        v[u] = i < n4 ? s4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) {
        const int32_t i = base + u * kRowThreads + (int32_t)threadIdx.x;
        if (i < n4) {
          f(score_key(v[u].x), 4 * i);
          f(score_key(v[u].y), 4 * i + 1);
          f(score_key(v[u].z), 4 * i + 2);
          f(score_key(v[u].w), 4 * i + 3);
        }
      }
    }
    done = n4 << 2;
  }
  for (int32_t base = done; base < n; base += kRowThreads * kRowUnroll) {
    float v[kRowUnroll];
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int32_t p = base + u * kRowThreads + (int32_t)threadIdx.x;
      v[u] = p < n ? sr[p] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int32_t p = base + u * kRowThreads + (int32_t)threadIdx.x;
      if (p < n) f(score_key(v[u]), p);
    }
  }
}

// stream_row on the float values.
template <typename F>
__device__ __forceinline__ void stream_row_f(const float* __restrict__ sr, int32_t n, F&& f) {
  int32_t done = 0;
  if (((uintptr_t)sr & 15u) == 0) {
    const float4* s4 = reinterpret_cast<const float4*>(sr);
    const int32_t n4 = n >> 2;
    for (int32_t base = 0; base < n4; base += kRowThreads * kRowUnroll) {
      float4 v[kRowUnroll];
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) {
        const int32_t i = base + u * kRowThreads + (int32_t)threadIdx.x;
        v[u] = i < n4 ? s4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) {
        const int32_t i = base + u * kRowThreads + (int32_t)threadIdx.x;
        if (i < n4) {
          f(v[u].x, 4 * i);
          f(v[u].y, 4 * i + 1);
          f(v[u].z, 4 * i + 2);
          f(v[u].w, 4 * i + 3);
        }
      }
    }
    done = n4 << 2;
  }
  for (int32_t base = done; base < n; base += kRowThreads * kRowUnroll) {
    float v[kRowUnroll];
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int32_t p = base + u * kRowThreads + (int32_t)threadIdx.x;
      v[u] = p < n ? sr[p] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int32_t p = base + u * kRowThreads + (int32_t)threadIdx.x;
      if (p < n) f(v[u], p);
    }
  }
}

// The float whose order key (score_key) is k.
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Digit holding the need-th largest member of a histogram of PER * 1024 bins
// ordered by digit value.  Returns the digit, the number of members in higher
// digits and the count of the digit itself (all block-uniform).
template <int PER>
__device__ void row_find_digit(const uint32_t* h, uint32_t need, uint32_t* scan,
                               uint32_t* digit, uint32_t* above, uint32_t* count) {
  const int top = PER * kRowThreads - 1 - (int)threadIdx.x * PER;
  uint32_t c[PER];
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    c[i] = h[top - i];
    s += c[i];
  }
  uint32_t* res = scan + kRowThreads / 64 + 1;
  if (threadIdx.x == 0) {
    res[0] = 0u;
    res[1] = 0u;
    res[2] = 0u;
  }
  uint32_t tot;
  const uint32_t ex = block_excl_scan<kRowThreads>(s, scan, &tot);
  if (ex < need && need <= ex + s) {
    uint32_t acc = ex;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (acc < need && need <= acc + c[i]) {
        res[0] = (uint32_t)(top - i);
        res[1] = acc;
        res[2] = c[i];
      }
      acc += c[i];
    }
  }
  __syncthreads();
  *digit = res[0];
  *above = res[1];
  *count = res[2];
  __syncthreads();
}

// Rows streamed from memory (not held in registers) ask for 8 waves per SIMD
// (the SGPR budget that allows), so that two rows' work-groups share a
// compute unit and one's barriers and loads overlap the other's work.
template <bool kHasHist, bool kPre>
__global__ __launch_bounds__(kRowThreads) __attribute__((amdgpu_waves_per_eu(kPre ? 1 : 8, kPre ? 4 : 8)))
void k_topk_row(const float* __restrict__ scores, int32_t N,
                const int32_t* __restrict__ n_valid, int32_t n_all, int32_t K,
                uint32_t* __restrict__ hist, int32_t zero_hist,
                const int32_t* __restrict__ cand_map, int32_t* __restrict__ out) {
  __shared__ RowLds L;
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t n = row_count(n_valid, n_all, row, N);
  const float* sr = scores + (size_t)row * N;
  const int32_t* mrow = cand_map ? cand_map + (size_t)row * N : nullptr;
  int32_t* orow = out + (size_t)row * K;

  // kPre (rows of at most kPreF4 * 4 * kRowThreads positions, a multiple of
  // 4, 16-byte aligned): the row's loads are issued here, before the
  // histogram is read, and consumed by the collection pass.
  float4 pre[kPre ? kPreF4 : 1];
  if (kPre && n > K) {
    const float4* s4 = reinterpret_cast<const float4*>(sr);
#pragma unroll
    for (int u = 0; u < kPreF4; ++u) {
      const int32_t i = u * kRowThreads + tid;
      pre[u] = 4 * i < n ? s4[i] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  auto visit = [&](auto&& f) { stream_row(sr, n, f); };
  // visit_pre on the float values (the order key is computed by the caller).
  auto visit_pre_f = [&](auto&& f) {
    if (kPre) {
#pragma unroll
      for (int u = 0; u < kPreF4; ++u) {
        const int32_t i = u * kRowThreads + tid;
        if (4 * i + 0 < n) f(pre[u].x, 4 * i + 0);
        if (4 * i + 1 < n) f(pre[u].y, 4 * i + 1);
        if (4 * i + 2 < n) f(pre[u].z, 4 * i + 2);
        if (4 * i + 3 < n) f(pre[u].w, 4 * i + 3);
      }
    } else {
      stream_row_f(sr, n, f);
    }
  };

  auto visit_pre = [&](auto&& f) {
    if (kPre) {
#pragma unroll
      for (int u = 0; u < kPreF4; ++u) {
        const int32_t i = u * kRowThreads + tid;
        if (4 * i + 0 < n) f(score_key(pre[u].x), 4 * i + 0);
        if (4 * i + 1 < n) f(score_key(pre[u].y), 4 * i + 1);
        if (4 * i + 2 < n) f(score_key(pre[u].z), 4 * i + 2);
        if (4 * i + 3 < n) f(score_key(pre[u].w), 4 * i + 3);
      }
    } else {
      stream_row(sr, n, f);
    }
  };

  // 1. Top-digit histogram: bits 61..50 of the composite = the top 12 key bits.
  if (kHasHist) {
    uint32_t* hr = hist + (size_t)row * kHistBins;
    for (int i = tid; i < kHistBins; i += kRowThreads) {
      L.hist[i] = hr[i];
      if (zero_hist) hr[i] = 0u;   // left zeroed for the next score kernel
    }
  }
  if (n <= K) {   // every valid position is selected
    for (int i = tid; i < K; i += kRowThreads) orow[i] = i < n ? (mrow ? mrow[i] : i) : -1;
    return;
  }
  // The first digit: 12 key bits from bit kbit up.  With a histogram from
  // the score kernel, or a row streamed from memory, it is the top 12 bits.
  // For a row held in registers it starts just below the bits that every key
  // of the row shares (the common prefix of its smallest and largest keys,
  // which all keys between them share too), so that the 4096 bins spread over
  // the values the row actually holds instead of the few that share its
  // exponent (fewer same-bin LDS atomics; no extra pass over memory).
  int kbit = 32 - kHistBits;
  uint32_t common = 0u;   // key bits above the first digit
  if (!kHasHist && !kPre) {
    for (int i = tid; i < kHistBins; i += kRowThreads) L.hist[i] = 0u;
    __syncthreads();
    visit_pre([&](uint32_t key, int32_t) {
      atomicAdd(&L.hist[key >> (32 - kHistBits)], 1u);
    });
  } else if (!kHasHist) {
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
    visit_pre([&](uint32_t key, int32_t) {
      kmin = min(kmin, key);
      kmax = max(kmax, key);
    });
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
      kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
    }
    uint32_t* red = L.ckey;   // free until the collection step
    if ((tid & 63) == 0) {
      red[tid >> 6] = kmin;
      red[kRowThreads / 64 + (tid >> 6)] = kmax;
    }
    for (int i = tid; i < kHistBins; i += kRowThreads) L.hist[i] = 0u;
    __syncthreads();
    kmin = red[0];
    kmax = red[kRowThreads / 64];
#pragma unroll
    for (int w = 1; w < kRowThreads / 64; ++w) {
      kmin = min(kmin, red[w]);
      kmax = max(kmax, red[kRowThreads / 64 + w]);
    }
    const uint32_t diff = kmin ^ kmax;
    const int h = diff ? 31 - __builtin_clz(diff) : 0;          // highest bit where keys differ
    kbit = h >= kHistBits - 1 ? h - (kHistBits - 1) : 0;
    common = kbit + kHistBits >= 32 ? 0u : kmax >> (kbit + kHistBits);
    const int kb = kbit;
    visit_pre([&](uint32_t key, int32_t) {
      atomicAdd(&L.hist[(key >> kb) & (kHistBins - 1)], 1u);
    });
  }
  __syncthreads();
  const uint32_t nm1 = (uint32_t)(n - 1);
  uint32_t d, ab, cnt;
  row_find_digit<kHistBins / kRowThreads>(L.hist, (uint32_t)K, L.scan, &d, &ab, &cnt);
  // Invariant: the composites whose bits above `shift` exceed `prefix` are
  // all selected (K - need of them); `need` more come from the `cnt`
  // composites whose bits above `shift` equal `prefix`.
  uint64_t prefix = ((uint64_t)common << kHistBits) | d;
  uint32_t need = (uint32_t)K - ab;
  int shift = 30 + kbit;
  bool all = cnt == need;

  // 2. Refine by streaming passes until the prefix's members fit in LDS.
  //    While the digit lies in the score bits (shift >= 30) every test is a
  //    32-bit compare of the score key.
  while (!all && cnt > (uint32_t)kRowCap && shift > 0) {
    const int w = shift < kRowDigit ? shift : kRowDigit;
    shift -= w;
    for (int i = tid; i < (1 << kRowDigit); i += kRowThreads) L.hist[i] = 0u;
    __syncthreads();
    const int sh = shift;
    const uint32_t mask = (1u << w) - 1u;
    if (sh >= 30) {
      const int ks = sh - 30;
      const uint32_t pre = (uint32_t)prefix;
      visit([&](uint32_t key, int32_t) {
        if ((key >> (ks + w)) == pre) atomicAdd(&L.hist[(key >> ks) & mask], 1u);
      });
    } else {
      visit([&](uint32_t key, int32_t p) {
        const uint64_t c = composite(key, p, nm1);
        if ((c >> (sh + w)) == prefix) atomicAdd(&L.hist[(uint32_t)(c >> sh) & mask], 1u);
      });
    }
    __syncthreads();
    row_find_digit<(1 << kRowDigit) / kRowThreads>(L.hist, need, L.scan, &d, &ab, &cnt);
    prefix = (prefix << w) | d;
    need -= ab;
    all = cnt == need;
  }

  // 3. Mark everything above the prefix; copy the prefix's members to LDS.
  for (int i = tid; i < ((n + 31) >> 5); i += kRowThreads) L.bitmap[i] = 0u;
  if (tid == 0) L.ccount = 0u;
  __syncthreads();
  {
    const int sh = shift;
    const bool take_eq = all;
    auto hit = [&](uint32_t key, int32_t p, bool above, bool equal) {
      if (above || (take_eq && equal)) {
        atomicOr(&L.bitmap[p >> 5], 1u << (p & 31));
      } else if (equal) {
        const uint32_t slot = atomicAdd(&L.ccount, 1u);
        if (slot < (uint32_t)kRowCap) {
          L.ckey[slot] = key;
          L.cpos[slot] = p;
        }
      }
    };
    // The prefix lies in the score bits: with lo / hi the floats whose order
    // keys are prefix << ks and (prefix + 1) << ks, a score is above the
    // prefix iff s >= hi and inside it iff lo <= s < hi (order keys are
    // monotone in the real value), so most elements cost two compares.  The
    // lowest keys (-inf and below) have no float bound (their pattern is a
    // NaN): there the keys themselves are compared.
    bool fast = sh >= 30;
    bool top = false;
    float flo = 0.f, fhi = 0.f;
    if (fast) {
      const int ks = sh - 30;
      const uint32_t pre = (uint32_t)prefix;
      const uint32_t klo = pre << ks;
      top = (ks == 0) ? (pre == 0xFFFFFFFFu) : ((pre + 1u) >> (32 - ks)) != 0u;
      const uint32_t khi = top ? 0xFFFFFFFFu : (pre + 1u) << ks;
      flo = key_float(klo);
      fhi = key_float(khi);
      fast = !__builtin_isnan(flo) && (top || !__builtin_isnan(fhi));
    }
    if (fast) {
      visit_pre_f([&](float s, int32_t p) {
        if (s >= flo) {
          const bool above = !top && s >= fhi;
          hit(score_key(s), p, above, !above);
        }
      });
    } else {
      visit_pre([&](uint32_t key, int32_t p) {
        const uint64_t hi = composite(key, p, nm1) >> sh;
        if (hi >= prefix) hit(key, p, hi > prefix, hi == prefix);
      });
    }
  }
  __syncthreads();

  // 4. Radix passes over the LDS members, then mark the chosen ones.
  if (!all) {
    const uint32_t C = L.ccount;   // == cnt <= kRowCap
    while (!all && shift > 0) {
      const int w = shift < kRowDigit ? shift : kRowDigit;
      shift -= w;
      for (int i = tid; i < (1 << kRowDigit); i += kRowThreads) L.hist[i] = 0u;
      __syncthreads();
      for (uint32_t i = tid; i < C; i += kRowThreads) {
        const uint64_t c = composite(L.ckey[i], L.cpos[i], nm1);
        if ((c >> (shift + w)) == prefix)
          atomicAdd(&L.hist[(uint32_t)(c >> shift) & ((1u << w) - 1u)], 1u);
      }
      __syncthreads();
      row_find_digit<(1 << kRowDigit) / kRowThreads>(L.hist, need, L.scan, &d, &ab, &cnt);
      prefix = (prefix << w) | d;
      need -= ab;
      all = cnt == need;
    }
    for (uint32_t i = tid; i < C; i += kRowThreads) {
      const int32_t p = L.cpos[i];
      if ((composite(L.ckey[i], p, nm1) >> shift) >= prefix)
        atomicOr(&L.bitmap[p >> 5], 1u << (p & 31));
    }
    __syncthreads();
  }

  // 5. Ascending output through the bitmap.  The loop that writes positions
  //    holds no loads (a load feeding a store in the same loop makes every
  //    store wait for all earlier memory operations).  Up to 2 * kRowCap
  //    positions go to LDS first and are written (mapped) with coalesced
  //    stores afterwards.
  // The ceil(n / 32) bitmap words in use are spread evenly over the threads
  // (one word each for rows up to 32768), so that the per-bit loops below
  // run on every wave instead of a few.
  constexpr int WPT = kRowWords / kRowThreads;   // at most 8 words per thread
  const int nwords = (n + 31) >> 5;
  const int wpt = (nwords + kRowThreads - 1) / kRowThreads;
  uint32_t wv[WPT];
  uint32_t c = 0;
#pragma unroll
  for (int w = 0; w < WPT; ++w) {
    const int wi = tid * wpt + w;
    wv[w] = (w < wpt && wi < nwords) ? L.bitmap[wi] : 0u;
    c += __popc(wv[w]);
  }
  uint32_t tot;
  const uint32_t pos0 = block_excl_scan<kRowThreads>(c, L.scan, &tot);
  int32_t* opos = reinterpret_cast<int32_t*>(L.ckey);   // ckey and cpos: 2 * kRowCap ints
  const bool staged = K <= 2 * kRowCap;
  uint32_t pos = pos0;
#pragma unroll
  for (int w = 0; w < WPT; ++w) {
    uint32_t m = wv[w];
    while (m) {
      const int bit = __ffs(m) - 1;
      m &= m - 1;
      const int32_t p = (tid * wpt + w) * 32 + bit;
      if (pos < (uint32_t)K) {
        if (staged) opos[pos] = p;
        else if (!mrow) orow[pos] = p;
      }
      ++pos;
    }
  }
  if (staged) {   // coalesced stores (scattered 4-byte stores issue slowly)
    __syncthreads();
    if (mrow)
      for (uint32_t i = tid; i < (uint32_t)K; i += kRowThreads) orow[i] = i < tot ? mrow[opos[i]] : -1;
    else
      for (uint32_t i = tid; i < (uint32_t)K; i += kRowThreads) orow[i] = i < tot ? opos[i] : -1;
    return;
  }
  if (mrow) {   // K > 2 * kRowCap with a map: direct mapped stores
    pos = pos0;
#pragma unroll
    for (int w = 0; w < WPT; ++w) {
      uint32_t m = wv[w];
      while (m) {
        const int bit = __ffs(m) - 1;
        m &= m - 1;
        const int32_t p = (tid * wpt + w) * 32 + bit;
        if (pos < (uint32_t)K) orow[pos] = mrow[p];
        ++pos;
      }
    }
  }
  for (uint32_t i = tot + tid; i < (uint32_t)K; i += kRowThreads) orow[i] = -1;
}

// ---------------------------------------------------------------------------
// Sliced select: a row is cut into slices of kFinalThreads * PT positions;
// one work-group per slice keeps a superset of the slice's Top-K
// (k_topk_slice) and one work-group per row selects the row's Top-K from the
// slices' keepers (k_topk_final).  A slice's Top-K under the (key, lower
// position) order holds every element of the row's Top-K that lies in the
// slice (an element the slice drops has K better ones in the slice alone), so
// the union of the slices' keepers holds the row's Top-K.  A slice keeps
// everything at or above the radix digit that holds its K-th key, as long as
// that fits its topk_slot_count(K) slots (one radix pass, usually), otherwise
// it refines as the exact select does.  Rows of at most kFinalMaxN positions
// go to k_topk_final directly.
//
// Both levels run one block select.  Elements are loaded with coalesced
// 16-byte loads: thread t holds G = PT / 4 groups of 4, group u covering the
// block's positions 4096 u + 4 t .. 4096 u + 4 t + 3, so the block's
// position order is (group, thread, element); the kept elements leave in
// that order through one block scan of per-group counts (packed two to a
// word).  Work-groups are 1024 threads: with one wave per SIMD every
// dependent step of these short phases waits its full latency (measured: an
// LDS clear and barrier take 437 ns on 256 threads, 120 ns on 1024).  Every
// phase ends in one barrier: the histogram is double-buffered (a pass clears
// the other buffer) and the scans and digit searches rotate their LDS slots.
// ---------------------------------------------------------------------------

constexpr int kFinalThreads = 1024;
constexpr int kSelNW = kFinalThreads / 64;

// LDS of the block select on NT threads.  A scan slot holds every wave's
// packed group counts: NT / 64 waves x (PT / 8) words, at most 32 words for
// the NT x PT <= 16384 elements a block selects from.
template <int NT>
struct BlockSelLdsT {
  alignas(16) uint32_t hist[2][kHistBins];   // double-buffered histogram; output staging afterwards
  uint32_t scan[4][32];                      // rotating scan slots
  uint32_t res[4][4];                        // rotating digit-search results
  uint32_t red[3][NT / 64];                  // count, min, max per wave
};
using BlockSelLds = BlockSelLdsT<kFinalThreads>;

__device__ __forceinline__ uint32_t key_hi(uint32_t k, int sh) { return sh >= 32 ? 0u : k >> sh; }

// Zero a 4096-bin LDS histogram (16-byte aligned) with NT threads, 16 bytes
// per store.
template <int NT>
__device__ __forceinline__ void clear_hist(uint32_t* h) {
  static_assert(kHistBins % (4 * NT) == 0, "whole 16-byte stores per thread");
#pragma unroll
  for (int i = 0; i < kHistBins / (4 * NT); ++i)
    reinterpret_cast<uint4*>(h)[threadIdx.x + NT * i] = make_uint4(0u, 0u, 0u, 0u);
}

// Sum, minimum and maximum over the 64 lanes of a wave, in lane 63: DPP row
// shifts within each row of 16, then the row results added with readlane.
struct Wred {
  uint32_t sum, mn, mx;
};
template <int CTRL>
__device__ __forceinline__ void wred_step(uint32_t& s, uint32_t& mn, uint32_t& mx) {
  // a lane with no source in its row reads the identity (0 for the sum and
  // the maximum, all ones for the minimum)
  s += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s, CTRL, 0xF, 0xF, true);
  mn = min(mn, (uint32_t)__builtin_amdgcn_update_dpp((int)0xFFFFFFFFu, (int)mn, CTRL, 0xF, 0xF, false));
  mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ Wred wave_reduce3(uint32_t s, uint32_t mn, uint32_t mx) {
  wred_step<0x111>(s, mn, mx);   // row_shr:1
  wred_step<0x112>(s, mn, mx);   // row_shr:2
  wred_step<0x114>(s, mn, mx);   // row_shr:4
  wred_step<0x118>(s, mn, mx);   // row_shr:8
  Wred r;
  r.sum = (uint32_t)__builtin_amdgcn_readlane((int)s, 15) + (uint32_t)__builtin_amdgcn_readlane((int)s, 31) +
          (uint32_t)__builtin_amdgcn_readlane((int)s, 47) + (uint32_t)__builtin_amdgcn_readlane((int)s, 63);
  r.mn = min(min((uint32_t)__builtin_amdgcn_readlane((int)mn, 15), (uint32_t)__builtin_amdgcn_readlane((int)mn, 31)),
             min((uint32_t)__builtin_amdgcn_readlane((int)mn, 47), (uint32_t)__builtin_amdgcn_readlane((int)mn, 63)));
  r.mx = max(max((uint32_t)__builtin_amdgcn_readlane((int)mx, 15), (uint32_t)__builtin_amdgcn_readlane((int)mx, 31)),
             max((uint32_t)__builtin_amdgcn_readlane((int)mx, 47), (uint32_t)__builtin_amdgcn_readlane((int)mx, 63)));
  return r;
}

// Exclusive prefix (in position order) and total of G per-group counts
// (each < 2^16) over the block: fields of 16 bits, two groups to a word,
// scanned together; one barrier.  `slot` must not have been used by the
// previous three calls.
template <int NT, int G>
__device__ void scan_groups(const uint32_t (&c)[G], uint32_t* slot, uint32_t (&pre)[G],
                            uint32_t (&tot)[G]) {
  constexpr int W = (G + 1) / 2;
  constexpr int NW = NT / 64;
  const int wave = threadIdx.x >> 6;
  uint32_t v[W], x[W];
#pragma unroll
  for (int w = 0; w < W; ++w) {
    v[w] = c[2 * w] | (2 * w + 1 < G ? c[2 * w + 1] << 16 : 0u);
    x[w] = wave_incl_scan(v[w]);
    slot[wave * W + w] = (uint32_t)__builtin_amdgcn_readlane((int)x[w], 63);   // every lane
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < W; ++w) {
    uint32_t before, all;
    wave_prefix<NW>(slot + w, W, &before, &all);
    const uint32_t ex = before + x[w] - v[w];
    pre[2 * w] = ex & 0xFFFFu;
    tot[2 * w] = all & 0xFFFFu;
    if (2 * w + 1 < G) {
      pre[2 * w + 1] = ex >> 16;
      tot[2 * w + 1] = all >> 16;
    }
  }
}

// Digit holding the need-th largest of the 2^w bins (counted from the top):
// the digit, the count above it and its own count (block-uniform); two
// barriers, `slot` / `rs` as in scan_groups.
template <int NT>
__device__ void find_digit_c(const uint32_t (&c)[kHistBins / NT], int top, uint32_t need,
                             uint32_t* slot, uint32_t* rs, uint32_t* digit, uint32_t* above,
                             uint32_t* count);

template <int NT>
__device__ void find_digit(const uint32_t* h, int w, uint32_t need, uint32_t* slot, uint32_t* rs,
                           uint32_t* digit, uint32_t* above, uint32_t* count) {
  constexpr int kPer = kHistBins / NT;                // bins per thread at most
  const int nb = 1 << w;
  const int per = (nb + NT - 1) / NT;
  const int top = nb - 1 - (int)threadIdx.x * per;    // thread 0 owns the highest bins
  uint32_t c[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) c[i] = (i < per && top - i >= 0) ? h[top - i] : 0u;
  find_digit_c<NT>(c, top, need, slot, rs, digit, above, count);
}

// find_digit on this thread's bins in registers: c[i] is bin top - i (0 past
// the thread's share or below bin 0).
template <int NT>
__device__ void find_digit_c(const uint32_t (&c)[kHistBins / NT], int top, uint32_t need,
                             uint32_t* slot, uint32_t* rs, uint32_t* digit, uint32_t* above,
                             uint32_t* count) {
  constexpr int kPer = kHistBins / NT;
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) s += c[i];
  const int wave = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan(s);
  slot[wave] = (uint32_t)__builtin_amdgcn_readlane((int)x, 63);   // every lane: no branch
  __syncthreads();
  uint32_t before, all;
  wave_prefix<NT / 64>(slot, 1, &before, &all);
  const uint32_t ex = before + x - s;
  // the bin holding the need-th count (selects; one lane stores)
  uint32_t acc = ex, fd = 0u, fa = 0u, fc = 0u;
  bool hit = false;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const bool hi = acc < need && need <= acc + c[i];
    fd = hi ? (uint32_t)(top - i) : fd;
    fa = hi ? acc : fa;
    fc = hi ? c[i] : fc;
    hit = hit || hi;
    acc += c[i];
  }
  if (hit) {
    rs[0] = fd;
    rs[1] = fa;
    rs[2] = fc;
  }
  __syncthreads();
  *digit = rs[0];
  *above = rs[1];
  *count = rs[2];
}

// The K largest of the block's elements (key 0: absent; no score maps to it),
// equal keys going to the earlier element in position order, or a superset
// of them: at most `budget` (>= K) elements, all those at or above the radix
// digit that holds the K-th key once that group fits the budget.  sel[i] is
// set for the kept elements of this thread; returns how many are kept
// (min(K, present) when budget == K).  `round` counts the rotating slots used.
template <int NT, int PT>
__device__ uint32_t block_select(const uint32_t (&key)[PT], uint32_t K, uint32_t budget,
                                 BlockSelLdsT<NT>& L, bool (&sel)[PT], int& round) {
  constexpr int G = PT / 4;
  constexpr int NW = NT / 64;
  static_assert(NW * ((G + 1) / 2) <= 32, "the group scan fits a 32-word slot");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t cnt = 0, kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    if (key[i]) {
      ++cnt;
      kmin = min(kmin, key[i]);
      kmax = max(kmax, key[i]);
    }
  }
  const Wred wr = wave_reduce3(cnt, kmin, kmax);
  L.red[0][wave] = wr.sum;   // wave-uniform values, every lane stores
  L.red[1][wave] = wr.mn;
  L.red[2][wave] = wr.mx;
  clear_hist<NT>(L.hist[0]);
  __syncthreads();
  // the block's count, minimum and maximum: lane k takes wave k's values
  uint32_t tot, rs = 0u, rn = 0xFFFFFFFFu, rx = 0u;
  {
    const int k = lane < NW ? lane : 0;
    rs = lane < NW ? L.red[0][k] : 0u;
    rn = lane < NW ? L.red[1][k] : 0xFFFFFFFFu;
    rx = lane < NW ? L.red[2][k] : 0u;
    wred_step<0x111>(rs, rn, rx);
    wred_step<0x112>(rs, rn, rx);
    wred_step<0x114>(rs, rn, rx);
    wred_step<0x118>(rs, rn, rx);
    tot = (uint32_t)__builtin_amdgcn_readlane((int)rs, NW - 1);
    kmin = (uint32_t)__builtin_amdgcn_readlane((int)rn, NW - 1);
    kmax = (uint32_t)__builtin_amdgcn_readlane((int)rx, NW - 1);
  }
  if (tot <= budget) {
#pragma unroll
    for (int i = 0; i < PT; ++i) sel[i] = key[i] != 0u;
    return tot;
  }
  // bits at and above `shift` are fixed in `prefix`; every present key shares
  // the bits above the highest one where kmin and kmax differ
  const uint32_t diff = kmin ^ kmax;
  int shift = diff ? 32 - __builtin_clz(diff) : 0;
  uint32_t prefix = key_hi(kmax, shift);
  uint32_t need = K;
  uint32_t group = tot;   // elements matching the prefix
  bool all = false;       // every element matching the prefix is kept
  int buf = 0;
  while (shift > 0) {
    const int w = shift < kHistBits ? shift : kHistBits;
    const int sh = shift - w;
    const uint32_t mask = (1u << w) - 1u;
    uint32_t* h = L.hist[buf];
#pragma unroll
    for (int i = 0; i < PT; ++i)
      if (key[i] && key_hi(key[i], shift) == prefix) atomicAdd(&h[(key[i] >> sh) & mask], 1u);
    clear_hist<NT>(L.hist[buf ^ 1]);
    __syncthreads();
    uint32_t d, ab, c;
    find_digit<NT>(h, w, need, L.scan[round & 3], L.res[round & 3], &d, &ab, &c);
    ++round;
    buf ^= 1;
    prefix = (prefix << w) | d;
    need -= ab;
    group = c;
    shift = sh;
    if (K - need + c <= budget) {   // (budget == K: exactly when the group is needed whole)
      all = true;
      break;
    }
  }
  // above the prefix: kept; equal to it: kept when the group fits, otherwise
  // (equal keys) the earliest `need` of them in position order
  bool eq[PT];
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const uint32_t hk = key_hi(key[i], shift);
    eq[i] = key[i] && hk == prefix;
    sel[i] = key[i] && hk > prefix;
  }
  if (all) {
#pragma unroll
    for (int i = 0; i < PT; ++i) sel[i] = sel[i] || eq[i];
    return K - need + group;
  }
  uint32_t tc[G], pre[G], gt[G];
#pragma unroll
  for (int u = 0; u < G; ++u) {
    tc[u] = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) tc[u] += eq[4 * u + j] ? 1u : 0u;
  }
  scan_groups<NT, G>(tc, L.scan[round & 3], pre, gt);
  ++round;
  uint32_t before = 0;
#pragma unroll
  for (int u = 0; u < G; ++u) {
    uint32_t rank = before + pre[u];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (eq[4 * u + j]) {
        sel[4 * u + j] = rank < need;
        ++rank;
      }
    }
    before += gt[u];
  }
  return K;
}

// Output index (in position order) of each kept element of this thread: one
// scan of the per-group kept counts.
template <int NT, int PT>
__device__ void kept_order(const bool (&sel)[PT], BlockSelLdsT<NT>& L, int& round, uint32_t (&oidx)[PT]) {
  constexpr int G = PT / 4;
  uint32_t kc[G], pre[G], gt[G];
#pragma unroll
  for (int u = 0; u < G; ++u) {
    kc[u] = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) kc[u] += sel[4 * u + j] ? 1u : 0u;
  }
  scan_groups<NT, G>(kc, L.scan[round & 3], pre, gt);
  ++round;
  uint32_t before = 0;
#pragma unroll
  for (int u = 0; u < G; ++u) {
    uint32_t o = before + pre[u];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      oidx[4 * u + j] = o;
      o += sel[4 * u + j] ? 1u : 0u;
    }
    before += gt[u];
  }
}

// Slice s of row r (positions s * 1024 PT ..): a superset of its K largest
// keys (at most `slots`), keys and positions in ascending position order, then
// key 0 up to `slots` (slots [r][s][0 .. slots)).
template <int NT, int PT>
__global__ __launch_bounds__(NT)
void k_topk_slice(const float* __restrict__ scores, int32_t N, const int32_t* __restrict__ n_valid,
                  int32_t n_all, int32_t K, int32_t slots, uint32_t* __restrict__ ckey,
                  int32_t* __restrict__ cpos) {
  constexpr int G = PT / 4;
  constexpr int GS = 4 * NT;   // positions per element group
  __shared__ BlockSelLdsT<NT> L;
  const int row = blockIdx.y, s = blockIdx.x;
  const int32_t n = row_count(n_valid, n_all, row, N);
  const int32_t b0 = s * (NT * PT) + 4 * (int32_t)threadIdx.x;   // group 0's first position
  const float* sr = scores + (size_t)row * N;
  uint32_t key[PT];
  const bool vec = (N & 3) == 0 && ((uintptr_t)scores & 15u) == 0;
#pragma unroll
  for (int u = 0; u < G; ++u) {
    const int32_t p = b0 + GS * u;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (vec) {
      if (p < n) v = *reinterpret_cast<const float4*>(sr + p);   // p + 3 < N: N is a multiple of 4
    } else {
      v.x = p < n ? sr[p] : 0.f;
      v.y = p + 1 < n ? sr[p + 1] : 0.f;
      v.z = p + 2 < n ? sr[p + 2] : 0.f;
      v.w = p + 3 < n ? sr[p + 3] : 0.f;
    }
    key[4 * u + 0] = p + 0 < n ? score_key(v.x) : 0u;
    key[4 * u + 1] = p + 1 < n ? score_key(v.y) : 0u;
    key[4 * u + 2] = p + 2 < n ? score_key(v.z) : 0u;
    key[4 * u + 3] = p + 3 < n ? score_key(v.w) : 0u;
  }
  bool sel[PT];
  int round = 0;
  const uint32_t kept = block_select<NT, PT>(key, (uint32_t)K, (uint32_t)slots, L, sel, round);
  uint32_t oidx[PT];
  kept_order<NT, PT>(sel, L, round, oidx);
  const size_t base = ((size_t)row * gridDim.x + s) * slots;
  // the keepers go out through LDS (coalesced stores) when they fit the
  // histogram buffers, which the select no longer needs
  const bool staged = 2 * kept <= 2 * kHistBins;
  uint32_t* sk = &L.hist[0][0];
  int32_t* sp = reinterpret_cast<int32_t*>(sk + kept);
#pragma unroll
  for (int u = 0; u < G; ++u)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 4 * u + j;
      if (sel[i]) {
        if (staged) {
          sk[oidx[i]] = key[i];
          sp[oidx[i]] = b0 + GS * u + j;
        } else {
          ckey[base + oidx[i]] = key[i];
          cpos[base + oidx[i]] = b0 + GS * u + j;
        }
      }
    }
  if (staged) {
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < kept; i += NT) {
      ckey[base + i] = sk[i];
      cpos[base + i] = sp[i];
    }
  }
  for (uint32_t i = kept + threadIdx.x; i < (uint32_t)slots; i += NT) ckey[base + i] = 0u;
}

// Fused score -> Top-K (flat rows): work-group (s, r) scores slice s of row
// r (entries 4096 s .. 4096 s + 4095, one query row per sequence) straight
// into LDS and keeps that slice's superset of its K largest, as k_topk_slice
// does from scores in memory; k_topk_final then selects the row's Top-K from
// the keepers.  The scores never go to memory, and the slice select's launch
// and its read of them go away.  16 waves of 256 entries each, streamed as
// the scan kernel streams them (same lanes, same arithmetic: the same float
// for every entry), with batches of kFusedUnroll loads per lane, the next
// batch in flight while one is scored.
constexpr int kFusedSlice = kScoreSlice;                  // entries per work-group
static_assert(kFusedSlice == 4 * kFinalThreads, "a fused slice is one element group");
constexpr int kFusedEPW = kFusedSlice / (kFinalThreads / 64);   // 256 per wave
constexpr int kFusedUnroll = 8;

__global__ __launch_bounds__(kFinalThreads)
void k_score_slice(const uint8_t* __restrict__ key, int64_t M, const uint8_t* __restrict__ q_idx,
                   const float* __restrict__ w_idx, const int32_t* __restrict__ len, PoolMap map,
                   int32_t K, int32_t slots, uint32_t* __restrict__ ckey,
                   int32_t* __restrict__ cpos) {
  __shared__ BlockSelLds L;
  __shared__ __attribute__((aligned(16))) uint32_t sk[kFusedSlice];   // order keys, 0: absent
  const int row = blockIdx.y, s = blockIdx.x;
  const int b = row;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, sub = lane & 31, head = sub >> 2;
  const int64_t vis = len ? (int64_t)len[b] : M;
  const int64_t g0 = (int64_t)s * kFusedSlice;
  const int wofs = wave * kFusedEPW;

  float qf[16];
  const uint8_t* qsrc = q_idx + (size_t)row * kKeyRow + sub * 16;
  load_q_slice(qsrc, qf);
  const float wh = w_idx[(size_t)row * kHI + head];
  const uint8_t* kb = key + sub * 16;

  constexpr int kBatch = 2 * kFusedUnroll;                  // entries per batch of a wave
  constexpr int kIters = kFusedEPW / kBatch;
  u32x4 v[2][kFusedUnroll];
  bool ok[2][kFusedUnroll];
  auto issue = [&](int it, int bi) __attribute__((always_inline)) {
    const int64_t p0 = g0 + wofs + it * kBatch;
    // a batch's 16 entries lie in one page (pages hold >= 64 entries)
    const int64_t roff = map.pages ? (p0 < vis ? pool_row(map, b, p0, M) : 0) - p0
                                   : (int64_t)b * M;
#pragma unroll
    for (int u = 0; u < kFusedUnroll; ++u) {
      const int64_t p = p0 + 2 * u + half;
      const bool valid = p < vis;
      ok[bi][u] = valid;
      // absent entries read the query row (their key is 0 whatever they hold)
      const uint8_t* src = valid ? kb + (roff + p) * kKeyRow : qsrc;
      v[bi][u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
    }
  };
  issue(0, 0);
#pragma unroll 2
  for (int it = 0; it < kIters; ++it) {
    const int cb = it & 1;
    if (it + 1 < kIters) issue(it + 1, cb ^ 1);
    __builtin_amdgcn_sched_barrier(0);     // the next batch issues before this one is used
#pragma unroll
    for (int u = 0; u < kFusedUnroll; ++u) {
      const float r = entry_score(v[cb][u], qf, wh);
      if (sub == 0) sk[wofs + it * kBatch + 2 * u + half] = ok[cb][u] ? score_key(r) : 0u;
    }
  }
  __syncthreads();

  // thread t: slice positions 4 t .. 4 t + 3 (group 0 of k_topk_slice<4>)
  const u32x4 kv = *reinterpret_cast<const u32x4*>(&sk[4 * threadIdx.x]);
  uint32_t keyv[4] = {kv[0], kv[1], kv[2], kv[3]};
  bool sel[4];
  int round = 0;
  const uint32_t kept = block_select<kFinalThreads, 4>(keyv, (uint32_t)K, (uint32_t)slots, L, sel, round);
  uint32_t oidx[4];
  kept_order<kFinalThreads, 4>(sel, L, round, oidx);
  const size_t base = ((size_t)row * gridDim.x + s) * slots;
  const int32_t b0 = s * kFusedSlice + 4 * (int32_t)threadIdx.x;
  // the keepers go out through LDS (coalesced stores): the slice's own keys
  // are no longer needed
  __syncthreads();
  int32_t* sp = reinterpret_cast<int32_t*>(&L.hist[0][0]);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (sel[j]) {
      sk[oidx[j]] = keyv[j];
      sp[oidx[j]] = b0 + j;
    }
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < kept; i += kFinalThreads) {
    ckey[base + i] = sk[i];
    cpos[base + i] = sp[i];
  }
  for (uint32_t i = kept + threadIdx.x; i < (uint32_t)slots; i += kFinalThreads) ckey[base + i] = 0u;
}

// Row r's Top-K as ascending entries (through cand when given), -1 padded.
// Elements: `total` slots of keepers (ckey / cpos from k_topk_slice, in
// position order, total a multiple of 4) or, with total == 0, the row's own
// scores (N <= NT * PT).
// (8 waves per SIMD: with more than about 100 SGPRs a SIMD holds 7 waves and
// a compute unit only one 1024-thread work-group)
template <int NT, int PT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(8, 8)))
void k_topk_final(const float* __restrict__ scores, int32_t N, const int32_t* __restrict__ n_valid,
                  int32_t n_all, int32_t total, const uint32_t* __restrict__ ckey,
                  const int32_t* __restrict__ cpos, int32_t K, const int32_t* __restrict__ cand_map,
                  int32_t* __restrict__ out) {
  constexpr int G = PT / 4;
  constexpr int GS = 4 * NT;   // positions per element group
  __shared__ BlockSelLdsT<NT> L;
  const int row = blockIdx.x;
  const int32_t b0 = 4 * (int32_t)threadIdx.x;
  uint32_t key[PT];
  int32_t pos[PT];
  if (total == 0) {
    // the row's own scores; with a candidate list, each element's entry
    // number comes in with its score (no lookup after the select)
    const int32_t n = row_count(n_valid, n_all, row, N);
    const float* sr = scores + (size_t)row * N;
    const int32_t* mr = cand_map ? cand_map + (size_t)row * N : nullptr;
    const bool vec = (N & 3) == 0 && ((uintptr_t)scores & 15u) == 0 &&
                     ((uintptr_t)cand_map & 15u) == 0;
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int32_t p = b0 + GS * u;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      int4 m = make_int4(p, p + 1, p + 2, p + 3);
      if (vec) {
        if (p < n) {
          v = *reinterpret_cast<const float4*>(sr + p);
          if (mr) m = *reinterpret_cast<const int4*>(mr + p);
        }
      } else {
        v.x = p < n ? sr[p] : 0.f;
        v.y = p + 1 < n ? sr[p + 1] : 0.f;
        v.z = p + 2 < n ? sr[p + 2] : 0.f;
        v.w = p + 3 < n ? sr[p + 3] : 0.f;
        if (mr) {
          m.x = p < n ? mr[p] : 0;
          m.y = p + 1 < n ? mr[p + 1] : 0;
          m.z = p + 2 < n ? mr[p + 2] : 0;
          m.w = p + 3 < n ? mr[p + 3] : 0;
        }
      }
      key[4 * u + 0] = p + 0 < n ? score_key(v.x) : 0u;
      key[4 * u + 1] = p + 1 < n ? score_key(v.y) : 0u;
      key[4 * u + 2] = p + 2 < n ? score_key(v.z) : 0u;
      key[4 * u + 3] = p + 3 < n ? score_key(v.w) : 0u;
      pos[4 * u + 0] = m.x;
      pos[4 * u + 1] = m.y;
      pos[4 * u + 2] = m.z;
      pos[4 * u + 3] = m.w;
    }
  } else {
    const uint32_t* kr = ckey + (size_t)row * total;
    const int32_t* pr = cpos + (size_t)row * total;
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int32_t e = b0 + GS * u;
      u32x4 kv = {0u, 0u, 0u, 0u};
      u32x4 pv = {0u, 0u, 0u, 0u};
      if (e < total) {   // total is a multiple of 4
        kv = *reinterpret_cast<const u32x4*>(kr + e);
        pv = *reinterpret_cast<const u32x4*>(pr + e);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        key[4 * u + j] = kv[j];
        pos[4 * u + j] = (int32_t)pv[j];
      }
    }
  }
  bool sel[PT];
  int round = 0;
  const uint32_t chosen = block_select<NT, PT>(key, (uint32_t)K, (uint32_t)K, L, sel, round);
  uint32_t oidx[PT];
  kept_order<NT, PT>(sel, L, round, oidx);
  int32_t* orow = out + (size_t)row * K;
  // keepers' positions still go through the candidate list (the row's own
  // elements carry their entry numbers already)
  const int32_t* mrow = cand_map && total > 0 ? cand_map + (size_t)row * N : nullptr;
  // positions go out through LDS (coalesced stores, and the map lookups of a
  // candidate list one per thread) when they fit the histogram buffers
  const bool staged = chosen <= 2 * kHistBins;
  int32_t* sp = reinterpret_cast<int32_t*>(&L.hist[0][0]);
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    if (sel[i]) {
      if (staged) sp[oidx[i]] = pos[i];
      else orow[oidx[i]] = mrow ? mrow[pos[i]] : pos[i];
    }
  }
  if (staged) {
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < chosen; i += NT) {
      const int32_t p = sp[i];
      orow[i] = mrow ? mrow[p] : p;
    }
  }
  for (uint32_t i = chosen + threadIdx.x; i < (uint32_t)K; i += NT) orow[i] = -1;
}

// ---------------------------------------------------------------------------
// Group select for many long rows whose scores come with the maximum of every
// run of 16 positions (the chunked-prefill score kernel writes both).  Take
// the K best runs under the (run maximum, lower run) order: every position of
// the row's Top-K lies in one of them.  (An entry x in any other run rho has
// K runs each better than rho; each one's maximum beats x under the (score,
// lower position) order, by a larger score or, at an equal score, by lying in
// an earlier run, so x has K better entries.)  Any set of runs that holds
// those K, such as every run whose maximum reaches some bound, serves as well.
// One 512-thread work-group per row (K <= 512):
//  1. a block select over the run maxima (in run order) marks the K best
//     runs, or, when that takes fewer radix passes, every run at or above a
//     digit boundary as long as they are at most 512; a run holding no
//     visible position takes no part;
//  2. the marked runs are listed in LDS in ascending order by one block scan;
//  3. their positions (at most 8192), in ascending order, are the elements of
//     a block select of the row's K largest under the (key, lower position)
//     order, written out ascending as the final select does.
// ---------------------------------------------------------------------------
constexpr int kRunLen = 16;                              // positions per run
constexpr int kGroupThreads = 512;
constexpr int kGroupPT = 16;                             // gathered positions per thread
constexpr int kGroupRuns = kGroupThreads * kGroupPT / kRunLen;   // runs one work-group gathers (512)

// (512-thread work-groups at 8 waves per SIMD, as the register budgets then
// allow: four rows share a compute unit, and one's loads and barriers
// overlap the others' work)
template <int PG>
__global__ __launch_bounds__(kGroupThreads) __attribute__((amdgpu_waves_per_eu(8, 8)))
void k_topk_group(const float* __restrict__ scores, int32_t N, const float* __restrict__ gmax,
                  const int32_t* __restrict__ n_valid, int32_t n_all, int32_t K,
                  int32_t* __restrict__ out) {
  constexpr int NT = kGroupThreads;
  constexpr int GG = PG / 4;
  constexpr int PT = kGroupPT;
  constexpr int GT = PT / 4;
  __shared__ BlockSelLdsT<NT> L;
  __shared__ int32_t runs[kGroupRuns];
  // rows 4 k .. 4 k + 3 share the 128-byte lines of run maxima: with R a
  // multiple of 32 they go to work-groups w, w + 8, w + 16, w + 24, which the
  // dispatch places on one XCD
  const int R = gridDim.x, w = blockIdx.x;
  const int row = (R & 31) ? w : 32 * (w >> 5) + 4 * (w & 7) + ((w >> 3) & 3);
  const int tid = threadIdx.x;
  const int32_t n = row_count(n_valid, n_all, row, N);
  const int32_t nr = (n + kRunLen - 1) / kRunLen;        // runs holding a visible position

  // 1. run maxima, run r = 4 NT u + 4 tid + j at [r / 8][row][r % 8]
  uint32_t rk[PG];
#pragma unroll
  for (int u = 0; u < GG; ++u) {
    const int32_t r = 4 * NT * u + 4 * tid;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r < nr) v = *reinterpret_cast<const float4*>(gmax + ((size_t)(r >> 3) * R + row) * 8 + (r & 7));
    rk[4 * u + 0] = r + 0 < nr ? score_key(v.x) : 0u;
    rk[4 * u + 1] = r + 1 < nr ? score_key(v.y) : 0u;
    rk[4 * u + 2] = r + 2 < nr ? score_key(v.z) : 0u;
    rk[4 * u + 3] = r + 3 < nr ? score_key(v.w) : 0u;
  }
  bool top[PG];
  int round = 0;
  block_select<NT, PG>(rk, (uint32_t)K, (uint32_t)kGroupRuns, L, top, round);

  // 2. the marked runs (at most kGroupRuns: the select keeps at most its
  //    budget), listed in ascending order
  uint32_t c[GG], pre[GG], tot[GG];
#pragma unroll
  for (int u = 0; u < GG; ++u) {
    c[u] = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) c[u] += top[4 * u + j] ? 1u : 0u;
  }
  scan_groups<NT, GG>(c, L.scan[round & 3], pre, tot);
  ++round;
  uint32_t nrun = 0;
  {
    uint32_t base = 0;
#pragma unroll
    for (int u = 0; u < GG; ++u) {
      uint32_t o = base + pre[u];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (top[4 * u + j] && o < (uint32_t)kGroupRuns) runs[o++] = 4 * NT * u + 4 * tid + j;
      base += tot[u];
    }
    nrun = base < (uint32_t)kGroupRuns ? base : (uint32_t)kGroupRuns;
  }
  __syncthreads();

  // 3. element e = 4 NT u + 4 tid + j is position kRunLen runs[e / kRunLen] + e % kRunLen
  const int32_t ne = (int32_t)nrun * kRunLen;
  const float* sr = scores + (size_t)row * N;
  auto position = [&](int32_t e) { return kRunLen * runs[e / kRunLen] + (e % kRunLen); };
  uint32_t key[PT];
#pragma unroll
  for (int u = 0; u < GT; ++u) {
    const int32_t e = 4 * NT * u + 4 * tid;
    const int32_t p = e < ne ? position(e) : 0;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    // p is a multiple of 4; when N is not, the load is only 4-byte aligned
    // and the last group of a row reads up to 3 values past it (masked
    // below), still inside the workspace, whose visible counts follow the
    // scores
    if (e < ne && p < n) v = *reinterpret_cast<const float4*>(sr + p);
    key[4 * u + 0] = e < ne && p + 0 < n ? score_key(v.x) : 0u;
    key[4 * u + 1] = e < ne && p + 1 < n ? score_key(v.y) : 0u;
    key[4 * u + 2] = e < ne && p + 2 < n ? score_key(v.z) : 0u;
    key[4 * u + 3] = e < ne && p + 3 < n ? score_key(v.w) : 0u;
  }
  bool sel[PT];
  const uint32_t chosen = block_select<NT, PT>(key, (uint32_t)K, (uint32_t)K, L, sel, round);
  uint32_t oidx[PT];
  kept_order<NT, PT>(sel, L, round, oidx);
  int32_t* orow = out + (size_t)row * K;
  int32_t* sp = reinterpret_cast<int32_t*>(&L.hist[0][0]);   // chosen <= K <= 2 kHistBins
#pragma unroll
  for (int u = 0; u < GT; ++u) {
    const int32_t e = 4 * NT * u + 4 * tid;
    if (e >= ne) continue;
    const int32_t p = position(e);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (sel[4 * u + j]) sp[oidx[4 * u + j]] = p + j;
  }
  __syncthreads();
  for (uint32_t i = tid; i < chosen; i += NT) orow[i] = sp[i];
  for (uint32_t i = chosen + tid; i < (uint32_t)K; i += NT) orow[i] = -1;
}

// ---------------------------------------------------------------------------
// Threshold-bin select for a few long rows and a large K (the hierarchical
// Full layer's Top-P with its Top-K): after the histogram pass over the row's
// top 12 key bits, k_topk_bin_collect keeps every position whose top digit
// is at or above the digit holding the K0-th largest key, a superset of the
// row's Top-K0 (which holds its Top-K1, K1 <= K0), each 4096-position chunk
// into a region of its own in position order (one block scan, no atomics),
// and counts the members of the K0-th and the K1-th key's bins by their next
// 12 bits (fine histograms, device-scope atomics).  k_topk_bin_final then
// selects, per row, the K0 and the K1 largest of the kept elements exactly
// under the (key, lower position) order: the kept list goes to LDS (direct
// global-to-LDS transfers, 16384 elements a tile); the first 24 bits of each
// threshold come from the two histograms and one pass over the list's low
// bytes gives the last 8; ties go to the earlier element and both lists are
// written ascending, the two selects of a row in work-groups of their own.
// The histograms must be zeroed before the histogram pass (the decode step's
// scan clears them on the side); nothing here clears them.
// ---------------------------------------------------------------------------
constexpr int kBinThreads = 256;
constexpr int kBinPer = kBinChunk / kBinThreads;     // 16 consecutive positions per thread

__global__ __launch_bounds__(kBinThreads)
void k_topk_bin_collect(const float* __restrict__ scores, int32_t N, const int32_t* __restrict__ n_valid,
                        int32_t n_all, const uint32_t* __restrict__ hist, int32_t K0, int32_t K1,
                        uint32_t* __restrict__ fine, uint32_t* __restrict__ rkey,
                        int32_t* __restrict__ rpos, uint32_t* __restrict__ rcnt) {
  __shared__ uint32_t lds[kBinThreads / 64 + 5];
  const int row = blockIdx.y, c = blockIdx.x, nch = gridDim.x;
  const int32_t n = row_count(n_valid, n_all, row, N);
  const int32_t c0 = c * kBinChunk;
  const int32_t p0 = c0 + kBinPer * (int32_t)threadIdx.x;
  const float* sr = scores + (size_t)row * N;
  uint32_t key[kBinPer];
  const bool vec = (N & 3) == 0 && ((uintptr_t)scores & 15u) == 0;
#pragma unroll
  for (int u = 0; u < kBinPer / 4; ++u) {
    const int32_t p = p0 + 4 * u;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (vec) {
      if (p < n) v = *reinterpret_cast<const float4*>(sr + p);   // p + 3 < N: N is a multiple of 4
    } else {
      v.x = p < n ? sr[p] : 0.f;
      v.y = p + 1 < n ? sr[p + 1] : 0.f;
      v.z = p + 2 < n ? sr[p + 2] : 0.f;
      v.w = p + 3 < n ? sr[p + 3] : 0.f;
    }
    key[4 * u + 0] = p + 0 < n ? score_key(v.x) : 0u;
    key[4 * u + 1] = p + 1 < n ? score_key(v.y) : 0u;
    key[4 * u + 2] = p + 2 < n ? score_key(v.z) : 0u;
    key[4 * u + 3] = p + 3 < n ? score_key(v.w) : 0u;
  }
  int bin[2];
  uint32_t above[2];
  threshold_bins<kBinThreads>(hist + (size_t)row * kHistBins, (uint32_t)K0, (uint32_t)K1, lds, bin,
                              above);
  const int b0 = n > K0 ? bin[0] : -1;      // every present position when the row has no more than K0
  const int b1 = K1 > 0 && n > K1 ? bin[1] : -1;
  // the threshold bins' members by their next 12 bits (the final select's
  // second digit): a few hundred per chunk, added straight to the row's fine
  // histograms
  uint32_t* fr = fine + (size_t)row * 2 * kHistBins;
#pragma unroll
  for (int i = 0; i < kBinPer; ++i) {
    const int d = (int)(key[i] >> (32 - kHistBits));
    const uint32_t f = (key[i] >> (32 - 2 * kHistBits)) & (kHistBins - 1);
    if (key[i] && b0 >= 0 && d == b0) atomicAdd(&fr[f], 1u);
    if (key[i] && b1 >= 0 && d == b1) atomicAdd(&fr[kHistBins + f], 1u);
  }
  uint32_t cnt = 0;
#pragma unroll
  for (int i = 0; i < kBinPer; ++i) cnt += key[i] && (int)(key[i] >> (32 - kHistBits)) >= b0 ? 1u : 0u;
  uint32_t tot;
  uint32_t o = block_excl_scan<kBinThreads>(cnt, lds, &tot);
  const size_t base = ((size_t)row * nch + c) * kBinChunk;
#pragma unroll
  for (int i = 0; i < kBinPer; ++i) {
    if (key[i] && (int)(key[i] >> (32 - kHistBits)) >= b0) {
      rkey[base + o] = key[i];
      rpos[base + o] = p0 + i;
      ++o;
    }
  }
  if (threadIdx.x == 0) rcnt[(size_t)row * nch + c] = tot;
}

// Direct global -> LDS transfer of 4 bytes per lane: lane l's word lands at
// lds_dst + 4 l (lds_dst wave-uniform); lanes outside EXEC transfer nothing.
__device__ __forceinline__ void dma4(const void* src, void* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_dst, 4, 0, 0);
}

// One select's threshold over the kept list: elements whose key bits at and
// above `shift` exceed `prefix` are chosen, and of those equal to it the
// first `take` in list order.
struct BinThr {
  int shift;
  uint32_t prefix;
  uint32_t take;
};

constexpr int kBinList = kFinalThreads * 16;   // kept elements per LDS tile

struct BinLds {
  uint32_t key[kBinList + 64];       // a tile of the kept list, list order (+ one transfer of slack)
  int32_t pos[kBinList + 64];
  uint32_t h[2][256];                // low-byte histograms of the two 24-bit threshold groups
  uint32_t pre[kBinMaxChunks + 1];   // chunk offsets in the kept list
  uint32_t scan[4][8 * kSelNW];      // rotating scan slots (up to 16 fields)
  uint32_t res[4][4];
};

// One select of a row per work-group: blockIdx.y = 0 takes the K0 largest
// into out0, 1 the K1 largest into out1 (the two run side by side; they
// share only the kept list and the histograms, which neither writes).
__global__ __launch_bounds__(kFinalThreads)
void k_topk_bin_final(int32_t N, const int32_t* __restrict__ n_valid, int32_t n_all,
                      const uint32_t* __restrict__ hist, const uint32_t* __restrict__ fine,
                      int32_t nch, const uint32_t* __restrict__ rkey, const int32_t* __restrict__ rpos,
                      const uint32_t* __restrict__ rcnt, int32_t K0, int32_t* __restrict__ out0,
                      int32_t K1, int32_t* __restrict__ out1) {
  constexpr int kPer = kHistBins / kFinalThreads;   // 4 bins of each histogram per thread
  static_assert(kPer == 4, "one 16-byte slice of each histogram per thread");
  __shared__ __attribute__((aligned(16))) BinLds L;
  const int row = blockIdx.x, which = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t n = row_count(n_valid, n_all, row, N);
  const int32_t K = which == 0 ? K0 : K1;
  int32_t* orow = (which == 0 ? out0 : out1) + (size_t)row * K;
  // one round trip for the chunk counts and this thread's share of the row
  // histogram and of this select's fine histogram
  const uint32_t v = tid < nch ? rcnt[(size_t)row * nch + tid] : 0u;
  uint32_t hc[kPer], fc[kPer];
  hist_slice(hist + (size_t)row * kHistBins, hc);
  hist_slice(fine + ((size_t)row * 2 + which) * kHistBins, fc);
  int round = 0;
  {
    uint32_t tot;
    const uint32_t ex = block_excl_scan<kFinalThreads>(v, L.scan[0], &tot);
    if (tid < nch) L.pre[tid] = ex;
    L.pre[nch] = tot;      // every thread, the same value
  }
  __syncthreads();
  const uint32_t T = L.pre[nch];
  const int ntiles = (int)((T + kBinList - 1) / kBinList);

  // list tile t into LDS: each wave transfers its chunks' share, 64 at a time;
  // wait_tile() before reading it
  auto issue_tile = [&](int t) {
    const uint32_t lo = (uint32_t)t * kBinList;
    const uint32_t hi = T - lo < (uint32_t)kBinList ? T : lo + kBinList;
    for (int c = wave; c < nch; c += kSelNW) {
      const uint32_t pc = L.pre[c];
      const uint32_t a = pc > lo ? pc : lo;
      const uint32_t b = L.pre[c + 1] < hi ? L.pre[c + 1] : hi;
      const uint32_t* ks = rkey + ((size_t)row * nch + c) * kBinChunk;
      const int32_t* ps = rpos + ((size_t)row * nch + c) * kBinChunk;
      for (uint32_t e = a; e < b; e += 64) {
        if (e + lane < b) {
          dma4(ks + (e + lane - pc), &L.key[e - lo]);
          dma4(ps + (e + lane - pc), &L.pos[e - lo]);
        }
      }
    }
  };
  auto wait_tile = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this wave's transfers have landed
    __syncthreads();
  };
  auto tile_count = [&](int t) -> uint32_t {
    const uint32_t lo = (uint32_t)t * kBinList;
    return T - lo < (uint32_t)kBinList ? T - lo : (uint32_t)kBinList;
  };
  // keys of group u for this thread (0: absent or past the tile's cnt elements)
  auto group_keys = [&](int u, uint32_t cnt, uint32_t (&k4)[4]) {
    const uint32_t e = 4096u * u + 4u * tid;
    const uint4 kv = *reinterpret_cast<const uint4*>(&L.key[e]);
    k4[0] = e + 0 < cnt ? kv.x : 0u;
    k4[1] = e + 1 < cnt ? kv.y : 0u;
    k4[2] = e + 2 < cnt ? kv.z : 0u;
    k4[3] = e + 3 < cnt ? kv.w : 0u;
  };
  if (ntiles > 0) issue_tile(0);   // in flight while the threshold is found

  // The threshold.  A row with at most K present positions keeps all of
  // them.  Otherwise the first 24 bits come from the row histogram and the
  // threshold bin's fine histogram; unless that whole 24-bit group is
  // chosen, one pass over the list's low bytes gives the last 8.
  BinThr th{32, 0u, T};
  bool pass = false;
  if (n > K) {
    int bin[2];
    uint32_t above[2];
    threshold_bins_c<kFinalThreads>(hc, (uint32_t)K, 0u, L.scan[round & 3], bin, above);
    ++round;
    uint32_t d, ab, c;
    find_digit_c<kFinalThreads>(fc, kHistBins - 1 - kPer * tid, (uint32_t)K - above[0],
                                L.scan[round & 3], L.res[round & 3], &d, &ab, &c);
    ++round;
    th = BinThr{32 - 2 * kHistBits, ((uint32_t)bin[0] << kHistBits) | d, (uint32_t)K - above[0] - ab};
    pass = c != th.take;
  }
  if (ntiles > 0) wait_tile();
  if (pass) {
    for (int i = tid; i < 256; i += kFinalThreads) L.h[0][i] = 0u;
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
      if (t > 0) {
        __syncthreads();   // every thread is done with the previous tile
        issue_tile(t);
        wait_tile();
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        uint32_t k4[4];
        group_keys(u, tile_count(t), k4);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (k4[j] && (k4[j] >> 8) == th.prefix) atomicAdd(&L.h[0][k4[j] & 255u], 1u);
      }
    }
    __syncthreads();
    uint32_t d, ab, c;
    find_digit<kFinalThreads>(L.h[0], 8, th.take, L.scan[round & 3], L.res[round & 3], &d, &ab, &c);
    ++round;
    th = BinThr{0, (th.prefix << 8) | d, th.take - ab};
    if (ntiles > 1) {
      __syncthreads();
      issue_tile(0);
      wait_tile();
    }
  }

  // Output: an element's index in the list is the number chosen before it
  // in list order, (greater before) + min(equal before, take).  A tile's
  // share is staged in the key array (dead once its counts are scanned) and
  // stored coalesced.
  uint32_t gb = 0, eb = 0;
  for (int t = 0; t < ntiles; ++t) {
    if (t > 0) {
      __syncthreads();   // the staged share of the last tile has been stored
      issue_tile(t);
      wait_tile();
    }
    const uint32_t cnt = tile_count(t);
    uint32_t mg = 0u, me = 0u;   // bit 4 u + j: element greater than / equal to the threshold prefix
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t k4[4];
      group_keys(u, cnt, k4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t hk = key_hi(k4[j], th.shift);
        mg |= k4[j] && hk > th.prefix ? 1u << (4 * u + j) : 0u;
        me |= k4[j] && hk == th.prefix ? 1u << (4 * u + j) : 0u;
      }
    }
    uint32_t f[8], pf[8], tt[8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      f[2 * u] = __builtin_popcount((mg >> (4 * u)) & 15u);
      f[2 * u + 1] = __builtin_popcount((me >> (4 * u)) & 15u);
    }
    scan_groups<kFinalThreads, 8>(f, L.scan[round & 3], pf, tt);   // its barrier: every key read
    ++round;
    const uint32_t ob = gb + (eb < th.take ? eb : th.take);   // chosen before this tile
    int32_t* stage = reinterpret_cast<int32_t*>(L.key);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t g = gb + pf[2 * u], e = eb + pf[2 * u + 1];
      const int4 pv = *reinterpret_cast<const int4*>(&L.pos[4096 * u + 4 * tid]);
      const int32_t ps[4] = {pv.x, pv.y, pv.z, pv.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool gt = (mg >> (4 * u + j)) & 1u, eq = (me >> (4 * u + j)) & 1u;
        const uint32_t o = g + (e < th.take ? e : th.take);
        if ((gt || (eq && e < th.take)) && o < (uint32_t)K) stage[o - ob] = ps[j];
        g += gt ? 1u : 0u;
        e += eq ? 1u : 0u;
      }
      gb += tt[2 * u];
      eb += tt[2 * u + 1];
    }
    const uint32_t oe = gb + (eb < th.take ? eb : th.take);
    const uint32_t m = (oe < (uint32_t)K ? oe : (uint32_t)K) - (ob < (uint32_t)K ? ob : (uint32_t)K);
    __syncthreads();
    for (uint32_t i = tid; i < m; i += kFinalThreads) orow[ob + i] = stage[i];
  }
  const uint32_t chosen = gb + (eb < th.take ? eb : th.take);
  for (uint32_t i = chosen + tid; i < (uint32_t)K; i += kFinalThreads) orow[i] = -1;
}

__global__ void k_fill_u32(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t k = i; k < n; k += stride) p[k] = v;
}

__global__ void k_copy_i32(int32_t* __restrict__ d, const int32_t* __restrict__ s, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t k = i; k < n; k += stride) d[k] = s[k];
}

}  // namespace

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  k_fill_u32<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p, n, v);
  return hipGetLastError();
}

hipError_t launch_fill_zero(uint32_t* p, int64_t n, hipStream_t s) { return launch_fill_u32(p, n, 0u, s); }

hipError_t launch_copy_i32(int32_t* d, const int32_t* src, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  k_copy_i32<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(d, src, n);
  return hipGetLastError();
}

hipError_t launch_topk_rows(const float* scores, int32_t R, int32_t N,
                            const int32_t* n_valid, int32_t n_all, int32_t K,
                            uint32_t* hist, bool zero_hist, const int32_t* cand,
                            int32_t* out, hipStream_t s) {
  if (N > kRowMaxN) return hipErrorInvalidValue;
  const dim3 grid((unsigned)R), block(kRowThreads);
  const bool pre = (N & 3) == 0 && N <= kPreF4 * 4 * kRowThreads && ((uintptr_t)scores & 15u) == 0;
  const int zh = zero_hist ? 1 : 0;
  if (hist) {
    if (pre)
      k_topk_row<true, true><<<grid, block, 0, s>>>(scores, N, n_valid, n_all, K, hist, zh, cand, out);
    else
      k_topk_row<true, false><<<grid, block, 0, s>>>(scores, N, n_valid, n_all, K, hist, zh, cand, out);
  } else {
    if (pre)
      k_topk_row<false, true><<<grid, block, 0, s>>>(scores, N, n_valid, n_all, K, nullptr, 0, cand, out);
    else
      k_topk_row<false, false><<<grid, block, 0, s>>>(scores, N, n_valid, n_all, K, nullptr, 0, cand, out);
  }
  return hipGetLastError();
}

// The slice and final selects run on 1024 threads (16 waves on a CU).
// Measured at 128K decode: slice 5.8 / 6.4 / 8.8 us and final 6.7 / 8.2 /
// 12.8 us on 1024 / 512 / 256 threads (the same slices, 4 / 8 / 16
// positions a thread): the per-wave steps cost fewer issue cycles on fewer
// waves, but their dependent latencies are no longer hidden.
template <int NT>
hipError_t launch_final_nt(dim3 grid, hipStream_t s, int64_t elems, const float* scores, int32_t N,
                           const int32_t* n_valid, int32_t n_all, int32_t total,
                           const uint32_t* ckey, const int32_t* cpos, int32_t K,
                           const int32_t* cand, int32_t* out) {
  const dim3 block(NT);
  if (elems <= NT * 4)
    k_topk_final<NT, 4><<<grid, block, 0, s>>>(scores, N, n_valid, n_all, total, ckey, cpos, K, cand, out);
  else if (elems <= NT * 8)
    k_topk_final<NT, 8><<<grid, block, 0, s>>>(scores, N, n_valid, n_all, total, ckey, cpos, K, cand, out);
  else
    k_topk_final<NT, 16><<<grid, block, 0, s>>>(scores, N, n_valid, n_all, total, ckey, cpos, K, cand, out);
  return hipGetLastError();
}

// k_topk_final over `elems` elements per row (at most kFinalMaxN).
hipError_t launch_final(dim3 grid, hipStream_t s, int64_t elems, const float* scores, int32_t N,
                        const int32_t* n_valid, int32_t n_all, int32_t total, const uint32_t* ckey,
                        const int32_t* cpos, int32_t K, const int32_t* cand, int32_t* out) {
  static_assert(kFinalThreads * 16 >= kFinalMaxN, "one work-group holds the largest final select");
  return launch_final_nt<kFinalThreads>(grid, s, elems, scores, N, n_valid, n_all, total, ckey, cpos, K,
                                        cand, out);
}

hipError_t launch_topk_sliced(const float* scores, int32_t R, int32_t N,
                              const int32_t* n_valid, int32_t n_all, const int32_t* cand,
                              int32_t K, int32_t* out, void* ws, hipStream_t s) {
  const TopkSlicing sl = topk_slicing(R, N, K);
  if (!sl.taken || R <= 0 || K <= 0) return hipErrorInvalidValue;
  uint32_t* ckey = nullptr;
  int32_t* cpos = nullptr;
  int64_t elems = N;
  int32_t total = 0;
  if (sl.S > 0) {
    if (!ws) return hipErrorInvalidValue;
    ckey = (uint32_t*)ws;
    cpos = (int32_t*)((char*)ws + align256((size_t)R * sl.S * sl.slots * 4));
    // a slice of 1024 pt positions
    const dim3 grid((unsigned)sl.S, (unsigned)R), block(kFinalThreads);
    if (sl.pt == 4)
      k_topk_slice<kFinalThreads, 4><<<grid, block, 0, s>>>(scores, N, n_valid, n_all, K, sl.slots, ckey, cpos);
    else if (sl.pt == 8)
      k_topk_slice<kFinalThreads, 8><<<grid, block, 0, s>>>(scores, N, n_valid, n_all, K, sl.slots, ckey, cpos);
    else
      k_topk_slice<kFinalThreads, 16><<<grid, block, 0, s>>>(scores, N, n_valid, n_all, K, sl.slots, ckey, cpos);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    total = sl.S * sl.slots;
    elems = total;
  }
  return launch_final(dim3((unsigned)R), s, elems, scores, N, n_valid, n_all, total, ckey, cpos, K,
                      cand, out);
}

hipError_t launch_topk_group(const float* scores, const float* gmax, int32_t R, int32_t N,
                             const int32_t* n_valid, int32_t n_all, int32_t K, int32_t* out,
                             hipStream_t s) {
  if (!topk_group_taken(N, K) || R <= 0 || (N & 3) || ((uintptr_t)scores & 15u) ||
      ((uintptr_t)gmax & 15u))
    return hipErrorInvalidValue;
  const dim3 grid((unsigned)R), block(kGroupThreads);
  const int32_t need = (N + kRunLen - 1) / kRunLen;
  if (need <= 8 * kGroupThreads)
    k_topk_group<8><<<grid, block, 0, s>>>(scores, N, gmax, n_valid, n_all, K, out);
  else
    k_topk_group<16><<<grid, block, 0, s>>>(scores, N, gmax, n_valid, n_all, K, out);
  return hipGetLastError();
}

hipError_t launch_score_topk(const uint8_t* key, int32_t B, int64_t M, const uint8_t* q_idx,
                             const float* w_idx, const int32_t* len, const PoolMap& map,
                             int32_t K, int32_t* out, void* ws, hipStream_t s) {
  const TopkSlicing sl = score_topk_slicing(B, M, K);
  if (!sl.taken || !ws) return hipErrorInvalidValue;
  uint32_t* ckey = (uint32_t*)ws;
  int32_t* cpos = (int32_t*)((char*)ws + align256((size_t)B * sl.S * sl.slots * 4));
  k_score_slice<<<dim3((unsigned)sl.S, (unsigned)B), dim3(kFinalThreads), 0, s>>>(
      key, M, q_idx, w_idx, len, map, K, sl.slots, ckey, cpos);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int32_t total = sl.S * sl.slots;
  return launch_final(dim3((unsigned)B), s, total, nullptr, (int32_t)M, len, (int32_t)M, total, ckey,
                      cpos, K, nullptr, out);
}

hipError_t launch_topk_bin_select(const float* scores, int32_t R, int32_t N,
                                  const int32_t* n_valid, int32_t n_all, uint32_t* hist,
                                  int32_t K0, int32_t* out0, int32_t K1, int32_t* out1, void* ws,
                                  hipStream_t s) {
  const int32_t nch = (N + kBinChunk - 1) / kBinChunk;
  if (!ws || nch > kBinMaxChunks || K0 <= 0 || K1 < 0 || K1 > K0) return hipErrorInvalidValue;
  const size_t reg = align256((size_t)R * nch * kBinChunk * 4);
  char* p = (char*)ws;
  uint32_t* rkey = (uint32_t*)p;  p += reg;
  int32_t* rpos = (int32_t*)p;    p += reg;
  uint32_t* rcnt = (uint32_t*)p;
  uint32_t* fine = hist + (size_t)R * kHistBins;   // [R][2][4096] after the row histograms
  k_topk_bin_collect<<<dim3((unsigned)nch, (unsigned)R), dim3(kBinThreads), 0, s>>>(
      scores, N, n_valid, n_all, hist, K0, K1, fine, rkey, rpos, rcnt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_topk_bin_final<<<dim3((unsigned)R, K1 > 0 ? 2u : 1u), dim3(kFinalThreads), 0, s>>>(
      N, n_valid, n_all, hist, fine, nch, rkey, rpos, rcnt, K0, out0, K1, out1);
  return hipGetLastError();
}

hipError_t launch_topk_hist(const float* scores, int32_t R, int32_t N,
                            const int32_t* n_valid, int32_t n_all,
                            uint32_t* hist, hipStream_t s) {
  const dim3 grid((unsigned)((N + kChunk - 1) / kChunk), (unsigned)R);
  k_topk_hist<<<grid, dim3(kSelThreads), 0, s>>>(scores, N, n_valid, n_all, hist);
  return hipGetLastError();
}

static SelectSet select_set(int32_t K, const TopkWs& ws, const int32_t* cand, int32_t* out) {
  return SelectSet{K, ws.counters, ws.sel, ws.candk, ws.candp, ws.cap, cand, out};
}

static hipError_t launch_collect_finish(const float* scores, int32_t R, int32_t N,
                                        const int32_t* n_valid, int32_t n_all, uint32_t* hist,
                                        bool zero_hist, const SelectSet& t0, const SelectSet& t1,
                                        hipStream_t s) {
  const dim3 grid((unsigned)((N + kChunk - 1) / kChunk), (unsigned)R);
  k_topk_collect<<<grid, dim3(kSelThreads), 0, s>>>(scores, N, n_valid, n_all, hist, t0, t1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_topk_finish<<<dim3((unsigned)R, t1.K > 0 ? 2u : 1u), dim3(kFinThreads), 0, s>>>(
      scores, N, n_valid, n_all, hist, zero_hist ? 1 : 0, t0, t1);
  return hipGetLastError();
}

hipError_t launch_topk_select(const float* scores, int32_t R, int32_t N,
                              const int32_t* n_valid, int32_t n_all,
                              const int32_t* cand, int32_t K, int32_t* out,
                              const TopkWs& ws, bool zero_hist, hipStream_t s) {
  const SelectSet none{};
  return launch_collect_finish(scores, R, N, n_valid, n_all, ws.hist, zero_hist,
                               select_set(K, ws, cand, out), none, s);
}

hipError_t launch_topk_select2(const float* scores, int32_t R, int32_t N,
                               const int32_t* n_valid, int32_t n_all,
                               int32_t K0, int32_t* out0, const TopkWs& ws0,
                               int32_t K1, int32_t* out1, const TopkWs& ws1,
                               bool zero_hist, hipStream_t s) {
  return launch_collect_finish(scores, R, N, n_valid, n_all, ws0.hist, zero_hist,
                               select_set(K0, ws0, nullptr, out0), select_set(K1, ws1, nullptr, out1),
                               s);
}

}  // namespace csa2

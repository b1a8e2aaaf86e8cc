// Top-K select with the lower-index tie-break, ascending output.
//
// The pages say only that Full and Reindex layers select Top-K entries from
// the indexer scores ("DeepSeek V4.1-Flash Cuts KV Cache by 437x", paragraph
// on the three operating modes); equal scores going to the lower pool index
// and the ascending output order are this library's fixed conventions.
//
// Every (score, position) pair maps to a unique composite order key
//   key32(score) : (n - 1 - position)
// (key32 is the order-preserving uint32 image of the float), so the K largest
// composites are exactly the wanted set.  The select is a radix select:
//  1. histogram of the top 12 key bits per row (fused into the score kernel,
//     or k_topk_hist), giving the bin b* that holds the K-th largest key;
//  2. k_topk_collect (many work-groups per row) appends positions in bins
//     above b* to a list and the (key, position) pairs inside b* to a
//     candidate list, with one wave-aggregated atomic per wave;
//  3. k_topk_finish (one work-group per row) resolves the rest of the
//     composite with 10-bit radix passes over the candidates only, marks the
//     chosen positions in an LDS bitmap and writes them in ascending order
//     with a block prefix sum.  If the candidate list overflowed its slots,
//     the same passes read the candidates straight from the score row.
// Ties, -0 vs +0, rows with fewer than K valid positions and N up to 2^30 are
// all handled exactly; the result is deterministic.
#include "csa2_internal.h"

namespace csa2 {
namespace {

constexpr int kSelThreads = 256;
constexpr int kChunk = 4096;              // positions per collect / hist work-group
constexpr int kFinThreads = 1024;
constexpr int kSegBits = 18;              // bitmap segment of 2^18 positions (32 KiB)
constexpr int kSeg = 1 << kSegBits;
constexpr int kSegWords = kSeg / 32;      // 8192
constexpr int kCompBits = 50;             // 20 low key bits + 30 position bits
constexpr int kDigit = 10;

__device__ __forceinline__ int32_t row_count(const int32_t* n_valid, int32_t n_all,
                                             int row, int32_t N) {
  int32_t n = n_valid ? n_valid[row] : n_all;
  return n < 0 ? 0 : (n > N ? N : n);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Exclusive prefix sum over the NT threads of a block; *total receives the sum.
// lds must hold NT/64 + 1 words and is free again on return.
template <int NT>
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t* lds, uint32_t* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) lds[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t acc = 0;
    for (int w = 0; w < NT / 64; ++w) {
      const uint32_t c = lds[w];
      lds[w] = acc;
      acc += c;
    }
    lds[NT / 64] = acc;
  }
  __syncthreads();
  const uint32_t r = lds[wave] + x - v;
  *total = lds[NT / 64];
  __syncthreads();
  return r;
}

// Bin of the K-th largest key in a 4096-bin histogram (bins ordered by key).
// *above = number of keys in higher bins; above < K <= above + h[bin].
// lds: NT/64 + 3 words.  Returns bin -1 if the histogram holds fewer than K.
template <int NT>
__device__ void threshold_bin(const uint32_t* h, uint32_t K, uint32_t* lds,
                              int* bin, uint32_t* above) {
  constexpr int PER = kHistBins / NT;
  const int top = kHistBins - 1 - (int)threadIdx.x * PER;  // thread 0 owns the highest bins
  uint32_t c[PER];
  uint32_t s = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    c[i] = h[top - i];
    s += c[i];
  }
  if (threadIdx.x == 0) {
    lds[NT / 64 + 1] = 0xFFFFFFFFu;
    lds[NT / 64 + 2] = 0u;
  }
  uint32_t tot;
  const uint32_t ex = block_excl_scan<NT>(s, lds, &tot);
  if (ex < K && K <= ex + s) {
    uint32_t acc = ex;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (acc + c[i] >= K) {
        lds[NT / 64 + 1] = (uint32_t)(top - i);
        lds[NT / 64 + 2] = acc;
        break;
      }
      acc += c[i];
    }
  }
  __syncthreads();
  *bin = (int)lds[NT / 64 + 1];
  *above = lds[NT / 64 + 2];
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

__global__ __launch_bounds__(kSelThreads)
void k_topk_collect(const float* __restrict__ scores, int32_t N,
                    const int32_t* __restrict__ n_valid, int32_t n_all, int32_t K,
                    const uint32_t* __restrict__ hist, uint32_t* __restrict__ counters,
                    int32_t* __restrict__ sel, uint32_t* __restrict__ candk,
                    int32_t* __restrict__ candp, int32_t cap) {
  __shared__ uint32_t lds[kSelThreads / 64 + 3];
  const int row = blockIdx.y;
  const int32_t n = row_count(n_valid, n_all, row, N);
  if (n <= K) return;
  const int64_t c0 = (int64_t)blockIdx.x * kChunk;
  if (c0 >= n) return;
  int bstar;
  uint32_t above;
  threshold_bin<kSelThreads>(hist + (size_t)row * kHistBins, (uint32_t)K, lds, &bstar, &above);
  const float* sr = scores + (size_t)row * N;
  uint32_t* cnt = counters + (size_t)row * kCounterWords;
  int32_t* srow = sel + (size_t)row * K;
  uint32_t* ckr = candk + (size_t)row * cap;
  int32_t* cpr = candp + (size_t)row * cap;
  const int lane = threadIdx.x & 63;
  for (int i = 0; i < kChunk / kSelThreads; ++i) {
    const int64_t p = c0 + i * kSelThreads + threadIdx.x;
    const bool in = p < n;
    const uint32_t key = in ? score_key(sr[p]) : 0u;
    const int bin = (int)(key >> (32 - kHistBits));
    const bool gt = in && bin > bstar;
    const bool eq = in && bin == bstar;
    const uint64_t mg = __ballot(gt);
    const uint64_t me = __ballot(eq);
    uint32_t bg = 0, be = 0;
    if (lane == 0) {
      if (mg) bg = atomicAdd(&cnt[0], (uint32_t)__popcll(mg));
      if (me) be = atomicAdd(&cnt[1], (uint32_t)__popcll(me));
    }
    bg = __shfl(bg, 0, 64);
    be = __shfl(be, 0, 64);
    if (gt) {
      const uint32_t r = bg + lanes_below(mg);
      if (r < (uint32_t)K) srow[r] = (int32_t)p;
    }
    if (eq) {
      const uint32_t r = be + lanes_below(me);
      if (r < (uint32_t)cap) {
        ckr[r] = key;
        cpr[r] = (int32_t)p;
      }
    }
  }
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

__global__ __launch_bounds__(kFinThreads)
void k_topk_finish(const float* __restrict__ scores, int32_t N,
                   const int32_t* __restrict__ n_valid, int32_t n_all, int32_t K,
                   const uint32_t* __restrict__ hist, const uint32_t* __restrict__ counters,
                   const int32_t* __restrict__ sel, const uint32_t* __restrict__ candk,
                   const int32_t* __restrict__ candp, int32_t cap,
                   const int32_t* __restrict__ cand_map, int32_t* __restrict__ out) {
  __shared__ uint32_t lds[kFinThreads / 64 + 8];
  __shared__ uint32_t rh[1 << kDigit];
  __shared__ uint32_t bitmap[kSegWords];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int32_t n = row_count(n_valid, n_all, row, N);
  int32_t* orow = out + (size_t)row * K;
  const int32_t* mrow = cand_map ? cand_map + (size_t)row * N : nullptr;
  if (n <= K) {
    for (int i = tid; i < K; i += kFinThreads) orow[i] = i < n ? (mrow ? mrow[i] : i) : -1;
    return;
  }
  int bstar;
  uint32_t above;
  threshold_bin<kFinThreads>(hist + (size_t)row * kHistBins, (uint32_t)K, lds, &bstar, &above);
  if (bstar < 0) {  // inconsistent histogram: cannot happen for valid inputs
    for (int i = tid; i < K; i += kFinThreads) orow[i] = -1;
    return;
  }
  const uint32_t ccount = counters[(size_t)row * kCounterWords + 1];
  const bool overflow = ccount > (uint32_t)cap;
  const uint32_t C = overflow ? 0u : ccount;
  const uint32_t* ck = candk + (size_t)row * cap;
  const int32_t* cp = candp + (size_t)row * cap;
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
  const int32_t* srow = sel + (size_t)row * K;
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
#pragma unroll
    for (int w = 0; w < WPT; ++w) {
      uint32_t m = wv[w];
      while (m) {
        const int bit = __ffs(m) - 1;
        m &= m - 1;
        const int64_t p = s0 + (int64_t)(tid * WPT + w) * 32 + bit;
        if (pos < (uint32_t)K) orow[pos] = mrow ? mrow[p] : (int32_t)p;
        ++pos;
      }
    }
    written += tot;
    __syncthreads();
  }
  for (uint32_t i = written + tid; i < (uint32_t)K; i += kFinThreads) orow[i] = -1;
}

__global__ void k_fill_zero(uint32_t* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t k = i; k < n; k += stride) p[k] = 0u;
}

__global__ void k_copy_i32(int32_t* __restrict__ d, const int32_t* __restrict__ s, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t k = i; k < n; k += stride) d[k] = s[k];
}

}  // namespace

hipError_t launch_fill_zero(uint32_t* p, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  k_fill_zero<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(p, n);
  return hipGetLastError();
}

hipError_t launch_copy_i32(int32_t* d, const int32_t* src, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  k_copy_i32<<<dim3((unsigned)blocks), dim3(256), 0, s>>>(d, src, n);
  return hipGetLastError();
}

hipError_t launch_topk_hist(const float* scores, int32_t R, int32_t N,
                            const int32_t* n_valid, int32_t n_all,
                            uint32_t* hist, hipStream_t s) {
  const dim3 grid((unsigned)((N + kChunk - 1) / kChunk), (unsigned)R);
  k_topk_hist<<<grid, dim3(kSelThreads), 0, s>>>(scores, N, n_valid, n_all, hist);
  return hipGetLastError();
}

hipError_t launch_topk_select(const float* scores, int32_t R, int32_t N,
                              const int32_t* n_valid, int32_t n_all,
                              const int32_t* cand, int32_t K, int32_t* out,
                              const TopkWs& ws, hipStream_t s) {
  const dim3 grid((unsigned)((N + kChunk - 1) / kChunk), (unsigned)R);
  k_topk_collect<<<grid, dim3(kSelThreads), 0, s>>>(scores, N, n_valid, n_all, K, ws.hist,
                                                    ws.counters, ws.sel, ws.candk, ws.candp, ws.cap);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  k_topk_finish<<<dim3((unsigned)R), dim3(kFinThreads), 0, s>>>(
      scores, N, n_valid, n_all, K, ws.hist, ws.counters, ws.sel, ws.candk, ws.candp, ws.cap,
      cand, out);
  return hipGetLastError();
}

}  // namespace csa2

// Internal definitions shared by the CSA2 HIP translation units (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace csa2 {

// Fixed model shapes (latent, indexer and head widths).
constexpr int kD = 512;          // latent width (shared K/V)
constexpr int kLatRow = kD / 2;  // E2M1 bytes per latent row
constexpr int kScaleRow = kD / 32;  // E8M0 scales per latent row
constexpr int kHI = 8;           // indexer heads
constexpr int kDI = 64;          // indexer head width
constexpr int kKeyRow = kHI * kDI;  // E4M3 bytes per indexer key row
constexpr int kH = 16;           // attention heads

// Top-K
constexpr int kHistBits = 12;               // first radix digit: top 12 key bits
constexpr int kHistBins = 1 << kHistBits;   // 4096
constexpr int kMaxK = 16384;
constexpr int kMaxTopkN = 1 << 30;          // row length limit (composite key packs 30 bits)
constexpr int kRowMaxN = 1 << 18;           // rows up to this length can take the one-work-group select
constexpr int kRowSplitN = 32768;           // longer rows, when there are few, take the multi-work-group select
constexpr int kRowSplitR = 256;             // "few": fewer rows than this

// Which select a (rows, row length) shape takes.
inline bool topk_multi_wg(int64_t R, int64_t N) {
  return N > kRowMaxN || (N > kRowSplitN && R < kRowSplitR);
}
constexpr int kCounterWords = 4;            // per row: [0]=above count, [1]=candidate count, [2]=bin, [3]=above the bin

// Sliced select: rows of at most kFinalMaxN positions take one work-group;
// longer rows (on fewer than kRowSplitR rows) are cut into S slices of
// 1024 * pt positions, each slice's keepers (a superset of its Top-K, at most
// `slots`) found by one work-group, then the row's Top-K from all keepers,
// which must fit one work-group (S * slots <= kFinalMaxN).
constexpr int kFinalMaxN = 16384;
struct TopkSlicing {
  bool taken;      // the sliced select takes this shape
  int32_t S;       // slices (0: the row itself goes to the final select)
  int32_t pt;      // positions per thread of a slice (slice = 1024 pt)
  int32_t slots;   // keepers per slice
};
inline int32_t topk_slot_count(int64_t K) {
  // room for the threshold digit's group beyond K; a multiple of 64 (the
  // final select reads the keepers 16 bytes at a time)
  const int64_t extra = K / 4 > 64 ? K / 4 : 64;
  return (int32_t)((K + extra + 63) / 64 * 64);
}
inline TopkSlicing topk_slicing(int64_t R, int64_t N, int64_t K) {
  TopkSlicing t{false, 0, 0, 0};
  if (N <= kFinalMaxN) {   // the row itself goes to one work-group
    t.taken = true;
    return t;
  }
  if (R >= kRowSplitR) return t;   // many long rows: the one-work-group row select
  const int64_t slots = topk_slot_count(K);
  // the smallest slice that gives at most one round of work-groups (a slice
  // must hold several times K to filter anything, and all keepers must fit
  // the final select), else the largest slice that fits
  for (int pt = 4; pt <= 16; pt *= 2) {
    const int64_t len = 1024 * pt;
    const int64_t S = (N + len - 1) / len;
    if (len < 4 * K || S * slots > kFinalMaxN) continue;
    t.taken = true;
    t.S = (int32_t)S;
    t.pt = pt;
    t.slots = (int32_t)slots;
    if (R * S <= 256) break;
  }
  return t;
}

// Attention
constexpr int kAttnStepKeys = 32;           // keys per step of the attention kernel
constexpr int kAttnMaxSplits = 63;          // splits per row (the merge holds them and an
                                            // incoming result in one wave)
constexpr int kAttnFillGroups = 2048;       // decode: splits never give more work-groups than this
constexpr int kAttnSplitRows = 512;         // query rows from which one work-group per row fills the chip

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Where a sequence's pool entry lives.  Contiguous pools hold sequence b's
// entry e at row b * M + e; paged pools at row page * 2^lg2 + e mod 2^lg2,
// page = pages[b][e >> lg2] (a per-sequence page table into shared arrays).
struct PoolMap {
  const int32_t* pages;   // NULL: contiguous [B][M]; else [B][np] physical page numbers
  int32_t lg2;            // entries per page = 1 << lg2
  int32_t np;             // pages per sequence = M >> lg2
};
__device__ __forceinline__ int64_t pool_row(const PoolMap& m, int64_t b, int64_t e, int64_t M) {
  if (!m.pages) return b * M + e;
  return ((int64_t)m.pages[b * m.np + (e >> m.lg2)] << m.lg2) | (e & ((int64_t(1) << m.lg2) - 1));
}

// Order-preserving map of a float score to uint32 (-0 folded onto +0):
// a > b as reals  <=>  key(a) > key(b).
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Workspace carving for Top-K over R rows of N with up to K selected.
struct TopkWs {
  uint32_t* hist;      // [R][kHistBins]
  uint32_t* counters;  // [R][kCounterWords]
  int32_t* sel;        // [R][K]   positions strictly above the threshold bin
  uint32_t* candk;     // [R][cap] keys of positions inside the threshold bin
  int32_t* candp;      // [R][cap] their positions
  int32_t cap;
};

// One select of the multi-work-group path: its K, per-row counters
// ([0] count above the threshold bin, [1] bin members, [2] the bin, [3] the
// count above it as found from the histogram), lists and output.
struct SelectSet {
  int32_t K;
  uint32_t* counters;
  int32_t* sel;
  uint32_t* candk;
  int32_t* candp;
  int32_t cap;
  const int32_t* cand_map;
  int32_t* out;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline int32_t topk_cap(int64_t R, int64_t N) {
  // Candidate slots per row: every position for modest row counts, otherwise
  // 16384 (the finish step re-scans the row when a threshold bin overflows).
  int64_t c = (int64_t(1) << 25) / (R > 0 ? R : 1);
  if (c < 16384) c = 16384;
  if (c > N) c = N;
  return (int32_t)(c > 0 ? c : 1);
}

// Slice keepers of the sliced select: keys and positions [R][S][slots].
inline size_t topk_slice_ws_bytes(int64_t R, int64_t N, int64_t K) {
  const TopkSlicing s = topk_slicing(R, N, K);
  return s.S > 0 ? align256((size_t)(R * s.S * s.slots * 4)) * 2 : 0;
}

// Fused score -> Top-K of flat rows (one query row per sequence): slices of
// kScoreSlice entries scored and filtered in LDS, then the final select,
// which must hold every slice's keepers.
constexpr int kScoreSlice = 4096;
inline TopkSlicing score_topk_slicing(int64_t R, int64_t N, int64_t K) {
  TopkSlicing t{false, 0, 4, 0};
  if (R <= 0 || N <= 0 || K <= 0) return t;
  const int64_t S = (N + kScoreSlice - 1) / kScoreSlice;
  const int64_t slots = topk_slot_count(K);
  if (S * slots > kFinalMaxN) return t;
  t.taken = true;
  t.S = (int32_t)S;
  t.slots = (int32_t)slots;
  return t;
}
inline size_t score_topk_ws_bytes(int64_t R, int64_t N, int64_t K) {
  const TopkSlicing s = score_topk_slicing(R, N, K);
  return s.taken ? align256((size_t)(R * s.S * s.slots * 4)) * 2 : 0;
}

// Threshold-bin select (a few long rows, a large K, up to two selects from
// one histogram): every position at or above the threshold bin, per
// 4096-position chunk, keys and positions [R][chunks][4096] and counts
// [R][chunks].
// Its histograms (row [R][4096], then the threshold bins' next digit
// [R][2][4096], topk_bin_hist_words) must be zeroed before each select; the
// select leaves them filled.
constexpr int kBinChunk = 4096;
constexpr int kBinMaxChunks = 256;   // rows up to 2^20 positions
inline bool topk_bin_taken(int64_t N) { return N > 0 && N <= (int64_t)kBinChunk * kBinMaxChunks; }
inline int64_t topk_bin_hist_words(int64_t R) { return R * kHistBins * 3; }
inline size_t topk_bin_ws_bytes(int64_t R, int64_t N) {
  const int64_t nch = (N + kBinChunk - 1) / kBinChunk;
  return 2 * align256((size_t)(R * nch * kBinChunk * 4)) + align256((size_t)(R * nch * 4));
}

inline size_t topk_ws_bytes(int64_t R, int64_t N, int64_t K) {
  int64_t cap = topk_cap(R, N);
  return align256(R * kHistBins * 4) + align256(R * kCounterWords * 4) +
         align256(R * K * 4) + align256(R * cap * 4) * 2;
}

inline TopkWs topk_ws_carve(void* ws, int64_t R, int64_t N, int64_t K) {
  TopkWs t;
  char* p = (char*)ws;
  t.cap = topk_cap(R, N);
  t.hist = (uint32_t*)p;     p += align256(R * kHistBins * 4);
  t.counters = (uint32_t*)p; p += align256(R * kCounterWords * 4);
  t.sel = (int32_t*)p;       p += align256(R * K * 4);
  t.candk = (uint32_t*)p;    p += align256(R * (int64_t)t.cap * 4);
  t.candp = (int32_t*)p;
  return t;
}


// ---------------------------------------------------------------------------
// Launchers (each returns the hipError_t of its launch)
// ---------------------------------------------------------------------------

// Zero n 32-bit words (a kernel, so that it is safe inside captured graphs).
hipError_t launch_fill_zero(uint32_t* p, int64_t n, hipStream_t s);

// Up to three spans of 32-bit words that a launch zeroes on the side, for the
// launches after it on the stream (n = 0: unused).  The scan takes them when
// they are 16-byte aligned multiples of 4 words that its grid covers, 16
// bytes per thread; otherwise fill launches ahead of it clear them.
struct ZeroSpans {
  uint32_t* p[3];
  int64_t n[3];
};

// Indexer scores; see csa2_index_score.  len (optional, [B]): sequence b has
// len[b] <= M entries (a ragged batch); entries at or past it score -inf.
// zero (optional): spans the scan's first work-groups clear as well (one
// fill launch fewer ahead of a select that needs zeroed counters).
hipError_t launch_index_score(const uint8_t* key, int32_t B, int64_t M,
                              const uint8_t* q_idx, const float* w_idx,
                              int32_t Q, int64_t pos0, int32_t ratio,
                              const int32_t* cand, int32_t N, float* scores,
                              uint32_t* hist, const int32_t* len, const PoolMap& map,
                              hipStream_t s, const ZeroSpans* zero = nullptr);

// Top-K pieces.  n_valid: device [R] or NULL (then n_all applies to every row).
// launch_topk_rows: one work-group per row, N <= kRowMaxN.  hist: NULL (the
// kernel builds its own) or the rows' top-12-bit histograms [R][kHistBins]
// from the score kernel, zeroed after use when zero_hist is set.
hipError_t launch_topk_rows(const float* scores, int32_t R, int32_t N,
                            const int32_t* n_valid, int32_t n_all, int32_t K,
                            uint32_t* hist, bool zero_hist, const int32_t* cand,
                            int32_t* out, hipStream_t s);
// Group select (rows longer than kFinalMaxN whose scores come with the
// maximum of every run of 16 positions, gmax [ceil(N / 128)][R][8] as the
// prefill score kernel writes it; N a multiple of 4; 16-byte aligned): the
// Top-K of each row from the K best runs, K <= 512.
inline bool topk_group_taken(int64_t N, int64_t K) {
  return N > kFinalMaxN && N <= (int64_t)16 * 8192 && K > 0 && K <= 512;
}
// run maxima per row, with the padding of the last 128-entry tile
inline int64_t topk_group_runs(int64_t N) { return 8 * ((N + 127) / 128); }
hipError_t launch_topk_group(const float* scores, const float* gmax, int32_t R, int32_t N,
                             const int32_t* n_valid, int32_t n_all, int32_t K, int32_t* out,
                             hipStream_t s);
// Sliced select (topk_slicing(R, N, K).taken): ws holds topk_slice_ws_bytes.
hipError_t launch_topk_sliced(const float* scores, int32_t R, int32_t N,
                              const int32_t* n_valid, int32_t n_all, const int32_t* cand,
                              int32_t K, int32_t* out, void* ws, hipStream_t s);
// Fused score -> Top-K of B flat rows (score_topk_slicing(B, M, K).taken):
// the indexer score of every visible entry and the row's Top-K, without
// writing the scores; ws holds score_topk_ws_bytes.
hipError_t launch_score_topk(const uint8_t* key, int32_t B, int64_t M, const uint8_t* q_idx,
                             const float* w_idx, const int32_t* len, const PoolMap& map,
                             int32_t K, int32_t* out, void* ws, hipStream_t s);
hipError_t launch_topk_hist(const float* scores, int32_t R, int32_t N,
                            const int32_t* n_valid, int32_t n_all,
                            uint32_t* hist, hipStream_t s);
// Threshold-bin select on scores whose histogram is in hist (topk_bin_taken(N);
// hist holds topk_bin_hist_words words, zeroed on entry, filled on return):
// the K0 largest of each row to out0 and the K1 largest (K1 <= K0; 0: none)
// to out1, both ascending; ws holds topk_bin_ws_bytes; hist is left zeroed.
hipError_t launch_topk_bin_select(const float* scores, int32_t R, int32_t N,
                                  const int32_t* n_valid, int32_t n_all, uint32_t* hist,
                                  int32_t K0, int32_t* out0, int32_t K1, int32_t* out1, void* ws,
                                  hipStream_t s);
// Multi-work-group select on scores whose histogram is in ws.hist and whose
// counters are zero; leaves the counters (and, with zero_hist, the
// histogram) zeroed.
hipError_t launch_topk_select(const float* scores, int32_t R, int32_t N,
                              const int32_t* n_valid, int32_t n_all,
                              const int32_t* cand, int32_t K, int32_t* out,
                              const TopkWs& ws, bool zero_hist, hipStream_t s);
// Two selects of the same rows in one collect pass and one finish launch
// (one work-group per row and select): K0 into out0 with ws0's lists and K1
// into out1 with ws1's; both read ws0.hist (ws1's histogram is not used).
// Both outputs are unmapped (global positions).
hipError_t launch_topk_select2(const float* scores, int32_t R, int32_t N,
                               const int32_t* n_valid, int32_t n_all,
                               int32_t K0, int32_t* out0, const TopkWs& ws0,
                               int32_t K1, int32_t* out1, const TopkWs& ws1,
                               bool zero_hist, hipStream_t s);

// Attention over up to K gathered FP4 entries and up to W FP8 window rows per
// query row, on the matrix cores.  The row's keys are taken kAttnStepKeys per
// step (global steps first, then window steps).  Prefill runs one work-group
// per row; decode cuts a row's steps into `splits` runs of `cps` steps, one
// work-group each, whose partials (opart, ml) a merge launch combines.  The
// result, merged with an incoming (o_in, lse_in) when lse_in is given (they
// may alias o / lse), is written to o and lse.
struct AttnArgs {
  const uint8_t* latent;  // pool rows [.][kLatRow] (see PoolMap)
  const uint8_t* scale;   // pool rows [.][kScaleRow]
  int64_t M;
  PoolMap map;
  const int32_t* idx;     // [rows][K]
  int32_t K;
  const uint8_t* swa;     // [B][swa_rows][kD]
  int32_t W;
  int32_t swa_rows;       // rows per sequence in swa (Q + W - 1)
  int64_t pos0;           // prefill: position of query 0; window row t + r of query t is
                          // position pos0 + t - (W - 1) + r, rows before 0 are skipped
                          // (< 0: every row is a token; required for split launches)
  const uint16_t* q;      // [rows][kH][kD] bf16
  int32_t Q;              // query rows per sequence
  int32_t rows;           // B * Q
  float* opart;           // [rows][splits][kH][kD]  (split launches)
  float* ml;              // [rows][splits][kH][2]   (split launches)
  float* o;               // [rows][kH][kD]
  float* lse;             // [rows][kH]
  const float* o_in;      // NULL or [rows][kH][kD]
  const float* lse_in;    // NULL or [rows][kH]
};
// Steps of one row's keys.
int32_t attn_steps(int32_t K, int32_t W);
// The most splits a decode launch of `rows` rows uses (bounds its workspace).
int32_t attn_max_splits(int64_t rows, int32_t steps);
struct AttnPlan {
  int32_t splits;   // work-groups per row (1: one, writing o and lse itself)
  int32_t cps;      // decode: steps per work-group (0: the one-work-group-per-row kernel)
};
// Decode: splits per row from an estimate of the launch (splits > 1 needs the
// workspace of attn_ws_bytes).  AttnPlan{1, 0}: one work-group per row, no
// workspace (prefill).
AttnPlan attn_plan(int64_t rows, int32_t steps);
hipError_t launch_attn(const AttnArgs& a, const AttnPlan& plan, hipStream_t s);
// Decode attention workspace: per (row, split) one [kH][kD] unnormalised
// output and kH (reference, sum) pairs, for the splits attn_plan gives the
// shape (nothing when it takes one work-group per row).
struct AttnWs {
  float* opart;
  float* ml;
};
inline int64_t attn_ws_splits(int64_t rows, int32_t steps) {
  const AttnPlan p = attn_plan(rows, steps);
  return p.splits > 1 ? p.splits : 0;
}
inline size_t attn_ws_bytes(int64_t rows, int32_t steps) {
  const int64_t S = attn_ws_splits(rows, steps);
  return align256(rows * S * kH * kD * 4) + align256(rows * S * kH * 2 * 4);
}
inline AttnWs attn_ws_carve(void* ws, int64_t rows, int32_t steps) {
  const int64_t S = attn_ws_splits(rows, steps);
  AttnWs w;
  w.opart = (float*)ws;
  w.ml = (float*)((char*)ws + align256(rows * S * kH * kD * 4));
  return w;
}

// Write side: new pool entries (slot outside [0, M): skipped) and new window
// rows into a ring of W rows (only the last W of T tokens are written).
hipError_t launch_pool_append(uint8_t* latent, uint8_t* scale, uint8_t* idx_key, int32_t B,
                              int32_t M, const float* x_lat, const float* x_key, const int32_t* slot,
                              int32_t T, const PoolMap& map, hipStream_t s);
hipError_t launch_window_append(uint8_t* swa, int32_t B, int32_t W, const float* x, int64_t pos0,
                                int32_t T, hipStream_t s);

// Chunked prefill (Q > 1 query tokens per sequence), matrix-core kernels.
// Scores [B][Q][N] of pool entries 0 .. N-1 (N <= M) for every query (no
// candidate list, no histogram); invisible entries get -inf.  n_valid
// (optional, [B][Q]) receives each query's count of visible entries.  gmax
// (optional, [ceil(N / 128)][B Q][8]) receives the largest visible score of
// every run of 16 entries (-inf for a run the query cannot see), at
// [e / 128][b Q + q][e % 128 / 16] for the run starting at entry e.
hipError_t launch_prefill_score(const uint8_t* key, int32_t B, int64_t M, int32_t N,
                                const uint8_t* q_idx, const float* w_idx, int32_t Q, int64_t pos0,
                                int32_t ratio, float* scores, int32_t* n_valid, const int32_t* len,
                                const PoolMap& map, hipStream_t s, float* gmax = nullptr);
// Fill n 32-bit words with v.
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s);
// Copy n int32 (Reuse layers that ask for their indices).
hipError_t launch_copy_i32(int32_t* dst, const int32_t* src, int64_t n, hipStream_t s);

}  // namespace csa2

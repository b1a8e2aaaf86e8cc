// Host side of the C ABI: argument validation, workspace carving and the
// per-layer Full / Reindex / Reuse dispatch.  Every check runs before the
// first HIP call, so argument errors never touch the device.
#include "csa2.h"
#include "csa2_internal.h"

#include <mutex>

using namespace csa2;

namespace {

bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
constexpr int32_t kMinPageLog2 = 6;   // a scan wave's 64 entries lie in one page
bool al4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

csa2_status check_pool(const csa2_pool* p) {
  if (!p || !p->latent || !p->scale || !p->idx_key) return CSA2_ERR_NULL;
  if (p->B <= 0 || p->M <= 0 || p->M > kMaxTopkN) return CSA2_ERR_SHAPE;
  if (p->D != kD || p->HI != kHI || p->DI != kDI) return CSA2_ERR_SHAPE;
  if (p->pages && (p->page_log2 < kMinPageLog2 || p->page_log2 > 30 ||
                   (p->M & ((1 << p->page_log2) - 1)) != 0))
    return CSA2_ERR_SHAPE;
  if (!al16(p->latent) || !al16(p->scale) || !al16(p->idx_key) || !al4(p->len) ||
      !al4(p->pages))
    return CSA2_ERR_ALIGN;
  return CSA2_OK;
}

PoolMap pool_map(const csa2_pool* p) {
  PoolMap m{};
  m.pages = p->pages;
  m.lg2 = p->pages ? p->page_log2 : 0;
  m.np = p->pages ? p->M >> p->page_log2 : 0;
  return m;
}

csa2_status hip_status(hipError_t e) { return e == hipSuccess ? CSA2_OK : CSA2_ERR_HIP; }

constexpr int32_t kMaxW = 4096;
constexpr int32_t kMaxRows = 65535;  // grid.y limit for row-indexed launches

// Workspace of a stand-alone decode attention call (at least 256 bytes, as
// every call that takes a workspace asks for some).
size_t attn_call_ws_bytes(int64_t rows, int32_t steps) {
  const size_t b = attn_ws_bytes(rows, steps);
  return b > 256 ? b : 256;
}

// Top-K workspace: the sliced select's winners when it takes the shape,
// otherwise the multi-work-group scratch (nothing for the one-work-group
// row select).
size_t topk_call_ws_bytes(int64_t R, int64_t N, int64_t K) {
  if (topk_slicing(R, N, K).taken) {
    const size_t b = topk_slice_ws_bytes(R, N, K);
    return b > 256 ? b : 256;
  }
  return topk_multi_wg(R, N) ? topk_ws_bytes(R, N, K) : 256;
}

// Sliced-select winners for any row length up to Nmax (prefill chunks see a
// growing prefix of the pool).
size_t topk_slice_ws_max(int64_t R, int64_t Nmax, int64_t K) {
  // the keepers of a taken shape fit kFinalMaxN per row; many rows are never
  // sliced
  if (R >= kRowSplitR) return 0;
  size_t b = topk_slice_ws_bytes(R, Nmax, K);
  if (Nmax > kFinalMaxN) {
    const size_t cap = align256((size_t)(R * kFinalMaxN * 4)) * 2;
    b = b > cap ? b : cap;
  }
  return b;
}

// How a decode step selects: the sliced select for the Top-K (and for the
// Top-P of a hierarchical Full layer) when it takes the shape, otherwise
// the one-work-group row select or the multi-work-group select (`big`),
// whose histogram and counters live in the workspace.  (The fused score ->
// Top-K of csa2_score_topk is not used here: on the decode shapes its one
// 1024-thread work-group per compute unit streams the keys slower than the
// scan kernel's many small ones, more than the slice launch it saves.)
// A hierarchical Full layer whose Top-P the sliced select cannot take selects
// its Top-P and Top-K together with the threshold-bin select (`bin`) when the
// rows allow it.
struct DecodeSelect {
  bool sliced_k, sliced_p, bin, big;
};
DecodeSelect decode_select(int64_t B, int64_t M, int64_t K, int64_t P) {
  DecodeSelect d;
  d.sliced_k = topk_slicing(B, M, K).taken;
  d.sliced_p = P > 0 && topk_slicing(B, M, P).taken;
  d.bin = P > 0 && !d.sliced_p && topk_multi_wg(B, M) && topk_bin_taken(M);
  d.big = topk_multi_wg(B, M) && (!d.sliced_k || (P > 0 && !d.sliced_p && !d.bin));
  return d;
}

// decode_layers workspace: scores [B][N] | multi-work-group Top-K scratch
// (only when the select takes several work-groups per row; twice with a
// candidate pool, whose Top-P and the layer's Top-K are selected together)
// | candidate pool | attention partials.  The scans
// build no histogram: a fused one costs more in cross-XCD atomics than the
// 4 bytes per entry a Top-K pass reads (the row kernel builds its own from
// the row it holds; the multi-work-group select gets one histogram pass).
struct DecodeWs {
  float* scores;
  DecodeSelect sel;
  bool big;
  uint32_t* hist;  // threshold-bin select: the Full layer's histograms (topk_bin_hist_words)
  void* bin;       // threshold-bin select: kept elements per chunk
  void* slice;     // sliced-select winners
  TopkWs t;
  TopkWs t2;   // the Top-K's lists when the Top-P is selected beside it
  int32_t* cand;
  float* opart;
  float* ml;
};

size_t decode_slice_ws_bytes(int64_t B, int64_t M, int64_t K, int64_t P) {
  const DecodeSelect sel = decode_select(B, M, K, P);
  size_t b = sel.sliced_k ? topk_slice_ws_bytes(B, M, K) : 0;
  if (sel.sliced_p && topk_slice_ws_bytes(B, M, P) > b) b = topk_slice_ws_bytes(B, M, P);
  // a hierarchical Reindex layer selects K among its P candidates
  if (P > 0 && topk_slicing(B, P, K).S > 0 && topk_slice_ws_bytes(B, P, K) > b) b = topk_slice_ws_bytes(B, P, K);
  return b;
}

size_t decode_ws_bytes(int64_t B, int64_t M, int64_t K, int64_t P, int64_t W) {
  const int64_t N = P > M ? P : M;
  const int64_t Kmax = P > K ? P : K;
  const int32_t steps = attn_steps((int32_t)K, (int32_t)W);
  const DecodeSelect sel = decode_select(B, M, K, P);
  const bool big = sel.big;
  return align256(B * N * 4) + (big ? topk_ws_bytes(B, M, Kmax) : 0) +
         (big && P > 0 ? topk_ws_bytes(B, M, K) : 0) +
         (sel.bin ? align256(topk_bin_hist_words(B) * 4) + topk_bin_ws_bytes(B, M) : 0) +
         align256(B * (P > 0 ? P : 1) * 4) + decode_slice_ws_bytes(B, M, K, P) +
         attn_ws_bytes(B, steps);
}

DecodeWs decode_ws_carve(void* ws, int64_t B, int64_t M, int64_t K, int64_t P, int64_t W) {
  DecodeWs d{};
  const int64_t N = P > M ? P : M;
  const int64_t Kmax = P > K ? P : K;
  char* p = (char*)ws;
  d.scores = (float*)p;
  p += align256(B * N * 4);
  d.sel = decode_select(B, M, K, P);
  d.big = d.sel.big;
  if (d.big) {
    d.t = topk_ws_carve(p, B, M, Kmax);
    p += topk_ws_bytes(B, M, Kmax);
    if (P > 0) {
      d.t2 = topk_ws_carve(p, B, M, K);
      p += topk_ws_bytes(B, M, K);
    }
  }
  if (d.sel.bin) {
    d.hist = (uint32_t*)p;
    p += align256(topk_bin_hist_words(B) * 4);
    d.bin = p;
    p += topk_bin_ws_bytes(B, M);
  }
  d.cand = (int32_t*)p;
  p += align256(B * (P > 0 ? P : 1) * 4);
  d.slice = p;
  p += decode_slice_ws_bytes(B, M, K, P);
  const AttnWs w = attn_ws_carve(p, B, attn_steps((int32_t)K, (int32_t)W));
  d.opart = w.opart;
  d.ml = w.ml;
  return d;
}

// Multi-work-group Top-K on scores whose histogram is ready in t.hist (the
// counters are zero; the finish step leaves them zero again).
csa2_status select_rows_big(const float* scores, int32_t R, int32_t N, const int32_t* n_valid,
                            int32_t n_all, const int32_t* cand, int32_t K, int32_t* out,
                            const TopkWs& t, bool zero_hist, hipStream_t s) {
  return hip_status(launch_topk_select(scores, R, N, n_valid, n_all, cand, K, out, t, zero_hist, s));
}

// Zero the histogram and the per-row counters (adjacent in the workspace).
csa2_status zero_hist_counters(const TopkWs& t, int64_t R, hipStream_t s) {
  const int64_t words = (int64_t)((char*)t.counters - (char*)t.hist) / 4 + R * kCounterWords;
  return hip_status(launch_fill_zero(t.hist, words, s));
}

// Mode schedule and per-layer arguments of a layer array (decode or prefill).
csa2_status check_layers(const csa2_layer* layers, int32_t L, int32_t W) {
  if (layers[0].mode != CSA2_FULL) return CSA2_ERR_SCHEDULE;
  for (int32_t l = 0; l < L; ++l) {
    const csa2_layer& y = layers[l];
    if (y.mode != CSA2_FULL && y.mode != CSA2_REINDEX && y.mode != CSA2_REUSE)
      return CSA2_ERR_SCHEDULE;
    if (!y.q || !y.o || !y.lse) return CSA2_ERR_NULL;
    if (W > 0 && !y.swa) return CSA2_ERR_NULL;
    if (y.mode != CSA2_REUSE && (!y.q_idx || !y.w_idx || !y.idx_out)) return CSA2_ERR_NULL;
    if (!al16(y.q) || !al16(y.o) || !al4(y.lse) || (y.swa && !al16(y.swa)) ||
        (y.q_idx && y.mode != CSA2_REUSE && !al16(y.q_idx)) ||
        (y.w_idx && y.mode != CSA2_REUSE && !al4(y.w_idx)) || (y.idx_out && !al4(y.idx_out)))
      return CSA2_ERR_ALIGN;
  }
  return CSA2_OK;
}

// Whether a prefill chunk of R rows of N positions takes the group select.
inline bool prefill_group(int64_t R, int64_t N, int64_t K) {
  return R >= kRowSplitR && topk_group_taken(N, K);
}

// prefill_layers workspace: scores [B*Q][M] (a chunk uses a row length N <= M)
// | visible counts [B*Q] | multi-work-group Top-K scratch when the rows are
// few and long | sliced-select keepers | run maxima [B*Q][runs] of the group
// select.
size_t prefill_ws_bytes(int64_t B, int64_t Q, int64_t M, int64_t K) {
  const int64_t R = B * Q;
  const bool grp = R >= kRowSplitR && M > kFinalMaxN && K > 0 && K <= 512;   // some N <= M takes it
  return align256(R * M * 4) + align256(R * 4) + (topk_multi_wg(R, M) ? topk_ws_bytes(R, M, K) : 0) +
         topk_slice_ws_max(R, M, K) +
         (grp ? align256((size_t)R * topk_group_runs(M < 16 * 8192 ? M : 16 * 8192) * 4) : 0);
}

// Entries that some query of a chunk can see, rounded up to a multiple of 4
// (at most M) so that score rows stay 16-byte aligned: the score row length.
int64_t prefill_scan_entries(int64_t M, int32_t Q, int64_t pos0, int32_t ratio) {
  int64_t v = pos0 < 0 ? M : (pos0 + Q) / ratio;
  if (v > M) v = M;
  v = (v + 3) & ~int64_t(3);
  return v < M ? v : M;
}

}  // namespace

extern "C" {

const char* csa2_status_string(csa2_status s) {
  switch (s) {
    case CSA2_OK: return "ok";
    case CSA2_ERR_NULL: return "required pointer is NULL";
    case CSA2_ERR_SHAPE: return "size out of range or unsupported";
    case CSA2_ERR_ALIGN: return "pointer not 16-byte aligned";
    case CSA2_ERR_SCHEDULE: return "invalid layer mode schedule";
    case CSA2_ERR_WORKSPACE: return "workspace missing or too small";
    case CSA2_ERR_HIP: return "HIP launch or runtime error";
    case CSA2_ERR_SCRATCH: return "step needs more than the library's static scratch";
  }
  return "unknown status";
}

const char* csa2_version(void) { return "csa2-mi355x 0.1.0 gfx950"; }

size_t csa2_workspace_bytes(int op, int32_t B, int32_t Q, int32_t M, int32_t K, int32_t P,
                            int32_t W, int32_t H) {
  if (B <= 0 || Q <= 0) return 0;
  switch (op) {
    case CSA2_OP_TOPK:
      if (M <= 0 || K <= 0 || K > kMaxK || M > kMaxTopkN) return 0;
      return topk_call_ws_bytes(B, M, K);
    case CSA2_OP_SPARSE_ATTN:
      if (K <= 0 || K > kMaxK || H != kH) return 0;
      return Q > 1 ? 256 : attn_call_ws_bytes((int64_t)B * Q, attn_steps(K, 0));
    case CSA2_OP_SWA_MERGE:
      if (W < 0 || W > kMaxW || H != kH) return 0;
      return Q > 1 ? 256 : attn_call_ws_bytes((int64_t)B * Q, attn_steps(0, W));
    case CSA2_OP_PREFILL_LAYERS:
      if (M <= 0 || K <= 0 || K > kMaxK || W < 0 || W > kMaxW || H != kH ||
          (int64_t)B * Q > kMaxRows)
        return 0;
      return prefill_ws_bytes(B, Q, M, K);
    case CSA2_OP_DECODE_LAYERS:
      if (M <= 0 || K <= 0 || K > kMaxK || P < 0 || P > kMaxK || (P > 0 && P < K) ||
          W < 0 || W > kMaxW || H != kH)
        return 0;
      return decode_ws_bytes(B, M, K, P, W);
    case CSA2_OP_SCORE_TOPK:
      if (K <= 0 || K > kMaxK || M > kMaxTopkN || !score_topk_slicing(B, M, K).taken) return 0;
      return score_topk_ws_bytes(B, M, K);
  }
  return 0;
}

csa2_status csa2_index_score(const csa2_pool* pool, const uint8_t* q_idx, const float* w_idx,
                             int32_t Q, int64_t pos0, int32_t ratio, const int32_t* cand,
                             int32_t P, float* scores, uint32_t* hist, hipStream_t stream) {
  csa2_status st = check_pool(pool);
  if (st != CSA2_OK) return st;
  if (!q_idx || !w_idx || !scores) return CSA2_ERR_NULL;
  if (Q <= 0 || (int64_t)pool->B * Q > kMaxRows) return CSA2_ERR_SHAPE;
  if (pos0 >= 0 && ratio <= 0) return CSA2_ERR_SHAPE;
  if (cand && (P <= 0 || P > kMaxTopkN)) return CSA2_ERR_SHAPE;
  if (!al16(q_idx) || !al4(w_idx) || !al4(scores) || (hist && !al4(hist)) || (cand && !al4(cand)))
    return CSA2_ERR_ALIGN;
  if (Q > 1 && !cand) {   // chunked prefill: matrix-core contraction
    if (hist) return CSA2_ERR_SHAPE;
    return hip_status(launch_prefill_score(pool->idx_key, pool->B, pool->M, pool->M, q_idx, w_idx,
                                           Q, pos0, pos0 >= 0 ? ratio : 1, scores, nullptr,
                                           pool->len, pool_map(pool), stream));
  }
  const int32_t N = cand ? P : pool->M;
  return hip_status(launch_index_score(pool->idx_key, pool->B, pool->M, q_idx, w_idx, Q, pos0,
                                       pos0 >= 0 ? ratio : 1, cand, N, scores, hist, pool->len,
                                       pool_map(pool), stream));
}

csa2_status csa2_topk(const float* scores, int32_t R, int32_t N, const int32_t* n_valid,
                      const int32_t* cand, int32_t K, int32_t* idx, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  if (!scores || !idx) return CSA2_ERR_NULL;
  if (R <= 0 || R > kMaxRows || N <= 0 || N > kMaxTopkN || K <= 0 || K > kMaxK)
    return CSA2_ERR_SHAPE;
  if (!al4(scores) || !al4(idx) || (n_valid && !al4(n_valid)) || (cand && !al4(cand)))
    return CSA2_ERR_ALIGN;
  if (!ws || ws_bytes < topk_call_ws_bytes(R, N, K)) return CSA2_ERR_WORKSPACE;
  if (!al16(ws)) return CSA2_ERR_ALIGN;
  if (topk_slicing(R, N, K).taken)
    return hip_status(launch_topk_sliced(scores, R, N, n_valid, N, cand, K, idx, ws, stream));
  if (!topk_multi_wg(R, N))
    return hip_status(launch_topk_rows(scores, R, N, n_valid, N, K, nullptr, false, cand, idx,
                                       stream));
  const TopkWs t = topk_ws_carve(ws, R, N, K);
  csa2_status st = zero_hist_counters(t, R, stream);
  if (st != CSA2_OK) return st;
  st = hip_status(launch_topk_hist(scores, R, N, n_valid, N, t.hist, stream));
  if (st != CSA2_OK) return st;
  return hip_status(launch_topk_select(scores, R, N, n_valid, N, cand, K, idx, t, false, stream));
}

csa2_status csa2_score_topk(const csa2_pool* pool, const uint8_t* q_idx, const float* w_idx,
                            int32_t K, int32_t* idx, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  csa2_status st = check_pool(pool);
  if (st != CSA2_OK) return st;
  if (!q_idx || !w_idx || !idx) return CSA2_ERR_NULL;
  if (pool->B > kMaxRows || pool->M > kMaxTopkN || K <= 0 || K > kMaxK ||
      !score_topk_slicing(pool->B, pool->M, K).taken)
    return CSA2_ERR_SHAPE;
  if (!al16(q_idx) || !al4(w_idx) || !al4(idx)) return CSA2_ERR_ALIGN;
  if (!ws || ws_bytes < score_topk_ws_bytes(pool->B, pool->M, K)) return CSA2_ERR_WORKSPACE;
  if (!al16(ws)) return CSA2_ERR_ALIGN;
  return hip_status(launch_score_topk(pool->idx_key, pool->B, pool->M, q_idx, w_idx, pool->len,
                                      pool_map(pool), K, idx, ws, stream));
}

// Attention of `rows` query rows in the workspace of a stand-alone call:
// split decode rows (Q == 1), one work-group per token for a prefill chunk.
static csa2_status attend_rows(AttnArgs& a, void* ws, int64_t rows, int32_t steps,
                               hipStream_t stream) {
  if (a.Q > 1) return hip_status(launch_attn(a, AttnPlan{1, 0}, stream));
  const AttnWs w = attn_ws_carve(ws, rows, steps);
  a.opart = w.opart;
  a.ml = w.ml;
  return hip_status(launch_attn(a, attn_plan(rows, steps), stream));
}

csa2_status csa2_sparse_attn(const csa2_pool* pool, const uint16_t* q, int32_t Q, int32_t H,
                             const int32_t* idx, int32_t K, float* o, float* lse, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  csa2_status st = check_pool(pool);
  if (st != CSA2_OK) return st;
  if (!q || !idx || !o || !lse) return CSA2_ERR_NULL;
  if (Q <= 0 || H != kH || K <= 0 || K > kMaxK || (int64_t)pool->B * Q > kMaxRows)
    return CSA2_ERR_SHAPE;
  if (!al16(q) || !al4(idx) || !al16(o) || !al4(lse)) return CSA2_ERR_ALIGN;
  const int64_t rows = (int64_t)pool->B * Q;
  const int32_t steps = attn_steps(K, 0);
  const size_t need = Q > 1 ? 256 : attn_call_ws_bytes(rows, steps);
  if (!ws || ws_bytes < need) return CSA2_ERR_WORKSPACE;
  if (!al16(ws)) return CSA2_ERR_ALIGN;
  AttnArgs a{};
  a.latent = pool->latent;
  a.scale = pool->scale;
  a.M = pool->M;
  a.map = pool_map(pool);
  a.idx = idx;
  a.K = K;
  a.swa = nullptr;
  a.W = 0;
  a.swa_rows = 0;
  a.pos0 = -1;
  a.q = q;
  a.Q = Q;
  a.rows = (int32_t)rows;
  a.o = o;
  a.lse = lse;
  a.o_in = nullptr;
  a.lse_in = nullptr;
  return attend_rows(a, ws, rows, steps, stream);
}

csa2_status csa2_swa_merge(const uint16_t* q, int32_t B, int32_t Q, int32_t H, int32_t D,
                           const uint8_t* swa, int32_t W, float* o, float* lse, void* ws,
                           size_t ws_bytes, hipStream_t stream) {
  if (!q || !o || !lse) return CSA2_ERR_NULL;
  if (B <= 0 || Q <= 0 || H != kH || D != kD || W < 0 || W > kMaxW ||
      (int64_t)B * Q > kMaxRows)
    return CSA2_ERR_SHAPE;
  if (W > 0 && !swa) return CSA2_ERR_NULL;
  if (!al16(q) || !al16(o) || !al4(lse) || (swa && !al16(swa))) return CSA2_ERR_ALIGN;
  const int64_t rows = (int64_t)B * Q;
  const int32_t steps = attn_steps(0, W);
  if (!ws || ws_bytes < (Q > 1 ? 256 : attn_call_ws_bytes(rows, steps))) return CSA2_ERR_WORKSPACE;
  if (!al16(ws)) return CSA2_ERR_ALIGN;
  if (W == 0) return CSA2_OK;  // nothing to merge: (o, lse) unchanged
  AttnArgs a{};
  a.latent = nullptr;
  a.scale = nullptr;
  a.M = 0;
  a.idx = nullptr;
  a.K = 0;
  a.swa = swa;
  a.W = W;
  a.swa_rows = Q + W - 1;
  a.pos0 = -1;
  a.q = q;
  a.Q = Q;
  a.rows = (int32_t)rows;
  a.o = o;
  a.lse = lse;
  a.o_in = o;
  a.lse_in = lse;
  return attend_rows(a, ws, rows, steps, stream);
}

}  // extern "C"

namespace {

// Argument checks shared by the decode entry points: the pool, the sizes and
// the schedule.
csa2_status check_decode_args(const csa2_pool* pool, const csa2_layer* layers, int32_t L,
                              int32_t H, int32_t K, int32_t P, int32_t W) {
  csa2_status st = check_pool(pool);
  if (st != CSA2_OK) return st;
  if (!layers) return CSA2_ERR_NULL;
  if (L <= 0 || H != kH || K <= 0 || K > kMaxK || P < 0 || P > kMaxK || (P > 0 && P < K) ||
      W < 0 || W > kMaxW || pool->B > kMaxRows)
    return CSA2_ERR_SHAPE;
  return check_layers(layers, L, W);
}

// ... and the caller's workspace.
csa2_status check_decode(const csa2_pool* pool, const csa2_layer* layers, int32_t L, int32_t H,
                         int32_t K, int32_t P, int32_t W, void* ws, size_t ws_bytes) {
  const csa2_status st = check_decode_args(pool, layers, L, H, K, P, W);
  if (st != CSA2_OK) return st;
  if (!ws || ws_bytes < decode_ws_bytes(pool->B, pool->M, K, P, W)) return CSA2_ERR_WORKSPACE;
  if (!al16(ws)) return CSA2_ERR_ALIGN;
  return CSA2_OK;
}

// The layer whose indices layer l uses: itself (Full / Reindex) or the most
// recent Full or Reindex layer before it (layer 0 is Full).
int32_t source_layer(const csa2_layer* layers, int32_t l) {
  int32_t s = l;
  while (s > 0 && layers[s].mode == CSA2_REUSE) --s;
  return s;
}

// Layer l of a decode step: its index work (Full / Reindex), the copy a
// Reuse layer asks for, and its attention.  zero: what a Full (or flat
// Reindex) layer's scan clears on the side for its selects.
csa2_status decode_one(const csa2_pool* pool, const csa2_layer* layers, int32_t l, int32_t K,
                       int32_t P, int32_t W, const DecodeWs& d, const AttnPlan& plan,
                       const ZeroSpans* zero, hipStream_t stream) {
  const int64_t B = pool->B, M = pool->M;
  const int32_t n_cand = (int32_t)(P < M ? P : M);
  const csa2_layer& y = layers[l];
  csa2_status st = CSA2_OK;
  if (y.mode == CSA2_FULL || (y.mode == CSA2_REINDEX && P == 0)) {
    st = hip_status(launch_index_score(pool->idx_key, (int32_t)B, M, y.q_idx, y.w_idx, 1, -1, 1,
                                       nullptr, (int32_t)M, d.scores, nullptr, pool->len,
                                       pool_map(pool), stream, zero));
    if (st != CSA2_OK) return st;
    const bool want_p = y.mode == CSA2_FULL && P > 0;
    if (want_p && d.sel.bin) {
      // Top-P and the layer's Top-K from one histogram and one collect pass
      st = hip_status(launch_topk_hist(d.scores, (int32_t)B, (int32_t)M, pool->len, (int32_t)M,
                                       d.hist, stream));
      if (st != CSA2_OK) return st;
      st = hip_status(launch_topk_bin_select(d.scores, (int32_t)B, (int32_t)M, pool->len,
                                             (int32_t)M, d.hist, P, d.cand, K, y.idx_out, d.bin,
                                             stream));
    } else if (d.sel.sliced_k && (!want_p || d.sel.sliced_p)) {
      if (want_p) {
        st = hip_status(launch_topk_sliced(d.scores, (int32_t)B, (int32_t)M, pool->len, (int32_t)M,
                                           nullptr, P, d.cand, d.slice, stream));
        if (st != CSA2_OK) return st;
      }
      st = hip_status(launch_topk_sliced(d.scores, (int32_t)B, (int32_t)M, pool->len, (int32_t)M,
                                         nullptr, K, y.idx_out, d.slice, stream));
    } else if (!d.big) {
      if (want_p) {
        st = hip_status(launch_topk_rows(d.scores, (int32_t)B, (int32_t)M, pool->len, (int32_t)M, P,
                                         nullptr, false, nullptr, d.cand, stream));
        if (st != CSA2_OK) return st;
      }
      st = hip_status(launch_topk_rows(d.scores, (int32_t)B, (int32_t)M, pool->len, (int32_t)M, K,
                                       nullptr, false, nullptr, y.idx_out, stream));
    } else {
      st = hip_status(launch_topk_hist(d.scores, (int32_t)B, (int32_t)M, pool->len, (int32_t)M,
                                       d.t.hist, stream));
      if (st != CSA2_OK) return st;
      if (want_p) {
        // Top-P and the layer's Top-K from one histogram, one collect pass
        // over the scores and one finish launch (the two selects of a row
        // run on two work-groups side by side)
        st = hip_status(launch_topk_select2(d.scores, (int32_t)B, (int32_t)M, pool->len,
                                            (int32_t)M, P, d.cand, d.t, K, y.idx_out, d.t2, true,
                                            stream));
      } else {
        st = select_rows_big(d.scores, (int32_t)B, (int32_t)M, pool->len, (int32_t)M, nullptr, K,
                             y.idx_out, d.t, true, stream);
      }
    }
    if (st != CSA2_OK) return st;
  } else if (y.mode == CSA2_REINDEX) {  // hierarchical: score inside the candidate pool
    st = hip_status(launch_index_score(pool->idx_key, (int32_t)B, M, y.q_idx, y.w_idx, 1, -1, 1,
                                       d.cand, P, d.scores, nullptr, pool->len, pool_map(pool),
                                       stream));
    if (st != CSA2_OK) return st;
    // a ragged sequence has min(P, len) candidates (the selects clamp len to P)
    if (topk_slicing(B, P, K).taken)
      st = hip_status(launch_topk_sliced(d.scores, (int32_t)B, P, pool->len, n_cand, d.cand, K,
                                         y.idx_out, d.slice, stream));
    else
      st = hip_status(launch_topk_rows(d.scores, (int32_t)B, P, pool->len, n_cand, K, nullptr,
                                       false, d.cand, y.idx_out, stream));
    if (st != CSA2_OK) return st;
  }
  const int32_t* cur = layers[source_layer(layers, l)].idx_out;
  if (y.mode == CSA2_REUSE && y.idx_out && y.idx_out != cur) {
    st = hip_status(launch_copy_i32(y.idx_out, cur, B * K, stream));
    if (st != CSA2_OK) return st;
  }

  AttnArgs a{};
  a.latent = pool->latent;
  a.scale = pool->scale;
  a.M = M;
  a.map = pool_map(pool);
  a.idx = cur;
  a.K = K;
  a.swa = y.swa;
  a.W = W;
  a.swa_rows = W;
  a.pos0 = -1;
  a.q = y.q;
  a.Q = 1;
  a.rows = (int32_t)B;
  a.opart = d.opart;
  a.ml = d.ml;
  a.o_in = nullptr;
  a.lse_in = nullptr;
  a.o = y.o;
  a.lse = y.lse;
  return hip_status(launch_attn(a, plan, stream));
}

// What a Full layer's selects need zeroed on entry: the multi-work-group
// select's histograms and counters (which it leaves zeroed again) and the
// threshold-bin select's histograms (which it leaves filled).  The layer's
// scan clears them on the side; nullptr when nothing is needed.
const ZeroSpans* full_layer_zero(const DecodeWs& d, int64_t B, int32_t P, ZeroSpans* z) {
  *z = ZeroSpans{{nullptr, nullptr, nullptr}, {0, 0, 0}};
  int k = 0;
  auto add = [&](uint32_t* p, int64_t n) {
    z->p[k] = p;
    z->n[k] = n;
    ++k;
  };
  auto hist_counters = [&](const TopkWs& t) {
    return (int64_t)((char*)t.counters - (char*)t.hist) / 4 + B * kCounterWords;
  };
  if (d.big) {
    add(d.t.hist, hist_counters(d.t));
    if (P > 0) add(d.t2.hist, hist_counters(d.t2));
  }
  if (d.sel.bin) add(d.hist, topk_bin_hist_words(B));
  return k > 0 ? z : nullptr;
}

// Every layer of a decode step on a checked, large enough workspace.  What
// must start at zero (the selects' histograms and counters) is cleared by
// each Full layer's scan on the side, a kernel like every other step of the
// call (so the call can be captured in a graph); everything else in the
// workspace is written before it is read.
csa2_status decode_step(const csa2_pool* pool, const csa2_layer* layers, int32_t L, int32_t K,
                        int32_t P, int32_t W, int32_t* src_layer, void* ws, hipStream_t stream) {
  const int64_t B = pool->B;
  const DecodeWs d = decode_ws_carve(ws, B, pool->M, K, P, W);
  const AttnPlan plan = attn_plan(B, attn_steps(K, W));
  ZeroSpans zs;
  const ZeroSpans* zero = full_layer_zero(d, B, P, &zs);
  csa2_status st = CSA2_OK;
  for (int32_t l = 0; l < L; ++l) {
    st = decode_one(pool, layers, l, K, P, W, d, plan, zero, stream);
    if (st != CSA2_OK) return st;
    if (src_layer) src_layer[l] = source_layer(layers, l);
  }
  return CSA2_OK;
}

}  // namespace

// Workspace of csa2_decode_layers_noalloc: one array per GPU in the
// library's own device memory, held from the library's load on that GPU to
// the end of the process.  Host code never hands the array's name to a
// kernel or a copy (on the host it names a stand-in, not device memory): it
// asks HIP for the array's address on each device once and uses that.
static __device__ __align__(256) uint8_t scratch[CSA2_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kScratchBytes = CSA2_NOALLOC_SCRATCH_BYTES;
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchDevices] = {};

// The array's address on the current device (looked up on the first call
// made with that device current), or a HIP error.
hipError_t scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

csa2_status csa2_decode_layers(const csa2_pool* pool, const csa2_layer* layers, int32_t L,
                               int32_t H, int32_t K, int32_t P, int32_t W, int32_t* src_layer,
                               void* ws, size_t ws_bytes, hipStream_t stream) {
  const csa2_status st = check_decode(pool, layers, L, H, K, P, W, ws, ws_bytes);
  if (st != CSA2_OK) return st;
  return decode_step(pool, layers, L, K, P, W, src_layer, ws, stream);
}

csa2_status csa2_decode_layer(const csa2_pool* pool, const csa2_layer* layers, int32_t L,
                              int32_t l, int32_t H, int32_t K, int32_t P, int32_t W,
                              int32_t* src_layer, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (l < 0 || l >= L) return CSA2_ERR_SHAPE;
  csa2_status st = check_decode(pool, layers, L, H, K, P, W, ws, ws_bytes);
  if (st != CSA2_OK) return st;
  const int64_t B = pool->B;
  const DecodeWs d = decode_ws_carve(ws, B, pool->M, K, P, W);
  const AttnPlan plan = attn_plan(B, attn_steps(K, W));
  const csa2_layer& y = layers[l];
  ZeroSpans zs;
  const ZeroSpans* zero = (y.mode == CSA2_FULL || (y.mode == CSA2_REINDEX && P == 0))
                              ? full_layer_zero(d, B, P, &zs) : nullptr;
  st = decode_one(pool, layers, l, K, P, W, d, plan, zero, stream);
  if (st == CSA2_OK && src_layer) *src_layer = source_layer(layers, l);
  return st;
}

csa2_status csa2_decode_layers_noalloc(const csa2_pool* pool, const csa2_layer* layers,
                                       int32_t L, int32_t H, int32_t K, int32_t P, int32_t W,
                                       int32_t* src_layer, hipStream_t stream) {
  const csa2_status st = check_decode_args(pool, layers, L, H, K, P, W);
  if (st != CSA2_OK) return st;
  if (decode_ws_bytes(pool->B, pool->M, K, P, W) > kScratchBytes) return CSA2_ERR_SCRATCH;
  void* ws = nullptr;
  const hipError_t e = scratch_on_current_device(&ws);
  if (e != hipSuccess) return CSA2_ERR_HIP;
  return decode_step(pool, layers, L, K, P, W, src_layer, ws, stream);
}

csa2_status csa2_prefill_layers(const csa2_pool* pool, const csa2_layer* layers, int32_t L,
                                int32_t Q, int64_t pos0, int32_t ratio, int32_t H, int32_t K,
                                int32_t W, int32_t* src_layer, void* ws, size_t ws_bytes,
                                hipStream_t stream) {
  csa2_status st = check_pool(pool);
  if (st != CSA2_OK) return st;
  if (!layers) return CSA2_ERR_NULL;
  if (L <= 0 || Q <= 0 || H != kH || K <= 0 || K > kMaxK || W < 0 || W > kMaxW ||
      (int64_t)pool->B * Q > kMaxRows || (pos0 >= 0 && ratio <= 0))
    return CSA2_ERR_SHAPE;
  st = check_layers(layers, L, W);
  if (st != CSA2_OK) return st;
  const int64_t B = pool->B, M = pool->M, R = B * Q;
  if (!ws || ws_bytes < prefill_ws_bytes(B, Q, M, K)) return CSA2_ERR_WORKSPACE;
  if (!al16(ws)) return CSA2_ERR_ALIGN;

  // A chunk scores only the entries its last query can see (early chunks of
  // a growing pool see a prefix); none visible: no index work at all.
  const int64_t N = prefill_scan_entries(M, Q, pos0, ratio);
  char* p = (char*)ws;
  float* scores = (float*)p;
  p += align256(R * M * 4);
  int32_t* n_valid = (int32_t*)p;
  p += align256(R * 4);
  const bool grp = N > 0 && prefill_group(R, N, K);
  const bool sliced = N > 0 && !grp && topk_slicing(R, N, K).taken;
  const bool big = N > 0 && !grp && !sliced && topk_multi_wg(R, N);
  const TopkWs t = big ? topk_ws_carve(p, R, N, K) : TopkWs{};
  void* slice_ws = p + (topk_multi_wg(R, M) ? topk_ws_bytes(R, M, K) : 0);
  float* gmax = grp ? (float*)((char*)slice_ws + topk_slice_ws_max(R, M, K)) : nullptr;

  const int32_t* cur = nullptr;
  int32_t cur_layer = -1;
  for (int32_t l = 0; l < L; ++l) {
    const csa2_layer& y = layers[l];
    if (y.mode == CSA2_FULL || y.mode == CSA2_REINDEX) {
      if (N == 0) {
        st = hip_status(launch_fill_u32((uint32_t*)y.idx_out, R * K, 0xFFFFFFFFu, stream));
      } else {
        st = hip_status(launch_prefill_score(pool->idx_key, (int32_t)B, M, (int32_t)N, y.q_idx,
                                             y.w_idx, Q, pos0, pos0 >= 0 ? ratio : 1, scores,
                                             n_valid, pool->len, pool_map(pool), stream, gmax));
        if (st != CSA2_OK) return st;
        if (grp) {
          st = hip_status(launch_topk_group(scores, gmax, (int32_t)R, (int32_t)N, n_valid,
                                            (int32_t)N, K, y.idx_out, stream));
        } else if (sliced) {
          st = hip_status(launch_topk_sliced(scores, (int32_t)R, (int32_t)N, n_valid, (int32_t)N,
                                             nullptr, K, y.idx_out, slice_ws, stream));
        } else if (!big) {
          st = hip_status(launch_topk_rows(scores, (int32_t)R, (int32_t)N, n_valid, (int32_t)N, K,
                                           nullptr, false, nullptr, y.idx_out, stream));
        } else {
          st = zero_hist_counters(t, R, stream);
          if (st != CSA2_OK) return st;
          st = hip_status(launch_topk_hist(scores, (int32_t)R, (int32_t)N, n_valid, (int32_t)N,
                                           t.hist, stream));
          if (st != CSA2_OK) return st;
          st = hip_status(launch_topk_select(scores, (int32_t)R, (int32_t)N, n_valid, (int32_t)N,
                                             nullptr, K, y.idx_out, t, false, stream));
        }
      }
      if (st != CSA2_OK) return st;
      cur = y.idx_out;
      cur_layer = l;
    } else if (y.idx_out && y.idx_out != cur) {  // Reuse that asks for its indices
      st = hip_status(launch_copy_i32(y.idx_out, cur, R * K, stream));
      if (st != CSA2_OK) return st;
    }
    if (src_layer) src_layer[l] = cur_layer;

    // the selected entries and the window rows in one pass (one softmax)
    AttnArgs a{};
    a.latent = pool->latent;
    a.scale = pool->scale;
    a.M = M;
    a.map = pool_map(pool);
    a.idx = cur;
    a.K = N > 0 ? K : 0;
    a.swa = y.swa;
    a.W = W;
    a.swa_rows = Q + W - 1;
    a.pos0 = pos0;
    a.q = y.q;
    a.Q = Q;
    a.rows = (int32_t)R;
    a.o = y.o;
    a.lse = y.lse;
    a.o_in = nullptr;
    a.lse_in = nullptr;
    st = hip_status(launch_attn(a, AttnPlan{1, 0}, stream));
    if (st != CSA2_OK) return st;
  }
  return CSA2_OK;
}

csa2_status csa2_pool_append(uint8_t* latent, uint8_t* scale, uint8_t* idx_key, int32_t B,
                             int32_t M, const float* x_latent, const float* x_key,
                             const int32_t* slot, int32_t T, const int32_t* pages,
                             int32_t page_log2, hipStream_t stream) {
  if (!latent || !scale || !idx_key || !x_latent || !x_key || !slot) return CSA2_ERR_NULL;
  if (B <= 0 || M <= 0 || T < 0) return CSA2_ERR_SHAPE;
  if (pages && (page_log2 < kMinPageLog2 || page_log2 > 30 || (M & ((1 << page_log2) - 1)) != 0))
    return CSA2_ERR_SHAPE;
  if (!al16(x_latent) || !al16(x_key) || !al4(slot) || ((uintptr_t)latent & 7u) ||
      ((uintptr_t)idx_key & 7u) || !al4(pages))
    return CSA2_ERR_ALIGN;
  if (T == 0) return CSA2_OK;
  PoolMap map{};
  map.pages = pages;
  map.lg2 = pages ? page_log2 : 0;
  map.np = pages ? M >> page_log2 : 0;
  return hip_status(launch_pool_append(latent, scale, idx_key, B, M, x_latent, x_key, slot, T, map,
                                       stream));
}

// Host tier: one sequence's entries (or window ring) between page-locked host
// memory and the device arrays, by the copy engines on the caller's stream.
static csa2_status pool_transfer(uint8_t* latent, uint8_t* scale, uint8_t* idx_key, int32_t B,
                                 int32_t M, int32_t seq, int32_t entry0, int32_t n,
                                 uint8_t* h_latent, uint8_t* h_scale, uint8_t* h_key, bool to_device,
                                 hipStream_t stream) {
  if (!latent || !scale || !idx_key || !h_latent || !h_scale || !h_key) return CSA2_ERR_NULL;
  if (B <= 0 || M <= 0 || seq < 0 || seq >= B || entry0 < 0 || n < 0 || (int64_t)entry0 + n > M)
    return CSA2_ERR_SHAPE;
  if (n == 0) return CSA2_OK;
  const size_t e0 = (size_t)seq * (size_t)M + (size_t)entry0;
  const hipMemcpyKind kind = to_device ? hipMemcpyHostToDevice : hipMemcpyDeviceToHost;
  const struct { uint8_t* dev; uint8_t* host; size_t row; } parts[3] = {
      {latent, h_latent, (size_t)kLatRow}, {scale, h_scale, (size_t)kScaleRow},
      {idx_key, h_key, (size_t)kKeyRow}};
  for (const auto& q : parts) {
    uint8_t* d = q.dev + e0 * q.row;
    const size_t bytes = (size_t)n * q.row;
    const hipError_t e = to_device ? hipMemcpyAsync(d, q.host, bytes, kind, stream)
                                   : hipMemcpyAsync(q.host, d, bytes, kind, stream);
    if (e != hipSuccess) return CSA2_ERR_HIP;
  }
  return CSA2_OK;
}

csa2_status csa2_pool_restore(uint8_t* latent, uint8_t* scale, uint8_t* idx_key, int32_t B,
                              int32_t M, int32_t seq, int32_t entry0, int32_t n,
                              const uint8_t* h_latent, const uint8_t* h_scale, const uint8_t* h_key,
                              hipStream_t stream) {
  return pool_transfer(latent, scale, idx_key, B, M, seq, entry0, n, const_cast<uint8_t*>(h_latent),
                       const_cast<uint8_t*>(h_scale), const_cast<uint8_t*>(h_key), true, stream);
}

csa2_status csa2_pool_offload(const uint8_t* latent, const uint8_t* scale, const uint8_t* idx_key,
                              int32_t B, int32_t M, int32_t seq, int32_t entry0, int32_t n,
                              uint8_t* h_latent, uint8_t* h_scale, uint8_t* h_key,
                              hipStream_t stream) {
  return pool_transfer(const_cast<uint8_t*>(latent), const_cast<uint8_t*>(scale),
                       const_cast<uint8_t*>(idx_key), B, M, seq, entry0, n, h_latent, h_scale, h_key,
                       false, stream);
}

static csa2_status swa_transfer(uint8_t* swa, int32_t B, int32_t W, int32_t seq, uint8_t* h_swa,
                                bool to_device, hipStream_t stream) {
  if (!swa || !h_swa) return CSA2_ERR_NULL;
  if (B <= 0 || W <= 0 || seq < 0 || seq >= B) return CSA2_ERR_SHAPE;
  uint8_t* d = swa + (size_t)seq * (size_t)W * kD;
  const size_t bytes = (size_t)W * kD;
  const hipError_t e = to_device ? hipMemcpyAsync(d, h_swa, bytes, hipMemcpyHostToDevice, stream)
                                 : hipMemcpyAsync(h_swa, d, bytes, hipMemcpyDeviceToHost, stream);
  return e == hipSuccess ? CSA2_OK : CSA2_ERR_HIP;
}

csa2_status csa2_swa_restore(uint8_t* swa, int32_t B, int32_t W, int32_t seq, const uint8_t* h_swa,
                             hipStream_t stream) {
  return swa_transfer(swa, B, W, seq, const_cast<uint8_t*>(h_swa), true, stream);
}

csa2_status csa2_swa_offload(const uint8_t* swa, int32_t B, int32_t W, int32_t seq, uint8_t* h_swa,
                             hipStream_t stream) {
  return swa_transfer(const_cast<uint8_t*>(swa), B, W, seq, h_swa, false, stream);
}

csa2_status csa2_swa_append(uint8_t* swa, int32_t B, int32_t W, const float* x, int64_t pos0,
                            int32_t T, hipStream_t stream) {
  if (!swa || !x) return CSA2_ERR_NULL;
  if (B <= 0 || W <= 0 || T < 0 || pos0 < 0) return CSA2_ERR_SHAPE;
  if (!al16(x) || ((uintptr_t)swa & 7u)) return CSA2_ERR_ALIGN;
  if (T == 0) return CSA2_OK;
  return hip_status(launch_window_append(swa, B, W, x, pos0, T, stream));
}

}  // extern "C"

/*
 * csa2.h - C ABI of the CSA2 (Compressed Sparse Attention 2) hot path for
 * AMD Instinct MI355X (gfx950).
 *
 * CSA2 keeps one global KV pool for all layers and gives every layer one of
 * three static modes (Full / Reindex / Reuse); a hierarchical candidate pool
 * serves very long contexts; the global entries are FP4 (E2M1) restored to
 * real values at run time and a sliding window of FP8 rows covers nearby
 * tokens.  Sources: "DeepSeek V4.1-Flash Cuts KV Cache by 437x With New CED
 * and CSA2 Architecture" (paragraphs on CSA2 storage, the three operating
 * modes, sliding window attention and FP4 quantisation) and "DeepSeek V4.1
 * Flash Architecture Breakdown" (sections "How does the cache compress along
 * three dimensions at once?" and "How are cache precision and storage
 * arranged?").  The pages give no formulas, sizes or layouts; the readings
 * used here are stated per function.
 *
 * Conventions for every entry point
 *  - All array pointers are DEVICE pointers unless marked "host".  Arrays are
 *    dense, row-major, in the shapes given.  The caller owns every buffer; the
 *    library allocates no device memory and keeps no global state.
 *  - Work is enqueued on `stream` (0 = the null stream) and returns without
 *    synchronising.  Outputs are fully overwritten.
 *  - Argument and schedule errors are detected on the host and returned
 *    before any HIP call is made.  A failed launch returns CSA2_ERR_HIP.
 *    Faults inside kernels surface at the caller's next synchronisation.
 *  - Device-side preconditions (not checked): no NaN E4M3 codes (0x7F, 0xFF),
 *    E8M0 scale codes 0..252, selected indices in [-1, M), candidate lists
 *    strictly ascending with -1 padding only at the end.
 *  - Results are deterministic: the same inputs give bit-identical outputs.
 *  - Fixed model shapes: latent width D = 512, indexer HI = 8 heads of
 *    DI = 64, attention heads H = 16.  Other values return CSA2_ERR_SHAPE.
 *
 * Number formats
 *  - E4M3: OCP FP8 E4M3 (bias 7, max 448, no infinity).
 *  - E2M1: OCP FP4, two codes per byte, element 2i in the LOW nibble of byte i.
 *  - E8M0: OCP block scale 2^(x-127), one per 32 consecutive latent elements.
 *  - bf16: the upper 16 bits of an IEEE binary32, passed as uint16_t.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum csa2_status {
  CSA2_OK = 0,
  CSA2_ERR_NULL = 1,       /* a required pointer is NULL */
  CSA2_ERR_SHAPE = 2,      /* a size is out of range or unsupported */
  CSA2_ERR_ALIGN = 3,      /* a pointer is not 16-byte aligned */
  CSA2_ERR_SCHEDULE = 4,   /* invalid per-layer mode schedule */
  CSA2_ERR_WORKSPACE = 5,  /* workspace missing or too small */
  CSA2_ERR_HIP = 6,        /* a HIP launch or runtime call failed */
  CSA2_ERR_SCRATCH = 7     /* the call needs more than the static scratch */
} csa2_status;

/* Size of the device array that csa2_decode_layers_noalloc works in (one
 * per GPU, in the library's own device memory until the process ends). */
#define CSA2_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

enum { CSA2_FULL = 0, CSA2_REINDEX = 1, CSA2_REUSE = 2 };

/* Which call a workspace size is asked for (csa2_workspace_bytes). */
enum {
  CSA2_OP_TOPK = 0,
  CSA2_OP_SPARSE_ATTN = 1,
  CSA2_OP_SWA_MERGE = 2,
  CSA2_OP_DECODE_LAYERS = 3,
  CSA2_OP_PREFILL_LAYERS = 4,
  CSA2_OP_SCORE_TOPK = 5
};

/* The shared global KV pool: B sequences of up to M compressed entries each,
 * stored as rows of three arrays (structure of arrays):
 *   latent  [rows][D/2]     E2M1 codes of the D-wide shared K/V latent
 *   scale   [rows][D/32]    E8M0 block scales of the latent
 *   idx_key [rows][HI][DI]  E4M3 indexer keys
 *   len     NULL: every sequence holds M entries.  Otherwise device [B]
 *           int32 in [0, M]: sequence b holds entries 0 .. len[b]-1 (a
 *           ragged batch, the serving shape); the scans read no key past
 *           len[b], such entries score -inf and are never selected.  (Not
 *           checked on the device: values outside [0, M] are not allowed.)
 *   pages   NULL: contiguous, sequence b's entry e is row b * M + e (arrays
 *           of B * M rows).  Otherwise device [B][M >> page_log2] int32: a
 *           page table; entry e of sequence b is row
 *           pages[b][e >> page_log2] * 2^page_log2 + (e mod 2^page_log2), so
 *           sequences hold their entries in pages of 2^page_log2 rows of
 *           shared arrays (a paged pool; pages need not be distinct or in
 *           order).  page_log2 in [6, 30] and M a multiple of the page size.
 *           (Not checked on the device: page numbers must address rows that
 *           exist.)
 * latent, scale and idx_key must be 16-byte aligned, len and pages 4-byte
 * aligned.  Selected indices (idx outputs and inputs) are always entry
 * numbers e, never rows. */
typedef struct csa2_pool {
  const uint8_t* latent;
  const uint8_t* scale;
  const uint8_t* idx_key;
  int32_t B, M, D, HI, DI;
  const int32_t* len;
  const int32_t* pages;
  int32_t page_log2;
} csa2_pool;

/* One layer of a decode step (one query token per sequence).
 *   mode    CSA2_FULL, CSA2_REINDEX or CSA2_REUSE
 *   q_idx   [B][HI][DI] E4M3 indexer query   (Full / Reindex; ignored for Reuse)
 *   w_idx   [B][HI] float indexer head weights (Full / Reindex; ignored for Reuse)
 *   q       [B][H][D] bf16 attention query (already scaled by 1/sqrt(D))
 *   swa     [B][W][D] E4M3 sliding-window rows (may be NULL when W == 0)
 *   o       [B][H][D] float output
 *   lse     [B][H] float output, natural-log sum of exp of the logits
 *   idx_out [B][K] int32 selected global entries, ascending, -1 padded.
 *           Required for Full / Reindex; for Reuse it may be NULL, otherwise
 *           it receives a copy of the source layer's indices. */
typedef struct csa2_layer {
  int32_t mode;
  const uint8_t* q_idx;
  const float* w_idx;
  const uint16_t* q;
  const uint8_t* swa;
  float* o;
  float* lse;
  int32_t* idx_out;
} csa2_layer;

/* Indexer scores of pool entries.
 * Reading (the pages give no formula): for query row r = (b, t) and pool
 * entry j,  s = sum_h w[r][h] * ReLU(sum_i q_idx[r][h][i] * idx_key[b][j][h][i])
 * with E4M3 operands, fp32 products (exact) and fp32 accumulation; ReLU maps
 * x <= 0 to +0.  The pages' Full layer scores the whole context, a Reindex
 * layer re-scores with its own indexer, and in the hierarchical case it
 * scores only inside the candidate pool ("... Cuts KV Cache by 437x",
 * paragraph on the three operating modes).
 *   pool    the pool (B, M used)
 *   q_idx   [B][Q][HI][DI] E4M3;  w_idx [B][Q][HI] float
 *   Q       query tokens per sequence (1 for decode)
 *   pos0    < 0: every entry is visible.  >= 0: query t sits at position
 *           pos0 + t and sees the first min(M, (pos0 + t + 1) / ratio) entries
 *           (an entry is visible once its last token is); scores of
 *           invisible positions are written as -inf.
 *   ratio   tokens per pool entry (used only when pos0 >= 0; must be >= 1)
 *   cand    NULL: score all M entries, N = M.  Otherwise [B][P] ascending
 *           global entry numbers, -1 padded; N = P, and position p scores
 *           entry cand[b][p] (-inf for -1).
 *   scores  [B][Q][N] float output
 *   hist    NULL, or [B*Q][4096] uint32 histogram that the call ADDS the
 *           score keys' top 12 bits to (see csa2_topk); caller zeroes it.
 *           Must be NULL when Q > 1 and cand is NULL (CSA2_ERR_SHAPE).
 * With Q > 1 and no candidate list (a chunked-prefill step) the scores are
 * computed as a matrix-core contraction of the Q queries against 128-entry
 * tiles (E4M3 widened exactly to bf16, fp32 accumulation); the result meets
 * the same fp32 bound as the Q == 1 path. */
csa2_status csa2_index_score(const csa2_pool* pool, const uint8_t* q_idx,
                             const float* w_idx, int32_t Q, int64_t pos0,
                             int32_t ratio, const int32_t* cand, int32_t P,
                             float* scores, uint32_t* hist, hipStream_t stream);

/* Top-K selection per row.
 * The pages' Full and Reindex layers pick the Top-K entries from the indexer
 * scores, over the whole context or, in the hierarchical case, within the
 * candidate pool ("DeepSeek V4.1-Flash Cuts KV Cache by 437x", paragraph on
 * the three operating modes; "DeepSeek V4.1 Flash Architecture Breakdown",
 * section "How does the cache compress along three dimensions at once?").
 * Readings (the pages fix neither): ties go to the lower index, and the
 * selection is returned in ascending index order.
 * For each of R rows of N scores, select the K largest among the first
 * n_valid[r] positions (all N when n_valid is NULL).  Equal scores are broken
 * toward the LOWER position (= lower global entry, since candidate lists are
 * ascending).  The selection is written as ascending entry numbers (through
 * cand when given), padded with -1 when fewer than K positions are valid.
 * Scores compare as real numbers (-0 == +0); NaN scores are not allowed.
 *   scores  [R][N] float;  n_valid NULL or [R] int32
 *   cand    NULL (output positions) or [R][N] int32 position -> entry map
 *   idx     [R][K] int32 output
 *   ws      workspace of at least csa2_workspace_bytes(CSA2_OP_TOPK, R, 1, N, K, 0, 0, 0)
 * Limits: 1 <= K <= 16384; 1 <= N <= 2^30 (the select orders (score,
 * position) pairs as one 62-bit key with 30 position bits); 1 <= R <= 65535
 * (rows are a grid dimension of the launches).  Other values return
 * CSA2_ERR_SHAPE. */
csa2_status csa2_topk(const float* scores, int32_t R, int32_t N,
                      const int32_t* n_valid, const int32_t* cand, int32_t K,
                      int32_t* idx, void* ws, size_t ws_bytes,
                      hipStream_t stream);

/* Indexer score and Top-K of a flat decode row in one pass: the result of
 * csa2_index_score (Q = 1, no candidate list, every entry of the sequence's
 * length visible) followed by csa2_topk with n_valid = the pool's lengths,
 * bit for bit, without writing the scores.  The Full layer scores the
 * context and selects its Top-K entries ("DeepSeek V4.1-Flash Cuts KV Cache
 * by 437x", paragraph on the three operating modes); the single pass is this
 * library's fusion of those two steps.  Each work-group scores 4096 entries
 * of one row into LDS and keeps a superset of their Top-K (every member of
 * the row's Top-K that lies among them); one work-group per row then selects
 * the Top-K from all keepers.
 *   pool    the pool (B, M, len, pages used)
 *   q_idx   [B][HI][DI] E4M3;  w_idx [B][HI] float
 *   idx     [B][K] int32 output: ascending entry numbers, -1 padded
 *   ws      at least csa2_workspace_bytes(CSA2_OP_SCORE_TOPK, B, 1, M, K, 0, 0, 0)
 * Limits: 1 <= K <= 16384 and ceil(M / 4096) * (K + max(K / 4, 64), rounded
 * up to a multiple of 64) <= 16384 (every keeper fits the final select; M
 * up to 114688 at K = 512), 1 <= B <= 65535.  Other shapes return
 * CSA2_ERR_SHAPE (csa2_workspace_bytes returns 0 for them). */
csa2_status csa2_score_topk(const csa2_pool* pool, const uint8_t* q_idx, const float* w_idx,
                            int32_t K, int32_t* idx, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/* Attention over selected FP4 global entries.
 * Every layer attends over the entries its index selects, held as FP4 (E2M1)
 * and restored to real values for the computation ("DeepSeek V4.1-Flash Cuts
 * KV Cache by 437x", paragraphs on the three operating modes and on FP4
 * quantisation; "DeepSeek V4.1 Flash Architecture Breakdown", section "How are
 * cache precision and storage arranged?").  Readings: key = value = the
 * latent row (shared K/V), softmax scale 1 (q carries 1/sqrt(D)).
 * Per query row (b, t) and head h, the keys (= values) are the dequantised
 * latent rows c_j[i] = E2M1(code) * 2^(scale - 127) of the selected entries
 * (idx != -1); logits z_j = q[h] . c_j (scale 1); o[h] = sum softmax(z)_j c_j
 * and lse[h] = log sum exp(z).  No selected entry gives o = 0, lse = -inf.
 * Computed on the matrix cores: the dequantised values and q enter as bf16
 * (exact for every E2M1 value times a scale code 0..252), products and sums
 * in fp32, and the softmax weights are split into two bf16 halves (relative
 * rounding below 2^-16).  Decode rows (Q == 1) are cut into runs of keys on
 * separate work-groups whose partial results (in the workspace) a merge
 * combines; prefill rows (Q > 1) take one work-group each.
 *   q    [B][Q][H][D] bf16;  idx [B][Q][K] int32 in [-1, M)
 *   o    [B][Q][H][D] float;  lse [B][Q][H] float
 *   ws   at least csa2_workspace_bytes(CSA2_OP_SPARSE_ATTN, B, Q, M, K, 0, 0, H)
 *        (256 bytes when Q > 1) */
csa2_status csa2_sparse_attn(const csa2_pool* pool, const uint16_t* q,
                             int32_t Q, int32_t H, const int32_t* idx,
                             int32_t K, float* o, float* lse, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/* Sliding-window attention merged into an earlier result.
 * Query row (b, t) attends to the W E4M3 rows t .. t+W-1 of swa[b] (the
 * window of the newest tokens including its own) and the result is merged
 * with the incoming (o, lse) as one softmax over the union of both key sets:
 *   lse' = log(e^lse + e^lse_w),  o' = (e^lse o + e^lse_w o_w) / e^lse'.
 * The pages pair the sparse global entries with an FP8 sliding window for
 * nearby tokens ("... Cuts KV Cache by 437x", paragraph on sliding window
 * attention); merging by log-sum-exp is an exact rewrite of one softmax.
 *   q    [B][Q][H][D] bf16;  swa [B][Q+W-1][D] E4M3
 *   o    [B][Q][H][D] float, in/out;  lse [B][Q][H] float, in/out
 *   ws   at least csa2_workspace_bytes(CSA2_OP_SWA_MERGE, B, Q, 0, 0, 0, W, H) */
csa2_status csa2_swa_merge(const uint16_t* q, int32_t B, int32_t Q, int32_t H,
                           int32_t D, const uint8_t* swa, int32_t W, float* o,
                           float* lse, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/* One decode step through a static per-layer mode schedule over one pool.
 * The pages give every layer one of three static modes over one shared pool
 * and index: Full builds the index from scratch, Reindex re-scores with the
 * layer's own indexer, Reuse takes the previous layer's indices with no index
 * work; for very long contexts the indexer is hierarchical and later layers
 * search only a candidate pool ("DeepSeek V4.1-Flash Cuts KV Cache by 437x",
 * paragraphs on the three operating modes and on CSA2 storage; "DeepSeek V4.1
 * Flash Architecture Breakdown", section "How does the cache compress along
 * three dimensions at once?").  Readings: Reuse takes the most recent Full or
 * Reindex layer; the first layer must be Full; each layer has its own query,
 * indexer query and window.
 * Layers run in order.  Full: score all M entries, select Top-K; with P > 0
 * it also builds the candidate pool = Top-P of the same scores (ascending).
 * Reindex: with P == 0 score all M with its own indexer; with P > 0 score only
 * the candidate pool.  Reuse: no index work, take the indices of the most
 * recent Full or Reindex layer.  Then every layer attends over its selected
 * entries plus its W window rows (one softmax).  The first layer must be Full.
 *   layers     host array [L]
 *   K          selected entries per layer (1..16384); P: 0 = flat, else K <= P
 *   W          window rows per layer (0..4096)
 *   src_layer  NULL or host [L] output: the layer whose indices each layer
 *              uses (itself for Full / Reindex)
 *   ws         at least csa2_workspace_bytes(CSA2_OP_DECODE_LAYERS, B, 1, M, K, P, W, H) */
csa2_status csa2_decode_layers(const csa2_pool* pool, const csa2_layer* layers,
                               int32_t L, int32_t H, int32_t K, int32_t P,
                               int32_t W, int32_t* src_layer, void* ws,
                               size_t ws_bytes, hipStream_t stream);

/* Layer l alone of the decode step csa2_decode_layers describes: the shape
 * of a model that runs each layer's attention between its other work.  The
 * schedule (layers, L) is checked whole.  Layers 0 .. l-1 must have run (by
 * this call or by csa2_decode_layers) on the same pool, layer array and
 * workspace: a Reuse layer reads its source layer's idx_out, and a Reindex
 * layer of a hierarchical step (P > 0) scores the candidate pool that the
 * Full layer left in the workspace.  Results equal those of
 * csa2_decode_layers, bit for bit.
 *   l          0 <= l < L (else CSA2_ERR_SHAPE)
 *   src_layer  NULL or host int32 output: the layer whose indices l uses
 *   other arguments as in csa2_decode_layers (same workspace size) */
csa2_status csa2_decode_layer(const csa2_pool* pool, const csa2_layer* layers, int32_t L,
                              int32_t l, int32_t H, int32_t K, int32_t P, int32_t W,
                              int32_t* src_layer, void* ws, size_t ws_bytes, hipStream_t stream);

/* csa2_decode_layers for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  The caller still passes the pool, the layers' inputs and their
 * outputs; the workspace is a fixed array of CSA2_NOALLOC_SCRATCH_BYTES per
 * GPU inside the library.  No device memory is allocated or freed by the
 * call (the array's address on the current device is looked up once, on the
 * first call made with that device current).  The stream must belong to the
 * current device.
 *   Limit: a step whose csa2_workspace_bytes(CSA2_OP_DECODE_LAYERS, B, 1, M,
 *   K, P, W, H) exceeds CSA2_NOALLOC_SCRATCH_BYTES returns CSA2_ERR_SCRATCH
 *   before any HIP call (64 MiB holds, e.g., B = 64 at M = 65536 or B = 8 at
 *   M = 262144 with P = 8192, K = 512, W = 128).
 *   Races: every call on one GPU shares that GPU's array and leaves its
 *   contents behind; calls whose work overlaps on the device (calls on
 *   different streams, or from several host threads, without an ordering
 *   between them) race and their results are undefined.  Calls in order on
 *   one stream are safe; the call clears what must start at zero itself.
 *   Other arguments, results and errors as in csa2_decode_layers (results
 *   equal, bit for bit); CSA2_ERR_HIP when the array's address cannot be
 *   obtained. */
csa2_status csa2_decode_layers_noalloc(const csa2_pool* pool, const csa2_layer* layers,
                                       int32_t L, int32_t H, int32_t K, int32_t P, int32_t W,
                                       int32_t* src_layer, hipStream_t stream);

/* One chunk of Q tokens per sequence (chunked prefill) through the same
 * static per-layer mode schedule as csa2_decode_layers.  The pages name
 * prefill as the cost that CSA2's index reuse cuts and give every layer its
 * mode there as in decode ("... Cuts KV Cache by 437x", paragraphs on prefill
 * cost and the three operating modes).  Per query token the layer does what
 * it does in decode, within that token's causal limits: query t sits at
 * position pos0 + t, sees the first min(M, (pos0 + t + 1) / ratio) pool
 * entries (an entry is visible once its last token is), and attends to its
 * window rows of positions max(0, pos0 + t - W + 1) .. pos0 + t.  Full and
 * Reindex score the visible entries with their own indexer (a matrix-core
 * contraction of the chunk's queries against the pool, as in
 * csa2_index_score) and select Top-K (csa2_topk's rules; a token that sees
 * fewer than K entries selects all of them, -1 padded); Reuse takes the
 * indices of the most recent Full or Reindex layer, token by token.  Each
 * layer's selected entries and window rows form one softmax in one pass.
 * There is no candidate pool in prefill (reading: the chunk's Q queries
 * share one pass over the keys, which is what the candidate pool saves a
 * single decode token).  A chunk reads only the entries its last query can
 * see, so successive chunks over a pool that grows by csa2_pool_append cost
 * what they can see, not M.  The first layer must be Full.
 *   layers     host array [L]; per layer (shapes per chunk):
 *                q_idx [B][Q][HI][DI] E4M3, w_idx [B][Q][HI] float (Full /
 *                Reindex), q [B][Q][H][D] bf16, o [B][Q][H][D] float,
 *                lse [B][Q][H] float, idx_out [B][Q][K] int32 (required for
 *                Full / Reindex; optional for Reuse, then a copy),
 *                swa [B][Q+W-1][D] E4M3: row r holds position
 *                pos0 - (W - 1) + r; rows at positions below 0 are not read.
 *   Q          query tokens per sequence (B * Q <= 65535)
 *   pos0       position of the chunk's first token; < 0: no causal limit
 *              (every entry and every window row visible)
 *   ratio      tokens per pool entry (>= 1 when pos0 >= 0)
 *   K          1..16384;  W  0..4096
 *   src_layer  NULL or host [L] output, as in csa2_decode_layers
 *   ws         at least csa2_workspace_bytes(CSA2_OP_PREFILL_LAYERS, B, Q, M, K, 0, W, H)
 * Errors: as csa2_decode_layers (CSA2_ERR_SCHEDULE when layer 0 is not Full
 * or a mode is unknown). */
csa2_status csa2_prefill_layers(const csa2_pool* pool, const csa2_layer* layers,
                                int32_t L, int32_t Q, int64_t pos0, int32_t ratio,
                                int32_t H, int32_t K, int32_t W, int32_t* src_layer,
                                void* ws, size_t ws_bytes, hipStream_t stream);

/* New pool entries, encoded into the stored formats in place: the write side
 * of a Full layer, which generates the global KV and the index data that
 * later layers reuse, stored in FP4 ("... Cuts KV Cache by 437x", paragraphs
 * on the three operating modes and FP4 quantisation).
 * Reading (the pages give no encoding rule): each latent row becomes MXFP4 -
 * per block of 32 elements an E8M0 scale 2^s, s = floor(log2(amax)) - 2
 * clamped to [-127, 127] (0 for an all-zero block), elements divided by it
 * and rounded to the nearest E2M1 value, ties to the even code, saturating at
 * 6, signs kept; element 2i in the low nibble of byte i.  Each index key row
 * becomes E4M3, clamped to +-448, nearest value, ties to the even code.
 *   latent, scale, idx_key  the pool arrays (rows of 256, 16 and 512 bytes;
 *                           [B][M] rows when contiguous), written in place
 *   x_latent  [B][T][512] float;  x_key [B][T][8][64] float (finite)
 *   slot      [B][T] int32: entry number receiving row t of sequence b;
 *             rows whose slot is outside [0, M) are skipped.  Two rows of one
 *             sequence naming the same slot is a caller error (race).
 *   pages, page_log2  NULL for a contiguous pool, or its page table (as in
 *             csa2_pool): an entry is written to the row it maps to.  Rows
 *             written by one call must be distinct (two slots that map to
 *             one row, through shared pages, race like a repeated slot).
 * Errors: CSA2_ERR_NULL, CSA2_ERR_SHAPE (B, M <= 0, T < 0, a page size
 * outside [2^6, 2^30] or not dividing M), CSA2_ERR_ALIGN (x_latent, x_key
 * not 16-byte aligned, pool arrays not 8-byte aligned).
 * T == 0 returns CSA2_OK without a launch. */
csa2_status csa2_pool_append(uint8_t* latent, uint8_t* scale, uint8_t* idx_key,
                             int32_t B, int32_t M, const float* x_latent,
                             const float* x_key, const int32_t* slot, int32_t T,
                             const int32_t* pages, int32_t page_log2,
                             hipStream_t stream);

/* New tokens into the FP8 sliding window ("... Cuts KV Cache by 437x",
 * paragraphs on sliding window attention and FP8 storage), kept as a ring of
 * W rows per sequence: token position p lives in row p mod W, so the ring
 * always holds the newest W tokens (their order does not change the window
 * attention, one softmax over the set).  Encoding: E4M3 as for index keys.
 *   swa   [B][W][512] E4M3 ring, written in place
 *   x     [B][T][512] float: tokens pos0 .. pos0+T-1 (only the last W of
 *         them are written when T > W)
 * Errors: CSA2_ERR_NULL, CSA2_ERR_SHAPE (B, W <= 0, T < 0, pos0 < 0),
 * CSA2_ERR_ALIGN (x not 16-byte aligned, swa not 8-byte aligned). */
csa2_status csa2_swa_append(uint8_t* swa, int32_t B, int32_t W, const float* x,
                            int64_t pos0, int32_t T, hipStream_t stream);

/* Host tier: one sequence's pool entries between host memory and the device
 * pool, by the copy engines on `stream`.  The pages keep the runtime copy of
 * the KV in HBM and a longer-lived copy outside it: the sliding-window KV in a
 * host-memory pool and the global KV in a persistent cache ("DeepSeek V4.1
 * Flash Architecture Breakdown", section "How are cache precision and storage
 * arranged?"; "... Cuts KV Cache by 437x", paragraph on the cache tiers).
 * These calls move the stored bytes unchanged (the FP4 / FP8 encodings are
 * the transfer format: 784 B per pool entry, 196 B per token at 4 tokens per
 * entry).
 *   latent, scale, idx_key  the device pool arrays [B][M][256], [B][M][16],
 *                           [B][M][8][64]
 *   seq, entry0, n          entries entry0 .. entry0+n-1 of sequence seq
 *   h_latent, h_scale, h_key  host [n][256], [n][16], [n][8][64] (host
 *                           pointers; page-locked memory, e.g. hipHostMalloc,
 *                           lets the copies run asynchronously beside
 *                           kernels on other streams; pageable memory works but
 *                           the call may block until the copy is done)
 * Restore copies host -> device, offload device -> host.  Errors:
 * CSA2_ERR_NULL, CSA2_ERR_SHAPE (B, M <= 0, seq outside [0, B), entry0 < 0,
 * n < 0, entry0 + n > M), CSA2_ERR_HIP (a copy could not be enqueued).
 * n == 0 returns CSA2_OK without a copy. */
csa2_status csa2_pool_restore(uint8_t* latent, uint8_t* scale, uint8_t* idx_key,
                              int32_t B, int32_t M, int32_t seq, int32_t entry0,
                              int32_t n, const uint8_t* h_latent,
                              const uint8_t* h_scale, const uint8_t* h_key,
                              hipStream_t stream);
csa2_status csa2_pool_offload(const uint8_t* latent, const uint8_t* scale,
                              const uint8_t* idx_key, int32_t B, int32_t M,
                              int32_t seq, int32_t entry0, int32_t n,
                              uint8_t* h_latent, uint8_t* h_scale, uint8_t* h_key,
                              hipStream_t stream);

/* One sequence's window ring ([W][512] E4M3, as csa2_swa_append keeps it)
 * between host memory h_swa [W][512] and the device rings swa [B][W][512].
 * Errors: CSA2_ERR_NULL, CSA2_ERR_SHAPE (B, W <= 0, seq outside [0, B)),
 * CSA2_ERR_HIP. */
csa2_status csa2_swa_restore(uint8_t* swa, int32_t B, int32_t W, int32_t seq,
                             const uint8_t* h_swa, hipStream_t stream);
csa2_status csa2_swa_offload(const uint8_t* swa, int32_t B, int32_t W, int32_t seq,
                             uint8_t* h_swa, hipStream_t stream);

/* Workspace bytes needed by an entry point (op = CSA2_OP_*).  Arguments that
 * an op does not use are ignored.  For CSA2_OP_TOPK, B is the row count R and
 * M the row length N.  Returns 0 for an unknown op or bad sizes. */
size_t csa2_workspace_bytes(int op, int32_t B, int32_t Q, int32_t M, int32_t K,
                            int32_t P, int32_t W, int32_t H);

/* Static, human-readable name of a status code. */
const char* csa2_status_string(csa2_status s);

/* Library version string (static). */
const char* csa2_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */

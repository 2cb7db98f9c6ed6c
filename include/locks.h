/*
 * locks.h - C ABI of the Locks decode-step library for AMD Instinct MI355X
 * (gfx950): page-local rank-r key summaries, query-aware page selection and
 * sparse paged decode attention.
 *
 * Method: "Locks: Page-Local Compact Key Summaries for Efficient Long-Context
 * Decoding" (J. Hwang, arXiv 2607.24555), cited as [Locks].
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All array arguments are DEVICE pointers into memory the caller allocated
 *   and owns (the library never allocates, frees or keeps device memory, and
 *   holds no mutable global state). Arrays are dense, row-major, and must be
 *   16-byte aligned; element types are given per argument.
 * - Every call only validates its arguments on the host and enqueues kernels
 *   on `stream` (a hipStream_t; NULL = the default stream). It never
 *   synchronises and never reads device memory on the host, so it may be
 *   captured into a HIP graph.
 * - Return value: LOCKS_OK (0) or a negative status (see below). A non-OK
 *   status means nothing was enqueued, except LOCKS_E_HIP, which reports a
 *   launch failure from the HIP runtime.
 * - num_blocks >= 1 for every call with work that reads a paged pool (an id
 *   outside the pool still issues its loads at block 0, result discarded).
 * - Data-dependent checks are done on the device: a block id outside
 *   [0, num_blocks) is skipped (its page scores -inf and is never selected;
 *   in decode the slot contributes nothing), a negative sequence length counts
 *   as 0 and a length above max_pages * page_size is clamped to it.
 *
 * Paged layouts (P = page_size, d = head_dim, r = rank, e = element bytes)
 *   K pool, V pool   [num_blocks][num_kv_heads][P][d]     kv_dtype
 *   block_table      [batch][max_pages] int32: physical block of logical page j
 *   seq_lens         [batch] int32: tokens T in the cache (current token included)
 *   summary pool     [num_blocks][num_kv_heads][record], one record per
 *                    (block, KV head), summary_dtype elements:
 *                        mu[d] | V^T[r][d] | C[P][r]
 *                    record bytes = e * (d + r*d + P*r)
 *   q                [batch][num_q_heads][d] kv_dtype; query head g belongs
 *                    to KV head g / G, G = num_q_heads / num_kv_heads
 *   selected         [batch][num_kv_heads][budget_pages] int32 logical page ids,
 *                    ascending, padded with -1
 * A sequence with T tokens has J = ceil(T/P) pages; the first floor(T/P) are
 * complete. Page J-1 is the current page (partial when P does not divide T).
 *
 * LOCKS_I4 summary records ([Locks] §4 "i4" storage, App. C.7 byte model),
 * in this byte order:
 *   V codes     r rows of d/2 bytes: basis vector rho as 4-bit fields n in
 *               1..15, value s_V[rho] * (n - 8)
 *   mu codes    2 rows of d/2 bytes: the high, then the low 4 bits of the
 *               centroid's 8-bit codes b in 1..255, value s_mu * (b - 128)
 *   C codes     P rows of r bytes: token i's codes b, value s_C[i] * (b - 128)
 *   scales      r + 1 + P bf16: s_V[0..r-1], s_mu, s_C[0..P-1]
 *   padding     zero bytes up to a multiple of 16
 *   In a row of 4-bit fields, element a (0 <= a < d) lives in the 32-bit
 *   little-endian word w = ((a % 32) / 8) * (d / 32) + a / 32, at bits
 *   4m .. 4m+3 with m = e/2 for even e = a % 8 and m = 4 + (e-1)/2 for odd e.
 *   Size: ((r + 2) d/2 + P r + 2 (1 + r + P)) rounded up to 16 bytes, i.e. the
 *   pages' d r/2 + P r + d bytes before scales plus 2 (r + P + 1) of scales.
 */
#ifndef LOCKS_H
#define LOCKS_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  LOCKS_OK = 0,
  LOCKS_E_INVALID_ARG = -1,  /* null pointer, negative size, k < 2, bad scale ... */
  LOCKS_E_UNSUPPORTED = -2,  /* a shape or dtype this library has no kernel for */
  LOCKS_E_WORKSPACE = -3,    /* workspace pointer NULL or smaller than required */
  LOCKS_E_HIP = -4           /* the HIP runtime reported a launch error          */
};

/* LOCKS_I4 is a summary_dtype only: the quantized summary storage of [Locks]
 * §4 and App. C.7 (4-bit basis, 8-bit centroid and coefficients, bf16
 * scales), layout below. */
typedef enum { LOCKS_BF16 = 0, LOCKS_F32 = 1, LOCKS_I4 = 2 } locks_dtype_t;

typedef struct locks_config {
  int32_t head_dim;      /* d: 64 or 128                                          */
  int32_t page_size;     /* P: 16, 32 or 64 tokens per page                       */
  int32_t rank;          /* r: 1 .. min(15, P - 1)                                */
  int32_t num_q_heads;   /* H_q                                                   */
  int32_t num_kv_heads;  /* H_kv >= 1; G = H_q / H_kv must be 1, 2, 4 or 8        */
  int32_t budget_pages;  /* k = ceil(b / P) page slots per (sequence, KV head), >= 2 */
  int32_t kv_dtype;      /* locks_dtype_t of q, K, V and the attention output     */
  int32_t summary_dtype; /* locks_dtype_t of the summary records: kv_dtype, or
                            LOCKS_I4 with kv_dtype LOCKS_BF16 and rank 1, 2, 4 or 8 */
  float softmax_scale;   /* logit scale, normally 1/sqrt(d); finite and > 0       */
} locks_config_t;

/* Human-readable name of a status code (static string, never NULL). */
const char* locks_status_string(int status);

/* Library ABI version (this header: 1). */
int locks_version(void);

/* Bytes of one summary record: e*(d + r*d + P*r) for bf16 / fp32 records,
 * the LOCKS_I4 size below for quantized ones; 0 when cfg is invalid or
 * unsupported. [Locks] §4: a page stores its centroid mu_j, its basis V_j and
 * its per-token coefficients C_j. */
size_t locks_summary_record_bytes(const locks_config_t* cfg);

/* Workspace bytes needed by locks_score_select, locks_sparse_decode,
 * locks_decode_step and locks_decode_step_cached for a batch of `batch`
 * sequences of at most `max_pages` pages (one buffer of this size serves all
 * four, in any interleaving).
 * Writes *bytes; returns a status.
 * The workspace must be zero-filled once before its first use: its first
 * bytes hold control words (per-(sequence, KV head) arrival counters) that
 * every call returns to zero and that no call uses as scratch; each call's
 * scratch ends at the end of the buffer. A workspace sized for a batch also
 * serves calls with fewer sequences of at most as many pages. Calls that share
 * a workspace must not overlap in time (same stream, or synchronised). */
int locks_workspace_size(const locks_config_t* cfg, int32_t batch, int32_t max_pages,
                         size_t* bytes);

/* (a1) Summary build, [Locks] §3-§4: for each physical block id in
 * block_ids[n_ids] (device int32) and each KV head h, fit to the P keys
 * k_i of that (block, head) tile
 *     mu = (1/P) sum_i k_i,   D = [k_i - mu]_i  (P x d),
 *     V  = top-r eigenvectors of H = D^T D (orthonormal, d x r),
 *     C  = D V  (P x r),
 * and store (mu, V^T, C) rounded to summary_dtype (round-to-nearest-even)
 * into the record of (block, h) in summary_pool. For LOCKS_I4 each group (the
 * centroid, each basis vector, each token's coefficient row) is quantized
 * symmetrically: scale = bf16(max|x| / L) with L = 127 (8-bit) or 7 (4-bit),
 * code = round-half-even(x / scale) in fp32, scale 0 for an all-zero group.
 * Keys are read as stored; the fit is computed in fp32 (centred keys, Gram
 * matrix on the matrix cores, subspace iteration with Rayleigh-Ritz steps; see
 * locks_build_summaries_ex). Within an eigenvalue cluster any orthonormal
 * basis of the subspace is an equally valid result; each basis vector is
 * sign-fixed so its largest-magnitude entry is positive.
 * Only summarise complete pages. Ids outside [0, num_blocks) are skipped;
 * duplicate ids race. n_ids == 0 enqueues nothing. */
int locks_build_summaries(const locks_config_t* cfg, const void* k_pool, int64_t num_blocks,
                          const int32_t* block_ids, int32_t n_ids, void* summary_pool,
                          hipStream_t stream);

/* locks_build_summaries with a report of every fit. The top-r eigenvectors
 * are reached through the P x P dual Gram M = D D^T by subspace iteration on
 * a 16-column block with a Rayleigh-Ritz step after every product M X from
 * the third on ([Locks] App. A.2: the page's top-r right singular vectors);
 * a fit has converged when each of its r leading Ritz pairs has a residual
 * ||M u - theta u|| <= 2^-10 times the largest Ritz value and every leading
 * m-subspace (m <= r) whose Ritz gap exceeds 2^-7 of the largest Ritz value
 * has a residual norm <= 2^-6 of that gap (an angle of about 2^-6 to the
 * exact subspace by the sin-theta bound). P = 16 pages are
 * solved on the whole 16-dimensional space in one step. fit_info ([n_ids]
 * [num_kv_heads] int32, device, may be NULL) receives for the tile
 * (block_ids[t], h) the number of products taken, negated when the bound was
 * not met within the cap of 32 products (the record then holds the last
 * Ritz basis). Entries of skipped ids are left untouched. */
int locks_build_summaries_ex(const locks_config_t* cfg, const void* k_pool, int64_t num_blocks,
                             const int32_t* block_ids, int32_t n_ids, void* summary_pool,
                             int32_t* fit_info, hipStream_t stream);

/* (a2) Page scoring, [Locks] §4 Eq. (2): for every sequence b, query head g
 * and complete page j < floor(T_b / P), with mu, V, C the summary of
 * block_table[b][j] for KV head g / G,
 *     head_scores[b][g][j] = (q.mu) * scale + log sum_i exp(((V^T q).c_i) * scale)
 * computed from the stored summary values in fp32 (for LOCKS_I4, the values
 * code * scale). Entries j >= floor(T_b/P) are left untouched. head_scores:
 * [batch][H_q][max_pages] fp32. */
int locks_page_score(const locks_config_t* cfg, const void* q, const void* summary_pool,
                     int64_t num_blocks, const int32_t* block_table, const int32_t* seq_lens,
                     int32_t batch, int32_t max_pages, float* head_scores, hipStream_t stream);

/* (a3 + a4) Share-average combine and selection, [Locks] §2 and §4. Per
 * (sequence, KV head) with J pages and Jc complete pages:
 *   log Z_g  = log sum_{j<Jc} exp(s_g(j))                 (per query head)
 *   sigma_j  = log( (1/G) sum_g exp(s_g(j) - log Z_g) )   (log of the share average)
 * If J <= k every page 0..J-1 is selected. Otherwise the sink page 0 and the
 * current page J-1 are always selected and the other k-2 slots take the
 * complete pages outside {0, J-1} with the largest sigma (ties: lower page
 * id), by radix selection on the fp32 keys. selected receives the ids in
 * ascending order, padded with -1. page_sigma ([batch][H_kv][max_pages]
 * fp32) receives sigma_j for j < Jc when J > k and is left untouched
 * otherwise; it is also the selector's scratch. head_scores as written by
 * locks_page_score. */
int locks_select_pages(const locks_config_t* cfg, const float* head_scores,
                       const int32_t* seq_lens, int32_t batch, int32_t max_pages,
                       int32_t* selected, float* page_sigma, hipStream_t stream);

/* locks_page_score followed by locks_select_pages, with the head scores and
 * page keys kept in the caller's workspace (ws, ws_bytes >=
 * locks_workspace_size). Reads no candidate key or value ([Locks] §4). */
int locks_score_select(const locks_config_t* cfg, const void* q, const void* summary_pool,
                       int64_t num_blocks, const int32_t* block_table, const int32_t* seq_lens,
                       int32_t batch, int32_t max_pages, int32_t* selected, void* ws,
                       size_t ws_bytes, hipStream_t stream);

/* (a5) Sparse decode attention over the selected pages, [Locks] §2: for
 * query head g of sequence b, over every valid token i of the pages listed
 * in selected[b][g / G] (the current page contributes its T - (J-1)*P valid
 * tokens; -1 slots are skipped) with the original K and V,
 *     out[b][g] = sum_i softmax_i(q_g . k_i * scale) v_i,
 *     lse[b][g] = log sum_i exp(q_g . k_i * scale)
 * Split-K over page slots with an LSE merge, fp32 accumulation; out is
 * [batch][H_q][d] in kv_dtype (round-to-nearest-even), lse (may be NULL)
 * [batch][H_q] fp32. A (sequence, KV head) with no valid slot gives out = 0,
 * lse = -inf. ws as for locks_score_select. */
int locks_sparse_decode(const locks_config_t* cfg, const void* q, const void* k_pool,
                        const void* v_pool, int64_t num_blocks, const int32_t* block_table,
                        const int32_t* seq_lens, const int32_t* selected, int32_t batch,
                        int32_t max_pages, void* out, float* lse, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* One whole decode step, [Locks] §2 and §4: locks_score_select, then
 * locks_sparse_decode on the page ids it wrote, sharing one workspace (ws as
 * for locks_score_select). `selected`, out and lse are those two calls'
 * results. */
int locks_decode_step(const locks_config_t* cfg, const void* q, const void* summary_pool,
                      const void* k_pool, const void* v_pool, int64_t num_blocks,
                      const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
                      int32_t max_pages, int32_t* selected, void* out, float* lse, void* ws,
                      size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * (f4) Hot-page cache for K/V held in host memory, [Locks] §5.3 Table 3 and
 * App. B.4.2: the full K/V stays in host memory and the pages used often are
 * kept in a smaller cache in GPU memory. The pages specify no cache policy;
 * this library's is second-chance (clock) replacement over (block, KV head)
 * tiles of P x d keys and values, the unit one selection reads:
 *   - a selected tile resident in the cache is a hit: its slot is marked used
 *     this step and referenced. A tile that was copied while its page was
 *     incomplete (page J-1 with T % P != 0) is copied again on its next use
 *     (a refresh), since tokens may have been appended since.
 *   - each selected tile that is not resident (the first page slot naming it,
 *     in (sequence, KV head, slot) order, when several page slots name one
 *     tile) takes the next evictable slot of a clock hand that walks the
 *     slots cyclically: slots used this step (taken ones included) are
 *     skipped, a referenced slot
 *     loses its reference mark and is passed, an unreferenced one is taken
 *     (its old tile leaves the cache); the hand stops just past the last
 *     slot taken.
 *   - taken and refreshed tiles are copied from the K/V pools into their
 *     slots, then the decode reads every selected tile from the cache.
 * Cache buffer (device memory the caller allocates and owns; its layout from
 * locks_hot_cache_layout; fields in this order, each 256-byte aligned):
 *   STATS    int64[8]: hits, misses, refreshes, shared (page slots served by
 *            a tile another page slot of the step named), failed (page slots
 *            left unserved: a cache initialised for another capacity or pool),
 *            steps; accumulated by every call
 *   META     int64[2]: capacity and num_blocks * H_kv it was initialised for
 *   CLOCK    int32[2]: hand, step number
 *   SLOT_OF  int32[num_blocks * H_kv]: slot holding tile blk * H_kv + h, or -1
 *   TILE_OF, STAMP, FLAGS  int32[capacity]: tile held (or -1), last step
 *            that used the slot, flags (1 referenced, 2 copied incomplete)
 *   K, V     [capacity][P][d] kv_dtype: the cached tiles
 */
enum {
  LOCKS_HOT_CACHE_STATS = 0,
  LOCKS_HOT_CACHE_META,
  LOCKS_HOT_CACHE_CLOCK,
  LOCKS_HOT_CACHE_SLOT_OF,
  LOCKS_HOT_CACHE_TILE_OF,
  LOCKS_HOT_CACHE_STAMP,
  LOCKS_HOT_CACHE_FLAGS,
  LOCKS_HOT_CACHE_K,
  LOCKS_HOT_CACHE_V,
  LOCKS_HOT_CACHE_FIELDS
};

/* Byte offsets of the LOCKS_HOT_CACHE_FIELDS fields (offsets may be NULL)
 * and the total size (*bytes) of the cache buffer of a pool of num_blocks
 * blocks with `capacity` tile slots (both >= 1; num_blocks * H_kv < 2^31 - 1).
 * Host only. */
int locks_hot_cache_layout(const locks_config_t* cfg, int64_t num_blocks, int32_t capacity,
                           int64_t* offsets, size_t* bytes);

/* Empty the cache buffer (no tile resident, counters zero, hand at slot 0)
 * and record capacity and num_blocks in it. Required before the first
 * locks_decode_step_cached call on the buffer, and whenever the pool's blocks
 * get new contents other than tokens appended to incomplete pages. */
int locks_hot_cache_init(const locks_config_t* cfg, void* cache, int64_t num_blocks, int32_t capacity,
                         hipStream_t stream);

/* locks_decode_step with the K/V pools read through the hot-page cache:
 * locks_score_select, then the cache admission (above) of the selected tiles
 * and the copies of the missing and refreshed ones from k_pool / v_pool, then
 * the sparse decode over the cached tiles. Results (selected, out, lse) equal
 * locks_decode_step's on the same inputs bit for bit. k_pool / v_pool are
 * normally host memory the device can read (pinned, hipHostMalloc); they are
 * only read for the copied tiles. capacity >= batch * H_kv * budget_pages
 * (else LOCKS_E_INVALID_ARG), and every call on one cache buffer passes the
 * cfg, num_blocks and capacity it was initialised with. ws as for
 * locks_decode_step; calls that share a cache buffer must not overlap in
 * time. */
int locks_decode_step_cached(const locks_config_t* cfg, const void* q, const void* summary_pool,
                             const void* k_pool, const void* v_pool, int64_t num_blocks,
                             const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
                             int32_t max_pages, int32_t* selected, void* out, float* lse, void* cache,
                             int32_t capacity, void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* LOCKS_H */

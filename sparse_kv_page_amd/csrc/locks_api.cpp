// Host side of the Locks C ABI: argument validation, workspace layout and
// kernel dispatch. Every entry point decides OK/error from its arguments
// alone, then only enqueues work on the caller's stream.
#include "../../include/locks.h"

#include <cmath>
#include <cstddef>

#include "kernels.h"

namespace {

constexpr int kMaxK = 1024;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int elem_bytes(int dtype) { return dtype == LOCKS_BF16 ? 2 : 4; }

int check_config(const locks_config_t* c) {
  if (!c) return LOCKS_E_INVALID_ARG;
  if (c->head_dim <= 0 || c->page_size <= 0 || c->rank <= 0 || c->num_q_heads <= 0 ||
      c->num_kv_heads <= 0 || c->budget_pages < 2)
    return LOCKS_E_INVALID_ARG;
  if (!std::isfinite(c->softmax_scale) || !(c->softmax_scale > 0.f)) return LOCKS_E_INVALID_ARG;
  if (c->kv_dtype != LOCKS_BF16 && c->kv_dtype != LOCKS_F32) return LOCKS_E_INVALID_ARG;
  if (c->summary_dtype != LOCKS_BF16 && c->summary_dtype != LOCKS_F32 && c->summary_dtype != LOCKS_I4)
    return LOCKS_E_INVALID_ARG;
  if (c->num_q_heads % c->num_kv_heads != 0) return LOCKS_E_INVALID_ARG;
  const int G = c->num_q_heads / c->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return LOCKS_E_UNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128) return LOCKS_E_UNSUPPORTED;
  if (c->page_size != 16 && c->page_size != 32 && c->page_size != 64) return LOCKS_E_UNSUPPORTED;
  if (c->rank > 15 || c->rank > c->page_size - 1) return LOCKS_E_UNSUPPORTED;
  if (c->budget_pages > kMaxK) return LOCKS_E_UNSUPPORTED;
  if (c->summary_dtype == LOCKS_I4) {
    // quantized records: bf16 queries on the bf16 matrix cores, ranks 1/2/4/8
    if (c->kv_dtype != LOCKS_BF16) return LOCKS_E_UNSUPPORTED;
    if (c->rank != 1 && c->rank != 2 && c->rank != 4 && c->rank != 8) return LOCKS_E_UNSUPPORTED;
  } else if (c->summary_dtype != c->kv_dtype) {
    return LOCKS_E_UNSUPPORTED;
  }
  return LOCKS_OK;
}

int check_batch(int32_t batch, int32_t max_pages) {
  if (batch < 0 || max_pages < 0) return LOCKS_E_INVALID_ARG;
  if (batch > 0 && max_pages < 1) return LOCKS_E_INVALID_ARG;
  if (batch > 65535) return LOCKS_E_UNSUPPORTED;  // grid dimension
  // page offsets and token counts stay inside int32
  if ((int64_t)max_pages * 64 > (int64_t)0x7fffffff) return LOCKS_E_UNSUPPORTED;
  return LOCKS_OK;
}

int64_t rec_elems(const locks_config_t* c) {
  return (int64_t)c->head_dim * (1 + c->rank) + (int64_t)c->page_size * c->rank;
}

int64_t rec_bytes(const locks_config_t* c) {
  if (c->summary_dtype == LOCKS_I4) return locks::i4_record_bytes(c->head_dim, c->rank, c->page_size);
  return rec_elems(c) * elem_bytes(c->summary_dtype);
}

// Workspace layout, shared by every entry point that takes a workspace:
//   control words at the front: the decode arrival counters, one int32 per
//     (sequence, KV head); zero between calls, never written as scratch
//   scratch at the back (overwritten by every call), ending at the end of the
//     buffer:
//     score/select: head scores, page keys
//     decode:       split partials
//     decode step:  the two above in turn
// Control words sit in front of every scratch region, and a call with fewer
// sequences uses a prefix of the control words of a call with more and a
// shorter scratch ending at the same place, so calls of different entry points
// and batch sizes may share one workspace sized for the largest of them.
size_t ctl_bytes(const locks_config_t* c, int32_t batch) {
  return align_up((size_t)batch * c->num_kv_heads * sizeof(int32_t));
}

// first scratch byte of a call needing `scratch` bytes: as late as the buffer
// allows, 256-byte aligned (at or past the control words, since ws_bytes >=
// control + scratch and the control region is a multiple of 256 bytes)
uint8_t* scratch_base(void* ws, size_t ws_bytes, size_t scratch) {
  return static_cast<uint8_t*>(ws) + (ws_bytes - scratch) / kAlign * kAlign;
}

size_t score_ws_bytes(const locks_config_t* c, int32_t batch, int32_t max_pages) {
  const size_t scores = (size_t)batch * c->num_q_heads * max_pages * sizeof(float);
  const size_t sigma = (size_t)batch * c->num_kv_heads * max_pages * sizeof(float);
  return ctl_bytes(c, batch) + align_up(scores) + align_up(sigma);
}

// pages per split of a launch over `batch` sequences
int decode_pages_per_split(const locks_config_t* c, int32_t batch) {
  const int tpw = locks::decode_tiles_per_wave((int64_t)batch * c->num_kv_heads, c->budget_pages, c->page_size,
                                                c->kv_dtype == LOCKS_F32);
  return locks::decode_pages_per_split(c->page_size, tpw);
}

int decode_splits(const locks_config_t* c, int32_t batch) {
  const int pps = decode_pages_per_split(c, batch);
  return (c->budget_pages + pps - 1) / pps;
}

// sized for the most splits any batch uses, so a workspace sized for one
// batch serves every smaller batch
size_t decode_ws_bytes(const locks_config_t* c, int32_t batch) {
  const size_t rows = (size_t)batch * c->num_q_heads * locks::decode_max_splits(c->budget_pages, c->page_size);
  return ctl_bytes(c, batch) + align_up(rows * c->head_dim * sizeof(float)) +
         align_up(rows * sizeof(float));
}

int hip_status(hipError_t e) { return e == hipSuccess ? LOCKS_OK : LOCKS_E_HIP; }

locks::ScoreArgs score_args(const locks_config_t* cfg, const void* q, const void* summary_pool,
                            int64_t num_blocks, const int32_t* block_table, const int32_t* seq_lens,
                            int32_t max_pages, float* head_scores) {
  locks::ScoreArgs a{};
  a.q = q;
  a.sum_pool = static_cast<const uint8_t*>(summary_pool);
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.scores = head_scores;
  a.num_blocks = num_blocks;
  a.rec_elems = rec_elems(cfg);
  a.Hkv = cfg->num_kv_heads;
  a.G = cfg->num_q_heads / cfg->num_kv_heads;
  a.P = cfg->page_size;
  a.r = cfg->rank;
  a.max_pages = max_pages;
  a.scale = cfg->softmax_scale;
  return a;
}

locks::SelectArgs select_args(const locks_config_t* cfg, const float* head_scores, const int32_t* seq_lens,
                              int32_t max_pages, int32_t* selected, float* page_sigma) {
  locks::SelectArgs a{};
  a.scores = head_scores;
  a.seq_lens = seq_lens;
  a.selected = selected;
  a.sigma = page_sigma;
  a.Hkv = cfg->num_kv_heads;
  a.G = cfg->num_q_heads / cfg->num_kv_heads;
  a.P = cfg->page_size;
  a.k = cfg->budget_pages;
  a.max_pages = max_pages;
  a.idbits = 1;
  while (a.idbits < 31 && (int64_t(1) << a.idbits) < max_pages) ++a.idbits;
  return a;
}

locks::DecodeArgs decode_args(const locks_config_t* cfg, const void* q, const void* k_pool, const void* v_pool,
                              int64_t num_blocks, const int32_t* block_table, const int32_t* seq_lens,
                              const int32_t* selected, int32_t batch, int32_t max_pages, void* out, float* lse,
                              int32_t* counters, float* part_o, float* part_lse) {
  locks::DecodeArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.selected = selected;
  a.counters = counters;
  a.part_o = part_o;
  a.part_lse = part_lse;
  a.out = out;
  a.lse = lse;
  a.num_blocks = num_blocks;
  a.Hkv = cfg->num_kv_heads;
  a.G = cfg->num_q_heads / cfg->num_kv_heads;
  a.P = cfg->page_size;
  a.k = cfg->budget_pages;
  a.max_pages = max_pages;
  a.pages_per_split = decode_pages_per_split(cfg, batch);
  a.splits = decode_splits(cfg, batch);
  a.scale = cfg->softmax_scale;
  return a;
}

// score -> select on a checked workspace
int enqueue_score_select(const locks_config_t* cfg, const void* q, const void* summary_pool, int64_t num_blocks,
                         const int32_t* block_table, const int32_t* seq_lens, int32_t batch, int32_t max_pages,
                         int32_t* selected, void* ws, size_t ws_bytes, hipStream_t stream) {
  uint8_t* region = scratch_base(ws, ws_bytes, score_ws_bytes(cfg, batch, max_pages) - ctl_bytes(cfg, batch));
  float* scores = reinterpret_cast<float*>(region);
  float* sigma = reinterpret_cast<float*>(region +
                                          align_up((size_t)batch * cfg->num_q_heads * max_pages * sizeof(float)));
  locks::ScoreArgs sa = score_args(cfg, q, summary_pool, num_blocks, block_table, seq_lens, max_pages, scores);
  const hipError_t e = cfg->summary_dtype == LOCKS_I4
                           ? locks::launch_page_score_i4(sa, cfg->head_dim, batch, stream)
                           : locks::launch_page_score(sa, cfg->kv_dtype, cfg->head_dim, batch, stream);
  if (e != hipSuccess) return LOCKS_E_HIP;
  locks::SelectArgs a = select_args(cfg, scores, seq_lens, max_pages, selected, sigma);
  return hip_status(locks::launch_select(a, batch, stream));
}

// split-K decode on a checked workspace (arrival counters at its front)
int enqueue_sparse_decode(const locks_config_t* cfg, const void* q, const void* k_pool, const void* v_pool,
                          int64_t num_blocks, const int32_t* block_table, const int32_t* seq_lens,
                          const int32_t* selected, int32_t batch, int32_t max_pages, void* out, float* lse, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  // partial rows laid out for the most splits any batch uses (the workspace layout)
  const size_t rows = (size_t)batch * cfg->num_q_heads * locks::decode_max_splits(cfg->budget_pages, cfg->page_size);
  uint8_t* region = scratch_base(ws, ws_bytes, decode_ws_bytes(cfg, batch) - ctl_bytes(cfg, batch));
  locks::DecodeArgs a = decode_args(cfg, q, k_pool, v_pool, num_blocks, block_table, seq_lens, selected,
                                    batch, max_pages, out, lse, static_cast<int32_t*>(ws),
                                    reinterpret_cast<float*>(region),
                                    reinterpret_cast<float*>(region + align_up(rows * cfg->head_dim * sizeof(float))));
  return hip_status(locks::launch_sparse_decode(a, cfg->kv_dtype, cfg->head_dim, batch, stream));
}

// per-call lists of the cached decode step (page-slot tiles, tile map,
// copies, victims, copy count); they sit just below the decode scratch, which
// is written after them, and may overlap the score scratch, consumed before
size_t cache_ws_bytes(const locks_config_t* cfg, int32_t batch) {
  const size_t n = (size_t)batch * cfg->num_kv_heads * cfg->budget_pages;
  return n ? 5 * align_up(n * sizeof(int32_t)) + kAlign : 0;
}

size_t step_ws_bytes(const locks_config_t* cfg, int32_t batch, int32_t max_pages) {
  const size_t a = score_ws_bytes(cfg, batch, max_pages);
  const size_t b = decode_ws_bytes(cfg, batch) + cache_ws_bytes(cfg, batch);
  return a > b ? a : b;
}

// Hot-page cache buffer: counters, what it was initialised for, clock state,
// then the maps and the cached K and V tiles, each region 256-byte aligned.
struct CacheLayout {
  size_t off[LOCKS_HOT_CACHE_FIELDS];
  size_t bytes;
};

CacheLayout cache_layout(const locks_config_t* cfg, int64_t num_blocks, int32_t capacity) {
  const size_t tiles = (size_t)num_blocks * cfg->num_kv_heads;
  const size_t tile_bytes = (size_t)cfg->page_size * cfg->head_dim * elem_bytes(cfg->kv_dtype);
  const size_t sizes[LOCKS_HOT_CACHE_FIELDS] = {
      locks::kCacheStats * sizeof(int64_t), 2 * sizeof(int64_t), 2 * sizeof(int32_t), tiles * sizeof(int32_t),
      (size_t)capacity * sizeof(int32_t), (size_t)capacity * sizeof(int32_t), (size_t)capacity * sizeof(int32_t),
      (size_t)capacity * tile_bytes, (size_t)capacity * tile_bytes};
  CacheLayout L{};
  size_t at = 0;
  for (int i = 0; i < LOCKS_HOT_CACHE_FIELDS; ++i) {
    L.off[i] = at;
    at += align_up(sizes[i]);
  }
  L.bytes = at;
  return L;
}

int check_cache(const locks_config_t* cfg, int64_t num_blocks, int32_t capacity) {
  if (num_blocks < 1 || capacity < 1) return LOCKS_E_INVALID_ARG;
  // tile ids and page-slot claims are int32
  if (num_blocks * cfg->num_kv_heads >= (int64_t)0x7fffffff) return LOCKS_E_UNSUPPORTED;
  return LOCKS_OK;
}

locks::CacheArgs cache_args(const locks_config_t* cfg, void* cache, int64_t num_blocks, int32_t capacity) {
  const CacheLayout L = cache_layout(cfg, num_blocks, capacity);
  uint8_t* c = static_cast<uint8_t*>(cache);
  locks::CacheArgs a{};
  a.stats = reinterpret_cast<long long*>(c + L.off[LOCKS_HOT_CACHE_STATS]);
  a.meta = reinterpret_cast<long long*>(c + L.off[LOCKS_HOT_CACHE_META]);
  a.state = reinterpret_cast<int32_t*>(c + L.off[LOCKS_HOT_CACHE_CLOCK]);
  a.slot_of = reinterpret_cast<int32_t*>(c + L.off[LOCKS_HOT_CACHE_SLOT_OF]);
  a.tile_of = reinterpret_cast<int32_t*>(c + L.off[LOCKS_HOT_CACHE_TILE_OF]);
  a.stamp = reinterpret_cast<int32_t*>(c + L.off[LOCKS_HOT_CACHE_STAMP]);
  a.flags = reinterpret_cast<int32_t*>(c + L.off[LOCKS_HOT_CACHE_FLAGS]);
  a.k_slots = c + L.off[LOCKS_HOT_CACHE_K];
  a.v_slots = c + L.off[LOCKS_HOT_CACHE_V];
  a.num_blocks = num_blocks;
  a.tile_bytes = (int64_t)cfg->page_size * cfg->head_dim * elem_bytes(cfg->kv_dtype);
  a.Hkv = cfg->num_kv_heads;
  a.P = cfg->page_size;
  a.k = cfg->budget_pages;
  a.capacity = capacity;
  return a;
}

// argument checks shared by the two whole-step entry points
int check_step(const locks_config_t* cfg, const void* q, const void* summary_pool, const void* k_pool,
               const void* v_pool, int64_t num_blocks, const int32_t* block_table, const int32_t* seq_lens,
               int32_t batch, int32_t max_pages, const int32_t* selected, const void* out) {
  int st = check_config(cfg);
  if (st != LOCKS_OK) return st;
  st = check_batch(batch, max_pages);
  if (st != LOCKS_OK) return st;
  if (num_blocks < 0) return LOCKS_E_INVALID_ARG;
  if (batch == 0) return LOCKS_OK;
  if (num_blocks == 0) return LOCKS_E_INVALID_ARG;  // an empty pool cannot be read
  if (!q || !summary_pool || !k_pool || !v_pool || !block_table || !seq_lens || !selected || !out)
    return LOCKS_E_INVALID_ARG;
  return LOCKS_OK;
}

}  // namespace

extern "C" {

const char* locks_status_string(int status) {
  switch (status) {
    case LOCKS_OK: return "ok";
    case LOCKS_E_INVALID_ARG: return "invalid argument";
    case LOCKS_E_UNSUPPORTED: return "unsupported shape or dtype";
    case LOCKS_E_WORKSPACE: return "workspace missing or too small";
    case LOCKS_E_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int locks_version(void) { return 1; }

size_t locks_summary_record_bytes(const locks_config_t* cfg) {
  if (check_config(cfg) != LOCKS_OK) return 0;
  return (size_t)rec_bytes(cfg);
}

int locks_workspace_size(const locks_config_t* cfg, int32_t batch, int32_t max_pages, size_t* bytes) {
  int st = check_config(cfg);
  if (st != LOCKS_OK) return st;
  if (!bytes) return LOCKS_E_INVALID_ARG;
  st = check_batch(batch, max_pages);
  if (st != LOCKS_OK) return st;
  *bytes = step_ws_bytes(cfg, batch, max_pages);
  return LOCKS_OK;
}

int locks_build_summaries(const locks_config_t* cfg, const void* k_pool, int64_t num_blocks,
                          const int32_t* block_ids, int32_t n_ids, void* summary_pool,
                          hipStream_t stream) {
  return locks_build_summaries_ex(cfg, k_pool, num_blocks, block_ids, n_ids, summary_pool, nullptr, stream);
}

int locks_build_summaries_ex(const locks_config_t* cfg, const void* k_pool, int64_t num_blocks,
                             const int32_t* block_ids, int32_t n_ids, void* summary_pool,
                             int32_t* fit_info, hipStream_t stream) {
  int st = check_config(cfg);
  if (st != LOCKS_OK) return st;
  if (n_ids < 0 || num_blocks < 0) return LOCKS_E_INVALID_ARG;
  if (n_ids == 0) return LOCKS_OK;
  if (!k_pool || !block_ids || !summary_pool) return LOCKS_E_INVALID_ARG;
  if (cfg->num_kv_heads > 65535) return LOCKS_E_UNSUPPORTED;
  locks::BuildArgs a{};
  a.k_pool = k_pool;
  a.block_ids = block_ids;
  a.sum_pool = static_cast<uint8_t*>(summary_pool);
  a.num_blocks = num_blocks;
  a.rec_elems = rec_elems(cfg);
  a.rec_bytes = rec_bytes(cfg);
  a.fit_info = fit_info;
  a.Hkv = cfg->num_kv_heads;
  a.P = cfg->page_size;
  a.r = cfg->rank;
  a.n = n_ids;
  return hip_status(locks::launch_build(a, cfg->kv_dtype, cfg->head_dim, cfg->summary_dtype == LOCKS_I4, stream));
}

int locks_page_score(const locks_config_t* cfg, const void* q, const void* summary_pool,
                     int64_t num_blocks, const int32_t* block_table, const int32_t* seq_lens,
                     int32_t batch, int32_t max_pages, float* head_scores, hipStream_t stream) {
  int st = check_config(cfg);
  if (st != LOCKS_OK) return st;
  st = check_batch(batch, max_pages);
  if (st != LOCKS_OK) return st;
  if (num_blocks < 0) return LOCKS_E_INVALID_ARG;
  if (batch == 0) return LOCKS_OK;
  if (num_blocks == 0) return LOCKS_E_INVALID_ARG;  // an empty pool cannot be read
  if (!q || !summary_pool || !block_table || !seq_lens || !head_scores) return LOCKS_E_INVALID_ARG;
  locks::ScoreArgs a = score_args(cfg, q, summary_pool, num_blocks, block_table, seq_lens, max_pages, head_scores);
  if (cfg->summary_dtype == LOCKS_I4) return hip_status(locks::launch_page_score_i4(a, cfg->head_dim, batch, stream));
  return hip_status(locks::launch_page_score(a, cfg->kv_dtype, cfg->head_dim, batch, stream));
}

int locks_select_pages(const locks_config_t* cfg, const float* head_scores, const int32_t* seq_lens,
                       int32_t batch, int32_t max_pages, int32_t* selected, float* page_sigma,
                       hipStream_t stream) {
  int st = check_config(cfg);
  if (st != LOCKS_OK) return st;
  st = check_batch(batch, max_pages);
  if (st != LOCKS_OK) return st;
  if (batch == 0) return LOCKS_OK;
  if (!head_scores || !seq_lens || !selected || !page_sigma) return LOCKS_E_INVALID_ARG;
  locks::SelectArgs a = select_args(cfg, head_scores, seq_lens, max_pages, selected, page_sigma);
  a.want_sigma = 1;
  return hip_status(locks::launch_select(a, batch, stream));
}

int locks_score_select(const locks_config_t* cfg, const void* q, const void* summary_pool,
                       int64_t num_blocks, const int32_t* block_table, const int32_t* seq_lens,
                       int32_t batch, int32_t max_pages, int32_t* selected, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
  int st = check_config(cfg);
  if (st != LOCKS_OK) return st;
  st = check_batch(batch, max_pages);
  if (st != LOCKS_OK) return st;
  if (num_blocks < 0) return LOCKS_E_INVALID_ARG;
  if (batch == 0) return LOCKS_OK;
  if (num_blocks == 0) return LOCKS_E_INVALID_ARG;  // an empty pool cannot be read
  if (!q || !summary_pool || !block_table || !seq_lens || !selected) return LOCKS_E_INVALID_ARG;
  if (!ws || ws_bytes < score_ws_bytes(cfg, batch, max_pages)) return LOCKS_E_WORKSPACE;
  return enqueue_score_select(cfg, q, summary_pool, num_blocks, block_table, seq_lens, batch, max_pages, selected,
                              ws, ws_bytes, stream);
}

int locks_sparse_decode(const locks_config_t* cfg, const void* q, const void* k_pool,
                        const void* v_pool, int64_t num_blocks, const int32_t* block_table,
                        const int32_t* seq_lens, const int32_t* selected, int32_t batch,
                        int32_t max_pages, void* out, float* lse, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  int st = check_config(cfg);
  if (st != LOCKS_OK) return st;
  st = check_batch(batch, max_pages);
  if (st != LOCKS_OK) return st;
  if (num_blocks < 0) return LOCKS_E_INVALID_ARG;
  if (batch == 0) return LOCKS_OK;
  if (num_blocks == 0) return LOCKS_E_INVALID_ARG;  // an empty pool cannot be read
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !selected || !out)
    return LOCKS_E_INVALID_ARG;
  if (!ws || ws_bytes < decode_ws_bytes(cfg, batch)) return LOCKS_E_WORKSPACE;
  return enqueue_sparse_decode(cfg, q, k_pool, v_pool, num_blocks, block_table, seq_lens, selected, batch,
                               max_pages, out, lse, ws, ws_bytes, stream);
}

int locks_decode_step(const locks_config_t* cfg, const void* q, const void* summary_pool, const void* k_pool,
                      const void* v_pool, int64_t num_blocks, const int32_t* block_table,
                      const int32_t* seq_lens, int32_t batch, int32_t max_pages, int32_t* selected,
                      void* out, float* lse, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_step(cfg, q, summary_pool, k_pool, v_pool, num_blocks, block_table, seq_lens, batch, max_pages,
                      selected, out);
  if (st != LOCKS_OK || batch == 0) return st;
  if (!ws || ws_bytes < step_ws_bytes(cfg, batch, max_pages)) return LOCKS_E_WORKSPACE;
  // the head scores and page keys of the first call are consumed before the
  // second call's partials overwrite them (same stream)
  st = enqueue_score_select(cfg, q, summary_pool, num_blocks, block_table, seq_lens, batch, max_pages, selected, ws,
                            ws_bytes, stream);
  if (st != LOCKS_OK) return st;
  return enqueue_sparse_decode(cfg, q, k_pool, v_pool, num_blocks, block_table, seq_lens, selected, batch,
                               max_pages, out, lse, ws, ws_bytes, stream);
}

int locks_hot_cache_layout(const locks_config_t* cfg, int64_t num_blocks, int32_t capacity,
                           int64_t* offsets, size_t* bytes) {
  int st = check_config(cfg);
  if (st != LOCKS_OK) return st;
  st = check_cache(cfg, num_blocks, capacity);
  if (st != LOCKS_OK) return st;
  if (!bytes) return LOCKS_E_INVALID_ARG;
  const CacheLayout L = cache_layout(cfg, num_blocks, capacity);
  if (offsets)
    for (int i = 0; i < LOCKS_HOT_CACHE_FIELDS; ++i) offsets[i] = (int64_t)L.off[i];
  *bytes = L.bytes;
  return LOCKS_OK;
}

int locks_hot_cache_init(const locks_config_t* cfg, void* cache, int64_t num_blocks, int32_t capacity,
                         hipStream_t stream) {
  int st = check_config(cfg);
  if (st != LOCKS_OK) return st;
  st = check_cache(cfg, num_blocks, capacity);
  if (st != LOCKS_OK) return st;
  if (!cache) return LOCKS_E_INVALID_ARG;
  locks::CacheArgs a = cache_args(cfg, cache, num_blocks, capacity);
  return hip_status(locks::launch_cache_init(a, num_blocks * cfg->num_kv_heads, stream));
}

int locks_decode_step_cached(const locks_config_t* cfg, const void* q, const void* summary_pool,
                             const void* k_pool, const void* v_pool, int64_t num_blocks,
                             const int32_t* block_table, const int32_t* seq_lens, int32_t batch,
                             int32_t max_pages, int32_t* selected, void* out, float* lse, void* cache,
                             int32_t capacity, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_step(cfg, q, summary_pool, k_pool, v_pool, num_blocks, block_table, seq_lens, batch, max_pages,
                      selected, out);
  if (st != LOCKS_OK || batch == 0) return st;
  st = check_cache(cfg, num_blocks, capacity);
  if (st != LOCKS_OK) return st;
  if (!cache) return LOCKS_E_INVALID_ARG;
  const int64_t n = (int64_t)batch * cfg->num_kv_heads * cfg->budget_pages;
  if (n > capacity) return LOCKS_E_INVALID_ARG;  // one step's tiles must fit
  if (!ws || ws_bytes < step_ws_bytes(cfg, batch, max_pages)) return LOCKS_E_WORKSPACE;
  st = enqueue_score_select(cfg, q, summary_pool, num_blocks, block_table, seq_lens, batch, max_pages, selected, ws,
                            ws_bytes, stream);
  if (st != LOCKS_OK) return st;
  // the lists sit below the decode scratch
  const size_t dec_scratch = decode_ws_bytes(cfg, batch) - ctl_bytes(cfg, batch);
  uint8_t* lists = scratch_base(ws, ws_bytes, dec_scratch) - cache_ws_bytes(cfg, batch);
  const size_t list = align_up((size_t)n * sizeof(int32_t));
  locks::CacheArgs a = cache_args(cfg, cache, num_blocks, capacity);
  a.selected = selected;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.tile_e = reinterpret_cast<int32_t*>(lists);
  a.map = reinterpret_cast<int32_t*>(lists + list);
  a.fill = reinterpret_cast<int32_t*>(lists + 2 * list);
  a.victims = reinterpret_cast<int32_t*>(lists + 4 * list);
  a.fill_count = reinterpret_cast<int32_t*>(lists + 5 * list);
  a.k_src = k_pool;
  a.v_src = v_pool;
  a.max_pages = max_pages;
  a.batch = batch;
  if (locks::launch_cache_admit(a, stream) != hipSuccess) return LOCKS_E_HIP;
  if (locks::launch_cache_fill(a, stream) != hipSuccess) return LOCKS_E_HIP;
  const size_t rows = (size_t)batch * cfg->num_q_heads * locks::decode_max_splits(cfg->budget_pages, cfg->page_size);
  uint8_t* region = scratch_base(ws, ws_bytes, dec_scratch);
  locks::DecodeArgs d = decode_args(cfg, q, a.k_slots, a.v_slots, num_blocks, block_table, seq_lens, selected,
                                    batch, max_pages, out, lse, static_cast<int32_t*>(ws),
                                    reinterpret_cast<float*>(region),
                                    reinterpret_cast<float*>(region + align_up(rows * cfg->head_dim * sizeof(float))));
  d.tile_map = a.map;
  d.map_tiles = capacity;
  return hip_status(locks::launch_sparse_decode(d, cfg->kv_dtype, cfg->head_dim, batch, stream));
}

}  // extern "C"

// Kernel argument blocks and launchers of the Locks library (host + device).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace locks {

struct ScoreArgs {
  const void* q;              // [B][Hq][D] kv dtype
  const uint8_t* sum_pool;    // [blocks][Hkv][record]
  const int32_t* block_table; // [B][max_pages]
  const int32_t* seq_lens;    // [B]
  float* scores;              // [B][Hq][max_pages]
  int64_t num_blocks;
  int64_t rec_elems;          // elements per record
  int Hkv, G, P, r, max_pages;
  int ppw;                    // pages per wave, set by the launcher (<= 128 LDS-staged, else <= 64)
  int head_major;             // LDS-staged scorer: a workgroup's waves take adjacent KV heads
  float scale;
};

struct SelectArgs {
  const float* scores;        // [B][Hq][max_pages]
  const int32_t* seq_lens;    // [B]
  int32_t* selected;          // [B][Hkv][k]
  float* sigma;               // [B][Hkv][max_pages]
  int want_sigma;             // 0: sigma is scratch only (not left as an output)
  int Hkv, G, P, k, max_pages;
  int idbits;                 // bits that hold any page id < max_pages (>= 1)
};

struct DecodeArgs {
  const void* q;              // [B][Hq][D]
  const void* k_pool;         // [blocks][Hkv][P][D]
  const void* v_pool;
  const int32_t* block_table; // [B][max_pages]
  const int32_t* seq_lens;    // [B]
  const int32_t* selected;    // [B][Hkv][k]
  float* part_o;              // [B][Hkv][splits][G][D]
  float* part_lse;            // [B][Hkv][splits][G]
  int32_t* counters;          // [B][Hkv] arrival counters, zero between calls
  void* out;                  // [B][Hq][D] kv dtype
  float* lse;                 // [B][Hq] or null
  // [B][Hkv][k] tile per page slot, or null. Null: slot j of (b, h) reads
  // tile block_table[b][j] * Hkv + h of the pools. Else: it reads tile
  // tile_map[(b Hkv + h) k + slot] of pools of map_tiles [P][D] tiles (a
  // negative entry contributes nothing).
  const int32_t* tile_map;
  int64_t num_blocks;
  int64_t map_tiles;
  int Hkv, G, P, k, max_pages;
  int pages_per_split, splits;
  float scale;
};

struct BuildArgs {
  const void* k_pool;         // [blocks][Hkv][P][D]
  const int32_t* block_ids;   // [n]
  uint8_t* sum_pool;          // [blocks][Hkv][record]
  int64_t num_blocks;
  int64_t rec_elems;          // elements per record (bf16 / fp32 records)
  int64_t rec_bytes;          // bytes per record
  int32_t* fit_info;          // [n][Hkv] products of the eigensolver (negative: bound not met), or null
  int Hkv, P, r, n;
};

// Hot-page cache of host-resident K/V tiles in device memory: persistent
// state in the caller's cache buffer, per-call lists in the workspace.
struct CacheArgs {
  const int32_t* selected;    // [B][Hkv][k] logical pages of this step
  const int32_t* block_table; // [B][max_pages]
  const int32_t* seq_lens;    // [B]
  long long* stats;           // [kCacheStats] counters, accumulated
  long long* meta;            // [2] capacity, tiles: what the state was initialised for
  int32_t* state;             // [2] clock hand, step
  int32_t* slot_of;           // [tiles] cache slot holding a (block, head) tile, or -1
  int32_t* tile_of;           // [C] tile held by a slot, or -1
  int32_t* stamp;             // [C] last step that used the slot
  int32_t* flags;             // [C] kCacheRef | kCachePartial
  int32_t* tile_e;            // [n] workspace: tile of each page slot, or -1
  int32_t* map;               // [n] workspace: cache slot of each page slot (the decode's tile map)
  int32_t* fill;              // [n][2] workspace: (slot, tile) copies of this step
  int32_t* victims;           // [n] workspace
  int32_t* fill_count;        // [1] workspace
  const void* k_src;          // K / V pools, [tiles][P][D] (normally in host memory)
  const void* v_src;
  void* k_slots;              // [C][P][D] cached tiles
  void* v_slots;
  int64_t num_blocks;
  int64_t tile_bytes;         // P * D * element bytes
  int Hkv, P, k, max_pages, batch, capacity;
};
constexpr int kCacheRef = 1;      // used since the clock hand last passed the slot
constexpr int kCachePartial = 2;  // copied while its page was incomplete: copied again on its next use
// counters: hits, misses, refreshes, shared, failed, steps
constexpr int kCacheStats = 8;

// Quantized ("i4") summary record of one (block, KV head), bytes:
//   r + 2 nibble rows of d/2 bytes: the basis vectors' 4-bit codes (excess 8),
//     then the high and the low nibbles of the centroid's 8-bit codes
//     (excess 128); element a of a row lives in 32-bit word
//     (a % 32) / 8 * (d / 32) + a / 32, nibble e / 2 (even e) or 4 + e / 2
//     (odd e), e = a % 8
//   P rows of r bytes: the coefficient codes (excess 128)
//   r + 1 + P bf16 scales: basis vectors, centroid, tokens
//   zero padding to a multiple of 16 bytes
constexpr int i4_head_bytes(int d, int r) { return (r + 2) * (d / 2); }
constexpr int i4_scale_offset(int d, int r, int P) { return i4_head_bytes(d, r) + P * r; }
constexpr int i4_record_bytes(int d, int r, int P) {
  return (i4_scale_offset(d, r, P) + 2 * (1 + r + P) + 15) / 16 * 16;
}

hipError_t launch_page_score(const ScoreArgs& a, int dtype, int D, int batch, hipStream_t s);
hipError_t launch_select(const SelectArgs& a, int batch, hipStream_t s);
hipError_t launch_sparse_decode(const DecodeArgs& a, int dtype, int D, int batch, hipStream_t s);
int decode_pages_per_split(int page_size, int tiles_per_wave);
// tiles per wave for `units` (sequence, KV head) units of k pages
int decode_tiles_per_wave(int64_t units, int k, int page_size, bool f32);
// the most splits any launch uses (the workspace is sized for it)
int decode_max_splits(int k, int page_size);
// dtype: 0 bf16, 1 fp32 keys; i4: write quantized records (bf16 keys only)
hipError_t launch_build(const BuildArgs& a, int dtype, int D, bool i4, hipStream_t s);
// cache state for `tiles` tiles and `capacity` slots: empty, counters zero
hipError_t launch_cache_init(const CacheArgs& a, int64_t tiles, hipStream_t s);
// look up this step's tiles, evict, list the copies, write the tile map
hipError_t launch_cache_admit(const CacheArgs& a, hipStream_t s);
// copy the listed tiles from the pools into their slots
hipError_t launch_cache_fill(const CacheArgs& a, hipStream_t s);
// page scores from quantized records (bf16 q)
hipError_t launch_page_score_i4(const ScoreArgs& a, int D, int batch, hipStream_t s);

}  // namespace locks

// (f4) Hot-page cache in device memory for K/V pools held in host memory,
// [Locks] §5.3 Table 3 and App. B.4.2: the full K/V stays in host memory and
// the pages used often are kept in a smaller GPU cache. The pages name no
// policy; this one is second-chance (clock) replacement over (block, KV head)
// tiles, the unit a selection reads:
//
//   - every page slot a step selects is a tile t = block * Hkv + h;
//   - a tile resident in slot s is a hit: s is marked used this step and
//     referenced; a tile copied while its page was still incomplete is copied
//     again (a refresh), since tokens may have been appended since;
//   - each missing tile (the first page slot naming it, when several do) takes
//     the next evictable slot from the clock hand: the hand walks the slots in
//     order, skips slots used this step (a taken slot counts as used), clears
//     the reference mark of a referenced slot and passes on, and takes an
//     unreferenced one; it stops just past the last slot taken. Missing tiles take victims in page-slot
//     order (sequence, KV head, slot);
//   - taken and refreshed tiles are then copied from the pools into their
//     slots, and the decode reads every selected tile from the cache.
//
// A capacity of at least batch * Hkv * k slots guarantees a slot for every
// missing tile: at most that many slots are used in one step.
//
// Page slots of one step that name the same tile (blocks shared between
// sequences) are served by one slot. When such a tile is resident and was
// copied while incomplete, each of them may see the incomplete mark and
// list the copy (the same bytes twice) and count a refresh.
//
// The admission runs in one workgroup of 1024 threads (a step selects a few
// thousand tiles); the state its threads share lives in global memory,
// accessed with workgroup-scope atomics, so that each phase sees the previous
// phase's stores after the workgroup barrier.
#include "common.h"
#include "kernels.h"

#include <climits>

namespace locks {

namespace {

constexpr int kAdmitThreads = 1024;
constexpr int kAdmitWaves = kAdmitThreads / 64;
constexpr int kFillThreads = 256;
constexpr int kFillUnroll = 4;

enum { kStatHits = 0, kStatMisses, kStatRefreshes, kStatShared, kStatFailed, kStatSteps };

__device__ __forceinline__ int ld_wg(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void st_wg(int32_t* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

struct AdmitLds {
  int wtot[kAdmitWaves];
  int last;
  int nfill;
  int cnt[kCacheStats];
};

// exclusive prefix count of `f` over the workgroup's threads (in thread
// order); every thread must call it
__device__ int scan_flag(bool f, AdmitLds& L, int& total) {
  const unsigned long long m = __ballot(f);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int ex = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) L.wtot[w] = __popcll(m);
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kAdmitWaves; ++i) {
    const int t = L.wtot[i];
    base += i < w ? t : 0;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return base + ex;
}

// page slot e = (b Hkv + h) k + i: its tile, or -1, and whether its page is complete
__device__ __forceinline__ int slot_tile(const CacheArgs& a, int e, bool& complete) {
  const int unit = e / a.k;
  const int b = unit / a.Hkv, h = unit - b * a.Hkv;
  const int j = a.selected[e];
  const int T = clamp_len(a.seq_lens[b], a.max_pages, a.P);
  const int J = (T + a.P - 1) / a.P;
  complete = false;
  if (j < 0 || j >= J) return -1;
  const int blk = a.block_table[(int64_t)b * a.max_pages + j];
  if (blk < 0 || (int64_t)blk >= a.num_blocks) return -1;
  complete = (int64_t)(j + 1) * a.P <= T;
  return blk * a.Hkv + h;
}

__global__ __launch_bounds__(kAdmitThreads) void cache_admit_kernel(CacheArgs a) {
  __shared__ AdmitLds L;
  const int tid = threadIdx.x;
  const int n = a.batch * a.Hkv * a.k;
  const int C = a.capacity;
  if (tid < kCacheStats) L.cnt[tid] = 0;
  if (tid == 0) L.nfill = 0;
  __syncthreads();
  // a cache initialised for another capacity or pool: serve nothing
  if (a.meta[0] != C || a.meta[1] != a.num_blocks * a.Hkv) {
    for (int e = tid; e < n; e += kAdmitThreads) a.map[e] = -1;
    if (tid == 0) {
      a.fill_count[0] = 0;
      a.stats[kStatFailed] += n;
    }
    return;
  }
  const int cur = a.state[1] + 1;

  // 1. lookups: hits and refreshes take their slot; misses claim their tile
  //    for the lowest page slot naming it (slot_of holds INT_MIN + e meanwhile)
  for (int e = tid; e < n; e += kAdmitThreads) {
    bool complete;
    const int t = slot_tile(a, e, complete);
    a.tile_e[e] = t;
    if (t < 0) {
      a.map[e] = -1;
      continue;
    }
    const int s = ld_wg(a.slot_of + t);
    if (s >= 0) {
      a.map[e] = s;
      const int f = ld_wg(a.flags + s);
      st_wg(a.stamp + s, cur);
      st_wg(a.flags + s, kCacheRef | (complete ? 0 : kCachePartial));
      if (f & kCachePartial) {
        const int q = atomicAdd(&L.nfill, 1);
        a.fill[2 * q] = s;
        a.fill[2 * q + 1] = t;
        atomicAdd(&L.cnt[kStatRefreshes], 1);
      } else {
        atomicAdd(&L.cnt[kStatHits], 1);
      }
    } else {
      a.map[e] = -2;
      __hip_atomic_fetch_min(a.slot_of + t, INT_MIN + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
  __syncthreads();

  // 2. owners (the claiming page slot of each missing tile) ranked in page-slot order
  int M = 0;
  for (int c = 0; c < n; c += kAdmitThreads) {
    const int e = c + tid;
    bool own = false;
    if (e < n && a.map[e] == -2) own = ld_wg(a.slot_of + a.tile_e[e]) == INT_MIN + e;
    int tot;
    const int r = scan_flag(own, L, tot);
    if (own) a.map[e] = -3 - (M + r);
    M += tot;
  }

  // 3. the clock hand finds M victims (slots not used this step, unreferenced)
  int hand = a.state[0];
  int got = 0;
  const int W = C < kAdmitThreads ? C : kAdmitThreads;
  const int max_rounds = 2 * ((C + W - 1) / W) + 2;  // two turns clear every reference mark
  for (int it = 0; it < max_rounds && got < M; ++it) {
    const bool in = tid < W;
    int s = hand + tid;
    if (s >= C) s -= C;
    const int stp = in ? ld_wg(a.stamp + s) : cur;
    const int fl = in ? ld_wg(a.flags + s) : 0;
    const bool ev = in && stp != cur && !(fl & kCacheRef);
    int tot;
    const int r = scan_flag(ev, L, tot);
    const int need = M - got;
    int last = W - 1;  // offset of the last slot the hand passes
    if (tot >= need) {
      if (ev && r == need - 1) L.last = tid;
      __syncthreads();
      last = L.last;
      __syncthreads();
    }
    if (ev && r < need) {
      st_wg(a.victims + got + r, s);
      st_wg(a.stamp + s, cur);  // taken: a second turn of the hand skips it
    }
    if (in && tid <= last && stp != cur && (fl & kCacheRef)) st_wg(a.flags + s, fl & ~kCacheRef);
    hand += last + 1;
    if (hand >= C) hand -= C;
    got += tot < need ? tot : need;
    __syncthreads();  // the next round may revisit these slots (C < 2 W)
  }

  // 4. owners move into their victims' slots
  for (int e = tid; e < n; e += kAdmitThreads) {
    const int m = a.map[e];
    if (m > -3) continue;
    const int rank = -3 - m;
    const int t = a.tile_e[e];
    if (rank < got) {
      const int s = ld_wg(a.victims + rank);
      const int old = ld_wg(a.tile_of + s);
      if (old >= 0) st_wg(a.slot_of + old, -1);
      bool complete;
      slot_tile(a, e, complete);
      st_wg(a.slot_of + t, s);
      st_wg(a.tile_of + s, t);
      st_wg(a.stamp + s, cur);
      st_wg(a.flags + s, kCacheRef | (complete ? 0 : kCachePartial));
      a.map[e] = s;
      const int q = atomicAdd(&L.nfill, 1);
      a.fill[2 * q] = s;
      a.fill[2 * q + 1] = t;
      atomicAdd(&L.cnt[kStatMisses], 1);
    } else {
      st_wg(a.slot_of + t, -1);
      a.map[e] = -1;
      atomicAdd(&L.cnt[kStatFailed], 1);
    }
  }
  __syncthreads();

  // 5. page slots naming a tile another page slot claimed share its slot
  for (int e = tid; e < n; e += kAdmitThreads) {
    if (a.map[e] != -2) continue;
    a.map[e] = ld_wg(a.slot_of + a.tile_e[e]);
    atomicAdd(&L.cnt[kStatShared], 1);
  }
  __syncthreads();
  if (tid == 0) {
    a.fill_count[0] = L.nfill;
    a.state[0] = hand;
    a.state[1] = cur;
    a.stats[kStatSteps] += 1;
  }
  if (tid < kStatSteps) a.stats[tid] += L.cnt[tid];
}

// one tile copy per workgroup iteration: 16-byte words, kFillUnroll loads of
// K and V in flight per thread before the stores
__global__ __launch_bounds__(kFillThreads) void cache_fill_kernel(CacheArgs a) {
  const int cnt = a.fill_count[0];
  const int64_t words = a.tile_bytes / 16;
  for (int q = blockIdx.x; q < cnt; q += gridDim.x) {
    const int s = a.fill[2 * q], t = a.fill[2 * q + 1];
    const u32x4_t* ks = reinterpret_cast<const u32x4_t*>(static_cast<const uint8_t*>(a.k_src) + t * a.tile_bytes);
    const u32x4_t* vs = reinterpret_cast<const u32x4_t*>(static_cast<const uint8_t*>(a.v_src) + t * a.tile_bytes);
    u32x4_t* kd = reinterpret_cast<u32x4_t*>(static_cast<uint8_t*>(a.k_slots) + s * a.tile_bytes);
    u32x4_t* vd = reinterpret_cast<u32x4_t*>(static_cast<uint8_t*>(a.v_slots) + s * a.tile_bytes);
    for (int64_t w0 = threadIdx.x; w0 < words; w0 += kFillThreads * kFillUnroll) {
      u32x4_t kb[kFillUnroll], vb[kFillUnroll];
#pragma unroll
      for (int u = 0; u < kFillUnroll; ++u) {
        const int64_t w = w0 + u * kFillThreads;
        if (w < words) {
          kb[u] = ks[w];
          vb[u] = vs[w];
        }
      }
#pragma unroll
      for (int u = 0; u < kFillUnroll; ++u) {
        const int64_t w = w0 + u * kFillThreads;
        if (w < words) {
          kd[w] = kb[u];
          vd[w] = vb[u];
        }
      }
    }
  }
}

__global__ void cache_init_kernel(CacheArgs a, int64_t tiles) {
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = i0; i < tiles; i += stride) a.slot_of[i] = -1;
  for (int64_t i = i0; i < a.capacity; i += stride) {
    a.tile_of[i] = -1;
    a.stamp[i] = -1;
    a.flags[i] = 0;
  }
  if (i0 < kCacheStats) a.stats[i0] = 0;
  if (i0 == 0) {
    a.meta[0] = a.capacity;
    a.meta[1] = tiles;
    a.state[0] = 0;
    a.state[1] = 0;
  }
}

}  // namespace

hipError_t launch_cache_init(const CacheArgs& a, int64_t tiles, hipStream_t stream) {
  const int64_t most = tiles > a.capacity ? tiles : a.capacity;
  int64_t blocks = (most + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(cache_init_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a, tiles);
  return hipGetLastError();
}

hipError_t launch_cache_admit(const CacheArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(cache_admit_kernel, dim3(1), dim3(kAdmitThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_cache_fill(const CacheArgs& a, hipStream_t stream) {
  const int n = a.batch * a.Hkv * a.k;
  const int grid = n < 1024 ? (n > 0 ? n : 1) : 1024;
  hipLaunchKernelGGL(cache_fill_kernel, dim3(grid), dim3(kFillThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace locks

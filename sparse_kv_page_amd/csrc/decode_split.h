// Device code of the split-K sparse decode, [Locks] §2. See sparse_decode.hip.
#pragma once

#include "common.h"
#include "kernels.h"

namespace locks {

constexpr int kDecWaves = 8;
constexpr int kDecThreads = kDecWaves * 64;
constexpr int kDecTile = 16;
// 16-token tiles per wave: 8 (16 pages of 64 per 8-wave workgroup) or 4
// (8 pages) when the grid still holds a workgroup per CU, else 2 (more,
// smaller splits). The largest that fills the chip is taken: fewer, longer
// workgroups keep fewer loads in flight per CU, which the scattered tiles are
// served faster with.
constexpr int kDecTilesPerWaveXL = 8;
constexpr int kDecTilesPerWaveLarge = 4;
constexpr int kDecTilesPerWaveSmall = 2;
// tiles whose K/V loads a wave keeps in flight: one (the next tile's loads go
// out before the current tile is computed). Fewer requests in flight served
// the scattered tiles faster than issuing every load at once (16.7 vs
// 17.9 us at 128K context, batch 8).
constexpr int kDecLoadDepth = 1;

namespace dec_detail {

template <typename T, int D>
struct QkMfma;

template <int D>
struct QkMfma<bf16_t, D> {
  static constexpr int kSteps = D / 32;
  using Op = bf16x8_t;
  static __device__ __forceinline__ Op zero() { return Op{0, 0, 0, 0, 0, 0, 0, 0}; }
  // row element offset of step s for lane group kg
  static __device__ __forceinline__ int off(int s, int kg) { return s * 32 + kg * 8; }
  static __device__ __forceinline__ Op load_nt(const bf16_t* p) { return __builtin_bit_cast(Op, ld_nt4(p)); }
  static __device__ __forceinline__ Op load(const bf16_t* p) { return *reinterpret_cast<const Op*>(p); }
  static __device__ __forceinline__ f32x4_t mfma(Op a, Op b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <int D>
struct QkMfma<float, D> {
  static constexpr int kSteps = D / 4;
  using Op = float;
  static __device__ __forceinline__ Op zero() { return 0.f; }
  static __device__ __forceinline__ int off(int s, int kg) { return s * 4 + kg; }
  static __device__ __forceinline__ Op load_nt(const float* p) { return __uint_as_float(ld_nt1(p)); }
  static __device__ __forceinline__ Op load(const float* p) { return *p; }
  static __device__ __forceinline__ f32x4_t mfma(Op a, Op b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// 8 consecutive V elements of one row as raw words (bf16: 4 words, fp32: 8)
template <typename T>
struct VRow {
  static constexpr int kWords = 8 * (int)sizeof(T) / 4;
  uint32_t w[kWords];
  __device__ __forceinline__ void load(const T* p) { ld_nt_words<kWords>(p, w); }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < kWords; ++i) w[i] = 0u;
  }
  __device__ __forceinline__ float at(int e) const {
    if constexpr (sizeof(T) == 2) return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
    else return __uint_as_float(w[e]);
  }
};

}  // namespace dec_detail

template <int D, int GQ>
struct alignas(16) DecodeLds {
  float pbuf[kDecWaves][4][GQ][4];
  float abuf[kDecWaves][GQ];
  // per wave: its current K tile (bf16, staged for the MFMA operand layout)
  // while it streams, then its output partials for the workgroup merge
  union alignas(16) WaveBuf {
    float mo[4][GQ][D];
    uint8_t kst[kDecTile * D * 2];
  } wv[kDecWaves];
  float mm[kDecWaves][GQ];
  float ml[kDecWaves][GQ];
  int last_s;
};


// One split (workgroup of kDecWaves waves, TPW tiles each) of the unit (b, h);
// `splits` splits per unit.
template <typename T, int D, int GQ, int TPW>
__device__ __forceinline__ void decode_split(const DecodeArgs& a, int split, int h, int b, int splits,
                                             DecodeLds<D, GQ>& lds) {
  using namespace dec_detail;
  using Q = QkMfma<T, D>;
  constexpr int G = GQ;
  constexpr int NC = D / 8;  // 8-wide column slices; PV lanes: 16 slices x 4 token groups per pass
  static_assert(NC % 8 == 0, "d must be a multiple of 64");
  constexpr int kColPasses = NC >= 16 ? NC / 16 : 1;  // d = 64: lanes with c >= 8 idle
  auto& pbuf = lds.pbuf;
  auto& abuf = lds.abuf;
  auto& mm = lds.mm;
  auto& ml = lds.ml;
  int& last_s = lds.last_s;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);  // uniform: tile lookups use scalar loads
  const int P = a.P;
  const int Hq = a.Hkv * G;
  const int Tl = __builtin_amdgcn_readfirstlane(clamp_len(a.seq_lens[b], a.max_pages, P));
  const int J = (Tl + P - 1) / P;
  const int64_t unit = (int64_t)b * a.Hkv + h;
  const int32_t* sel = a.selected + unit * a.k;
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;
  const T* kp = reinterpret_cast<const T*>(a.k_pool);
  const T* vp = reinterpret_cast<const T*>(a.v_pool);
  const float zscale = a.scale * kLog2e;
  const int tiles_per_page = P / kDecTile;

  // MFMA roles: n = head column / token row inside a tile, kg = k group
  const int n = lane & 15;
  const int kg = lane >> 4;
  // PV roles: c = 8-column slice, tg = token group (4 tokens)
  const int c = lane & 15;
  const int tg = lane >> 4;
  const bool c_ok = c < NC;

  typename Q::Op qb[Q::kSteps];
  {
    const T* qrow = reinterpret_cast<const T*>(a.q) + ((int64_t)b * Hq + (int64_t)h * G + (n < G ? n : 0)) * D;
#pragma unroll
    for (int s = 0; s < Q::kSteps; ++s) qb[s] = n < G ? Q::load(qrow + Q::off(s, kg)) : Q::zero();
  }

  // ---- locate this wave's tiles (scalar loads), then issue every K/V load ----
  int ntok[TPW];
  int64_t tile_off[TPW];
  int jsel[TPW];
  int slots[TPW];
  const int slot_end = min((split + 1) * a.pages_per_split, a.k);
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int ti = wave_u + kDecWaves * i;
    const int slot = split * a.pages_per_split + ti / tiles_per_page;
    slots[i] = slot;
    jsel[i] = slot < slot_end ? sel[slot] : -1;
  }
  const int32_t* tmap = a.tile_map ? a.tile_map + unit * a.k : nullptr;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int ti = wave_u + kDecWaves * i;
    const int sub = ti % tiles_per_page;
    const int j = jsel[i];
    int nt = 0;
    int64_t off = 0;
    if (j >= 0 && j < J) {
      int64_t tile = -1;
      if (tmap) {
        const int m = tmap[slots[i]];
        if (m >= 0 && (int64_t)m < a.map_tiles) tile = m;
      } else {
        const int blk = bt[j];
        if (blk >= 0 && (int64_t)blk < a.num_blocks) tile = (int64_t)blk * a.Hkv + h;
      }
      if (tile >= 0) {
        nt = min(P, Tl - j * P) - sub * kDecTile;
        nt = nt < 0 ? 0 : (nt > kDecTile ? kDecTile : nt);
        off = (tile * P + sub * kDecTile) * D;
      }
    }
    ntok[i] = nt;
    tile_off[i] = off;
  }
  // Loads are unconditional (an empty tile reads row 0 of the pool, a lane
  // past the valid tokens reads the tile's first row) so that no load sits
  // inside a branch; K rows past ntok only reach S rows that are masked to
  // -inf, and V rows past ntok are zeroed below.
  // bf16: the K tile (16 rows of D) is loaded as contiguous 1 KiB blocks (lane
  // l takes bytes 16 l .. 16 l + 15 of each) and rearranged through the
  // wave's LDS buffer into the MFMA operand layout (lane (n, kg) needs row n);
  // the 16-byte chunks of a row are XOR-swizzled by row so those reads are
  // free of bank conflicts. fp32 K rows, and the two-tile variant (whose
  // register budget is 128 and would spill the staging), load the operand
  // layout straight into registers.
  constexpr bool kLdsK = sizeof(T) == 2 && TPW >= 4;
  constexpr int kRowBytes = D * 2;
  auto kswz = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };
  typename Q::Op ka[kLdsK ? 1 : TPW][Q::kSteps];
  u32x4_t kraw[kLdsK ? TPW : 1][Q::kSteps];
  VRow<T> vr[TPW][kColPasses][4];
  const int cc = c_ok ? c : 0;
  auto load_tile = [&](int i) {
    const T* kt = kp + tile_off[i];
    const T* vt = vp + tile_off[i];
    if constexpr (kLdsK) {
#pragma unroll
      for (int s = 0; s < Q::kSteps; ++s) kraw[i][s] = ld_nt4(kt + s * 512 + lane * 8);
    } else {
      const int krow = n < ntok[i] ? n : 0;
#pragma unroll
      for (int s = 0; s < Q::kSteps; ++s) ka[i][s] = Q::load_nt(kt + (int64_t)krow * D + Q::off(s, kg));
    }
#pragma unroll
    for (int cp = 0; cp < kColPasses; ++cp)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tok = 4 * tg + e;
        vr[i][cp][e].load(vt + (int64_t)(tok < ntok[i] ? tok : 0) * D + (cp * 16 + cc) * 8);
      }
  };
  // the first kDecLoadDepth tiles' loads go out now, each later tile's when
  // the tile kDecLoadDepth before it is about to be computed
  constexpr int kDepth = kDecLoadDepth < TPW ? kDecLoadDepth : TPW;
#pragma unroll
  for (int i = 0; i < kDepth; ++i) load_tile(i);

  // ---- online softmax and P V over the tiles ----
  float m_run = -INFINITY, l_run = 0.f;  // head n, valid in lanes n < G
  float o[kColPasses][G][8];
#pragma unroll
  for (int cp = 0; cp < kColPasses; ++cp)
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[cp][g][e] = 0.f;

#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    if (i + kDepth < TPW) load_tile(i + kDepth);
    if (ntok[i] < kDecTile || !c_ok) {
#pragma unroll
      for (int cp = 0; cp < kColPasses; ++cp)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (!c_ok || 4 * tg + e >= ntok[i]) vr[i][cp][e].zero();
    }
    if (ntok[i] == 0) continue;
    if constexpr (kLdsK) {
      // rows past ntok hold other tokens' (or unused) keys; their logits are
      // masked to -inf below
      uint8_t* ks = lds.wv[wave].kst;
#pragma unroll
      for (int s = 0; s < Q::kSteps; ++s) {
        const int e0 = s * 512 + lane * 8;
        const int r = e0 / D;
        *reinterpret_cast<u32x4_t*>(ks + r * kRowBytes + (((e0 % D) / 8) ^ kswz(r)) * 16) = kraw[i][s];
      }
      wave_lds_sync();
    }
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < Q::kSteps; ++s) {
      if constexpr (kLdsK) {
        const typename Q::Op kop = *reinterpret_cast<const typename Q::Op*>(
            lds.wv[wave].kst + n * kRowBytes + ((4 * s + kg) ^ kswz(n)) * 16);
        acc = Q::mfma(kop, qb[s], acc);
      } else {
        acc = Q::mfma(ka[i][s], qb[s], acc);
      }
    }
    // lane holds S[token 4 kg + e][head n]
    float z[4];
    float mt = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      z[e] = 4 * kg + e < ntok[i] ? acc[e] * zscale : -INFINITY;
      mt = fmaxf(mt, z[e]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16, kWave));
    mt = fmaxf(mt, __shfl_xor(mt, 32, kWave));
    const float m_new = fmaxf(m_run, mt);          // finite: the tile has a valid token
    const float alpha = exp2_fast(m_run - m_new);  // m_run = -inf -> 0
    float pe[4];
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pe[e] = exp2_fast(z[e] - m_new);
      ps += pe[e];
    }
    ps += __shfl_xor(ps, 16, kWave);
    ps += __shfl_xor(ps, 32, kWave);
    l_run = l_run * alpha + ps;
    m_run = m_new;
    if (n < G) {
      *reinterpret_cast<f32x4_t*>(&pbuf[wave][kg][n][0]) = f32x4_t{pe[0], pe[1], pe[2], pe[3]};
      if (kg == 0) abuf[wave][n] = alpha;
    }
    wave_lds_sync();
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float al = abuf[wave][g];
      const f32x4_t pv = *reinterpret_cast<const f32x4_t*>(&pbuf[wave][tg][g][0]);
#pragma unroll
      for (int cp = 0; cp < kColPasses; ++cp)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float x = o[cp][g][e] * al;
          x = fmaf(pv[0], vr[i][cp][0].at(e), x);
          x = fmaf(pv[1], vr[i][cp][1].at(e), x);
          x = fmaf(pv[2], vr[i][cp][2].at(e), x);
          x = fmaf(pv[3], vr[i][cp][3].at(e), x);
          o[cp][g][e] = x;
        }
    }
    wave_lds_sync();
  }

  // ---- merge the waves of the workgroup ----
  if (c_ok) {
#pragma unroll
    for (int cp = 0; cp < kColPasses; ++cp)
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float* dst = &lds.wv[wave].mo[tg][g][(cp * 16 + c) * 8];
        *reinterpret_cast<f32x4_t*>(dst) = f32x4_t{o[cp][g][0], o[cp][g][1], o[cp][g][2], o[cp][g][3]};
        *reinterpret_cast<f32x4_t*>(dst + 4) = f32x4_t{o[cp][g][4], o[cp][g][5], o[cp][g][6], o[cp][g][7]};
      }
  }
  if (kg == 0 && n < G) { mm[wave][n] = m_run; ml[wave][n] = l_run; }
  __syncthreads();

  // Partials are published with device-scope (write-through) stores and read
  // back with device-scope loads, so no cache-wide write-back or invalidate
  // is needed: the stores of every wave are complete (vmcnt 0) before the
  // arrival counter moves, and the merging workgroup loads only after it has
  // seen the last arrival.
  float* part_o = a.part_o + (unit * splits + split) * (int64_t)(G * D);
  float* part_l = a.part_lse + (unit * splits + split) * (int64_t)G;
  for (int x = threadIdx.x; x < G * D; x += kDecThreads) {
    const int g = x / D;
    const int e = x - g * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, mm[w][g]);
    float L = 0.f, O = 0.f;
    if (M > -INFINITY) {
      // branch-free, so the LDS reads of all waves go out together: a wave
      // without tokens has mm = -inf (weight exp2(-inf) = 0) and o = 0
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) {
        const float cw = exp2_fast(mm[w][g] - M);
        L = fmaf(cw, ml[w][g], L);
        const auto& mw = lds.wv[w].mo;
        O = fmaf(cw, (mw[0][g][e] + mw[1][g][e]) + (mw[2][g][e] + mw[3][g][e]), O);
      }
    }
    __hip_atomic_store(&part_o[x], L > 0.f ? O / L : 0.f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (e == 0)
      __hip_atomic_store(&part_l[g], L > 0.f ? (M + log2_fast(L)) * kLn2 : -INFINITY, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- the last workgroup of this (sequence, KV head) merges the splits ----
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's partial stores are done
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = atomicAdd(&a.counters[unit], 1);
    last_s = prev == splits - 1;
  }
  __syncthreads();
  if (!last_s) return;
  const float* po = a.part_o + unit * splits * (int64_t)(G * D);
  const float* pl = a.part_lse + unit * splits * (int64_t)G;
  // every output of this thread (kNx of them) and splits in chunks of
  // kMergeChunk: all loads of a chunk are issued before any is used, then the
  // chunk is folded into a running (M, L, O) per output. Up to 4 or 8 splits
  // take one chunk of 4 or 8 (no clamped duplicate loads); with one chunk
  // either way the fold is the same arithmetic.
  constexpr int kNx = (G * D + kDecThreads - 1) / kDecThreads;
  float M[kNx], L[kNx], O[kNx];
#pragma unroll
  for (int xi = 0; xi < kNx; ++xi) { M[xi] = -INFINITY; L[xi] = 0.f; O[xi] = 0.f; }
  auto merge = [&](auto chunk) {
    constexpr int kMergeChunk = decltype(chunk)::value;
    for (int s0 = 0; s0 < splits; s0 += kMergeChunk) {
      float ls[kNx][kMergeChunk], ov[kNx][kMergeChunk];
#pragma unroll
      for (int xi = 0; xi < kNx; ++xi) {
        const int x = threadIdx.x + kDecThreads * xi;
        const int xc = x < G * D ? x : 0;
        const int g = xc / D;
#pragma unroll
        for (int i = 0; i < kMergeChunk; ++i) {
          const int sp = s0 + i < splits ? s0 + i : splits - 1;
          ls[xi][i] = __hip_atomic_load(&pl[sp * G + g], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ov[xi][i] = __hip_atomic_load(&po[(int64_t)sp * G * D + xc], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
#pragma unroll
      for (int xi = 0; xi < kNx; ++xi) {
        float Mc = M[xi];
#pragma unroll
        for (int i = 0; i < kMergeChunk; ++i)
          if (s0 + i < splits) Mc = fmaxf(Mc, ls[xi][i]);
        if (Mc > -INFINITY) {
          const float r = exp2_fast((M[xi] - Mc) * kLog2e);  // M = -inf -> 0
          L[xi] *= r;
          O[xi] *= r;
#pragma unroll
          for (int i = 0; i < kMergeChunk; ++i) {
            if (s0 + i < splits && ls[xi][i] > -INFINITY) {
              const float cw = exp2_fast((ls[xi][i] - Mc) * kLog2e);
              L[xi] += cw;
              O[xi] = fmaf(cw, ov[xi][i], O[xi]);
            }
          }
          M[xi] = Mc;
        }
      }
    }
  };
  if (splits <= 4)
    merge(std::integral_constant<int, 4>{});
  else if (splits <= 8)
    merge(std::integral_constant<int, 8>{});
  else
    merge(std::integral_constant<int, 16>{});
  T* out = reinterpret_cast<T*>(a.out) + ((int64_t)b * Hq + (int64_t)h * G) * D;
#pragma unroll
  for (int xi = 0; xi < kNx; ++xi) {
    const int x = threadIdx.x + kDecThreads * xi;
    if (x >= G * D) continue;
    const int g = x / D;
    out[x] = Elem<T>::from_f32(L[xi] > 0.f ? O[xi] / L[xi] : 0.f);
    if (a.lse && x % D == 0)
      a.lse[(int64_t)b * Hq + (int64_t)h * G + g] = L[xi] > 0.f ? M[xi] + log2_fast(L[xi]) * kLn2 : -INFINITY;
  }
  if (threadIdx.x == 0) atomicExch(&a.counters[unit], 0);
}

}  // namespace locks

// Device code of the share-average combine and top-(k-2) selection, [Locks]
// §2, §4. See select.hip for the method.
#pragma once

#include "common.h"
#include "kernels.h"

namespace locks {

constexpr int kSelBins = 1024;
constexpr int kSelDigit = 10;

namespace sel_detail {

// ---- wave-wide helpers on DPP (no LDS permutes) ----
// inclusive prefix sum over the 64 lanes: row_shr 1/2/4/8 inside each row of
// 16 lanes, then row_bcast 15 / 31 carry the row totals forward
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// max / min of a uint32 over the wave (uniform result)
template <bool kMax>
__device__ __forceinline__ uint32_t wave_minmax_u32(uint32_t v) {
  auto op = [](uint32_t x, uint32_t y) { return kMax ? (x > y ? x : y) : (x < y ? x : y); };
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppXor1, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppXor2, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppHalfMirror, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kDppMirror, 0xf, 0xf, false));
  const uint32_t r0 = __builtin_amdgcn_readlane((int)v, 0), r1 = __builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane((int)v, 32), r3 = __builtin_amdgcn_readlane((int)v, 48);
  return op(op(r0, r1), op(r2, r3));
}

// float max / sum over the wave (uniform result)
__device__ __forceinline__ float wave_max(float v) {
  v = group_max<16>(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum<16>(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// exclusive scan over a block of NW waves; `tot` receives the block total. One
// barrier: the caller puts another barrier between two uses of the same wsum.
template <int NW>
__device__ __forceinline__ int block_excl_scan(int v, int* wsum, int& tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int inc = wave_incl_scan(v);
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  int before = 0;
  tot = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int x = wsum[w];
    before += w < wave ? x : 0;
    tot += x;
  }
  return before + inc - v;
}

}  // namespace sel_detail

template <int NT, int KEYS, int BITS = 1>
struct alignas(16) SelectLds {
  uint32_t keys[KEYS];
  uint32_t bits[BITS];  // chosen-page bitmap of the register path (BITS words)
  uint32_t hist[2][kSelBins];
  int pick_s[3];
  float red_m[NT / 64][8];
  float red_s[NT / 64][8];
  uint32_t redu[NT / 64][2];
  int wsum[NT / 64];
};

// Combine and selection of the unit (b, h) by a workgroup of NT threads for
// GQ query heads per KV head (a compile-time count: the per-head loops are
// straight-line code). NPT > 0 keeps pages tid, tid + NT, ... (NPT of them,
// max_pages <= NT * NPT) in registers; NPT = 0 loops over global memory.
// KEYS: page keys kept in LDS (longer contexts keep them in the sigma buffer).
template <int NT, int NPT, int KEYS, int GQ, int BITS>
__device__ __forceinline__ void select_unit(const SelectArgs& a, int b, int h, SelectLds<NT, KEYS, BITS>& L) {
  using namespace sel_detail;
  constexpr int kSelThreads = NT;
  constexpr int kSelWaves = NT / 64;
  constexpr int kSelLdsKeys = KEYS;
  auto& keys_lds = L.keys;
  auto& hist = L.hist;
  auto& red_m = L.red_m;
  auto& red_s = L.red_s;
  auto& redu = L.redu;
  auto& wsum = L.wsum;
  auto& pick_s = L.pick_s;


  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int P = a.P, k = a.k;
  constexpr int G = GQ;
  const float* srow = a.scores + ((int64_t)b * a.Hkv * G + (int64_t)h * G) * a.max_pages;
  // the register path loads its scores before the length is known (pages up
  // to max_pages are addressable), so both loads are in flight together
  // (register page i of thread t is page 4 (t + NT (i / 4)) + i % 4: runs of
  // four pages, read with 16-byte loads when rows are 16-byte aligned)
  constexpr int kRegs = NPT > 0 ? NPT : 1;
  static_assert(NPT % 4 == 0, "register pages come in runs of four");
  auto page_of = [&](int i) { return 4 * (tid + kSelThreads * (i >> 2)) + (i & 3); };
  float sc[kRegs][GQ];
  if constexpr (NPT > 0) {
    const bool vec = (a.max_pages & 3) == 0 && (reinterpret_cast<uintptr_t>(a.scores) & 15) == 0;
#pragma unroll
    for (int i4 = 0; i4 < NPT / 4; ++i4) {
      const int j0 = page_of(4 * i4);
#pragma unroll
      for (int g = 0; g < GQ; ++g) {
        if (g < G && vec && j0 < a.max_pages) {
          const f32x4_t v = *reinterpret_cast<const f32x4_t*>(srow + (int64_t)g * a.max_pages + j0);
#pragma unroll
          for (int e = 0; e < 4; ++e) sc[4 * i4 + e][g] = v[e];
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sc[4 * i4 + e][g] = (g < G && j0 + e < a.max_pages) ? srow[(int64_t)g * a.max_pages + j0 + e] : 0.f;
        }
      }
    }
  }
  const int T = __builtin_amdgcn_readfirstlane(clamp_len(a.seq_lens[b], a.max_pages, P));
  const int J = (T + P - 1) / P;
  const int Jc = T / P;
  int32_t* sel_row = a.selected + ((int64_t)b * a.Hkv + h) * k;
  auto put = [&](int pos, int j) { sel_row[pos] = j; };

  if (J <= k) {
    for (int t = tid; t < k; t += kSelThreads) put(t, t < J ? t : -1);
    return;
  }

  float* sig_row = a.sigma + ((int64_t)b * a.Hkv + h) * a.max_pages;
  const bool keys_in_lds = Jc <= kSelLdsKeys;
  uint32_t* keys = keys_in_lds ? keys_lds : reinterpret_cast<uint32_t*>(sig_row);
  auto is_cand = [&](int j) { return (j >= 1) & (j < Jc) & (j != J - 1); };
  for (int x = tid; x < kSelBins; x += kSelThreads) hist[0][x] = 0;
  if constexpr (NPT > 4) {
    static_assert(BITS * 32 >= NT * NPT, "bitmap covers the register pages");
    for (int x = tid; x < BITS; x += kSelThreads) L.bits[x] = 0;
  }

  // ---- per-head normaliser log Z_g ----
  float mx[GQ];
#pragma unroll
  for (int g = 0; g < GQ; ++g) mx[g] = -INFINITY;
  float lz[GQ], inv_z[GQ];  // log Z_g, and the factor that turns a kept exponential into exp(s - log Z_g)
  float ex[kRegs][GQ];      // register path: exp(s_g(j) - the wave's max_g), kept for sigma
  if constexpr (NPT > 0) {
    // One barrier: every wave sums 2^(s - m_w) against its own maximum m_w
    // (DPP inside the wave) and publishes (m_w, sum_w); then lane w of every
    // row of 16 takes wave w's pair, and M = max m_w,
    // Z = sum_w sum_w 2^(m_w - M) come from DPP over the row.
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int j = page_of(i);
#pragma unroll
      for (int g = 0; g < GQ; ++g) {
        if (!(g < G && j < Jc)) sc[i][g] = -INFINITY;
        mx[g] = fmaxf(mx[g], sc[i][g]);
      }
    }
    float wm[GQ], sm[GQ];
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      wm[g] = g < G ? wave_max(mx[g]) : -INFINITY;
      sm[g] = 0.f;
    }
#pragma unroll
    for (int i = 0; i < NPT; ++i)
#pragma unroll
      for (int g = 0; g < GQ; ++g) {
        ex[i][g] = 0.f;
        if (g < G && wm[g] > -INFINITY) {
          ex[i][g] = exp2_fast((sc[i][g] - wm[g]) * kLog2e);
          sm[g] += ex[i][g];
        }
      }
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      if (g < G) {
        const float r = wave_sum(sm[g]);
        if (lane == 0) {
          red_m[wave][g] = wm[g];
          red_s[wave][g] = r;
        }
      }
    }
    __syncthreads();
    static_assert(kSelWaves <= 16, "one row of lanes per wave pair");
    // straight-line code (every lane loads a row, rows past the waves are
    // masked), so the heads' dependent DPP chains interleave
    const int wv = lane & 15;
    const bool wv_ok = wv < kSelWaves;
    const int wvc = wv_ok ? wv : 0;
    float m_w[GQ], e_w[GQ];
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      const float m0 = red_m[wvc][g], s0 = red_s[wvc][g];
      m_w[g] = wv_ok ? m0 : -INFINITY;
      e_w[g] = wv_ok ? s0 : 0.f;
    }
#pragma unroll
    for (int g = 0; g < GQ; ++g) mx[g] = group_max<16>(m_w[g]);
#pragma unroll
    for (int g = 0; g < GQ; ++g) e_w[g] = m_w[g] > -INFINITY ? e_w[g] * exp2_fast((m_w[g] - mx[g]) * kLog2e) : 0.f;
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      const float l2z = log2_fast(group_sum<16>(e_w[g]));
      const bool live = mx[g] > -INFINITY;
      lz[g] = live ? mx[g] + l2z * kLn2 : -INFINITY;
      // exp(m_w,g - M) / Z as one exponential, 2^((m_w,g - M) log2 e - log2 Z)
      inv_z[g] = live && wm[g] > -INFINITY ? exp2_fast((wm[g] - mx[g]) * kLog2e - l2z) : 0.f;
    }
  } else {
    // block max, then block sum of 2^(s - max); each reduction is DPP
    // inside the waves, one LDS exchange and one barrier, with every thread
    // combining the wave results itself
    for (int j = tid; j < Jc; j += kSelThreads)
#pragma unroll
      for (int g = 0; g < GQ; ++g)
        if (g < G) mx[g] = fmaxf(mx[g], srow[(int64_t)g * a.max_pages + j]);
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      if (g < G) {
        const float r = wave_max(mx[g]);
        if (lane == 0) red_m[wave][g] = r;
      }
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      if (g < G) {
        float r = red_m[0][g];
#pragma unroll
        for (int w = 1; w < kSelWaves; ++w) r = fmaxf(r, red_m[w][g]);
        mx[g] = r;
      }
    }
    float sm[GQ];
#pragma unroll
    for (int g = 0; g < GQ; ++g) sm[g] = 0.f;
    for (int j = tid; j < Jc; j += kSelThreads)
#pragma unroll
      for (int g = 0; g < GQ; ++g)
        if (g < G && mx[g] > -INFINITY) sm[g] += exp2_fast((srow[(int64_t)g * a.max_pages + j] - mx[g]) * kLog2e);
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      if (g < G) {
        const float r = wave_sum(sm[g]);
        if (lane == 0) red_s[wave][g] = r;
      }
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      lz[g] = -INFINITY;
      inv_z[g] = 0.f;
      if (g < G && mx[g] > -INFINITY) {
        float r = red_s[0][g];
#pragma unroll
        for (int w = 1; w < kSelWaves; ++w) r += red_s[w][g];
        lz[g] = mx[g] + log2_fast(r) * kLn2;
      }
    }
  }

  // ---- sigma_j, its sortable key, and the spread of candidate keys ----
  const float log2G = log2_fast((float)G);
  uint32_t kmax = 0u, kmin = 0xffffffffu;
  auto sigma_key = [&](int j, const float* sv) {
    float tg[GQ];
    float m = -INFINITY;
#pragma unroll
    for (int g = 0; g < GQ; ++g) {
      tg[g] = -INFINITY;
      if (g < G && lz[g] > -INFINITY) {
        tg[g] = (sv[g] - lz[g]) * kLog2e;
        m = fmaxf(m, tg[g]);
      }
    }
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < GQ; ++g)
      if (g < G && m > -INFINITY) s += exp2_fast(tg[g] - m);
    const float sigma = m > -INFINITY ? (m + log2_fast(s) - log2G) * kLn2 : -INFINITY;
    const uint32_t key = float_key(sigma);
    if (keys_in_lds) {
      keys[j] = key;
      if (a.want_sigma) sig_row[j] = sigma;
    } else {
      sig_row[j] = __uint_as_float(key);  // global scratch holds the key; rewritten below
    }
    if (is_cand(j)) {
      kmax = key > kmax ? key : kmax;
      kmin = key < kmin ? key : kmin;
    }
  };
  // register path: sigma_j = log(sum_g e_g(j) f_g) - log G from the kept
  // exponentials e_g(j) = exp(s_g(j) - m_w,g) and f_g = exp(m_w,g - log Z_g)
  // (one logarithm per page); a page whose sum falls below 2^-60 (terms near
  // or below the fp32 range) takes the per-page-max form above on its scores
  // read again. The key stays in a register.
  uint32_t kreg[kRegs];
  if constexpr (NPT > 0) {
    float sg[kRegs], vs[kRegs];
    bool low = false;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      float v = 0.f;
#pragma unroll
      for (int g = 0; g < GQ; ++g) v = fmaf(ex[i][g], inv_z[g], v);
      vs[i] = v;
      sg[i] = (log2_fast(v) - log2G) * kLn2;
      low = low || (page_of(i) < Jc && !(v >= 0x1p-60f));
    }
    if (__ballot(low) != 0) {  // rare: some sum below 2^-60 in this wave
#pragma unroll
      for (int i = 0; i < NPT; ++i) {
        const int j = page_of(i);
        if (j < Jc && !(vs[i] >= 0x1p-60f)) {
          float tg[GQ];
          float m = -INFINITY;
#pragma unroll
          for (int g = 0; g < GQ; ++g) {
            tg[g] = -INFINITY;
            if (lz[g] > -INFINITY) {
              tg[g] = (srow[(int64_t)g * a.max_pages + j] - lz[g]) * kLog2e;  // the scores read again
              m = fmaxf(m, tg[g]);
            }
          }
          float su = 0.f;
#pragma unroll
          for (int g = 0; g < GQ; ++g)
            if (m > -INFINITY) su += exp2_fast(tg[g] - m);
          sg[i] = m > -INFINITY ? (m + log2_fast(su) - log2G) * kLn2 : -INFINITY;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int j = page_of(i);
      const uint32_t key = float_key(sg[i]);
      kreg[i] = j < Jc ? key : 0u;
      if (a.want_sigma && j < Jc) sig_row[j] = sg[i];
      const bool cand = is_cand(j);
      kmax = cand && key > kmax ? key : kmax;
      kmin = cand && key < kmin ? key : kmin;
    }
  } else {
    for (int j = tid; j < Jc; j += kSelThreads) {
      float sv[GQ];
#pragma unroll
      for (int g = 0; g < GQ; ++g) sv[g] = g < G ? srow[(int64_t)g * a.max_pages + j] : 0.f;
      sigma_key(j, sv);
    }
  }
  kmax = wave_minmax_u32<true>(kmax);
  kmin = wave_minmax_u32<false>(kmin);
  if (lane == 0) { redu[wave][0] = kmax; redu[wave][1] = kmin; }
  __syncthreads();  // also publishes keys[] and the cleared hist[0]
  kmax = redu[0][0];
  kmin = redu[0][1];
#pragma unroll
  for (int w = 1; w < kSelWaves; ++w) {
    kmax = redu[w][0] > kmax ? redu[w][0] : kmax;
    kmin = redu[w][1] < kmin ? redu[w][1] : kmin;
  }
  // uniform (every lane read the same words): the radix bounds live in SGPRs
  kmax = __builtin_amdgcn_readfirstlane(kmax);
  kmin = __builtin_amdgcn_readfirstlane(kmin);

  // ---- radix select of the K best candidates ----
  int ncand = Jc - 1 - ((J - 1 >= 1 && J - 1 < Jc) ? 1 : 0);
  if (ncand < 0) ncand = 0;
  const int K = min(k - 2, ncand);
  const int idb = a.idbits;
  const uint64_t idmask = ((uint64_t)1 << idb) - 1;
  auto key64 = [&](int j) -> uint64_t { return ((uint64_t)keys[j] << idb) | (idmask - (uint64_t)j); };

  // highest bit in which two candidate keys can differ: within sigma's key
  // when the keys differ, else within the page id
  int hi = kmax != kmin ? idb + 32 - __builtin_clz(kmax ^ kmin) : idb;
  // common bits above `hi` (taken from the largest key)
  uint64_t prefix = (((uint64_t)kmax << idb) >> hi) << hi;
  int kr = K;
  const bool take_all = K == 0 || K >= ncand;  // nothing to rank: none wanted, or every candidate fits
  int cur = 0;
  while (!take_all && hi > 0) {
    const int lo = hi > kSelDigit ? hi - kSelDigit : 0;
    const uint32_t dmask = (1u << (hi - lo)) - 1u;
    uint32_t* hc = hist[cur];
    if constexpr (NPT > 0) {
#pragma unroll
      for (int i = 0; i < NPT; ++i) {
        const int j = page_of(i);
        if (j >= Jc || !is_cand(j)) continue;
        const uint64_t kv = ((uint64_t)kreg[i] << idb) | (idmask - (uint64_t)j);
        if ((kv >> hi) != (prefix >> hi)) continue;
        atomicAdd(&hc[(uint32_t)(kv >> lo) & dmask], 1u);
      }
    } else {
      for (int j = tid; j < Jc; j += kSelThreads) {
        if (!is_cand(j)) continue;
        const uint64_t kv = key64(j);
        if ((kv >> hi) != (prefix >> hi)) continue;
        atomicAdd(&hc[(uint32_t)(kv >> lo) & dmask], 1u);
      }
    }
    __syncthreads();
    // bins in descending order, kPer per thread; the next pass's buffer is
    // cleared meanwhile
    static_assert(kSelBins % kSelThreads == 0, "every thread scans the same number of bins");
    constexpr int kPer = kSelBins / kSelThreads;
    const int top = kSelBins - 1 - tid * kPer;
    int local = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) local += (int)hc[top - i];
#pragma unroll
    for (int i = 0; i < kPer; ++i) hist[cur ^ 1][top - i] = 0;
    int tot;
    const int before = block_excl_scan<kSelWaves>(local, wsum, tot);
    if (before < kr && before + local >= kr) {
      int acc = before;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int c = (int)hc[top - i];
        if (acc + c >= kr) {
          pick_s[0] = top - i;
          pick_s[1] = kr - acc;  // still needed from this bin
          pick_s[2] = c;
          break;
        }
        acc += c;
      }
    }
    __syncthreads();
    const int dsel = __builtin_amdgcn_readfirstlane(pick_s[0]);
    const int need = __builtin_amdgcn_readfirstlane(pick_s[1]);
    const int cnt = __builtin_amdgcn_readfirstlane(pick_s[2]);
    prefix |= (uint64_t)dsel << lo;
    hi = lo;
    kr = need;
    cur ^= 1;
    if (cnt == need) break;  // the whole bin is taken
  }

  // ---- ascending output: sink, current and the chosen candidates ----
  auto chosen = [&](int j) -> bool {
    if (j == 0 || j == J - 1) return true;
    if (!is_cand(j) || K == 0) return false;
    if (take_all) return true;
    return (key64(j) >> hi) >= (prefix >> hi);
  };
  static_assert(NPT == 0 || NPT == 4 || NPT == 8, "register pages: 4 or 8 per thread");
  if constexpr (NPT == 4) {
    // the thread's register pages are 4 tid .. 4 tid + 3: their chosen flags,
    // a block scan of the counts, and the writes at ascending positions
    // (straight-line flags: every term is evaluated, none behind a branch)
    bool cf[4];
    int cnt = 0;
    const uint64_t pfx = prefix >> hi;
    const bool rank_any = K != 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = page_of(i);
      const uint64_t kv = ((uint64_t)kreg[i] << idb) | (idmask - (uint64_t)j);
      const bool ranked = take_all | ((kv >> hi) >= pfx);
      const bool c = (j < J) & ((j == 0) | (j == J - 1) | (is_cand(j) & rank_any & ranked));
      cf[i] = c;
      cnt += c ? 1 : 0;
    }
    int total;
    int pos = block_excl_scan<kSelWaves>(cnt, wsum, total);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (cf[i]) {
        if (pos < k) put(pos, page_of(i));
        ++pos;
      }
    }
    for (int t = total + tid; t < k; t += kSelThreads) put(t, -1);
    return;
  }
  if constexpr (NPT > 0) {
    // chosen pages set bits of an LDS bitmap; thread t then takes bits
    // NPT t .. NPT t + NPT - 1 (one word holds them) and writes them at the
    // count of bits before them (ascending ids)
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int j = page_of(i);
      if (j >= J) continue;
      bool c = j == 0 || j == J - 1;
      if (!c && is_cand(j) && K != 0)
        c = take_all || ((((uint64_t)kreg[i] << idb) | (idmask - (uint64_t)j)) >> hi) >= (prefix >> hi);
      if (c) atomicOr(&L.bits[j >> 5], 1u << (j & 31));
    }
    __syncthreads();
    static_assert(32 % NPT == 0, "a thread's bits sit in one word");
    // every wave counts the bits of all words (lane l takes words kWpl l ..)
    // and prefix-sums them, so no block scan is needed
    constexpr int kWpl = (BITS + 63) / 64;
    int wex[kWpl];  // bits before each of the lane's words, within the lane
    int c = 0;
#pragma unroll
    for (int u = 0; u < kWpl; ++u) {
      const int x = lane * kWpl + u;
      wex[u] = c;
      c += x < BITS ? __builtin_popcount(L.bits[x]) : 0;
    }
    const int inc = wave_incl_scan(c);
    const int total = __builtin_amdgcn_readlane(inc, 63);
    const int b0 = NPT * tid;
    const int wi = b0 >> 5;  // the word of this thread's bits, held by lane wi / kWpl
    int wpre = 0;
#pragma unroll
    for (int u = 0; u < kWpl; ++u) {
      const int v = __shfl(inc - c + wex[u], wi / kWpl, 64);
      wpre = wi % kWpl == u ? v : wpre;
    }
    const uint32_t word = L.bits[wi];
    const int off = b0 & 31;
    const uint32_t mine = (word >> off) & ((1u << NPT) - 1u);
    int pos = wpre + __builtin_popcount(word & ((1u << off) - 1u));
#pragma unroll
    for (int e = 0; e < NPT; ++e) {
      if ((mine >> e) & 1u) {
        if (pos < k) put(pos, b0 + e);
        ++pos;
      }
    }
    for (int t = total + tid; t < k; t += kSelThreads) put(t, -1);
    return;
  }
  const int ppt = (J + kSelThreads - 1) / kSelThreads;
  const int j0 = tid * ppt;
  const int j1 = min(J, j0 + ppt);
  int cnt = 0;
  for (int j = j0; j < j1; ++j) cnt += chosen(j) ? 1 : 0;
  int total;
  int pos = block_excl_scan<kSelWaves>(cnt, wsum, total);
  for (int j = j0; j < j1; ++j) {
    if (chosen(j)) {
      if (pos < k) put(pos, j);
      ++pos;
    }
  }
  for (int t = total + tid; t < k; t += kSelThreads) put(t, -1);

  // when the keys lived in the global scratch, leave sigma there as documented
  if (!keys_in_lds && a.want_sigma) {
    __syncthreads();
    for (int j = tid; j < Jc; j += kSelThreads) {
      const uint32_t key = keys[j];
      const uint32_t u = (key & 0x80000000u) ? (key & 0x7fffffffu) : ~key;
      sig_row[j] = key == 0u ? __uint_as_float(0x7fc00000u) : __uint_as_float(u);
    }
  }
}

}  // namespace locks

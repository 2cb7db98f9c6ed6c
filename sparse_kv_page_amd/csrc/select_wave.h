// Share-average combine and top-(k-2) selection of one (sequence, KV head) by
// a single wave, [Locks] §2, §4, run by the page scorer's last workgroup of
// that unit once every page score of the unit is written.
//
// The arithmetic is the workgroup selector's (select_unit.h), operation for
// operation, so both give the same bits: the 512-thread selector keeps pages
// t, t + 512, t + 1024, t + 1536 in thread t, i.e. in lane t % 64 of wave
// t / 64. Here lane l keeps pages l + 64 i (i = w + 8 i'), so it holds the
// pages of "virtual thread" l + 64 w of every wave w of that selector: the
// per-head sums of 2^(s - max) are formed per virtual thread in the same
// order, reduced with the same wave reduction per virtual wave, and the eight
// wave totals added in wave order. sigma and its key follow the same
// expressions. The selection itself is exact on those keys: the K-th largest
// candidate key is found bit by bit (wave-wide counts from ballots), every
// key above it is taken, and ties at it go to the lower page ids.
#pragma once

#include "common.h"
#include "kernels.h"
#include "select_unit.h"

namespace locks {

// pages per lane of the one-wave selection for GQ query heads per KV head:
// its scores stay in registers (128 per lane), so it serves units of at most
// 64 * kSelWaveNpl<GQ> pages
template <int GQ>
constexpr int kSelWaveNpl = 128 / GQ;

// Scores of the unit were written by other workgroups with device-scope
// stores before their arrival was counted; they are read with device-scope
// loads.
template <int GQ>
__device__ __forceinline__ void select_wave(const float* scores, const int32_t* seq_lens, int32_t* selected,
                                            int b, int h, int Hkv, int P, int k, int max_pages) {
  using namespace sel_detail;
  constexpr int G = GQ;
  constexpr int NPL = kSelWaveNpl<GQ>;
  constexpr int kVWaves = 8;   // waves of the 512-thread selector
  constexpr int kVPages = 4;   // pages per thread of that selector
  static_assert(NPL <= kVWaves * kVPages && NPL % kVWaves == 0, "lane pages map onto the selector's threads");

  const int lane = threadIdx.x & 63;
  const float* srow = scores + ((int64_t)b * Hkv * G + (int64_t)h * G) * max_pages;
  const int T = __builtin_amdgcn_readfirstlane(clamp_len(seq_lens[b], max_pages, P));
  const int J = (T + P - 1) / P;
  const int Jc = T / P;
  int32_t* sel_row = selected + ((int64_t)b * Hkv + h) * k;
  if (J <= k) {
    for (int t = lane; t < k; t += 64) sel_row[t] = t < J ? t : -1;
    return;
  }
  auto is_cand = [&](int j) { return j >= 1 && j < Jc && j != J - 1; };

  float sc[NPL][G];
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int j = lane + 64 * i;
#pragma unroll
    for (int g = 0; g < G; ++g)
      sc[i][g] = j < Jc ? __hip_atomic_load(srow + (int64_t)g * max_pages + j, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT)
                        : -INFINITY;
  }

  // ---- per-head normaliser log Z_g ----
  float lz[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < NPL; ++i) m = fmaxf(m, sc[i][g]);
    const float mx = wave_max(m);
    lz[g] = -INFINITY;
    if (mx > -INFINITY) {
      float r = 0.f;
#pragma unroll
      for (int w = 0; w < kVWaves; ++w) {
        float part = 0.f;
#pragma unroll
        for (int ip = 0; ip < kVPages; ++ip) {
          const int i = w + kVWaves * ip;
          if (i < NPL) part += exp2_fast((sc[i][g] - mx) * kLog2e);
        }
        const float tot = wave_sum(part);
        r = w == 0 ? tot : r + tot;
      }
      lz[g] = mx + log2_fast(r) * kLn2;
    }
  }

  // ---- sigma_j and its sortable key (0 for pages that are not candidates) ----
  const float log2G = log2_fast((float)G);
  uint32_t key[NPL];
  uint32_t kmax = 0u, kmin = 0xffffffffu;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int j = lane + 64 * i;
    float tg[G];
    float m = -INFINITY;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      tg[g] = -INFINITY;
      if (lz[g] > -INFINITY) {
        tg[g] = (sc[i][g] - lz[g]) * kLog2e;
        m = fmaxf(m, tg[g]);
      }
    }
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g)
      if (m > -INFINITY) s += exp2_fast(tg[g] - m);
    const float sigma = m > -INFINITY ? (m + log2_fast(s) - log2G) * kLn2 : -INFINITY;
    const bool c = is_cand(j);
    key[i] = c ? float_key(sigma) : 0u;
    if (c) {
      kmax = key[i] > kmax ? key[i] : kmax;
      kmin = key[i] < kmin ? key[i] : kmin;
    }
  }
  kmax = wave_minmax_u32<true>(kmax);
  kmin = wave_minmax_u32<false>(kmin);

  int ncand = Jc - 1 - ((J - 1 >= 1 && J - 1 < Jc) ? 1 : 0);
  if (ncand < 0) ncand = 0;
  const int K = min(k - 2, ncand);
  const bool take_all = K >= ncand;

  // ---- v = the K-th largest candidate key, one bit at a time below the
  // bits every candidate shares; count(key >= v) >= K holds throughout ----
  auto count_ge = [&](uint32_t c) {
    int n = 0;
#pragma unroll
    for (int i = 0; i < NPL; ++i) n += __popcll(__ballot(key[i] >= c));
    return n;
  };
  uint32_t v = 0u;
  int n_gt = 0;
  if (!take_all && K > 0) {
    const int hb = kmax != kmin ? 31 - __builtin_clz(kmax ^ kmin) : -1;
    v = hb < 0 ? kmax : (hb == 31 ? 0u : (kmax >> (hb + 1)) << (hb + 1));
    for (int bit = hb; bit >= 0; --bit) {
      const uint32_t c = v | (1u << bit);
      if (count_ge(c) >= K) v = c;
    }
    // non-candidates hold 0 < v (every candidate key is at least float_key(-inf))
    n_gt = v == 0xffffffffu ? 0 : count_ge(v + 1u);
  }
  const int need_ties = K - n_gt;

  // ---- ascending output: sink, current and the chosen candidates ----
  const uint64_t below = (1ull << lane) - 1ull;
  int base = 0, tie_base = 0;
#pragma unroll
  for (int i = 0; i < NPL; ++i) {
    const int j = lane + 64 * i;
    const bool c = is_cand(j);
    const bool tie = !take_all && K > 0 && c && key[i] == v;
    const uint64_t tm = __ballot(tie);
    const int trank = tie_base + __popcll(tm & below);
    tie_base += __popcll(tm);
    bool ch = j == 0 || j == J - 1;
    if (c) ch = take_all || (K > 0 && (key[i] > v || (tie && trank < need_ties)));
    ch = ch && j < J;
    const uint64_t cm = __ballot(ch);
    const int pos = base + __popcll(cm & below);
    if (ch && pos < k) sel_row[pos] = j;
    base += __popcll(cm);
  }
  for (int t = base + lane; t < k; t += 64) sel_row[t] = -1;
}

}  // namespace locks

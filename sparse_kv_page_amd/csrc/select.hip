// (a3 + a4) Share-average combine and top-(k-2) page selection, [Locks] §2, §4.
//
// One workgroup per (sequence, KV head). From the per-head page scores s_g(j)
// of the Jc complete pages:
//   log Z_g  = log sum_j exp(s_g(j))
//   sigma_j  = log((1/G) sum_g exp(s_g(j) - log Z_g))   (log of the share average)
// Pages 0 (sink) and J-1 (current) are always kept; the other k-2 slots take
// the largest sigma among the remaining complete pages, ties to the lower
// page id. The ranking runs as a radix select over 64-bit keys
// (order-preserving image of sigma, then the complemented page id) with 8-bit
// digits and an LDS histogram, most significant digit first; it stops as soon
// as the bucket holding the k-2'th key is taken whole.
#include "common.h"
#include "kernels.h"

namespace locks {

constexpr int kSelThreads = 256;
constexpr int kSelMaxK = 1024;
constexpr int kSelLdsKeys = 16384;  // sigma keys kept in LDS up to this many pages

namespace {

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace

__global__ __launch_bounds__(kSelThreads) void select_kernel(SelectArgs a) {
  extern __shared__ uint32_t keys_lds[];
  __shared__ float red[kSelThreads / 64][8];
  __shared__ float logz_s[8];
  __shared__ float mx_s[8];
  __shared__ uint32_t hist[256];
  __shared__ int32_t list[kSelMaxK];
  __shared__ int list_n;
  __shared__ uint32_t dig_s;
  __shared__ int kr_s;
  __shared__ int done_s;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int P = a.P, G = a.G, k = a.k;
  const int T = clamp_len(a.seq_lens[b], a.max_pages, P);
  const int J = (T + P - 1) / P;
  const int Jc = T / P;
  int32_t* sel_row = a.selected + ((int64_t)b * a.Hkv + h) * k;

  if (J <= k) {
    for (int t = tid; t < k; t += kSelThreads) sel_row[t] = t < J ? t : -1;
    return;
  }

  const float* srow = a.scores + ((int64_t)b * a.Hkv * G + (int64_t)h * G) * a.max_pages;
  float* sig_row = a.sigma + ((int64_t)b * a.Hkv + h) * a.max_pages;
  const bool keys_in_lds = Jc <= kSelLdsKeys;
  uint32_t* keys = keys_in_lds ? keys_lds : reinterpret_cast<uint32_t*>(sig_row);

  // ---- per-head normaliser log Z_g ----
  float mx[8], sm[8];
#pragma unroll
  for (int g = 0; g < 8; ++g) { mx[g] = -INFINITY; sm[g] = 0.f; }
  for (int j = tid; j < Jc; j += kSelThreads)
#pragma unroll
    for (int g = 0; g < 8; ++g)
      if (g < G) mx[g] = fmaxf(mx[g], srow[(int64_t)g * a.max_pages + j]);
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    if (g < G) {
      float v = wave_max(mx[g]);
      if (lane == 0) red[wave][g] = v;
    }
  }
  __syncthreads();
  if (tid < G) {
    float v = red[0][tid];
    for (int w = 1; w < kSelThreads / 64; ++w) v = fmaxf(v, red[w][tid]);
    mx_s[tid] = v;
  }
  __syncthreads();
#pragma unroll
  for (int g = 0; g < 8; ++g) mx[g] = g < G ? mx_s[g] : -INFINITY;
  for (int j = tid; j < Jc; j += kSelThreads)
#pragma unroll
    for (int g = 0; g < 8; ++g)
      if (g < G && mx[g] > -INFINITY)
        sm[g] += exp2_fast((srow[(int64_t)g * a.max_pages + j] - mx[g]) * kLog2e);
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    if (g < G) {
      float v = wave_sum(sm[g]);
      if (lane == 0) red[wave][g] = v;
    }
  }
  __syncthreads();
  if (tid < G) {
    float v = 0.f;
    for (int w = 0; w < kSelThreads / 64; ++w) v += red[w][tid];
    logz_s[tid] = mx_s[tid] > -INFINITY ? mx_s[tid] + log2_fast(v) * kLn2 : -INFINITY;
  }
  __syncthreads();

  // ---- sigma_j = log of the share average, and its sortable key ----
  float lz[8];
#pragma unroll
  for (int g = 0; g < 8; ++g) lz[g] = g < G ? logz_s[g] : 0.f;
  const float log2G = log2_fast((float)G);
  for (int j = tid; j < Jc; j += kSelThreads) {
    float tg[8];
    float m = -INFINITY;
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      tg[g] = -INFINITY;
      if (g < G && lz[g] > -INFINITY) {
        tg[g] = (srow[(int64_t)g * a.max_pages + j] - lz[g]) * kLog2e;
        m = fmaxf(m, tg[g]);
      }
    }
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < 8; ++g)
      if (g < G && m > -INFINITY) s += exp2_fast(tg[g] - m);
    const float sigma = m > -INFINITY ? (m + log2_fast(s) - log2G) * kLn2 : -INFINITY;
    const uint32_t key = float_key(sigma);
    if (keys_in_lds) {
      keys[j] = key;
      sig_row[j] = sigma;
    } else {
      sig_row[j] = __uint_as_float(key);  // global scratch holds the key; rewritten below
    }
  }
  if (tid == 0) list_n = 0;
  __syncthreads();

  // ---- radix select of the top K candidates ----
  int ncand = Jc - 1 - ((J - 1 >= 1 && J - 1 < Jc) ? 1 : 0);
  if (ncand < 0) ncand = 0;
  const int K = min(k - 2, ncand);
  auto is_cand = [&](int j) { return j >= 1 && j < Jc && j != J - 1; };
  auto key64 = [&](int j) -> uint64_t {
    return ((uint64_t)keys[j] << 32) | (uint64_t)(0xffffffffu - (uint32_t)j);
  };

  uint64_t prefix = 0;
  int shift = 64;
  int kr = K;
  if (K > 0) {
    for (int pass = 0; pass < 8; ++pass) {
      shift -= 8;
      for (int x = tid; x < 256; x += kSelThreads) hist[x] = 0;
      __syncthreads();
      for (int j = tid; j < Jc; j += kSelThreads) {
        if (!is_cand(j)) continue;
        const uint64_t kv = key64(j);
        if (pass > 0 && (kv >> (shift + 8)) != (prefix >> (shift + 8))) continue;
        atomicAdd(&hist[(uint32_t)(kv >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (wave == 0) {
        const uint32_t c0 = hist[4 * lane + 0], c1 = hist[4 * lane + 1];
        const uint32_t c2 = hist[4 * lane + 2], c3 = hist[4 * lane + 3];
        const int cs = (int)(c0 + c1 + c2 + c3);
        int S = cs;  // inclusive suffix sum over lanes >= lane
        for (int o = 1; o < 64; o <<= 1) {
          const int v = __shfl_down(S, o, 64);
          if (lane + o < 64) S += v;
        }
        const uint64_t bal = __ballot(S >= kr);
        const int L = 63 - __builtin_clzll(bal);
        if (lane == L) {
          int above = S - cs;
          int dsel, cnt;
          if (above + (int)c3 >= kr) {
            dsel = 4 * lane + 3; cnt = (int)c3;
          } else if (above + (int)(c3 + c2) >= kr) {
            above += (int)c3; dsel = 4 * lane + 2; cnt = (int)c2;
          } else if (above + (int)(c3 + c2 + c1) >= kr) {
            above += (int)(c3 + c2); dsel = 4 * lane + 1; cnt = (int)c1;
          } else {
            above += (int)(c3 + c2 + c1); dsel = 4 * lane; cnt = (int)c0;
          }
          dig_s = (uint32_t)dsel;
          kr_s = kr - above;
          done_s = (cnt == kr - above) ? 1 : 0;
        }
      }
      __syncthreads();
      prefix |= (uint64_t)dig_s << shift;
      kr = kr_s;
      const int done = done_s;
      __syncthreads();
      if (done) break;
    }
  }

  // ---- gather the chosen ids, then place them in ascending order ----
  for (int j = tid; j < Jc; j += kSelThreads) {
    if (K > 0 && is_cand(j) && (key64(j) >> shift) >= (prefix >> shift)) {
      const int pos = atomicAdd(&list_n, 1);
      if (pos < kSelMaxK) list[pos] = j;
    }
  }
  __syncthreads();
  if (tid == 0) {
    const int n0 = list_n;
    list[n0] = 0;
    list[n0 + 1] = J - 1;
    list_n = n0 + 2;
  }
  __syncthreads();
  const int nl = list_n;
  for (int t = tid; t < nl; t += kSelThreads) {
    const int v = list[t];
    int rank = 0;
    for (int x = 0; x < nl; ++x) rank += list[x] < v ? 1 : 0;
    if (rank < k) sel_row[rank] = v;
  }
  for (int t = nl + tid; t < k; t += kSelThreads) sel_row[t] = -1;

  // when the keys lived in the global scratch, leave sigma there as documented
  if (!keys_in_lds) {
    __syncthreads();
    for (int j = tid; j < Jc; j += kSelThreads) {
      const uint32_t key = keys[j];
      const uint32_t u = (key & 0x80000000u) ? (key & 0x7fffffffu) : ~key;
      sig_row[j] = key == 0u ? __uint_as_float(0x7fc00000u) : __uint_as_float(u);
    }
  }
}

hipError_t launch_select(const SelectArgs& a, int batch, hipStream_t stream) {
  const int lds_keys = a.max_pages < kSelLdsKeys ? a.max_pages : kSelLdsKeys;
  dim3 grid(a.Hkv, batch);
  hipLaunchKernelGGL(select_kernel, grid, dim3(kSelThreads), (size_t)lds_keys * 4, stream, a);
  return hipGetLastError();
}

}  // namespace locks

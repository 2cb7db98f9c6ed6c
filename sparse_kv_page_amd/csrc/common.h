// Device helpers shared by the Locks kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace locks {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;

typedef uint16_t bf16_t;  // bfloat16 storage bits

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

// float -> bfloat16 bits, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  // round to nearest even; a NaN keeps its top bits and becomes quiet. Both
  // results are formed and one selected, so no branch is generated.
  const uint32_t u = __float_as_uint(f);
  const uint32_t rne = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  const uint32_t nan = (u >> 16) | 0x40u;
  return (bf16_t)((u & 0x7fffffffu) > 0x7f800000u ? nan : rne);
}

// Storage element helpers: T is bf16_t or float.
template <typename T> struct Elem;
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ bf16_t from_f32(float f) { return f32_to_bf16(f); }
};
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ float from_f32(float f) { return f; }
};

// Raw hardware 2^x and log2(x) (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// Make this wave's LDS writes visible to its own later LDS reads and stop the
// compiler from moving memory accesses across the point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, kWave); }

// ---- cross-lane helpers (DPP inside a 16-lane row, LDS permute across rows) ----
// DPP controls: quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror, row_mirror.
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// All-reduce (max or sum) over aligned groups of N lanes, N in {1,2,4,8,16,32,64}.
// Every lane of a group ends with the group's result.
template <int N>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (N >= 2) v = fmaxf(v, dpp_f<kDppXor1>(v));
  if constexpr (N >= 4) v = fmaxf(v, dpp_f<kDppXor2>(v));
  if constexpr (N >= 8) v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  if constexpr (N >= 16) v = fmaxf(v, dpp_f<kDppMirror>(v));
  if constexpr (N >= 32) v = fmaxf(v, __shfl_xor(v, 16, kWave));
  if constexpr (N >= 64) v = fmaxf(v, __shfl_xor(v, 32, kWave));
  return v;
}
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp_f<kDppXor1>(v);
  if constexpr (N >= 4) v += dpp_f<kDppXor2>(v);
  if constexpr (N >= 8) v += dpp_f<kDppHalfMirror>(v);
  if constexpr (N >= 16) v += dpp_f<kDppMirror>(v);
  if constexpr (N >= 32) v += __shfl_xor(v, 16, kWave);
  if constexpr (N >= 64) v += __shfl_xor(v, 32, kWave);
  return v;
}

// Streaming (non-temporal) loads: data read once per step bypasses cache reuse.
__device__ __forceinline__ u32x4_t ld_nt4(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}
__device__ __forceinline__ u32x2_t ld_nt2(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
}
__device__ __forceinline__ uint32_t ld_nt1(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}

// NW 32-bit words from a 4*NW-byte block aligned to min(16, 4*NW) bytes.
template <int NW>
__device__ __forceinline__ void ld_nt_words(const void* p, uint32_t* w) {
  const uint8_t* b = reinterpret_cast<const uint8_t*>(p);
  if constexpr (NW % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
      const u32x4_t v = ld_nt4(b + 16 * i);
      w[4 * i] = v[0]; w[4 * i + 1] = v[1]; w[4 * i + 2] = v[2]; w[4 * i + 3] = v[3];
    }
  } else if constexpr (NW % 2 == 0) {
#pragma unroll
    for (int i = 0; i < NW / 2; ++i) {
      const u32x2_t v = ld_nt2(b + 8 * i);
      w[2 * i] = v[0]; w[2 * i + 1] = v[1];
    }
  } else {
#pragma unroll
    for (int i = 0; i < NW; ++i) w[i] = ld_nt1(b + 4 * i);
  }
}

// Order-preserving map of a float onto uint32 (larger float -> larger key);
// NaN maps below -inf so it is never preferred.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Tokens actually present in a sequence, clamped to the page table.
__device__ __forceinline__ int clamp_len(int T, int max_pages, int P) {
  long long cap = (long long)max_pages * P;
  if (T < 0) return 0;
  return (long long)T > cap ? (int)cap : T;
}

}  // namespace locks

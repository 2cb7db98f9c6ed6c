// (a1) Summary build, [Locks] §3-§4: for one (physical block, KV head) tile of
// P keys, fit
//   mu = (1/P) sum_i k_i,  D = K - 1 mu^T,
//   V  = top-r eigenvectors of H = D^T D (d x d),  C = D V,
// and store (mu, V^T, C) in the summary record.
//
// The top-r eigenvectors of D^T D are the top-r right singular vectors of D
// ([Locks] App. A.2), reached here through the P x P dual Gram M = D D^T
// (P <= d for every supported shape): if M u = theta u with theta > 0, then
// v = D^T u / sqrt(theta) is a unit eigenvector of D^T D with the same
// eigenvalue. One workgroup (4 waves) per tile, all in LDS and registers:
//  1. Keys -> registers; the centroid is a plain fp32 mean; the centred keys
//     D = K - mu are kept in LDS, for bf16 keys as bf16 hi + lo parts (their
//     sum is D to about 2^-16 relative), so the Gram needs no uncentred
//     subtraction whatever the keys' common offset.
//  2. M = D D^T on the matrix cores: v_mfma_f32_16x16x32_bf16 on hi.hi +
//     hi.lo + lo.hi (exact bf16 products, fp32 sums) for bf16 keys,
//     v_mfma_f32_16x16x4_f32 for fp32 keys. Wave w computes the 16-row block
//     w of M; by symmetry its MFMA outputs already are the A operand of M X
//     for those rows (k index permuted as k = 16 I + 4 g + i), so M never
//     leaves registers.
//  3. Top-r eigenvectors of M: for P = 16 one Rayleigh-Ritz step on the whole
//     space (X = I, exact); for P >= 32 subspace iteration on a 16-column
//     block started from signed Hadamard columns, X <- orth(M X) by
//     Cholesky-QR (columns that collapse are replaced by pseudo-random
//     vectors), from the third product on each followed by a Rayleigh-Ritz
//     step: T = X^T M X (16 x 16) diagonalised by parallel
//     cyclic Jacobi, Ritz vectors U = X W, Ritz values theta. The fit has
//     converged when (a) every one of the r leading Ritz pairs has a residual
//     ||M u_i - theta_i u_i|| <= 2^-10 theta_1, i.e. each vector is exact for
//     a Gram within 2^-10 of the stored one (below the bf16 rounding of the
//     keys themselves), and (b) every leading m-subspace (m <= r) whose Ritz
//     gap theta_m - theta_(m+1) exceeds 2^-7 theta_1 has a residual
//     ||R_m||_F <= 2^-6 (theta_m - theta_(m+1)), which by the sin-theta bound
//     puts it within an angle of about 2^-6 of the exact one; otherwise the
//     iteration continues from M U. The number of products, and whether the
//     bounds were met within the cap, are reported by
//     locks_build_summaries_ex.
//  4. V = D^T U_r (matrix cores), normalised and made orthonormal to fp32
//     level by one Newton-Schulz step (the columns of Ritz vectors are already
//     nearly orthogonal), or, when the r-th Ritz value is tiny against the
//     first, by Cholesky-QR (a second pass when a column vanished and was
//     replaced); each column sign-fixed so its largest-magnitude entry is
//     positive (lowest index on ties).
//  5. C = D V in fp32 from the unrounded V (matrix cores); mu, V, C are rounded
//     to the summary dtype independently. Quantized ("i4") records, [Locks] §4
//     and App. C.7: per group (the centroid, each basis vector, each token's
//     coefficient row) scale = bf16(max|x| / L), L = 127 for the 8-bit centroid
//     and coefficients and 7 for the 4-bit basis, and code =
//     round-half-even(x / scale), all in fp32 (correctly rounded division).
#include <utility>

#include "common.h"
#include "kernels.h"

namespace locks {

constexpr int kBlk = 16;                    // block size of the subspace iteration
constexpr int kFirstRitzCheck = 3;          // the product after which the first Rayleigh-Ritz step comes (P >= 32)
constexpr int kMaxProducts = 32;            // cap on products M X
constexpr float kRitzTol = 1.0f / 1024.0f;  // residual bound of every pair, relative to the largest Ritz value
constexpr float kGapFloor = 1.0f / 128.0f;  // a Ritz gap above this fraction of the largest value is significant
constexpr float kSubspaceTol = 1.0f / 64.0f;   // residual bound of a leading subspace, relative to its gap
constexpr int kMaxSweeps = 12;              // Jacobi sweeps of one Rayleigh-Ritz step
constexpr float kJacobiAbs = 0x1p-20f;      // off-diagonal entries below this fraction of the largest diagonal are converged
constexpr float kJacobiStop = 0x1p-10f;     // a sweep whose largest rotated entry is below this fraction is the last

namespace {

__device__ __forceinline__ float hash_unit(uint32_t a, uint32_t b, uint32_t salt) {
  uint32_t x = a * 0x9E3779B1u ^ (b + 97u * salt) * 0x85EBCA77u;
  x ^= x >> 15; x *= 0x2C1B3C6Du;
  x ^= x >> 12; x *= 0x297A2D39u;
  x ^= x >> 15;
  return (float)(x >> 8) * (1.0f / 8388608.0f) - 1.0f;  // [-1, 1)
}

__device__ __forceinline__ float rdl(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// v of lane `src` of the wave
__device__ __forceinline__ float lane_at(int src, float v) {
  return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(v)));
}

// v of lane (lane ^ X), X known at compile time: DPP where a quad or row
// permutation expresses it (quad_perm [1,0,3,2], [2,3,0,1], [3,2,1,0],
// row_half_mirror, row_ror:8, row_mirror), the LDS swizzle inside 32 lanes,
// a permute beyond
template <int X>
__device__ __forceinline__ float lane_xor(float v) {
  static_assert(X > 0 && X < 64, "lane xor");
  const int iv = __float_as_int(v);
  int r;
  if constexpr (X == 1) r = __builtin_amdgcn_mov_dpp(iv, 0xB1, 0xF, 0xF, true);
  else if constexpr (X == 2) r = __builtin_amdgcn_mov_dpp(iv, 0x4E, 0xF, 0xF, true);
  else if constexpr (X == 3) r = __builtin_amdgcn_mov_dpp(iv, 0x1B, 0xF, 0xF, true);
  else if constexpr (X == 7) r = __builtin_amdgcn_mov_dpp(iv, 0x141, 0xF, 0xF, true);
  else if constexpr (X == 8) r = __builtin_amdgcn_mov_dpp(iv, 0x128, 0xF, 0xF, true);
  else if constexpr (X == 15) r = __builtin_amdgcn_mov_dpp(iv, 0x140, 0xF, 0xF, true);
  else if constexpr (X < 32) r = __builtin_amdgcn_ds_swizzle(iv, (X << 10) | 0x1F);  // and 31, xor X
  else r = __builtin_amdgcn_ds_bpermute((int)(((threadIdx.x & 63) ^ X) << 2), iv);
  return __int_as_float(r);
}

// v of lane N of the lane's row of 16 (DPP row_newbcast)
template <int N>
__device__ __forceinline__ float row_lane(float v) {
  static_assert(N >= 0 && N < 16, "row lane");
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + N, 0xF, 0xF, true));
}

// row_lane<n> for an n that is a constant once loops are unrolled
__device__ __forceinline__ float row_lane_at(float v, int n) {
  switch (n) {
    case 0: return row_lane<0>(v);
    case 1: return row_lane<1>(v);
    case 2: return row_lane<2>(v);
    case 3: return row_lane<3>(v);
    case 4: return row_lane<4>(v);
    case 5: return row_lane<5>(v);
    case 6: return row_lane<6>(v);
    case 7: return row_lane<7>(v);
    case 8: return row_lane<8>(v);
    case 9: return row_lane<9>(v);
    case 10: return row_lane<10>(v);
    case 11: return row_lane<11>(v);
    case 12: return row_lane<12>(v);
    case 13: return row_lane<13>(v);
    case 14: return row_lane<14>(v);
    default: return row_lane<15>(v);
  }
}

template <int... Ns>
__device__ __forceinline__ void bcast_row16_impl(float v, float (&out)[16], std::integer_sequence<int, Ns...>) {
  ((out[Ns] = row_lane<Ns>(v)), ...);
}
// out[N] = v of lane N of the lane's row of 16, N = 0..15
__device__ __forceinline__ void bcast_row16(float v, float (&out)[16]) {
  bcast_row16_impl(v, out, std::make_integer_sequence<int, 16>{});
}

// a[k] for a per-lane k in 0..3, as a two-level select on the bits of k
// (an indexed form is compiled to a store and load through LDS)
__device__ __forceinline__ float pick4(const float (&a)[4], int k) {
  const float l = (k & 1) ? a[1] : a[0];
  const float u = (k & 1) ? a[3] : a[2];
  return (k & 2) ? u : l;
}

// One round of parallel cyclic Jacobi on a 16 x 16 symmetric T held by one
// wave: lane (g, j) = (lane >> 4, lane & 15) owns column n = j ^ 4 g (every
// row of 16 lanes holds all columns, the column that equals one of the lane
// row's own rows 4 g + i sitting at position i) and holds t4[i] = T[4 g + i][n],
// w4[i] = W[4 g + i][n] and dg = T[n][n]. Round t rotates the 8 disjoint
// pairs {p, p ^ t}: T <- J^T T J, W <- W J, with J[p][p] = J[q][q] = c,
// J[p][q] = s, J[q][p] = -s for p < q. Every lane forms the rotation of its
// own column's pair {lo, hi} from the diagonal entries (its own and lane
// lane ^ t's, which owns column n ^ t) and T[hi][lo] read from column lo, so
// the two columns of a pair form the same rotation. The entries the two-sided
// update combines, T[x][q], T[x ^ t][n] and T[x ^ t][q] for q = n ^ t, sit in
// lanes lane ^ t, lane ^ 16 (t >> 2) ^ (t & 12) and lane ^ 16 (t >> 2) ^ (t & 3)
// and are requested at the start, as none depends on this round's rotation;
// the rotation (c, J[x ^ t][x]) of row x = 4 g + i is broadcast from position
// i of the lane's row. A pair rotates only while |T[hi][lo]| exceeds
// floor_abs; the tangent is sign(d) e / (|d| + sqrt(d^2 + e^2)),
// d = T[hi][hi] - T[lo][lo], e = 2 T[hi][lo] (|tan| <= 1), and the diagonal
// moves by -/+ tan T[hi][lo] (the annihilated entry's exact effect on the
// pair's diagonal); `big` records an entry above stop_abs.
template <int t>
__device__ __forceinline__ void jacobi_round(float (&t4)[4], float (&w4)[4], float& dg, float floor_abs,
                                             float stop_abs, bool& big) {
  constexpr int hb = t >= 8 ? 8 : (t >= 4 ? 4 : (t >= 2 ? 2 : 1));  // p < p ^ t iff (p & hb) == 0
  constexpr int gx = 16 * (t >> 2);  // lane offset of the row partners' row group
  constexpr int it = t & 3;          // element offset of the row partners
  const int lane = threadIdx.x & 63;
  const int g = lane >> 4;
  const int n = (lane & 15) ^ (4 * g);
  const bool first = (n & hb) == 0;  // n is the pair's lo
  const int lo = first ? n : (n ^ t), hi = lo ^ t;
  const float oself = pick4(t4, (n & 3) ^ it);                      // T[4 g + ((n ^ t) & 3)][n]
  const float apq = lane_at(4 * (hi & 12) + (lo ^ (hi & 12)), oself);  // T[hi][lo]: column lo in row group hi >> 2
  const float dq = lane_xor<t>(dg);                                   // T[n ^ t][n ^ t]
  float xq[4], xr[4], xrq[4], wq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xq[i] = lane_xor<t>(t4[i]);  // T[4 g + i][n ^ t]
    wq[i] = lane_xor<t>(w4[i]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (t < 4) {
      xr[i] = t4[i ^ it];    // T[(4 g + i) ^ t][n]
      xrq[i] = xq[i ^ it];   // T[(4 g + i) ^ t][n ^ t]
    } else {
      xr[i] = lane_xor<gx ^ (t & 12)>(t4[i ^ it]);
      xrq[i] = lane_xor<gx ^ it>(t4[i ^ it]);
    }
  }
  // every exchange is issued before the rotation waits for T[hi][lo]
  __builtin_amdgcn_sched_barrier(0);
  const float app = first ? dg : dq, aqq = first ? dq : dg;
  const float d = aqq - app, e = 2.f * apq;
  const float rt = __builtin_amdgcn_sqrtf(fmaf(d, d, e * e));
  const float tr = (d >= 0.f ? e : -e) * __builtin_amdgcn_rcpf(fabsf(d) + rt);
  const float tt = fabsf(apq) > floor_abs ? tr : 0.f;
  big = big || fabsf(apq) > stop_abs;
  const float c = __builtin_amdgcn_rsqf(fmaf(tt, tt, 1.f));
  const float s = tt * c;
  const float on = first ? -s : s;  // J[n ^ t][n]
  const float ta = tt * apq;
  dg = first ? dg - ta : dg + ta;
  const float cx[4] = {row_lane<0>(c), row_lane<1>(c), row_lane<2>(c), row_lane<3>(c)};
  const float ox[4] = {row_lane<0>(on), row_lane<1>(on), row_lane<2>(on), row_lane<3>(on)};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a0 = c * t4[i] + on * xq[i];   // (T J)[x][n]
    const float a1 = c * xr[i] + on * xrq[i];  // (T J)[x ^ t][n]
    t4[i] = cx[i] * a0 + ox[i] * a1;
    w4[i] = c * w4[i] + on * wq[i];
  }
}

template <int... ts>
__device__ __forceinline__ void jacobi_sweep(std::integer_sequence<int, ts...>, float (&t4)[4], float (&w4)[4],
                                             float& dg, float floor_abs, float stop_abs, bool& big) {
  (jacobi_round<ts + 1>(t4, w4, dg, floor_abs, stop_abs, big), ...);
}

// Centred keys in LDS: row-major [P][D], 16-byte chunks XOR-swizzled by row so
// that 16 lanes reading one chunk of 16 different rows hit distinct banks.
template <typename T, int D, int P>
struct CentredKeys;

template <int D, int P>
struct CentredKeys<bf16_t, D, P> {
  static constexpr int kChunks = D / 8;  // 16-byte chunks per row
  bf16_t hi[P * D];
  bf16_t lo[P * D];
  static __device__ __forceinline__ int chunk_off(int row, int chunk) {
    return row * D + ((chunk ^ (row & (kChunks - 1))) << 3);
  }
  __device__ __forceinline__ float at(int row, int a) const {
    const int o = chunk_off(row, a >> 3) + (a & 7);
    return bf16_to_f32(hi[o]) + bf16_to_f32(lo[o]);
  }
};

template <int D, int P>
struct CentredKeys<float, D, P> {
  static constexpr int kChunks = D / 4;
  float v[P * D];
  static __device__ __forceinline__ int chunk_off(int row, int chunk) {
    return row * D + ((chunk ^ (row & (kChunks - 1))) << 2);
  }
  __device__ __forceinline__ float at(int row, int a) const { return v[chunk_off(row, a >> 2) + (a & 3)]; }
};

template <typename T, int D, int P>
struct alignas(16) BuildLds {
  CentredKeys<T, D, P> dk;
  float mu[D];
  float X[P][kBlk];        // orthonormal block; at the end the Ritz vectors U
  float Y[P][kBlk];        // M X, then M U; at the end C = D V
  float Vb[D][kBlk];       // D^T U, then the orthonormal basis V
  float Gp[4][kBlk][kBlk]; // the waves' partial Gram matrices (and centroid partial sums)
  float RiW[4][kBlk][kBlk];  // each wave's R^-1 of the Cholesky-QR
  float Wo[kBlk][kBlk];    // eigenvectors of T, descending eigenvalue order
  float th[kBlk];          // Ritz values, descending
  float dg[kBlk];          // diagonal of the diagonalised T
  float res[4][kBlk];      // partial squared residual norms
  int flag;
};

}  // namespace

template <typename T, int D, int P, bool I4>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void build_kernel(BuildArgs a) {
  constexpr int NB = P / 16;  // 16-row blocks of M (and of X, Y, C)
  constexpr int DB = D / 16;  // 16-row blocks of V
  static_assert(P == 16 || P == 32 || P == 64, "page size");
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(sizeof(BuildLds<T, D, P>) <= 64 * 1024, "LDS budget");
  __shared__ BuildLds<T, D, P> L;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int ln = lane & 15;  // MFMA column / row-in-tile
  const int lg = lane >> 4;  // MFMA k group / row group
  const int h = blockIdx.y;
  const int r = a.r;
  const int blk = a.block_ids[blockIdx.x];
  if (blk < 0 || (int64_t)blk >= a.num_blocks) return;  // uniform for the workgroup
  const T* tile = reinterpret_cast<const T*>(a.k_pool) + ((int64_t)blk * a.Hkv + h) * (int64_t)P * D;

  // ---- 1. keys -> registers, centroid, centred keys -> LDS ----
  {
    constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
    constexpr int CPR = D / EPC;         // chunks per row
    constexpr int NCHUNK = P * CPR;      // chunks in the tile
    constexpr int NCH = (NCHUNK + 255) / 256;  // chunks per thread
    static_assert(64 % CPR == 0 && (NCHUNK >= 256 ? NCHUNK % 256 == 0 : 256 % NCHUNK == 0), "chunk split");
    u32x4_t raw[NCH];
#pragma unroll
    for (int m = 0; m < NCH; ++m) {
      const int c = tid + 256 * m;
      raw[m] = c < NCHUNK ? *reinterpret_cast<const u32x4_t*>(tile + (int64_t)c * EPC) : u32x4_t{0u, 0u, 0u, 0u};
    }
    // thread t holds chunk column t % CPR of rows t / CPR + (256 / CPR) m
    const int cc = tid % CPR;
    float part[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) {
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < NCH; ++m) s += Elem<T>::load(reinterpret_cast<const T*>(&raw[m]) + e);
      part[e] = s;
    }
    // lanes with the same chunk column are CPR apart: fold the wave, then the waves
#pragma unroll
    for (int o = CPR; o < 64; o <<= 1)
#pragma unroll
      for (int e = 0; e < EPC; ++e) part[e] += __shfl_xor(part[e], o, 64);
    float* msum = &L.Gp[0][0][0];  // [4][D]
    if (lane < CPR) {
#pragma unroll
      for (int e = 0; e < EPC; ++e) msum[wave * D + cc * EPC + e] = part[e];
    }
    __syncthreads();
    if (tid < D) L.mu[tid] = ((msum[tid] + msum[D + tid]) + (msum[2 * D + tid] + msum[3 * D + tid])) / (float)P;
    __syncthreads();
#pragma unroll
    for (int m = 0; m < NCH; ++m) {
      if (tid + 256 * m >= NCHUNK) continue;
      const int row = (tid + 256 * m) / CPR;
      if constexpr (sizeof(T) == 2) {
        uint32_t wh[4], wl[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const uint32_t w = raw[m][e2];
          const float d0 = bf16_lo(w) - L.mu[cc * 8 + 2 * e2];
          const float d1 = bf16_hi(w) - L.mu[cc * 8 + 2 * e2 + 1];
          const bf16_t h0 = f32_to_bf16(d0), h1 = f32_to_bf16(d1);
          const bf16_t l0 = f32_to_bf16(d0 - bf16_to_f32(h0)), l1 = f32_to_bf16(d1 - bf16_to_f32(h1));
          wh[e2] = (uint32_t)h0 | ((uint32_t)h1 << 16);
          wl[e2] = (uint32_t)l0 | ((uint32_t)l1 << 16);
        }
        const int o = CentredKeys<T, D, P>::chunk_off(row, cc);
        *reinterpret_cast<u32x4_t*>(&L.dk.hi[o]) = u32x4_t{wh[0], wh[1], wh[2], wh[3]};
        *reinterpret_cast<u32x4_t*>(&L.dk.lo[o]) = u32x4_t{wl[0], wl[1], wl[2], wl[3]};
      } else {
        const float* f = reinterpret_cast<const float*>(&raw[m]);
        const int o = CentredKeys<T, D, P>::chunk_off(row, cc);
        *reinterpret_cast<f32x4_t*>(&L.dk.v[o]) =
            f32x4_t{f[0] - L.mu[cc * 4], f[1] - L.mu[cc * 4 + 1], f[2] - L.mu[cc * 4 + 2], f[3] - L.mu[cc * 4 + 3]};
      }
    }
  }
  __syncthreads();

  // ---- 2. M = D D^T: wave w < NB holds hreg[I][i] = M[16 I + 4 lg + i][16 w + ln] ----
  f32x4_t hreg[NB];
  if (wave < NB) {
#pragma unroll
    for (int I = 0; I < NB; ++I) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int s = 0; s < D / 32; ++s) {
          const int oa = CentredKeys<T, D, P>::chunk_off(16 * I + ln, 4 * s + lg);
          const int ob = CentredKeys<T, D, P>::chunk_off(16 * wave + ln, 4 * s + lg);
          const bf16x8_t ah = *reinterpret_cast<const bf16x8_t*>(&L.dk.hi[oa]);
          const bf16x8_t al = *reinterpret_cast<const bf16x8_t*>(&L.dk.lo[oa]);
          const bf16x8_t bh = *reinterpret_cast<const bf16x8_t*>(&L.dk.hi[ob]);
          const bf16x8_t bl = *reinterpret_cast<const bf16x8_t*>(&L.dk.lo[ob]);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
        }
      } else {
#pragma unroll 8
        for (int s = 0; s < D / 4; ++s)
          acc = __builtin_amdgcn_mfma_f32_16x16x4f32(L.dk.at(16 * I + ln, 4 * s + lg), L.dk.at(16 * wave + ln, 4 * s + lg),
                                                     acc, 0, 0, 0);
      }
      hreg[I] = acc;
    }
  }

  // ---- helpers ----
  // Every wave, in registers, lane l taking column c = l & 15 of the block
  // Gram G (am[r] = G[r][c], gd = G[c][c]; every row of 16 lanes holds the
  // whole matrix, and entries of other columns come by row broadcast):
  // column scaling S (columns with a vanishing norm are dead), Cholesky
  // S G S = L L^T (right-looking: step j broadcasts column j, and lane c
  // keeps row c of L in lrow[]; a column whose pivot is 1e-12 or less is dead
  // and gets a zero column of L and a zero reciprocal pivot, so it neither
  // updates the others nor survives the inverse), then column c of L^-1 by
  // forward substitution and row c of Ri = S L^-T to this wave's RiW (dead
  // columns zero). Returns the dead-column mask (uniform).
  auto chol_rinv = [&](float* am, float gd) -> uint32_t {
    const int col = ln;
    float dmax = gd;
    dmax = fmaxf(dmax, lane_xor<1>(dmax));
    dmax = fmaxf(dmax, lane_xor<2>(dmax));
    dmax = fmaxf(dmax, lane_xor<4>(dmax));
    dmax = fmaxf(dmax, lane_xor<8>(dmax));
    const bool live = gd > 1e-30f * fmaxf(dmax, 1e-30f);
    const float sc = live ? __builtin_amdgcn_rsqf(gd) : 0.f;
    float sr[kBlk];
    bcast_row16(sc, sr);
#pragma unroll
    for (int r = 0; r < kBlk; ++r) am[r] *= sr[r] * sc;
    // the chain of pivots uses the hardware reciprocal square root (about
    // 1 ulp): the factor only has to orthonormalise the block to fp32 level
    uint32_t dead = 0u;
    float invd[kBlk];  // 1 / L[j][j], 0 for a dead column
    float lrow[kBlk];  // L[c][j] for j <= c
#pragma unroll
    for (int j = 0; j < kBlk; ++j) {
      const float vjj = row_lane_at(am[j], j);  // (S G S - ...)[j][j], from lane j
      const bool ok = vjj > 1e-12f;                // the same in every lane; a dead row's entries are 0
      invd[j] = ok ? __builtin_amdgcn_rsqf(vjj) : 0.f;
      dead |= ok ? 0u : 1u << j;
      lrow[j] = am[j] * invd[j];
      const float f = -lrow[j] * invd[j];  // -L[c][j] / L[j][j]
      // am[r] -= L[r][j] L[c][j] = column j's entry r times f
#pragma unroll
      for (int r = j + 1; r < kBlk; ++r) am[r] = fmaf(row_lane_at(am[r], j), f, am[r]);
    }
    // z = L^-1 e_c, column by column (L[i][k] is lane i's lrow[k]). Step k
    // broadcasts lrow[k] + 0 z[k], which cannot be formed before z[k]: the
    // broadcasts of every step hoisted to the start were live at once and
    // cost registers the second wave of a SIMD needs.
    float z[kBlk];
#pragma unroll
    for (int i = 0; i < kBlk; ++i) z[i] = i == col ? 1.f : 0.f;
#pragma unroll
    for (int k = 0; k < kBlk; ++k) {
      z[k] *= invd[k];
      const float nz = -z[k];
      const float lk = fmaf(0.f, z[k], lrow[k]);
#pragma unroll
      for (int i = k + 1; i < kBlk; ++i) z[i] = fmaf(row_lane_at(lk, i), nz, z[i]);
    }
    // Ri[c][b] = s_c (L^-1)[b][c]
    if (lane < kBlk) {
#pragma unroll
      for (int c = 0; c < kBlk; c += 4)
        *reinterpret_cast<f32x4_t*>(&L.RiW[wave][col][c]) = f32x4_t{sc * z[c], sc * z[c + 1], sc * z[c + 2], sc * z[c + 3]};
    }
    return __builtin_amdgcn_readfirstlane(dead);
  };

  // Cholesky-QR of the NR x 16 rows in `src` (LDS, row-major) into `dst`
  // (may be `src`): wave w takes the 16-row tiles w, w + 4, ...; dead columns
  // become pseudo-random vectors (call again to orthonormalise those). The
  // Gram partials are formed here unless the product that wrote `src` left
  // them in Gp (`gram_ready`, after a workgroup barrier). Returns the
  // dead-column mask (uniform).
  auto cholqr = [&](const float (*src)[kBlk], float (*dst)[kBlk], int NR, uint32_t salt,
                    bool gram_ready) -> uint32_t {
    if (!gram_ready) {
      f32x4_t m = {0.f, 0.f, 0.f, 0.f};
      for (int t = wave; t < NR / 16; t += 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = src[16 * t + 4 * lg + i][ln];
          m = __builtin_amdgcn_mfma_f32_16x16x4f32(v, v, m, 0, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) L.Gp[wave][4 * lg + i][ln] = m[i];
      __syncthreads();
    }
    float am[kBlk];
#pragma unroll
    for (int c = 0; c < kBlk; c += 4) {
      f32x4_t v = *reinterpret_cast<const f32x4_t*>(&L.Gp[0][ln][c]);
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        const f32x4_t u = *reinterpret_cast<const f32x4_t*>(&L.Gp[w][ln][c]);
        v[0] += u[0]; v[1] += u[1]; v[2] += u[2]; v[3] += u[3];
      }
      am[c] = v[0]; am[c + 1] = v[1]; am[c + 2] = v[2]; am[c + 3] = v[3];
    }
    const float gd = ((L.Gp[0][ln][ln] + L.Gp[1][ln][ln]) + L.Gp[2][ln][ln]) + L.Gp[3][ln][ln];
    const uint32_t dead = chol_rinv(am, gd);
    wave_lds_sync();  // RiW[wave] visible to the wave
    const bool dcol = (dead >> ln) & 1u;
    for (int t = wave; t < NR / 16; t += 4) {
      f32x4_t x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k0 = 0; k0 < kBlk; k0 += 4)
        x = __builtin_amdgcn_mfma_f32_16x16x4f32(src[16 * t + ln][k0 + lg], L.RiW[wave][k0 + lg][ln], x, 0, 0, 0);
      wave_lds_sync();  // every lane's reads of the tile are done before it is overwritten (src == dst)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * t + 4 * lg + i;
        dst[row][ln] = dcol ? hash_unit((uint32_t)row, (uint32_t)ln, salt) : x[i];
      }
    }
    __syncthreads();
    return dead;
  };

  // One Newton-Schulz step towards orthonormal columns for the first r
  // columns of the NR x 16 rows in `buf` (columns r.. become zero):
  // buf <- buf S (3/2 I - 1/2 S G S), G = buf^T buf, S = diag(G)^-1/2, which
  // takes columns whose pairwise cosines are at most e to at most about
  // 3/2 e^2 (the same two barriers as cholqr, no serial factorisation).
  // Returns the largest cosine it started from (uniform: every wave forms
  // the same value from the same sums).
  auto ns_orth = [&](float (*buf)[kBlk], int NR, int ncols) -> float {
    f32x4_t m = {0.f, 0.f, 0.f, 0.f};
    for (int t = wave; t < NR / 16; t += 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float v = buf[16 * t + 4 * lg + i][ln];
        m = __builtin_amdgcn_mfma_f32_16x16x4f32(v, v, m, 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) L.Gp[wave][4 * lg + i][ln] = m[i];
    __syncthreads();
    auto gsum = [&](int x, int y) { return (L.Gp[0][x][y] + L.Gp[1][x][y]) + (L.Gp[2][x][y] + L.Gp[3][x][y]); };
    const float sj = ln < ncols ? __builtin_amdgcn_rsqf(gsum(ln, ln)) : 0.f;
    float cmax = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * lg + i;
      const float si = row < ncols ? __builtin_amdgcn_rsqf(gsum(row, row)) : 0.f;
      const float cs = si * gsum(row, ln) * sj;  // cosine of columns row, ln
      cmax = row != ln ? fmaxf(cmax, fabsf(cs)) : cmax;
      L.RiW[wave][row][ln] = si * ((row == ln ? 1.5f : 0.f) - 0.5f * cs);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) cmax = fmaxf(cmax, __shfl_xor(cmax, o, 64));
    wave_lds_sync();  // RiW[wave] visible to the wave
    for (int t = wave; t < NR / 16; t += 4) {
      f32x4_t x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k0 = 0; k0 < kBlk; k0 += 4)
        x = __builtin_amdgcn_mfma_f32_16x16x4f32(buf[16 * t + ln][k0 + lg], L.RiW[wave][k0 + lg][ln], x, 0, 0, 0);
      wave_lds_sync();  // every lane's reads of the tile are done before it is overwritten
#pragma unroll
      for (int i = 0; i < 4; ++i) buf[16 * t + 4 * lg + i][ln] = x[i];
    }
    __syncthreads();
    return __shfl(cmax, 0, 64);
  };

  // Y = M X for this wave's rows (wave < NB): lane (ln, lg) -> Y[16 wave + 4 lg + i][ln]
  // With `gram`, also this wave's partial Y^T Y of its rows into Gp (the
  // Gram the Cholesky-QR of Y starts from; waves without rows write zeros).
  auto product = [&](bool gram) {
    f32x4_t y = {0.f, 0.f, 0.f, 0.f};
    if (wave < NB) {
#pragma unroll
      for (int I = 0; I < NB; ++I)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          y = __builtin_amdgcn_mfma_f32_16x16x4f32(hreg[I][i], L.X[16 * I + 4 * lg + i][ln], y, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) L.Y[16 * wave + 4 * lg + i][ln] = y[i];
    }
    if (gram) {
      f32x4_t m = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) m = __builtin_amdgcn_mfma_f32_16x16x4f32(y[i], y[i], m, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) L.Gp[wave][4 * lg + i][ln] = m[i];
    }
  };

  // Rayleigh quotient T = (G + G^T) / 2 of the summed partials G in Gp,
  // diagonalised by parallel cyclic Jacobi in one wave's registers (wave 0;
  // jacobi_round): about 465 shader cycles a round (0.2 us). Measured slower:
  // 256 threads each owning one entry of T and W in LDS with a barrier per
  // round (0.38 us a round); one wave keeping T and W^T in the matrix-core
  // layout, each round as twelve v_mfma_f32_16x16x4_f32 (0.42 us); this wave
  // layout with the diagonal gathered every round and the rows' rotations
  // recomputed from gathered tangents (0.38 us), then with the diagonal kept
  // per lane and the rotations read by permute (0.28 us), then fetched by row
  // broadcast (0.24 us) before the exchanges were issued ahead of the wait
  // for T[hi][lo]. A pair is rotated only while its
  // off-diagonal entry exceeds 2^-20 of the largest diagonal entry t_max
  // (about the largest eigenvalue): a smaller entry moves an eigenvector by
  // at most 2^-20 t_max / gap, and the Ritz pairs are only used where the
  // gap is a sizeable fraction of t_max. Pairs of two small eigenvalues
  // therefore stop rotating as soon as their coupling is small against
  // t_max. The sweeps stop after one that rotated no entry above 2^-10 t_max
  // (the next sweep's would be of about its square). Stopping at 2^-7 saved
  // a sweep in half the tiles but not its time, and cost fp32 fits their
  // accuracy. Then Wo = W in descending order of eigenvalue, th = those
  // eigenvalues (ties by index).
  auto jacobi = [&]() {
    if (wave != 0) return;
    const int cn = ln ^ (4 * lg);  // this lane's column
    float t4[4], w4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int x = 4 * lg + i;
      const float v = (L.Gp[0][x][cn] + L.Gp[1][x][cn]) + (L.Gp[2][x][cn] + L.Gp[3][x][cn]);
      const float vt = (L.Gp[0][cn][x] + L.Gp[1][cn][x]) + (L.Gp[2][cn][x] + L.Gp[3][cn][x]);
      t4[i] = 0.5f * (v + vt);
      w4[i] = x == cn ? 1.f : 0.f;
    }
    // T[cn][cn] from the lane whose row group holds row cn and whose column is cn
    float dg = lane_at(16 * (cn >> 2) + (cn & 3), pick4(t4, cn & 3));
    float tmax = fabsf(dg);
    tmax = fmaxf(tmax, lane_xor<1>(tmax));
    tmax = fmaxf(tmax, lane_xor<2>(tmax));
    tmax = fmaxf(tmax, lane_xor<4>(tmax));
    tmax = fmaxf(tmax, lane_xor<8>(tmax));
    const float floor_abs = kJacobiAbs * tmax;
    const float stop_abs = kJacobiStop * tmax;
    for (int sweep = 0; sweep < kMaxSweeps; ++sweep) {
      bool big = false;
      jacobi_sweep(std::make_integer_sequence<int, kBlk - 1>{}, t4, w4, dg, floor_abs, stop_abs, big);
      if (__ballot(big) == 0) break;  // uniform
    }
    const float dv = dg;
    if (lane < kBlk) L.dg[cn] = dv;
    wave_lds_sync();
    int rank = 0;
#pragma unroll
    for (int j = 0; j < kBlk; ++j) {
      const float u = L.dg[j];
      rank += (u > dv || (u == dv && j < cn)) ? 1 : 0;
    }
    if (lane < kBlk) L.th[rank] = dv;
#pragma unroll
    for (int i = 0; i < 4; ++i) L.Wo[4 * lg + i][rank] = w4[i];
  };

  // ---- 3. top-r eigenvectors of M into X ----
  int products = 0;
  bool converged = false;
  if constexpr (NB == 1) {
    for (int e = tid; e < kBlk * kBlk; e += 256) L.X[e / kBlk][e % kBlk] = (e / kBlk == e % kBlk) ? 1.f : 0.f;
  } else {
    // an orthonormal start without a factorisation: 16 columns of the
    // P x P Sylvester-Hadamard matrix, rows with pseudo-random signs, / sqrt(P)
    const float inv = 1.0f / sqrtf((float)P);
    for (int e = tid; e < P * kBlk; e += 256) {
      const int i = e / kBlk, j = e % kBlk;
      const float sg = hash_unit((uint32_t)i, 0u, 1u) < 0.f ? -inv : inv;
      L.X[i][j] = (__builtin_popcount(i & j) & 1) ? -sg : sg;
    }
  }
  __syncthreads();
  const int first_rr = NB == 1 ? 1 : kFirstRitzCheck;
  while (true) {
    product(products + 1 < first_rr);
    ++products;
    if (products < first_rr) {
      __syncthreads();
      cholqr(L.Y, L.X, P, 3u + (uint32_t)products, true);
      continue;
    }
    // Rayleigh-Ritz: T = X^T Y (waves < NB each its rows), summed and symmetrised by wave 0
    {
      f32x4_t m = {0.f, 0.f, 0.f, 0.f};
      if (wave < NB) {
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < 4; ++i)
          m = __builtin_amdgcn_mfma_f32_16x16x4f32(L.X[16 * wave + 4 * lg + i][ln], L.Y[16 * wave + 4 * lg + i][ln], m,
                                                   0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) L.Gp[wave][4 * lg + i][ln] = m[i];
    }
    __syncthreads();
    jacobi();
    __syncthreads();
    // Ritz vectors U = X Wo (into X) and M U = Y Wo (into Y); residual norms of the r leading pairs
    {
      float r2 = 0.f;
      if (wave < NB) {
        f32x4_t z = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < kBlk; k0 += 4) {
          const float wo = L.Wo[k0 + lg][ln];
          z = __builtin_amdgcn_mfma_f32_16x16x4f32(L.Y[16 * wave + ln][k0 + lg], wo, z, 0, 0, 0);
          u = __builtin_amdgcn_mfma_f32_16x16x4f32(L.X[16 * wave + ln][k0 + lg], wo, u, 0, 0, 0);
        }
        const float thn = L.th[ln];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = z[i] - thn * u[i];
          r2 = fmaf(e, e, r2);
        }
        wave_lds_sync();  // reads of the X and Y rows done before they are overwritten
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          L.X[16 * wave + 4 * lg + i][ln] = u[i];
          L.Y[16 * wave + 4 * lg + i][ln] = z[i];
        }
      }
      r2 += __shfl_xor(r2, 16, 64);
      r2 += __shfl_xor(r2, 32, 64);
      if (lane < kBlk) L.res[wave][lane] = r2;
    }
    __syncthreads();
    {
      // the same decision in every thread (uniform): every leading pair within
      // the backward bound, and every leading subspace whose Ritz gap is
      // significant within the sin-theta bound ||R_m||_F <= kSubspaceTol * gap
      const float th0 = fmaxf(L.th[0], 0.f);
      const float pair2 = (kRitzTol * th0) * (kRitzTol * th0);
      float acc2 = 0.f;
      bool ok = true;
      for (int m = 1; m <= r; ++m) {
        const float rm2 = (L.res[0][m - 1] + L.res[1][m - 1]) + (L.res[2][m - 1] + L.res[3][m - 1]);
        acc2 += rm2;
        ok = ok && rm2 <= pair2;
        const float gap = L.th[m - 1] - L.th[m];
        if (gap > kGapFloor * th0) ok = ok && acc2 <= (kSubspaceTol * gap) * (kSubspaceTol * gap);
      }
      converged = NB == 1 || ok;
    }
    if (converged || products >= kMaxProducts) break;
    // continue from M U
    cholqr(L.Y, L.X, P, 50u + (uint32_t)products, false);
  }
  if (tid == 0 && a.fit_info) a.fit_info[(int64_t)blockIdx.x * a.Hkv + h] = converged ? products : -products;

  // ---- 4. V = D^T U (columns beyond r are Ritz vectors too and are carried along) ----
  for (int b = wave; b < DB; b += 4) {
    f32x4_t v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int s = 0; s < P / 4; ++s)
      v = __builtin_amdgcn_mfma_f32_16x16x4f32(L.dk.at(4 * s + lg, 16 * b + ln), L.X[4 * s + lg][ln], v, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) L.Vb[16 * b + 4 * lg + i][ln] = v[i];
  }
  __syncthreads();
  // The columns D^T u_i of Ritz vectors are orthogonal up to the Jacobi
  // sweeps' remaining coupling (about 2^-20 theta_1) against norms
  // sqrt(theta_i), so unless the r-th Ritz value is tiny against the first,
  // a Newton-Schulz step makes them orthonormal (a second one when the
  // first found cosines above 2^-10); otherwise (a page of nearly lower rank)
  // Cholesky-QR, which also replaces vanishing columns.
  const float th0 = L.th[0], thr = L.th[r - 1];
  if (th0 > 0.f && thr > 0x1p-16f * th0 && th0 < 3.0e38f) {
    if (ns_orth(L.Vb, D, r) > 0x1p-10f) ns_orth(L.Vb, D, r);
  } else if (cholqr(L.Vb, L.Vb, D, 101u, false)) {
    cholqr(L.Vb, L.Vb, D, 102u, false);  // a replaced column is orthonormalised by a second pass
  }
  // sign: largest-magnitude entry positive (lowest index on ties). Wave 0:
  // lane (q, c) = (lane >> 4, lane & 15) scans rows q, q + 4, ... of column
  // c, the four quarters of a column (lanes c, c + 16, c + 32, c + 48) are
  // combined, and each lane flips its own rows.
  if (wave == 0) {
    float vq[D / 4];
#pragma unroll
    for (int k = 0; k < D / 4; ++k) vq[k] = L.Vb[lg + 4 * k][ln];
    float best = -1.f, bv = 1.f;
    int arg = D;
#pragma unroll
    for (int k = 0; k < D / 4; ++k) {
      const bool gt = fabsf(vq[k]) > best;
      best = gt ? fabsf(vq[k]) : best;
      arg = gt ? lg + 4 * k : arg;
      bv = gt ? vq[k] : bv;
    }
#pragma unroll
    for (int o = 16; o < 64; o <<= 1) {
      const float ob = __shfl_xor(best, o, 64), ov = __shfl_xor(bv, o, 64);
      const int oa = __shfl_xor(arg, o, 64);
      if (ob > best || (ob == best && oa < arg)) { best = ob; arg = oa; bv = ov; }
    }
    // (every entry NaN: no argument, the sign stays)
    if (ln < r && bv < 0.f) {
#pragma unroll
      for (int k = 0; k < D / 4; ++k) L.Vb[lg + 4 * k][ln] = -vq[k];
    }
  }
  __syncthreads();

  // ---- 5. C = D V (wave w < NB, rows 16 w ..), into Y; then the record ----
  if (wave < NB) {
    f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int s = 0; s < D / 4; ++s)
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(L.dk.at(16 * wave + ln, 4 * s + lg), L.Vb[4 * s + lg][ln], c, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) L.Y[16 * wave + 4 * lg + i][ln] = c[i];
  }
  __syncthreads();

  if constexpr (I4) {
    float* sq = &L.Gp[0][0][0];  // scales in record order: basis vectors, centroid, tokens
    // group scales: the waves take the basis vectors and the centroid, the
    // first P threads their token's coefficient row
    for (int gi = wave; gi < r + 1; gi += 4) {
      float m = 0.f;
      for (int row = lane; row < D; row += 64) m = fmaxf(m, fabsf(gi == r ? L.mu[row] : L.Vb[row][gi]));
      for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      if (lane == 0) sq[gi] = bf16_to_f32(f32_to_bf16(m / (gi == r ? 127.f : 7.f)));
    }
    if (tid < P) {
      float m = 0.f;
      for (int rho = 0; rho < r; ++rho) m = fmaxf(m, fabsf(L.Y[tid][rho]));
      sq[r + 1 + tid] = bf16_to_f32(f32_to_bf16(m / 127.f));
    }
    __syncthreads();
    auto code = [](float x, float s, float Lv) -> int {
      if (!(s > 0.f)) return 0;
      return (int)fminf(fmaxf(__builtin_rintf(x / s), -Lv), Lv);
    };
    uint8_t* rec = a.sum_pool + ((int64_t)blk * a.Hkv + h) * a.rec_bytes;
    constexpr int WPR = D / 8;  // 32-bit words per nibble row
    for (int t = tid; t < (r + 2) * WPR; t += 256) {
      const int row = t / WPR, wi = t - row * WPR;
      const int kg = wi / (D / 32), st = wi - kg * (D / 32);
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int el = st * 32 + kg * 8 + e;
        uint32_t nib;
        if (row < r) {
          nib = (uint32_t)(code(L.Vb[el][row], sq[row], 7.f) + 8);
        } else {
          const uint32_t byte = (uint32_t)(code(L.mu[el], sq[r], 127.f) + 128);
          nib = row == r ? byte >> 4 : byte & 15u;
        }
        word |= nib << (4 * ((e & 1) ? 4 + (e >> 1) : (e >> 1)));
      }
      *reinterpret_cast<uint32_t*>(rec + row * (D / 2) + wi * 4) = word;
    }
    uint8_t* crec = rec + (r + 2) * (D / 2);
    for (int e = tid; e < P * r; e += 256) {
      const int i = e / r, rho = e - i * r;
      crec[e] = (uint8_t)(code(L.Y[i][rho], sq[r + 1 + i], 127.f) + 128);
    }
    bf16_t* srec = reinterpret_cast<bf16_t*>(crec + P * r);
    for (int t = tid; t < 1 + r + P; t += 256) srec[t] = f32_to_bf16(sq[t]);
    for (int t = (r + 2) * (D / 2) + P * r + 2 * (1 + r + P) + tid; t < a.rec_bytes; t += 256) rec[t] = 0;
    return;
  }
  T* rec = reinterpret_cast<T*>(a.sum_pool) + ((int64_t)blk * a.Hkv + h) * a.rec_elems;
  for (int d0 = tid; d0 < D; d0 += 256) rec[d0] = Elem<T>::from_f32(L.mu[d0]);
  for (int e = tid; e < r * D; e += 256) {
    const int rho = e / D, d0 = e - rho * D;
    rec[D + e] = Elem<T>::from_f32(L.Vb[d0][rho]);
  }
  T* crec = rec + (int64_t)D * (1 + r);
  for (int e = tid; e < P * r; e += 256) {
    const int i = e / r, rho = e - i * r;
    crec[e] = Elem<T>::from_f32(L.Y[i][rho]);
  }
}

namespace {
template <typename T, int D, bool I4>
void launch_p(const BuildArgs& a, dim3 grid, hipStream_t stream) {
  switch (a.P) {
    case 16: hipLaunchKernelGGL((build_kernel<T, D, 16, I4>), grid, dim3(256), 0, stream, a); break;
    case 32: hipLaunchKernelGGL((build_kernel<T, D, 32, I4>), grid, dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL((build_kernel<T, D, 64, I4>), grid, dim3(256), 0, stream, a); break;
  }
}
}  // namespace

hipError_t launch_build(const BuildArgs& a, int dtype, int D, bool i4, hipStream_t stream) {
  dim3 grid(a.n, a.Hkv);
  if (dtype == 0 && i4) {
    if (D == 64) launch_p<bf16_t, 64, true>(a, grid, stream);
    else launch_p<bf16_t, 128, true>(a, grid, stream);
  } else if (dtype == 0) {
    if (D == 64) launch_p<bf16_t, 64, false>(a, grid, stream);
    else launch_p<bf16_t, 128, false>(a, grid, stream);
  } else {
    if (D == 64) launch_p<float, 64, false>(a, grid, stream);
    else launch_p<float, 128, false>(a, grid, stream);
  }
  return hipGetLastError();
}

}  // namespace locks

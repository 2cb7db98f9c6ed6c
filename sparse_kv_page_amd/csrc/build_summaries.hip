// (a1) Summary build, [Locks] §3-§4: for one (physical block, KV head) tile of
// P keys, fit
//   mu = (1/P) sum_i k_i,  D = K - 1 mu^T,  H = D^T D (d x d),
//   V  = top-r eigenvectors of H,  C = D V,
// and store (mu, V^T, C) in the summary record.
//
// One workgroup (4 waves) per tile, everything in LDS and registers:
//  1. K is staged transposed in LDS; mu is a plain fp32 mean.
//  2. Gram on the matrix cores. bf16 keys: H = K^T K - P mu mu^T with
//     v_mfma_f32_16x16x16_bf16 (exact bf16 products, fp32 accumulation);
//     fp32 keys are centred first and use v_mfma_f32_16x16x4_f32. Wave w
//     computes the 16-row tiles it owns against every column tile; because H
//     is symmetric the MFMA output registers already are the A operand of
//     H X for those rows, with the k index permuted as
//     k(step = 4*tile + i, lane group lg) = 16*tile + 4*lg + i.
//     H therefore never leaves registers.
//  3. Subspace iteration on a 16-column block X: Y = H X (fp32 MFMA), then
//     X = Y R^-1 from a Cholesky factor of the column-scaled Gram Y^T Y
//     (columns that collapse are replaced by fresh pseudo-random vectors).
//     Each pass has two workgroup barriers: the waves' partial Grams meet in
//     LDS, then every wave factors the 16 x 16 Gram and inverts the factor
//     in registers (lane l holds row l, broadcasts by readlane) and forms its
//     own rows of X on the matrix cores.
//  4. A second Cholesky-QR pass, then Rayleigh-Ritz: T = X^T H X (16 x 16)
//     diagonalised by parallel cyclic Jacobi (8 disjoint rotations per
//     round applied in one pass, stopping once the off-diagonal mass is
//     negligible); the r largest Ritz pairs give V = X W_r, each column
//     sign-fixed so its largest-magnitude entry is positive (lowest index on
//     ties).
//  5. C = D V in fp32 from the unrounded V; mu, V, C are rounded to the
//     summary dtype independently. Quantized ("i4") records, [Locks] §4 and
//     App. C.7: per group (the centroid, each basis vector, each token's
//     coefficient row) scale = bf16(max|x| / L), L = 127 for the 8-bit
//     centroid and coefficients and 7 for the 4-bit basis, and code =
//     round-half-even(x / scale), all in fp32 (correctly rounded division).
#include "common.h"
#include "kernels.h"

namespace locks {

constexpr int kBuildIters = 10;   // subspace iterations
constexpr int kJacobiSweeps = 8;  // sweeps of the 16 x 16 Rayleigh-Ritz problem
constexpr int kBlk = 16;          // block size of the subspace iteration

namespace {

__device__ __forceinline__ float hash_unit(uint32_t a, uint32_t b, uint32_t salt) {
  uint32_t x = a * 0x9E3779B1u ^ (b + 97u * salt) * 0x85EBCA77u;
  x ^= x >> 15; x *= 0x2C1B3C6Du;
  x ^= x >> 12; x *= 0x297A2D39u;
  x ^= x >> 15;
  return (float)(x >> 8) * (1.0f / 8388608.0f) - 1.0f;  // [-1, 1)
}

template <typename T>
struct GramOp;

template <>
struct GramOp<bf16_t> {
  static constexpr int kStep = 16;  // tokens per MFMA
  // kt row r holds the keys of dimension r over tokens (stride in elements)
  static __device__ __forceinline__ f32x4_t mfma(const bf16_t* kt, int stride, int ra, int rb, int tok0,
                                                 int lane, f32x4_t c) {
    const int t = tok0 + 4 * (lane >> 4);
    const bf16x4_t av = *reinterpret_cast<const bf16x4_t*>(kt + (ra + (lane & 15)) * stride + t);
    const bf16x4_t bv = *reinterpret_cast<const bf16x4_t*>(kt + (rb + (lane & 15)) * stride + t);
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bv, c, 0, 0, 0);
  }
};

template <>
struct GramOp<float> {
  static constexpr int kStep = 4;
  static __device__ __forceinline__ f32x4_t mfma(const float* kt, int stride, int ra, int rb, int tok0,
                                                 int lane, f32x4_t c) {
    const int t = tok0 + (lane >> 4);
    const float av = kt[(ra + (lane & 15)) * stride + t];
    const float bv = kt[(rb + (lane & 15)) * stride + t];
    return __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, c, 0, 0, 0);
  }
};

}  // namespace

template <typename T, int D, bool I4>
__global__ __launch_bounds__(256) void build_kernel(BuildArgs a) {
  constexpr int NT = D / 16;          // row tiles of H
  constexpr int RTW = NT / 4;         // row tiles per wave
  constexpr int KT_STRIDE = 64 + 4;   // LDS row stride of the transposed keys
  __shared__ __attribute__((aligned(16))) T kt[D * KT_STRIDE];
  __shared__ float mu[D];
  __shared__ __attribute__((aligned(16))) float X[D][kBlk];
  __shared__ __attribute__((aligned(16))) float Y[D][kBlk];
  __shared__ __attribute__((aligned(16))) float Mp[4][kBlk][kBlk];
  __shared__ __attribute__((aligned(16))) float RiW[4][kBlk][kBlk];  // each wave's copy of R^-1
  __shared__ float Ms[2][kBlk][kBlk + 1];  // Rayleigh quotient, ping-pong
  __shared__ float Wm[2][kBlk][kBlk + 1];  // its eigenvectors, ping-pong
  __shared__ float jsc[kBlk], joc[kBlk];   // rotation of the index's pair: self / other coefficient
  __shared__ int jpt[kBlk];                // partner index
  __shared__ int order[kBlk];
  __shared__ int cur_s;  // which Ms / Wm buffer holds the result

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = blockIdx.y;
  const int P = a.P, r = a.r;
  const int blk = a.block_ids[blockIdx.x];
  if (blk < 0 || (int64_t)blk >= a.num_blocks) return;  // uniform for the workgroup
  const T* tile = reinterpret_cast<const T*>(a.k_pool) + ((int64_t)blk * a.Hkv + h) * (int64_t)P * D;

  // ---- 1. keys -> LDS (transposed), centroid ----
  {
    constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
    const int chunks = P * D / EPC;
    for (int c = tid; c < chunks; c += 256) {
      const int e0 = c * EPC;
      const int i = e0 / D;
      const int a0 = e0 - i * D;
      const u32x4_t w = *reinterpret_cast<const u32x4_t*>(tile + e0);
      const T* v = reinterpret_cast<const T*>(&w);
#pragma unroll
      for (int x = 0; x < EPC; ++x) kt[(a0 + x) * KT_STRIDE + i] = v[x];
    }
  }
  __syncthreads();
  for (int d0 = tid; d0 < D; d0 += 256) {
    float s = 0.f;
    for (int i = 0; i < P; ++i) s += Elem<T>::load(&kt[d0 * KT_STRIDE + i]);
    mu[d0] = s / (float)P;
  }
  __syncthreads();
  if constexpr (sizeof(T) == 4) {  // fp32 keys: centre in place
    for (int e = tid; e < D * P; e += 256) {
      const int d0 = e / P, i = e - d0 * P;
      kt[d0 * KT_STRIDE + i] -= mu[d0];
    }
    __syncthreads();
  }

  // ---- 2. Gram matrix: hreg[t][c][i] = H[16*tc + lane%16][16*c + 4*(lane/16) + i], tc = wave*RTW + t ----
  f32x4_t hreg[RTW][NT];
#pragma unroll
  for (int t = 0; t < RTW; ++t) {
    const int tc = wave * RTW + t;
#pragma unroll
    for (int c = 0; c < NT; ++c) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      for (int k0 = 0; k0 < P; k0 += GramOp<T>::kStep)
        acc = GramOp<T>::mfma(kt, KT_STRIDE, 16 * c, 16 * tc, k0, lane, acc);
      if constexpr (sizeof(T) == 2) {
        const float mrow = mu[16 * tc + (lane & 15)] * (float)P;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] -= mrow * mu[16 * c + 4 * (lane >> 4) + i];
      }
      hreg[t][c] = acc;
    }
  }

  // helpers ---------------------------------------------------------------
  // Y = H X for this wave's rows; ytile[t][i] = Y[16*tc + 4*(lane/16) + i][lane%16]
  auto matmul_hx = [&](f32x4_t* ytile) {
#pragma unroll
    for (int t = 0; t < RTW; ++t) ytile[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NT; ++c) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float bx = X[16 * c + 4 * (lane >> 4) + i][lane & 15];
#pragma unroll
        for (int t = 0; t < RTW; ++t)
          ytile[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(hreg[t][c][i], bx, ytile[t], 0, 0, 0);
      }
    }
  };
  // partial Gram of the rows in `rows` (same layout as ytile) against `cols`
  auto partial_gram = [&](const f32x4_t* rows, const f32x4_t* cols) {
    f32x4_t m = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < RTW; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) m = __builtin_amdgcn_mfma_f32_16x16x4f32(rows[t][i], cols[t][i], m, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) Mp[wave][4 * (lane >> 4) + i][lane & 15] = m[i];
  };
  auto load_x_tiles = [&](f32x4_t* xt) {
#pragma unroll
    for (int t = 0; t < RTW; ++t) {
      const int tc = wave * RTW + t;
#pragma unroll
      for (int i = 0; i < 4; ++i) xt[t][i] = X[16 * tc + 4 * (lane >> 4) + i][lane & 15];
    }
  };
  auto store_y_tiles = [&](const f32x4_t* yt) {
#pragma unroll
    for (int t = 0; t < RTW; ++t) {
      const int tc = wave * RTW + t;
#pragma unroll
      for (int i = 0; i < 4; ++i) Y[16 * tc + 4 * (lane >> 4) + i][lane & 15] = yt[t][i];
    }
  };
  // Sum Mp into Ms[0] (wave 0), symmetrised.
  auto reduce_gram = [&]() {
    if (wave == 0) {
      for (int e = lane; e < kBlk * kBlk; e += 64) {
        const int i = e / kBlk, j = e % kBlk;
        const float v = Mp[0][i][j] + Mp[1][i][j] + Mp[2][i][j] + Mp[3][i][j];
        const float vt = Mp[0][j][i] + Mp[1][j][i] + Mp[2][j][i] + Mp[3][j][i];
        Ms[0][i][j] = 0.5f * (v + vt);
      }
    }
  };
  auto rdl = [](float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); };
  // Every wave, in registers (lane l holds row l & 15 of the block Gram M in
  // a[]): column scaling S (columns with a vanishing norm are dead), Cholesky
  // S M S = L L^T (right-looking; a column whose pivot vanishes is dead and
  // gets L = unit column), then L^-1 column by column (lane c forms column c)
  // and Ri = S L^-T with dead columns zeroed, written to this wave's RiW.
  // Returns the dead-column mask (uniform).
  auto chol_rinv = [&](float* am) -> uint32_t {
    const int row = lane & 15;
    float sd[kBlk];
    float dmax = 0.f;
#pragma unroll
    for (int j = 0; j < kBlk; ++j) {
      sd[j] = rdl(am[j], j);  // diagonal
      dmax = fmaxf(dmax, sd[j]);
    }
    uint32_t dead = 0u;
#pragma unroll
    for (int j = 0; j < kBlk; ++j) {
      const bool dd = !(sd[j] > 1e-30f * fmaxf(dmax, 1e-30f));
      dead |= dd ? 1u << j : 0u;
      sd[j] = dd ? 0.f : __builtin_amdgcn_rsqf(sd[j]);
    }
    float srow = 0.f;
#pragma unroll
    for (int j = 0; j < kBlk; ++j) srow = row == j ? sd[j] : srow;
#pragma unroll
    for (int c = 0; c < kBlk; ++c) am[c] *= srow * sd[c];
    // the chain of pivots uses the hardware reciprocal square root (about
    // 1 ulp): the factor only has to orthonormalise the block to fp32 level
    float invd[kBlk];  // 1 / L[j][j]
#pragma unroll
    for (int j = 0; j < kBlk; ++j) {
      const float vjj = rdl(am[j], j);
      const bool ok = vjj > 1e-12f && !((dead >> j) & 1u);
      const float rj = ok ? __builtin_amdgcn_rsqf(vjj) : 1.0f;
      invd[j] = rj;
      const float lij = row > j ? (ok ? am[j] * rj : 0.f) : (row == j ? (ok ? vjj * rj : 1.0f) : 0.f);
      am[j] = lij;
      dead |= ok ? 0u : 1u << j;
#pragma unroll
      for (int k = j + 1; k < kBlk; ++k) am[k] = fmaf(-lij, rdl(lij, k), am[k]);
    }
    // li[i] = (L^-1)[i][row]
    float li[kBlk];
#pragma unroll
    for (int i = 0; i < kBlk; ++i) {
      float t = row == i ? 1.f : 0.f;
#pragma unroll
      for (int k = 0; k < i; ++k) t = fmaf(-rdl(am[k], i), li[k], t);
      li[i] = t * invd[i];
    }
    // Ri[row][j] = s_row * (L^-1)[j][row] for j >= row, live j
    if (lane < kBlk) {
#pragma unroll
      for (int j = 0; j < kBlk; ++j) RiW[wave][row][j] = (j >= row && !((dead >> j) & 1u)) ? srow * li[j] : 0.f;
    }
    return dead;
  };
  // One Cholesky-QR pass of the block Y whose rows owned by this wave are in
  // yt: X = Y Ri for the wave's rows (matrix cores), dead columns replaced by
  // fresh pseudo-random vectors, X -> LDS. Two workgroup barriers.
  auto cholqr = [&](const f32x4_t* yt, uint32_t salt) {
    store_y_tiles(yt);  // read back below by this wave only
    partial_gram(yt, yt);
    __syncthreads();
    float am[kBlk];
    {
      const int row = lane & 15;
#pragma unroll
      for (int c = 0; c < kBlk; c += 4) {
        f32x4_t v = *reinterpret_cast<const f32x4_t*>(&Mp[0][row][c]);
#pragma unroll
        for (int w = 1; w < 4; ++w) {
          const f32x4_t u = *reinterpret_cast<const f32x4_t*>(&Mp[w][row][c]);
          v[0] += u[0]; v[1] += u[1]; v[2] += u[2]; v[3] += u[3];
        }
        am[c] = v[0]; am[c + 1] = v[1]; am[c + 2] = v[2]; am[c + 3] = v[3];
      }
    }
    const uint32_t dead = chol_rinv(am);
    wave_lds_sync();  // RiW[wave] and this wave's Y rows are visible to the wave
    const bool dcol = (dead >> (lane & 15)) & 1u;
#pragma unroll
    for (int t = 0; t < RTW; ++t) {
      const int tc = wave * RTW + t;
      f32x4_t x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k0 = 0; k0 < kBlk; k0 += 4)
        x = __builtin_amdgcn_mfma_f32_16x16x4f32(Y[16 * tc + (lane & 15)][k0 + (lane >> 4)],
                                                 RiW[wave][k0 + (lane >> 4)][lane & 15], x, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * tc + 4 * (lane >> 4) + i;
        X[row][lane & 15] = dcol ? hash_unit((uint32_t)row, (uint32_t)(lane & 15), salt) : x[i];
      }
    }
    __syncthreads();  // X complete
  };

  // ---- 3. subspace iteration ----
  f32x4_t yt[RTW];
#pragma unroll
  for (int t = 0; t < RTW; ++t) {
    const int tc = wave * RTW + t;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      yt[t][i] = hash_unit((uint32_t)(16 * tc + 4 * (lane >> 4) + i), (uint32_t)(lane & 15), 1u);
  }
  cholqr(yt, 2u);
  for (int it = 0; it < kBuildIters; ++it) {
    matmul_hx(yt);
    cholqr(yt, 3u + (uint32_t)it);
  }
  // second pass for orthonormality
  load_x_tiles(yt);
  cholqr(yt, 101u);

  // ---- 4. Rayleigh-Ritz: T = X^T H X, diagonalised by cyclic Jacobi ----
  int cur = 0;
  {
    f32x4_t xt[RTW];
    load_x_tiles(xt);
    matmul_hx(yt);
    partial_gram(xt, yt);
    __syncthreads();
    reduce_gram();  // Ms[0] = T (symmetrised)
    if (wave == 0) {
      for (int e = lane; e < kBlk * kBlk; e += 64) Wm[0][e / kBlk][e % kBlk] = (e / kBlk == e % kBlk) ? 1.f : 0.f;
      wave_lds_sync();
      // Each round rotates 8 disjoint index pairs (round-robin schedule) at
      // once: T <- R T R^T, W <- W R^T in one pass per element into the other
      // buffer. A pair is rotated only while its off-diagonal entry is
      // significant both against its own diagonal entries and against 1e-7
      // of the trace (fp32 rounding leaves about one ulp of the largest
      // eigenvalue behind); the sweeps stop after one in which no pair was.
      float tr = lane < kBlk ? Ms[0][lane][lane] : 0.f;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) tr += __shfl_xor(tr, o, 64);
      const float floor_abs = 1e-7f * fabsf(tr);
      const int ey = lane & 15;  // this lane's column in the update pass
      for (int sweep = 0; sweep < kJacobiSweeps; ++sweep) {
        bool any = false;
        for (int rnd = 0; rnd < kBlk - 1; ++rnd) {
          if (lane < 8) {
            int p, q;
            if (lane == 0) { p = kBlk - 1; q = rnd; }
            else { p = (rnd + lane) % (kBlk - 1); q = (rnd - lane + (kBlk - 1)) % (kBlk - 1); }
            const float apq = Ms[cur][p][q];
            const float app = Ms[cur][p][p], aqq = Ms[cur][q][q];
            float c = 1.f, sn = 0.f;
            if (fabsf(apq) > floor_abs && fabsf(apq) > 1e-6f * sqrtf(fabsf(app * aqq))) {
              any = true;
              const float theta = (aqq - app) * __builtin_amdgcn_rcpf(2.f * apq);
              const float tt = (theta >= 0.f ? 1.f : -1.f) *
                               __builtin_amdgcn_rcpf(fabsf(theta) + sqrtf(theta * theta + 1.f));
              c = __builtin_amdgcn_rsqf(tt * tt + 1.f);
              sn = tt * c;
            }
            jsc[p] = c; joc[p] = -sn; jpt[p] = q;
            jsc[q] = c; joc[q] = sn;  jpt[q] = p;
          }
          wave_lds_sync();
          {
            const int py = jpt[ey];
            const float sy = jsc[ey], oy = joc[ey];
#pragma unroll
            for (int k = 0; k < kBlk * kBlk / 64; ++k) {
              const int x = (lane >> 4) + 4 * k;
              const int px = jpt[x];
              const float sx = jsc[x], ox = joc[x];
              Ms[cur ^ 1][x][ey] = sx * (sy * Ms[cur][x][ey] + oy * Ms[cur][x][py]) +
                                   ox * (sy * Ms[cur][px][ey] + oy * Ms[cur][px][py]);
              Wm[cur ^ 1][x][ey] = sy * Wm[cur][x][ey] + oy * Wm[cur][x][py];
            }
          }
          wave_lds_sync();
          cur ^= 1;
        }
        if (!__builtin_amdgcn_ballot_w64(any)) break;
      }
      // descending order of the Ritz values, ties by index
      if (lane < kBlk) {
        const float v = Ms[cur][lane][lane];
        int rank = 0;
        for (int j = 0; j < kBlk; ++j) {
          const float u = Ms[cur][j][j];
          rank += (u > v || (u == v && j < lane)) ? 1 : 0;
        }
        order[rank] = lane;
      }
    }
    if (tid == 0) cur_s = cur;
    __syncthreads();
  }
  const int cw = cur_s;
  // V = X W[:, order[0..r-1]] into Y[:, 0..r-1]
  for (int e = tid; e < D * kBlk; e += 256) {
    const int row = e / kBlk, rho = e % kBlk;
    if (rho < r) {
      const int col = order[rho];
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < kBlk; ++j) s += X[row][j] * Wm[cw][j][col];
      Y[row][rho] = s;
    }
  }
  __syncthreads();
  // sign: largest-magnitude entry positive (lowest index on ties)
  for (int rho = wave; rho < r; rho += 4) {
    float best = -1.f;
    int arg = D;
    for (int row = lane; row < D; row += 64) {
      const float m = fabsf(Y[row][rho]);
      if (m > best) { best = m; arg = row; }
    }
    for (int o = 32; o > 0; o >>= 1) {
      const float ob = __shfl_xor(best, o, 64);
      const int oa = __shfl_xor(arg, o, 64);
      if (ob > best || (ob == best && oa < arg)) { best = ob; arg = oa; }
    }
    if (arg >= D) arg = 0;  // only when every entry is NaN
    const float sg = Y[arg][rho] < 0.f ? -1.f : 1.f;
    wave_lds_sync();
    for (int row = lane; row < D; row += 64) Y[row][rho] *= sg;
  }
  __syncthreads();

  // ---- 5. C = D V and the record ----
  if constexpr (I4) {
    float* Cs = &X[0][0];      // C [P][r]; X is free from here on
    float* sq = &Mp[0][0][0];  // scales in record order: basis vectors, centroid, tokens
    for (int e = tid; e < P * r; e += 256) {
      const int i = e / r, rho = e - i * r;
      float s = 0.f;
      for (int d0 = 0; d0 < D; ++d0) s = fmaf(Elem<T>::load(&kt[d0 * KT_STRIDE + i]) - mu[d0], Y[d0][rho], s);
      Cs[e] = s;
    }
    __syncthreads();
    // group scales: the waves take the basis vectors and the centroid, the
    // first P threads their token's coefficient row
    for (int gi = wave; gi < r + 1; gi += 4) {
      float m = 0.f;
      for (int row = lane; row < D; row += 64) m = fmaxf(m, fabsf(gi == r ? mu[row] : Y[row][gi]));
      for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      if (lane == 0) sq[gi] = bf16_to_f32(f32_to_bf16(m / (gi == r ? 127.f : 7.f)));
    }
    if (tid < P) {
      float m = 0.f;
      for (int rho = 0; rho < r; ++rho) m = fmaxf(m, fabsf(Cs[tid * r + rho]));
      sq[r + 1 + tid] = bf16_to_f32(f32_to_bf16(m / 127.f));
    }
    __syncthreads();
    auto code = [](float x, float s, float L) -> int {
      if (!(s > 0.f)) return 0;
      return (int)fminf(fmaxf(__builtin_rintf(x / s), -L), L);
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
          nib = (uint32_t)(code(Y[el][row], sq[row], 7.f) + 8);
        } else {
          const uint32_t byte = (uint32_t)(code(mu[el], sq[r], 127.f) + 128);
          nib = row == r ? byte >> 4 : byte & 15u;
        }
        word |= nib << (4 * ((e & 1) ? 4 + (e >> 1) : (e >> 1)));
      }
      *reinterpret_cast<uint32_t*>(rec + row * (D / 2) + wi * 4) = word;
    }
    uint8_t* crec = rec + (r + 2) * (D / 2);
    for (int e = tid; e < P * r; e += 256) crec[e] = (uint8_t)(code(Cs[e], sq[r + 1 + e / r], 127.f) + 128);
    bf16_t* srec = reinterpret_cast<bf16_t*>(crec + P * r);
    for (int t = tid; t < 1 + r + P; t += 256) srec[t] = f32_to_bf16(sq[t]);
    for (int t = (r + 2) * (D / 2) + P * r + 2 * (1 + r + P) + tid; t < a.rec_bytes; t += 256) rec[t] = 0;
    return;
  }
  T* rec = reinterpret_cast<T*>(a.sum_pool) + ((int64_t)blk * a.Hkv + h) * a.rec_elems;
  for (int d0 = tid; d0 < D; d0 += 256) rec[d0] = Elem<T>::from_f32(mu[d0]);
  for (int e = tid; e < r * D; e += 256) {
    const int rho = e / D, d0 = e - rho * D;
    rec[D + e] = Elem<T>::from_f32(Y[d0][rho]);
  }
  T* crec = rec + (int64_t)D * (1 + r);
  for (int e = tid; e < P * r; e += 256) {
    const int i = e / r, rho = e - i * r;
    float s = 0.f;
    for (int d0 = 0; d0 < D; ++d0) {
      float kv = Elem<T>::load(&kt[d0 * KT_STRIDE + i]);
      if constexpr (sizeof(T) == 2) kv -= mu[d0];
      s = fmaf(kv, Y[d0][rho], s);
    }
    crec[e] = Elem<T>::from_f32(s);
  }
}

hipError_t launch_build(const BuildArgs& a, int dtype, int D, bool i4, hipStream_t stream) {
  dim3 grid(a.n, a.Hkv);
  if (dtype == 0 && i4) {
    if (D == 64) hipLaunchKernelGGL((build_kernel<bf16_t, 64, true>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((build_kernel<bf16_t, 128, true>), grid, dim3(256), 0, stream, a);
  } else if (dtype == 0) {
    if (D == 64) hipLaunchKernelGGL((build_kernel<bf16_t, 64, false>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((build_kernel<bf16_t, 128, false>), grid, dim3(256), 0, stream, a);
  } else {
    if (D == 64) hipLaunchKernelGGL((build_kernel<float, 64, false>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((build_kernel<float, 128, false>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace locks

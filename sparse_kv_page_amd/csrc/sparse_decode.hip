// (a5) Sparse paged decode attention over the selected pages, [Locks] §2:
// the softmax is renormalised over the tokens of the selected pages only and
// uses the original K/V.
//
// Split-K: a workgroup handles `pages_per_split` consecutive slots of one
// (sequence, KV head)'s selected list; each of its 4 waves takes one page at
// a time for all G query heads of the group.
//   scores  S = K q^T on the matrix cores (16 tokens x 16 head-columns per
//           MFMA, G columns used), masked past the page's valid tokens,
//   online softmax in base 2 (running max / sum per head),
//   output  o_g += p_g(i) v_i on the VALU: each lane owns an 8-wide slice of
//           d for a quarter (d=128) or an eighth (d=64) of the tokens, so the
//           V rows are read with coalesced 16-byte loads.
// The waves' states merge through LDS; each workgroup writes one normalised
// partial (o, lse) per head, and merge_kernel combines the splits by LSE.
#include "common.h"
#include "kernels.h"

namespace locks {

constexpr int kDecWaves = 4;

namespace {

template <typename T, int D>
struct QkMfma;

template <int D>
struct QkMfma<bf16_t, D> {
  static constexpr int kSteps = D / 32;
  using Op = bf16x8_t;
  static __device__ __forceinline__ Op load(const bf16_t* row, int s, int kg, bool ok) {
    if (!ok) return bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    return *reinterpret_cast<const bf16x8_t*>(row + s * 32 + kg * 8);
  }
  static __device__ __forceinline__ f32x4_t mfma(Op a, Op b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <int D>
struct QkMfma<float, D> {
  static constexpr int kSteps = D / 4;
  using Op = float;
  static __device__ __forceinline__ Op load(const float* row, int s, int kg, bool ok) {
    return ok ? row[s * 4 + kg] : 0.f;
  }
  static __device__ __forceinline__ f32x4_t mfma(Op a, Op b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// 8 consecutive elements of a V row as floats.
__device__ __forceinline__ void load8(const bf16_t* p, float* v) {
  const u32x4_t w = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) { v[2 * e] = bf16_lo(w[e]); v[2 * e + 1] = bf16_hi(w[e]); }
}
__device__ __forceinline__ void load8(const float* p, float* v) {
  const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
  const f32x4_t b = *reinterpret_cast<const f32x4_t*>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) { v[e] = a[e]; v[4 + e] = b[e]; }
}

}  // namespace

template <typename T, int D>
__global__ __launch_bounds__(256) void sparse_decode_kernel(DecodeArgs a) {
  using Q = QkMfma<T, D>;
  constexpr int NS = D / 8;         // 8-wide d slices
  constexpr int TPS = 64 / NS;      // tokens per PV step
  __shared__ __attribute__((aligned(16))) float pbuf[kDecWaves][64][8];
  __shared__ float abuf[kDecWaves][8];
  __shared__ __attribute__((aligned(16))) float mo[kDecWaves][8][D];
  __shared__ float mm[kDecWaves][8];
  __shared__ float ml[kDecWaves][8];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int P = a.P, G = a.G;
  const int Hq = a.Hkv * G;
  const int Tl = clamp_len(a.seq_lens[b], a.max_pages, P);
  const int J = (Tl + P - 1) / P;
  const int32_t* sel = a.selected + ((int64_t)b * a.Hkv + h) * a.k;
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;
  const T* kp = reinterpret_cast<const T*>(a.k_pool);
  const T* vp = reinterpret_cast<const T*>(a.v_pool);
  const float zscale = a.scale * kLog2e;

  // MFMA lane roles: n = head column / token row in tile, kg = k group
  const int n = lane & 15;
  const int kg = lane >> 4;
  typename Q::Op qb[Q::kSteps];
  {
    const T* qrow = reinterpret_cast<const T*>(a.q) + ((int64_t)b * Hq + (int64_t)h * G + (n < G ? n : 0)) * D;
#pragma unroll
    for (int s = 0; s < Q::kSteps; ++s) qb[s] = Q::load(qrow, s, kg, n < G);
  }
  // PV lane roles
  const int tg = lane / NS;
  const int ts = lane % NS;

  float m_run = -INFINITY, l_run = 0.f;  // valid in lanes with n < G
  float o[8][8];
#pragma unroll
  for (int g = 0; g < 8; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[g][e] = 0.f;

  const int slot_end = min((split + 1) * a.pages_per_split, a.k);
  for (int slot = split * a.pages_per_split + wave; slot < slot_end; slot += kDecWaves) {
    const int j = sel[slot];
    if (j < 0 || j >= J) continue;
    const int blk = bt[j];
    if (blk < 0 || (int64_t)blk >= a.num_blocks) continue;
    int ntok = Tl - j * P;
    ntok = ntok > P ? P : ntok;
    const T* ktile = kp + ((int64_t)blk * a.Hkv + h) * (int64_t)P * D;
    const T* vtile = vp + ((int64_t)blk * a.Hkv + h) * (int64_t)P * D;

    // ---- S = K q^T, 16 tokens per tile ----
    f32x4_t acc[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      acc[tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      if (tt * 16 < P) {
        const int tok = tt * 16 + n;
        const T* krow = ktile + (int64_t)tok * D;
#pragma unroll
        for (int s = 0; s < Q::kSteps; ++s) acc[tt] = Q::mfma(Q::load(krow, s, kg, tok < ntok), qb[s], acc[tt]);
      }
    }
    // lane holds S[token = tt*16 + 4*kg + i][head n]
    float pmax = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = tt * 16 + 4 * kg + i;
        const float z = (tt * 16 < P && tok < ntok) ? acc[tt][i] * zscale : -INFINITY;
        acc[tt][i] = z;
        pmax = fmaxf(pmax, z);
      }
    pmax = fmaxf(pmax, shfl_xor(pmax, 16));
    pmax = fmaxf(pmax, shfl_xor(pmax, 32));
    const float m_new = fmaxf(m_run, pmax);  // finite: ntok >= 1
    const float alpha = exp2_fast(m_run - m_new);  // m_run = -inf -> 0
    float psum = 0.f;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = tt * 16 + 4 * kg + i;
        if (tt * 16 < P) {
          const float p = exp2_fast(acc[tt][i] - m_new);
          psum += p;
          if (n < G) pbuf[wave][tok][n] = p;
        }
      }
    psum += shfl_xor(psum, 16);
    psum += shfl_xor(psum, 32);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (kg == 0 && n < G) abuf[wave][n] = alpha;
    wave_lds_sync();

    // ---- o_g = alpha_g o_g + sum_i p_g(i) v_i ----
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      if (g < G) {
        const float al = abuf[wave][g];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[g][e] *= al;
      }
    }
    for (int i = tg; i < ntok; i += TPS) {
      float v[8];
      load8(vtile + (int64_t)i * D + ts * 8, v);
      const f32x4_t pa = *reinterpret_cast<const f32x4_t*>(&pbuf[wave][i][0]);
      const f32x4_t pb = *reinterpret_cast<const f32x4_t*>(&pbuf[wave][i][4]);
      const float pg[8] = {pa[0], pa[1], pa[2], pa[3], pb[0], pb[1], pb[2], pb[3]};
#pragma unroll
      for (int g = 0; g < 8; ++g)
        if (g < G)
#pragma unroll
          for (int e = 0; e < 8; ++e) o[g][e] = fmaf(pg[g], v[e], o[g][e]);
    }
    wave_lds_sync();
  }

  // ---- reduce the token groups of each wave, then merge the waves ----
#pragma unroll
  for (int g = 0; g < 8; ++g)
    if (g < G)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        for (int off = NS; off < 64; off <<= 1) o[g][e] += shfl_xor(o[g][e], off);
  if (tg == 0) {
#pragma unroll
    for (int g = 0; g < 8; ++g)
      if (g < G)
#pragma unroll
        for (int e = 0; e < 8; ++e) mo[wave][g][ts * 8 + e] = o[g][e];
  }
  if (kg == 0 && n < G) { mm[wave][n] = m_run; ml[wave][n] = l_run; }
  __syncthreads();

  for (int x = threadIdx.x; x < G * D; x += 256) {
    const int g = x / D;
    const int e = x - g * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, mm[w][g]);
    float L = 0.f, O = 0.f;
    if (M > -INFINITY) {
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) {
        if (mm[w][g] > -INFINITY) {
          const float c = exp2_fast(mm[w][g] - M);
          L += c * ml[w][g];
          O += c * mo[w][g][e];
        }
      }
    }
    const int64_t row = ((int64_t)b * Hq + (int64_t)h * G + g) * a.splits + split;
    a.part_o[row * D + e] = L > 0.f ? O / L : 0.f;
    if (e == 0) a.part_lse[row] = L > 0.f ? (M + log2_fast(L)) * kLn2 : -INFINITY;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(D) void merge_kernel(DecodeArgs a) {
  const int row = blockIdx.x;  // b * Hq + head
  const int e = threadIdx.x;
  const float* pl = a.part_lse + (int64_t)row * a.splits;
  const float* po = a.part_o + (int64_t)row * a.splits * D;
  float M = -INFINITY;
  for (int s = 0; s < a.splits; ++s) M = fmaxf(M, pl[s]);
  float L = 0.f, O = 0.f;
  if (M > -INFINITY) {
    for (int s = 0; s < a.splits; ++s) {
      if (pl[s] > -INFINITY) {
        const float c = exp2_fast((pl[s] - M) * kLog2e);
        L += c;
        O += c * po[(int64_t)s * D + e];
      }
    }
  }
  T* out = reinterpret_cast<T*>(a.out) + (int64_t)row * D;
  out[e] = Elem<T>::from_f32(L > 0.f ? O / L : 0.f);
  if (a.lse && e == 0) a.lse[row] = L > 0.f ? M + log2_fast(L) * kLn2 : -INFINITY;
}

hipError_t launch_sparse_decode(const DecodeArgs& a, int dtype, int D, int batch, hipStream_t stream) {
  dim3 grid(a.splits, a.Hkv, batch);
  const int rows = batch * a.Hkv * a.G;
#define LAUNCH(T, DD)                                                                     \
  do {                                                                                    \
    hipLaunchKernelGGL((sparse_decode_kernel<T, DD>), grid, dim3(256), 0, stream, a);     \
    hipError_t e_ = hipGetLastError();                                                    \
    if (e_ != hipSuccess) return e_;                                                      \
    hipLaunchKernelGGL((merge_kernel<T, DD>), dim3(rows), dim3(DD), 0, stream, a);        \
  } while (0)
  if (dtype == 0) {
    if (D == 64) LAUNCH(bf16_t, 64); else LAUNCH(bf16_t, 128);
  } else {
    if (D == 64) LAUNCH(float, 64); else LAUNCH(float, 128);
  }
#undef LAUNCH
  return hipGetLastError();
}

}  // namespace locks

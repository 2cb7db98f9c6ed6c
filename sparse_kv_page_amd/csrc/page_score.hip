// (a2) Page scoring: reconstructed page log-sum-exp of every complete page,
// [Locks] §4 Eq. (2):
//   shat_j(q_g) = (q_g . mu_j) * scale + log sum_i exp(((V_j^T q_g) . c_i) * scale)
//
// Work unit: one wave scores one page at a time for all G query heads of a
// KV head; a workgroup of 4 waves covers a chunk of pages of one
// (sequence, KV head). Summary records are streamed once with 16-byte loads.
//
// Phase A (matrix cores): the r basis rows and the centroid of the record form
// the 16 rows of an MFMA A operand (rows r+1..15 are zero) and the G query
// heads the columns of the B operand, so one 16x16 product per 32-wide slice
// of d gives w_g = V^T q_g (rows 0..r-1) and q_g . mu (row r) for all heads
// at once. bf16 x bf16 products are exact and accumulate in fp32.
// Phase B (VALU): each head owns 64/G lanes, each lane reconstructs the
// logits of P*G/64 tokens from the coefficient rows staged in LDS, and the
// page LSE is reduced across the head's lanes (max, then sum of 2^x).
#include "common.h"
#include "kernels.h"

namespace locks {

namespace {

template <typename T, int D>
struct ScoreMfma;

// bf16: v_mfma_f32_16x16x32_bf16. Lane l supplies row/col (l % 16) and the
// k-range 8*(l/16) .. +8 of each 32-wide k step.
template <int D>
struct ScoreMfma<bf16_t, D> {
  static constexpr int kSteps = D / 32;
  bf16x8_t a[kSteps];
  __device__ __forceinline__ void load_a(const bf16_t* row, bool ok, int kg) {
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      if (ok) {
        a[s] = *reinterpret_cast<const bf16x8_t*>(row + s * 32 + kg * 8);
      } else {
        a[s] = bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
  }
  static __device__ __forceinline__ void load_b(bf16x8_t* b, const bf16_t* qrow, bool ok, int kg) {
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      if (ok) b[s] = *reinterpret_cast<const bf16x8_t*>(qrow + s * 32 + kg * 8);
      else b[s] = bf16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
  using BType = bf16x8_t;
  __device__ __forceinline__ f32x4_t product(const BType* b) const {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], b[s], acc, 0, 0, 0);
    return acc;
  }
};

// fp32: v_mfma_f32_16x16x4_f32. Lane l supplies row/col (l % 16) and k = l/16
// of each 4-wide k step.
template <int D>
struct ScoreMfma<float, D> {
  static constexpr int kSteps = D / 4;
  float a[kSteps];
  __device__ __forceinline__ void load_a(const float* row, bool ok, int kg) {
#pragma unroll
    for (int s = 0; s < kSteps; ++s) a[s] = ok ? row[s * 4 + kg] : 0.f;
  }
  using BType = float;
  static __device__ __forceinline__ void load_b(float* b, const float* qrow, bool ok, int kg) {
#pragma unroll
    for (int s = 0; s < kSteps; ++s) b[s] = ok ? qrow[s * 4 + kg] : 0.f;
  }
  __device__ __forceinline__ f32x4_t product(const BType* b) const {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
    return acc;
  }
};

// Coefficient row of token i from the staged C block (P x r, row-major).
template <typename T, int RT>
__device__ __forceinline__ float logit_from_lds(const T* cb, int i, int r, const float* w) {
  float z = 0.f;
  if constexpr (RT > 0) {
    const T* row = cb + i * RT;
#pragma unroll
    for (int rho = 0; rho < RT; ++rho) z = fmaf(w[rho], Elem<T>::load(row + rho), z);
  } else {
    const T* row = cb + i * r;
#pragma unroll
    for (int rho = 0; rho < 16; ++rho)
      if (rho < r) z = fmaf(w[rho], Elem<T>::load(row + rho), z);
  }
  return z;
}

}  // namespace

constexpr int kScoreWaves = 4;
constexpr int kCBufBytes = 64 * 15 * 4;  // largest C block: P=64, r=15, fp32

template <typename T, int D, int RT>
__global__ __launch_bounds__(256) void page_score_kernel(ScoreArgs a) {
  using M = ScoreMfma<T, D>;
  constexpr int kMaxChunks = RT > 0 ? (64 * RT * (int)sizeof(T) + 1023) / 1024 : 4;
  __shared__ __attribute__((aligned(16))) float wbuf[kScoreWaves][16][16];
  __shared__ __attribute__((aligned(16))) uint8_t cbuf[kScoreWaves][kCBufBytes];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int b = blockIdx.z;
  const int h = blockIdx.y;
  const int P = a.P, r = a.r, G = a.G;
  const int Hq = a.Hkv * G;
  const int T_b = clamp_len(a.seq_lens[b], a.max_pages, P);
  const int Jc = T_b / P;
  const int p0 = (blockIdx.x * kScoreWaves + wave) * a.ppw;
  if (p0 >= Jc) return;
  const int np = min(a.ppw, Jc - p0);

  // block ids of this wave's pages: lane t holds page p0 + t
  const int32_t* bt_row = a.block_table + (int64_t)b * a.max_pages;
  int my_bid = lane < np ? bt_row[p0 + lane] : -1;

  // B operand: query heads as columns
  const int n = lane & 15;
  const int kg = lane >> 4;
  typename M::BType qb[M::kSteps];
  M::load_b(qb, reinterpret_cast<const T*>(a.q) + ((int64_t)b * Hq + (int64_t)h * G + (n < G ? n : 0)) * D,
            n < G, kg);

  // A operand rows: 0..r-1 basis rows, r centroid, others zero
  const int m = lane & 15;
  const bool row_ok = m <= r;
  const int64_t row_off = m < r ? (int64_t)D * (1 + m) : 0;
  const int64_t rec_elems = a.rec_elems;
  const int64_t c_off_bytes = (int64_t)D * (1 + r) * sizeof(T);
  const int c_bytes = P * r * (int)sizeof(T);

  // phase-B lane layout
  const int lph = 64 / G;
  const int g = lane / lph;
  const int u = lane - g * lph;
  const int tpl = (P + lph - 1) / lph;
  const float zscale = a.scale * kLog2e;
  float* out_row = a.scores + ((int64_t)b * Hq + (int64_t)h * G + g) * a.max_pages;

  auto rec_of = [&](int bid) -> const T* {
    return reinterpret_cast<const T*>(a.sum_pool) + ((int64_t)bid * a.Hkv + h) * rec_elems;
  };
  auto bid_ok = [&](int bid) { return bid >= 0 && (int64_t)bid < a.num_blocks; };

  M cur, nxt;
  u32x4_t ccur[kMaxChunks], cnxt[kMaxChunks];
  auto load_page = [&](int t, M& mm, u32x4_t* cc) {
    const int bid = __builtin_amdgcn_readlane(my_bid, t);
    const bool ok = bid_ok(bid);
    const T* rec = rec_of(ok ? bid : 0);
    mm.load_a(rec + row_off, ok && row_ok, kg);
    const uint8_t* cb = reinterpret_cast<const uint8_t*>(rec) + c_off_bytes;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      const int off = c * 1024 + lane * 16;
      if (ok && off < c_bytes) cc[c] = *reinterpret_cast<const u32x4_t*>(cb + off);
      else cc[c] = u32x4_t{0u, 0u, 0u, 0u};
    }
  };

  load_page(0, cur, ccur);
  for (int t = 0; t < np; ++t) {
    if (t + 1 < np) load_page(t + 1, nxt, cnxt);
    const int bid = __builtin_amdgcn_readlane(my_bid, t);
    const bool ok = bid_ok(bid);

    // phase A
    f32x4_t acc = cur.product(qb);
    *reinterpret_cast<f32x4_t*>(&wbuf[wave][n][kg * 4]) = acc;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      const int off = c * 1024 + lane * 16;
      if (off < c_bytes) *reinterpret_cast<u32x4_t*>(&cbuf[wave][off]) = ccur[c];
    }
    wave_lds_sync();

    // phase B
    float w[16];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      f32x4_t v = *reinterpret_cast<const f32x4_t*>(&wbuf[wave][g][q4 * 4]);
      w[q4 * 4 + 0] = v[0]; w[q4 * 4 + 1] = v[1]; w[q4 * 4 + 2] = v[2]; w[q4 * 4 + 3] = v[3];
    }
    const float mq = wbuf[wave][g][r];  // q . mu
    const T* cbt = reinterpret_cast<const T*>(&cbuf[wave][0]);
    float z[8];
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const int i = u * tpl + tt;
      z[tt] = -INFINITY;
      if (tt < tpl && i < P) {
        z[tt] = logit_from_lds<T, RT>(cbt, i, r, w) * zscale;
        mx = fmaxf(mx, z[tt]);
      }
    }
    for (int o = 1; o < lph; o <<= 1) mx = fmaxf(mx, shfl_xor(mx, o));
    float sm = 0.f;
#pragma unroll
    for (int tt = 0; tt < 8; ++tt)
      if (tt < tpl) sm += exp2_fast(z[tt] - mx);  // exp2(-inf) = 0
    for (int o = 1; o < lph; o <<= 1) sm += shfl_xor(sm, o);
    if (u == 0) {
      const float s = mq * a.scale + (mx + log2_fast(sm)) * kLn2;
      out_row[p0 + t] = ok ? s : -INFINITY;
    }
    wave_lds_sync();
    if (t + 1 < np) {
      cur = nxt;
#pragma unroll
      for (int c = 0; c < kMaxChunks; ++c) ccur[c] = cnxt[c];
    }
  }
}

#define LOCKS_SCORE_INST(T, D, RT) template __global__ void page_score_kernel<T, D, RT>(ScoreArgs);
#define LOCKS_SCORE_INST_R(T, D) \
  LOCKS_SCORE_INST(T, D, 0) LOCKS_SCORE_INST(T, D, 1) LOCKS_SCORE_INST(T, D, 2) \
  LOCKS_SCORE_INST(T, D, 4) LOCKS_SCORE_INST(T, D, 8)
LOCKS_SCORE_INST_R(bf16_t, 64)
LOCKS_SCORE_INST_R(bf16_t, 128)
LOCKS_SCORE_INST_R(float, 64)
LOCKS_SCORE_INST_R(float, 128)

hipError_t launch_page_score(const ScoreArgs& args, int dtype, int D, int batch, hipStream_t stream) {
  const int pages_per_wg = kScoreWaves * args.ppw;
  dim3 grid((args.max_pages + pages_per_wg - 1) / pages_per_wg, args.Hkv, batch);
  dim3 block(256);
  const int RT = (args.r == 1 || args.r == 2 || args.r == 4 || args.r == 8) ? args.r : 0;
#define LAUNCH(T, DD, R) \
  hipLaunchKernelGGL((page_score_kernel<T, DD, R>), grid, block, 0, stream, args)
#define LAUNCH_R(T, DD)                 \
  switch (RT) {                         \
    case 1: LAUNCH(T, DD, 1); break;    \
    case 2: LAUNCH(T, DD, 2); break;    \
    case 4: LAUNCH(T, DD, 4); break;    \
    case 8: LAUNCH(T, DD, 8); break;    \
    default: LAUNCH(T, DD, 0); break;   \
  }
  if (dtype == 0) {
    if (D == 64) { LAUNCH_R(bf16_t, 64) } else { LAUNCH_R(bf16_t, 128) }
  } else {
    if (D == 64) { LAUNCH_R(float, 64) } else { LAUNCH_R(float, 128) }
  }
#undef LAUNCH_R
#undef LAUNCH
  return hipGetLastError();
}

}  // namespace locks

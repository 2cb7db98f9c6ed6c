// (a2) Page scoring: reconstructed page log-sum-exp of every complete page,
// [Locks] §4 Eq. (2):
//   shat_j(q_g) = (q_g . mu_j) * scale + log sum_i exp(((V_j^T q_g) . c_i) * scale)
//
// Work unit: one wave scores a run of consecutive pages of one (sequence,
// KV head) for all G query heads of the group, one page per iteration, with
// the next page's record already in flight (non-temporal 16-byte loads: every
// record is read once per step). Waves per unit and pages per wave are sized
// on the host so that the whole grid is resident at once.
//
// Per page:
//  A (matrix cores): the r basis rows and the centroid of the record are the
//    first r+1 rows of a 16-row MFMA A operand and the G query
//    heads the columns of the B operand, so one 16x16 product per 32-wide
//    slice of d yields w_g = V^T q_g (rows 0..r-1) and q_g . mu (row r) for
//    all heads. bf16 x bf16 products are exact; accumulation is fp32.
//  B (VALU): the 64 lanes split into G groups of 64/G, one per head; a lane
//    reads the coefficient rows of its TPL consecutive tokens straight from
//    the record, forms their logits w_g . c_i, and the page LSE is reduced
//    across the head's lanes with DPP (max, then sum of 2^(z - max)).
//    The LDS-staged kernel (score_lds.h) forms these logits on the matrix
//    cores instead at rank 8 or 4 with G = 4, four pages per product.
#include "common.h"
#include "kernels.h"
#include "score_lds.h"

#include <atomic>

namespace locks {

namespace {

// Coefficient rho of token tt from the lane's packed words (RT > 0 layout:
// TPL tokens x RT elements, row-major).
template <typename T, int RT>
__device__ __forceinline__ float coef(const uint32_t* w, int tt, int rho) {
  if constexpr (sizeof(T) == 2) {
    const int e = tt * RT + rho;
    return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
  } else {
    return __uint_as_float(w[tt * RT + rho]);
  }
}

}  // namespace


// T: storage type; D: head dim; RT: rank (2, 4, 8) or 0 for any rank <= 15;
// GQ: query heads per KV head; TPL: tokens per lane = max(1, P / (64 / GQ)).
template <typename T, int D, int RT, int GQ, int TPL>
__global__ __launch_bounds__(256) void page_score_kernel(ScoreArgs a) {
  using M = ScoreMfma<T, D>;
  constexpr int kWRows = RT > 0 ? RT + 1 : 16;
  constexpr int kWVec = (kWRows + 3) / 4;
  constexpr int kCWords = RT > 0 ? TPL * RT * (int)sizeof(T) / 4 : 1;
  __shared__ __attribute__((aligned(16))) float wbuf[kScoreWaves][16][16];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int b = blockIdx.z;
  const int h = blockIdx.y;
  const int P = a.P, r = RT > 0 ? RT : a.r;
  constexpr int G = GQ;
  const int Hq = a.Hkv * G;
  const int T_b = clamp_len(a.seq_lens[b], a.max_pages, P);
  const int Jc = T_b / P;
  const int p0 = (blockIdx.x * kScoreWaves + wave) * a.ppw;
  if (p0 >= Jc) return;
  const int np = min(a.ppw, Jc - p0);

  // block ids of this wave's pages: lane t holds page p0 + t (ppw <= 64)
  const int32_t* bt_row = a.block_table + (int64_t)b * a.max_pages;
  const int my_bid = lane < np ? bt_row[p0 + lane] : -1;

  // MFMA roles: n = head column (B) / record row (A), kg = k group
  const int n = lane & 15;
  const int kg = lane >> 4;
  typename M::Op qb[M::kSteps];
  M::load_b(qb, reinterpret_cast<const T*>(a.q) + ((int64_t)b * Hq + (int64_t)h * G + (n < G ? n : 0)) * D,
            n < G, kg);
  // A rows: basis row n for n < r, else the centroid (rows past r repeat it;
  // their outputs are never read)
  const int row_off = n < r ? D * (1 + n) : 0;
  const int64_t rec_elems = a.rec_elems;
  const int c_off = D * (1 + r);                    // elements before the C block

  // phase-B roles: head g owns lanes [g*lph, (g+1)*lph); lane u of it owns
  // tokens u*TPL .. u*TPL + TPL - 1
  constexpr int lph = 64 / G;
  const int g = lane / lph;
  const int u = lane - g * lph;
  const bool tok_ok = u * TPL < P;
  const int c_lane = c_off + (tok_ok ? u * TPL * r : 0);
  // logit bias: 0 for the lane's real tokens, -inf for slots past P
  float zbias[TPL];
#pragma unroll
  for (int tt = 0; tt < TPL; ++tt) zbias[tt] = u * TPL + tt < P ? 0.f : -INFINITY;
  const float zscale = a.scale * kLog2e;
  float* out_row = a.scores + ((int64_t)b * Hq + (int64_t)h * G + g) * a.max_pages + p0;

  auto bid_ok = [&](int bid) { return bid >= 0 && (int64_t)bid < a.num_blocks; };
  auto rec_of = [&](int bid) -> const T* {
    return reinterpret_cast<const T*>(a.sum_pool) + ((int64_t)(bid_ok(bid) ? bid : 0) * a.Hkv + h) * rec_elems;
  };

  typename M::Op abuf0[M::kSteps], abuf1[M::kSteps];
  uint32_t cbuf0[kCWords], cbuf1[kCWords];
  auto load_page = [&](int t, typename M::Op* av, uint32_t* cv) {
    const T* rec = rec_of(__builtin_amdgcn_readlane(my_bid, t));
    M::load_a(av, rec + row_off, kg);
    if constexpr (RT > 0) ld_nt_words<kCWords>(rec + c_lane, cv);
  };

  auto score_page = [&](int t, typename M::Op* av, const uint32_t* cv) {
    const int bid = __builtin_amdgcn_readlane(my_bid, t);
    // ---- A: w_g and q_g . mu on the matrix cores ----
    const f32x4_t acc = M::product(av, qb);
    *reinterpret_cast<f32x4_t*>(&wbuf[wave][n][kg * 4]) = acc;
    wave_lds_sync();
    float w[kWVec * 4];
#pragma unroll
    for (int v = 0; v < kWVec; ++v) {
      const f32x4_t x = *reinterpret_cast<const f32x4_t*>(&wbuf[wave][g][v * 4]);
      w[4 * v] = x[0]; w[4 * v + 1] = x[1]; w[4 * v + 2] = x[2]; w[4 * v + 3] = x[3];
    }
    const float qmu = RT > 0 ? w[RT] : wbuf[wave][g][r];
    wave_lds_sync();  // wbuf is rewritten by the next page

    // ---- B: token logits and the page LSE of head g ----
    float z[TPL];
    if constexpr (RT > 0) {
      float ws[RT];
#pragma unroll
      for (int rho = 0; rho < RT; ++rho) ws[rho] = w[rho] * zscale;
#pragma unroll
      for (int tt = 0; tt < TPL; ++tt) {
        float s = 0.f;
#pragma unroll
        for (int rho = 0; rho < RT; ++rho) s = fmaf(ws[rho], coef<T, RT>(cv, tt, rho), s);
        z[tt] = s;
      }
    } else {
      const T* cb = rec_of(bid) + c_lane;
#pragma unroll
      for (int tt = 0; tt < TPL; ++tt) {
        float s = 0.f;
#pragma unroll
        for (int rho = 0; rho < 15; ++rho)
          if (rho < r) s = fmaf(w[rho] * zscale, Elem<T>::load(cb + tt * r + rho), s);
        z[tt] = s;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < TPL; ++tt) {
      z[tt] += zbias[tt];
      mx = fmaxf(mx, z[tt]);
    }
    mx = group_max<lph>(mx);
    float sm = 0.f;
#pragma unroll
    for (int tt = 0; tt < TPL; ++tt) sm += exp2_fast(z[tt] - mx);  // exp2(-inf) = 0
    sm = group_sum<lph>(sm);
    if (u == 0) {
      const float s = qmu * a.scale + (mx + log2_fast(sm)) * kLn2;
      out_row[t] = bid_ok(bid) ? s : -INFINITY;
    }
  };

  // two register sets in turn: page t+1 is in flight while page t is scored
  load_page(0, abuf0, cbuf0);
  for (int t = 0; t < np; t += 2) {
    if (t + 1 < np) load_page(t + 1, abuf1, cbuf1);
    score_page(t, abuf0, cbuf0);
    if (t + 1 >= np) break;
    if (t + 2 < np) load_page(t + 2, abuf0, cbuf0);
    score_page(t + 1, abuf1, cbuf1);
  }
}

// LDS-staged variant (bf16 records, rank 1/2/4/8, G * P >= 64): see score_lds.h.
template <int D, int RT, int GQ, int P>
__global__ __launch_bounds__(kScoreLdsWaves * 64, 2) void page_score_lds_kernel(ScoreArgs a) {
  __shared__ ScoreLds<D, RT, GQ, P> lds;
  const int wave = threadIdx.x >> 6;
  if (a.head_major) {  // grid (page ranges, H_kv / waves, batch): adjacent heads, same pages
    const int h = __builtin_amdgcn_readfirstlane(blockIdx.y * kScoreLdsWaves + wave);
    score_wave_lds<D, RT, GQ, P>(a, blockIdx.z, h, __builtin_amdgcn_readfirstlane(blockIdx.x * a.ppw), a.ppw, lds);
  } else {  // grid (page ranges / waves, H_kv, batch): consecutive page ranges of one head
    const int p0 = __builtin_amdgcn_readfirstlane((blockIdx.x * kScoreLdsWaves + wave) * a.ppw);
    score_wave_lds<D, RT, GQ, P>(a, blockIdx.z, blockIdx.y, p0, a.ppw, lds);
  }
}

namespace {

// Resident waves the device holds for one kernel (cached per kernel/device).
int resident_waves(const void* fn, int threads) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fn, threads, 0) != hipSuccess || blocks <= 0)
    blocks = 1;
  return cus * blocks * (threads / 64);
}

template <typename KernelTag>
int cached_waves(const void* fn, int threads = 256) {
  static std::atomic<int> cached{0};
  int waves = cached.load(std::memory_order_relaxed);
  if (waves == 0) {
    waves = resident_waves(fn, threads);
    cached.store(waves, std::memory_order_relaxed);
  }
  return waves;
}

// pages per wave (at most max_ppw) and grid for one round of `waves`
// resident waves
dim3 score_grid(ScoreArgs& a, int batch, int waves, int max_ppw) {
  const int64_t total = (int64_t)batch * a.Hkv * a.max_pages;
  int64_t ppw = (total + waves - 1) / waves;
  ppw = ppw < 1 ? 1 : (ppw > max_ppw ? max_ppw : ppw);
  a.ppw = (int)ppw;
  const int waves_per_unit = (int)((a.max_pages + ppw - 1) / ppw);
  return dim3((waves_per_unit + kScoreWaves - 1) / kScoreWaves, a.Hkv, batch);
}

template <int D, int RT, int GQ, int P>
struct LdsTag {};

template <int D, int RT, int GQ, int P>
hipError_t launch_lds(ScoreArgs a, int batch, hipStream_t stream) {
  const void* fn = reinterpret_cast<const void*>(&page_score_lds_kernel<D, RT, GQ, P>);
  constexpr int kThreads = kScoreLdsWaves * 64;
  dim3 grid = score_grid(a, batch, cached_waves<LdsTag<D, RT, GQ, P>>(fn, kThreads), kScoreMaxPpw);
  a.head_major = a.Hkv % kScoreLdsWaves == 0;
  if (a.head_major) {
    grid = dim3((a.max_pages + a.ppw - 1) / a.ppw, a.Hkv / kScoreLdsWaves, batch);
  } else {
    const int waves_per_unit = (a.max_pages + a.ppw - 1) / a.ppw;
    grid = dim3((waves_per_unit + kScoreLdsWaves - 1) / kScoreLdsWaves, a.Hkv, batch);
  }
  hipLaunchKernelGGL((page_score_lds_kernel<D, RT, GQ, P>), grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D, int RT, int GQ, int TPL>
struct RegTag {};

template <typename T, int D, int RT, int GQ, int TPL>
hipError_t launch_one(ScoreArgs a, int batch, hipStream_t stream) {
  const int waves = cached_waves<RegTag<T, D, RT, GQ, TPL>>(
      reinterpret_cast<const void*>(&page_score_kernel<T, D, RT, GQ, TPL>));
  // one round of resident waves; a wave keeps its block ids in one VGPR, so
  // at most 64 pages per wave
  const dim3 grid = score_grid(a, batch, waves, 64);
  hipLaunchKernelGGL((page_score_kernel<T, D, RT, GQ, TPL>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

// (G, tokens per lane) pairs reachable with P in {16, 32, 64}
template <int D, int RT>
hipError_t launch_lds_pg(const ScoreArgs& a, int batch, hipStream_t s) {
  switch (a.G * 100 + a.P) {
    case 416: return launch_lds<D, RT, 4, 16>(a, batch, s);
    case 432: return launch_lds<D, RT, 4, 32>(a, batch, s);
    case 464: return launch_lds<D, RT, 4, 64>(a, batch, s);
    case 816: return launch_lds<D, RT, 8, 16>(a, batch, s);
    case 832: return launch_lds<D, RT, 8, 32>(a, batch, s);
    case 864: return launch_lds<D, RT, 8, 64>(a, batch, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int D, int RT>
hipError_t launch_tpl(const ScoreArgs& a, int batch, hipStream_t s) {
  if constexpr (sizeof(T) == 2 && RT > 0) {
    if (a.G == 4 || a.G == 8) return launch_lds_pg<D, RT>(a, batch, s);
  }
  if constexpr (RT == 1) {
    return launch_tpl<T, D, 0>(a, batch, s);  // the register kernel's packed layout needs RT >= 2
  } else {
    const int lph = 64 / a.G;
    const int tpl = a.P > lph ? a.P / lph : 1;
    switch (a.G * 16 + tpl) {
      case 1 * 16 + 1: return launch_one<T, D, RT, 1, 1>(a, batch, s);
      case 2 * 16 + 1: return launch_one<T, D, RT, 2, 1>(a, batch, s);
      case 2 * 16 + 2: return launch_one<T, D, RT, 2, 2>(a, batch, s);
      case 4 * 16 + 1: return launch_one<T, D, RT, 4, 1>(a, batch, s);
      case 4 * 16 + 2: return launch_one<T, D, RT, 4, 2>(a, batch, s);
      case 4 * 16 + 4: return launch_one<T, D, RT, 4, 4>(a, batch, s);
      case 8 * 16 + 2: return launch_one<T, D, RT, 8, 2>(a, batch, s);
      case 8 * 16 + 4: return launch_one<T, D, RT, 8, 4>(a, batch, s);
      case 8 * 16 + 8: return launch_one<T, D, RT, 8, 8>(a, batch, s);
      default: return hipErrorInvalidValue;
    }
  }
}

template <typename T, int D>
hipError_t launch_rank(const ScoreArgs& a, int batch, hipStream_t s) {
  switch (a.r) {
    case 1: return launch_tpl<T, D, 1>(a, batch, s);
    case 2: return launch_tpl<T, D, 2>(a, batch, s);
    case 4: return launch_tpl<T, D, 4>(a, batch, s);
    case 8: return launch_tpl<T, D, 8>(a, batch, s);
    default: return launch_tpl<T, D, 0>(a, batch, s);
  }
}

}  // namespace

hipError_t launch_page_score(const ScoreArgs& args, int dtype, int D, int batch, hipStream_t stream) {
  if (dtype == 0) return D == 64 ? launch_rank<bf16_t, 64>(args, batch, stream)
                                 : launch_rank<bf16_t, 128>(args, batch, stream);
  return D == 64 ? launch_rank<float, 64>(args, batch, stream) : launch_rank<float, 128>(args, batch, stream);
}

}  // namespace locks

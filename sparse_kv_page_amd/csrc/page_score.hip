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
#include "common.h"
#include "kernels.h"

#include <atomic>
#include <type_traits>

namespace locks {

namespace {

template <typename T, int D>
struct ScoreMfma;

// bf16: v_mfma_f32_16x16x32_bf16. Lane l supplies row/col (l % 16) and the
// k-range 8*(l/16) .. +8 of each 32-wide k step.
template <int D>
struct ScoreMfma<bf16_t, D> {
  static constexpr int kSteps = D / 32;
  using Op = bf16x8_t;
  static __device__ __forceinline__ void load_a(Op* a, const bf16_t* row, int kg) {
#pragma unroll
    for (int s = 0; s < kSteps; ++s) a[s] = __builtin_bit_cast(Op, ld_nt4(row + s * 32 + kg * 8));
  }
  static __device__ __forceinline__ void load_b(Op* b, const bf16_t* qrow, bool ok, int kg) {
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
      b[s] = ok ? *reinterpret_cast<const Op*>(qrow + s * 32 + kg * 8) : Op{0, 0, 0, 0, 0, 0, 0, 0};
  }
  static __device__ __forceinline__ f32x4_t product(const Op* a, const Op* b) {
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
  using Op = float;
  static __device__ __forceinline__ void load_a(Op* a, const float* row, int kg) {
#pragma unroll
    for (int s = 0; s < kSteps; ++s) a[s] = __uint_as_float(ld_nt1(row + s * 4 + kg));
  }
  static __device__ __forceinline__ void load_b(Op* b, const float* qrow, bool ok, int kg) {
#pragma unroll
    for (int s = 0; s < kSteps; ++s) b[s] = ok ? qrow[s * 4 + kg] : 0.f;
  }
  static __device__ __forceinline__ f32x4_t product(const Op* a, const Op* b) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kSteps; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], acc, 0, 0, 0);
    return acc;
  }
};

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

constexpr int kScoreWaves = 4;

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

// ---------------------------------------------------------------------------
// LDS-staged variant for bf16 summaries with rank 2, 4 or 8 and G * P >= 64.
//
// Each wave keeps a ring of NS record slots in LDS and fills them with
// direct global->LDS loads (global_load_lds_dwordx4, non-temporal), so NS-1
// records per wave are in flight without holding registers. The 16-byte
// chunks of every row of the mu / V^T block are XOR-swizzled by their row
// index on the way in (the source address is per lane), which makes the
// row-wise MFMA operand reads conflict-free. Coefficient rows are read
// token-strided (lane u of a head takes tokens u, u + 64/G, ...), again
// conflict-free, with the G head groups reading the same addresses.
// ---------------------------------------------------------------------------
namespace {

typedef __attribute__((address_space(3))) void* lds_void_ptr;

constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14); }

__device__ __forceinline__ void compiler_fence() { __asm__ __volatile__("" ::: "memory"); }

// One direct global->LDS load of 16 bytes per active lane, non-temporal: lane
// i writes LDS bytes [lds + 16 i, lds + 16 i + 16). Issued from inline
// assembly so that the compiler does not guard every later LDS read with a
// wait for all outstanding loads; completion is awaited explicitly with
// s_waitcnt vmcnt before a slot is read. M0 is saved and restored.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  uint32_t saved;
  __asm__ __volatile__(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off nt\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(src)
      : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_void_ptr)(p);
}

// wait until at most n vector-memory instructions of this wave are pending
template <int I>
__device__ __forceinline__ void wait_vm_const() {
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(I));
}

template <int STEP, int MAXN>
__device__ __forceinline__ void wait_vm_pages(int pages) {
  // pages in 0 .. MAXN; the immediate must be a constant, hence the switch
  switch (pages) {
    case 0: wait_vm_const<0>(); break;
    case 1: if constexpr (MAXN >= 1) wait_vm_const<1 * STEP>(); break;
    case 2: if constexpr (MAXN >= 2) wait_vm_const<2 * STEP>(); break;
    case 3: if constexpr (MAXN >= 3) wait_vm_const<3 * STEP>(); break;
    case 4: if constexpr (MAXN >= 4) wait_vm_const<4 * STEP>(); break;
    case 5: if constexpr (MAXN >= 5) wait_vm_const<5 * STEP>(); break;
    case 6: if constexpr (MAXN >= 6) wait_vm_const<6 * STEP>(); break;
    default: if constexpr (MAXN >= 7) wait_vm_const<7 * STEP>(); break;
  }
  compiler_fence();
}

template <int D, int RT, int P, int G>
struct LdsRec {
  static constexpr int kE = 2;
  static constexpr int kHeadBytes = kE * D * (1 + RT);      // mu | V^T
  static constexpr int kBytes = kHeadBytes + kE * P * RT;   // + C
  static constexpr int kChunks = kBytes / 16;
  static constexpr int kInstr = (kChunks + 63) / 64;        // DMA instructions per record
  static constexpr int kTail = kChunks - (kInstr - 1) * 64; // lanes of the last one
  static constexpr int kRowChunks = kE * D / 16;            // 16-byte chunks per row
  static constexpr int kHeadChunks = kHeadBytes / 16;
  static constexpr int kBudget = 80 * 1024;                 // LDS bytes per workgroup
  static constexpr int kExtra = 4 * (2 * G * 16 + 64 * G) * 4; // w and score staging of 4 waves
  static constexpr int kNs0 = (kBudget - kExtra) / (4 * kBytes);
  static constexpr int kNs = kNs0 < 2 ? 2 : (kNs0 > 8 ? 8 : kNs0);
  static_assert(kBytes % 16 == 0, "records are whole 16-byte chunks");
  // LDS chunk x holds global chunk swz(x) (an involution inside each row)
  static __device__ __forceinline__ int swz(int x) {
    if (x >= kHeadChunks) return x;
    const int row = x / kRowChunks;
    return row * kRowChunks + ((x % kRowChunks) ^ (row % kRowChunks));
  }
};

}  // namespace

template <int D, int RT, int GQ, int P>
__global__ __launch_bounds__(256, 2) void page_score_lds_kernel(ScoreArgs a) {
  using M = ScoreMfma<bf16_t, D>;
  using R = LdsRec<D, RT, P, GQ>;
  constexpr int G = GQ;
  constexpr int lph = 64 / G;
  constexpr int TPL = P / lph;
  constexpr int NS = R::kNs;
  constexpr int kWVec = (RT + 1 + 3) / 4;
  static_assert(TPL >= 1 && TPL * lph == P, "P * G must be a multiple of 64");
  __shared__ __attribute__((aligned(16))) uint8_t slots[kScoreWaves][NS][R::kBytes];
  __shared__ __attribute__((aligned(16))) float wbuf[kScoreWaves][2][G][16];
  __shared__ __attribute__((aligned(16))) float sbuf[kScoreWaves][64][G];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int b = blockIdx.z;
  const int h = blockIdx.y;
  const int Hq = a.Hkv * G;
  const int p0 = __builtin_amdgcn_readfirstlane((blockIdx.x * kScoreWaves + wave) * a.ppw);
  if (p0 >= a.max_pages) return;
  // block ids are loaded before the length is known (entries up to max_pages
  // are addressable), so the two loads are in flight together
  const int32_t* bt_row = a.block_table + (int64_t)b * a.max_pages;
  int my_bid = lane < a.ppw && p0 + lane < a.max_pages ? bt_row[p0 + lane] : -1;
  const int T_b = __builtin_amdgcn_readfirstlane(clamp_len(a.seq_lens[b], a.max_pages, P));
  const int Jc = T_b / P;
  if (p0 >= Jc) return;
  const int np = min(a.ppw, Jc - p0);

  const int n = lane & 15;
  const int kg = lane >> 4;
  typename M::Op qb[M::kSteps];
  M::load_b(qb, reinterpret_cast<const bf16_t*>(a.q) + ((int64_t)b * Hq + (int64_t)h * G + (n < G ? n : 0)) * D,
            n < G, kg);
  // settle the ordinary loads before the record loads start (the wait counts
  // below assume only record loads are pending)
  wait_vm_const<0>();
  my_bid = __builtin_amdgcn_mov_dpp(my_bid, 0xE4, 0xf, 0xf, false);  // identity; orders the use after the wait
  const int g = lane / lph;
  const int u = lane - g * lph;
  const float zscale = a.scale * kLog2e;

  auto bid_ok = [&](int bid) { return bid >= 0 && (int64_t)bid < a.num_blocks; };
  const uint8_t* pool = a.sum_pool + (int64_t)h * R::kBytes;
  const int64_t blk_stride = (int64_t)a.Hkv * R::kBytes;

  // per-lane DMA source offsets (swizzled) for each instruction of a record
  int src_off[R::kInstr];
#pragma unroll
  for (int j = 0; j < R::kInstr; ++j) {
    const int x = 64 * j + lane;
    src_off[j] = (x < R::kChunks ? R::swz(x) : 0) * 16;
  }
  // MFMA A operand: LDS row of record row n (basis row n, or the centroid)
  const int arow = n < RT ? n + 1 : 0;
  int a_off[M::kSteps];
#pragma unroll
  for (int s = 0; s < M::kSteps; ++s) {
    const int c = s * 4 + kg;
    a_off[s] = (arow * R::kRowChunks + (c ^ (arow % R::kRowChunks))) * 16;
  }

  auto issue = [&](int t, int slot) {
    const int bid = __builtin_amdgcn_readlane(my_bid, t);
    const uint8_t* rec = pool + (int64_t)(bid_ok(bid) ? bid : 0) * blk_stride;
    const uint32_t dst = lds_addr(&slots[wave][slot][0]);
#pragma unroll
    for (int j = 0; j < R::kInstr; ++j) {
      if (j < R::kInstr - 1 || lane < R::kTail) dma16(rec + src_off[j], dst + j * 1024);
    }
  };

  const int npre = np < NS ? np : NS;
  for (int t = 0; t < npre; ++t) issue(t, t);

  // Two pages per iteration: their dependent chains (LDS reads -> MFMA ->
  // transpose through LDS -> logits -> DPP reductions) interleave, which hides
  // the chain latency the two resident waves per SIMD cannot.
  auto score_pages = [&](auto npg_tag, int t, int s0) {
    constexpr int NPG = decltype(npg_tag)::value;
    const uint8_t* rec[NPG];
    rec[0] = &slots[wave][s0][0];
    if constexpr (NPG == 2) rec[1] = &slots[wave][s0 + 1 == NS ? 0 : s0 + 1][0];

    // ---- A: w_g and q_g . mu ----
    typename M::Op av[NPG][M::kSteps];
#pragma unroll
    for (int p = 0; p < NPG; ++p)
#pragma unroll
      for (int s = 0; s < M::kSteps; ++s) av[p][s] = *reinterpret_cast<const bf16x8_t*>(rec[p] + a_off[s]);
    f32x4_t acc[NPG];
#pragma unroll
    for (int p = 0; p < NPG; ++p) acc[p] = M::product(av[p], qb);
    if (n < G) {
#pragma unroll
      for (int p = 0; p < NPG; ++p) *reinterpret_cast<f32x4_t*>(&wbuf[wave][p][n][kg * 4]) = acc[p];
    }
    wave_lds_sync();
    float ws[NPG][RT], qmu[NPG];
#pragma unroll
    for (int p = 0; p < NPG; ++p) {
      float w[kWVec * 4];
#pragma unroll
      for (int v = 0; v < kWVec; ++v) {
        const f32x4_t x = *reinterpret_cast<const f32x4_t*>(&wbuf[wave][p][g][v * 4]);
        w[4 * v] = x[0]; w[4 * v + 1] = x[1]; w[4 * v + 2] = x[2]; w[4 * v + 3] = x[3];
      }
      qmu[p] = w[RT];
#pragma unroll
      for (int rho = 0; rho < RT; ++rho) ws[p][rho] = w[rho] * zscale;
    }

    // ---- B: logits of the lane's tokens u, u + lph, ... ----
    float z[NPG][TPL];
#pragma unroll
    for (int p = 0; p < NPG; ++p) {
      const uint8_t* cb = rec[p] + R::kHeadBytes;
#pragma unroll
      for (int tt = 0; tt < TPL; ++tt) {
        const int tok = u + lph * tt;
        uint32_t cw[RT / 2];
        if constexpr (RT == 8) {
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(cb + tok * 16);
          cw[0] = v[0]; cw[1] = v[1]; cw[2] = v[2]; cw[3] = v[3];
        } else if constexpr (RT == 4) {
          const u32x2_t v = *reinterpret_cast<const u32x2_t*>(cb + tok * 8);
          cw[0] = v[0]; cw[1] = v[1];
        } else {
          cw[0] = *reinterpret_cast<const uint32_t*>(cb + tok * 4);
        }
        float sacc = 0.f;
#pragma unroll
        for (int rho = 0; rho < RT; ++rho)
          sacc = fmaf(ws[p][rho], (rho & 1) ? bf16_hi(cw[rho >> 1]) : bf16_lo(cw[rho >> 1]), sacc);
        z[p][tt] = sacc;
      }
    }
    float mx[NPG], sm[NPG];
#pragma unroll
    for (int p = 0; p < NPG; ++p) {
      mx[p] = z[p][0];
#pragma unroll
      for (int tt = 1; tt < TPL; ++tt) mx[p] = fmaxf(mx[p], z[p][tt]);
    }
#pragma unroll
    for (int p = 0; p < NPG; ++p) mx[p] = group_max<lph>(mx[p]);
#pragma unroll
    for (int p = 0; p < NPG; ++p) {
      sm[p] = 0.f;
#pragma unroll
      for (int tt = 0; tt < TPL; ++tt) sm[p] += exp2_fast(z[p][tt] - mx[p]);
    }
#pragma unroll
    for (int p = 0; p < NPG; ++p) sm[p] = group_sum<lph>(sm[p]);
    if (u == 0) {
#pragma unroll
      for (int p = 0; p < NPG; ++p) {
        const int bid = __builtin_amdgcn_readlane(my_bid, t + p);
        const float sc = qmu[p] * a.scale + (mx[p] + log2_fast(sm[p])) * kLn2;
        sbuf[wave][t + p][g] = bid_ok(bid) ? sc : -INFINITY;
      }
    }
  };

  int slot = 0;
  int t = 0;
  for (; t + 1 < np; t += 2) {
    wait_vm_pages<R::kInstr, NS - 1>(min(np, t + NS) - (t + 2));  // records issued after page t+1
    score_pages(std::integral_constant<int, 2>{}, t, slot);
    // every read of these two slots has been consumed; refill them
    const int s1 = slot + 1 == NS ? 0 : slot + 1;
    if (t + NS < np) issue(t + NS, slot);
    if (t + 1 + NS < np) issue(t + 1 + NS, s1);
    slot = s1 + 1 == NS ? 0 : s1 + 1;
  }
  if (t < np) {
    wait_vm_pages<R::kInstr, NS - 1>(0);
    score_pages(std::integral_constant<int, 1>{}, t, slot);
  }
  wave_lds_sync();
  // coalesced store of the wave's scores: lane t writes page p0 + t of each head
  float* out = a.scores + ((int64_t)b * Hq + (int64_t)h * G) * a.max_pages + p0;
  if (lane < np) {
#pragma unroll
    for (int gg = 0; gg < G; ++gg) out[(int64_t)gg * a.max_pages + lane] = sbuf[wave][lane][gg];
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
int cached_waves(const void* fn) {
  static std::atomic<int> cached{0};
  int waves = cached.load(std::memory_order_relaxed);
  if (waves == 0) {
    waves = resident_waves(fn, 256);
    cached.store(waves, std::memory_order_relaxed);
  }
  return waves;
}

// pages per wave and grid for one round of `waves` resident waves
dim3 score_grid(ScoreArgs& a, int batch, int waves) {
  const int64_t total = (int64_t)batch * a.Hkv * a.max_pages;
  int64_t ppw = (total + waves - 1) / waves;
  ppw = ppw < 1 ? 1 : (ppw > 64 ? 64 : ppw);
  a.ppw = (int)ppw;
  const int waves_per_unit = (int)((a.max_pages + ppw - 1) / ppw);
  return dim3((waves_per_unit + kScoreWaves - 1) / kScoreWaves, a.Hkv, batch);
}

template <int D, int RT, int GQ, int P>
struct LdsTag {};

template <int D, int RT, int GQ, int P>
hipError_t launch_lds(ScoreArgs a, int batch, hipStream_t stream) {
  const void* fn = reinterpret_cast<const void*>(&page_score_lds_kernel<D, RT, GQ, P>);
  const dim3 grid = score_grid(a, batch, cached_waves<LdsTag<D, RT, GQ, P>>(fn));
  hipLaunchKernelGGL((page_score_lds_kernel<D, RT, GQ, P>), grid, dim3(256), 0, stream, a);
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
  const dim3 grid = score_grid(a, batch, waves);
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

template <typename T, int D>
hipError_t launch_rank(const ScoreArgs& a, int batch, hipStream_t s) {
  switch (a.r) {
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

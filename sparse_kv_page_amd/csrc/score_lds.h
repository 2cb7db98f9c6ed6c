// Device code of the page scorer: MFMA operand helpers, direct global->LDS
// record loads and the LDS-staged per-wave scoring of a run of pages,
// [Locks] §4 Eq. (2).
#pragma once

#include "common.h"
#include "kernels.h"

#include <type_traits>

namespace locks {

constexpr int kScoreWaves = 4;
// waves of an LDS-staged scorer workgroup; with H_kv a multiple of it they
// take adjacent KV heads of the same pages, whose records are adjacent in
// the pool (a block's heads are stored together), so a workgroup's record
// loads cover one contiguous run per page
constexpr int kScoreLdsWaves = 4;
constexpr int kScoreMaxPpw = 128;  // pages per wave of the LDS-staged scorer (block ids in two VGPRs)
constexpr int kScorePagesPerIter = 4;  // at most this many pages scored together (interleaved chains)

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
  static __device__ __forceinline__ f32x4_t product(const Op* a, const Op* b, f32x4_t acc = {0.f, 0.f, 0.f, 0.f}) {
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

// ---------------------------------------------------------------------------
// LDS-staged variant for bf16 summaries with rank 1, 2, 4 or 8 and G * P >= 64.
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
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f2_t;

__host__ __device__ constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | (((n >> 4) & 3) << 14); }

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
  // pages in 0 .. MAXN (<= 11, STEP * MAXN <= 63); the immediate must be a constant, hence the switch
  static_assert(MAXN <= 11 && STEP * MAXN <= 63, "vmcnt range");
  switch (pages) {
    case 0: wait_vm_const<0>(); break;
    case 1: if constexpr (MAXN >= 1) wait_vm_const<1 * STEP>(); break;
    case 2: if constexpr (MAXN >= 2) wait_vm_const<2 * STEP>(); break;
    case 3: if constexpr (MAXN >= 3) wait_vm_const<3 * STEP>(); break;
    case 4: if constexpr (MAXN >= 4) wait_vm_const<4 * STEP>(); break;
    case 5: if constexpr (MAXN >= 5) wait_vm_const<5 * STEP>(); break;
    case 6: if constexpr (MAXN >= 6) wait_vm_const<6 * STEP>(); break;
    case 7: if constexpr (MAXN >= 7) wait_vm_const<7 * STEP>(); break;
    case 8: if constexpr (MAXN >= 8) wait_vm_const<8 * STEP>(); break;
    case 9: if constexpr (MAXN >= 9) wait_vm_const<9 * STEP>(); break;
    case 10: if constexpr (MAXN >= 10) wait_vm_const<10 * STEP>(); break;
    default: if constexpr (MAXN >= 11) wait_vm_const<11 * STEP>(); break;
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
  // LDS bytes per workgroup (2 per CU at 4 waves): 4 ring slots at the
  // 128K-context batch-8 shape, measured faster than 5 (fewer record loads in flight)
  // and than 3
  static constexpr int kBudget = 17 * 1024 * kScoreLdsWaves;
  static constexpr int kExtra = kScoreLdsWaves * (kScorePagesPerIter * G * 16 + kScoreMaxPpw * G) * 4;  // w and score staging
  static constexpr int kNs0 = (kBudget - kExtra) / (kScoreLdsWaves * kBytes);
  static constexpr int kNs = kNs0 < 2 ? 2 : (kNs0 > 8 ? 8 : kNs0);
  static_assert(kBytes % 16 == 0, "records are whole 16-byte chunks");
  // LDS chunk x holds global chunk swz(x) (an involution inside each row)
  static __device__ __forceinline__ int swz(int x) {
    if (x >= kHeadChunks) return x;
    const int row = x / kRowChunks;
    return row * kRowChunks + ((x % kRowChunks) ^ (row % kRowChunks));
  }
};

template <int D, int RT, int GQ, int P>
struct alignas(16) ScoreLds {
  using R = LdsRec<D, RT, P, GQ>;
  uint8_t slots[kScoreLdsWaves][R::kNs][R::kBytes];
  float wbuf[kScoreLdsWaves][kScorePagesPerIter][GQ][16];
  float sbuf[kScoreLdsWaves][kScoreMaxPpw][GQ];
};

// One wave scores pages [p0, p0 + min(ppw, Jc - p0)) of the unit (b, h) for
// all G heads (ppw <= kScoreMaxPpw, p0 wave-uniform).
template <int D, int RT, int GQ, int P>
__device__ __forceinline__ void score_wave_lds(const ScoreArgs& a, int b, int h, int p0, int ppw,
                                               ScoreLds<D, RT, GQ, P>& L) {
  using M = ScoreMfma<bf16_t, D>;
  using R = LdsRec<D, RT, P, GQ>;
  constexpr int G = GQ;
  constexpr int lph = 64 / G;
  constexpr int TPL = P / lph;
  constexpr int NS = R::kNs;
  constexpr int kWVec = (RT + 1 + 3) / 4;
  static_assert(TPL >= 1 && TPL * lph == P, "P * G must be a multiple of 64");
  auto& slots = L.slots;
  auto& wbuf = L.wbuf;
  auto& sbuf = L.sbuf;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int Hq = a.Hkv * G;
  if (p0 >= a.max_pages) return;
  // block ids are loaded before the length is known (entries up to max_pages
  // are addressable), so the two loads are in flight together
  const int32_t* bt_row = a.block_table + (int64_t)b * a.max_pages;
  // lane l holds the block ids of pages l and 64 + l of the range
  int my_bid = lane < ppw && p0 + lane < a.max_pages ? bt_row[p0 + lane] : -1;
  int my_bid2 = lane + 64 < ppw && p0 + 64 + lane < a.max_pages ? bt_row[p0 + 64 + lane] : -1;
  const int T_b = __builtin_amdgcn_readfirstlane(clamp_len(a.seq_lens[b], a.max_pages, P));
  const int Jc = T_b / P;
  if (p0 >= Jc) return;
  const int np = min(ppw, Jc - p0);

  const int n = lane & 15;
  const int kg = lane >> 4;
  typename M::Op qb[M::kSteps];
  M::load_b(qb, reinterpret_cast<const bf16_t*>(a.q) + ((int64_t)b * Hq + (int64_t)h * G + (n < G ? n : 0)) * D,
            n < G, kg);
  // settle the ordinary loads before the record loads start (the wait counts
  // below assume only record loads are pending)
  wait_vm_const<0>();
  my_bid = __builtin_amdgcn_mov_dpp(my_bid, 0xE4, 0xf, 0xf, false);  // identity; orders the use after the wait
  my_bid2 = __builtin_amdgcn_mov_dpp(my_bid2, 0xE4, 0xf, 0xf, false);
  auto bid_at = [&](int t) {  // t wave-uniform
    const int b0 = __builtin_amdgcn_readlane(my_bid, t & 63);
    const int b1 = __builtin_amdgcn_readlane(my_bid2, t & 63);
    return t < 64 ? b0 : b1;
  };
  const int g = lane / lph;
  const int u = lane - g * lph;
  const float zscale = a.scale * kLog2e;

  auto bid_ok = [&](int bid) { return bid >= 0 && (int64_t)bid < a.num_blocks; };
  const uint8_t* pool = a.sum_pool + (int64_t)h * R::kBytes;
  const int64_t blk_stride = (int64_t)a.Hkv * R::kBytes;
  // Short records (small ranks): each page's record offset and validity are
  // formed once per wave on the VALU (lane l holds pages l and 64 + l), so a
  // page's load address is two lane reads. Long records keep the per-page
  // scalar form: the extra registers slowed the rank-8 launch.
  constexpr bool kLaneOffsets = R::kBytes <= 1024;
  uint64_t off1 = 0, off2 = 0, okm1 = 0, okm2 = 0;
  if constexpr (kLaneOffsets) {
    const bool ok1 = bid_ok(my_bid), ok2 = bid_ok(my_bid2);
    okm1 = __ballot(ok1);
    okm2 = __ballot(ok2);
    off1 = (uint64_t)(ok1 ? my_bid : 0) * (uint64_t)blk_stride;
    off2 = (uint64_t)(ok2 ? my_bid2 : 0) * (uint64_t)blk_stride;
  }
  auto ok_at = [&](int t) {  // t wave-uniform
    if constexpr (kLaneOffsets) return (((t < 64 ? okm1 : okm2) >> (t & 63)) & 1u) != 0;
    else return bid_ok(bid_at(t));
  };
  auto rec_at = [&](int t) {
    if constexpr (kLaneOffsets) {
      const uint64_t o = t < 64 ? off1 : off2;
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)o, t & 63);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(o >> 32), t & 63);
      return pool + (((uint64_t)hi << 32) | lo);
    } else {
      const int bid = bid_at(t);
      return pool + (int64_t)(bid_ok(bid) ? bid : 0) * blk_stride;
    }
  };

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
    const uint8_t* rec = rec_at(t);
    const uint32_t dst = lds_addr(&slots[wave][slot][0]);
#pragma unroll
    for (int j = 0; j < R::kInstr; ++j) {
      if (j < R::kInstr - 1 || lane < R::kTail) dma16(rec + src_off[j], dst + j * 1024);
    }
  };

  const int npre = np < NS ? np : NS;
  for (int t = 0; t < npre; ++t) issue(t, t);

  // Token logits on the matrix cores (rank 8 or 4, 4 query heads per KV
  // head): for up to 4 pages at once,
  //   Z[token][4 p + g] = sum_rho C_p[token][rho] w_(p,g)[rho] * scale * log2(e)
  // is one v_mfma_f32_16x16x32_bf16 (rank 8) or v_mfma_f32_16x16x16_bf16
  // (rank 4) per 16 tokens and per half of w. A row = token, k = r p + rho (a
  // lane's k group kg is page p: the token's coefficient row, read from LDS as
  // it is stored); B is block-diagonal, column 4 p + g holding w_(p,g) in k
  // rows r p .. r p + r - 1 and zero elsewhere. w is split into bf16 hi + lo
  // (RNE twice, relative error below 2^-17), so every product is exact and
  // the sums are fp32 as on the VALU path. Lane (n, kg) then holds tokens
  // 16 m + 4 kg .. + 3 of column n = (page n / 4, head n % 4); the page LSE
  // takes the lane's values and the three other k groups' (xor 16, 32).
  constexpr bool kMfmaB = (RT == 8 || RT == 4) && G == 4 && P >= 16;
  auto score_pages_mfma_b = [&](auto npg_tag, int t, const uint8_t* const* rec) {
    constexpr int NPG = decltype(npg_tag)::value;
    constexpr int kTiles = P / 16;
    constexpr int kW = RT >= 2 ? RT / 2 : 1;  // packed bf16 pairs per lane operand (one page's k range)
    const int cp = n >> 2, cg = n & 3;        // the lane's column: page, head
    const uint8_t* rec_k = rec[0];            // the page of the lane's k group (A)
    bool ok[NPG];
#pragma unroll
    for (int p = 0; p < NPG; ++p) {
      if (p > 0 && kg == p) rec_k = rec[p];
      ok[p] = ok_at(t + p);
    }
    const bool col_ok = cp < NPG;
    const bool mine = col_ok && kg == cp;
    float wv[RT >= 4 ? RT : 4];
#pragma unroll
    for (int v = 0; v < RT / 4; ++v) {
      const f32x4_t x = *reinterpret_cast<const f32x4_t*>(&wbuf[wave][cp][cg][4 * v]);
      wv[4 * v] = x[0] * zscale; wv[4 * v + 1] = x[1] * zscale;
      wv[4 * v + 2] = x[2] * zscale; wv[4 * v + 3] = x[3] * zscale;
    }
    const float qmu_c = wbuf[wave][cp][cg][RT];
    uint32_t bh[kW], bl[kW];
#pragma unroll
    for (int e = 0; e < kW; ++e) {
      const f2_t x = {mine ? wv[2 * e] : 0.f, mine ? wv[2 * e + 1] : 0.f};
      const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
      const f2_t r = {x[0] - bf16_lo(h), x[1] - bf16_hi(h)};
      bh[e] = h;
      bl[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2_t));
    }
    const uint8_t* cb = rec_k + R::kHeadBytes;
    float z[kTiles][4];
#pragma unroll
    for (int m = 0; m < kTiles; ++m) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (RT == 8) {
        const bf16x8_t A = *reinterpret_cast<const bf16x8_t*>(cb + (16 * m + n) * 16);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8_t, u32x4_t{bh[0], bh[1], bh[2], bh[3]}),
                                                      acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8_t, u32x4_t{bl[0], bl[1], bl[2], bl[3]}),
                                                      acc, 0, 0, 0);
      } else {
        const bf16x4_t A = *reinterpret_cast<const bf16x4_t*>(cb + (16 * m + n) * 8);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, __builtin_bit_cast(bf16x4_t, u32x2_t{bh[0], bh[1]}), acc, 0,
                                                        0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, __builtin_bit_cast(bf16x4_t, u32x2_t{bl[0], bl[1]}), acc, 0,
                                                        0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) z[m][i] = acc[i];
    }
    float mx = z[0][0];
#pragma unroll
    for (int m = 0; m < kTiles; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, z[m][i]);
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    float sm = 0.f;
#pragma unroll
    for (int m = 0; m < kTiles; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm += exp2_fast(z[m][i] - mx);
    sm += shfl_xor(sm, 16);
    sm += shfl_xor(sm, 32);
    bool okc = false;
#pragma unroll
    for (int p = 0; p < NPG; ++p) okc = cp == p ? ok[p] : okc;
    if (kg == 0 && col_ok) {
      const float sc = qmu_c * a.scale + (mx + log2_fast(sm)) * kLn2;
      sbuf[wave][t + cp][cg] = okc ? sc : -INFINITY;
    }
  };

  // Several pages per iteration: their dependent chains (LDS reads -> MFMA ->
  // transpose through LDS -> logits -> DPP reductions) interleave, which hides
  // the chain latency the two resident waves per SIMD cannot (4 pages measured
  // faster than 2 or 3 at 128K context, batch 8).
  auto score_pages = [&](auto npg_tag, int t, int s0) {
    constexpr int NPG = decltype(npg_tag)::value;
    const uint8_t* rec[NPG];
    rec[0] = &slots[wave][s0][0];
#pragma unroll
    for (int p = 1; p < NPG; ++p) rec[p] = &slots[wave][(s0 + p) % NS][0];

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
    if constexpr (kMfmaB) {
      score_pages_mfma_b(std::integral_constant<int, NPG>{}, t, rec);
    } else {
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
        uint32_t cw[RT > 1 ? RT / 2 : 1];
        if constexpr (RT == 8) {
          const u32x4_t v = *reinterpret_cast<const u32x4_t*>(cb + tok * 16);
          cw[0] = v[0]; cw[1] = v[1]; cw[2] = v[2]; cw[3] = v[3];
        } else if constexpr (RT == 4) {
          const u32x2_t v = *reinterpret_cast<const u32x2_t*>(cb + tok * 8);
          cw[0] = v[0]; cw[1] = v[1];
        } else if constexpr (RT == 2) {
          cw[0] = *reinterpret_cast<const uint32_t*>(cb + tok * 4);
        } else {
          cw[0] = *reinterpret_cast<const uint16_t*>(cb + tok * 2);  // one coefficient, low half
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
        const float sc = qmu[p] * a.scale + (mx[p] + log2_fast(sm[p])) * kLn2;
        sbuf[wave][t + p][g] = ok_at(t + p) ? sc : -INFINITY;
      }
    }
    }
  };

  int slot = 0;
  int t = 0;
  // one slot beyond an iteration's pages stays in flight across iterations
  constexpr int KI = NS - 1 < kScorePagesPerIter ? (NS - 1 < 1 ? 1 : NS - 1) : kScorePagesPerIter;
  for (; t + KI - 1 < np; t += KI) {
    wait_vm_pages<R::kInstr, NS - 1>(min(np, t + NS) - (t + KI));  // records issued after page t+KI-1
    score_pages(std::integral_constant<int, KI>{}, t, slot);
    // every read of these slots has been consumed; refill them
#pragma unroll
    for (int p = 0; p < KI; ++p)
      if (t + p + NS < np) issue(t + p + NS, (slot + p) % NS);
    slot = (slot + KI) % NS;
  }
  // the last pages one at a time (all issued already: t + NS >= np here)
  for (; t < np; ++t) {
    wait_vm_pages<R::kInstr, NS - 1>(min(np, t + NS) - (t + 1));
    score_pages(std::integral_constant<int, 1>{}, t, slot);
    slot = slot + 1 == NS ? 0 : slot + 1;
  }
  wave_lds_sync();
  // coalesced store of the wave's scores: lane t writes page p0 + t of each head
  float* out = a.scores + ((int64_t)b * Hq + (int64_t)h * G) * a.max_pages + p0;
  if (lane < np) {
#pragma unroll
    for (int gg = 0; gg < G; ++gg) out[(int64_t)gg * a.max_pages + lane] = sbuf[wave][lane][gg];
  }
  if (lane + 64 < np) {
#pragma unroll
    for (int gg = 0; gg < G; ++gg) out[(int64_t)gg * a.max_pages + lane + 64] = sbuf[wave][lane + 64][gg];
  }
}

}  // namespace locks

// (a2) Page scoring on quantized ("i4") summaries: [Locks] §4 Eq. (2)
// evaluated on the stored values of the i4 storage (§4, App. C.7: 4-bit
// basis, 8-bit centroid and coefficients, bf16 scales; the record layout is
// described next to i4_record_bytes):
//   s_g(j) = s_mu (mu_code . q_g) * scale
//          + log sum_i exp( s_C[i] sum_rho C_code[i][rho] s_V[rho] (V_code[rho] . q_g) * scale )
//
// The wave structure is the bf16 LDS-staged scorer's: a ring of record
// slots per wave filled by direct global->LDS loads (16-byte chunks of the
// nibble rows XOR-swizzled by row), several pages per iteration, scores
// staged in LDS and stored coalesced. What differs is the operand decode:
//  * MFMA A operand from 4-bit fields. A 32-bit word holds 8 consecutive
//    elements, element e at nibble e/2 (even e) or 4 + e/2 (odd e), so
//      ((w >> 4j) << 3) & 0x00780078 | 0x41804180
//    is the exact bf16 pair (16 + field(2j), 16 + field(2j+1)): two
//    instructions per pair. The MFMA against q then gives
//    A = sum_a (16 + field_a) q_a, and one MFMA per wave against the
//    constant operand 16 gives A16 = 16 sum_a q_a, which removes the offset
//    and the excess of the codes (applied in the MFMA output layout, where
//    each lane scales its own four rows):
//      basis rows (field = code + 8):       code . q = A - 1.5 A16
//      centroid (byte = code + 128 = 16 hi + lo, hi and lo in two rows):
//                                            code . q = 16 A_hi + A_lo - 25 A16
//  * coefficient bytes are excess 128, one conversion instruction each, and
//    sum_rho (b_rho - 128) w_rho = sum_rho b_rho w_rho - 128 sum_rho w_rho.
#include "common.h"
#include "kernels.h"
#include "score_lds.h"

#include <atomic>
#include <type_traits>

namespace locks {

// Pages per wave, at most. A 128K-context batch of 8 has 32 per wave in one
// resident round at 64-token pages; 16-token pages then run four rounds,
// and the later rounds' workgroups go to whichever CUs free up first, which
// evens out the tail: measured faster than two rounds of 64 (by 7.5 us at
// rank 4, level at rank 8), than one round of 128 (block ids in two VGPRs)
// and than eight rounds of 16.
constexpr int kI4MaxPpw = 32;
constexpr int kI4Budget = 40 * 1024;  // LDS bytes per workgroup: 4 workgroups per CU
constexpr int kI4PagesPerIter = kScorePagesPerIter;  // at most this many pages scored together
constexpr int kI4MaxNs = 8;           // ring slots per wave

template <int D, int RT, int P, int G>
struct I4Rec {
  static constexpr int kRowBytes = D / 2;
  static constexpr int kHeadBytes = i4_head_bytes(D, RT);
  static constexpr int kScaleOff = i4_scale_offset(D, RT, P);
  static constexpr int kBytes = i4_record_bytes(D, RT, P);
  static constexpr int kChunks = kBytes / 16;
  static constexpr int kInstr = (kChunks + 63) / 64;         // DMA instructions per record
  static constexpr int kTail = kChunks - (kInstr - 1) * 64;  // lanes of the last one
  static constexpr int kRowChunks = kRowBytes / 16;          // 4 (d = 128) or 2 (d = 64)
  static constexpr int kHeadChunks = kHeadBytes / 16;
  static constexpr int kExtra = 4 * (kI4PagesPerIter * G * 16 + kI4MaxPpw * G) * 4;
  static constexpr int kNs0 = (kI4Budget - kExtra) / (4 * kBytes);
  static constexpr int kNs = kNs0 < 2 ? 2 : (kNs0 > kI4MaxNs ? kI4MaxNs : kNs0);
  static_assert(kBytes % 16 == 0 && kHeadBytes % 16 == 0, "whole 16-byte chunks");
  // LDS chunk x holds global chunk swz(x) (an involution inside each nibble row)
  static __device__ __forceinline__ int swz(int x) {
    if (x >= kHeadChunks) return x;
    const int row = x / kRowChunks;
    return row * kRowChunks + ((x % kRowChunks) ^ (row % kRowChunks));
  }
};

template <int D, int RT, int GQ, int P>
struct alignas(16) ScoreI4Lds {
  using R = I4Rec<D, RT, P, GQ>;
  uint8_t slots[kScoreWaves][R::kNs][R::kBytes];
  float wbuf[kScoreWaves][kI4PagesPerIter][GQ][16];
  float sbuf[kScoreWaves][kI4MaxPpw][GQ];
};

constexpr uint32_t kNibMask = 0x00780078u;  // one nibble at mantissa bits 3..6 of each bf16 half
constexpr uint32_t kNibBias = 0x41804180u;  // bf16 16.0 in both halves

// (x & m) | b in one instruction; m and b are held in VGPRs (a VOP3 takes no
// literal here, and the compiler would otherwise split it into two)
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t b) {
  uint32_t r;
  __asm__("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(m), "v"(b));
  return r;
}

// bf16 pairs (16 + field) of the 8 nibbles of w, in element order; m, b =
// kNibMask, kNibBias in VGPRs
__device__ __forceinline__ bf16x8_t nibbles_to_bf16(uint32_t w, uint32_t m, uint32_t b) {
  const u32x4_t v = {and_or(w << 3, m, b), and_or(w >> 1, m, b), and_or(w >> 5, m, b), and_or(w >> 9, m, b)};
  return __builtin_bit_cast(bf16x8_t, v);
}

// One wave scores pages [p0, p0 + min(ppw, Jc - p0)) of the unit (b, h) for
// all G heads (ppw <= kI4MaxPpw, p0 wave-uniform).
template <int D, int RT, int GQ, int P>
__device__ __forceinline__ void score_wave_i4(const ScoreArgs& a, int b, int h, int p0, int ppw,
                                              ScoreI4Lds<D, RT, GQ, P>& L) {
  using M = ScoreMfma<bf16_t, D>;
  using R = I4Rec<D, RT, P, GQ>;
  constexpr int G = GQ;
  constexpr int lph = 64 / G;                    // lanes per head
  constexpr bool kPartial = P < lph;             // lanes u >= P hold no token
  constexpr int TPL = kPartial ? 1 : P / lph;    // tokens per lane
  constexpr int NS = R::kNs;
  constexpr int kSteps = M::kSteps;
  constexpr int kWVec = (RT + 1 + 3) / 4;        // scaled basis rows and the centroid term
  constexpr int kCi = RT % 4;                    // the centroid's rows RT, RT + 1 sit in lane group RT / 4
  constexpr bool kMfmaB = (RT == 8 || RT == 4) && G == 4 && P >= 16;  // phase B on the matrix cores
  auto& slots = L.slots;
  auto& wbuf = L.wbuf;
  auto& sbuf = L.sbuf;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int Hq = a.Hkv * G;
  if (p0 >= a.max_pages) return;
  const int32_t* bt_row = a.block_table + (int64_t)b * a.max_pages;
  int my_bid = lane < ppw && p0 + lane < a.max_pages ? bt_row[p0 + lane] : -1;
  const int T_b = __builtin_amdgcn_readfirstlane(clamp_len(a.seq_lens[b], a.max_pages, P));
  const int Jc = T_b / P;
  if (p0 >= Jc) return;
  const int np = min(ppw, Jc - p0);

  const int n = lane & 15;
  const int kg = lane >> 4;
  typename M::Op qb[kSteps];
  M::load_b(qb, reinterpret_cast<const bf16_t*>(a.q) + ((int64_t)b * Hq + (int64_t)h * G + (n < G ? n : 0)) * D,
            n < G, kg);
  // settle the ordinary loads before the record loads start (the wait counts
  // below assume only record loads are pending)
  wait_vm_const<0>();
  my_bid = __builtin_amdgcn_mov_dpp(my_bid, 0xE4, 0xf, 0xf, false);  // identity; orders the use after the wait
  const int g = lane / lph;
  const int u = lane - g * lph;
  const float zscale = a.scale * kLog2e;

  uint32_t nib_m, nib_b;  // the decode constants, in VGPRs
  __asm__("v_mov_b32 %0, %1" : "=v"(nib_m) : "i"(kNibMask));
  __asm__("v_mov_b32 %0, %1" : "=v"(nib_b) : "i"(kNibBias));
  // A16 = 16 sum_a q_n[a] for the lane's MFMA column n: one MFMA against the
  // constant 16 (every output row holds it)
  float a16;
  {
    typename M::Op cop[kSteps];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) cop[s] = nibbles_to_bf16(0u, nib_m, nib_b);
    a16 = M::product(cop, qb)[0];
  }
  const f32x4_t a16_init = {-1.5f * a16, -1.5f * a16, -1.5f * a16, -1.5f * a16};

  auto bid_ok = [&](int bid) { return bid >= 0 && (int64_t)bid < a.num_blocks; };
  const uint8_t* pool = a.sum_pool + (int64_t)h * R::kBytes;
  const int64_t blk_stride = (int64_t)a.Hkv * R::kBytes;
  // per page of the wave (lane t holds page p0 + t): its record's byte offset
  // (block 0 for an invalid id) and a validity mask, formed once on the VALU
  // so that a page's load address is two lane reads
  const bool my_ok = bid_ok(my_bid);
  const uint64_t ok_mask = __ballot(my_ok);
  const uint64_t my_off = (uint64_t)(my_ok ? my_bid : 0) * (uint64_t)blk_stride;
  const uint32_t off_lo = (uint32_t)my_off, off_hi = (uint32_t)(my_off >> 32);
  auto ok_at = [&](int t) { return ((ok_mask >> t) & 1u) != 0; };  // t wave-uniform, < 64
  auto rec_at = [&](int t) {
    const uint64_t o = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)off_hi, t) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((int)off_lo, t);
    return pool + o;
  };

  int src_off[R::kInstr];
#pragma unroll
  for (int j = 0; j < R::kInstr; ++j) {
    const int x = 64 * j + lane;
    src_off[j] = (x < R::kChunks ? R::swz(x) : 0) * 16;
  }
  // A operand: lane (n, kg) reads record row n (rows past the centroid's two
  // read row 0; their MFMA output rows are never used) at its k groups
  // Ranks 1, 2 and 4: a page has RT + 2 nibble rows (basis, centroid high
  // and low), so the 16 rows of one product hold kPack pages (4 at ranks 1
  // and 2, 2 at rank 4) instead of one, and the nibble decode (the bulk of
  // the VALU work per record) is shared: lane (n, kg) decodes row n % kRows
  // of the pack's page n / kRows. Rank 1 pads its 3 rows to 4 so that no
  // centroid pair straddles two lanes; pad rows and rows past the last whole
  // page decode row 0 (their output rows are never used).
  constexpr int kRows = RT == 1 ? 4 : RT + 2;
  constexpr int kPack = RT <= 4 ? 16 / kRows : 1;
  const int a_pp = kPack > 1 ? n / kRows : 0;
  const int arow = kPack > 1 ? (a_pp < kPack && n % kRows < RT + 2 ? n % kRows : 0) : (n < RT + 2 ? n : 0);
  auto row_off = [&](int row) {  // the lane's 16 (d = 128) or 8 (d = 64) bytes of nibble row `row`
    if constexpr (D == 128) return (row * R::kRowChunks + (kg ^ (row % R::kRowChunks))) * 16;
    else return (row * R::kRowChunks + ((kg >> 1) ^ (row % R::kRowChunks))) * 16 + (kg & 1) * 8;
  };
  const int a_off = row_off(arow);
  // Rank 8 (ten rows a page) splits a page's rows over two products: the
  // basis rows of two pages fill one product (lane row n: page n / 8, basis
  // row n % 8) and the centroid rows of up to eight pages another (lane row
  // n: page n / 2, centroid row RT + n % 2), three products for four pages
  // instead of four, each row decoded once.
  constexpr bool kSplit = RT == 8;
  const int a_off_b = row_off(n & 7);
  const int a_off_c = row_off(RT + (n & 1));

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

  // Phase B on the matrix cores (rank 8 or 4, 4 query heads per KV head): the
  // logits of up to 4 pages come from one v_mfma_f32_16x16x32_bf16 (rank 8) or
  // v_mfma_f32_16x16x16_bf16 (rank 4) per 16 tokens and per half of w,
  //   Z[token][4 p + g] = sum_rho code_p[token][rho] w_(p,g)[rho] - 128 sum_rho w_(p,g)[rho],
  // with A row = token, k = r p + rho (a lane's k group kg is the page p)
  // and B block-diagonal: column 4 p + g holds w_(p,g) in k rows r p .. r p + r - 1
  // and zero elsewhere. Coefficient bytes are exact in bf16; w is split into
  // bf16 hi + lo (RNE twice: relative error below 2^-17), so every product is
  // exact and the sums are fp32 as on the VALU path. Lane (n, kg) then holds
  // tokens 16 m + 4 kg .. + 3 of column n = (page n / 4, head n % 4); its page
  // LSE takes the lane's values and the three other k groups' (xor 16, 32).
  auto score_pages_mfma_b = [&](auto npg_tag, int t, const uint8_t* const* rec) {
    constexpr int NPG = decltype(npg_tag)::value;
    constexpr int kTiles = P / 16;
    constexpr int kW = RT >= 2 ? RT / 2 : 1;  // packed bf16 pairs per lane operand (one page's k range)
    const int cp = n >> 2, cg = n & 3;  // the lane's column: page, head
    const uint8_t* rec_k = rec[0];      // the page of the lane's k group (A)
    const uint8_t* rec_c = rec[0];      // the page of the lane's column (token scales)
    bool ok[NPG];
#pragma unroll
    for (int p = 0; p < NPG; ++p) {
      if (p > 0 && kg == p) rec_k = rec[p];
      if (p > 0 && cp == p) rec_c = rec[p];
      ok[p] = ok_at(t + p);
    }
    const bool col_ok = cp < NPG;
    const bool mine = col_ok && kg == cp;
    float wv[RT >= 4 ? RT : 4];
#pragma unroll
    for (int v = 0; v < RT / 4; ++v) {
      const f32x4_t x = *reinterpret_cast<const f32x4_t*>(&wbuf[wave][cp][cg][4 * v]);
      wv[4 * v] = x[0]; wv[4 * v + 1] = x[1]; wv[4 * v + 2] = x[2]; wv[4 * v + 3] = x[3];
    }
    const float qmu_c = wbuf[wave][cp][cg][RT];
    float wsum_c = 0.f;
#pragma unroll
    for (int rho = 0; rho < RT; ++rho) wsum_c += wv[rho];
    const float init = col_ok ? -128.f * wsum_c : 0.f;
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
    const uint8_t* tsc = rec_c + R::kScaleOff + 2 * (RT + 1);
    float z[kTiles][4];
#pragma unroll
    for (int m = 0; m < kTiles; ++m) {
      // the RT coefficient bytes of token 16 m + n of the lane's page, exact in bf16
      uint32_t cw[RT >= 4 ? RT / 4 : 1];
      if constexpr (RT == 8) {
        const u32x2_t v = *reinterpret_cast<const u32x2_t*>(cb + (16 * m + n) * 8);
        cw[0] = v[0]; cw[1] = v[1];
      } else {
        cw[0] = *reinterpret_cast<const uint32_t*>(cb + (16 * m + n) * 4);
      }
      uint32_t av[kW];
#pragma unroll
      for (int e = 0; e < kW; ++e) {
        const uint32_t wd = cw[e >> 1];
        const int sh = 16 * (e & 1);
        const f2_t x = {(float)((wd >> sh) & 0xffu), (float)((wd >> (sh + 8)) & 0xffu)};
        av[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
      }
      f32x4_t acc = {init, init, init, init};
      if constexpr (RT == 8) {
        // v_mfma_f32_16x16x32_bf16: the lane's k range is 8 kg .. 8 kg + 7
        const bf16x8_t A = __builtin_bit_cast(bf16x8_t, u32x4_t{av[0], av[1], av[2], av[3]});
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8_t, u32x4_t{bh[0], bh[1], bh[2], bh[3]}),
                                                      acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, __builtin_bit_cast(bf16x8_t, u32x4_t{bl[0], bl[1], bl[2], bl[3]}),
                                                      acc, 0, 0, 0);
      } else {
        // v_mfma_f32_16x16x16_bf16: the lane's k range is 4 kg .. 4 kg + 3
        const bf16x4_t A = __builtin_bit_cast(bf16x4_t, u32x2_t{av[0], av[1]});
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, __builtin_bit_cast(bf16x4_t, u32x2_t{bh[0], bh[1]}), acc, 0,
                                                        0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, __builtin_bit_cast(bf16x4_t, u32x2_t{bl[0], bl[1]}), acc, 0,
                                                        0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float st = bf16_to_f32(*reinterpret_cast<const bf16_t*>(tsc + 2 * (16 * m + 4 * kg + i)));
        z[m][i] = st * acc[i];
      }
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
      const float s = qmu_c + (mx + log2_fast(sm)) * kLn2;
      sbuf[wave][t + cp][cg] = okc ? s : -INFINITY;
    }
  };

  // Phase A with kPack pages per product: the lane's output rows 4 kg + i
  // (i = 0..3) are row r % kRows of the pack's page r / kRows; basis rows are
  // scaled as in the one-page form, a centroid pair (always rows i, i + 1 of
  // one lane) gives the centroid term, and each value goes to its
  // (page, head, row) slot of the LDS exchange.
  int o_pr[4], o_lr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o_pr[i] = (4 * kg + i) / kRows;
    o_lr[i] = (4 * kg + i) % kRows;
  }
  auto score_rows_packed = [&](auto npg_tag, const uint8_t* const* rec) {
    constexpr int NPG = decltype(npg_tag)::value;
    constexpr int NQ = (NPG + kPack - 1) / kPack;
    // a centroid pair (rows RT, RT + 1 of a page) never straddles two lanes
    static_assert(kPack == 1 || (kRows % 4 == 0 && RT % 4 <= 2) || (kRows % 2 == 0 && RT % 2 == 0),
                  "centroid pairs inside one lane's four rows");
    typename M::Op av[NQ][kSteps];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const uint8_t* ra = rec[q * kPack];
#pragma unroll
      for (int pp = 1; pp < kPack; ++pp)
        if (q * kPack + pp < NPG && a_pp == pp) ra = rec[q * kPack + pp];
      if constexpr (D == 128) {
        const u32x4_t w = *reinterpret_cast<const u32x4_t*>(ra + a_off);
#pragma unroll
        for (int st = 0; st < kSteps; ++st) av[q][st] = nibbles_to_bf16(w[st], nib_m, nib_b);
      } else {
        const u32x2_t w = *reinterpret_cast<const u32x2_t*>(ra + a_off);
#pragma unroll
        for (int st = 0; st < kSteps; ++st) av[q][st] = nibbles_to_bf16(w[st], nib_m, nib_b);
      }
    }
    float sc[NQ][4];
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint8_t* rr = rec[q * kPack];
#pragma unroll
        for (int pp = 1; pp < kPack; ++pp)
          if (q * kPack + pp < NPG && o_pr[i] == pp) rr = rec[q * kPack + pp];
        const int li = o_lr[i] < RT ? o_lr[i] : RT;
        sc[q][i] = bf16_to_f32(*reinterpret_cast<const bf16_t*>(rr + R::kScaleOff + 2 * li));
      }
    f32x4_t acc[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) acc[q] = M::product(av[q], qb, a16_init);
    // every lane stores every row (no branches): rows with no slot (other
    // heads, centroid low and pad rows, pages past the pack) go to entry 15
    // of page 0, head 0, which the exchange never reads (it holds at most
    // RT + 1 <= 9 entries per head)
    float* const dummy = &wbuf[wave][0][0][15];
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int page = q * kPack + o_pr[i];
        const bool live = n < G && o_pr[i] < kPack && page < NPG;
        const bool is_c = i < 3 && o_lr[i] == RT;
        const float vb = acc[q][i] * (sc[q][i] * zscale);
        const float vc = (16.f * acc[q][i] + acc[q][(i + 1) & 3] + 0.5f * a16) * sc[q][i] * a.scale;
        const bool st = live && (is_c || o_lr[i] < RT);
        const int pg = page < NPG ? page : 0;
        const int hd = n < G ? n : 0;
        const int ix = o_lr[i] < RT ? o_lr[i] : RT;
        float* const dst = st ? &wbuf[wave][pg][hd][ix] : dummy;
        *dst = is_c ? vc : vb;
      }
  };

  // Rank-8 split form. Basis product q: lane (n, kg) holds basis rows
  // 4 (kg % 2) .. + 3 of page 2 q + kg / 2 for head n (scales in one 8-byte
  // read); centroid product: rows 4 kg .. 4 kg + 3 are the (high, low) pairs
  // of pages 2 kg and 2 kg + 1.
  auto score_rows_split = [&](auto npg_tag, const uint8_t* const* rec) {
    constexpr int NPG = decltype(npg_tag)::value;
    constexpr int NB = (NPG + 1) / 2;
    typename M::Op ab[NB][kSteps], ac[kSteps];
    auto decode = [&](typename M::Op* dst, const uint8_t* src) {
      if constexpr (D == 128) {
        const u32x4_t w = *reinterpret_cast<const u32x4_t*>(src);
#pragma unroll
        for (int st = 0; st < kSteps; ++st) dst[st] = nibbles_to_bf16(w[st], nib_m, nib_b);
      } else {
        const u32x2_t w = *reinterpret_cast<const u32x2_t*>(src);
#pragma unroll
        for (int st = 0; st < kSteps; ++st) dst[st] = nibbles_to_bf16(w[st], nib_m, nib_b);
      }
    };
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const uint8_t* ra = (2 * q + 1 < NPG && n >= 8) ? rec[2 * q + 1] : rec[2 * q];
      decode(ab[q], ra + a_off_b);
    }
    {
      const uint8_t* ra = rec[0];
#pragma unroll
      for (int p = 1; p < NPG; ++p)
        if ((n >> 1) == p) ra = rec[p];
      decode(ac, ra + a_off_c);
    }
    // scales: the basis product's page for this lane, and the centroid scale
    // of the two pages whose rows the lane holds in the centroid product
    u32x2_t sb[NB];
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const uint8_t* rs = (2 * q + 1 < NPG && kg >= 2) ? rec[2 * q + 1] : rec[2 * q];
      sb[q] = *reinterpret_cast<const u32x2_t*>(rs + R::kScaleOff + 8 * (kg & 1));
    }
    float smu[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint8_t* rs = rec[0];
#pragma unroll
      for (int p = 1; p < NPG; ++p)
        if (2 * kg + e == p) rs = rec[p];
      smu[e] = bf16_to_f32(*reinterpret_cast<const bf16_t*>(rs + R::kScaleOff + 2 * RT));
    }
    f32x4_t accb[NB];
#pragma unroll
    for (int q = 0; q < NB; ++q) accb[q] = M::product(ab[q], qb, a16_init);
    const f32x4_t accc = M::product(ac, qb, a16_init);
    float* const dummy = &wbuf[wave][0][0][15];
#pragma unroll
    for (int q = 0; q < NB; ++q) {
      const int page = 2 * q + (kg >> 1);
      f32x4_t o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = accb[q][i] * (((i & 1) ? bf16_hi(sb[q][i >> 1]) : bf16_lo(sb[q][i >> 1])) * zscale);
      if (n < G && page < NPG) *reinterpret_cast<f32x4_t*>(&wbuf[wave][page][n][4 * (kg & 1)]) = o;
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int page = 2 * kg + e;
      const float cent = (16.f * accc[2 * e] + accc[2 * e + 1] + 0.5f * a16) * smu[e] * a.scale;
      float* const dst = (n < G && page < NPG) ? &wbuf[wave][page < NPG ? page : 0][n < G ? n : 0][RT] : dummy;
      *dst = cent;
    }
  };

  auto score_pages = [&](auto npg_tag, int t, int s0) {
    constexpr int NPG = decltype(npg_tag)::value;
    const uint8_t* rec[NPG];
    rec[0] = &slots[wave][s0][0];
#pragma unroll
    for (int p = 1; p < NPG; ++p) rec[p] = &slots[wave][(s0 + p) % NS][0];

    // ---- A: code . q for the basis rows and the centroid's nibble rows ----
    if constexpr (kPack > 1) {
      score_rows_packed(std::integral_constant<int, NPG>{}, rec);
    } else if constexpr (kSplit) {
      score_rows_split(std::integral_constant<int, NPG>{}, rec);
    } else {
    typename M::Op av[NPG][kSteps];
#pragma unroll
    for (int p = 0; p < NPG; ++p) {
      if constexpr (D == 128) {
        const u32x4_t w = *reinterpret_cast<const u32x4_t*>(rec[p] + a_off);
#pragma unroll
        for (int s = 0; s < kSteps; ++s) av[p][s] = nibbles_to_bf16(w[s], nib_m, nib_b);
      } else {
        const u32x2_t w = *reinterpret_cast<const u32x2_t*>(rec[p] + a_off);
#pragma unroll
        for (int s = 0; s < kSteps; ++s) av[p][s] = nibbles_to_bf16(w[s], nib_m, nib_b);
      }
    }
    // Lane (n, kg) holds rows 4kg .. 4kg+3 of head n. The products start
    // from -1.5 A16, so a basis row holds A' = A - 1.5 A16 = code . q; the
    // lane scales its rows where they are (scales s_V[4kg .. 4kg+3], or s_mu
    // at index RT, in one 8-byte read, issued before the products):
    //   basis row rho < RT:   A' s_V[rho] * scale * log2(e)
    //   row RT (centroid):    (16 A'_hi + A'_lo + 0.5 A16) s_mu * scale
    //                         (= (16 A_hi + A_lo - 25 A16) s_mu * scale)
    // then the G heads' rows go through LDS to the lanes that own the head.
    u32x2_t sv[NPG];
#pragma unroll
    for (int p = 0; p < NPG; ++p) sv[p] = *reinterpret_cast<const u32x2_t*>(rec[p] + R::kScaleOff + 8 * kg);
    f32x4_t acc[NPG];
#pragma unroll
    for (int p = 0; p < NPG; ++p) acc[p] = M::product(av[p], qb, a16_init);
#pragma unroll
    for (int p = 0; p < NPG; ++p) {
      f32x4_t o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = acc[p][i] * (((i & 1) ? bf16_hi(sv[p][i >> 1]) : bf16_lo(sv[p][i >> 1])) * zscale);
      const float smu = (kCi & 1) ? bf16_hi(sv[p][kCi >> 1]) : bf16_lo(sv[p][kCi >> 1]);
      const float cent = (16.f * acc[p][kCi] + acc[p][kCi + 1] + 0.5f * a16) * smu * a.scale;
      if (kg == RT / 4) o[kCi] = cent;
      if (n < G) *reinterpret_cast<f32x4_t*>(&wbuf[wave][p][n][kg * 4]) = o;
    }
    }
    wave_lds_sync();
    if constexpr (kMfmaB) {
      score_pages_mfma_b(std::integral_constant<int, NPG>{}, t, rec);
    } else {
    float ws[NPG][RT], wsum[NPG], qmu[NPG];
#pragma unroll
    for (int p = 0; p < NPG; ++p) {
      float w[kWVec * 4];
#pragma unroll
      for (int v = 0; v < kWVec; ++v) {
        const f32x4_t x = *reinterpret_cast<const f32x4_t*>(&wbuf[wave][p][g][v * 4]);
        w[4 * v] = x[0]; w[4 * v + 1] = x[1]; w[4 * v + 2] = x[2]; w[4 * v + 3] = x[3];
      }
      qmu[p] = w[RT];
      float sum = 0.f;
#pragma unroll
      for (int rho = 0; rho < RT; ++rho) {
        ws[p][rho] = w[rho];
        sum += w[rho];
      }
      wsum[p] = -128.f * sum;
    }

    // ---- B: logits of the lane's tokens u, u + lph, ... ----
    float z[NPG][TPL];
#pragma unroll
    for (int p = 0; p < NPG; ++p) {
      const uint8_t* cb = rec[p] + R::kHeadBytes;
      const uint8_t* tsc = rec[p] + R::kScaleOff + 2 * (RT + 1);
#pragma unroll
      for (int tt = 0; tt < TPL; ++tt) {
        int tok = u + lph * tt;
        if constexpr (kPartial) tok = tok < P ? tok : 0;
        uint32_t cw[(RT + 3) / 4];
        if constexpr (RT == 8) {
          const u32x2_t v = *reinterpret_cast<const u32x2_t*>(cb + tok * 8);
          cw[0] = v[0]; cw[1] = v[1];
        } else if constexpr (RT == 4) {
          cw[0] = *reinterpret_cast<const uint32_t*>(cb + tok * 4);
        } else if constexpr (RT == 2) {
          cw[0] = *reinterpret_cast<const uint16_t*>(cb + tok * 2);
        } else {
          cw[0] = cb[tok];
        }
        float sacc = wsum[p];  // holds -128 sum_rho w_rho: the codes' excess
#pragma unroll
        for (int rho = 0; rho < RT; ++rho)
          sacc = fmaf(ws[p][rho], (float)((cw[rho >> 2] >> (8 * (rho & 3))) & 0xffu), sacc);
        const float st = bf16_to_f32(*reinterpret_cast<const bf16_t*>(tsc + 2 * tok));
        float zz = st * sacc;
        if constexpr (kPartial) zz = u < P ? zz : -INFINITY;
        z[p][tt] = zz;
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
        const float s = qmu[p] + (mx[p] + log2_fast(sm[p])) * kLn2;
        sbuf[wave][t + p][g] = ok_at(t + p) ? s : -INFINITY;
      }
    }
    }
  };

  int slot = 0;
  int t = 0;
  constexpr int KI = NS - 1 < kI4PagesPerIter ? (NS - 1 < 1 ? 1 : NS - 1) : kI4PagesPerIter;
  for (; t + KI - 1 < np; t += KI) {
    wait_vm_pages<R::kInstr, NS - 1>(min(np, t + NS) - (t + KI));  // records issued after page t+KI-1
    score_pages(std::integral_constant<int, KI>{}, t, slot);
#pragma unroll
    for (int p = 0; p < KI; ++p)
      if (t + p + NS < np) issue(t + p + NS, (slot + p) % NS);
    slot = (slot + KI) % NS;
  }
  for (; t < np; ++t) {
    wait_vm_pages<R::kInstr, NS - 1>(min(np, t + NS) - (t + 1));
    score_pages(std::integral_constant<int, 1>{}, t, slot);
    slot = slot + 1 == NS ? 0 : slot + 1;
  }
  wave_lds_sync();
  float* out = a.scores + ((int64_t)b * Hq + (int64_t)h * G) * a.max_pages + p0;
  if (lane < np) {
#pragma unroll
    for (int gg = 0; gg < G; ++gg) out[(int64_t)gg * a.max_pages + lane] = sbuf[wave][lane][gg];
  }
}

template <int D, int RT, int GQ, int P>
__global__ __launch_bounds__(256, 4) void page_score_i4_kernel(ScoreArgs a) {
  __shared__ ScoreI4Lds<D, RT, GQ, P> lds;
  const int wave = threadIdx.x >> 6;
  const int p0 = __builtin_amdgcn_readfirstlane((blockIdx.x * kScoreWaves + wave) * a.ppw);
  score_wave_i4<D, RT, GQ, P>(a, blockIdx.z, blockIdx.y, p0, a.ppw, lds);
}

namespace {

template <int D, int RT, int GQ, int P>
hipError_t launch_i4(ScoreArgs a, int batch, hipStream_t stream) {
  static_assert(sizeof(ScoreI4Lds<D, RT, GQ, P>) <= kI4Budget, "LDS budget");
  static std::atomic<int> cached{0};
  int waves = cached.load(std::memory_order_relaxed);
  if (waves == 0) {
    int dev = 0, cus = 0, blocks = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &blocks, reinterpret_cast<const void*>(&page_score_i4_kernel<D, RT, GQ, P>), 256, 0) != hipSuccess ||
        blocks <= 0)
      blocks = 1;
    waves = cus * blocks * kScoreWaves;
    cached.store(waves, std::memory_order_relaxed);
  }
  // pages per wave for one round of resident waves, at most kI4MaxPpw (then
  // several rounds)
  const int64_t total = (int64_t)batch * a.Hkv * a.max_pages;
  int64_t ppw = (total + waves - 1) / waves;
  ppw = ppw < 1 ? 1 : (ppw > kI4MaxPpw ? kI4MaxPpw : ppw);
  a.ppw = (int)ppw;
  const int waves_per_unit = (int)((a.max_pages + ppw - 1) / ppw);
  const dim3 grid((waves_per_unit + kScoreWaves - 1) / kScoreWaves, a.Hkv, batch);
  hipLaunchKernelGGL((page_score_i4_kernel<D, RT, GQ, P>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <int D, int RT, int GQ>
hipError_t launch_i4_p(const ScoreArgs& a, int batch, hipStream_t s) {
  switch (a.P) {
    case 16: return launch_i4<D, RT, GQ, 16>(a, batch, s);
    case 32: return launch_i4<D, RT, GQ, 32>(a, batch, s);
    case 64: return launch_i4<D, RT, GQ, 64>(a, batch, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D, int RT>
hipError_t launch_i4_g(const ScoreArgs& a, int batch, hipStream_t s) {
  switch (a.G) {
    case 1: return launch_i4_p<D, RT, 1>(a, batch, s);
    case 2: return launch_i4_p<D, RT, 2>(a, batch, s);
    case 4: return launch_i4_p<D, RT, 4>(a, batch, s);
    case 8: return launch_i4_p<D, RT, 8>(a, batch, s);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t launch_i4_r(const ScoreArgs& a, int batch, hipStream_t s) {
  switch (a.r) {
    case 1: return launch_i4_g<D, 1>(a, batch, s);
    case 2: return launch_i4_g<D, 2>(a, batch, s);
    case 4: return launch_i4_g<D, 4>(a, batch, s);
    case 8: return launch_i4_g<D, 8>(a, batch, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_page_score_i4(const ScoreArgs& a, int D, int batch, hipStream_t stream) {
  return D == 64 ? launch_i4_r<64>(a, batch, stream) : launch_i4_r<128>(a, batch, stream);
}

}  // namespace locks

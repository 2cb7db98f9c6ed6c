// (a5) Sparse paged decode attention over the selected pages, [Locks] §2:
// the softmax is renormalised over the tokens of the selected pages only and
// uses the original K/V.
//
// Split-K: a workgroup takes `pages_per_split` consecutive slots of one
// (sequence, KV head)'s selected list, cut into 16-token tiles; its 8 waves
// take the tiles in turn (TPW each), a wave loading its next tile while it
// computes the current one (non-temporal loads: the tiles are read once per
// step).
// Per tile, for all G query heads of the group:
//   S = K q^T on the matrix cores (16 tokens x 16 head columns, G used),
//   online softmax in base 2 (running max / sum per head),
//   o_g = alpha_g o_g + sum_i p_g(i) v_i on the VALU: lane (c, t) owns the
//   8-column slice c of d for tokens 4t .. 4t+3, so V rows are read with
//   coalesced 16-byte loads.
// The waves' states merge through LDS into one normalised partial (o, lse) per
// head and split. The last workgroup of a (sequence, KV head) to finish
// (per-unit arrival counter in the workspace, reset by that workgroup) merges
// the splits by LSE and writes the output.
#include "common.h"
#include "kernels.h"
#include "decode_split.h"

namespace locks {

// Register budget: two tiles per wave with bf16 and G <= 4 fits 4 waves per
// SIMD; four tiles per wave, G = 8 and fp32 take more registers. An 8-wave
// workgroup per CU holds every workgroup of grids like 128K context at batch 8.
template <typename T, int D, int GQ, int TPW>
__global__ __launch_bounds__(kDecThreads, (sizeof(T) == 2 && GQ <= 4 && TPW <= 2) ? 4 : 2) void sparse_decode_kernel(
    DecodeArgs a) {
  __shared__ DecodeLds<D, GQ> lds;
  decode_split<T, D, GQ, TPW>(a, blockIdx.x, blockIdx.y, blockIdx.z, gridDim.x, lds);
}

int decode_pages_per_split(int page_size, int tiles_per_wave) {
  return kDecWaves * tiles_per_wave * kDecTile / page_size;
}

// Eight or four tiles per wave cut the splits (a shorter merge, fewer loads
// in flight per CU) while the grid still holds at least 256 workgroups (one
// per CU); smaller grids and fp32 (whose larger kernels spill) keep two.
int decode_tiles_per_wave(int64_t units, int k, int page_size, bool f32) {
  if (f32) return kDecTilesPerWaveSmall;
  for (int tpw : {kDecTilesPerWaveXL, kDecTilesPerWaveLarge}) {
    const int pps = decode_pages_per_split(page_size, tpw);
    if (units * ((k + pps - 1) / pps) >= 256) return tpw;
  }
  return kDecTilesPerWaveSmall;
}

int decode_max_splits(int k, int page_size) {
  const int pps = decode_pages_per_split(page_size, kDecTilesPerWaveSmall);
  return (k + pps - 1) / pps;
}

namespace {
template <typename T, int D, int G>
void launch_tpw(const DecodeArgs& a, dim3 grid, hipStream_t stream, int tpw) {
  if constexpr (sizeof(T) == 2) {
    if (tpw == kDecTilesPerWaveXL) {
      hipLaunchKernelGGL((sparse_decode_kernel<T, D, G, kDecTilesPerWaveXL>), grid, dim3(kDecThreads), 0, stream, a);
      return;
    }
    if (tpw == kDecTilesPerWaveLarge) {
      hipLaunchKernelGGL((sparse_decode_kernel<T, D, G, kDecTilesPerWaveLarge>), grid, dim3(kDecThreads), 0, stream, a);
      return;
    }
  }
  hipLaunchKernelGGL((sparse_decode_kernel<T, D, G, kDecTilesPerWaveSmall>), grid, dim3(kDecThreads), 0, stream, a);
}
}  // namespace

hipError_t launch_sparse_decode(const DecodeArgs& a, int dtype, int D, int batch, hipStream_t stream) {
  dim3 grid(a.splits, a.Hkv, batch);
  // tiles per wave of the host's split plan (pages_per_split = waves * tiles * 16 / P)
  const int tpw = dtype == 0 ? a.pages_per_split * a.P / (kDecWaves * kDecTile) : kDecTilesPerWaveSmall;
#define LAUNCH(T, DD, GG) launch_tpw<T, DD, GG>(a, grid, stream, tpw)
#define LAUNCH_G(T, DD)                  \
  switch (a.G) {                         \
    case 1: LAUNCH(T, DD, 1); break;     \
    case 2: LAUNCH(T, DD, 2); break;     \
    case 4: LAUNCH(T, DD, 4); break;     \
    default: LAUNCH(T, DD, 8); break;    \
  }
  if (dtype == 0) {
    if (D == 64) { LAUNCH_G(bf16_t, 64) } else { LAUNCH_G(bf16_t, 128) }
  } else {
    if (D == 64) { LAUNCH_G(float, 64) } else { LAUNCH_G(float, 128) }
  }
#undef LAUNCH_G
#undef LAUNCH
  return hipGetLastError();
}

}  // namespace locks

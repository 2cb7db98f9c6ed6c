// (a5) Sparse paged decode attention over the selected pages, [Locks] §2:
// the softmax is renormalised over the tokens of the selected pages only and
// uses the original K/V.
//
// Split-K: a workgroup takes `pages_per_split` consecutive slots of one
// (sequence, KV head)'s selected list, cut into 16-token tiles; its 4 waves
// take the tiles in turn (kDecTilesPerWave each), with every K and V load of
// a wave issued up front (non-temporal: the tiles are read once per step).
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

// bf16 with G <= 4: 4 workgroups (16 waves) per CU, so the whole grid of the
// common shapes is resident at once; G = 8 and fp32 need more registers.
template <typename T, int D, int GQ>
__global__ __launch_bounds__(256, (sizeof(T) == 2 && GQ <= 4) ? 4 : 2) void sparse_decode_kernel(DecodeArgs a) {
  __shared__ DecodeLds<D, GQ> lds;
  decode_split<T, D, GQ>(a, blockIdx.x, blockIdx.y, blockIdx.z, gridDim.x, lds);
}

int decode_pages_per_split(int page_size) { return kDecTilesPerWg * kDecTile / page_size; }

hipError_t launch_sparse_decode(const DecodeArgs& a, int dtype, int D, int batch, hipStream_t stream) {
  dim3 grid(a.splits, a.Hkv, batch);
#define LAUNCH(T, DD, GG) \
  hipLaunchKernelGGL((sparse_decode_kernel<T, DD, GG>), grid, dim3(256), 0, stream, a)
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

// (a3 + a4) Share-average combine and top-(k-2) page selection, [Locks] §2, §4.
//
// One workgroup (512 or 1024 threads) per (sequence, KV head). From the per-head page
// scores s_g(j) of the Jc complete pages:
//   log Z_g  = log sum_j exp(s_g(j))
//   sigma_j  = log((1/G) sum_g exp(s_g(j) - log Z_g))   (log of the share average)
// Pages 0 (sink) and J-1 (current) are always kept; the other k-2 slots take
// the largest sigma among the remaining complete pages, ties to the lower
// page id.
//
// Scores are read once: thread t keeps pages t, t + NT, ... (up to NPT of
// them) in registers for both the normaliser and sigma. A generic variant
// (NPT = 0) loops over global memory for longer contexts.
//
// Ranking: every candidate gets the composite key
//   key(j) = (order-preserving image of sigma_j) << idbits | (2^idbits - 1 - j)
// which is unique and orders by (sigma desc, id asc). The bits above the
// highest bit in which two candidates differ are common and skipped; the rest
// is radix-selected with 11-bit digits (2048-bin LDS histogram, most
// significant digit first), stopping as soon as the bin holding the K-th key
// is taken whole. The chosen pages are written in ascending order by a
// block-wide scan over page flags.
#include "common.h"
#include "kernels.h"
#include "select_unit.h"

namespace locks {

constexpr int kSelLdsKeys = 16384;  // sigma keys kept in LDS up to this many pages

// NT threads, NPT register pages per thread (0: loop over global memory)
template <int NT, int NPT>
__global__ __launch_bounds__(NT) void select_kernel(SelectArgs a) {
  __shared__ SelectLds<NT, kSelLdsKeys> lds;
  select_unit<NT, NPT, kSelLdsKeys>(a, blockIdx.y, blockIdx.x, lds);
}

// Up to 2048 pages, 512 threads with 4 pages each: the selection is a chain
// of block-wide steps, and a smaller block shortens every barrier (measured
// faster than 1024 threads x 2 pages). Longer contexts use 1024 threads.
hipError_t launch_select(const SelectArgs& a, int batch, hipStream_t stream) {
  dim3 grid(a.Hkv, batch);
  if (a.max_pages <= 512 * 4)
    hipLaunchKernelGGL((select_kernel<512, 4>), grid, dim3(512), 0, stream, a);
  else if (a.max_pages <= 1024 * 8)
    hipLaunchKernelGGL((select_kernel<1024, 8>), grid, dim3(1024), 0, stream, a);
  else
    hipLaunchKernelGGL((select_kernel<1024, 0>), grid, dim3(1024), 0, stream, a);
  return hipGetLastError();
}

}  // namespace locks

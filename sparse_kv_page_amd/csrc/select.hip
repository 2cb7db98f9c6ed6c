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
// is radix-selected with 10-bit digits (1024-bin LDS histogram, most
// significant digit first), stopping as soon as the bin holding the K-th key
// is taken whole. The chosen pages are written in ascending order by a
// block-wide scan over page flags.
#include "common.h"
#include "kernels.h"
#include "select_unit.h"

namespace locks {

constexpr int kSelLdsKeys = 16384;  // sigma keys kept in LDS up to this many pages

// NT threads, NPT register pages per thread (0: loop over global memory), GQ
// query heads per KV head
template <int NT, int NPT, int GQ>
__global__ __launch_bounds__(NT) void select_kernel(SelectArgs a) {
  // the register path keeps its keys in registers; with eight pages per
  // thread (not consecutive) its output goes through an LDS bitmap
  constexpr int kKeys = NPT > 0 ? 1 : kSelLdsKeys;
  constexpr int kBits = NPT > 4 ? (NT * NPT + 31) / 32 : 1;
  __shared__ SelectLds<NT, kKeys, kBits> lds;
  select_unit<NT, NPT, kKeys, GQ, kBits>(a, blockIdx.y, blockIdx.x, lds);
}

namespace {
template <int NT, int NPT>
void launch_g(const SelectArgs& a, dim3 grid, hipStream_t stream) {
  switch (a.G) {
    case 1: hipLaunchKernelGGL((select_kernel<NT, NPT, 1>), grid, dim3(NT), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((select_kernel<NT, NPT, 2>), grid, dim3(NT), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((select_kernel<NT, NPT, 4>), grid, dim3(NT), 0, stream, a); break;
    default: hipLaunchKernelGGL((select_kernel<NT, NPT, 8>), grid, dim3(NT), 0, stream, a); break;
  }
}
}  // namespace

// Up to 2048 pages, 512 threads with 4 pages each: the selection is a chain
// of block-wide steps, and a smaller block shortens every barrier (measured
// faster than 1024 threads x 2 pages). Longer contexts use 1024 threads.
hipError_t launch_select(const SelectArgs& a, int batch, hipStream_t stream) {
  dim3 grid(a.Hkv, batch);
  if (a.max_pages <= 512 * 4)
    launch_g<512, 4>(a, grid, stream);
  else if (a.max_pages <= 1024 * 8)
    launch_g<1024, 8>(a, grid, stream);
  else
    launch_g<1024, 0>(a, grid, stream);
  return hipGetLastError();
}

}  // namespace locks

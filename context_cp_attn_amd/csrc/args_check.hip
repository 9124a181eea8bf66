// Precondition check of the position and segment-id arrays of an attention call.
//
// The attention kernels classify whole tiles from the first and last entries of a
// tile's positions and segment ids, which is exact only when positions increase
// strictly and segment ids never decrease along a row (the causal test is
// kpos <= qpos, the segment test equality of ids; block positions: handbook
// "Context parallelism: Ring Attention and Ulysses", §"Ring Attention"; per-token
// segment ids and positions: MaxText PR "Add Packing Support for Context
// Parallelism (Ring Attention)").  These kernels test exactly those rules, plus
// non-negative positions (so qpos - kpos cannot overflow), and report violations
// as bits of one int32; they change nothing else.
#include "launch.h"

namespace cp {
namespace {

__global__ void check_clear_kernel(int* flags) { *flags = 0; }

// blockIdx.y selects the array: 0 q_pos, 1 k_pos (strict, >= 0), 2 q_seg, 3 k_seg
// (non-decreasing within each of the B rows).
__global__ __launch_bounds__(256) void check_order_kernel(const int* q_pos, const int* k_pos, const int* q_seg,
                                                          const int* k_seg, int64_t B, int64_t Sq, int64_t Sk,
                                                          int* flags) {
  const int which = blockIdx.y;
  const int* a = which == 0 ? q_pos : which == 1 ? k_pos : which == 2 ? q_seg : k_seg;
  if (a == nullptr) return;
  const bool is_pos = which < 2;
  const int64_t n = (which & 1) ? Sk : Sq;
  const int64_t total = is_pos ? n : B * n;
  bool bad = false;
  for (int64_t t = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; t < total;
       t += int64_t(gridDim.x) * blockDim.x) {
    const int x = a[t];
    if (is_pos && x < 0) bad = true;
    if ((t % n) + 1 < n) {
      const int y = a[t + 1];
      bad |= is_pos ? !(x < y) : !(x <= y);
    }
  }
  if (bad) atomicOr(flags, 1 << which);
}

}  // namespace

hipError_t launch_check_args(const int* q_pos, const int* k_pos, const int* q_seg, const int* k_seg, int64_t B,
                             int64_t Sq, int64_t Sk, int* flags, hipStream_t s) {
  hipLaunchKernelGGL(check_clear_kernel, dim3(1), dim3(1), 0, s, flags);
  const int64_t most = B * (Sq > Sk ? Sq : Sk);
  const int64_t blocks = (most + 255) / 256 < 1024 ? (most + 255) / 256 : 1024;
  hipLaunchKernelGGL(check_order_kernel, dim3(unsigned(blocks), 4), dim3(256), 0, s, q_pos, k_pos, q_seg, k_seg, B,
                     Sq, Sk, flags);
  return hipGetLastError();
}

}  // namespace cp

// In-place log-sum-exp merge of a ring step's block result into the running result.
// Handbook "Context parallelism: Ring Attention and Ulysses", self-test answers and
// §"Ring Attention": lse = log(e^lse1 + e^lse2), o = o1 e^(lse1-lse) + o2 e^(lse2-lse).
//
// HBM-bound streaming kernel: each thread owns 4 consecutive float32 of one
// (b, s, h) row of the accumulator (16-byte loads and stores); the D/4 threads of a
// row sit in one wavefront (D/4 divides 64), so every lane reads the old lse_acc of
// its row in the same instruction before the row's first lane writes the new one.
#include "common.h"
#include "launch.h"
#include "prof.h"

namespace cp {
namespace {

constexpr int kThreads = 256;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

template <bool kBf16>
__global__ __launch_bounds__(kThreads) void lse_merge_kernel(float* __restrict__ acc,
                                                             float* __restrict__ lse_acc,
                                                             const void* __restrict__ blk,
                                                             const float* __restrict__ lse_blk,
                                                             int S, int H, int D4,
                                                             int64_t nvec) {
  const int64_t t = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (t >= nvec) return;
  const int64_t row = t / D4;            // (b, s, h) row index in [B*S*H]
  const int c = int(t - row * D4);       // which 4-float column group
  const int h = int(row % H);
  const int64_t bs = row / H;
  const int s = int(bs % S);
  const int64_t b = bs / S;
  const int64_t li = (b * H + h) * int64_t(S) + s;  // lse index [b][h][s]
  const MergeWeights w = merge_weights(lse_acc[li], lse_blk[li]);
  const float wa = w.wa, wb = w.wb;
  f32x4 a = *reinterpret_cast<const f32x4*>(acc + t * 4);
  f32x4 x;
  if constexpr (kBf16) {
    const u16x4 r = *reinterpret_cast<const u16x4*>(static_cast<const uint16_t*>(blk) + t * 4);
    x = f32x4{bf16_to_f32(r.x), bf16_to_f32(r.y), bf16_to_f32(r.z), bf16_to_f32(r.w)};
  } else {
    x = *reinterpret_cast<const f32x4*>(static_cast<const float*>(blk) + t * 4);
  }
  f32x4 o;
  o.x = a.x * wa + x.x * wb;
  o.y = a.y * wa + x.y * wb;
  o.z = a.z * wa + x.z * wb;
  o.w = a.w * wa + x.w * wb;
  *reinterpret_cast<f32x4*>(acc + t * 4) = o;
  if (c == 0) lse_acc[li] = w.lse;
}

}  // namespace

hipError_t launch_lse_merge(int64_t B, int64_t S, int64_t H, int64_t D, float* acc, float* lse_acc,
                            const void* blk, const float* lse_blk, int blk_is_bf16, hipStream_t s) {
  const int64_t nvec = B * S * H * (D / 4);
  const unsigned grid = unsigned((nvec + kThreads - 1) / kThreads);
  ProfScope ps(s, kProfLseMerge);
  if (blk_is_bf16)
    hipLaunchKernelGGL(lse_merge_kernel<true>, dim3(grid), dim3(kThreads), 0, s, acc, lse_acc, blk,
                       lse_blk, int(S), int(H), int(D / 4), nvec);
  else
    hipLaunchKernelGGL(lse_merge_kernel<false>, dim3(grid), dim3(kThreads), 0, s, acc, lse_acc,
                       blk, lse_blk, int(S), int(H), int(D / 4), nvec);
  return hipGetLastError();
}

}  // namespace cp

// In-place log-sum-exp merge of a ring step's block result into the running result.
// Handbook "Context parallelism: Ring Attention and Ulysses", self-test answers and
// §"Ring Attention": lse = log(e^lse1 + e^lse2), o = o1 e^(lse1-lse) + o2 e^(lse2-lse).
//
// HBM-bound streaming kernel: each thread moves two 16-byte vectors (4 consecutive
// float32 of a (b, s, h) row of the accumulator each, kThreads vectors apart); the
// D/4 threads of a row sit in one wavefront (D/4 divides 64), so every lane reads the
// old lse_acc of its row in the same instruction before the row's first lane writes
// the new one.  Index math is 32-bit (a 64-bit division is a long instruction
// sequence); the entry point rejects sizes whose vector indices would not fit.
#include "common.h"
#include "launch.h"
#include "prof.h"

namespace cp {
namespace {

constexpr int kThreads = 256;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4 __attribute__((ext_vector_type(4)));

constexpr int kVPT = 2;  // vectors per thread: both loads issued before the stores

using I = uint32_t;

template <bool kBf16>
__global__ __launch_bounds__(kThreads) void lse_merge_kernel(float* __restrict__ acc,
                                                             float* __restrict__ lse_acc,
                                                             const void* __restrict__ blk,
                                                             const float* __restrict__ lse_blk,
                                                             I S, I H, I D4, I nvec) {
  // vectors t0 + u * kThreads, u < kVPT; the D4 lanes of a row are consecutive
  // threads of one wavefront for every u
  const I t0 = I(blockIdx.x) * I(kThreads * kVPT) + I(threadIdx.x);
  f32x4 a[kVPT], x[kVPT];
  MergeWeights w[kVPT];
  I li[kVPT];
#pragma unroll
  for (int u = 0; u < kVPT; ++u) {
    const I t = t0 + I(u * kThreads);
    if (t >= nvec) continue;
    const I row = t / D4;  // (b, s, h) row index in [B*S*H]
    const I h = row % H;
    const I bs = row / H;
    const I sI = bs % S;
    const I b = bs / S;
    li[u] = (b * H + h) * S + sI;  // lse index [b][h][s]
    w[u] = merge_weights(lse_acc[li[u]], lse_blk[li[u]]);
    a[u] = *reinterpret_cast<const f32x4*>(acc + int64_t(t) * 4);
    if constexpr (kBf16) {
      const u16x4 r = *reinterpret_cast<const u16x4*>(static_cast<const uint16_t*>(blk) + int64_t(t) * 4);
      x[u] = f32x4{bf16_to_f32(r.x), bf16_to_f32(r.y), bf16_to_f32(r.z), bf16_to_f32(r.w)};
    } else {
      x[u] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(blk) + int64_t(t) * 4);
    }
  }
#pragma unroll
  for (int u = 0; u < kVPT; ++u) {
    const I t = t0 + I(u * kThreads);
    if (t >= nvec) continue;
    const float wa = w[u].wa, wb = w[u].wb;
    f32x4 o;
    o.x = a[u].x * wa + x[u].x * wb;
    o.y = a[u].y * wa + x[u].y * wb;
    o.z = a[u].z * wa + x[u].z * wb;
    o.w = a[u].w * wa + x[u].w * wb;
    *reinterpret_cast<f32x4*>(acc + int64_t(t) * 4) = o;
    if (t % D4 == 0) lse_acc[li[u]] = w[u].lse;
  }
}

template <bool kBf16>
void launch_merge_t(int64_t B, int64_t S, int64_t H, int64_t D, float* acc, float* lse_acc, const void* blk,
                    const float* lse_blk, hipStream_t s) {
  const int64_t nvec = B * S * H * (D / 4);
  const unsigned grid = unsigned((nvec + kThreads * kVPT - 1) / (kThreads * kVPT));
  hipLaunchKernelGGL((lse_merge_kernel<kBf16>), dim3(grid), dim3(kThreads), 0, s, acc, lse_acc, blk, lse_blk,
                     I(S), I(H), I(D / 4), I(nvec));
}

}  // namespace

hipError_t launch_lse_merge(int64_t B, int64_t S, int64_t H, int64_t D, float* acc, float* lse_acc,
                            const void* blk, const float* lse_blk, int blk_is_bf16, hipStream_t s) {
  // the caller keeps B*S*H*D/4 + 512 below 2^31, so every vector index fits
  ProfScope ps(s, kProfLseMerge);
  if (blk_is_bf16)
    launch_merge_t<true>(B, S, H, D, acc, lse_acc, blk, lse_blk, s);
  else
    launch_merge_t<false>(B, S, H, D, acc, lse_acc, blk, lse_blk, s);
  return hipGetLastError();
}

}  // namespace cp

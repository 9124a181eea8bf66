// Row-per-wavefront attention kernels (forward and backward).
//
// These serve the float32 problems (small head counts and sequence lengths, e.g.
// the handbook's toy data) and bf16 head dims the matrix-core kernels are not
// built for (any D <= 128 other than 32, 64, 128, e.g. 16).  All arithmetic is
// float32; bf16 inputs are widened on load and the bf16 output is rounded to
// nearest even.  One
// wavefront owns one row; a lane holds head-dim elements d = lane + 64*t, dot
// products are wavefront sums, and keys are visited one at a time with the online
// softmax.
//
// Definition: handbook "Context parallelism: Ring Attention and Ulysses",
// §"Which operations partition directly" (attention with offsets returning the
// log-sum-exp); gradient: the softmax-attention VJP with Delta_i = dO_i . O_i.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "prof.h"

namespace cp {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

CP_DEVICE int qpos_of(const AttnProblem& p, int i) { return p.q_pos ? p.q_pos[i] : p.q_offset + i; }
CP_DEVICE int kpos_of(const AttnProblem& p, int j) { return p.k_pos ? p.k_pos[j] : p.k_offset + j; }

// NT = ceil(D / 64) elements per lane.  kMerge = true (fused ring step): out is the
// float32 accumulator and lse the accumulator's lse, merged in place.
template <typename T, bool kMerge>
using OutT = typename std::conditional<kMerge, float, T>::type;

template <typename T, int NT, bool kMerge>
__global__ __launch_bounds__(kThreads) void fwd_rowwise_kernel(AttnProblem p, const T* __restrict__ q,
                                                               const T* __restrict__ k,
                                                               const T* __restrict__ v,
                                                               OutT<T, kMerge>* __restrict__ out,
                                                               float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int h = blockIdx.y, b = blockIdx.z;
  if (i >= p.Sq) return;
  const int g = h / (p.Hq / p.Hkv);
  const int D = p.D;
  const MaskSpec ms = make_mask_spec(p.causal, p.window, p.q_seg != nullptr);
  const T* qr = q + ((int64_t(b) * p.Sq + i) * p.Hq + h) * D;
  float qv[NT], acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int d = lane + 64 * t;
    qv[t] = d < D ? Elem<T>::load(qr + d) : 0.0f;
    acc[t] = 0.0f;
  }
  const int qp = qpos_of(p, i);
  const int qs = ms.has_seg ? p.q_seg[int64_t(b) * p.Sq + i] : 0;
  float m = -INFINITY, l = 0.0f;
  for (int j = 0; j < p.Sk; ++j) {
    const int ks = ms.has_seg ? p.k_seg[int64_t(b) * p.Sk + j] : 0;
    if (!pair_visible(ms, qp, kpos_of(p, j), qs, ks)) continue;
    const T* kr = k + ((int64_t(b) * p.Sk + j) * p.Hkv + g) * D;
    const T* vr = v + ((int64_t(b) * p.Sk + j) * p.Hkv + g) * D;
    float dot = 0.0f;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int d = lane + 64 * t;
      if (d < D) dot += qv[t] * Elem<T>::load(kr + d);
    }
    const float s = wave_sum(dot) * p.scale;
    const float mn = fmaxf(m, s);
    const float alpha = expf(m - mn);  // m = -inf on the first visible key -> 0
    const float pr = expf(s - mn);
    l = l * alpha + pr;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int d = lane + 64 * t;
      acc[t] = acc[t] * alpha + (d < D ? pr * Elem<T>::load(vr + d) : 0.0f);
    }
    m = mn;
  }
  OutT<T, kMerge>* orow = out + ((int64_t(b) * p.Sq + i) * p.Hq + h) * D;
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  const float lse_blk = l > 0.0f ? m + logf(l) : -INFINITY;
  const int64_t li = (int64_t(b) * p.Hq + h) * p.Sq + i;
  if constexpr (kMerge) {
    // every lane reads the old lse (one wave-wide load) before lane 0 writes it
    const MergeWeights w = merge_weights(lse[li], lse_blk);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int d = lane + 64 * t;
      if (d < D) orow[d] = orow[d] * w.wa + acc[t] * inv * w.wb;
    }
    if (lane == 0) lse[li] = w.lse;
  } else {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int d = lane + 64 * t;
      if (d < D) Elem<T>::store(orow + d, acc[t] * inv);
    }
    if (lane == 0) lse[li] = lse_blk;
  }
}

// Delta[b,h,i] = sum_d dO[b,i,h,d] * O[b,i,h,d]; one wavefront per row.
template <typename T, int NT>
__global__ __launch_bounds__(kThreads) void delta_rowwise_kernel(int B, int Sq, int Hq, int D,
                                                                 const T* __restrict__ out,
                                                                 const T* __restrict__ dout,
                                                                 float* __restrict__ delta) {
  const int lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * kWaves + (threadIdx.x >> 6);  // (b, i, h)
  if (row >= int64_t(B) * Sq * Hq) return;
  const T* o = out + row * D;
  const T* g = dout + row * D;
  float x = 0.0f;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int d = lane + 64 * t;
    if (d < D) x += Elem<T>::load(o + d) * Elem<T>::load(g + d);
  }
  x = wave_sum(x);
  if (lane == 0) {
    const int h = int(row % Hq);
    const int64_t bi = row / Hq;
    const int i = int(bi % Sq);
    const int64_t b = bi / Sq;
    delta[(b * Hq + h) * Sq + i] = x;
  }
}

// dQ: one wavefront per (b, i, h) query row.
template <typename T, int NT>
__global__ __launch_bounds__(kThreads) void dq_rowwise_kernel(AttnProblem p, const T* __restrict__ q,
                                                              const T* __restrict__ k,
                                                              const T* __restrict__ v,
                                                              const float* __restrict__ lse,
                                                              const T* __restrict__ dout,
                                                              const float* __restrict__ delta,
                                                              float* __restrict__ dq, int accumulate) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int h = blockIdx.y, b = blockIdx.z;
  if (i >= p.Sq) return;
  const int g = h / (p.Hq / p.Hkv);
  const int D = p.D;
  const MaskSpec ms = make_mask_spec(p.causal, p.window, p.q_seg != nullptr);
  const int64_t qrow = ((int64_t(b) * p.Sq + i) * p.Hq + h) * D;
  float qv[NT], gv[NT], acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int d = lane + 64 * t;
    qv[t] = d < D ? Elem<T>::load(q + qrow + d) : 0.0f;
    gv[t] = d < D ? Elem<T>::load(dout + qrow + d) : 0.0f;
    acc[t] = 0.0f;
  }
  const int64_t li = (int64_t(b) * p.Hq + h) * p.Sq + i;
  const float L = lse[li];
  const float dl = delta[li];
  if (L != -INFINITY) {
    const int qp = qpos_of(p, i);
    const int qs = ms.has_seg ? p.q_seg[int64_t(b) * p.Sq + i] : 0;
    for (int j = 0; j < p.Sk; ++j) {
      const int ks = ms.has_seg ? p.k_seg[int64_t(b) * p.Sk + j] : 0;
      if (!pair_visible(ms, qp, kpos_of(p, j), qs, ks)) continue;
      const T* kr = k + ((int64_t(b) * p.Sk + j) * p.Hkv + g) * D;
      const T* vr = v + ((int64_t(b) * p.Sk + j) * p.Hkv + g) * D;
      float sdot = 0.0f, pdot = 0.0f;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int d = lane + 64 * t;
        if (d < D) {
          sdot += qv[t] * Elem<T>::load(kr + d);
          pdot += gv[t] * Elem<T>::load(vr + d);
        }
      }
      const float s = wave_sum(sdot) * p.scale;
      const float dp = wave_sum(pdot);
      const float pr = expf(s - L);
      const float ds = pr * (dp - dl) * p.scale;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int d = lane + 64 * t;
        if (d < D) acc[t] += ds * Elem<T>::load(kr + d);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int d = lane + 64 * t;
    if (d < D) dq[qrow + d] = accumulate ? dq[qrow + d] + acc[t] : acc[t];
  }
}

// dK, dV: one wavefront per (b, j, g) key row, summing over the group's query heads.
template <typename T, int NT>
__global__ __launch_bounds__(kThreads) void dkdv_rowwise_kernel(AttnProblem p, const T* __restrict__ q,
                                                                const T* __restrict__ k,
                                                                const T* __restrict__ v,
                                                                const float* __restrict__ lse,
                                                                const T* __restrict__ dout,
                                                                const float* __restrict__ delta,
                                                                float* __restrict__ dk,
                                                                float* __restrict__ dv,
                                                                int accumulate) {
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int g = blockIdx.y, b = blockIdx.z;
  if (j >= p.Sk) return;
  const int G = p.Hq / p.Hkv;
  const int D = p.D;
  const MaskSpec ms = make_mask_spec(p.causal, p.window, p.q_seg != nullptr);
  const int64_t krow = ((int64_t(b) * p.Sk + j) * p.Hkv + g) * D;
  float kv[NT], vv[NT], ak[NT], av[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int d = lane + 64 * t;
    kv[t] = d < D ? Elem<T>::load(k + krow + d) : 0.0f;
    vv[t] = d < D ? Elem<T>::load(v + krow + d) : 0.0f;
    ak[t] = av[t] = 0.0f;
  }
  const int kp = kpos_of(p, j);
  const int ks = ms.has_seg ? p.k_seg[int64_t(b) * p.Sk + j] : 0;
  for (int hh = 0; hh < G; ++hh) {
    const int h = g * G + hh;
    for (int i = 0; i < p.Sq; ++i) {
      const int qs = ms.has_seg ? p.q_seg[int64_t(b) * p.Sq + i] : 0;
      if (!pair_visible(ms, qpos_of(p, i), kp, qs, ks)) continue;
      const int64_t li = (int64_t(b) * p.Hq + h) * p.Sq + i;
      const float L = lse[li];
      if (L == -INFINITY) continue;
      const int64_t qrow = ((int64_t(b) * p.Sq + i) * p.Hq + h) * D;
      float sdot = 0.0f, pdot = 0.0f;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int d = lane + 64 * t;
        if (d < D) {
          sdot += Elem<T>::load(q + qrow + d) * kv[t];
          pdot += Elem<T>::load(dout + qrow + d) * vv[t];
        }
      }
      const float s = wave_sum(sdot) * p.scale;
      const float dp = wave_sum(pdot);
      const float pr = expf(s - L);
      const float ds = pr * (dp - delta[li]) * p.scale;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int d = lane + 64 * t;
        if (d < D) {
          av[t] += pr * Elem<T>::load(dout + qrow + d);
          ak[t] += ds * Elem<T>::load(q + qrow + d);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int d = lane + 64 * t;
    if (d < D) {
      dk[krow + d] = accumulate ? dk[krow + d] + ak[t] : ak[t];
      dv[krow + d] = accumulate ? dv[krow + d] + av[t] : av[t];
    }
  }
}

template <typename T, int NT, bool kMerge>
hipError_t fwd_nt(const AttnProblem& p, const T* q, const T* k, const T* v, OutT<T, kMerge>* out, float* lse,
                  hipStream_t s) {
  dim3 grid((p.Sq + kWaves - 1) / kWaves, p.Hq, p.B);
  ProfScope ps(s, kMerge ? kProfFwdMergeRowwise : kProfFwdRowwise);
  hipLaunchKernelGGL((fwd_rowwise_kernel<T, NT, kMerge>), grid, dim3(kThreads), 0, s, p, q, k, v, out, lse);
  return hipGetLastError();
}

template <typename T, int NT>
hipError_t bwd_nt(const AttnProblem& p, const T* q, const T* k, const T* v, const T* out,
                  const float* lse, const T* dout, float* dq, float* dk, float* dv, int accumulate,
                  float* delta, bool rows_ready, hipStream_t s) {
  const int64_t rows = int64_t(p.B) * p.Sq * p.Hq;
  ProfScope ps(s, kProfBwdRowwise);
  if (!rows_ready)
    hipLaunchKernelGGL((delta_rowwise_kernel<T, NT>), dim3(unsigned((rows + kWaves - 1) / kWaves)),
                     dim3(kThreads), 0, s, p.B, p.Sq, p.Hq, p.D, out, dout, delta);
  hipLaunchKernelGGL((dq_rowwise_kernel<T, NT>), dim3((p.Sq + kWaves - 1) / kWaves, p.Hq, p.B),
                     dim3(kThreads), 0, s, p, q, k, v, lse, dout, delta, dq, accumulate);
  hipLaunchKernelGGL((dkdv_rowwise_kernel<T, NT>), dim3((p.Sk + kWaves - 1) / kWaves, p.Hkv, p.B),
                     dim3(kThreads), 0, s, p, q, k, v, lse, dout, delta, dk, dv, accumulate);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_f32(const AttnProblem& p, const float* q, const float* k, const float* v,
                               float* out, float* lse, hipStream_t s) {
  return p.D <= 64 ? fwd_nt<float, 1, false>(p, q, k, v, out, lse, s)
                   : fwd_nt<float, 2, false>(p, q, k, v, out, lse, s);
}

hipError_t launch_attn_fwd_merge_f32(const AttnProblem& p, const float* q, const float* k, const float* v,
                                     float* acc, float* lse_acc, hipStream_t s) {
  return p.D <= 64 ? fwd_nt<float, 1, true>(p, q, k, v, acc, lse_acc, s)
                   : fwd_nt<float, 2, true>(p, q, k, v, acc, lse_acc, s);
}

hipError_t launch_attn_bwd_f32(const AttnProblem& p, const float* q, const float* k, const float* v,
                               const float* out, const float* lse, const float* dout, float* dq,
                               float* dk, float* dv, int accumulate, float* delta, bool rows_ready,
                               hipStream_t s) {
  return p.D <= 64 ? bwd_nt<float, 1>(p, q, k, v, out, lse, dout, dq, dk, dv, accumulate, delta, rows_ready, s)
                   : bwd_nt<float, 2>(p, q, k, v, out, lse, dout, dq, dk, dv, accumulate, delta, rows_ready, s);
}

hipError_t launch_attn_fwd_rowwise_bf16(const AttnProblem& p, const void* q, const void* k, const void* v,
                                        void* out, float* lse, hipStream_t s) {
  using U = const uint16_t*;
  return p.D <= 64 ? fwd_nt<uint16_t, 1, false>(p, U(q), U(k), U(v), static_cast<uint16_t*>(out), lse, s)
                   : fwd_nt<uint16_t, 2, false>(p, U(q), U(k), U(v), static_cast<uint16_t*>(out), lse, s);
}

hipError_t launch_attn_fwd_merge_rowwise_bf16(const AttnProblem& p, const void* q, const void* k,
                                              const void* v, float* acc, float* lse_acc, hipStream_t s) {
  using U = const uint16_t*;
  return p.D <= 64 ? fwd_nt<uint16_t, 1, true>(p, U(q), U(k), U(v), acc, lse_acc, s)
                   : fwd_nt<uint16_t, 2, true>(p, U(q), U(k), U(v), acc, lse_acc, s);
}

hipError_t launch_attn_bwd_rowwise_bf16(const AttnProblem& p, const void* q, const void* k, const void* v,
                                        const void* out, const float* lse, const void* dout, float* dq,
                                        float* dk, float* dv, int accumulate, float* delta, bool rows_ready,
                                        hipStream_t s) {
  using U = const uint16_t*;
  return p.D <= 64 ? bwd_nt<uint16_t, 1>(p, U(q), U(k), U(v), U(out), lse, U(dout), dq, dk, dv, accumulate, delta, rows_ready, s)
                   : bwd_nt<uint16_t, 2>(p, U(q), U(k), U(v), U(out), lse, U(dout), dq, dk, dv, accumulate, delta, rows_ready, s);
}

}  // namespace cp

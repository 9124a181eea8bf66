// Internal helpers shared by the HIP kernels of libcp_attn (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define CP_DEVICE __device__ __forceinline__

namespace cp {

// ---- bf16 <-> f32 -------------------------------------------------------------
// bf16 is stored as its 16 raw bits.  Widening is exact (shift into the high half).
CP_DEVICE float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Narrowing rounds to nearest, ties to even, through the compiler's __bf16 cast
// (one v_cvt_pk_bf16_f32 on gfx950).
CP_DEVICE uint16_t f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}

CP_DEVICE uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  static CP_DEVICE float load(const float* p) { return *p; }
  static CP_DEVICE void store(float* p, float x) { *p = x; }
};
template <> struct Elem<uint16_t> {
  static CP_DEVICE float load(const uint16_t* p) { return bf16_to_f32(*p); }
  static CP_DEVICE void store(uint16_t* p, float x) { *p = f32_to_bf16(x); }
};

// ---- wave64 reductions ----------------------------------------------------------
CP_DEVICE float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// ---- visibility of a (query, key) pair -------------------------------------------
// Positions are global token indices in [0, 2^31); segments int32 document ids.  The
// key at kp is visible to the query at qp iff kp <= qp (causal), qp - kp < window
// (when a window is given; the host turns the causal rule on with any window, so a
// window means 0 <= qp - kp < window) and both carry the same segment id (when
// given).  With d = qp - kp in (-2^31, 2^31) the position rules are one unsigned
// range test, (d - lo) mod 2^32 < span:
//   causal:     lo = 0,          span = window, or 2^31 without one (d >= 0);
//   not causal: lo = 1 - 2^31,   span = 2^32 - 1 (any d).
struct MaskSpec {
  uint32_t lo, span;
  int has_seg;
};

inline __host__ __device__ MaskSpec make_mask_spec(int causal, int window, int has_seg) {
  if (causal || window) return MaskSpec{0u, window ? uint32_t(window) : (1u << 31), has_seg};
  return MaskSpec{1u - (1u << 31), 0xffffffffu, has_seg};
}

// Branch-free (bitwise) so that per-element masks compile to compares and selects.
CP_DEVICE bool pair_visible(const MaskSpec& m, int qp, int kp, int qs, int ks) {
  const bool pos = uint32_t(qp) - uint32_t(kp) - m.lo < m.span;
  const bool seg = (m.has_seg == 0) | (qs == ks);
  return pos & seg;
}

// Log-sum-exp merge of two parts of a row (handbook "Context parallelism: Ring
// Attention and Ulysses", self-test answers and the ring merge): the merged
// lse = log(e^la + e^lb) and the weights e^(la - lse), e^(lb - lse) of the parts.  A
// part with lse -inf has weight 0; both -inf gives lse = -inf and weights 0.
struct MergeWeights {
  float lse, wa, wb;
};
CP_DEVICE MergeWeights merge_weights(float la, float lb) {
  const float mx = fmaxf(la, lb);
  MergeWeights r{mx, 0.0f, 0.0f};
  if (mx != -INFINITY) {
    // computed from the larger part, so it cannot overflow
    r.lse = mx + log1pf(__expf(fminf(la, lb) - mx));
    r.wa = la == -INFINITY ? 0.0f : __expf(la - r.lse);
    r.wb = lb == -INFINITY ? 0.0f : __expf(lb - r.lse);
  }
  return r;
}

}  // namespace cp

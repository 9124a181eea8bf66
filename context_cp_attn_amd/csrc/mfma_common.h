// Shared pieces of the bf16 matrix-core attention kernels (gfx950, wave64).
//
// Operand conventions for v_mfma_f32_32x32x16_bf16 (A: 32xK16, B: K16x32, C/D 32x32):
//  * A fragment: lane l holds row (l % 32), 8 consecutive k-slots 8*(l/32)..+7;
//    B fragment: lane l holds column (l % 32), the same 8 k-slots.  Both sides of
//    a product load their k-slots with the same mapping, so the k order is free.
//  * C/D: lane l holds column (l % 32); register r holds row 8*(r/4) + 4*(l/32) + r%4.
//  * Loading the A rows of a product with bits 2 and 3 of the row index swapped
//    (perm_row) makes register r of lane half h hold row key_of_reg(r, h), so that
//    registers 8t..8t+7 are the 8 consecutive rows 16t + 8h + (0..7): exactly the
//    k-slots of a B fragment in the next product, with no data exchange.
#pragma once

#include "common.h"
#include "launch.h"

namespace cp {
namespace mfma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

CP_DEVICE f32x16 mma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

CP_DEVICE bf16x8 ld8(const uint16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }

// bf16 B/A fragment from 8 consecutive float registers
CP_DEVICE bf16x8 to_bf16x8(const f32x16& x, int base) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = static_cast<__bf16>(x[base + e]);
  return r;
}

CP_DEVICE constexpr int perm_row(int m) { return (m & 0x13) | ((m & 4) << 1) | ((m & 8) >> 1); }
CP_DEVICE constexpr int key_of_reg(int r, int h) { return 16 * (r >> 3) + 8 * h + (r & 7); }

CP_DEVICE float other_half(float x) { return __shfl_xor(x, 32, 64); }

// ---- tile classification -------------------------------------------------------
enum : int { kEmpty = 0, kPartial = 1, kFull = 2 };

// Extreme positions and segment ids of a run of tokens (both are monotone).
struct Span {
  int pos_lo, pos_hi, seg_lo, seg_hi;
};

CP_DEVICE int qpos_at(const AttnProblem& p, int i) { return p.q_pos ? p.q_pos[i] : p.q_offset + i; }
CP_DEVICE int kpos_at(const AttnProblem& p, int j) { return p.k_pos ? p.k_pos[j] : p.k_offset + j; }
CP_DEVICE int qseg_at(const AttnProblem& p, int b, int i) { return p.q_seg ? p.q_seg[int64_t(b) * p.Sq + i] : 0; }
CP_DEVICE int kseg_at(const AttnProblem& p, int b, int j) { return p.k_seg ? p.k_seg[int64_t(b) * p.Sk + j] : 0; }

CP_DEVICE Span q_span(const AttnProblem& p, int b, int r0, int r1) {
  return Span{qpos_at(p, r0), qpos_at(p, r1), qseg_at(p, b, r0), qseg_at(p, b, r1)};
}
CP_DEVICE Span k_span(const AttnProblem& p, int b, int j0, int j1) {
  return Span{kpos_at(p, j0), kpos_at(p, j1), kseg_at(p, b, j0), kseg_at(p, b, j1)};
}

// empty: no pair of the two runs is visible; full: every pair is (and nothing ragged)
CP_DEVICE int classify(const AttnProblem& p, const Span& q, const Span& k, bool ragged) {
  if (p.causal && k.pos_lo > q.pos_hi) return kEmpty;
  if (p.window && q.pos_lo - k.pos_hi >= p.window) return kEmpty;
  if (p.q_seg && (k.seg_hi < q.seg_lo || k.seg_lo > q.seg_hi)) return kEmpty;
  bool full = !ragged;
  if (p.causal) full = full && (k.pos_hi <= q.pos_lo);
  if (p.window) full = full && (q.pos_hi - k.pos_lo < p.window);
  if (p.q_seg) full = full && (q.seg_lo == q.seg_hi) && (k.seg_lo == k.seg_hi) && (q.seg_lo == k.seg_lo);
  return full ? kFull : kPartial;
}

// ---- a tile of NR token rows x D dims (bf16): global -> registers -> LDS ----------
// Work unit = 4 rows x 8 dims (four 16-byte loads); consecutive threads take
// consecutive 8-dim columns of the same 4 rows, so a load instruction of a wave
// reads whole rows.  The same registers can be stored row-major ([NR][ld]) or
// transposed ([D][ld]) into LDS.
template <int NR, int D, int NT>
struct RowTile {
  static constexpr int kUnits = (NR / 4) * (D / 8);
  static constexpr int kIter = (kUnits + NT - 1) / NT;
  static_assert(NR % 4 == 0 && D % 8 == 0, "tile shape");
  u32x4 r[kIter][4];

  CP_DEVICE void load(const uint16_t* __restrict__ base, int64_t row_stride, int row0, int nrows) {
#pragma unroll
    for (int it = 0; it < kIter; ++it) {
      const int u = int(threadIdx.x) + it * NT;
      const int r4 = u / (D / 8);
      const int d8 = u - r4 * (D / 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = r4 * 4 + e;
        r[it][e] = u32x4{0, 0, 0, 0};
        if (u < kUnits && row0 + row < nrows)
          r[it][e] = *reinterpret_cast<const u32x4*>(base + int64_t(row0 + row) * row_stride + d8 * 8);
      }
    }
  }

  CP_DEVICE void store_rows(uint16_t* lds, int ld) const {
#pragma unroll
    for (int it = 0; it < kIter; ++it) {
      const int u = int(threadIdx.x) + it * NT;
      const int r4 = u / (D / 8);
      const int d8 = u - r4 * (D / 8);
      if (u < kUnits) {
#pragma unroll
        for (int e = 0; e < 4; ++e) *reinterpret_cast<u32x4*>(lds + (r4 * 4 + e) * ld + d8 * 8) = r[it][e];
      }
    }
  }

  // transposed: row d of the LDS tile holds dim d of the NR tokens
  CP_DEVICE void store_cols(uint16_t* lds, int ld) const {
#pragma unroll
    for (int it = 0; it < kIter; ++it) {
      const int u = int(threadIdx.x) + it * NT;
      const int r4 = u / (D / 8);
      const int d8 = u - r4 * (D / 8);
      if (u < kUnits) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {  // dims 2w, 2w+1 live in 32-bit word w
          const uint32_t a0 = r[it][0][w], a1 = r[it][1][w], a2 = r[it][2][w], a3 = r[it][3][w];
          const u32x2 lo{(a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16)};
          const u32x2 hi{(a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u)};
          *reinterpret_cast<u32x2*>(lds + (d8 * 8 + 2 * w) * ld + r4 * 4) = lo;
          *reinterpret_cast<u32x2*>(lds + (d8 * 8 + 2 * w + 1) * ld + r4 * 4) = hi;
        }
      }
    }
  }
};

}  // namespace mfma
}  // namespace cp

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

// x of lane l combined with x of lane l ^ 32, in every lane.  v_permlane32_swap
// (one VALU op) hands each lane both halves' values: r[0] = x[l mod 32], r[1] =
// x[32 + l mod 32]; a cross-lane shuffle would be an LDS round trip.
CP_DEVICE float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
CP_DEVICE float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---- tile classification -------------------------------------------------------
enum : int { kEmpty = 0, kPartial = 1, kFull = 2 };

// Extreme positions and segment ids of a run of tokens (both are monotone).
struct Span {
  int pos_lo, pos_hi, seg_lo, seg_hi;
};
// Keeps v in a vector register, redefined here as far as the optimizer knows: values
// derived from it after this point are computed there, neither hoisted out of the
// loop around it nor kept live from earlier uses.
template <class T>
CP_DEVICE void pin(T& v) {
  asm volatile("" : "+v"(v));
}

// A span of wave-uniform rows, held in scalar registers (the compiler cannot always
// prove the uniformity of values loaded or derived from the wavefront index).
CP_DEVICE Span uniform(const Span& s) {
  return Span{__builtin_amdgcn_readfirstlane(s.pos_lo), __builtin_amdgcn_readfirstlane(s.pos_hi),
              __builtin_amdgcn_readfirstlane(s.seg_lo), __builtin_amdgcn_readfirstlane(s.seg_hi)};
}

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

// With positions strictly increasing and segment ids non-decreasing along q and
// along k (the documented preconditions the tile classification above already
// relies on), the key runs wholly before a query run's window / segments form a
// prefix of the key tiles, and those wholly after its causal horizon / segments a
// suffix: the live tiles of a run lie in one contiguous range, found by bisection
// instead of classifying every empty tile.
CP_DEVICE bool keys_before(const AttnProblem& p, const Span& q, const Span& k) {
  return (p.window && q.pos_lo - k.pos_hi >= p.window) || (p.q_seg && k.seg_hi < q.seg_lo);
}
CP_DEVICE bool keys_after(const AttnProblem& p, const Span& q, const Span& k) {
  return (p.causal && k.pos_lo > q.pos_hi) || (p.q_seg && k.seg_lo > q.seg_hi);
}

// Smallest x in [lo, hi) with pred(x), else hi; pred must be false ... false true ... true.
template <class Pred>
CP_DEVICE int first_true(int lo, int hi, Pred&& pred) {
  while (lo < hi) {
    const int mid = lo + (hi - lo) / 2;
    if (pred(mid))
      hi = mid;
    else
      lo = mid + 1;
  }
  return lo;
}

// The kernel instances without the one-tile-per-lane classification (kLane = false)
// are launched only for problems with no window and no segment ids.  Their copy of
// the problem says so at compile time, so that the code paths of windowed and
// segmented problems (per-tile classification from span loads, segment compares)
// are not compiled into them and take no registers there.
template <bool kLane>
CP_DEVICE AttnProblem specialize(const AttnProblem& p) {
  AttnProblem r = p;
  if constexpr (!kLane) {
    r.window = 0;
    r.q_seg = nullptr;
    r.k_seg = nullptr;
  }
  return r;
}

// ---- buffer resources ---------------------------------------------------------------
// A raw buffer resource over nbytes from base: loads past the end read as zeros in
// hardware, so ragged tiles need neither selects nor 64-bit address arithmetic.
CP_DEVICE __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(nbytes), 0x00020000);
}

// N consecutive dwords of src from element first (valid of them exist; the rest
// read as 0) into lds, copied by one wavefront with N / 64 LDS-DMA loads (lane i
// writes dword i of each 64) and, for N an odd multiple of 32, one more load by the
// lower half of the wavefront (the upper half's lanes do not load).
template <int N>
CP_DEVICE void dma_dwords(const void* src, int64_t first, int valid, void* lds, int lane) {
  static_assert(N % 32 == 0, "whole half-wavefronts");
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(reinterpret_cast<const uint8_t*>(src) + first * 4, uint32_t(valid > 0 ? valid : 0) * 4u);
  uint8_t* dst = static_cast<uint8_t*>(lds);
#pragma unroll
  for (int c = 0; c < N / 64; ++c)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + 256 * c), 4,
                                            lane * 4 + 256 * c, 0, 0, 0);
  if constexpr (N % 64 != 0) {
    constexpr int c = N / 64;
    if (lane < 32)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + 256 * c), 4,
                                              lane * 4 + 256 * c, 0, 0, 0);
  }
}

// ---- row-major LDS tiles filled by LDS-DMA, read as rows or transposed ------------
// A tile of NR token rows x D dims is stored unpadded, row-major, with the 16-byte
// chunk c of row r placed at chunk c ^ chunk_xor<D>(r).  The XOR functions make
// both access patterns bank-conflict free (64 banks x 4 bytes):
//  * row fragments (8 consecutive dims of one row; 16 lanes read 16 distinct rows,
//    the A rows of a product loaded with perm_row);
//  * transposed fragments (8 consecutive rows of one dim) read with
//    ds_read_b64_tr_b16, where each group of 16 lanes addresses a 4-row x 16-dim
//    block and lane j receives dim j of the 4 rows.
template <int D>
CP_DEVICE constexpr int chunk_xor(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else if constexpr (D == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  else return (r >> 2) & 3;
}

template <int D>
CP_DEVICE int rm_elem(int row, int chunk) { return row * D + ((chunk ^ chunk_xor<D>(row)) << 3); }

// 8 consecutive dims (chunk c) of one row
template <int D>
CP_DEVICE bf16x8 ld_row(const uint16_t* tile, int row, int c) { return ld8(tile + rm_elem<D>(row, c)); }

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Transposed fragment: lane l receives rows rbase + 8*(l/32) + e (e = 0..7) of dim
// dbase + (l % 32) -- the A/B fragment layout with k-slots over rows.
template <int D>
CP_DEVICE bf16x8 ld_tr(const uint16_t* tile, int rbase, int dbase) {
  const int l = int(threadIdx.x) & 63, g = l >> 4, i = l & 15;
  const int d = dbase + 16 * (g & 1) + 4 * (i & 3);
  const int r = rbase + 8 * (g >> 1) + (i >> 2);
  const uint16_t* p0 = tile + r * D + (((d >> 3) ^ chunk_xor<D>(r)) << 3) + (d & 7);
  const uint16_t* p1 = tile + (r + 4) * D + (((d >> 3) ^ chunk_xor<D>(r + 4)) << 3) + (d & 7);
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0));
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p1));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

// Stage NR rows x D dims into a swizzled row-major LDS tile with LDS-DMA: each
// wavefront instruction moves 64 consecutive 16-byte LDS chunks, lane i fetching
// the global chunk that belongs at LDS chunk i.  Rows at or beyond nrows read as
// zeros (buffer range check).  Completion is tracked by vmcnt: wait for it before
// the barrier that publishes the tile.
template <int NR, int D, int NT>
struct DmaTile {
  static constexpr int kChunks = NR * D / 8;
  static constexpr int kIter = (kChunks + NT - 1) / NT;
  static_assert(kChunks % 64 == 0 && NT % 64 == 0, "whole wavefronts");
  uint32_t voff[kIter];
  int wbase;  // first thread of this wavefront within the NT loading threads

  // tid: this thread's index among the NT threads that load the tile together
  CP_DEVICE void init(uint32_t row_stride_bytes, int tid) {
    wbase = __builtin_amdgcn_readfirstlane(tid & ~63);
#pragma unroll
    for (int it = 0; it < kIter; ++it) {
      const int s = it * NT + tid;
      const int row = s / (D / 8), slot = s % (D / 8);
      voff[it] = uint32_t(row) * row_stride_bytes + uint32_t(slot ^ chunk_xor<D>(row)) * 16u;
    }
  }

  // buffer resource of rows [row0, nrows) (rows past nrows read as zeros)
  CP_DEVICE static __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t* base, uint32_t row_stride_bytes, int row0,
                                                    int nrows) {
    const uint32_t skip = uint32_t(row0) * row_stride_bytes;
    const uint32_t valid = uint32_t(nrows - 1 - row0) * row_stride_bytes + uint32_t(D) * 2u;
    return make_rsrc(reinterpret_cast<const uint8_t*>(base) + skip, valid);
  }

  // one of the kIter loads of this thread (it < kIter)
  CP_DEVICE void load_iter(const __amdgpu_buffer_rsrc_t& rs, int it, uint16_t* lds_tile) const {
    const int s0 = it * NT + wbase;  // first chunk of this wavefront
    if (kChunks % NT == 0 || s0 < kChunks)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(lds_tile + s0 * 8),
                                               16, voff[it], 0, 0, 0);
  }

  CP_DEVICE void load(const uint16_t* base, uint32_t row_stride_bytes, int row0, int nrows, uint16_t* lds_tile) const {
    const __amdgpu_buffer_rsrc_t rs = rows_rsrc(base, row_stride_bytes, row0, nrows);
#pragma unroll
    for (int it = 0; it < kIter; ++it) load_iter(rs, it, lds_tile);
  }
};

// Issue N matrix products whose A operands come from LDS with each operand read
// kAhead products ahead of its use: load(i) returns product i's fragment, mul(i, f)
// issues it.  Scheduling fences keep the order, so the reads are in flight while
// earlier products run instead of each product waiting for its own read.
template <int N, int kAhead, class Load, class Mul>
CP_DEVICE void pipelined_products(Load&& load, Mul&& mul) {
  if constexpr (kAhead == 0) {
#pragma unroll
    for (int i = 0; i < N; ++i) mul(i, load(i));
  } else {
    bf16x8 frag[kAhead + 1];
#pragma unroll
    for (int i = 0; i < kAhead && i < N; ++i) frag[i] = load(i);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if (i + kAhead < N) frag[(i + kAhead) % (kAhead + 1)] = load(i + kAhead);
      __builtin_amdgcn_sched_barrier(0);
      mul(i, frag[i % (kAhead + 1)]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Wait for every outstanding memory operation of this wavefront (LDS-DMA included).
CP_DEVICE void wait_all() { __builtin_amdgcn_s_waitcnt(0); }

// Workgroup barrier after this wavefront's LDS operations only: its vector-memory
// loads (the LDS-DMA of later tiles) stay in flight.  __syncthreads() would wait for
// those too: its memory fence is lowered to s_waitcnt vmcnt(0) before s_barrier.
// The signal fences and scheduling barriers keep the compiler from moving LDS
// accesses across it (s_barrier alone is not a memory operation to the optimizer).
CP_DEVICE void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
  // s_waitcnt lgkmcnt(0), vmcnt and expcnt at their maxima (gfx9 encoding)
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

}  // namespace mfma
}  // namespace cp

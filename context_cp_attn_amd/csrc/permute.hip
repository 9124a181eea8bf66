// Data-movement kernels: the Ulysses sequence<->head relayout of all simulated ranks,
// the zigzag (dual-chunk-swap) reorder and the striped reorder.  Both are permutations of contiguous
// byte runs, so each is a streaming copy: every thread moves VPT vectors of VB bytes,
// writes are fully coalesced in output order and reads are coalesced within a run.
//
// Ulysses relayout: handbook "Context parallelism: Ring Attention and Ulysses",
// §"Ulysses" (seq_to_head / head_to_seq).  A run is one rank's head slice of one
// token: (H/P)*D elements.
// Zigzag: the same handbook, §"The zigzag partition" (rank r takes chunks r and
// 2P-1-r); a run is one chunk of S/(2P) token rows.
// Striped: MaxText PR "Add Packing Support for Context Parallelism (Ring Attention)",
// reorder strategy 1 (token t to rank t mod P); a run is one token row.
// Padding: transformers PR "[distributed] Context parallel module, with Ulysses",
// "What this PR brings" (sequences padded at their end to a multiple of the CP size).
#include "common.h"
#include "launch.h"
#include "prof.h"

namespace cp {
namespace {

constexpr int kThreads = 128;
constexpr int kVPT = 1;  // vectors per thread per pass: loads issued before stores

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int VB> struct Vec;
template <> struct Vec<16> { using T = u32x4; };
template <> struct Vec<8> { using T = u32x2; };
template <> struct Vec<4> { using T = uint32_t; };
template <> struct Vec<2> { using T = uint16_t; };
template <> struct Vec<1> { using T = uint8_t; };

// in [P][B][Sp][P][R] (source rank s, batch, row i, destination p, vector r)
// out [P][B][P][Sp][R] (destination p, batch, source s, row i, vector r)
// One grid slice per (s, b) input span of Sp*P*R vectors, read in order; every run of
// R vectors goes to its destination rank's rows.
template <typename V>
__global__ __launch_bounds__(kThreads) void ulysses_fwd_kernel(const V* __restrict__ in,
                                                               V* __restrict__ out, int P, int B,
                                                               int Sp, int R, int blocks_per_span,
                                                               int64_t group_vecs) {
  const int span = blockIdx.x / blocks_per_span;
  const int blk = blockIdx.x - span * blocks_per_span;
  const int s = span / B;
  const int b = span - s * B;
  in += int64_t(blockIdx.y) * group_vecs;  // independent groups (USP), stacked outermost
  out += int64_t(blockIdx.y) * group_vecs;
  const uint32_t PR = uint32_t(P) * uint32_t(R);
  const uint32_t n = uint32_t(Sp) * PR;  // fits in 32 bits (checked by the launcher)
  const V* src = in + int64_t(span) * n;
  // element (i, p, r) of the span goes to ((p*B + b)*P + s)*Sp*R + i*R + r
  V* dst = out + (int64_t(b) * P + s) * Sp * int64_t(R);
  const int64_t pstride = int64_t(B) * P * Sp * R;
  for (uint32_t base = uint32_t(blk) * kThreads * kVPT + threadIdx.x; base < n;
       base += uint32_t(blocks_per_span) * kThreads * kVPT) {
    V vals[kVPT];
#pragma unroll
    for (int u = 0; u < kVPT; ++u) {
      const uint32_t idx = base + uint32_t(u) * kThreads;
      if (idx < n) vals[u] = __builtin_nontemporal_load(src + idx);
    }
#pragma unroll
    for (int u = 0; u < kVPT; ++u) {
      const uint32_t idx = base + uint32_t(u) * kThreads;
      if (idx < n) {
        const uint32_t i = idx / PR;
        const uint32_t rem = idx - i * PR;
        const uint32_t p = rem / uint32_t(R);
        const uint32_t r = rem - p * uint32_t(R);
        __builtin_nontemporal_store(vals[u], dst + int64_t(p) * pstride + int64_t(i) * R + r);
      }
    }
  }
}

// in [P][B][P][Sp][R] (p, b, s, i, r) -> out [P][B][Sp][P][R] (s, b, i, p, r).
// One grid slice per (s, b) output span of Sp*P*R vectors.
template <typename V>
__global__ __launch_bounds__(kThreads) void ulysses_inv_kernel(const V* __restrict__ in,
                                                               V* __restrict__ out, int P, int B,
                                                               int Sp, int R, int blocks_per_span,
                                                               int64_t group_vecs) {
  const int span = blockIdx.x / blocks_per_span;
  const int blk = blockIdx.x - span * blocks_per_span;
  const int s = span / B;
  const int b = span - s * B;
  in += int64_t(blockIdx.y) * group_vecs;
  out += int64_t(blockIdx.y) * group_vecs;
  const uint32_t PR = uint32_t(P) * uint32_t(R);
  const uint32_t n = uint32_t(Sp) * PR;  // fits in 32 bits (checked by the launcher)
  V* dst = out + int64_t(span) * n;
  // element (p, i, r) of the source lives at ((p*B + b)*P + s)*Sp*R + i*R + r
  const V* src = in + (int64_t(b) * P + s) * Sp * int64_t(R);
  const int64_t pstride = int64_t(B) * P * Sp * R;
  for (uint32_t base = uint32_t(blk) * kThreads * kVPT + threadIdx.x; base < n;
       base += uint32_t(blocks_per_span) * kThreads * kVPT) {
    V vals[kVPT];
#pragma unroll
    for (int u = 0; u < kVPT; ++u) {
      const uint32_t idx = base + uint32_t(u) * kThreads;
      if (idx < n) {
        const uint32_t i = idx / PR;
        const uint32_t rem = idx - i * PR;
        const uint32_t p = rem / uint32_t(R);
        const uint32_t r = rem - p * uint32_t(R);
        vals[u] = __builtin_nontemporal_load(src + int64_t(p) * pstride + int64_t(i) * R + r);
      }
    }
#pragma unroll
    for (int u = 0; u < kVPT; ++u) {
      const uint32_t idx = base + uint32_t(u) * kThreads;
      if (idx < n) __builtin_nontemporal_store(vals[u], dst + idx);
    }
  }
}

// Relayout with every head replicated rep times (head j of the replicated set is
// head j / rep; Hl = H*rep/P of them per destination): in [P][B][Sp][H][R1] ->
// out [P][B][S][Hl][R1], written in output order (one grid slice per (p, b) span).
template <typename V>
__global__ __launch_bounds__(kThreads) void ulysses_rep_kernel(const V* __restrict__ in, V* __restrict__ out,
                                                               int P, int B, int Sp, int H, int Hl, int rep,
                                                               int R1, int blocks_per_span, int64_t group_in,
                                                               int64_t group_out) {
  const int span = blockIdx.x / blocks_per_span;
  const int blk = blockIdx.x - span * blocks_per_span;
  const int p = span / B;
  const int b = span - p * B;
  in += int64_t(blockIdx.y) * group_in;
  const uint32_t HR = uint32_t(Hl) * uint32_t(R1);
  const uint32_t n = uint32_t(Sp) * uint32_t(P) * HR;  // fits in 32 bits (checked by the launcher)
  V* dst = out + int64_t(blockIdx.y) * group_out + int64_t(span) * n;
  for (uint32_t base = uint32_t(blk) * kThreads * kVPT + threadIdx.x; base < n;
       base += uint32_t(blocks_per_span) * kThreads * kVPT) {
    V vals[kVPT];
#pragma unroll
    for (int u = 0; u < kVPT; ++u) {
      const uint32_t idx = base + uint32_t(u) * kThreads;
      if (idx < n) {
        const uint32_t row = idx / HR;
        const uint32_t rem = idx - row * HR;
        const uint32_t hh = rem / uint32_t(R1);
        const uint32_t v = rem - hh * uint32_t(R1);
        const uint32_t s = row / uint32_t(Sp);
        const uint32_t i = row - s * uint32_t(Sp);
        const uint32_t head = (uint32_t(p) * uint32_t(Hl) + hh) / uint32_t(rep);
        vals[u] = __builtin_nontemporal_load(in + ((int64_t(s) * B + b) * Sp + i) * (int64_t(H) * R1) +
                                             int64_t(head) * R1 + v);
      }
    }
#pragma unroll
    for (int u = 0; u < kVPT; ++u) {
      const uint32_t idx = base + uint32_t(u) * kThreads;
      if (idx < n) __builtin_nontemporal_store(vals[u], dst + idx);
    }
  }
}

// Inverse of the replicated relayout for float32 gradients: out [P][B][Sp][H][R1]
// receives, for head h, the sum of its rep copies j = h*rep + t (t = 0..rep-1, in
// that order) from in [P][B][S][Hl][R1].  One grid slice per (s, b) span.
template <typename V>
__global__ __launch_bounds__(kThreads) void ulysses_inv_sum_kernel(const V* __restrict__ in, V* __restrict__ out,
                                                                   int P, int B, int Sp, int H, int Hl, int rep,
                                                                   int R1, int blocks_per_span, int64_t group_in,
                                                                   int64_t group_out) {
  const int span = blockIdx.x / blocks_per_span;
  const int blk = blockIdx.x - span * blocks_per_span;
  const int s = span / B;
  const int b = span - s * B;
  in += int64_t(blockIdx.y) * group_in;
  const uint32_t HR = uint32_t(H) * uint32_t(R1);
  const uint32_t n = uint32_t(Sp) * HR;
  V* dst = out + int64_t(blockIdx.y) * group_out + int64_t(span) * n;
  const int64_t S = int64_t(P) * Sp;
  for (uint32_t idx = uint32_t(blk) * kThreads + threadIdx.x; idx < n;
       idx += uint32_t(blocks_per_span) * kThreads) {
    const uint32_t i = idx / HR;
    const uint32_t rem = idx - i * HR;
    const uint32_t h = rem / uint32_t(R1);
    const uint32_t v = rem - h * uint32_t(R1);
    V acc{};
    for (int t = 0; t < rep; ++t) {
      const uint32_t j = h * uint32_t(rep) + uint32_t(t);
      const uint32_t p = j / uint32_t(Hl);
      const uint32_t hh = j - p * uint32_t(Hl);
      acc += __builtin_nontemporal_load(in + ((int64_t(p) * B + b) * S + int64_t(s) * Sp + i) * (int64_t(Hl) * R1) +
                                        int64_t(hh) * R1 + v);
    }
    __builtin_nontemporal_store(acc, dst + idx);
  }
}

// Chunk copy: the output slot j of batch b receives input chunk order(j) (forward)
// or the output chunk order(j) receives input slot j (inverse), where order(2r) = r
// and order(2r+1) = 2P-1-r.
template <typename V>
__global__ __launch_bounds__(kThreads) void zigzag_kernel(const V* __restrict__ in,
                                                          V* __restrict__ out, int P,
                                                          int64_t chunk_vecs, int inverse,
                                                          int blocks_per_span) {
  const int span = blockIdx.x / blocks_per_span;
  const int blk = blockIdx.x - span * blocks_per_span;
  const int nch = 2 * P;
  const int b = span / nch;
  const int slot = span - b * nch;
  const int r = slot >> 1;
  const int chunk = (slot & 1) ? (nch - 1 - r) : r;
  const int src_c = inverse ? slot : chunk;
  const int dst_c = inverse ? chunk : slot;
  const V* src = in + (int64_t(b) * nch + src_c) * chunk_vecs;
  V* dst = out + (int64_t(b) * nch + dst_c) * chunk_vecs;
  for (int64_t base = (int64_t(blk) * kThreads * kVPT) + threadIdx.x; base < chunk_vecs;
       base += int64_t(blocks_per_span) * kThreads * kVPT) {
    V vals[kVPT];
#pragma unroll
    for (int u = 0; u < kVPT; ++u) {
      const int64_t idx = base + int64_t(u) * kThreads;
      if (idx < chunk_vecs) vals[u] = __builtin_nontemporal_load(src + idx);
    }
#pragma unroll
    for (int u = 0; u < kVPT; ++u) {
      const int64_t idx = base + int64_t(u) * kThreads;
      if (idx < chunk_vecs) __builtin_nontemporal_store(vals[u], dst + idx);
    }
  }
}

// Striped reorder (token t -> rank t mod P; ranks' shares in rank order), c = S/P:
// forward, output row r*c + j of a batch takes input row j*P + r; the inverse takes
// it back.  Each block copies rows_per_block whole output rows (vector v of row o).
template <typename V>
__global__ __launch_bounds__(kThreads) void striped_kernel(const V* __restrict__ in, V* __restrict__ out,
                                                           int S, int P, int RV, int rows_per_block,
                                                           int64_t rows, int inverse) {
  const int64_t row0 = int64_t(blockIdx.x) * rows_per_block;
  const int c = S / P;
  const int n = rows_per_block * RV;
  for (int base = threadIdx.x; base < n; base += kThreads * kVPT) {
    V vals[kVPT];
    int64_t dst[kVPT];
#pragma unroll
    for (int u = 0; u < kVPT; ++u) {
      const int l = base + u * kThreads;
      dst[u] = -1;
      if (l < n) {
        const int lr = l / RV;
        const int v = l - lr * RV;
        const int64_t o = row0 + lr;  // output row over all batches
        if (o < rows) {
          const int64_t b = o / S;
          const int t = int(o - b * S);
          // forward: t = r*c + j <- j*P + r; inverse: t = j*P + r <- r*c + j
          const int src_t = inverse ? (t % P) * c + t / P : (t % c) * P + t / c;
          vals[u] = __builtin_nontemporal_load(in + (b * S + src_t) * RV + v);
          dst[u] = o * RV + v;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kVPT; ++u)
      if (dst[u] >= 0) __builtin_nontemporal_store(vals[u], out + dst[u]);
  }
}

// Pad (or truncate) every batch's sequence to S_out rows: rows t < min(S, S_out) are
// copied, rows t >= S are filled with a repeated 32-bit word.  Output-ordered, one
// grid slice per batch.  Vectors of VB bytes; fill is the word pattern as a vector.
template <typename V>
__global__ __launch_bounds__(kThreads) void pad_rows_kernel(const V* __restrict__ in, V* __restrict__ out,
                                                            int64_t S, int64_t S_out, int64_t RV, V fill,
                                                            int blocks_per_span) {
  const int b = blockIdx.x / blocks_per_span;
  const int blk = blockIdx.x - b * blocks_per_span;
  const int64_t n = S_out * RV;
  const int64_t copy = (S < S_out ? S : S_out) * RV;  // vectors of real rows
  const V* src = in + int64_t(b) * S * RV;
  V* dst = out + int64_t(b) * n;
  for (int64_t base = int64_t(blk) * kThreads * kVPT + threadIdx.x; base < n;
       base += int64_t(blocks_per_span) * kThreads * kVPT) {
    V vals[kVPT];
#pragma unroll
    for (int u = 0; u < kVPT; ++u) {
      const int64_t idx = base + int64_t(u) * kThreads;
      vals[u] = fill;
      if (idx < copy) vals[u] = __builtin_nontemporal_load(src + idx);
    }
#pragma unroll
    for (int u = 0; u < kVPT; ++u) {
      const int64_t idx = base + int64_t(u) * kThreads;
      if (idx < n) __builtin_nontemporal_store(vals[u], dst + idx);
    }
  }
}

int pick_vec_bytes(int64_t run_bytes, const void* a, const void* b) {
  const uintptr_t al = reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b);
  for (int vb = 16; vb > 1; vb >>= 1)
    if (run_bytes % vb == 0 && al % vb == 0) return vb;
  return 1;
}

// Blocks per span so that the whole grid has about 131072 small blocks (512 per CU
// of 256; a 256 MiB bf16 tensor then takes one 2 KiB pass per block: one 16-byte
// vector per thread) while a span never gets more blocks than it has work.  Many
// short blocks keep more loads in flight per CU than fewer blocks that each issue
// several loads before their stores.  Measured on the llama2-7b relayout shapes and
// the 64K-token reorder: from 16384 blocks of 256 threads x 4 vectors to this, the
// bf16 seq->head relayout 5.54 -> 6.25 TB/s, its inverse 5.59 -> 6.20, the 64K
// reorder 6.24 -> 6.45; in between, 65536 blocks of 256 x 1 reached 6.07 / 6.17 /
// 6.30 and 32768 of 256 x 2 5.71 / 5.79 / 6.25.
int blocks_for(int64_t spans, int64_t vecs_per_span) {
  const int64_t per_block = int64_t(kThreads) * kVPT;
  int64_t need = (vecs_per_span + per_block - 1) / per_block;
  int64_t want = (131072 + spans - 1) / spans;
  if (want < 1) want = 1;
  int64_t bps = need < want ? need : want;
  return int(bps < 1 ? 1 : bps);
}

template <int VB>
hipError_t ulysses_vb(const RelayoutProblem& r, const void* in, void* out, hipStream_t s) {
  using V = typename Vec<VB>::T;
  const int P = int(r.P), B = int(r.B), Sp = int(r.S / r.P);
  const int R = int((r.H / r.P) * r.D * r.eb / VB);
  const int64_t group_vecs = r.B * r.S * r.H * r.D * r.eb / VB;  // one group's tensor, either side
  const int64_t spans = int64_t(P) * B;
  const int bps = blocks_for(spans * r.G, int64_t(Sp) * P * R);
  const dim3 grid(unsigned(spans * bps), unsigned(r.G));
  ProfScope ps(s, r.inverse ? kProfUlyssesInv : kProfUlysses);
  if (!r.inverse)
    hipLaunchKernelGGL(ulysses_fwd_kernel<V>, grid, dim3(kThreads), 0, s, static_cast<const V*>(in),
                       static_cast<V*>(out), P, B, Sp, R, bps, group_vecs);
  else
    hipLaunchKernelGGL(ulysses_inv_kernel<V>, grid, dim3(kThreads), 0, s, static_cast<const V*>(in),
                       static_cast<V*>(out), P, B, Sp, R, bps, group_vecs);
  return hipGetLastError();
}

template <int VB>
hipError_t ulysses_rep_vb(const RelayoutProblem& r, const void* in, void* out, hipStream_t s) {
  using V = typename Vec<VB>::T;
  const int P = int(r.P), B = int(r.B), Sp = int(r.S / r.P), H = int(r.H), rep = int(r.rep);
  const int Hl = int(r.H * r.rep / r.P);
  const int R1 = int(r.D * r.eb / VB);
  const int64_t spans = int64_t(P) * B;
  const int bps = blocks_for(spans * r.G, int64_t(r.S) * Hl * R1);
  const dim3 grid(unsigned(spans * bps), unsigned(r.G));
  ProfScope ps(s, kProfUlysses);
  hipLaunchKernelGGL(ulysses_rep_kernel<V>, grid, dim3(kThreads), 0, s, static_cast<const V*>(in),
                     static_cast<V*>(out), P, B, Sp, H, Hl, rep, R1, bps, r.P * r.B * Sp * int64_t(H) * R1,
                     r.P * r.B * r.S * int64_t(Hl) * R1);
  return hipGetLastError();
}

template <typename F>  // float or f32x4
hipError_t ulysses_inv_sum_f(const RelayoutProblem& r, const void* in, void* out, hipStream_t s) {
  const int P = int(r.P), B = int(r.B), Sp = int(r.S / r.P), H = int(r.H), rep = int(r.rep);
  const int Hl = int(r.H * r.rep / r.P);
  const int R1 = int(r.D * 4 / int(sizeof(F)));
  const int64_t spans = int64_t(P) * B;
  const int bps = blocks_for(spans * r.G, int64_t(Sp) * H * R1);
  const dim3 grid(unsigned(spans * bps), unsigned(r.G));
  ProfScope ps(s, kProfUlyssesInv);
  hipLaunchKernelGGL(ulysses_inv_sum_kernel<F>, grid, dim3(kThreads), 0, s, static_cast<const F*>(in),
                     static_cast<F*>(out), P, B, Sp, H, Hl, rep, R1, bps, r.P * r.B * r.S * int64_t(Hl) * R1,
                     r.P * r.B * Sp * int64_t(H) * R1);
  return hipGetLastError();
}

template <int VB>
hipError_t zigzag_vb(const void* in, void* out, int B, int P, int64_t chunk_bytes, bool inverse,
                     hipStream_t s) {
  using V = typename Vec<VB>::T;
  const int64_t cv = chunk_bytes / VB;
  const int64_t spans = int64_t(B) * 2 * P;
  const int bps = blocks_for(spans, cv);
  ProfScope ps(s, kProfZigzag);
  hipLaunchKernelGGL(zigzag_kernel<V>, dim3(unsigned(spans * bps)), dim3(kThreads), 0, s,
                     static_cast<const V*>(in), static_cast<V*>(out), P, cv, inverse ? 1 : 0, bps);
  return hipGetLastError();
}

template <int VB>
hipError_t striped_vb(const void* in, void* out, int64_t B, int64_t S, int64_t row_bytes, int64_t P,
                      bool inverse, hipStream_t s) {
  using V = typename Vec<VB>::T;
  const int RV = int(row_bytes / VB);
  // whole rows per block, about kThreads * kVPT vectors each
  const int rpb = RV >= kThreads * kVPT ? 1 : (kThreads * kVPT) / RV;
  const int64_t rows = B * S;
  const int64_t blocks = (rows + rpb - 1) / rpb;
  ProfScope ps(s, kProfStriped);
  hipLaunchKernelGGL(striped_kernel<V>, dim3(unsigned(blocks)), dim3(kThreads), 0, s, static_cast<const V*>(in),
                     static_cast<V*>(out), int(S), int(P), RV, rpb, rows, inverse ? 1 : 0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_striped(const void* in, void* out, int64_t B, int64_t S, int64_t row_bytes, int64_t P,
                          bool inverse, hipStream_t s) {
  switch (pick_vec_bytes(row_bytes, in, out)) {
    case 16: return striped_vb<16>(in, out, B, S, row_bytes, P, inverse, s);
    case 8: return striped_vb<8>(in, out, B, S, row_bytes, P, inverse, s);
    case 4: return striped_vb<4>(in, out, B, S, row_bytes, P, inverse, s);
    case 2: return striped_vb<2>(in, out, B, S, row_bytes, P, inverse, s);
    default: return striped_vb<1>(in, out, B, S, row_bytes, P, inverse, s);
  }
}

hipError_t launch_pad_rows(const void* in, void* out, int64_t B, int64_t S, int64_t S_out, int64_t row_bytes,
                           uint32_t fill, hipStream_t s) {
  // fill words need 4-byte vectors at least; a zero fill admits any width
  int vb = pick_vec_bytes(row_bytes, in, out);
  if (fill != 0 && vb < 4) vb = 4;  // row_bytes % 4 == 0 is checked by the caller
  const int64_t RV = row_bytes / vb;
  const int bps = blocks_for(B, S_out * RV);
  ProfScope ps(s, kProfPadRows);
  const dim3 grid(unsigned(B * bps));
  switch (vb) {
    case 16:
      hipLaunchKernelGGL(pad_rows_kernel<u32x4>, grid, dim3(kThreads), 0, s, static_cast<const u32x4*>(in),
                         static_cast<u32x4*>(out), S, S_out, RV, u32x4{fill, fill, fill, fill}, bps);
      break;
    case 8:
      hipLaunchKernelGGL(pad_rows_kernel<u32x2>, grid, dim3(kThreads), 0, s, static_cast<const u32x2*>(in),
                         static_cast<u32x2*>(out), S, S_out, RV, u32x2{fill, fill}, bps);
      break;
    case 4:
      hipLaunchKernelGGL(pad_rows_kernel<uint32_t>, grid, dim3(kThreads), 0, s, static_cast<const uint32_t*>(in),
                         static_cast<uint32_t*>(out), S, S_out, RV, fill, bps);
      break;
    case 2:
      hipLaunchKernelGGL(pad_rows_kernel<uint16_t>, grid, dim3(kThreads), 0, s, static_cast<const uint16_t*>(in),
                         static_cast<uint16_t*>(out), S, S_out, RV, uint16_t(0), bps);
      break;
    default:
      hipLaunchKernelGGL(pad_rows_kernel<uint8_t>, grid, dim3(kThreads), 0, s, static_cast<const uint8_t*>(in),
                         static_cast<uint8_t*>(out), S, S_out, RV, uint8_t(0), bps);
  }
  return hipGetLastError();
}

hipError_t launch_relayout(const RelayoutProblem& r, const void* in, void* out, hipStream_t s) {
  if (r.rep == 1) {
    switch (pick_vec_bytes((r.H / r.P) * r.D * r.eb, in, out)) {
      case 16: return ulysses_vb<16>(r, in, out, s);
      case 8: return ulysses_vb<8>(r, in, out, s);
      case 4: return ulysses_vb<4>(r, in, out, s);
      case 2: return ulysses_vb<2>(r, in, out, s);
      default: return ulysses_vb<1>(r, in, out, s);
    }
  }
  if (r.inverse) {  // float32, copies summed
    if (pick_vec_bytes(r.D * 4, in, out) == 16) return ulysses_inv_sum_f<f32x4>(r, in, out, s);
    return ulysses_inv_sum_f<float>(r, in, out, s);
  }
  switch (pick_vec_bytes(r.D * r.eb, in, out)) {
    case 16: return ulysses_rep_vb<16>(r, in, out, s);
    case 8: return ulysses_rep_vb<8>(r, in, out, s);
    case 4: return ulysses_rep_vb<4>(r, in, out, s);
    case 2: return ulysses_rep_vb<2>(r, in, out, s);
    default: return ulysses_rep_vb<1>(r, in, out, s);
  }
}

hipError_t launch_zigzag(const void* in, void* out, int64_t B, int64_t S, int64_t row_bytes,
                         int64_t P, bool inverse, hipStream_t s) {
  const int64_t chunk = (S / (2 * P)) * row_bytes;
  switch (pick_vec_bytes(chunk, in, out)) {
    case 16: return zigzag_vb<16>(in, out, int(B), int(P), chunk, inverse, s);
    case 8: return zigzag_vb<8>(in, out, int(B), int(P), chunk, inverse, s);
    case 4: return zigzag_vb<4>(in, out, int(B), int(P), chunk, inverse, s);
    case 2: return zigzag_vb<2>(in, out, int(B), int(P), chunk, inverse, s);
    default: return zigzag_vb<1>(in, out, int(B), int(P), chunk, inverse, s);
  }
}

}  // namespace cp

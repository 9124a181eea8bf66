// Blockwise attention backward, bf16 in / float32 gradients, on the gfx950 matrix
// cores.  Deterministic: no atomics; every gradient element is written by one lane.
//
// Gradient of sum(dO * O) for O = softmax(scale * Q K^T) V restricted to visible
// pairs, given the rows' final O and lse (so ring blocks add up to the full
// gradient):  P = exp(scale*s - lse), Delta_i = dO_i . O_i, dV = P^T dO,
// dP = dO V^T, dS = P * (dP - Delta), dQ = scale dS K, dK = scale dS^T Q.
// Attention itself: handbook "Context parallelism: Ring Attention and Ulysses",
// §"Which operations partition directly"; its gradient is the textbook one.
//
// Two launches:
//  1. delta: Delta = rowsum(dO * O) into the caller's workspace [B,Hq,Sq].
//  2. one grid with two roles, each a workgroup of 8 wavefronts:
//     paired dK / dV role — owns 128 keys of a kv head; the two wavefronts of a SIMD
//       share 32 keys (one holds their V rows and accumulates dK, the other their K
//       rows and accumulates dV) and stream query tiles of the group's heads:
//       S = Q K^T and P once per block pair (P passed through LDS), dP = dO V^T,
//       dS, dK^T += Q^T dS, dV^T += dO^T P;
//     dQ role — owns 256 queries of a head (Q and dO fragments) and streams key
//       tiles: S^T = K Q^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T.
//     7 products per block pair of keys and queries (4 would be counted).  S and dP
//     are computed query-major in the pair role so P and dS are directly the B
//     operands of the next products.  Each LDS stage holds two row-major tiles (Q
//     and dO, or K and V), XOR-swizzled and filled by LDS-DMA; the operands needed
//     transposed (dO^T, Q^T, K^T) are read from the same tiles with the LDS
//     transpose read.  The role lists, each heaviest first, are interleaved in one
//     grid.
// Tiles are skipped / masked exactly as in the forward (empty / partial / full).
#include <type_traits>

#include "mfma_common.h"
#include "prof.h"

namespace cp {
namespace {

using namespace mfma;

// lse in the base-2 domain; a row with no visible key gets +inf so that every
// exp2(s*c - lse2) of it is exactly 0.
CP_DEVICE float lse2_of(float lse) { return lse == -INFINITY ? INFINITY : lse * kLog2e; }

// ---- 1. Delta (and the base-2 lse) ----------------------------------------------
// Both row arrays [B,Hq,Sq] go to the workspace, where the main kernel's pair role
// copy a query tile's values straight into LDS.
template <int D>
__global__ __launch_bounds__(256) void delta_kernel(int64_t rows, int Sq, int Hq,
                                                    const uint16_t* __restrict__ out,
                                                    const uint16_t* __restrict__ dout,
                                                    const float* __restrict__ lse,
                                                    float* __restrict__ delta, float* __restrict__ lse2) {
  constexpr int kLanesPerRow = D / 8;
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t row = t / kLanesPerRow;   // (b, i, h)
  const int c = int(t % kLanesPerRow);
  float x = 0.0f;
  if (row < rows) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(out + row * D + c * 8);
    const u32x4 g = *reinterpret_cast<const u32x4*>(dout + row * D + c * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      x += bf16_to_f32(uint16_t(a[w] & 0xffff)) * bf16_to_f32(uint16_t(g[w] & 0xffff));
      x += bf16_to_f32(uint16_t(a[w] >> 16)) * bf16_to_f32(uint16_t(g[w] >> 16));
    }
  }
#pragma unroll
  for (int o = kLanesPerRow / 2; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  if (row < rows && c == 0) {
    const int h = int(row % Hq);
    const int64_t bi = row / Hq;
    const int i = int(bi % Sq);
    const int64_t b = bi / Sq;
    const int64_t li = (b * Hq + h) * Sq + i;
    delta[li] = x;
    lse2[li] = lse2_of(lse[li]);
  }
}


// ---- 2. configuration and LDS stages ---------------------------------------------
template <int D_>
struct BwdCfg {
  static constexpr int D = D_;
  static constexpr int NW = 8;
  static constexpr int kThreads = 64 * NW;
  static constexpr int kRows = 32 * NW;  // queries per workgroup of the dQ role
  static constexpr int KS = D / 16;
  static constexpr int DB = D / 32;
  static constexpr int BN = 128;         // key tile of the dQ role
  static constexpr int KB = BN / 32;
  static constexpr int kTileN = BN * D;  // swizzled row-major tile
  // dQ stage: K rows, V rows, kpos, kseg
  static constexpr int kStageQ = 2 * kTileN * 2 + 2 * BN * 4;
  static constexpr int kAhead = 3;  // LDS operand reads issued this many products ahead
  // key-tile spans of the dQ role, cached (after its two stages) when they come from
  // position / segment arrays
  static constexpr int kSpanTiles = 1024;
  using TileN = DmaTile<BN, D, kThreads>;
  // paired dK / dV role: a workgroup owns 128 keys and walks query tiles of BMP rows;
  // its stages hold the Q and dO rows, lse2, delta, positions and segment ids of a
  // tile, spaced like the dQ role's stages, followed by the P buffer
  // ([QBLKP][4 key blocks][2 fragments][64 lanes] x 16 B)
  static constexpr int kPairKeys = 128;
  static constexpr int BMP = 96;
  static constexpr int QBLKP = BMP / 32;
  static constexpr int kTileMP = BMP * D;
  static constexpr int kStageP = 2 * kTileMP * 2 + 4 * BMP * 4;  // Q, dO, lse2, delta, qpos, qseg
  static constexpr int kStageMax = kStageQ > kStageP ? kStageQ : kStageP;
  static constexpr int kPBytes = QBLKP * 4 * 2 * 64 * 16;
  static constexpr int kLdsPair = 2 * kStageMax + kPBytes;
  using TileMP = DmaTile<BMP, D, kThreads>;
  // the general instance (windows, segment ids, position arrays) also caches the
  // spans of up to kSpanTilesP query tiles after the P buffer
  static constexpr int kSpanTilesP = 256;
  static constexpr int kLdsPairL = kLdsPair + kSpanTilesP * 16;
  static_assert(kLdsPairL <= 160 * 1024, "LDS of one workgroup");
  static_assert(2 * kStageMax + kSpanTiles * 16 <= kLdsPair, "the dQ role's spans fit the pair kernel's LDS");
  static_assert(BMP <= kThreads && BN <= kThreads, "one thread per row of the small arrays");
};

// Paired dK / dV role.  kLane: the general instance (windows, segment ids, position
// arrays); otherwise positions are offset + index and there is neither window nor
// segment ids.  A workgroup owns keys [j0, j0 + 128) of kv
// head g; wavefronts w and w + 4 (w < 4, the two wavefronts of one SIMD) own the same
// 32 keys j0 + 32w + (0..31), one per lane column: wavefront w accumulates dK and
// holds the keys' V rows, wavefront w + 4 accumulates dV and holds their K rows.
// For every query tile of BMP = 96 rows (three 32-query blocks) of every head of
// the group:
//   phase A: the dV wavefront forms S = Q K^T and P = exp(S - lse) of the three
//     blocks and writes P to LDS as the bf16 B fragments of the next products; the
//     dK wavefront meanwhile forms dP = dO V^T of the three blocks;
//   phase B: the dK wavefront forms dS = P (dP - Delta) and dK^T += Q^T dS, the dV
//     wavefront dV^T += dO^T P, both reading P from LDS.
// Each P (and each exponential) is computed once: 7 products per block pair of keys
// and queries with the dQ role, where separate dV and dK roles would take 8 (both
// recomputing S).  The phases are separated by a workgroup barrier, and in each
// phase both wavefronts of a SIMD run three products per block.
template <class C, bool kLane>
CP_DEVICE void pair_role(const AttnProblem& p, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                         const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
                         const float* __restrict__ lse2, const float* __restrict__ delta, float* __restrict__ dk,
                         float* __restrict__ dv, int accumulate, uint8_t* smem, int kt, int g, int b, int h_lo,
                         int h_end) {
  constexpr int BM = C::BMP, QB = C::QBLKP;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int pr = __builtin_amdgcn_readfirstlane(wave & 3);  // key block of the pair
  const bool is_dv = __builtin_amdgcn_readfirstlane(wave >> 2) != 0;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int G = p.Hq / p.Hkv;
  const int j0 = kt * C::kPairKeys;
  const int wj0 = j0 + pr * 32;
  const int64_t krs = int64_t(p.Hkv) * C::D;
  const int64_t qrs = int64_t(p.Hq) * C::D;

  const Span wg_k = uniform(k_span(p, b, j0, min(j0 + C::kPairKeys, p.Sk) - 1));
  const bool wave_live = wj0 < p.Sk;
  const Span wv_k = uniform(k_span(p, b, min(wj0, p.Sk - 1), min(wj0 + 32, p.Sk) - 1));

  // K rows (dV wavefront: S) or V rows (dK wavefront: dP) of this lane's key as B
  // fragments (k-slots = head dims)
  const int key = min(wj0 + l32, p.Sk - 1);
  const bool key_ok = wj0 + l32 < p.Sk;
  bf16x8 kvf[C::KS];
  {
    const uint16_t* kr = (is_dv ? k : v) + (int64_t(b) * p.Sk + key) * krs + int64_t(g) * C::D;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(kr + s * 16 + hi * 8);
      kvf[s] = __builtin_bit_cast(bf16x8, key_ok ? x : u32x4{0, 0, 0, 0});
    }
  }
  const int my_kpos = kLane ? kpos_at(p, key) : p.k_offset + key;
  const int my_kseg = kLane ? kseg_at(p, b, key) : 0;

  f32x16 acc[C::DB];  // dK^T (dK wavefront) or dV^T (dV wavefront)
#pragma unroll
  for (int d = 0; d < C::DB; ++d) acc[d] = f32x16{};

  const float c2 = p.scale * kLog2e;
  const int n_it = (p.Sq + BM - 1) / BM;
  // tiles (query head hh of the group's heads [h_lo, h_end), query tile it), walked
  // from the last query tile down with the heads innermost: every workgroup of this
  // role starts at the end of the sequence and sweeps down at about the same pace, so
  // the workgroups resident together read the same Q / dO tiles and the caches serve
  // most of them
  struct Tq {
    int hh, it;
  };
  auto step = [&](Tq t) {
    if (++t.hh == h_end) {
      t.hh = h_lo;
      --t.it;
    }
    return t;
  };
  // Spans of the query tiles: with position or segment arrays (general instance) each
  // is two dependent global loads, so up to kSpanTilesP of them are loaded once, in
  // parallel, into LDS after the P buffer.
  const bool span_cached = kLane && (p.q_pos != nullptr || p.q_seg != nullptr) && n_it <= C::kSpanTilesP;
  i32x4* span_l = reinterpret_cast<i32x4*>(smem + C::kLdsPair);
  if (span_cached) {
    for (int t = tid; t < n_it; t += C::kThreads) {
      const Span sp_ = q_span(p, b, t * BM, min(t * BM + BM, p.Sq) - 1);
      span_l[t] = i32x4{sp_.pos_lo, sp_.pos_hi, sp_.seg_lo, sp_.seg_hi};
    }
    __syncthreads();
  }
  auto qtile_span = [&](int it) {
    if (span_cached) {
      const i32x4 x = span_l[it];
      return Span{x[0], x[1], x[2], x[3]};
    }
    return q_span(p, b, it * BM, min(it * BM + BM, p.Sq) - 1);
  };
  // the query tiles live for this key block lie in [it_lo, it_hi) (queries wholly
  // after the keys' window / segments are a suffix, those wholly before the keys a
  // prefix)
  const int it_hi =
      kLane ? first_true(0, n_it, [&](int it) { return keys_before(p, qtile_span(it), wg_k); }) : n_it;
  const int it_lo = first_true(0, it_hi, [&](int it) { return !keys_after(p, qtile_span(it), wg_k); });
  // without a window or segment ids every query tile of [it_lo, it_hi) holds a visible
  // pair and a wavefront pair's classes run by range (empty ..., partial ..., full ...);
  // other problems classify up to 64 tiles at once, one per lane, else tile by tile
  const bool dense = !kLane || (!p.window && !p.q_seg);
  const bool lane_cls = kLane && !dense && it_hi - it_lo <= 64;
  uint64_t live_m = 0, wfull_m = 0, wpart_m = 0;
  if (lane_cls) {
    const int it = it_lo + lane;
    int cg = kEmpty, cw = kEmpty;
    if (it < it_hi) {
      const Span qs_ = qtile_span(it);
      cg = classify(p, qs_, wg_k, false);
      if (wave_live) cw = classify(p, qs_, wv_k, false);
    }
    live_m = __ballot(cg != kEmpty);
    wfull_m = __ballot(cw == kFull);
    wpart_m = __ballot(cw == kPartial);
  }
  // the live tile at or below t (heads innermost), or one with it = -1
  auto next_tile = [&](Tq t) {
    if (t.it >= it_hi) t = Tq{h_lo, it_hi - 1};
    if (lane_cls) {
      if (t.it < it_lo) return Tq{t.hh, -1};
      const int sh = t.it - it_lo;
      const uint64_t m = live_m & (sh == 63 ? ~uint64_t(0) : (uint64_t(2) << sh) - 1);
      if (!m) return Tq{t.hh, -1};
      const int it = it_lo + 63 - int(__builtin_clzll(m));
      return it == t.it ? t : Tq{h_lo, it};
    }
    while (!dense && t.it >= it_lo && classify(p, qtile_span(t.it), wg_k, false) == kEmpty) t = step(t);
    if (t.it < it_lo) t.it = -1;
    return t;
  };
  int it_wlo = 0, it_wfull = 0;
  if (dense && wave_live && p.causal) {
    it_wlo = first_true(it_lo, it_hi, [&](int it) { return !(wv_k.pos_lo > qtile_span(it).pos_hi); });
    it_wfull = first_true(it_wlo, it_hi, [&](int it) { return qtile_span(it).pos_lo >= wv_k.pos_hi; });
  }
  auto wave_class = [&](Tq t) {
    if (lane_cls) {
      const uint64_t bit = uint64_t(1) << (t.it - it_lo);
      return (wfull_m & bit) ? int(kFull) : (wpart_m & bit) ? int(kPartial) : int(kEmpty);
    }
    if (!dense) return wave_live ? classify(p, qtile_span(t.it), wv_k, false) : int(kEmpty);
    if (!wave_live || t.it < it_wlo) return int(kEmpty);
    return t.it >= it_wfull ? int(kFull) : int(kPartial);
  };
  typename C::TileMP tq, tg;
  const uint32_t qrs_bytes = uint32_t(qrs) * 2u;
  tq.init(qrs_bytes, tid);
  tg.init(qrs_bytes, tid);
  auto q_of = [&](uint8_t* base) { return reinterpret_cast<uint16_t*>(base); };
  auto g_of = [&](uint8_t* base) { return q_of(base) + C::kTileMP; };
  auto l_of = [&](uint8_t* base) { return reinterpret_cast<float*>(g_of(base) + C::kTileMP); };
  auto d_of = [&](uint8_t* base) { return l_of(base) + BM; };
  auto qp_of = [&](uint8_t* base) { return reinterpret_cast<int*>(d_of(base) + BM); };
  auto qs_of = [&](uint8_t* base) { return qp_of(base) + BM; };
  // per-row values of query tile i0 (rows past the end read as 0): lse2 and delta,
  // and in the general instance the positions / segment ids (LDS-DMA from their
  // arrays, or written as offset + row / 0)
  auto issue_rows = [&](int h, int i0, uint8_t* base) {
    const int64_t li0 = (int64_t(b) * p.Hq + h) * p.Sq + i0;
    if (wave == 0) dma_dwords<BM>(lse2, li0, p.Sq - i0, l_of(base), lane);
    if (wave == 1) dma_dwords<BM>(delta, li0, p.Sq - i0, d_of(base), lane);
    if constexpr (kLane) {
      if (p.q_pos) {
        if (wave == 2) dma_dwords<BM>(p.q_pos, i0, p.Sq - i0, qp_of(base), lane);
      } else if (tid < BM) {
        qp_of(base)[tid] = p.q_offset + i0 + tid;
      }
      if (p.q_seg) {
        if (wave == 3) dma_dwords<BM>(p.q_seg, int64_t(b) * p.Sq + i0, p.Sq - i0, qs_of(base), lane);
      } else if (tid < BM) {
        qs_of(base)[tid] = 0;
      }
    }
  };
  auto issue = [&](Tq t, uint8_t* base) {
    const int h = g * G + t.hh;
    const int i0 = t.it * BM;
    tq.load(q + int64_t(b) * p.Sq * qrs + int64_t(h) * C::D, qrs_bytes, i0, p.Sq, q_of(base));
    tg.load(dout + int64_t(b) * p.Sq * qrs + int64_t(h) * C::D, qrs_bytes, i0, p.Sq, g_of(base));
    issue_rows(h, i0, base);
  };
  // P fragment j of query block qb of this pair, this lane
  uint8_t* pbuf = smem + 2 * C::kStageMax;
  auto p_at = [&](int qb, int j) {
    return reinterpret_cast<bf16x8*>(pbuf + (((qb * 4 + pr) * 2 + j) * 64 + lane) * 16);
  };
  const MaskSpec ms = make_mask_spec(p.causal, kLane ? p.window : 0, kLane && p.q_seg != nullptr);

  Tq cur = next_tile(Tq{h_lo, it_hi - 1});
  if (cur.it >= it_lo) {
    issue(cur, smem);
    wait_all();
    __syncthreads();
    int buf = 0;
    while (true) {
      Tq nxt = next_tile(step(cur));
      const bool has_next = nxt.it >= it_lo;
      uint8_t* base = smem + buf * C::kStageMax;
      // The next tile's Q and dO rows are staged by 2 kIter LDS-DMA loads per thread.
      // Issued together they hold a wavefront for hundreds of cycles (the loads of
      // all eight wavefronts queue at the CU's address unit), so they are issued one
      // every other product of phase A instead (dma_step); lse2 and delta go first.
      uint8_t* nbase = smem + (buf ^ 1) * C::kStageMax;
      const int nh = g * G + nxt.hh;
      const int ni0 = max(nxt.it, 0) * BM;
      const auto rq = C::TileMP::rows_rsrc(q + int64_t(b) * p.Sq * qrs + int64_t(nh) * C::D, qrs_bytes, ni0, p.Sq);
      const auto rg =
          C::TileMP::rows_rsrc(dout + int64_t(b) * p.Sq * qrs + int64_t(nh) * C::D, qrs_bytes, ni0, p.Sq);
      if (has_next) issue_rows(nh, ni0, nbase);
      constexpr int kIt = C::TileMP::kIter;
      auto dma_step = [&](int j) {
        if (j < 2 * kIt && has_next) {
          if (j < kIt)
            tq.load_iter(rq, j, q_of(nbase));
          else
            tg.load_iter(rg, j - kIt, g_of(nbase));
        }
      };
      const int wcls = wave_class(cur);
      if (wcls == kEmpty) {
#pragma unroll
        for (int j = 0; j < 2 * kIt; ++j) dma_step(j);
      }
      const uint16_t* qs = q_of(base);
      const uint16_t* gs = g_of(base);
      const float* ls = l_of(base);
      const float* ds = d_of(base);
      const int qpos0 = p.q_offset + cur.it * BM;
      const int* qps = qp_of(base);  // general instance: the tile's positions / segment ids
      const int* qss = qs_of(base);
      // ---- phase A: dP (dK wavefront) or S and P (dV wavefront) of the three query
      // blocks.  The exponentials take as long as the products (the transcendental
      // unit runs at a quarter of the vector rate), so the dV wavefront spreads those
      // of each block over the products of the next one.
      f32x16 sp[QB];
      if (wcls != kEmpty) {
        if (!is_dv) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) sp[qb] = f32x16{};
          static_assert(QB * C::KS >= 4 * C::TileMP::kIter, "the DMA steps fit phase A's products");
          pipelined_products<QB * C::KS, C::kAhead>(
              [&](int i) { return ld_row<C::D>(gs, (i / C::KS) * 32 + perm_row(l32), 2 * (i % C::KS) + hi); },
              [&](int i, bf16x8 f) {
                sp[i / C::KS] = mma(f, kvf[i % C::KS], sp[i / C::KS]);
                if ((i & 1) == 0) dma_step(i / 2);
              });
          // dP - Delta now: this wavefront waits for the dV wavefront's exponentials
          // at the barrier anyway, and phase B (where it forms dS) is its long one
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const f32x4 d4 = *reinterpret_cast<const f32x4*>(ds + qb * 32 + key_of_reg(4 * jj, hi));
#pragma unroll
              for (int i = 0; i < 4; ++i) sp[qb][4 * jj + i] -= d4[i];
            }
        } else {
          // raised priority: the SIMD's matrix core serves this wavefront's S products
          // first, so its exponentials start early and overlap the dK wavefront's dP
          __builtin_amdgcn_s_setprio(1);
          auto phase_a = [&](auto masked) {
            constexpr bool kMasked = decltype(masked)::value;
            f32x4 l4[4];
            auto load_lse = [&](int qb) {
#pragma unroll
              for (int jj = 0; jj < 4; ++jj)
                l4[jj] = *reinterpret_cast<const f32x4*>(ls + qb * 32 + key_of_reg(4 * jj, hi));
            };
            // P = 2^(S c2 - lse2) of score r of block qb (masked on partial tiles)
            auto exp_at = [&](int qb, int r) {
              float x = fmaf(sp[qb][r], c2, -l4[r >> 2][r & 3]);
              if constexpr (kMasked) {
                const int row = qb * 32 + key_of_reg(r & ~3, hi) + (r & 3);
                if constexpr (kLane)
                  x = pair_visible(ms, qps[row], my_kpos, qss[row], my_kseg) ? x : -INFINITY;
                else
                  x = pair_visible(ms, qpos0 + row, my_kpos, 0, 0) ? x : -INFINITY;
              }
              sp[qb][r] = __builtin_amdgcn_exp2f(x);
            };
            auto store_p = [&](int qb) {
              *p_at(qb, 0) = to_bf16x8(sp[qb], 0);
              *p_at(qb, 1) = to_bf16x8(sp[qb], 8);
            };
            constexpr int kPer = 16 / C::KS;  // scores per product
            static_assert(kPer * C::KS == 16, "the products of a block cover the previous block's scores");
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
              if (qb > 0) load_lse(qb - 1);
              sp[qb] = f32x16{};
              pipelined_products<C::KS, C::kAhead>(
                  [&](int i) { return ld_row<C::D>(qs, qb * 32 + perm_row(l32), 2 * i + hi); },
                  [&](int i, bf16x8 f) {
                    sp[qb] = mma(f, kvf[i], sp[qb]);
                    if (((qb * C::KS + i) & 1) == 0) dma_step((qb * C::KS + i) / 2);
                    if (qb > 0) {
#pragma unroll
                      for (int j = 0; j < kPer; ++j) exp_at(qb - 1, kPer * i + j);
                    }
                  });
              if (qb > 0) store_p(qb - 1);
            }
            load_lse(QB - 1);
#pragma unroll
            for (int r = 0; r < 16; ++r) exp_at(QB - 1, r);
            store_p(QB - 1);
          };
          if (wcls == kPartial)
            phase_a(std::true_type{});
          else
            phase_a(std::false_type{});
          __builtin_amdgcn_s_setprio(0);
        }
      }
      // P is in LDS; the next tile's DMA stays in flight across this barrier
      lds_barrier();
      // ---- phase B: dK^T += Q^T dS (dK wavefront), dV^T += dO^T P (dV wavefront):
      // one product loop for both, reading Q^T or dO^T transposed from the stage
      if (wcls != kEmpty) {
        const uint16_t* at = is_dv ? gs : qs;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          bf16x8 bfrag[2] = {*p_at(qb, 0), *p_at(qb, 1)};
          if (!is_dv) {
            // dS = P (dP - Delta), in place of P (dP - Delta formed in phase A)
            f32x16 dp = sp[qb];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              // P of this key and row from its bf16 fragment (bf16 is the high half of a float)
              const uint32_t w = __builtin_bit_cast(u32x4, bfrag[r >> 3])[(r & 7) >> 1];
              const float pr_ = __uint_as_float((r & 1) ? (w & 0xffff0000u) : (w << 16));
              dp[r] = pr_ * dp[r];
            }
            bfrag[0] = to_bf16x8(dp, 0);
            bfrag[1] = to_bf16x8(dp, 8);
          }
          pipelined_products<2 * C::DB, C::kAhead>(
              [&](int i) { return ld_tr<C::D>(at, (qb * 2 + i / C::DB) * 16, (i % C::DB) * 32); },
              [&](int i, bf16x8 f) { acc[i % C::DB] = mma(f, bfrag[i / C::DB], acc[i % C::DB]); });
        }
      }
      if (has_next) {
        wait_all();
        __syncthreads();
      } else {
        __syncthreads();
        break;
      }
      cur = nxt;
      buf ^= 1;
    }
  }

  // epilogue: lane holds key column l32, dims d*32 + 8j + 4*hi + (0..3)
  if (!key_ok) return;
  const float sc = is_dv ? 1.0f : p.scale;
  int kcol = wj0 + l32;
  pin(kcol);  // the row address is formed here, not kept live from the prologue
  float* gr = (is_dv ? dv : dk) + ((int64_t(b) * p.Sk + kcol) * p.Hkv + g) * C::D;
#pragma unroll
  for (int d = 0; d < C::DB; ++d)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int off = d * 32 + 8 * j + 4 * hi;
      f32x4 a{acc[d][4 * j] * sc, acc[d][4 * j + 1] * sc, acc[d][4 * j + 2] * sc, acc[d][4 * j + 3] * sc};
      if (accumulate) a += *reinterpret_cast<const f32x4*>(gr + off);
      *reinterpret_cast<f32x4*>(gr + off) = a;
    }
}

// dQ role: a workgroup owns queries [q0, q0 + kRows) of head h; wavefront w owns
// queries q0 + 32w + (0..31), one per lane column.  kUse tells the kernels that call
// it apart: each kernel instantiates its own copy (the host compilation pass accepts
// one kernel's reference to a device-builtin function template specialization only).
template <class C, bool kLane, int kUse = 0>
CP_DEVICE void dq_role(const AttnProblem& p, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                       const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
                       const float* __restrict__ lse2, const float* __restrict__ delta, float* __restrict__ dq,
                       int accumulate, uint8_t* smem, int qt, int h, int b) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int g = h / (p.Hq / p.Hkv);
  const int q0 = qt * C::kRows;
  const int wq0 = q0 + wave * 32;
  const int64_t krs = int64_t(p.Hkv) * C::D;
  const int64_t qrs = int64_t(p.Hq) * C::D;

  const Span wg_q = uniform(q_span(p, b, q0, min(q0 + C::kRows, p.Sq) - 1));
  const bool wave_live = wq0 < p.Sq;
  const Span wv_q = uniform(q_span(p, b, min(wq0, p.Sq - 1), min(wq0 + 32, p.Sq) - 1));

  const int row = min(wq0 + l32, p.Sq - 1);
  const bool row_ok = wq0 + l32 < p.Sq;
  bf16x8 qf[C::KS], gf[C::KS];
  {
    const uint16_t* qr = q + (int64_t(b) * p.Sq + row) * qrs + int64_t(h) * C::D;
    const uint16_t* gr = dout + (int64_t(b) * p.Sq + row) * qrs + int64_t(h) * C::D;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(qr + s * 16 + hi * 8);
      const u32x4 y = *reinterpret_cast<const u32x4*>(gr + s * 16 + hi * 8);
      qf[s] = __builtin_bit_cast(bf16x8, row_ok ? x : u32x4{0, 0, 0, 0});
      gf[s] = __builtin_bit_cast(bf16x8, row_ok ? y : u32x4{0, 0, 0, 0});
    }
  }
  const int64_t li = (int64_t(b) * p.Hq + h) * p.Sq + row;
  const float my_lse2 = row_ok ? lse2[li] : INFINITY;
  const float my_delta = row_ok ? delta[li] : 0.0f;
  const int my_qpos = qpos_at(p, row);
  const int my_qseg = qseg_at(p, b, row);

  f32x16 acc[C::DB];
#pragma unroll
  for (int d = 0; d < C::DB; ++d) acc[d] = f32x16{};

  const float c2 = p.scale * kLog2e;
  const int n_kt = (p.Sk + C::BN - 1) / C::BN;
  const uint16_t* kbase = k + int64_t(b) * p.Sk * krs + int64_t(g) * C::D;
  const uint16_t* vbase = v + int64_t(b) * p.Sk * krs + int64_t(g) * C::D;

  // spans of the key tiles, cached in LDS when they come from arrays (as above)
  const bool span_cached = (p.k_pos != nullptr || p.k_seg != nullptr) && n_kt <= C::kSpanTiles;
  i32x4* span_l = reinterpret_cast<i32x4*>(smem + 2 * C::kStageMax);
  if (span_cached) {
    for (int t = tid; t < n_kt; t += C::kThreads) {
      const Span s = k_span(p, b, t * C::BN, min(t * C::BN + C::BN, p.Sk) - 1);
      span_l[t] = i32x4{s.pos_lo, s.pos_hi, s.seg_lo, s.seg_hi};
    }
    __syncthreads();
  }
  auto ktile_span = [&](int kt) {
    if (span_cached) {
      const i32x4 x = span_l[kt];
      return Span{x[0], x[1], x[2], x[3]};
    }
    return k_span(p, b, kt * C::BN, min(kt * C::BN + C::BN, p.Sk) - 1);
  };
  auto tile_class = [&](int kt, const Span& qsp) {
    return classify(p, qsp, ktile_span(kt), kt * C::BN + C::BN > p.Sk);
  };
  // the key tiles live for this query block lie in [kt_lo, kt_hi)
  const int kt_lo = first_true(0, n_kt, [&](int kt) { return !keys_before(p, wg_q, ktile_span(kt)); });
  const int kt_hi = first_true(kt_lo, n_kt, [&](int kt) { return keys_after(p, wg_q, ktile_span(kt)); });
  // without a window or segment ids: no classification inside [kt_lo, kt_hi)
  const bool dense = !p.window && !p.q_seg;
  // other problems with at most 64 key tiles in the range: all classified at once,
  // one tile per lane
  const bool lane_cls = kLane && !dense && kt_hi - kt_lo <= 64;
  uint64_t live_m = 0, wfull_m = 0, wpart_m = 0;
  if (lane_cls) {
    const int kt = kt_lo + lane;
    int cg = kEmpty, cw = kEmpty;
    if (kt < kt_hi) {
      const Span ks = ktile_span(kt);
      const bool ragged = kt * C::BN + C::BN > p.Sk;
      cg = classify(p, wg_q, ks, ragged);
      if (wave_live) cw = classify(p, wv_q, ks, ragged);
    }
    live_m = __ballot(cg != kEmpty);
    wfull_m = __ballot(cw == kFull);
    wpart_m = __ballot(cw == kPartial);
  }
  auto next_tile = [&](int kt) {
    kt = max(kt, kt_lo);
    if (lane_cls) {
      const uint64_t m = kt < kt_hi ? live_m >> (kt - kt_lo) : 0;
      return m ? kt + int(__builtin_ctzll(m)) : n_kt;
    }
    while (!dense && kt < kt_hi && tile_class(kt, wg_q) == kEmpty) ++kt;
    return kt < kt_hi ? kt : n_kt;
  };
  // this wavefront's class of a key tile; dense problems by range (full ... full,
  // partial ..., empty ...; the last tile is partial when ragged)
  int kt_full = n_kt, kt_wend = n_kt;
  if (dense && wave_live && p.causal) {
    kt_wend = first_true(kt_lo, kt_hi, [&](int kt) { return ktile_span(kt).pos_lo > wv_q.pos_hi; });
    kt_full = first_true(kt_lo, kt_wend, [&](int kt) { return ktile_span(kt).pos_hi > wv_q.pos_lo; });
  }
  auto wave_class = [&](int kt) {
    if (lane_cls) {
      const uint64_t bit = uint64_t(1) << (kt - kt_lo);
      return (wfull_m & bit) ? int(kFull) : (wpart_m & bit) ? int(kPartial) : int(kEmpty);
    }
    if (!dense) return tile_class(kt, wv_q);
    if (!wave_live || kt >= kt_wend) return int(kEmpty);
    return (kt < kt_full && kt * C::BN + C::BN <= p.Sk) ? int(kFull) : int(kPartial);
  };
  typename C::TileN tk, tv;
  const uint32_t krs_bytes = uint32_t(krs) * 2u;
  tk.init(krs_bytes, tid);
  tv.init(krs_bytes, tid);
  // stage: K rows, V rows, kpos, kseg
  auto ks_of = [&](uint8_t* base) { return reinterpret_cast<uint16_t*>(base); };
  auto vs_of = [&](uint8_t* base) { return ks_of(base) + C::kTileN; };
  auto kp_of = [&](uint8_t* base) { return reinterpret_cast<int*>(vs_of(base) + C::kTileN); };
  // key positions / segment ids of the tile straight into the stage (LDS-DMA from
  // their arrays, or written as offset + index / 0); keys past the end are masked by
  // their index
  static_assert(C::BN % 64 == 0, "whole wavefronts of keys");
  auto issue = [&](int kt, uint8_t* base) {
    tk.load(kbase, krs_bytes, kt * C::BN, p.Sk, ks_of(base));
    tv.load(vbase, krs_bytes, kt * C::BN, p.Sk, vs_of(base));
    int* kp = kp_of(base);
    const int j0 = kt * C::BN;
    const int wave = tid >> 6;
    if (p.k_pos) {
      if (wave == 0) dma_dwords<C::BN>(p.k_pos, j0, p.Sk - j0, kp, lane);
    } else if (tid < C::BN) {
      kp[tid] = p.k_offset + j0 + tid;
    }
    if (p.k_seg) {
      if (wave == 1) dma_dwords<C::BN>(p.k_seg, int64_t(b) * p.Sk + j0, p.Sk - j0, kp + C::BN, lane);
    } else if (tid < C::BN) {
      kp[C::BN + tid] = 0;
    }
  };
  auto publish = [&](uint8_t*) {
    wait_all();
    __syncthreads();
  };

  int cur = next_tile(0);
  if (cur < n_kt) {
    issue(cur, smem);
    publish(smem);
    int buf = 0;
    const MaskSpec ms = make_mask_spec(p.causal, p.window, p.q_seg != nullptr);
    while (true) {
      const int nxt = next_tile(cur + 1);
      const bool has_next = nxt < n_kt;
      uint8_t* nbase = smem + (buf ^ 1) * C::kStageMax;
      const int wcls = wave_class(cur);
      // The next stage's loads.  Issued by all eight wavefronts at once they queue at
      // the CU's address unit, so in the dense instance wavefronts w and w + 4 issue
      // theirs during key block w % 4 of this stage (the general instance, which also
      // stages positions / segment ids, would spill registers doing so).
      const int my_kb = kLane ? -1 : __builtin_amdgcn_readfirstlane(wave & 3);
      if (has_next && (wcls == kEmpty || my_kb < 0 || my_kb >= C::KB)) issue(nxt, nbase);
      if (wcls != kEmpty) {
        uint8_t* base = smem + buf * C::kStageMax;
        const uint16_t* ks = ks_of(base);
        const uint16_t* vs = vs_of(base);
        const int* kp = kp_of(base);
        const int* kg = kp + C::BN;
        const int nvalid = p.Sk - cur * C::BN;
        auto body = [&](auto masked) {
          constexpr bool kMasked = decltype(masked)::value;
#pragma unroll
          for (int kb = 0; kb < C::KB; ++kb) {
            if (!kLane && has_next && kb == my_kb) issue(nxt, nbase);
            // S^T = K Q^T and dP^T = V dO^T for 32 keys: lane column = this lane's query
            f32x16 s = f32x16{}, dp = f32x16{};
            const int arow = kb * 32 + perm_row(l32);
            pipelined_products<2 * C::KS, C::kAhead>(
                [&](int i) { return ld_row<C::D>((i & 1) ? vs : ks, arow, 2 * (i >> 1) + hi); },
                [&](int i, bf16x8 f) {
                  if (i & 1)
                    dp = mma(f, gf[i >> 1], dp);
                  else
                    s = mma(f, qf[i >> 1], s);
                });
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const int kk0 = kb * 32 + key_of_reg(4 * jj, hi);
              i32x4 kp4 = i32x4{0, 0, 0, 0}, kg4 = i32x4{0, 0, 0, 0};
              if constexpr (kMasked) {
                kp4 = *reinterpret_cast<const i32x4*>(kp + kk0);
                kg4 = *reinterpret_cast<const i32x4*>(kg + kk0);
              }
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int r = 4 * jj + i;
                float x = fmaf(s[r], c2, -my_lse2);
                if constexpr (kMasked)
                  x = ((kk0 + i < nvalid) & pair_visible(ms, my_qpos, kp4[i], my_qseg, kg4[i])) ? x : -INFINITY;
                const float pr = __builtin_amdgcn_exp2f(x);
                s[r] = pr * (dp[r] - my_delta);  // dS^T
              }
            }
            // dQ^T += K^T dS^T over the block's two 16-key k-steps (K^T read transposed)
            const bf16x8 sb[2] = {to_bf16x8(s, 0), to_bf16x8(s, 8)};
            pipelined_products<2 * C::DB, C::kAhead>(
                [&](int i) { return ld_tr<C::D>(ks, (kb * 2 + i / C::DB) * 16, (i % C::DB) * 32); },
                [&](int i, bf16x8 f) { acc[i % C::DB] = mma(f, sb[i / C::DB], acc[i % C::DB]); });
          }
        };
        if (wcls == kPartial)
          body(std::true_type{});
        else
          body(std::false_type{});
      }
      if (has_next)
        publish(nbase);
      else
        __syncthreads();
      if (!has_next) break;
      cur = nxt;
      buf ^= 1;
    }
  }

  if (!row_ok) return;
  int qrow = row;
  pin(qrow);  // the row address is formed here, not kept live from the prologue
  float* dqr = dq + (int64_t(b) * p.Sq + qrow) * qrs + int64_t(h) * C::D;
#pragma unroll
  for (int d = 0; d < C::DB; ++d)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int off = d * 32 + 8 * j + 4 * hi;
      f32x4 a{acc[d][4 * j] * p.scale, acc[d][4 * j + 1] * p.scale, acc[d][4 * j + 2] * p.scale,
              acc[d][4 * j + 3] * p.scale};
      if (accumulate) a += *reinterpret_cast<const f32x4*>(dqr + off);
      *reinterpret_cast<f32x4*>(dqr + off) = a;
    }
}

// ---- fused launch ------------------------------------------------------------------
// Key-side items (key blocks lowest first = heaviest under a causal mask) and
// query-side items (query blocks highest first) are merged at the ratio of their
// counts, then rotated within each round of 8 workgroups so that every XCD receives
// a fair share of each role.
struct BwdArgs {
  AttnProblem p;
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* lse2;   // [B,Hq,Sq] base-2 lse (workspace)
  const float* delta;  // [B,Hq,Sq] (workspace)
  float* dq;
  float* dk;
  float* dv;
  int accumulate;
  int n_kv;  // key-side items = B * Hkv * 128-key blocks * hsplit
  int n_q;   // query-side items = B * Hq * query blocks
  // key-side items of grouped-query problems on small grids take half of the group's
  // query heads each (hsplit = 2): the second half's dK / dV go to part
  // ([2][B,Sk,Hkv,D] float32, dK then dV) and a second kernel adds them
  int hsplit;
  float* part;
};

// One grid of paired dK / dV items (128 keys each; on small grouped-query grids
// split over two halves of the group's query heads) and dQ items.  kLane: the
// general instance (windows, segment ids, position arrays: per-tile classification
// of up to 64 tiles at once, masks from the staged positions / segment ids); the
// other instance serves problems whose positions are offset + index and carries
// none of that, so its register allocation is unaffected.
template <class C, bool kLane>
__global__ __launch_bounds__(C::kThreads) void attn_bwd_pair_kernel(BwdArgs a) {
  __shared__ __align__(16) uint8_t smem[kLane ? C::kLdsPairL : C::kLdsPair];
  const AttnProblem p = specialize<kLane>(a.p);
  const int64_t N = int64_t(a.n_kv) + a.n_q;
  // Workgroups go to the 8 XCDs round-robin by index.  Within each round of 8
  // consecutive workgroups the items are rotated by the round number, so that the
  // periodic role pattern of the interleaved list cannot alias with the XCD index.
  const int64_t u = blockIdx.x / 8;
  const int64_t width = N - 8 * u < 8 ? N - 8 * u : 8;
  const int64_t L = 8 * u + (blockIdx.x % 8 + u) % width;
  // head-split grids list every key-side item first (they are the heavy ones);
  // others interleave the two sides in proportion
  const bool kv_first = a.hsplit > 1;
  const int64_t before = kv_first ? (L < a.n_kv ? L : a.n_kv) : (L * a.n_kv) / N;  // key-side items before L
  const bool kv_side = kv_first ? L < a.n_kv : ((L + 1) * a.n_kv) / N > before;
  if (kv_side) {
    const int i = int(before);
    const int hs = a.hsplit;
    const int blk = i / hs;  // the head subsets of a key block are neighbours
    const int sub = i % hs;
    const int bg = blk % (p.B * p.Hkv);
    const int G = p.Hq / p.Hkv;
    const int64_t plane = int64_t(p.B) * p.Sk * p.Hkv * C::D;
    pair_role<C, kLane>(p, a.q, a.k, a.v, a.dout, a.lse2, a.delta, sub ? a.part : a.dk, sub ? a.part + plane : a.dv,
                 sub ? 0 : a.accumulate, smem, blk / (p.B * p.Hkv), bg % p.Hkv, bg / p.Hkv, sub * G / hs,
                 (sub + 1) * G / hs);
  } else {
    const int i = int(L - before);
    const int bh = i % (p.B * p.Hq);
    const int r = i / (p.B * p.Hq);
    const int n_qt = (p.Sq + C::kRows - 1) / C::kRows;
    dq_role<C, kLane, kLane ? 2 : 1>(p, a.q, a.k, a.v, a.dout, a.lse2, a.delta, a.dq, a.accumulate, smem,
                         p.causal ? n_qt - 1 - r : r, bh % p.Hq, bh / p.Hq);
  }
}

// dK += part[0], dV += part[1] over [B,Sk,Hkv,D] float32 (n4 vectors of 4 each):
// the second head subset's partial sums of the split key-side items.
__global__ __launch_bounds__(256) void head_split_sum_kernel(int64_t n4, float* dk, float* dv,
                                                             const float* part) {
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (t >= 2 * n4) return;
  const bool is_v = t >= n4;
  f32x4* o = reinterpret_cast<f32x4*>(is_v ? dv : dk) + (is_v ? t - n4 : t);
  *o += reinterpret_cast<const f32x4*>(part)[t];
}

// Key-side items per (kv head, key block) for this problem: 2 for problems with
// grouped heads whose grid is under 16 rounds of workgroups (one per CU); each
// key-side item then walks half of the group's query heads.  (Measured with the
// separate dK and dV roles the kernel had before the paired role; the item count
// below is the same: two per 256 keys then, one per 128 keys now.)  Without the split the
// key-side items, G times heavier than the query-side ones, set the time: on small
// grids the largest of them outlasts the average load of a CU, and on larger ones
// they leave the longer tail.  Measured (bf16, D=128, causal): 1.5-1.8x faster at
// 2-8K tokens with 8 q / 2 kv or 32 q / 8 kv heads, -20% at 16K and -6% at 32K with
// 8 / 2, -1.3% at 64K with 8 / 2 (12 rounds); never slower.  Beyond 16 rounds it is
// left off (not measured there).
constexpr int kHeadSplitRounds = 16;
int bwd_hsplit(const AttnProblem& p) {
  if (p.Hq / p.Hkv < 2) return 1;
  constexpr int kRows = 256;
  const int64_t items = 2 * int64_t(p.B) * p.Hkv * ((p.Sk + kRows - 1) / kRows) +
                        int64_t(p.B) * p.Hq * ((p.Sq + kRows - 1) / kRows);
  return items < kHeadSplitRounds * int64_t(device_cus()) ? 2 : 1;
}

template <int D>
hipError_t launch_d(const AttnProblem& p, const void* q, const void* k, const void* v, const void* out,
                    const float* lse, const void* dout, float* dq, float* dk, float* dv, int accumulate,
                    float* delta, bool rows_ready, hipStream_t s) {
  using U = const uint16_t*;
  const int64_t rows = int64_t(p.B) * p.Sq * p.Hq;
  const int64_t threads = rows * (D / 8);
  float* lse2 = delta + bwd_row_plane(rows);
  if (!rows_ready) {
    ProfScope ps(s, kProfBwdDelta);
    hipLaunchKernelGGL(delta_kernel<D>, dim3(unsigned((threads + 255) / 256)), dim3(256), 0, s, rows, p.Sq,
                       p.Hq, static_cast<U>(out), static_cast<U>(dout), lse, delta, lse2);
  }
  using C = BwdCfg<D>;
  static_assert(C::kRows == 256, "bwd_hsplit counts 256-row items");
  const int hs = bwd_hsplit(p);
  // the general instance takes windows, segment ids and position arrays
  const bool general = p.window || p.q_seg || p.q_pos || p.k_pos;
  BwdArgs a{p, static_cast<U>(q), static_cast<U>(k), static_cast<U>(v), static_cast<U>(dout), lse2, delta,
            dq, dk, dv, accumulate, p.B * p.Hkv * ((p.Sk + C::kPairKeys - 1) / C::kPairKeys) * hs,
            p.B * p.Hq * ((p.Sq + C::kRows - 1) / C::kRows), hs, delta + 2 * bwd_row_plane(rows)};
  {
    ProfScope ps(s, kProfBwdMfma);
    if (general)
      hipLaunchKernelGGL((attn_bwd_pair_kernel<C, true>), dim3(unsigned(a.n_kv + a.n_q)), dim3(C::kThreads), 0, s,
                         a);
    else
      hipLaunchKernelGGL((attn_bwd_pair_kernel<C, false>), dim3(unsigned(a.n_kv + a.n_q)), dim3(C::kThreads), 0, s,
                         a);
    if (hs > 1) {
      const int64_t n4 = int64_t(p.B) * p.Sk * p.Hkv * (D / 4);
      hipLaunchKernelGGL(head_split_sum_kernel, dim3(unsigned((2 * n4 + 255) / 256)), dim3(256), 0, s, n4, dk, dv,
                         a.part);
    }
  }
  return hipGetLastError();
}

}  // namespace

int64_t bwd_head_split_floats(const AttnProblem& p) {
  if (p.D != 32 && p.D != 64 && p.D != 128) return 0;
  return bwd_hsplit(p) > 1 ? 2 * int64_t(p.B) * p.Sk * p.Hkv * p.D : 0;
}

hipError_t launch_attn_bwd_bf16(const AttnProblem& p, const void* q, const void* k, const void* v,
                                const void* out, const float* lse, const void* dout, float* dq,
                                float* dk, float* dv, int accumulate, float* delta, bool rows_ready,
                                hipStream_t s) {
  switch (p.D) {
    case 128: return launch_d<128>(p, q, k, v, out, lse, dout, dq, dk, dv, accumulate, delta, rows_ready, s);
    case 64: return launch_d<64>(p, q, k, v, out, lse, dout, dq, dk, dv, accumulate, delta, rows_ready, s);
    case 32: return launch_d<32>(p, q, k, v, out, lse, dout, dq, dk, dv, accumulate, delta, rows_ready, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace cp

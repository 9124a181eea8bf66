// Blockwise causal attention forward, bf16 in / float32 accumulate, on the gfx950
// matrix cores.  Returns out and the per-row log-sum-exp at given query/key
// positions, with segment ids, a sliding window and grouped kv heads.
//
// Definition: handbook "Context parallelism: Ring Attention and Ulysses",
// §"Which operations partition directly" (attention with q_offset / k_offset
// returning the log-sum-exp that the ring merge needs).  Rows with no visible key
// give out = 0, lse = -inf.
//
// Design (CDNA4, wave64):
//  * A workgroup owns kRows = NW * 32 query rows of one (batch, q head); each
//    wavefront owns 32 rows, held in registers as bf16 MFMA operands.  The register
//    budget admits two wavefronts per SIMD, so one wave's matrix products overlap
//    the other's softmax.
//  * K/V tiles of BN keys stream through LDS, double-buffered, by LDS-DMA (buffer
//    loads that write LDS directly, no staging registers): the DMA of tile t+1 runs
//    while tile t is multiplied.  Both tiles are stored row-major with an XOR
//    swizzle of their 16-byte chunks; K rows are read as 16-byte fragments and V^T
//    fragments with the gfx950 LDS transpose read, conflict-free both ways.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    each lane then holds one query column, so the row max / row sum of the online
//    softmax need only one exchange between the two 32-lane halves.  The K rows are
//    loaded with bits 2 and 3 of the row index swapped, which makes each lane's
//    score registers exactly the 8 consecutive keys that the P^T operand of the
//    next product, O^T += V^T P^T, expects.
//  * Softmax in the base-2 domain (one v_exp_f32 per score).  The running max is
//    raised (and O, l rescaled) only when a row's max grows by more than 2^8;
//    otherwise the stale max is kept, which is exact because out = O / l uses the
//    same max in numerator and denominator, and keeps P <= 2^8.
//  * Tiles are classified per workgroup and per wavefront as empty (skipped: no
//    load, no math), full (no mask) or partial (elementwise mask) from the
//    extreme positions / segment ids of the tile, which are monotone; a
//    workgroup's walk is confined to the bisected range of key tiles that can hold
//    a visible pair.
//  * Causal grids run the heaviest query tiles of every head first.
//  * Grids with fewer query tiles than two rounds of workgroup slots split each
//    tile's live key tiles over two key groups: two wavefront groups of one
//    workgroup combining through LDS, or (with a workspace, >= 8192 keys and, at
//    D = 128, at most 1.5 query tiles per CU) two workgroups whose float32
//    partials a combine kernel merges.  In the fused ring step over a short block
//    the two groups of a workgroup synchronise each on its own after every tile.
#include <type_traits>

#include "mfma_common.h"
#include "prof.h"

namespace cp {
namespace {

using namespace mfma;

constexpr float kRescaleLog2 = 8.0f;  // lazy-rescale threshold (log2 units)
// longest live key-tile range (64-key tiles) of a fused ring step whose two key
// groups synchronise on their own (blocks of up to 4096 keys)
constexpr int kGroupSyncMaxTiles = 64;

// LDS reads at explicit byte addresses.  The forward keeps the lane-dependent part of
// every operand address in a few registers and adds the stage and product offsets as
// instruction immediates, so one register set serves every stage of both key groups.
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
CP_DEVICE uint32_t lds_addr(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint8_t*)p));
}
CP_DEVICE bf16x8 lds_ld8(uint32_t a) { return *(const lds_bf16x8*)(uintptr_t(a)); }
CP_DEVICE bf16x8 lds_tr8(uint32_t a0, uint32_t a1) {
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(uintptr_t(a0)));
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(uintptr_t(a1)));
  return __builtin_bit_cast(bf16x8, v8i16(__builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7)));
}

// NW row wavefronts (32 query rows each) per key group; NS key groups (1 or 2) that
// take alternate live key tiles of the same rows and combine their partial softmax
// states at the end (for grids too small to fill the chip with whole tiles).
// SPLIT: the NS = 2 key groups of a query tile are two workgroups instead of one
// (workgroup 2t + g is group g of tile t); each writes its partial (out, lse) to a
// float32 workspace and a second kernel combines the pair.
template <int D_, int NW_, int BN_, int NS_, bool SPLIT_ = false>
struct FwdCfg {
  static constexpr int D = D_, NW = NW_, BN = BN_, NS = NS_;
  static constexpr bool SPLIT = SPLIT_;
  static constexpr int kGroupThreads = 64 * NW;
  static constexpr int kThreads = SPLIT ? kGroupThreads : kGroupThreads * NS;
  static constexpr int kRows = 32 * NW;
  static constexpr int KS = D / 16;   // k-steps of S^T = K Q^T
  static constexpr int KB = BN / 32;  // 32-key blocks of a tile
  static constexpr int DB = D / 32;   // 32-row d blocks of O^T
  static constexpr int PT = BN / 16;  // k-steps of O^T += V^T P^T
  static constexpr int kTileElems = BN * D;  // swizzled row-major K or V tile
  static constexpr int kStageBytes = 2 * kTileElems * 2 + BN * 2 * 4;  // K, V, kpos, kseg
  static constexpr int kStagesBytes = (SPLIT ? 1 : NS) * 2 * kStageBytes;
  // spans of up to kSpanTiles key tiles, cached when they come from position /
  // segment arrays (a span is then two dependent global loads)
  static constexpr int kSpanTiles = 512;
  static constexpr int kLdsBytes = kStagesBytes + kSpanTiles * 16 + 16;  // + the key groups' arrival counters
  // exchange of the second key group's (o, m, l) per lane, over the stages
  static constexpr int kXchgBytes = NW * 64 * (DB * 16 + 2) * 4;
  static constexpr int kAhead = 2;  // LDS operand reads issued ahead of their product
  using Tile = DmaTile<BN, D, kGroupThreads>;
  static_assert(D % 32 == 0 && BN % 32 == 0, "tile shape");
  static_assert(NS == 1 || (NS == 2 && (SPLIT || kXchgBytes <= kStagesBytes)), "key groups");
  static_assert(!SPLIT || NS == 2, "a split pairs two key groups");
};

// kMerge = false: write out (bf16) and lse.  kMerge = true (fused ring step): merge
// the block's float32 result into acc [B,Sq,Hq,D] and lse (= lse_acc) in place.
// C::SPLIT: out / lse are ignored; the group's partial result goes to part_o
// [2][B,Sq,Hq,D] and part_l [2][B,Hq,Sq] (float32, normalised, natural-log lse).
// kLane enables the one-tile-per-lane classification of windowed or segmented
// problems (its own instance, so that dense problems run without its per-tile tests).
template <class C, bool kMerge, bool kLane>
CP_DEVICE void fwd_body(const AttnProblem& p, const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                        const uint16_t* __restrict__ v, uint16_t* __restrict__ out, float* __restrict__ acc,
                        float* __restrict__ lse, uint8_t* smem, float* __restrict__ part_o = nullptr,
                        float* __restrict__ part_l = nullptr) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wavefront
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int grp = C::SPLIT ? int(blockIdx.x & 1) : C::NS > 1 ? wave / C::NW : 0;  // key group
  const int rw = wave % C::NW;                    // row wavefront within the group
  const int gtid = tid % C::kGroupThreads;

  // heaviest query tiles of every (batch, head) first
  const int n_qt = (p.Sq + C::kRows - 1) / C::kRows;
  const int order = C::SPLIT ? int(blockIdx.x >> 1) : int(blockIdx.x);
  const int tile_rank = order / (p.B * p.Hq);
  const int bh = order - tile_rank * (p.B * p.Hq);
  const int qt = p.causal ? (n_qt - 1 - tile_rank) : tile_rank;
  const int h = bh % p.Hq;
  const int b = bh / p.Hq;
  const int g = h / (p.Hq / p.Hkv);
  const int q0 = qt * C::kRows;
  const int wq0 = q0 + rw * 32;
  const int64_t krs = int64_t(p.Hkv) * C::D;

  const uint16_t* kbase = k + int64_t(b) * p.Sk * krs + int64_t(g) * C::D;
  const uint16_t* vbase = v + int64_t(b) * p.Sk * krs + int64_t(g) * C::D;

  const Span wg_q = q_span(p, b, q0, min(q0 + C::kRows, p.Sq) - 1);
  if constexpr (kMerge) {
    // A block none of whose keys these rows can see leaves the running result as it
    // is: decided from the extreme positions / segment ids before any other load
    // (half the query tiles of a zigzag ring step see no key of a later block).
    const Span all_k = k_span(p, b, 0, p.Sk - 1);
    if (keys_after(p, wg_q, all_k) || keys_before(p, wg_q, all_k)) return;
  }
  const bool wave_live = wq0 < p.Sq;
  const Span wv_q = q_span(p, b, min(wq0, p.Sq - 1), min(wq0 + 32, p.Sq) - 1);
  const int n_kt = (p.Sk + C::BN - 1) / C::BN;

  // The K / V rows of the walk's first tile are requested now, before the key spans
  // that fix it: it is tile 0 (key group 1 of a split pair: tile 1) whenever these
  // rows see the first keys, as in every causal ring step.  Another first tile
  // waits for this DMA to land before its own is issued.
  typename C::Tile tk, tv;
  const uint32_t krs_bytes = uint32_t(krs) * 2u;
  tk.init(krs_bytes, gtid);
  tv.init(krs_bytes, gtid);
  const int spec_kt = C::NS > 1 ? grp : 0;
  const bool spec = spec_kt < n_kt;
  uint8_t* const stage0 = smem + ((C::SPLIT ? 0 : grp) * 2) * C::kStageBytes;
  if (spec) {
    tk.load(kbase, krs_bytes, spec_kt * C::BN, p.Sk, reinterpret_cast<uint16_t*>(stage0));
    tv.load(vbase, krs_bytes, spec_kt * C::BN, p.Sk, reinterpret_cast<uint16_t*>(stage0) + C::kTileElems);
  }

  // ---- Q fragments (B operand of S^T = K Q^T) and this lane's query position / segment
  const int row = min(wq0 + l32, p.Sq - 1);
  const bool row_ok = wq0 + l32 < p.Sq;
  bf16x8 qf[C::KS];
  {
    const uint16_t* qrow = q + ((int64_t(b) * p.Sq + row) * p.Hq + h) * C::D;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(qrow + ks * 16 + hi * 8);
      qf[ks] = __builtin_bit_cast(bf16x8, row_ok ? x : u32x4{0, 0, 0, 0});
    }
  }
  const int qp = qpos_at(p, row);
  const int qs = qseg_at(p, b, row);

  f32x16 o[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) o[db] = f32x16{};
  float m = -INFINITY, l = 0.0f;

  const float c2 = p.scale * kLog2e;

  // Spans of the key tiles.  With position or segment arrays each one is two
  // dependent global loads, which the walk and the per-wave classification would
  // wait for at every tile; all tiles' spans are then loaded once, in parallel,
  // into LDS (for up to kSpanTiles tiles).
  const bool span_cached = (p.k_pos != nullptr || p.k_seg != nullptr) && n_kt <= C::kSpanTiles;
  i32x4* span_l = reinterpret_cast<i32x4*>(smem + C::kStagesBytes);
  if (span_cached) {
    for (int t = tid; t < n_kt; t += C::kThreads) {
      const Span s = k_span(p, b, t * C::BN, min(t * C::BN + C::BN, p.Sk) - 1);
      span_l[t] = i32x4{s.pos_lo, s.pos_hi, s.seg_lo, s.seg_hi};
    }
    __syncthreads();
  }
  auto tile_span = [&](int kt) {
    if (span_cached) {
      const i32x4 x = span_l[kt];
      return Span{x[0], x[1], x[2], x[3]};
    }
    return k_span(p, b, kt * C::BN, min(kt * C::BN + C::BN, p.Sk) - 1);
  };
  auto tile_class = [&](int kt, const Span& qsp) {
    return classify(p, qsp, tile_span(kt), kt * C::BN + C::BN > p.Sk);
  };
  // the workgroup's live key tiles lie in [kt_lo, kt_hi); the walk stays inside
  const int kt_lo = first_true(0, n_kt, [&](int kt) { return !keys_before(p, wg_q, tile_span(kt)); });
  const int kt_hi = first_true(kt_lo, n_kt, [&](int kt) { return keys_after(p, wg_q, tile_span(kt)); });
  if constexpr (kMerge) {
    // no key of this block is visible to these rows: merging a weight-0 block
    // leaves the running result as it is, so nothing is read or written
    if (kt_lo >= kt_hi) {
      wait_all();  // the first tile's DMA must land before the workgroup's LDS is freed
      return;
    }
  }
  // Without a window or segment ids every tile of [kt_lo, kt_hi) holds a visible
  // pair (its first key is visible to the run's last query, positions increasing),
  // so the walk needs no classification there.
  const bool dense = !p.window && !p.q_seg;
  // Other problems with at most 64 tiles in [kt_lo, kt_hi) classify them all at once,
  // one tile per lane: ballots give the workgroup's live tiles and this wavefront's
  // full and partial tiles as bit masks over kt - kt_lo, and the walk becomes a bit
  // scan.
  const bool lane_cls = kLane && !dense && kt_hi - kt_lo <= 64;
  uint64_t live_m = 0, wfull_m = 0, wpart_m = 0;
  if (lane_cls) {
    const int kt = kt_lo + lane;
    int cg = kEmpty, cw = kEmpty;
    if (kt < kt_hi) {
      const Span ks = tile_span(kt);
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
  // This wavefront's class of a tile.  Dense problems are classified by range: along
  // the tile index the class runs full ... full, partial ... partial, empty ...
  // (positions increase), so two bisections per wavefront replace the per-tile
  // classification; the last tile is partial when ragged.
  int kt_full = n_kt, kt_wend = n_kt;
  if (dense && wave_live && p.causal) {
    kt_wend = first_true(kt_lo, kt_hi, [&](int kt) { return tile_span(kt).pos_lo > wv_q.pos_hi; });
    kt_full = first_true(kt_lo, kt_wend, [&](int kt) { return tile_span(kt).pos_hi > wv_q.pos_lo; });
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
  // Dense causal problems: the tiles below kt_wg_full are full for every row of the
  // workgroup (positions increase), so no wavefront masks them and their key
  // positions are not needed in LDS.
  int kt_wg_full = kt_lo;
  if (dense && p.causal && !p.k_pos)
    kt_wg_full = first_true(kt_lo, kt_hi, [&](int kt) {
      return kt * C::BN + C::BN > p.Sk || tile_span(kt).pos_hi > wg_q.pos_lo;
    });
  // stage layout: K tile, V tile (swizzled row-major), kpos, kseg
  // the tile's key positions and segment ids (stage_load adds its K / V rows)
  auto stage_aux = [&](int kt, uint8_t* stage) {
    int* kpos = reinterpret_cast<int*>(reinterpret_cast<uint16_t*>(stage) + 2 * C::kTileElems);
    int* kseg = kpos + C::BN;
    // key positions / segment ids: LDS-DMA from their arrays (one row wavefront of
    // the group each), or written as offset + index / 0; keys past the end are
    // masked by their index
    const int j0 = kt * C::BN;
    if (p.k_pos) {
      if (rw == 0) dma_dwords<C::BN>(p.k_pos, j0, p.Sk - j0, kpos, lane);
    } else if (kt >= kt_wg_full) {
      for (int t = gtid; t < C::BN; t += C::kGroupThreads) kpos[t] = p.k_offset + j0 + t;
    }
    // (segment ids are compared only when q_seg is given: no fill otherwise)
    if (p.k_seg) {
      if (rw == 1 % C::NW) dma_dwords<C::BN>(p.k_seg, int64_t(b) * p.Sk + j0, p.Sk - j0, kseg, lane);
    } else if (p.q_seg) {
      for (int t = gtid; t < C::BN; t += C::kGroupThreads) kseg[t] = 0;
    }
  };
  auto stage_load = [&](int kt, uint8_t* stage) {
    uint16_t* ks = reinterpret_cast<uint16_t*>(stage);
    tk.load(kbase, krs_bytes, kt * C::BN, p.Sk, ks);
    tv.load(vbase, krs_bytes, kt * C::BN, p.Sk, ks + C::kTileElems);
    stage_aux(kt, stage);
  };
  auto stage_of = [&](int buf) { return smem + ((C::SPLIT ? 0 : grp) * 2 + buf) * C::kStageBytes; };
  // Lane-dependent byte offsets (within this group's stage 0, the group's stage base
  // included) of the K row reads of S^T (one per k-step; the key block adds
  // kb * 32 rows) and of the two halves of the V^T transposed reads of O^T (one per
  // d block; the key step adds 16 rows).  The XOR swizzle of a row depends on the
  // row modulo 16 only, so these are the same for every key block / key step.
  uint32_t koff[C::KS], voff[2 * C::DB];
  {
    const uint32_t g0 = lds_addr(stage_of(0));
    const int pr = perm_row(l32);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) koff[ks] = g0 + 2u * uint32_t(rm_elem<C::D>(pr, 2 * ks + hi));
    const int gq = lane >> 4, iq = lane & 15;
    const int r = 8 * (gq >> 1) + (iq >> 2);
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      const int d = db * 32 + 16 * (gq & 1) + 4 * (iq & 3);
      const uint32_t vt = g0 + 2u * C::kTileElems;
      voff[2 * db] = vt + 2u * uint32_t(r * C::D + (((d >> 3) ^ chunk_xor<C::D>(r)) << 3) + (d & 7));
      voff[2 * db + 1] = vt + 2u * uint32_t((r + 4) * C::D + (((d >> 3) ^ chunk_xor<C::D>(r + 4)) << 3) + (d & 7));
    }
  }

  // Live tiles are taken in pairs (t0, t1): key group 0 multiplies t0, group 1 t1
  // (with one group, t1 is unused).  Every wavefront walks the same pair sequence,
  // so all of them meet the same barriers.
  int t0 = next_tile(0);
  int t1 = (C::NS > 1 && t0 < n_kt) ? next_tile(t0 + 1) : n_kt;
  if (t0 < n_kt) {
    int cur = grp == 0 ? t0 : t1;
    if (cur < n_kt) {
      if (spec && cur == spec_kt) {
        stage_aux(cur, stage_of(0));  // its K / V rows are already in flight
      } else {
        if (spec) wait_all();
        stage_load(cur, stage_of(0));
      }
    }
    int* arrivals = reinterpret_cast<int*>(smem + C::kStagesBytes + C::kSpanTiles * 16);
    if (tid < 2) arrivals[tid] = 0;
    wait_all();
    __syncthreads();
    const MaskSpec ms = make_mask_spec(p.causal, p.window, p.q_seg != nullptr);
    // In the fused ring step over a short block the two key groups synchronise each
    // on its own after every tile (each has its own stages), so they drift apart
    // instead of meeting at one workgroup barrier: every wavefront of the group
    // finishes its loads and LDS accesses, adds one to the group's counter and waits
    // until all NW have arrived at this tile.  Measured: the llama2-7b ring pass (32
    // live tiles per workgroup and step) 4% faster; long walks (hundreds of tiles)
    // 1.5-4% slower, so they keep the workgroup barrier.  The wait gives up after
    // 2^22 polls, a safety bound no correct run reaches.
    constexpr bool kGroupSync = kMerge && C::NS > 1 && !C::SPLIT;
    const bool gsync = kGroupSync && kt_hi - kt_lo <= kGroupSyncMaxTiles;
    int arrived = 0;
    auto group_barrier = [&]() {
      wait_all();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_sched_barrier(0);
      arrived += C::NW;
      if (lane == 0) __hip_atomic_fetch_add(&arrivals[grp], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      for (int spin = 0; spin < (1 << 22); ++spin) {
        const int now = __builtin_amdgcn_readfirstlane(
            __hip_atomic_load(&arrivals[grp], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
        if (now >= arrived) break;
        __builtin_amdgcn_s_sleep(1);
      }
      __builtin_amdgcn_sched_barrier(0);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };
    f32x16 s[C::KB];    // S^T of a tile between its products and its softmax
    bf16x8 pf[C::PT];   // P^T of a tile between its softmax and its V product
    // product lists: S^T = K Q^T from stage B's K tile (kb = i % KB, k-step i / KB)
    // and O^T += V^T P^T from stage B's V tile (d block i % DB, key step i / DB)
    constexpr int kNS = C::KS * C::KB, kNV = C::PT * C::DB;
    auto s_load = [&](auto bufc, int i) {
      constexpr uint32_t sb = decltype(bufc)::value * C::kStageBytes;
      return lds_ld8(koff[i / C::KB] + (sb + 2u * (i % C::KB) * 32 * C::D));
    };
    auto s_mul = [&](int i, bf16x8 f) { s[i % C::KB] = mma(f, qf[i / C::KB], s[i % C::KB]); };
    auto v_load = [&](auto bufc, int i) {
      const uint32_t rb = decltype(bufc)::value * C::kStageBytes + 2u * (i / C::DB) * 16 * C::D;
      return lds_tr8(voff[2 * (i % C::DB)] + rb, voff[2 * (i % C::DB) + 1] + rb);
    };
    auto v_mul = [&](int i, bf16x8 f) { o[i % C::DB] = mma(f, pf[i / C::DB], o[i % C::DB]); };
    auto pin_k = [&]() {
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) pin(koff[ks]);
    };
    auto pin_v = [&]() {
#pragma unroll
      for (int j = 0; j < 2 * C::DB; ++j) pin(voff[j]);
    };
    // mask of tile kt (class wcls; key positions / segment ids from stage B) and
    // its online softmax: s -> m, l (rescaling o) and pf
    auto softmax = [&](auto bufc, int kt, int wcls) {
      const uint16_t* ks_l = reinterpret_cast<const uint16_t*>(stage_of(decltype(bufc)::value));
      const int* kpos_l = reinterpret_cast<const int*>(ks_l + 2 * C::kTileElems);
      const int* kseg_l = kpos_l + C::BN;
      if (wcls == kPartial) {
        // keys of this lane's registers: key_of_reg(0, hi) plus a constant, so the
        // bound test compares constants with one per-lane limit
        const int lim = p.Sk - kt * C::BN - key_of_reg(0, hi);
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            // registers 4jj..4jj+3 hold 4 consecutive keys
            const int rel = kb * 32 + key_of_reg(4 * jj, 0);  // key - key_of_reg(0, hi)
            const int kk0 = kb * 32 + key_of_reg(4 * jj, hi);
            const i32x4 kp4 = *reinterpret_cast<const i32x4*>(kpos_l + kk0);
            const i32x4 kg4 = *reinterpret_cast<const i32x4*>(kseg_l + kk0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              // bitwise &: a short-circuit && here became one branch per element
              const bool vis = (rel + i < lim) & pair_visible(ms, qp, kp4[i], qs, kg4[i]);
              s[kb][4 * jj + i] = vis ? s[kb][4 * jj + i] : -INFINITY;
            }
          }
      }

      // online softmax (base 2) with lazy rescaling
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = max_halves(mx) * c2;
      if (__any(mx > m + kRescaleLog2)) {
        const float mnew = fmaxf(m, mx);
        const float alpha = __builtin_amdgcn_exp2f(m - (mnew == -INFINITY ? 0.0f : mnew));
        m = mnew;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < C::DB; ++db) o[db] *= alpha;
      }
      const float muse = m == -INFINITY ? 0.0f : m;
      float rs = 0.0f;
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(s[kb][r], c2, -muse));
          s[kb][r] = pv;
          rs += pv;
        }
      l += rs;
#pragma unroll
      for (int t = 0; t < C::PT; ++t) pf[t] = to_bf16x8(s[t >> 1], 8 * (t & 1));
    };
    // one tile per call, the stage index a compile-time constant (the loop below
    // alternates 0 and 1), so the swizzled LDS addresses of each stage are fixed
    auto iter = [&](auto bufc) -> bool {
      constexpr int buf = decltype(bufc)::value;
      const int n0 = next_tile((C::NS > 1 && t1 < n_kt ? t1 : t0) + 1);
      const int n1 = (C::NS > 1 && n0 < n_kt) ? next_tile(n0 + 1) : n_kt;
      const int nxt = grp == 0 ? n0 : n1;
      const bool has_next = n0 < n_kt;
      // the DMA of the next tile runs while this one is multiplied
      if (nxt < n_kt) stage_load(nxt, stage_of(buf ^ 1));
      const int wcls = (wave_live && cur < n_kt) ? wave_class(cur) : kEmpty;
      if (wcls != kEmpty) {
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) s[kb] = f32x16{};
        pin_k();
        pipelined_products<kNS, C::kAhead>([&](int i) { return s_load(bufc, i); }, s_mul);
        softmax(bufc, cur, wcls);
        pin_v();
        pipelined_products<kNV, C::kAhead>([&](int i) { return v_load(bufc, i); }, v_mul);
      }
      if (gsync) {
        group_barrier();
      } else {
        wait_all();
        __syncthreads();
      }
      t0 = n0;
      t1 = n1;
      cur = nxt;
      return has_next;
    };
    while (iter(std::integral_constant<int, 0>{}) && iter(std::integral_constant<int, 1>{})) {
    }
  } else if (spec) {
    // no live tile: the first tile's DMA lands before the stages are reused below
    wait_all();
    __syncthreads();
  }

  if constexpr (C::NS > 1 && !C::SPLIT) {
    // both groups are done with their stages, which the exchange below overlaps (with
    // group-local synchronisation the other group may still be in its walk)
    if constexpr (kMerge) __syncthreads();
    // combine the two key groups' partial states of each row (same lane layout):
    // m = max(m0, m1), o = o0 2^(m0-m) + o1 2^(m1-m), l likewise
    float* xo = reinterpret_cast<float*>(smem) + rw * (C::DB * 16) * 64 + lane;
    float* xm = reinterpret_cast<float*>(smem) + C::NW * (C::DB * 16) * 64 + rw * 64 + lane;
    float* xl = xm + C::NW * 64;
    if (grp == 1) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) xo[(db * 16 + r) * 64] = o[db][r];
      *xm = m;
      *xl = l;
    }
    __syncthreads();
    if (grp == 1) return;
    const float m1 = *xm, l1 = *xl;
    const float mn = fmaxf(m, m1);
    const float a0 = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m - mn);
    const float a1 = m1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - mn);
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] = o[db][r] * a0 + xo[(db * 16 + r) * 64] * a1;
    l = l * a0 + l1 * a1;
    m = mn;
  }

  // ---- epilogue: normalise; store out (bf16) and lse (natural log), or merge
  const float lt = sum_halves(l);
  if (!row_ok) return;
  const bool any = lt > 0.0f;
  const float inv = any ? 1.0f / lt : 0.0f;
  const float lse_blk = any ? (m + __log2f(lt)) * kLn2 : -INFINITY;
  const int64_t li = (int64_t(b) * p.Hq + h) * p.Sq + row;
  const int64_t orow = ((int64_t(b) * p.Sq + row) * p.Hq + h) * C::D;
  if constexpr (C::SPLIT) {
    // this group's normalised partial; a group with no visible key writes o = 0,
    // lse = -inf (weight 0 in the combine)
    const int64_t plane = int64_t(p.B) * p.Sq * p.Hq * C::D;
    float* prow = part_o + grp * plane + orow;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x16& a = o[db];
        *reinterpret_cast<f32x4*>(prow + db * 32 + 8 * j + 4 * hi) =
            f32x4{a[4 * j] * inv, a[4 * j + 1] * inv, a[4 * j + 2] * inv, a[4 * j + 3] * inv};
      }
    if (hi == 0) part_l[grp * (int64_t(p.B) * p.Hq * p.Sq) + li] = lse_blk;
  } else if constexpr (kMerge) {
    // both 32-lane halves read the row's old lse before either writes the new one
    const MergeWeights w = merge_weights(lse[li], lse_blk);
    const float fb = w.wb * inv;
    float* arow = acc + orow;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x16& a = o[db];
        f32x4* dst = reinterpret_cast<f32x4*>(arow + db * 32 + 8 * j + 4 * hi);
        const f32x4 old = *dst;
        *dst = f32x4{old[0] * w.wa + a[4 * j] * fb, old[1] * w.wa + a[4 * j + 1] * fb,
                     old[2] * w.wa + a[4 * j + 2] * fb, old[3] * w.wa + a[4 * j + 3] * fb};
      }
    if (hi == 0) lse[li] = w.lse;
  } else {
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x16& a = o[db];
        const u32x2 wv{pack_bf16x2(a[4 * j] * inv, a[4 * j + 1] * inv),
                       pack_bf16x2(a[4 * j + 2] * inv, a[4 * j + 3] * inv)};
        *reinterpret_cast<u32x2*>(out + orow + db * 32 + 8 * j + 4 * hi) = wv;
      }
    if (hi == 0) lse[li] = lse_blk;
  }
}

template <class C, bool kLane>
__global__ __launch_bounds__(C::kThreads, 2) void attn_fwd_mfma_kernel(AttnProblem pa, const uint16_t* q,
                                                                       const uint16_t* k, const uint16_t* v,
                                                                       uint16_t* out, float* lse) {
  __shared__ __align__(16) uint8_t smem[C::kLdsBytes];
  const AttnProblem p = specialize<kLane>(pa);
  fwd_body<C, false, kLane>(p, q, k, v, out, nullptr, lse, smem);
}

template <class C, bool kLane>
__global__ __launch_bounds__(C::kThreads, 2) void attn_fwd_merge_mfma_kernel(AttnProblem pa, const uint16_t* q,
                                                                             const uint16_t* k,
                                                                             const uint16_t* v, float* acc,
                                                                             float* lse_acc) {
  __shared__ __align__(16) uint8_t smem[C::kLdsBytes];
  const AttnProblem p = specialize<kLane>(pa);
  fwd_body<C, true, kLane>(p, q, k, v, nullptr, acc, lse_acc, smem);
}

template <class C, bool kLane>
__global__ __launch_bounds__(C::kThreads, 2) void attn_fwd_split_kernel(AttnProblem pa, const uint16_t* q,
                                                                        const uint16_t* k, const uint16_t* v,
                                                                        float* part_o, float* part_l) {
  __shared__ __align__(16) uint8_t smem[C::kLdsBytes];
  const AttnProblem p = specialize<kLane>(pa);
  fwd_body<C, false, kLane>(p, q, k, v, nullptr, nullptr, nullptr, smem, part_o, part_l);
}

// out = merge of the two partials of every (row, head), rounded to bf16, and the
// merged lse: the ring-step merge rule applied to the two key halves (weights
// e^(lse_g - lse), a -inf half has weight 0; both -inf gives out = 0, lse = -inf).
// One thread per 8 consecutive elements of a row.
template <int D>
__global__ __launch_bounds__(256) void split_combine_kernel(int64_t rows, int Sq, int Hq, const float* part_o,
                                                            const float* part_l, uint16_t* out, float* lse) {
  constexpr int kPer = D / 8;
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t row = t / kPer;  // (b, i, h) row of out
  if (row >= rows) return;
  const int c = int(t % kPer);
  const int h = int(row % Hq);
  const int64_t bi = row / Hq;
  const int i = int(bi % Sq);
  const int64_t b = bi / Sq;
  const int64_t li = (b * Hq + h) * Sq + i;
  const MergeWeights w = merge_weights(part_l[li], part_l[rows + li]);
  const int64_t e = row * D + c * 8;
  const int64_t plane = rows * D;
  const f32x4 a0 = *reinterpret_cast<const f32x4*>(part_o + e);
  const f32x4 a1 = *reinterpret_cast<const f32x4*>(part_o + e + 4);
  const f32x4 b0 = *reinterpret_cast<const f32x4*>(part_o + plane + e);
  const f32x4 b1 = *reinterpret_cast<const f32x4*>(part_o + plane + e + 4);
  const u32x4 r{pack_bf16x2(a0[0] * w.wa + b0[0] * w.wb, a0[1] * w.wa + b0[1] * w.wb),
                pack_bf16x2(a0[2] * w.wa + b0[2] * w.wb, a0[3] * w.wa + b0[3] * w.wb),
                pack_bf16x2(a1[0] * w.wa + b1[0] * w.wb, a1[1] * w.wa + b1[1] * w.wb),
                pack_bf16x2(a1[2] * w.wa + b1[2] * w.wb, a1[3] * w.wa + b1[3] * w.wb)};
  *reinterpret_cast<u32x4*>(out + e) = r;
  if (c == 0) lse[li] = w.lse;
}

template <class C, bool kMerge>
hipError_t launch_cfg(const AttnProblem& p, const void* q, const void* k, const void* v, void* out,
                      float* acc, float* lse, hipStream_t s) {
  const unsigned n = unsigned((p.Sq + C::kRows - 1) / C::kRows) * unsigned(p.Hq * p.B);
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kk = static_cast<const uint16_t*>(k);
  const auto* vv = static_cast<const uint16_t*>(v);
  const bool masked = p.window || p.q_seg;
  if constexpr (kMerge) {
    ProfScope ps(s, kProfFwdMergeMfma);
    if (masked)
      hipLaunchKernelGGL((attn_fwd_merge_mfma_kernel<C, true>), dim3(n), dim3(C::kThreads), 0, s, p, qq, kk, vv,
                         acc, lse);
    else
      hipLaunchKernelGGL((attn_fwd_merge_mfma_kernel<C, false>), dim3(n), dim3(C::kThreads), 0, s, p, qq, kk, vv,
                         acc, lse);
  } else {
    ProfScope ps(s, kProfFwdMfma);
    auto* o = static_cast<uint16_t*>(out);
    if (masked)
      hipLaunchKernelGGL((attn_fwd_mfma_kernel<C, true>), dim3(n), dim3(C::kThreads), 0, s, p, qq, kk, vv, o, lse);
    else
      hipLaunchKernelGGL((attn_fwd_mfma_kernel<C, false>), dim3(n), dim3(C::kThreads), 0, s, p, qq, kk, vv, o, lse);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_split(const AttnProblem& p, const void* q, const void* k, const void* v, void* out, float* lse,
                        float* ws, hipStream_t s) {
  using C = FwdCfg<D, 4, 64, 2, true>;
  const int64_t rows = int64_t(p.B) * p.Sq * p.Hq;
  float* part_o = ws;
  float* part_l = ws + 2 * rows * D;
  const unsigned n = 2u * unsigned((p.Sq + C::kRows - 1) / C::kRows) * unsigned(p.Hq * p.B);
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kk = static_cast<const uint16_t*>(k);
  const auto* vv = static_cast<const uint16_t*>(v);
  ProfScope ps(s, kProfFwdMfma);
  if (p.window || p.q_seg)
    hipLaunchKernelGGL((attn_fwd_split_kernel<C, true>), dim3(n), dim3(C::kThreads), 0, s, p, qq, kk, vv, part_o,
                       part_l);
  else
    hipLaunchKernelGGL((attn_fwd_split_kernel<C, false>), dim3(n), dim3(C::kThreads), 0, s, p, qq, kk, vv, part_o,
                       part_l);
  const int64_t threads = rows * (D / 8);
  hipLaunchKernelGGL(split_combine_kernel<D>, dim3(unsigned((threads + 255) / 256)), dim3(256), 0, s, rows, p.Sq,
                     p.Hq, part_o, part_l, static_cast<uint16_t*>(out), lse);
  return hipGetLastError();
}

// Workgroup slots of the device at two workgroups per CU.
int wg_slots() { return 2 * device_cus(); }

// Fewer query tiles than two rounds of workgroup slots: split each tile's keys over
// two wavefront groups, so the heaviest (causal) tiles no longer set the time.
template <int D, bool kMerge>
hipError_t launch_dim(const AttnProblem& p, const void* q, const void* k, const void* v, void* out,
                      float* acc, float* lse, hipStream_t s) {
  const int64_t tiles = int64_t((p.Sq + 127) / 128) * p.Hq * p.B;
  if (tiles < 2 * int64_t(wg_slots()))
    return launch_cfg<FwdCfg<D, 4, 64, 2>, kMerge>(p, q, k, v, out, acc, lse, s);
  return launch_cfg<FwdCfg<D, 4, 64, 1>, kMerge>(p, q, k, v, out, acc, lse, s);
}

template <bool kMerge>
hipError_t launch_d(const AttnProblem& p, const void* q, const void* k, const void* v, void* out,
                    float* acc, float* lse, hipStream_t s) {
  switch (p.D) {
    case 128: return launch_dim<128, kMerge>(p, q, k, v, out, acc, lse, s);
    case 64: return launch_dim<64, kMerge>(p, q, k, v, out, acc, lse, s);
    case 32: return launch_dim<32, kMerge>(p, q, k, v, out, acc, lse, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int device_cus() {
  static int cus_of[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cus_of[dev]) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    cus_of[dev] = cus;
  }
  return cus_of[dev];
}

// The combine pass moves 10 bytes per output element (two float32 partials in, bf16
// out); with fewer than 8192 keys that is no longer small next to the attention of
// the row (a 2048-key causal block measured slower split than unsplit).
constexpr int kSplitMinKeys = 8192;

// With D = 128 the split pays only up to about 1.5 query tiles per CU: measured on
// 256 CUs, 320 and 384 tiles ran 10% faster split, 448 and 512 tiles 4% and 7%
// faster as two-group workgroups (the combine pass and the partials' traffic then
// outweigh the finer granularity).  D = 64 still gained from the split at 512 tiles.
bool fwd_split_applies(const AttnProblem& p) {
  const int64_t tiles = int64_t((p.Sq + 127) / 128) * p.Hq * p.B;
  if (p.Sk < kSplitMinKeys) return false;
  if (p.D == 128) return 2 * tiles <= 3 * int64_t(device_cus());
  return tiles < 2 * int64_t(wg_slots());
}

size_t fwd_split_workspace_bytes(const AttnProblem& p) {
  const int64_t rows = int64_t(p.B) * p.Sq * p.Hq;
  return size_t(2 * rows * p.D + 2 * rows) * sizeof(float);
}

hipError_t launch_attn_fwd_split_bf16(const AttnProblem& p, const void* q, const void* k, const void* v,
                                      void* out, float* lse, float* ws, hipStream_t s) {
  switch (p.D) {
    case 128: return launch_split<128>(p, q, k, v, out, lse, ws, s);
    case 64: return launch_split<64>(p, q, k, v, out, lse, ws, s);
    case 32: return launch_split<32>(p, q, k, v, out, lse, ws, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_fwd_bf16(const AttnProblem& p, const void* q, const void* k, const void* v,
                                void* out, float* lse, hipStream_t s) {
  return launch_d<false>(p, q, k, v, out, nullptr, lse, s);
}

hipError_t launch_attn_fwd_merge_bf16(const AttnProblem& p, const void* q, const void* k, const void* v,
                                      float* acc, float* lse_acc, hipStream_t s) {
  return launch_d<true>(p, q, k, v, nullptr, acc, lse_acc, s);
}

}  // namespace cp

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
//  * A workgroup owns kRows = NW * 32 * QB query rows of one (batch, q head); each
//    wavefront owns 32*QB rows, held in registers as bf16 MFMA operands.
//  * K/V tiles of BN keys stream through LDS, double-buffered: the global loads of
//    tile t+1 are in flight while tile t is multiplied.  K is stored [key][d]; V is
//    stored transposed [d][key] so both products read 16-byte operand fragments.
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    each lane then holds one query column, so the row max / row sum of the online
//    softmax need only one exchange between the two 32-lane halves.  The K rows are
//    loaded with bits 2 and 3 of the row index swapped, which makes each lane's
//    score registers exactly the 8 consecutive keys that the P^T operand of the
//    next product, O^T += V^T P^T, expects.
//  * Softmax in the base-2 domain (one v_exp_f32 per score).
//  * Tiles are classified per workgroup and per wavefront as empty (skipped: no
//    load, no math), full (no mask) or partial (elementwise mask) from the
//    extreme positions / segment ids of the tile, which are monotone.
//  * Causal grids run the heaviest query tiles of every head first.
#include "common.h"
#include "launch.h"
#include "prof.h"

namespace cp {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

enum : int { kEmpty = 0, kPartial = 1, kFull = 2 };

// Extreme positions and segment ids of a run of rows (both sequences are monotone).
struct Span {
  int pos_lo, pos_hi, seg_lo, seg_hi;
};

CP_DEVICE int qpos_at(const AttnProblem& p, int i) { return p.q_pos ? p.q_pos[i] : p.q_offset + i; }
CP_DEVICE int kpos_at(const AttnProblem& p, int j) { return p.k_pos ? p.k_pos[j] : p.k_offset + j; }

CP_DEVICE Span q_span(const AttnProblem& p, int b, int r0, int r1) {
  Span s;
  s.pos_lo = qpos_at(p, r0);
  s.pos_hi = qpos_at(p, r1);
  s.seg_lo = p.q_seg ? p.q_seg[int64_t(b) * p.Sq + r0] : 0;
  s.seg_hi = p.q_seg ? p.q_seg[int64_t(b) * p.Sq + r1] : 0;
  return s;
}

CP_DEVICE Span k_span(const AttnProblem& p, int b, int j0, int j1) {
  Span s;
  s.pos_lo = kpos_at(p, j0);
  s.pos_hi = kpos_at(p, j1);
  s.seg_lo = p.k_seg ? p.k_seg[int64_t(b) * p.Sk + j0] : 0;
  s.seg_hi = p.k_seg ? p.k_seg[int64_t(b) * p.Sk + j1] : 0;
  return s;
}

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

CP_DEVICE float other_half(float x) { return __shfl_xor(x, 32, 64); }

template <int D_, int QB_, int NW_, int BN_>
struct FwdCfg {
  static constexpr int D = D_, QB = QB_, NW = NW_, BN = BN_;
  static constexpr int kThreads = 64 * NW;
  static constexpr int kWaveRows = 32 * QB;
  static constexpr int kRows = kWaveRows * NW;
  static constexpr int KS = D / 16;   // k-steps of S^T = K Q^T
  static constexpr int KB = BN / 32;  // 32-key blocks of a tile
  static constexpr int DB = D / 32;   // 32-row d blocks of O^T
  static constexpr int PT = BN / 16;  // k-steps of O^T += V^T P^T
  static constexpr int KLD = D + 8;   // K row pitch in LDS (elements): 16-byte skew per row
  static constexpr int VLD = BN + 8;  // V^T row pitch in LDS (elements)
  static constexpr int kKElems = BN * KLD;
  static constexpr int kVElems = D * VLD;
  static constexpr int kStageBytes = (kKElems + kVElems) * 2 + BN * 2 * 4;  // + kpos, kseg
  static constexpr int kLdsBytes = 2 * kStageBytes;
  static constexpr int kKChunks = BN * D / 8;        // 16-byte chunks of a K tile
  static constexpr int kKIter = (kKChunks + kThreads - 1) / kThreads;
  static constexpr int kVUnits = (BN / 4) * (D / 8);  // 4 keys x 8 dims of a V tile
  static constexpr int kVIter = (kVUnits + kThreads - 1) / kThreads;
  static_assert(D % 32 == 0 && BN % 32 == 0, "tile shape");
};

template <class C>
struct TileRegs {
  u32x4 k[C::kKIter];
  u32x4 v[C::kVIter][4];
};

template <class C>
CP_DEVICE void load_tile(const AttnProblem& p, const uint16_t* __restrict__ kb, const uint16_t* __restrict__ vb,
                         int j0, TileRegs<C>& r) {
  const int tid = threadIdx.x;
  const int64_t rs = int64_t(p.Hkv) * C::D;  // key row stride (elements)
#pragma unroll
  for (int it = 0; it < C::kKIter; ++it) {
    const int c = tid + it * C::kThreads;
    const int key = c / (C::D / 8);
    const int d8 = c - key * (C::D / 8);
    r.k[it] = u32x4{0, 0, 0, 0};
    if (c < C::kKChunks && j0 + key < p.Sk)
      r.k[it] = *reinterpret_cast<const u32x4*>(kb + int64_t(j0 + key) * rs + d8 * 8);
  }
#pragma unroll
  for (int it = 0; it < C::kVIter; ++it) {
    const int u = tid + it * C::kThreads;
    const int key4 = u / (C::D / 8);
    const int d8 = u - key4 * (C::D / 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int key = key4 * 4 + e;
      r.v[it][e] = u32x4{0, 0, 0, 0};
      if (u < C::kVUnits && j0 + key < p.Sk)
        r.v[it][e] = *reinterpret_cast<const u32x4*>(vb + int64_t(j0 + key) * rs + d8 * 8);
    }
  }
}

template <class C>
CP_DEVICE void store_tile(const AttnProblem& p, int b, int j0, const TileRegs<C>& r, uint8_t* stage) {
  uint16_t* ks = reinterpret_cast<uint16_t*>(stage);
  uint16_t* vt = ks + C::kKElems;
  int* kpos = reinterpret_cast<int*>(vt + C::kVElems);
  int* kseg = kpos + C::BN;
  const int tid = threadIdx.x;
#pragma unroll
  for (int it = 0; it < C::kKIter; ++it) {
    const int c = tid + it * C::kThreads;
    const int key = c / (C::D / 8);
    const int d8 = c - key * (C::D / 8);
    if (c < C::kKChunks) *reinterpret_cast<u32x4*>(ks + key * C::KLD + d8 * 8) = r.k[it];
  }
#pragma unroll
  for (int it = 0; it < C::kVIter; ++it) {
    const int u = tid + it * C::kThreads;
    const int key4 = u / (C::D / 8);
    const int d8 = u - key4 * (C::D / 8);
    if (u < C::kVUnits) {
      // transpose 4 keys x 8 dims into 8 rows of 4 consecutive keys
#pragma unroll
      for (int w = 0; w < 4; ++w) {  // dims 2w, 2w+1 live in 32-bit word w
        const uint32_t a0 = r.v[it][0][w], a1 = r.v[it][1][w], a2 = r.v[it][2][w], a3 = r.v[it][3][w];
        const u32x2 lo{(a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16)};
        const u32x2 hi{(a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u)};
        *reinterpret_cast<u32x2*>(vt + (d8 * 8 + 2 * w) * C::VLD + key4 * 4) = lo;
        *reinterpret_cast<u32x2*>(vt + (d8 * 8 + 2 * w + 1) * C::VLD + key4 * 4) = hi;
      }
    }
  }
  for (int t = tid; t < C::BN; t += C::kThreads) {
    const int j = j0 + t;
    const bool ok = j < p.Sk;
    kpos[t] = ok ? kpos_at(p, j) : 0;
    kseg[t] = (ok && p.k_seg) ? p.k_seg[int64_t(b) * p.Sk + j] : 0;
  }
}

// key index within a 32-key block held by score register r of lane half h
CP_DEVICE constexpr int key_of_reg(int r, int h) { return 16 * (r >> 3) + 8 * h + (r & 7); }
// K row loaded by lane row m (bits 2 and 3 swapped)
CP_DEVICE constexpr int perm_row(int m) { return (m & 0x13) | ((m & 4) << 1) | ((m & 8) >> 1); }

template <class C>
__global__ __launch_bounds__(C::kThreads) void attn_fwd_mfma_kernel(AttnProblem p,
                                                                    const uint16_t* __restrict__ q,
                                                                    const uint16_t* __restrict__ k,
                                                                    const uint16_t* __restrict__ v,
                                                                    uint16_t* __restrict__ out,
                                                                    float* __restrict__ lse) {
  __shared__ __align__(16) uint8_t smem[C::kLdsBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // heaviest query tiles of every (batch, head) first
  const int n_qt = (p.Sq + C::kRows - 1) / C::kRows;
  const int tile_rank = int(blockIdx.x) / (p.B * p.Hq);
  const int bh = int(blockIdx.x) - tile_rank * (p.B * p.Hq);
  const int qt = p.causal ? (n_qt - 1 - tile_rank) : tile_rank;
  const int h = bh % p.Hq;
  const int b = bh / p.Hq;
  const int g = h / (p.Hq / p.Hkv);
  const int q0 = qt * C::kRows;
  const int wq0 = q0 + wave * C::kWaveRows;

  const uint16_t* kbase = k + (int64_t(b) * p.Sk * p.Hkv + g) * C::D;
  const uint16_t* vbase = v + (int64_t(b) * p.Sk * p.Hkv + g) * C::D;

  const Span wg_q = q_span(p, b, q0, min(q0 + C::kRows, p.Sq) - 1);
  const bool wave_live = wq0 < p.Sq;
  const Span wv_q = q_span(p, b, min(wq0, p.Sq - 1), min(wq0 + C::kWaveRows, p.Sq) - 1);

  // ---- Q fragments (B operand of S^T = K Q^T) and per-lane query position / segment
  bf16x8 qf[C::QB][C::KS];
  int qp[C::QB], qs[C::QB];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const int row = wq0 + qb * 32 + l32;
    const bool ok = row < p.Sq;
    const int rr = ok ? row : p.Sq - 1;
    const uint16_t* qrow = q + ((int64_t(b) * p.Sq + rr) * p.Hq + h) * C::D;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      u32x4 x = u32x4{0, 0, 0, 0};
      if (ok) x = *reinterpret_cast<const u32x4*>(qrow + ks * 16 + hi * 8);
      qf[qb][ks] = __builtin_bit_cast(bf16x8, x);
    }
    qp[qb] = qpos_at(p, rr);
    qs[qb] = p.q_seg ? p.q_seg[int64_t(b) * p.Sq + rr] : 0;
  }

  f32x16 o[C::QB][C::DB];
  float m[C::QB], l[C::QB];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    m[qb] = -INFINITY;
    l[qb] = 0.0f;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) o[qb][db] = f32x16{};
  }

  const float c2 = p.scale * kLog2e;
  const int n_kt = (p.Sk + C::BN - 1) / C::BN;

  // first / next key tile with any visible pair for this workgroup
  auto tile_class = [&](int kt, const Span& qsp) {
    const int j0 = kt * C::BN;
    const int j1 = min(j0 + C::BN, p.Sk) - 1;
    return classify(p, qsp, k_span(p, b, j0, j1), j1 - j0 + 1 < C::BN);
  };
  auto next_tile = [&](int kt) {
    while (kt < n_kt && tile_class(kt, wg_q) == kEmpty) ++kt;
    return kt;
  };

  int cur = next_tile(0);
  if (cur < n_kt) {
    TileRegs<C> regs;
    load_tile<C>(p, kbase, vbase, cur * C::BN, regs);
    store_tile<C>(p, b, cur * C::BN, regs, smem);
    __syncthreads();
    int buf = 0;
    while (true) {
      const int nxt = next_tile(cur + 1);
      const bool has_next = nxt < n_kt;
      if (has_next) load_tile<C>(p, kbase, vbase, nxt * C::BN, regs);

      const int wcls = wave_live ? tile_class(cur, wv_q) : kEmpty;
      if (wcls != kEmpty) {
        const uint8_t* stage = smem + buf * C::kStageBytes;
        const uint16_t* ks_l = reinterpret_cast<const uint16_t*>(stage);
        const uint16_t* vt_l = ks_l + C::kKElems;
        const int* kpos_l = reinterpret_cast<const int*>(vt_l + C::kVElems);
        const int* kseg_l = kpos_l + C::BN;

        // S^T = K Q^T
        f32x16 s[C::QB][C::KB];
#pragma unroll
        for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
          for (int kb = 0; kb < C::KB; ++kb) s[qb][kb] = f32x16{};
#pragma unroll
        for (int kstep = 0; kstep < C::KS; ++kstep) {
#pragma unroll
          for (int kb = 0; kb < C::KB; ++kb) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(
                ks_l + (kb * 32 + perm_row(l32)) * C::KLD + kstep * 16 + hi * 8);
#pragma unroll
            for (int qb = 0; qb < C::QB; ++qb)
              s[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][kstep], s[qb][kb], 0, 0, 0);
          }
        }

        if (wcls == kPartial) {
          const int nvalid = p.Sk - cur * C::BN;
          const MaskSpec ms{p.causal, p.window, p.q_seg != nullptr};
#pragma unroll
          for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              // registers 4jj..4jj+3 hold 4 consecutive keys
              const int kk0 = kb * 32 + key_of_reg(4 * jj, hi);
              const i32x4 kp4 = *reinterpret_cast<const i32x4*>(kpos_l + kk0);
              const i32x4 kg4 = *reinterpret_cast<const i32x4*>(kseg_l + kk0);
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const bool valid = kk0 + i < nvalid;
#pragma unroll
                for (int qb = 0; qb < C::QB; ++qb) {
                  const bool vis = valid && pair_visible(ms, qp[qb], kp4[i], qs[qb], kg4[i]);
                  if (!vis) s[qb][kb][4 * jj + i] = -INFINITY;
                }
              }
            }
        }

        // online softmax (base 2) and P^T in bf16
#pragma unroll
        for (int qb = 0; qb < C::QB; ++qb) {
          float mx = -INFINITY;
#pragma unroll
          for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
          mx = fmaxf(mx, other_half(mx));
          const float mnew = fmaxf(m[qb], mx * c2);
          const float muse = (mnew == -INFINITY) ? 0.0f : mnew;
          const float alpha = __builtin_amdgcn_exp2f(m[qb] - muse);
          m[qb] = mnew;
          float rs = 0.0f;
#pragma unroll
          for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float pv = __builtin_amdgcn_exp2f(fmaf(s[qb][kb][r], c2, -muse));
              s[qb][kb][r] = pv;
              rs += pv;
            }
          l[qb] = l[qb] * alpha + rs;
#pragma unroll
          for (int db = 0; db < C::DB; ++db) o[qb][db] *= alpha;
        }

        // O^T += V^T P^T
#pragma unroll
        for (int t = 0; t < C::PT; ++t) {
          bf16x8 pf[C::QB];
#pragma unroll
          for (int qb = 0; qb < C::QB; ++qb)
#pragma unroll
            for (int e = 0; e < 8; ++e) pf[qb][e] = static_cast<__bf16>(s[qb][t >> 1][8 * (t & 1) + e]);
#pragma unroll
          for (int db = 0; db < C::DB; ++db) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(vt_l + (db * 32 + l32) * C::VLD + t * 16 + hi * 8);
#pragma unroll
            for (int qb = 0; qb < C::QB; ++qb)
              o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[qb], o[qb][db], 0, 0, 0);
          }
        }
      }

      if (has_next) store_tile<C>(p, b, nxt * C::BN, regs, smem + (buf ^ 1) * C::kStageBytes);
      __syncthreads();
      if (!has_next) break;
      cur = nxt;
      buf ^= 1;
    }
  }

  // ---- epilogue: normalise, store out (bf16) and lse (natural log)
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const float lt = l[qb] + other_half(l[qb]);
    const int row = wq0 + qb * 32 + l32;
    if (row >= p.Sq) continue;
    const bool any = lt > 0.0f;
    const float inv = any ? 1.0f / lt : 0.0f;
    uint16_t* orow = out + ((int64_t(b) * p.Sq + row) * p.Hq + h) * C::D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x16& a = o[qb][db];
        const u32x2 w{pack_bf16x2(a[4 * j] * inv, a[4 * j + 1] * inv),
                      pack_bf16x2(a[4 * j + 2] * inv, a[4 * j + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + db * 32 + 8 * j + 4 * hi) = w;
      }
    if (hi == 0)
      lse[(int64_t(b) * p.Hq + h) * p.Sq + row] = any ? (m[qb] + __log2f(lt)) * kLn2 : -INFINITY;
  }
}

template <class C>
hipError_t launch_cfg(const AttnProblem& p, const void* q, const void* k, const void* v, void* out,
                      float* lse, hipStream_t s) {
  dim3 grid(unsigned((p.Sq + C::kRows - 1) / C::kRows) * unsigned(p.Hq * p.B));
  ProfScope ps(s, kProfFwdMfma);
  hipLaunchKernelGGL(attn_fwd_mfma_kernel<C>, grid, dim3(C::kThreads), 0, s, p,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(out), lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const AttnProblem& p, const void* q, const void* k, const void* v,
                                void* out, float* lse, hipStream_t s) {
  switch (p.D) {
    case 128: return launch_cfg<FwdCfg<128, 1, 4, 64>>(p, q, k, v, out, lse, s);
    case 64: return launch_cfg<FwdCfg<64, 1, 4, 64>>(p, q, k, v, out, lse, s);
    case 32: return launch_cfg<FwdCfg<32, 1, 4, 64>>(p, q, k, v, out, lse, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace cp

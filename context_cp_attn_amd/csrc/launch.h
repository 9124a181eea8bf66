// Kernel launchers behind the C ABI.  Arguments are already validated by api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cp {

// Device-side description of one attention block (see cp_attn_args_t).
struct AttnProblem {
  int B, Sq, Sk, Hq, Hkv, D;
  int causal;
  int q_offset, k_offset;     // used when the position arrays are NULL
  const int* q_pos;           // [Sq] or NULL
  const int* k_pos;           // [Sk] or NULL
  const int* q_seg;           // [B,Sq] or NULL
  const int* k_seg;           // [B,Sk] or NULL
  int window;                 // 0 = none
  float scale;                // softmax scale (natural-log domain)
};

// forward
hipError_t launch_attn_fwd_bf16(const AttnProblem& p, const void* q, const void* k, const void* v,
                                void* out, float* lse, hipStream_t s);
hipError_t launch_attn_fwd_f32(const AttnProblem& p, const float* q, const float* k, const float* v,
                               float* out, float* lse, hipStream_t s);
// the same forward with each query tile's keys split over two workgroups whose
// float32 partials (ws, fwd_split_workspace_bytes) a second kernel combines; used
// when fwd_split_applies (too few query tiles to fill the device twice)
bool fwd_split_applies(const AttnProblem& p);
size_t fwd_split_workspace_bytes(const AttnProblem& p);
hipError_t launch_attn_fwd_split_bf16(const AttnProblem& p, const void* q, const void* k, const void* v,
                                      void* out, float* lse, float* ws, hipStream_t s);
// fused ring step: the block's result merged into acc [B,Sq,Hq,D] / lse_acc in place
hipError_t launch_attn_fwd_merge_bf16(const AttnProblem& p, const void* q, const void* k, const void* v,
                                      float* acc, float* lse_acc, hipStream_t s);
hipError_t launch_attn_fwd_merge_f32(const AttnProblem& p, const float* q, const float* k, const float* v,
                                     float* acc, float* lse_acc, hipStream_t s);

// bf16 head dims without a matrix-core kernel (D <= 128 other than 32, 64, 128):
// the row-per-wavefront kernels with bf16 loads / stores
hipError_t launch_attn_fwd_rowwise_bf16(const AttnProblem& p, const void* q, const void* k, const void* v,
                                        void* out, float* lse, hipStream_t s);
hipError_t launch_attn_fwd_merge_rowwise_bf16(const AttnProblem& p, const void* q, const void* k,
                                              const void* v, float* acc, float* lse_acc, hipStream_t s);
hipError_t launch_attn_bwd_rowwise_bf16(const AttnProblem& p, const void* q, const void* k, const void* v,
                                        const void* out, const float* lse, const void* dout, float* dq,
                                        float* dk, float* dv, int accumulate, float* delta, bool rows_ready,
                                        hipStream_t s);

// compute units of the current device (cached per device; 256 if it cannot be read)
int device_cus();

// backward workspace: delta [B,Hq,Sq] float32, then (bf16 matrix-core path) the
// base-2 lse [B,Hq,Sq] float32 starting bwd_row_plane(rows) floats in, then, where
// bwd_head_split_floats(p) > 0, that many floats of dK / dV partials starting
// 2 * bwd_row_plane(rows) floats in
inline int64_t bwd_row_plane(int64_t rows) { return (rows + 63) / 64 * 64; }
int64_t bwd_head_split_floats(const AttnProblem& p);
// rows_ready: the workspace's row arrays already hold this problem's values (an
// earlier call with the same out, lse and dout); the row pre-pass is skipped
hipError_t launch_attn_bwd_bf16(const AttnProblem& p, const void* q, const void* k, const void* v,
                                const void* out, const float* lse, const void* dout, float* dq,
                                float* dk, float* dv, int accumulate, float* delta, bool rows_ready,
                                hipStream_t s);
hipError_t launch_attn_bwd_f32(const AttnProblem& p, const float* q, const float* k, const float* v,
                               const float* out, const float* lse, const float* dout, float* dq,
                               float* dk, float* dv, int accumulate, float* delta, bool rows_ready,
                               hipStream_t s);

// precondition check of the position / segment arrays; writes a violation bit mask
hipError_t launch_check_args(const int* q_pos, const int* k_pos, const int* q_seg, const int* k_seg, int64_t B,
                             int64_t Sq, int64_t Sk, int* flags, hipStream_t s);

// data movement
hipError_t launch_lse_merge(int64_t B, int64_t S, int64_t H, int64_t D, float* acc, float* lse_acc,
                            const void* blk, const float* lse_blk, int blk_is_bf16, hipStream_t s);
// Ulysses relayout of G independent groups (see cp_relayout_args_t); validated sizes.
struct RelayoutProblem {
  int64_t G, P, B, S, H, D, eb, rep;
  bool inverse;
};
hipError_t launch_relayout(const RelayoutProblem& r, const void* in, void* out, hipStream_t s);
hipError_t launch_pad_rows(const void* in, void* out, int64_t B, int64_t S, int64_t S_out, int64_t row_bytes,
                           uint32_t fill, hipStream_t s);
hipError_t launch_zigzag(const void* in, void* out, int64_t B, int64_t S, int64_t row_bytes,
                         int64_t P, bool inverse, hipStream_t s);
hipError_t launch_striped(const void* in, void* out, int64_t B, int64_t S, int64_t row_bytes, int64_t P,
                          bool inverse, hipStream_t s);

}  // namespace cp

/*
 * cp_attn.h — C ABI of the context-parallel attention hot path on one MI355X (gfx950).
 *
 * Every compute entry point is asynchronous on the caller's HIP stream, allocates no
 * device memory, never synchronizes, and keeps no global state other than a
 * thread-local message describing the last failure (and the optional tracing
 * events of cp_prof_*).  All tensors are caller-owned, contiguous,
 * row-major device buffers; pointers must stay valid until the stream work ends.
 * Failures are reported by status code (never by abort); cp_last_error() gives the
 * detail.  Validation happens on the host before any launch, so an invalid call
 * touches no device memory.
 *
 * Sources of the operations (cited by page title and section):
 *   [H]  handbook "Context parallelism: Ring Attention and Ulysses"
 *   [MP] MaxText PR "Add Packing Support for Context Parallelism (Ring Attention)"
 *   [MU] MaxText PR "Add TPU Ulysses context parallelism"
 *   [HF] transformers PR "[distributed] Context parallel module, with Ulysses"
 */
#ifndef CP_ATTN_H
#define CP_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { CP_DTYPE_BF16 = 0, CP_DTYPE_F32 = 1 } cp_dtype_t;

typedef enum {
  CP_OK = 0,
  CP_ERR_INVALID = 1,      /* a size, shape relation or flag the operation does not admit
                              (also: sizes whose byte count would reach 2^62)            */
  CP_ERR_UNSUPPORTED = 2,  /* valid, but no kernel is compiled for it (head_dim, dtype)   */
  CP_ERR_ALIAS = 3,        /* an output buffer overlaps an input it must not overlap      */
  CP_ERR_HIP = 4           /* the HIP runtime reported an error at launch                 */
} cp_status_t;

/*
 * Problem description of one attention block, following [H] §"Which operations
 * partition directly": attention(q, k, v, causal, q_offset, k_offset) -> (out, lse),
 * with q [Sq, H, D], k/v [Sk, H, D], lse [H, Sq]; extended by a batch dimension,
 * grouped kv heads ([H] §"Ulysses", degree bounded by the kv head count), per-token
 * positions (needed by a zigzag rank's two chunks, [H] §"The zigzag partition"),
 * segment ids for packed documents ([MP] §Description, the segment_pos commit) and a
 * sliding window ([HF] §Tests).
 *
 * Key j is visible to query i iff all of:
 *   causal == 0  or  kpos[j] <= qpos[i]
 *   q_seg == NULL  or  q_seg[b,i] == k_seg[b,j]
 *   window == 0  or  0 <= qpos[i] - kpos[j] < window
 * where qpos[i] = q_pos ? q_pos[i] : q_offset + i (likewise kpos).  The pages name
 * the sliding window without defining it; it is read here as the window of the
 * window most recent keys up to and including the query's own position, so a
 * window implies the causal rule whatever causal says.
 * A query row with no visible key gets out = 0 and lse = -inf.
 */
typedef struct {
  int64_t batch;           /* B  >= 1                                                    */
  int64_t seqlen_q;        /* Sq >= 1                                                    */
  int64_t seqlen_k;        /* Sk >= 1                                                    */
  int64_t heads_q;         /* Hq >= 1, a multiple of heads_kv                            */
  int64_t heads_kv;        /* Hkv >= 1; query head h uses kv head h / (Hq / Hkv)          */
  int64_t head_dim;        /* D in [1, 128] (bf16 32/64/128 on the matrix cores)         */
  int32_t dtype;           /* cp_dtype_t of q, k, v, out, dout                           */
  int32_t causal;          /* 0 or 1                                                     */
  int64_t q_offset;        /* global position of query 0 when q_pos is NULL              */
  int64_t k_offset;        /* global position of key 0 when k_pos is NULL                */
  const int32_t* q_pos;    /* NULL or device [Sq] strictly increasing global positions    */
  const int32_t* k_pos;    /* NULL or device [Sk] strictly increasing global positions    */
  const int32_t* q_seg;    /* NULL or device [B, Sq] non-decreasing segment ids           */
  const int32_t* k_seg;    /* NULL or device [B, Sk]; non-NULL iff q_seg is non-NULL     */
  int64_t window;          /* 0 = no window; > 0 = sliding window width (implies causal) */
  float softmax_scale;     /* 0 -> 1/sqrt(head_dim)                                      */
} cp_attn_args_t;

/*
 * Blockwise attention forward.  q [B,Sq,Hq,D], k/v [B,Sk,Hkv,D] (dtype);
 * out [B,Sq,Hq,D] (dtype); lse [B,Hq,Sq] float32, natural log of the row's
 * sum of exp(scale * q.k) over visible keys.  bf16 inputs with D in {32, 64, 128}
 * are multiplied on the matrix cores (q, k, v, out 16-byte aligned); other D run on
 * row-per-wavefront kernels (element-aligned buffers).  Accumulation is float32;
 * a bf16 out is rounded to nearest even.  CP_ERR_UNSUPPORTED for D > 128, for
 * batch or heads_q above 65535, for one batch of q or of k/v of 2^31 bytes or more,
 * and for batch * heads_q * max(Sq, Sk) >= 2^31 (grid indices are 32-bit).
 * out/lse must not overlap q, k or v (CP_ERR_ALIAS).
 */
cp_status_t cp_attn_fwd(const cp_attn_args_t* args, const void* q, const void* k, const void* v,
                        void* out, float* lse, hipStream_t stream);

/*
 * The same forward with a caller-owned workspace, which lets the library split the
 * keys of every query tile over two workgroups when the problem has too few query
 * tiles (of 128 rows) to fill the current device twice and at least 8192 keys (bf16,
 * head_dim 32/64/128); the two float32 partial
 * results are then merged with the ring-step rule of cp_lse_merge ([H] §"Ring
 * Attention": the merge of two blocks of keys) by a second kernel.  Same results
 * as cp_attn_fwd within the bf16 tolerance (out is rounded once, after the merge).
 * cp_attn_fwd_workspace_size gives the bytes needed for args on the current
 * device (0: no split, workspace may be NULL); the workspace must be 16-byte
 * aligned and must not overlap q, k, v, out or lse (CP_ERR_ALIAS), otherwise as
 * cp_attn_fwd.
 */
size_t cp_attn_fwd_workspace_size(const cp_attn_args_t* args);
cp_status_t cp_attn_fwd_ws(const cp_attn_args_t* args, const void* q, const void* k, const void* v,
                           void* out, float* lse, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * Fused ring step ([H] §"Ring Attention": each step's block attention folded into
 * the running result; the merge of cp_lse_merge moved into the attention epilogue).
 * Computes the attention of q against k/v exactly as cp_attn_fwd, but instead of
 * writing the block's out/lse it merges them, in float32 (the block output is not
 * rounded to dtype), into the caller's running result in place:
 *   lse' = log(e^lse_acc + e^lse_blk)
 *   acc' = acc * e^(lse_acc - lse') + out_blk * e^(lse_blk - lse')
 * with the -inf rules of cp_lse_merge (a row with no visible key in this block has
 * weight 0).  out_acc [B,Sq,Hq,D] float32 (16-byte aligned on the matrix-core path) and lse_acc [B,Hq,Sq]
 * float32 are read and written; start a ring with out_acc = 0, lse_acc = -inf (rows
 * whose query tile sees no key of the block may be left untouched, which is the
 * same result for every state such a ring reaches).
 * out_acc/lse_acc must not overlap q, k, v or each other (CP_ERR_ALIAS).
 */
cp_status_t cp_attn_fwd_merge(const cp_attn_args_t* args, const void* q, const void* k, const void* v,
                              float* out_acc, float* lse_acc, hipStream_t stream);

/* Workspace bytes cp_attn_bwd needs for args on the current device (the backward
   of [HF] §Tests, stated with cp_attn_bwd below): two float32
   arrays of the rows [B,Hq,Sq], the per-row dO.O sums and the rows' lse in base 2;
   for bf16 problems (D 32, 64, 128) with grouped query heads whose backward grid is
   under 16 workgroups per compute unit, also float32 dK and dV partials
   [2][B,Sk,Hkv,D] (the key side's work is then split over two halves of each
   group's query heads and the halves are added in a fixed order). */
size_t cp_attn_bwd_workspace_size(const cp_attn_args_t* args);

/*
 * Blockwise attention backward: the gradient of sum(dout * out) with respect to q,
 * k and v for this block, given the rows' FINAL out and lse (for a ring step these are
 * the merged values over all blocks, so the per-block gradients add up to the full
 * gradient).  The pages ask for the backward next to the forward ([HF] §Tests:
 * forward and backward checked against plain attention) without stating it; this is
 * the textbook gradient of softmax attention, P = exp(scale*q.k - lse) on visible
 * pairs, Delta = rowsum(dout * out), dv = P^T dout, dS = P * (dout v^T - Delta),
 * dq = scale dS k, dk = scale dS^T q, and applying it per block with the final out
 * and lse is this library's reading of a ring backward.  dq [B,Sq,Hq,D], dk/dv [B,Sk,Hkv,D] float32; dk/dv are summed over the
 * query heads of each kv group.  accumulate = 1 adds into dq/dk/dv, 0 overwrites
 * them.  workspace: device memory of at least cp_attn_bwd_workspace_size(args)
 * bytes, 16-byte aligned, owned by the caller.  The result is deterministic (no
 * atomics).
 */
cp_status_t cp_attn_bwd(const cp_attn_args_t* args, const void* q, const void* k, const void* v,
                        const void* out, const float* lse, const void* dout,
                        float* dq, float* dk, float* dv, int32_t accumulate,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * cp_attn_bwd for the later steps of a ring backward (in the blockwise reading of
 * cp_attn_bwd, every step's block gradient uses the rows' same final out and lse;
 * the pages do not state a ring backward): the per-row values
 * the backward derives from out, lse and dout (the dO.O sums and the base-2 lse) are
 * taken from the workspace as an earlier cp_attn_bwd or cp_attn_bwd_rows_ready call
 * left them, instead of being recomputed.  The caller guarantees that the workspace
 * was last used by such a call, ordered before this one, with the same out, lse and
 * dout (same contents) and the same batch, heads_q, seqlen_q and dtype / head_dim;
 * the library cannot check this.  Arguments and errors as cp_attn_bwd.
 */
cp_status_t cp_attn_bwd_rows_ready(const cp_attn_args_t* args, const void* q, const void* k, const void* v,
                                   const void* out, const float* lse, const void* dout,
                                   float* dq, float* dk, float* dv, int32_t accumulate,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Allocation-free cp_attn_bwd, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same backward and kernels, with the workspace taken from a
 * scratch array that the library holds on every device it runs on until the
 * process ends (CP_ATTN_BWD_NOALLOC_MAX_BYTES per device), so the caller passes
 * inputs and outputs only.  Arguments, results and errors as cp_attn_bwd, plus
 * CP_ERR_UNSUPPORTED when cp_attn_bwd_workspace_size(args) exceeds that size.
 * Every call on a device shares that device's scratch, which keeps the last call's
 * contents: calls that can overlap in time on one device (other streams, other
 * host threads) race and must not be issued; calls ordered on one stream are safe.
 * No part of the scratch has to start at zero.  Nothing is allocated or freed.
 */
#define CP_ATTN_BWD_NOALLOC_MAX_BYTES (32u << 20)
cp_status_t cp_attn_bwd_noalloc(const cp_attn_args_t* args, const void* q, const void* k, const void* v,
                                const void* out, const float* lse, const void* dout,
                                float* dq, float* dk, float* dv, int32_t accumulate, hipStream_t stream);

/*
 * Debug check of the preconditions on args' arrays that the attention kernels rely
 * on but the host cannot see: q_pos / k_pos strictly increasing and >= 0 (the block
 * positions of [H] §"Ring Attention"), q_seg / k_seg non-decreasing along each of the
 * B rows (the per-token segment ids of [MP]).  Two small kernels on `stream` clear
 * *flags and set bit 0 (q_pos), 1 (k_pos), 2 (q_seg) or 3 (k_seg) for each array
 * that breaks its rule; NULL arrays are skipped, 0 means all hold.  flags: caller-
 * owned device int32, 4-byte aligned.  Asynchronous; read flags after the stream
 * work ends.  CP_ERR_INVALID for a NULL args/flags or invalid sizes.
 */
cp_status_t cp_attn_check_args(const cp_attn_args_t* args, int32_t* flags, hipStream_t stream);

/*
 * Ring-step merge, in place ([H] self-test answers and §"Ring Attention"):
 *   lse' = log(e^lse_acc + e^lse_blk)
 *   acc' = acc * e^(lse_acc - lse') + blk * e^(lse_blk - lse')
 * A part whose lse is -inf has weight 0 (both -inf gives acc' = 0, lse' = -inf).
 * out_acc [B,S,H,D] float32 (read and written), lse_acc [B,H,S] float32 (read and
 * written), out_blk [B,S,H,D] of blk_dtype, lse_blk [B,H,S] float32.  The two
 * written buffers (out_acc, lse_acc) may overlap neither each other nor either
 * read-only buffer (out_blk, lse_blk): CP_ERR_ALIAS.
 * CP_ERR_UNSUPPORTED when out_acc holds 32 GiB or more (B*S*H*D/4 >= 2^31 - 512
 * 16-byte vectors: the kernel indexes with 32-bit integers).
 */
cp_status_t cp_lse_merge(int64_t batch, int64_t seqlen, int64_t heads, int64_t head_dim,
                         float* out_acc, float* lse_acc, const void* out_blk,
                         const float* lse_blk, int32_t blk_dtype, hipStream_t stream);

/*
 * Ulysses sequence -> head relayout of all P ranks at once, as one local permute
 * ([H] §"Ulysses", seq_to_head; [MU] the forward all-to-all):
 *   in  [P][B][S/P][H][D]   (rank s holds sequence slice s, all heads)
 *   out [P][B][S][H/P][D]   (rank p holds the whole sequence, heads [p*H/P, (p+1)*H/P))
 *   out[p][b][s*(S/P)+i][hh][d] = in[s][b][i][p*(H/P)+hh][d]
 * seqlen is the full S; S % P == 0 and H % P == 0 (applied to k/v this is the
 * degree limit P <= H_kv) else CP_ERR_INVALID.  elem_bytes in {2, 4}.  Bit-exact.
 * in and out must not overlap (CP_ERR_ALIAS).
 */
cp_status_t cp_ulysses_relayout(const void* in, void* out, int64_t P, int64_t batch,
                                int64_t seqlen, int64_t heads, int64_t head_dim,
                                int64_t elem_bytes, hipStream_t stream);

/* Exact inverse of cp_ulysses_relayout ([H] §"Ulysses", head_to_seq):
 *   in [P][B][S][H/P][D] -> out [P][B][S/P][H][D].  Same arguments and errors. */
cp_status_t cp_ulysses_relayout_inv(const void* in, void* out, int64_t P, int64_t batch,
                                    int64_t seqlen, int64_t heads, int64_t head_dim,
                                    int64_t elem_bytes, hipStream_t stream);

/*
 * General Ulysses relayout ([H] §"Ulysses" and §Exercises: a degree above the kv
 * head count by replicating each kv head by group before the exchange, or Ulysses
 * within groups combined with ring attention across them, as in USP; [MU] names
 * the Ulysses x ring hybrid).  G independent groups stacked outermost (the ring
 * groups of USP; 1 for plain Ulysses); within a group P ranks, seqlen = the group's
 * whole sequence S, heads = H of the sequence-sharded tensor, each replicated rep
 * times (head j of the replicated set is head j / rep; H' = H*rep).
 *   inverse = 0: in [G][P][B][S/P][H][D] -> out [G][P][B][S][H'/P][D]
 *     out[g][p][b][s*(S/P)+i][hh][d] = in[g][s][b][i][(p*H'/P + hh) / rep][d]
 *   inverse = 1: in [G][P][B][S][H'/P][D] -> out [G][P][B][S/P][H][D]: the exact
 *     inverse for rep = 1; for rep > 1 each head receives the sum of its rep copies
 *     (copies t = 0..rep-1 added in that order; the gradient of the replication),
 *     float32 only (elem_bytes 4).
 * S % P == 0 and (H*rep) % P == 0, elem_bytes in {2, 4}, G <= 65535, else
 * CP_ERR_INVALID / CP_ERR_UNSUPPORTED.  Bit-exact except for the sums.  in and out
 * must not overlap (CP_ERR_ALIAS).  cp_ulysses_relayout(_inv) are G = 1, rep = 1.
 */
typedef struct {
  int64_t groups;      /* G >= 1                                                   */
  int64_t P;           /* Ulysses degree within a group                            */
  int64_t batch;       /* B >= 1                                                   */
  int64_t seqlen;      /* S: the sequence one group covers                         */
  int64_t heads;       /* H: heads of the sequence-sharded tensor                  */
  int64_t head_dim;    /* D                                                        */
  int64_t elem_bytes;  /* 2 or 4                                                   */
  int64_t rep;         /* >= 1: copies of every head                               */
  int32_t inverse;     /* 0: sequence -> heads; 1: heads -> sequence               */
} cp_relayout_args_t;

cp_status_t cp_ulysses_relayout_ex(const cp_relayout_args_t* args, const void* in, void* out,
                                   hipStream_t stream);

/*
 * Causal load-balancing reorder of whole token rows.  in/out [B][S][row_bytes]; the
 * output is the P ranks' shares in rank order, so a contiguous P-way split gives
 * rank r its share.  inverse = 1 undoes it.  Bit-exact.
 *   strategy 0 = DualChunkSwap ([H] §"The zigzag partition"; [MP] strategy 0): the
 *     sequence is cut into 2P chunks of S/(2P) rows and rank r gets chunk r then
 *     chunk 2P-1-r.  S % (2P) == 0 else CP_ERR_INVALID.
 *   strategy 1 = Striped ([MP] strategy 1): token t goes to rank t mod P, so rank r
 *     gets rows r, r+P, r+2P, ...  S % P == 0 else CP_ERR_INVALID.
 * Another strategy -> CP_ERR_INVALID.  in and out must not overlap (CP_ERR_ALIAS).
 */
cp_status_t cp_zigzag_reorder(const void* in, void* out, int64_t batch, int64_t seqlen,
                              int64_t row_bytes, int64_t P, int32_t strategy, int32_t inverse,
                              hipStream_t stream);

/*
 * Sequence padding to a multiple of the context-parallel degree ([HF] "What this
 * PR brings": sequences padded at their end before the masks are built; embeddings
 * zeros, positions continuing).  in [B][seqlen][row_bytes] -> out
 * [B][seqlen_out][row_bytes]: rows t < min(seqlen, seqlen_out) copied, rows
 * t >= seqlen filled with the 32-bit word `fill` repeated (0 for data; a fresh
 * segment id for int32 segment ids, so no real query sees a pad key);
 * seqlen_out < seqlen truncates (removes the padding of an output).  A non-zero
 * fill needs row_bytes % 4 == 0 (CP_ERR_INVALID).  Bit-exact.  in and out must
 * not overlap (CP_ERR_ALIAS).
 */
cp_status_t cp_pad_rows(const void* in, void* out, int64_t batch, int64_t seqlen, int64_t seqlen_out,
                        int64_t row_bytes, uint32_t fill, hipStream_t stream);

/*
 * Kernel tracing with HIP events (a measurement aid, off by default).  While
 * enabled, every kernel launch of the library is bracketed by two events recorded
 * on its stream; the events are created by the library on first use and reused.
 * cp_prof_read() waits for all events recorded so far, folds them into per-kernel
 * totals and returns the total milliseconds and launch count of one kernel id in
 * [0, cp_prof_kernel_count()) (CP_ERR_INVALID for another id or NULL outputs,
 * CP_ERR_HIP if an event query fails).  cp_prof_reset() waits for and discards
 * everything recorded.  Not for concurrent use from several host threads.
 */
void        cp_prof_enable(int32_t on);
void        cp_prof_reset(void);
int32_t     cp_prof_kernel_count(void);
const char* cp_prof_kernel_name(int32_t kernel);   /* "" for an unknown id */
cp_status_t cp_prof_read(int32_t kernel, double* total_ms, int64_t* launches);

/* Static name of a status code. */
const char* cp_status_string(cp_status_t status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* cp_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* CP_ATTN_H */

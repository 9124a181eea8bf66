// C ABI of libcp_attn: argument validation, error reporting and kernel dispatch.
// Every check runs on the host before any launch, so a rejected call touches no
// device memory.  Nothing here allocates or synchronizes.
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <initializer_list>
#include <mutex>
#include <string>

#include "cp_attn.h"
#include "launch.h"


namespace {

thread_local std::string g_last_error;

cp_status_t fail(cp_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

cp_status_t ok() {
  g_last_error.clear();
  return CP_OK;
}

cp_status_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(CP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool overlaps(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  if (!a || !b || abytes <= 0 || bbytes <= 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + uintptr_t(bbytes) && b0 < a0 + uintptr_t(abytes);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// a non-NULL, aligned stand-in for tensor pointers where only the sizes are checked
const void* const kProbe = reinterpret_cast<const void*>(uintptr_t(1) << 12);

// True when the product of the (positive) sizes is below 2^62: a byte count that a
// buffer can have.  Checked before any other arithmetic on caller sizes, so that
// none of it can overflow int64.
bool sizes_fit(std::initializer_list<int64_t> xs) {
  int64_t p = 1;
  for (const int64_t x : xs)
    if (__builtin_mul_overflow(p, x, &p)) return false;
  return p < (int64_t(1) << 62);
}

int64_t dtype_bytes(int32_t dt) { return dt == CP_DTYPE_BF16 ? 2 : 4; }

// bf16 problems with these head dims run on the matrix-core kernels; other bf16
// head dims up to 128 run on the row-per-wavefront kernels.
bool mfma_path(const cp_attn_args_t* a) {
  return a->dtype == CP_DTYPE_BF16 && (a->head_dim == 32 || a->head_dim == 64 || a->head_dim == 128);
}

// Shared validation of cp_attn_fwd / cp_attn_bwd arguments; fills the device problem.
cp_status_t check_attn(const cp_attn_args_t* a, const void* q, const void* k, const void* v,
                       cp::AttnProblem* p) {
  if (!a) return fail(CP_ERR_INVALID, "args is NULL");
  if (!q || !k || !v) return fail(CP_ERR_INVALID, "q, k and v must be non-NULL");
  if (a->batch < 1 || a->seqlen_q < 1 || a->seqlen_k < 1 || a->heads_q < 1 || a->heads_kv < 1 ||
      a->head_dim < 1)
    return fail(CP_ERR_INVALID,
                "sizes must be >= 1 (batch=%lld seqlen_q=%lld seqlen_k=%lld heads_q=%lld "
                "heads_kv=%lld head_dim=%lld)",
                (long long)a->batch, (long long)a->seqlen_q, (long long)a->seqlen_k,
                (long long)a->heads_q, (long long)a->heads_kv, (long long)a->head_dim);
  if (a->heads_q % a->heads_kv)
    return fail(CP_ERR_INVALID, "heads_q %lld is not a multiple of heads_kv %lld",
                (long long)a->heads_q, (long long)a->heads_kv);
  if (a->dtype != CP_DTYPE_BF16 && a->dtype != CP_DTYPE_F32)
    return fail(CP_ERR_INVALID, "unknown dtype %d", (int)a->dtype);
  if (a->causal != 0 && a->causal != 1) return fail(CP_ERR_INVALID, "causal must be 0 or 1");
  if (a->window < 0 || a->window > INT_MAX)
    return fail(CP_ERR_INVALID, "window %lld must be in [0, 2^31)", (long long)a->window);
  if ((a->q_seg == nullptr) != (a->k_seg == nullptr))
    return fail(CP_ERR_INVALID, "q_seg and k_seg must both be given or both be NULL");
  if (!(a->softmax_scale >= 0.0f) || std::isinf(a->softmax_scale))
    return fail(CP_ERR_INVALID, "softmax_scale must be finite and >= 0 (0 selects 1/sqrt(D))");
  if (a->seqlen_q > INT_MAX || a->seqlen_k > INT_MAX || a->batch > 65535 || a->heads_q > 65535)
    return fail(CP_ERR_UNSUPPORTED, "sizes beyond the launch grid (batch, heads_q <= 65535; seqlen < 2^31)");
  if (a->head_dim > 128)
    return fail(CP_ERR_UNSUPPORTED, "attention is built for head_dim <= 128 (got %lld)",
                (long long)a->head_dim);
  {
    // grid sizes and (batch, head, tile) indices are 32-bit: batch * heads_q * seqlen
    // (the longer of the two) rows at most 2^31 - 1; batch * heads_q < 2^32 here, so
    // the test divides instead of multiplying
    const int64_t bh = a->batch * a->heads_q;
    const int64_t s = a->seqlen_q > a->seqlen_k ? a->seqlen_q : a->seqlen_k;
    if (bh > INT_MAX / s)
      return fail(CP_ERR_UNSUPPORTED, "batch * heads_q * seqlen = %lld * %lld * %lld rows: 2^31 or more",
                  (long long)a->batch, (long long)a->heads_q, (long long)s);
  }
  {
    // the matrix-core kernels address one batch plane of a tensor with 32-bit offsets
    const int64_t eb = a->dtype == CP_DTYPE_BF16 ? 2 : 4;
    if (a->seqlen_q * a->heads_q * a->head_dim * eb >= (int64_t(1) << 31) ||
        a->seqlen_k * a->heads_kv * a->head_dim * eb >= (int64_t(1) << 31))
      return fail(CP_ERR_UNSUPPORTED, "one batch of q or k/v exceeds 2^31 bytes");
  }
  // (seqlen <= INT_MAX here, so the bounds are formed without overflow)
  if (!a->q_pos && (a->q_offset < 0 || a->q_offset > INT_MAX - a->seqlen_q))
    return fail(CP_ERR_INVALID, "q_offset %lld: positions must lie in [0, 2^31)", (long long)a->q_offset);
  if (!a->k_pos && (a->k_offset < 0 || a->k_offset > INT_MAX - a->seqlen_k))
    return fail(CP_ERR_INVALID, "k_offset %lld: positions must lie in [0, 2^31)", (long long)a->k_offset);
  if (mfma_path(a)) {
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
      return fail(CP_ERR_INVALID, "bf16 q, k, v must be 16-byte aligned");
  } else if (!aligned(q, dtype_bytes(a->dtype)) || !aligned(k, dtype_bytes(a->dtype)) ||
             !aligned(v, dtype_bytes(a->dtype))) {
    return fail(CP_ERR_INVALID, "q, k, v must be aligned to their element size");
  }
  p->B = int(a->batch);
  p->Sq = int(a->seqlen_q);
  p->Sk = int(a->seqlen_k);
  p->Hq = int(a->heads_q);
  p->Hkv = int(a->heads_kv);
  p->D = int(a->head_dim);
  // the window bounds qpos - kpos on both sides (0 <= qpos - kpos < window), so a
  // window carries the causal rule with it
  p->causal = (a->causal || a->window) ? 1 : 0;
  p->q_offset = int(a->q_pos ? 0 : a->q_offset);
  p->k_offset = int(a->k_pos ? 0 : a->k_offset);
  p->q_pos = a->q_pos;
  p->k_pos = a->k_pos;
  p->q_seg = a->q_seg;
  p->k_seg = a->k_seg;
  p->window = int(a->window);
  p->scale = a->softmax_scale > 0.0f ? a->softmax_scale : 1.0f / std::sqrt(float(a->head_dim));
  return CP_OK;
}

}  // namespace

extern "C" {

const char* cp_status_string(cp_status_t st) {
  switch (st) {
    case CP_OK: return "CP_OK";
    case CP_ERR_INVALID: return "CP_ERR_INVALID";
    case CP_ERR_UNSUPPORTED: return "CP_ERR_UNSUPPORTED";
    case CP_ERR_ALIAS: return "CP_ERR_ALIAS";
    case CP_ERR_HIP: return "CP_ERR_HIP";
  }
  return "CP_ERR_UNKNOWN";
}

const char* cp_last_error(void) { return g_last_error.c_str(); }

namespace {

// Workspace bytes of the split forward for args, 0 where it does not apply (the
// problem is invalid, not on the matrix-core path, or large enough to fill the
// current device with whole query tiles).
size_t fwd_workspace_bytes(const cp_attn_args_t* a) {
  if (!a || !mfma_path(a)) return 0;
  // the call's own validation (on stand-in pointers), without touching the caller's
  // last error
  cp::AttnProblem p;
  const std::string saved = g_last_error;
  const bool valid = check_attn(a, kProbe, kProbe, kProbe, &p) == CP_OK;
  g_last_error = saved;
  if (!valid || !cp::fwd_split_applies(p)) return 0;
  return (cp::fwd_split_workspace_bytes(p) + 255) & ~size_t(255);
}

cp_status_t fwd_impl(const cp_attn_args_t* a, const void* q, const void* k, const void* v, void* out, float* lse,
                     void* workspace, size_t workspace_bytes, bool with_ws, hipStream_t stream) {
  cp::AttnProblem p;
  cp_status_t st = check_attn(a, q, k, v, &p);
  if (st != CP_OK) return st;
  if (!out || !lse) return fail(CP_ERR_INVALID, "out and lse must be non-NULL");
  const size_t need = with_ws ? fwd_workspace_bytes(a) : 0;
  if (need) {
    if (!workspace || workspace_bytes < need)
      return fail(CP_ERR_INVALID, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
    if (!aligned(workspace, 16)) return fail(CP_ERR_INVALID, "workspace must be 16-byte aligned");
  }
  const int64_t eb = dtype_bytes(a->dtype);
  const int64_t qbytes = a->batch * a->seqlen_q * a->heads_q * a->head_dim * eb;
  const int64_t kbytes = a->batch * a->seqlen_k * a->heads_kv * a->head_dim * eb;
  const int64_t lbytes = a->batch * a->heads_q * a->seqlen_q * 4;
  for (const void* in : {q, k, v}) {
    const int64_t ib = (in == q) ? qbytes : kbytes;
    if (overlaps(out, qbytes, in, ib) || overlaps(lse, lbytes, in, ib))
      return fail(CP_ERR_ALIAS, "out/lse overlap an input");
  }
  if (overlaps(out, qbytes, lse, lbytes)) return fail(CP_ERR_ALIAS, "out overlaps lse");
  if (need) {
    const void* bufs[] = {q, k, v, out, lse};
    const int64_t bytes[] = {qbytes, kbytes, kbytes, qbytes, lbytes};
    for (int i = 0; i < 5; ++i)
      if (overlaps(workspace, int64_t(need), bufs[i], bytes[i]))
        return fail(CP_ERR_ALIAS, "the workspace overlaps an input or output");
  }
  hipError_t e;
  if (!aligned(out, mfma_path(a) ? 16 : eb) || !aligned(lse, 4))
    return fail(CP_ERR_INVALID, "out or lse is misaligned");
  if (need) {
    e = cp::launch_attn_fwd_split_bf16(p, q, k, v, out, lse, static_cast<float*>(workspace), stream);
  } else if (mfma_path(a)) {
    e = cp::launch_attn_fwd_bf16(p, q, k, v, out, lse, stream);
  } else if (a->dtype == CP_DTYPE_BF16) {
    e = cp::launch_attn_fwd_rowwise_bf16(p, q, k, v, out, lse, stream);
  } else {
    e = cp::launch_attn_fwd_f32(p, static_cast<const float*>(q), static_cast<const float*>(k),
                                static_cast<const float*>(v), static_cast<float*>(out), lse, stream);
  }
  return hip_status(e, "cp_attn_fwd launch");
}

}  // namespace

cp_status_t cp_attn_fwd(const cp_attn_args_t* a, const void* q, const void* k, const void* v, void* out,
                        float* lse, hipStream_t stream) {
  return fwd_impl(a, q, k, v, out, lse, nullptr, 0, false, stream);
}

size_t cp_attn_fwd_workspace_size(const cp_attn_args_t* a) { return fwd_workspace_bytes(a); }

cp_status_t cp_attn_fwd_ws(const cp_attn_args_t* a, const void* q, const void* k, const void* v, void* out,
                           float* lse, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return fwd_impl(a, q, k, v, out, lse, workspace, workspace_bytes, true, stream);
}

cp_status_t cp_attn_fwd_merge(const cp_attn_args_t* a, const void* q, const void* k, const void* v,
                              float* out_acc, float* lse_acc, hipStream_t stream) {
  cp::AttnProblem p;
  cp_status_t st = check_attn(a, q, k, v, &p);
  if (st != CP_OK) return st;
  if (!out_acc || !lse_acc) return fail(CP_ERR_INVALID, "out_acc and lse_acc must be non-NULL");
  if (!aligned(out_acc, mfma_path(a) ? 16 : 4)) return fail(CP_ERR_INVALID, "out_acc is misaligned");
  const int64_t eb = dtype_bytes(a->dtype);
  const int64_t qbytes = a->batch * a->seqlen_q * a->heads_q * a->head_dim * eb;
  const int64_t kbytes = a->batch * a->seqlen_k * a->heads_kv * a->head_dim * eb;
  const int64_t abytes = a->batch * a->seqlen_q * a->heads_q * a->head_dim * 4;
  const int64_t lbytes = a->batch * a->heads_q * a->seqlen_q * 4;
  for (const void* in : {q, k, v}) {
    const int64_t ib = (in == q) ? qbytes : kbytes;
    if (overlaps(out_acc, abytes, in, ib) || overlaps(lse_acc, lbytes, in, ib))
      return fail(CP_ERR_ALIAS, "out_acc/lse_acc overlap an input");
  }
  if (overlaps(out_acc, abytes, lse_acc, lbytes)) return fail(CP_ERR_ALIAS, "out_acc overlaps lse_acc");
  hipError_t e;
  if (!aligned(lse_acc, 4)) return fail(CP_ERR_INVALID, "lse_acc is misaligned");
  if (mfma_path(a)) {
    e = cp::launch_attn_fwd_merge_bf16(p, q, k, v, out_acc, lse_acc, stream);
  } else if (a->dtype == CP_DTYPE_BF16) {
    e = cp::launch_attn_fwd_merge_rowwise_bf16(p, q, k, v, out_acc, lse_acc, stream);
  } else {
    e = cp::launch_attn_fwd_merge_f32(p, static_cast<const float*>(q), static_cast<const float*>(k),
                                      static_cast<const float*>(v), out_acc, lse_acc, stream);
  }
  return hip_status(e, "cp_attn_fwd_merge launch");
}

cp_status_t cp_attn_check_args(const cp_attn_args_t* a, int32_t* flags, hipStream_t stream) {
  if (!a) return fail(CP_ERR_INVALID, "args is NULL");
  if (!flags || !aligned(flags, 4)) return fail(CP_ERR_INVALID, "flags must be a non-NULL, 4-byte aligned int32");
  if (a->batch < 1 || a->seqlen_q < 1 || a->seqlen_k < 1 || a->seqlen_q > INT_MAX || a->seqlen_k > INT_MAX ||
      a->batch > INT_MAX)
    return fail(CP_ERR_INVALID, "sizes must be >= 1 and seqlens < 2^31");
  if ((a->q_seg == nullptr) != (a->k_seg == nullptr))
    return fail(CP_ERR_INVALID, "q_seg and k_seg must both be given or both be NULL");
  const hipError_t e = cp::launch_check_args(a->q_pos, a->k_pos, a->q_seg, a->k_seg, a->batch, a->seqlen_q,
                                             a->seqlen_k, flags, stream);
  return hip_status(e, "cp_attn_check_args launch");
}

size_t cp_attn_bwd_workspace_size(const cp_attn_args_t* a) {
  if (!a || a->batch < 1 || a->heads_q < 1 || a->seqlen_q < 1 || !sizes_fit({a->batch, a->heads_q, a->seqlen_q, 8}))
    return 0;
  // two row arrays: delta and the base-2 lse
  const int64_t rows = a->batch * a->heads_q * a->seqlen_q;
  int64_t floats = 2 * cp::bwd_row_plane(rows);
  // then the dK / dV partials of a head-split backward (windowed or segmented
  // problems with grouped heads on small grids), for arguments the call accepts
  cp::AttnProblem p;
  const std::string saved = g_last_error;
  if (mfma_path(a) && check_attn(a, kProbe, kProbe, kProbe, &p) == CP_OK) floats += cp::bwd_head_split_floats(p);
  g_last_error = saved;
  return size_t(floats) * sizeof(float);
}

}  // extern "C"

namespace {

cp_status_t bwd_impl(const cp_attn_args_t* a, const void* q, const void* k, const void* v, const void* out,
                     const float* lse, const void* dout, float* dq, float* dk, float* dv, int32_t accumulate,
                     void* workspace, size_t workspace_bytes, bool rows_ready, hipStream_t stream) {
  cp::AttnProblem p;
  cp_status_t st = check_attn(a, q, k, v, &p);
  if (st != CP_OK) return st;
  if (!out || !lse || !dout || !dq || !dk || !dv)
    return fail(CP_ERR_INVALID, "out, lse, dout, dq, dk, dv must be non-NULL");
  if (accumulate != 0 && accumulate != 1) return fail(CP_ERR_INVALID, "accumulate must be 0 or 1");
  const size_t need = cp_attn_bwd_workspace_size(a);
  if (!workspace || workspace_bytes < need)
    return fail(CP_ERR_INVALID, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
  if (!aligned(workspace, 16)) return fail(CP_ERR_INVALID, "workspace must be 16-byte aligned");
  const int64_t eb = dtype_bytes(a->dtype);
  const int64_t qbytes = a->batch * a->seqlen_q * a->heads_q * a->head_dim * eb;
  const int64_t kbytes = a->batch * a->seqlen_k * a->heads_kv * a->head_dim * eb;
  const int64_t lbytes = a->batch * a->heads_q * a->seqlen_q * 4;
  const int64_t dqb = a->batch * a->seqlen_q * a->heads_q * a->head_dim * 4;
  const int64_t dkb = a->batch * a->seqlen_k * a->heads_kv * a->head_dim * 4;
  const void* ins[] = {q, k, v, out, lse, dout, workspace};
  const int64_t inb[] = {qbytes, kbytes, kbytes, qbytes, lbytes, qbytes, int64_t(need)};
  const void* outs[] = {dq, dk, dv};
  const int64_t outb[] = {dqb, dkb, dkb};
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 7; ++i)
      if (overlaps(outs[o], outb[o], ins[i], inb[i]))
        return fail(CP_ERR_ALIAS, "a gradient buffer overlaps an input or the workspace");
    for (int o2 = o + 1; o2 < 3; ++o2)
      if (overlaps(outs[o], outb[o], outs[o2], outb[o2]))
        return fail(CP_ERR_ALIAS, "gradient buffers overlap each other");
  }
  float* delta = static_cast<float*>(workspace);
  hipError_t e;
  if (!aligned(out, mfma_path(a) ? 16 : eb) || !aligned(dout, mfma_path(a) ? 16 : eb))
    return fail(CP_ERR_INVALID, "out or dout is misaligned");
  if (!aligned(lse, 4) || !aligned(dq, 4) || !aligned(dk, 4) || !aligned(dv, 4))
    return fail(CP_ERR_INVALID, "lse or a gradient buffer is misaligned");
  if (mfma_path(a)) {
    e = cp::launch_attn_bwd_bf16(p, q, k, v, out, lse, dout, dq, dk, dv, accumulate, delta, rows_ready, stream);
  } else if (a->dtype == CP_DTYPE_BF16) {
    e = cp::launch_attn_bwd_rowwise_bf16(p, q, k, v, out, lse, dout, dq, dk, dv, accumulate, delta, rows_ready,
                                         stream);
  } else {
    e = cp::launch_attn_bwd_f32(p, static_cast<const float*>(q), static_cast<const float*>(k),
                                static_cast<const float*>(v), static_cast<const float*>(out), lse,
                                static_cast<const float*>(dout), dq, dk, dv, accumulate, delta, rows_ready, stream);
  }
  return hip_status(e, "cp_attn_bwd launch");
}

}  // namespace

extern "C" {

cp_status_t cp_attn_bwd(const cp_attn_args_t* a, const void* q, const void* k, const void* v,
                        const void* out, const float* lse, const void* dout, float* dq, float* dk,
                        float* dv, int32_t accumulate, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  return bwd_impl(a, q, k, v, out, lse, dout, dq, dk, dv, accumulate, workspace, workspace_bytes, false, stream);
}

cp_status_t cp_attn_bwd_rows_ready(const cp_attn_args_t* a, const void* q, const void* k, const void* v,
                                   const void* out, const float* lse, const void* dout, float* dq, float* dk,
                                   float* dv, int32_t accumulate, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  return bwd_impl(a, q, k, v, out, lse, dout, dq, dk, dv, accumulate, workspace, workspace_bytes, true, stream);
}

}  // extern "C"

// ---- allocation-free backward ---------------------------------------------------
// The scratch memory of cp_attn_bwd_noalloc: a file-scope device array, one copy per
// device, alive until the process ends.  Host code never passes the array's name to
// a kernel (on the host it names a stand-in, not device memory): the device address
// of each device's copy is looked up once per device and kept.
static __device__ __align__(256) uint8_t scratch[CP_ATTN_BWD_NOALLOC_MAX_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices];

// Device address of the current device's copy of scratch (looked up on the first
// call on that device, with it current).
cp_status_t scratch_of_current_device(void** addr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(CP_ERR_UNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p || !aligned(p, 256)) return fail(CP_ERR_HIP, "hipGetSymbolAddress(scratch) gave an unusable address");
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return CP_OK;
}

}  // namespace

extern "C" {

cp_status_t cp_attn_bwd_noalloc(const cp_attn_args_t* a, const void* q, const void* k, const void* v,
                                const void* out, const float* lse, const void* dout, float* dq, float* dk,
                                float* dv, int32_t accumulate, hipStream_t stream) {
  cp::AttnProblem p;
  cp_status_t st = check_attn(a, q, k, v, &p);
  if (st != CP_OK) return st;
  const size_t need = cp_attn_bwd_workspace_size(a);
  if (need > size_t(CP_ATTN_BWD_NOALLOC_MAX_BYTES))
    return fail(CP_ERR_UNSUPPORTED,
                "this backward needs %zu bytes of scratch; the allocation-free entry point holds %zu "
                "(use cp_attn_bwd with a caller-owned workspace)",
                need, size_t(CP_ATTN_BWD_NOALLOC_MAX_BYTES));
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != CP_OK) return st;
  // every kernel of the backward writes the scratch bytes it later reads (row
  // arrays, head-split partials): nothing has to start at zero
  return bwd_impl(a, q, k, v, out, lse, dout, dq, dk, dv, accumulate, ws, size_t(CP_ATTN_BWD_NOALLOC_MAX_BYTES),
                  false, stream);
}

cp_status_t cp_lse_merge(int64_t batch, int64_t seqlen, int64_t heads, int64_t head_dim,
                         float* out_acc, float* lse_acc, const void* out_blk, const float* lse_blk,
                         int32_t blk_dtype, hipStream_t stream) {
  if (batch < 1 || seqlen < 1 || heads < 1 || head_dim < 1)
    return fail(CP_ERR_INVALID, "sizes must be >= 1");
  if (!sizes_fit({batch, seqlen, heads, head_dim, 4}))
    return fail(CP_ERR_INVALID, "sizes describe 2^62 bytes or more");
  if (blk_dtype != CP_DTYPE_BF16 && blk_dtype != CP_DTYPE_F32)
    return fail(CP_ERR_INVALID, "unknown blk_dtype %d", (int)blk_dtype);
  if (head_dim % 4 || 64 % (head_dim / 4))
    return fail(CP_ERR_UNSUPPORTED, "merge is built for head_dim in {4,8,16,32,64,128,256} (got %lld)",
                (long long)head_dim);
  if (!out_acc || !lse_acc || !out_blk || !lse_blk) return fail(CP_ERR_INVALID, "NULL buffer");
  if (batch * seqlen * heads > ((int64_t(1) << 31) - 512) / (head_dim / 4))
    return fail(CP_ERR_UNSUPPORTED, "merge of 2^31 - 512 or more 16-byte vectors (out_acc of 32 GiB or more)");
  if (!aligned(out_acc, 16) || !aligned(out_blk, blk_dtype == CP_DTYPE_BF16 ? 8 : 16))
    return fail(CP_ERR_INVALID, "out_acc must be 16-byte aligned, out_blk 8 (bf16) / 16 (f32)");
  // the written buffers (out_acc, lse_acc) overlap neither each other nor a read-only
  // one: a workgroup's in-place writes would race with other workgroups' reads
  const int64_t rows = batch * seqlen * heads;
  const int64_t acc_b = rows * head_dim * 4, blk_b = rows * head_dim * dtype_bytes(blk_dtype), lse_b = rows * 4;
  if (overlaps(out_acc, acc_b, out_blk, blk_b) || overlaps(out_acc, acc_b, lse_blk, lse_b) ||
      overlaps(lse_acc, lse_b, out_blk, blk_b) || overlaps(lse_acc, lse_b, lse_blk, lse_b) ||
      overlaps(out_acc, acc_b, lse_acc, lse_b))
    return fail(CP_ERR_ALIAS, "merge buffers overlap");
  return hip_status(cp::launch_lse_merge(batch, seqlen, heads, head_dim, out_acc, lse_acc, out_blk,
                                         lse_blk, blk_dtype == CP_DTYPE_BF16, stream),
                    "cp_lse_merge launch");
}

static cp_status_t relayout(const cp_relayout_args_t* a, const void* in, void* out, hipStream_t stream) {
  if (!a) return fail(CP_ERR_INVALID, "args is NULL");
  const int64_t G = a->groups, P = a->P, batch = a->batch, seqlen = a->seqlen, heads = a->heads,
                head_dim = a->head_dim, eb = a->elem_bytes, rep = a->rep;
  if (G < 1 || P < 1 || batch < 1 || seqlen < 1 || heads < 1 || head_dim < 1 || rep < 1)
    return fail(CP_ERR_INVALID, "sizes must be >= 1");
  if (!sizes_fit({G, batch, seqlen, heads, head_dim, 4, rep}) || !sizes_fit({P, P, batch}))
    return fail(CP_ERR_INVALID, "sizes describe 2^62 bytes or more");
  if (eb != 2 && eb != 4) return fail(CP_ERR_INVALID, "elem_bytes must be 2 or 4 (got %lld)", (long long)eb);
  if (a->inverse != 0 && a->inverse != 1) return fail(CP_ERR_INVALID, "inverse must be 0 or 1");
  if (seqlen % P)
    return fail(CP_ERR_INVALID, "seqlen %lld is not divisible by the Ulysses degree %lld",
                (long long)seqlen, (long long)P);
  if ((heads * rep) % P)
    return fail(CP_ERR_INVALID,
                "heads %lld x rep %lld is not divisible by the Ulysses degree %lld (the degree cannot exceed "
                "the head count -- for k/v the kv head count -- unless heads are replicated)",
                (long long)heads, (long long)rep, (long long)P);
  if (rep > 1 && a->inverse && eb != 4)
    return fail(CP_ERR_INVALID, "the inverse with replicated heads sums float32 gradients (elem_bytes 4)");
  if (!in || !out) return fail(CP_ERR_INVALID, "NULL buffer");
  const int64_t seq_bytes = G * P * batch * (seqlen / P) * heads * head_dim * eb;  // sequence-sharded side
  const int64_t head_bytes = seq_bytes * rep;                                      // head-sharded side
  const int64_t in_bytes = a->inverse ? head_bytes : seq_bytes;
  const int64_t out_bytes = a->inverse ? seq_bytes : head_bytes;
  if (overlaps(in, in_bytes, out, out_bytes)) return fail(CP_ERR_ALIAS, "in and out overlap");
  // one grid slice (32-bit element offsets) per source span [S/P][H] and destination
  // span [S][H*rep/P]
  const int64_t seq_span = (seqlen / P) * heads * head_dim * eb;
  const int64_t head_span = seqlen * (heads * rep / P) * head_dim * eb;
  if (seq_span >= (int64_t(1) << 31) || head_span >= (int64_t(1) << 31) || P * batch * P >= (int64_t(1) << 31) ||
      G > 65535)
    return fail(CP_ERR_UNSUPPORTED, "relayout span exceeds 2^31 bytes or more than 65535 groups");
  const cp::RelayoutProblem r{G, P, batch, seqlen, heads, head_dim, eb, rep, a->inverse != 0};
  return hip_status(cp::launch_relayout(r, in, out, stream), "cp_ulysses_relayout launch");
}

cp_status_t cp_ulysses_relayout_ex(const cp_relayout_args_t* args, const void* in, void* out,
                                   hipStream_t stream) {
  return relayout(args, in, out, stream);
}

cp_status_t cp_ulysses_relayout(const void* in, void* out, int64_t P, int64_t batch, int64_t seqlen,
                                int64_t heads, int64_t head_dim, int64_t elem_bytes,
                                hipStream_t stream) {
  const cp_relayout_args_t a{1, P, batch, seqlen, heads, head_dim, elem_bytes, 1, 0};
  return relayout(&a, in, out, stream);
}

cp_status_t cp_ulysses_relayout_inv(const void* in, void* out, int64_t P, int64_t batch,
                                    int64_t seqlen, int64_t heads, int64_t head_dim,
                                    int64_t elem_bytes, hipStream_t stream) {
  const cp_relayout_args_t a{1, P, batch, seqlen, heads, head_dim, elem_bytes, 1, 1};
  return relayout(&a, in, out, stream);
}

cp_status_t cp_zigzag_reorder(const void* in, void* out, int64_t batch, int64_t seqlen,
                              int64_t row_bytes, int64_t P, int32_t strategy, int32_t inverse,
                              hipStream_t stream) {
  if (batch < 1 || seqlen < 1 || row_bytes < 1 || P < 1) return fail(CP_ERR_INVALID, "sizes must be >= 1");
  if (!sizes_fit({batch, seqlen, row_bytes}) || !sizes_fit({batch, 2, P}))
    return fail(CP_ERR_INVALID, "sizes describe 2^62 bytes or more");
  if (strategy != 0 && strategy != 1) return fail(CP_ERR_INVALID, "unknown reorder strategy %d", (int)strategy);
  if (inverse != 0 && inverse != 1) return fail(CP_ERR_INVALID, "inverse must be 0 or 1");
  if (strategy == 0 && seqlen % (2 * P))
    return fail(CP_ERR_INVALID, "seqlen %lld is not divisible into 2P = %lld chunks", (long long)seqlen,
                (long long)(2 * P));
  if (strategy == 1 && seqlen % P)
    return fail(CP_ERR_INVALID, "seqlen %lld is not divisible by P = %lld", (long long)seqlen, (long long)P);
  if (!in || !out) return fail(CP_ERR_INVALID, "NULL buffer");
  const int64_t bytes = batch * seqlen * row_bytes;
  if (overlaps(in, bytes, out, bytes)) return fail(CP_ERR_ALIAS, "in and out overlap");
  if (strategy == 0) {
    if (batch * 2 * P >= (int64_t(1) << 31)) return fail(CP_ERR_UNSUPPORTED, "too many chunks");
    return hip_status(cp::launch_zigzag(in, out, batch, seqlen, row_bytes, P, inverse != 0, stream),
                      "cp_zigzag_reorder launch");
  }
  // striped: rows (and so blocks) and row bytes below 2^31
  if (row_bytes >= (int64_t(1) << 31) || batch * seqlen >= (int64_t(1) << 31))
    return fail(CP_ERR_UNSUPPORTED, "striped reorder beyond 2^31 rows or 2^31-byte rows");
  return hip_status(cp::launch_striped(in, out, batch, seqlen, row_bytes, P, inverse != 0, stream),
                    "cp_zigzag_reorder launch");
}

cp_status_t cp_pad_rows(const void* in, void* out, int64_t batch, int64_t seqlen, int64_t seqlen_out,
                        int64_t row_bytes, uint32_t fill, hipStream_t stream) {
  if (batch < 1 || seqlen < 1 || seqlen_out < 1 || row_bytes < 1) return fail(CP_ERR_INVALID, "sizes must be >= 1");
  if (!sizes_fit({batch, seqlen, row_bytes}) || !sizes_fit({batch, seqlen_out, row_bytes}))
    return fail(CP_ERR_INVALID, "sizes describe 2^62 bytes or more");
  if (fill != 0 && row_bytes % 4)
    return fail(CP_ERR_INVALID, "a non-zero fill word needs rows of whole 32-bit words (row_bytes %lld)",
                (long long)row_bytes);
  if (!in || !out) return fail(CP_ERR_INVALID, "NULL buffer");
  if (overlaps(in, batch * seqlen * row_bytes, out, batch * seqlen_out * row_bytes))
    return fail(CP_ERR_ALIAS, "in and out overlap");
  if (batch > 65535 * 64) return fail(CP_ERR_UNSUPPORTED, "batch too large");
  return hip_status(cp::launch_pad_rows(in, out, batch, seqlen, seqlen_out, row_bytes, fill, stream),
                    "cp_pad_rows launch");
}

}  // extern "C"

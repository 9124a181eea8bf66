// Optional kernel tracing with HIP events (off by default).  When enabled, every
// launch of the library is bracketed by two events recorded on the launch stream;
// cp_prof_read() waits for them and reports per-kernel totals.
#pragma once

#include <hip/hip_runtime.h>

namespace cp {

enum ProfKernel : int {
  kProfFwdMfma = 0,     // bf16 attention forward (matrix cores)
  kProfFwdRowwise,      // row-per-wavefront forward (float32, bf16 head dims without MFMA kernel)
  kProfBwdDelta,        // bf16 backward pre-pass: Delta = rowsum(dO * O)
  kProfBwdMfma,         // bf16 backward: dK/dV and dQ roles in one grid
  kProfBwdRowwise,      // row-per-wavefront backward (delta, dQ, dK/dV)
  kProfLseMerge,        // ring-step log-sum-exp merge
  kProfUlysses,         // sequence -> head relayout
  kProfUlyssesInv,      // head -> sequence relayout
  kProfZigzag,          // zigzag reorder (either direction)
  kProfFwdMergeMfma,    // bf16 forward with the ring merge fused into its epilogue
  kProfFwdMergeRowwise, // float32 forward with the fused ring merge
  kProfStriped,         // striped reorder (either direction)
  kProfPadRows,         // sequence padding / truncation
  kProfCount
};

bool prof_enabled();
void prof_begin(hipStream_t s, int kernel);
void prof_end(hipStream_t s);

struct ProfScope {
  bool on;
  hipStream_t s;
  ProfScope(hipStream_t st, int kernel) : on(prof_enabled()), s(st) {
    if (on) prof_begin(s, kernel);
  }
  ~ProfScope() {
    if (on) prof_end(s);
  }
};

}  // namespace cp

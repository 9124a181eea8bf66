// Kernel tracing with HIP events: see prof.h.  Events are created on first use
// while tracing is on and reused afterwards; nothing happens while it is off.
#include <atomic>
#include <mutex>
#include <vector>

#include "cp_attn.h"
#include "prof.h"

namespace cp {
namespace {

struct Record {
  int kernel;
  hipEvent_t start, stop;
};

std::atomic<bool> g_on{false};
std::mutex g_mu;
std::vector<Record> g_pending;        // recorded, not yet read
std::vector<hipEvent_t> g_free;       // reusable events
thread_local int t_open = -1;         // index of the record begun on this thread
double g_total_ms[kProfCount];
int64_t g_count[kProfCount];

const char* const kNames[kProfCount] = {
    "attn_fwd_mfma", "attn_fwd_rowwise", "attn_bwd_delta", "attn_bwd_mfma", "attn_bwd_rowwise",
    "lse_merge", "ulysses_relayout", "ulysses_relayout_inv", "zigzag_reorder", "attn_fwd_merge_mfma",
    "attn_fwd_merge_rowwise", "striped_reorder", "pad_rows"};

hipEvent_t take_event() {
  if (!g_free.empty()) {
    hipEvent_t e = g_free.back();
    g_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

bool prof_enabled() { return g_on.load(std::memory_order_relaxed); }

void prof_begin(hipStream_t s, int kernel) {
  std::lock_guard<std::mutex> lk(g_mu);
  Record r{kernel, take_event(), take_event()};
  if (!r.start || !r.stop) return;
  hipEventRecord(r.start, s);
  g_pending.push_back(r);
  t_open = int(g_pending.size()) - 1;
}

void prof_end(hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (t_open < 0 || t_open >= int(g_pending.size())) return;
  hipEventRecord(g_pending[t_open].stop, s);
  t_open = -1;
}

}  // namespace cp

extern "C" {

void cp_prof_enable(int32_t on) { cp::g_on.store(on != 0); }

void cp_prof_reset(void) {
  std::lock_guard<std::mutex> lk(cp::g_mu);
  for (auto& r : cp::g_pending) {
    hipEventSynchronize(r.stop);
    cp::g_free.push_back(r.start);
    cp::g_free.push_back(r.stop);
  }
  cp::g_pending.clear();
  for (int i = 0; i < cp::kProfCount; ++i) {
    cp::g_total_ms[i] = 0.0;
    cp::g_count[i] = 0;
  }
}

int32_t cp_prof_kernel_count(void) { return cp::kProfCount; }

const char* cp_prof_kernel_name(int32_t kernel) {
  return (kernel >= 0 && kernel < cp::kProfCount) ? cp::kNames[kernel] : "";
}

cp_status_t cp_prof_read(int32_t kernel, double* total_ms, int64_t* launches) {
  if (kernel < 0 || kernel >= cp::kProfCount || !total_ms || !launches) return CP_ERR_INVALID;
  std::lock_guard<std::mutex> lk(cp::g_mu);
  for (auto& r : cp::g_pending) {
    float ms = 0.0f;
    if (hipEventSynchronize(r.stop) != hipSuccess) return CP_ERR_HIP;
    if (hipEventElapsedTime(&ms, r.start, r.stop) != hipSuccess) return CP_ERR_HIP;
    cp::g_total_ms[r.kernel] += ms;
    cp::g_count[r.kernel] += 1;
    cp::g_free.push_back(r.start);
    cp::g_free.push_back(r.stop);
  }
  cp::g_pending.clear();
  *total_ms = cp::g_total_ms[kernel];
  *launches = cp::g_count[kernel];
  return CP_OK;
}

}  // extern "C"

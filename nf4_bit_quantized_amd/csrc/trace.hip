// Opt-in per-kernel timing with hipEvents (off by default; no cost when off).
#include <mutex>
#include <vector>

#include "trace.hpp"
#include "../../include/qlora.h"

namespace qlora {
namespace {

const char* const kNames[KID_COUNT] = {
    "nf4_quantize", "fwd_gemm", "dx_gemm", "lora_down_gemm", "lora_g_gemm", "lora_grad_gemm",
    "lora_db_gemm", "decode", "reduce", "fill_zero", "export", "adamw", "dropout", "decode_sum"};

struct Pending {
  int kid;
  hipEvent_t start, stop;
};

std::mutex g_mu;
uint32_t g_mask = 0;  // bit k set: launches of kernel k are bracketed
std::vector<Pending> g_pending;
std::vector<hipEvent_t> g_pool;
int64_t g_launches[KID_COUNT] = {};
double g_ms[KID_COUNT] = {};

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  // timing only: no system-scope fence (cache writeback and invalidation)
  // when the event is recorded, which would lengthen the bracketed interval
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

TraceScope::TraceScope(int kid, hipStream_t stream) : kid_(kid), stream_(stream) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!((g_mask >> kid) & 1u)) return;
  start_ = take_event();
  stop_ = take_event();
  if (!start_ || !stop_) return;
  active_ = hipEventRecord(start_, stream_) == hipSuccess;
}

TraceScope::~TraceScope() {
  if (!active_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  if (hipEventRecord(stop_, stream_) == hipSuccess) g_pending.push_back({kid_, start_, stop_});
}

KernelEvents::KernelEvents(int kid) : kid_(kid) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!((g_mask >> kid) & 1u)) return;
  start_ = take_event();
  stop_ = take_event();
  if (!start_ || !stop_) {
    if (start_) g_pool.push_back(start_);
    if (stop_) g_pool.push_back(stop_);
    start_ = stop_ = nullptr;
  }
}

KernelEvents::~KernelEvents() {
  if (!start_) return;
  std::lock_guard<std::mutex> lk(g_mu);
  g_pending.push_back({kid_, start_, stop_});
}

}  // namespace qlora

using namespace qlora;

extern "C" int qlora_trace_enable(int enable) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_mask = enable ? 0xFFFFFFFFu : 0u;
  return QLORA_OK;
}

extern "C" int qlora_trace_select(uint32_t kernel_mask) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_mask = kernel_mask;
  return QLORA_OK;
}

extern "C" const char* qlora_trace_kernel_name(int kernel) {
  return (kernel >= 0 && kernel < KID_COUNT) ? kNames[kernel] : nullptr;
}

extern "C" int qlora_trace_read(qlora_kernel_stat* stats, int max_stats, int* count, int reset) {
  if (!count || (max_stats > 0 && !stats)) return QLORA_ERR_NULL;
  std::lock_guard<std::mutex> lk(g_mu);
  int rc = QLORA_OK;
  for (const Pending& p : g_pending) {
    float ms = 0.0f;
    if (hipEventSynchronize(p.stop) != hipSuccess || hipEventElapsedTime(&ms, p.start, p.stop) != hipSuccess) {
      rc = QLORA_ERR_HIP;
    } else {
      g_launches[p.kid] += 1;
      g_ms[p.kid] += ms;
    }
    g_pool.push_back(p.start);
    g_pool.push_back(p.stop);
  }
  g_pending.clear();
  int n = 0;
  for (int k = 0; k < KID_COUNT; ++k) {
    if (g_launches[k] == 0) continue;
    if (n < max_stats) {
      stats[n].name = kNames[k];
      stats[n].launches = g_launches[k];
      stats[n].total_ms = g_ms[k];
    }
    ++n;
  }
  *count = n;
  if (reset) {
    for (int k = 0; k < KID_COUNT; ++k) {
      g_launches[k] = 0;
      g_ms[k] = 0.0;
    }
  }
  return rc;
}

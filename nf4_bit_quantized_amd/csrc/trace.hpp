// Opt-in per-kernel timing: when enabled, each launch of the library is
// bracketed by two hipEvents recorded on the launch stream.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace qlora {

enum KernelId : int {
  KID_QUANTIZE = 0,
  KID_FWD_GEMM,
  KID_DX_GEMM,
  KID_LORA_DOWN,
  KID_LORA_G,
  KID_LORA_DA,
  KID_LORA_DB,
  KID_DECODE,
  KID_REDUCE,
  KID_FILL,
  KID_EXPORT,
  KID_ADAMW,
  KID_DROPOUT,
  KID_DECODE_SUM,
  KID_COUNT
};

class TraceScope {
 public:
  TraceScope(int kid, hipStream_t stream);
  ~TraceScope();
  TraceScope(const TraceScope&) = delete;
  TraceScope& operator=(const TraceScope&) = delete;

 private:
  int kid_;
  hipStream_t stream_;
  hipEvent_t start_ = nullptr, stop_ = nullptr;
  bool active_ = false;
};

// Timing events attached to one kernel's own dispatch: when kernel kid is
// traced, start() and stop() are events for hipExtLaunchKernelGGL, which
// records them at the kernel's begin and end (no separate marker packets
// around it, whose processing would add to the interval); otherwise both are
// null and the launch is untimed.  The pair is queued for qlora_trace_read
// when the object goes out of scope, after the launch.
class KernelEvents {
 public:
  explicit KernelEvents(int kid);
  ~KernelEvents();
  KernelEvents(const KernelEvents&) = delete;
  KernelEvents& operator=(const KernelEvents&) = delete;
  hipEvent_t start() const { return start_; }
  hipEvent_t stop() const { return stop_; }

 private:
  int kid_;
  hipEvent_t start_ = nullptr, stop_ = nullptr;
};

}  // namespace qlora

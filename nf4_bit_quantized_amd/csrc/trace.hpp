// Opt-in per-kernel timing: when enabled, each launch of the library is
// bracketed by two hipEvents recorded on the launch stream.
#pragma once

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

}  // namespace qlora

// Opt-in per-kernel timing with HIP events (internal to libdocmask).
//
// While timing is enabled, every launcher brackets its kernel with a pair of
// events recorded on the launch stream; the elapsed times are summed per
// kernel class when the host asks for them.  Disabled (the default), a
// KernelTimer costs one relaxed atomic load.
#pragma once

#include <hip/hip_runtime.h>

namespace docmask {

enum KernelClass {
  KC_SCHEDULE = 0,   // validate + tile descriptors + need intervals + LPT orders, per schedule build
  KC_FWD = 1,
  KC_DELTA = 2,      // no separate launch: Delta is formed inside the dQ kernel
  KC_DKDV = 3,
  KC_DQ = 4,
  KC_MERGE = 5,
  KC_CONVERT = 6,
  KC_COPY = 7,       // KV exchange row copies
  KC_HEAD = 8,       // backward head pass (fp32 pairs at document starts)
  KC_COUNT = 9
};

bool timing_enabled();
void* timing_start(hipStream_t stream);                   // nullptr when disabled
void timing_stop(void* token, int kernel_class, hipStream_t stream);

class KernelTimer {
 public:
  KernelTimer(int kernel_class, hipStream_t stream)
      : token_(timing_enabled() ? timing_start(stream) : nullptr), cls_(kernel_class), stream_(stream) {}
  ~KernelTimer() {
    if (token_) timing_stop(token_, cls_, stream_);
  }
  KernelTimer(const KernelTimer&) = delete;
  KernelTimer& operator=(const KernelTimer&) = delete;

 private:
  void* token_;
  int cls_;
  hipStream_t stream_;
};

}  // namespace docmask

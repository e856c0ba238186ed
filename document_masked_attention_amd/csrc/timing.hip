// Opt-in per-kernel timing: event pool, pending pairs, per-class totals.
#include <atomic>
#include <mutex>
#include <vector>

#include "docmask.h"
#include "timing.h"

namespace docmask {
namespace {

struct Pair {
  hipEvent_t start, stop;
  int device;
  int cls;
};

struct Pooled {
  hipEvent_t ev;
  int device;
};

std::atomic<bool> g_enabled{false};
std::mutex g_mu;
std::vector<Pooled> g_pool;         // idle events, tagged with the device they were created on
std::vector<Pair> g_pending;        // recorded, not yet read
double g_total_ms[KC_COUNT];
long long g_launches[KC_COUNT];

hipEvent_t take_event(int device) {   // caller holds g_mu
  for (size_t i = 0; i < g_pool.size(); ++i) {
    if (g_pool[i].device == device) {
      hipEvent_t e = g_pool[i].ev;
      g_pool[i] = g_pool.back();
      g_pool.pop_back();
      return e;
    }
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

void give_back(hipEvent_t e, int device) { g_pool.push_back({e, device}); }

struct Token {
  hipEvent_t start;
  int device;
};

// Waits for and accumulates every pending pair; caller holds g_mu.
int drain(bool keep) {
  int status = DOCMASK_OK;
  for (const Pair& p : g_pending) {
    float ms = 0.f;
    if (hipEventSynchronize(p.stop) != hipSuccess || hipEventElapsedTime(&ms, p.start, p.stop) != hipSuccess) {
      status = DOCMASK_EHIP;
    } else if (keep) {
      g_total_ms[p.cls] += ms;
      g_launches[p.cls] += 1;
    }
    give_back(p.start, p.device);
    give_back(p.stop, p.device);
  }
  g_pending.clear();
  return status;
}

}  // namespace

bool timing_enabled() { return g_enabled.load(std::memory_order_relaxed); }

void* timing_start(hipStream_t stream) {
  int device = 0;
  if (hipGetDevice(&device) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  hipEvent_t e = take_event(device);
  if (!e) return nullptr;
  if (hipEventRecord(e, stream) != hipSuccess) {
    give_back(e, device);
    return nullptr;
  }
  return new Token{e, device};
}

void timing_stop(void* token, int kernel_class, hipStream_t stream) {
  Token* t = static_cast<Token*>(token);
  std::lock_guard<std::mutex> lock(g_mu);
  hipEvent_t e = take_event(t->device);
  if (e && hipEventRecord(e, stream) == hipSuccess) {
    g_pending.push_back({t->start, e, t->device, kernel_class});
  } else {
    give_back(t->start, t->device);
    if (e) give_back(e, t->device);
  }
  delete t;
}

}  // namespace docmask

using namespace docmask;

extern "C" {

int docmask_timing_enable(int enable) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (enable) {
    drain(false);
    for (int i = 0; i < KC_COUNT; ++i) {
      g_total_ms[i] = 0.0;
      g_launches[i] = 0;
    }
  }
  g_enabled.store(enable != 0, std::memory_order_relaxed);
  return DOCMASK_OK;
}

int docmask_timing_read(int kernel_class, double* total_ms, int64_t* launches) {
  if (kernel_class < 0 || kernel_class >= KC_COUNT || !total_ms || !launches) return DOCMASK_EINVAL;
  std::lock_guard<std::mutex> lock(g_mu);
  const int status = drain(true);
  *total_ms = g_total_ms[kernel_class];
  *launches = g_launches[kernel_class];
  return status;
}

const char* docmask_kernel_class_name(int kernel_class) {
  switch (kernel_class) {
    case KC_SCHEDULE: return "schedule";
    case KC_FWD: return "fwd_kernel";
    case KC_DELTA: return "delta (computed inside dq_kernel)";
    case KC_DKDV: return "dkdv_kernel";
    case KC_DQ: return "dq_kernel";
    case KC_MERGE: return "merge_kernel";
    case KC_CONVERT: return "f32_to_bf16_kernel";
    case KC_COPY: return "copy_rows_kernel";
    case KC_HEAD: return "head_kernel";
    default: return "unknown";
  }
}

}  // extern "C"

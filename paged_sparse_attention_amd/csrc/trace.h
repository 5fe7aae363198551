// trace.h -- optional per-kernel event tracing for the entry points.
//
// The caller hands in hipEvent_t handles it created (oomb_trace_events); while
// they are set, every kernel launch records one event just before and one
// just after itself on its own stream, so the caller can time each kernel.
// Nothing is allocated; with no events set the cost is one branch.  A filter
// (oomb_trace_only) limits the recording to the launches of one kernel, so
// that timing it costs two event records per launch and no more.
#pragma once

#include <hip/hip_runtime.h>
#include <string.h>

namespace oomb {

constexpr int kMaxTraced = 65536;

struct TraceState {
  void* const* events = nullptr;
  int capacity = 0;  // number of event handles
  int count = 0;     // launches recorded so far
  int error = 0;     // first hipEventRecord failure (hipError_t), 0 if none
  char only[64] = {};  // record only launches of this kernel; empty: every launch
  const char* names[kMaxTraced];
};
TraceState& trace_state();

// Brackets one launch: construct before hipLaunchKernelGGL, destroy after.
class Traced {
 public:
  Traced(hipStream_t st, const char* name) : st_(st) {
    TraceState& t = trace_state();
    on_ = t.events != nullptr && 2 * t.count + 1 < t.capacity && t.count < kMaxTraced &&
          (t.only[0] == 0 || strcmp(t.only, name) == 0);
    if (on_) {
      t.names[t.count] = name;
      const hipError_t e = hipEventRecord((hipEvent_t)t.events[2 * t.count], st_);
      if (e != hipSuccess && t.error == 0) t.error = (int)e;
    }
  }
  ~Traced() {
    if (on_) {
      TraceState& t = trace_state();
      const hipError_t e = hipEventRecord((hipEvent_t)t.events[2 * t.count + 1], st_);
      if (e != hipSuccess && t.error == 0) t.error = (int)e;
      ++t.count;
    }
  }

 private:
  hipStream_t st_;
  bool on_;
};

}  // namespace oomb

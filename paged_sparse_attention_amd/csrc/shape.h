// shape.h -- the validated shape of one chunk step, and the host-only parts of
// the library (descriptor validation, the host-side gradient add).  Plain C++:
// no HIP header, so that host.cpp also builds with a host compiler alone (the
// sanitizer tests build it with g++ under AddressSanitizer, UBSan and TSan).
#pragma once

#include <stdint.h>

#include "oomb.h"

namespace oomb {

// A validated descriptor.
struct Shape {
  int hq, hkv, d, ps, ps_log2, c, n, keff, n_slots, rep_cap;
  bool bf16;
  float scale;  // resolved softmax scale
};

// Checks every field of the descriptor against the limits documented in
// include/oomb.h and fills *s.  Returns OOMB_OK or the first failing status;
// never touches the device.
int validate_desc(const oomb_desc* d, Shape* s);

// compact block b of delta (selected (kv-head, page) blocks in sel order, then
// the chunk pages' blocks, kv-head fastest) += into its (host slot, kv-head)
// block of host_dk / host_dv, on up to n_threads host threads.  Entries of
// sel or the page table that are out of range are skipped.  Returns OOMB_OK;
// if a helper thread cannot be started, the calling thread does its share and
// the result is the same.  No exception leaves the function.
int host_accumulate_grads(const Shape& s, const float* delta_dk, const float* delta_dv, const int32_t* pt,
                          const int32_t* sel, float* host_dk, float* host_dv, int n_threads);

}  // namespace oomb

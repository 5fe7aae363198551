// check.hip -- validation of the device-resident tables a chunk step trusts:
// the selection (logical pages, ascending, below N per kv-head) and the page
// table (a distinct slot below n_slots for each of the N + C/ps logical pages).
// The attention kernels take these contents as given (an entry out of range is
// an out-of-bounds access), so a caller that builds them itself can run this
// check first.  The kernels here only read the tables: any contents are safe.
#include <hip/hip_runtime.h>

#include "launch.h"
#include "trace.h"

namespace oomb {

namespace {

// counts[4] and the per-slot use counters start at zero (a kernel, so that the
// check can be captured in a graph)
__global__ void check_clear_kernel(int32_t* counts, int32_t* slot_uses, int n_slots) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < 4) counts[i] = 0;
  for (int s = i; s < n_slots; s += gridDim.x * blockDim.x) slot_uses[s] = 0;
}

__global__ void check_tables_kernel(const int32_t* __restrict__ pt, const int32_t* __restrict__ sel, int hkv,
                                    int keff, int n, int n_pages, int n_slots, int32_t* counts,
                                    int32_t* slot_uses) {
  const int stride = gridDim.x * blockDim.x;
  const int i0 = blockIdx.x * blockDim.x + threadIdx.x;
  const int nsel = hkv * keff;
  for (int i = i0; i < nsel; i += stride) {
    const int v = sel[i];
    if (v < 0 || v >= n) atomicAdd(&counts[0], 1);
    if (i % keff + 1 < keff && sel[i + 1] <= v) atomicAdd(&counts[1], 1);
  }
  for (int p = i0; p < n_pages; p += stride) {
    const int s = pt[p];
    if (s < 0 || s >= n_slots)
      atomicAdd(&counts[2], 1);
    else if (atomicAdd(&slot_uses[s], 1) >= 1)
      atomicAdd(&counts[3], 1);
  }
}

}  // namespace

hipError_t launch_check_tables(const Shape& s, const int32_t* pt, const int32_t* sel, int32_t* counts,
                               int32_t* slot_uses, hipStream_t st) {
  const int n_pages = s.n + s.c / s.ps;
  const int grid_clear = std::min(1024, std::max(1, (s.n_slots + 255) / 256));
  const int work = std::max(s.hkv * s.keff, n_pages);
  const int grid = std::min(1024, std::max(1, (work + 255) / 256));
  {
    Traced tr(st, "check_clear_kernel");
    hipLaunchKernelGGL(check_clear_kernel, dim3(grid_clear), dim3(256), 0, st, counts, slot_uses, s.n_slots);
  }
  Traced tr(st, "check_tables_kernel");
  hipLaunchKernelGGL(check_tables_kernel, dim3(grid), dim3(256), 0, st, pt, sel, s.hkv, s.keff, s.n, n_pages,
                     s.n_slots, counts, slot_uses);
  return hipGetLastError();
}

}  // namespace oomb

// Per-launch device timing (HIP event pairs on the launch stream, summed on
// read) and the launch status check, shared by the kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdio>
#include <vector>

#include "../ff_internal.h"

namespace ff {

// Kernel families timed separately (the fields of ff_kernel_times).
enum { kAttn = 0, kMerge, kPublish, kAnchor, kLayout, kBwdPre, kBwdDq, kBwdDk, kBwdDv, kKinds };

struct Profiler {
  struct Rec { int kind; hipEvent_t a, b; };
  std::vector<Rec> pending;
  std::vector<hipEvent_t> pool;
  int64_t count[kKinds] = {};
  double ms[kKinds] = {};
  unsigned families = ~0u;         // kinds that get event pairs
  hipEvent_t get() {
    if (!pool.empty()) { hipEvent_t e = pool.back(); pool.pop_back(); return e; }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};

namespace {

struct Timed {
  Profiler* p; int kind; hipStream_t s; hipEvent_t a = nullptr, b = nullptr;
  Timed(Profiler* p_, int k, hipStream_t s_) : p(p_), kind(k), s(s_) {
    if (p && ((p->families >> k) & 1u)) { a = p->get(); b = p->get(); if (a) (void)hipEventRecord(a, s); }
  }
  ~Timed() {
    if (p && a && b) { (void)hipEventRecord(b, s); p->pending.push_back({kind, a, b}); }
  }
};

int launch_ok() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    std::fprintf(stderr, "ff: kernel launch failed: %s\n", hipGetErrorString(e));
    return FF_E_HIP;
  }
  return 0;
}

}  // namespace
}  // namespace ff

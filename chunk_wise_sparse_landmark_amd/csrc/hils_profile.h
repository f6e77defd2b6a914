// Optional per-launch HIP-event recording for one kernel family (profiling).
#pragma once
#include <hip/hip_runtime.h>

namespace hils {

enum KernelId {
  kGenericSelect = 1, kGenericAttend = 2, kGenericBwdRows = 3, kGenericBwdChunks = 4,
  kDecodeScore = 5, kDecodeMerge = 6, kDecodeAttend = 7,
  kPrefillSelect = 8, kPrefillAttend = 9, kPrefillBwdRows = 10, kPrefillBwdChunks = 11,
  kLandmarks = 12, kLandmarksBwd = 13,
  kKernelIdEnd = 14
};

struct ProfileSlot {
  int kernel = 0;
  hipEvent_t const* starts = nullptr;
  hipEvent_t const* stops = nullptr;
  int n = 0;
  int next = 0;
};

ProfileSlot& profile_slot();

// A failed event record only loses that timing: the caller reads the events
// back with hipEventElapsedTime, which then reports the error; the launch
// status is not affected.
inline void prof_begin(int kernel, hipStream_t st) {
  ProfileSlot& p = profile_slot();
  if (p.kernel == kernel && p.next < p.n) (void)hipEventRecord(p.starts[p.next], st);
}
inline void prof_end(int kernel, hipStream_t st) {
  ProfileSlot& p = profile_slot();
  if (p.kernel == kernel && p.next < p.n) (void)hipEventRecord(p.stops[p.next++], st);
}

}  // namespace hils

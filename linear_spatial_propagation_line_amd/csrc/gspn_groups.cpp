// Host-side helpers for launches that give each plane one compute unit:
// the device's compute-unit count, helper streams, and plane groups that run
// their chains of launches on their own streams.
#include <algorithm>
#include <cstdlib>
#include <functional>
#include <mutex>

#include "gspn_launch.hpp"

namespace gspn {

// compute units of the current device (cached per device)
int cu_count() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> lk(mu);
  if (!cache[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// up to three non-blocking, default-priority helper streams per device,
// created on first use and kept for the life of the process
hipStream_t aux_stream(int i) {
  static std::mutex mu;
  static hipStream_t cache[64][kMaxGroups - 1] = {};
  int dev = 0;
  if (i < 0 || i >= kMaxGroups - 1) return nullptr;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lk(mu);
  if (!cache[dev][i] && hipStreamCreateWithFlags(&cache[dev][i], hipStreamNonBlocking) != hipSuccess)
    cache[dev][i] = nullptr;
  return cache[dev][i];
}

// number of plane groups (GSPN_TPIPE_GROUPS=1..4 overrides, for measurements)
int tpipe_groups(int64_t planes) {
  if (const char* v = std::getenv("GSPN_TPIPE_GROUPS")) {
    const int n = std::atoi(v);
    if (n >= 1 && n <= kMaxGroups) return static_cast<int>(std::min<int64_t>(n, planes));
  }
  const int cus = cu_count();
  return (planes > cus && planes < 2 * cus) ? 2 : 1;
}

hipError_t run_plane_groups(int64_t planes, hipStream_t stream,
                            const std::function<hipError_t(int64_t, int64_t, hipStream_t)>& fn) {
  const int ngroups = tpipe_groups(planes);
  if (ngroups <= 1) return fn(0, planes, stream);
  hipStream_t streams[kMaxGroups] = {stream, stream, stream, stream};
  hipEvent_t fork = nullptr, join[kMaxGroups] = {};
  hipError_t e = hipEventCreateWithFlags(&fork, hipEventDisableTiming);
  for (int g = 1; g < ngroups && e == hipSuccess; ++g) {
    streams[g] = aux_stream(g - 1);
    if (!streams[g]) e = hipErrorOutOfMemory;
    if (e == hipSuccess) e = hipEventCreateWithFlags(&join[g], hipEventDisableTiming);
  }
  if (e == hipSuccess) e = hipEventRecord(fork, stream);
  for (int g = 1; g < ngroups && e == hipSuccess; ++g) e = hipStreamWaitEvent(streams[g], fork, 0);
  for (int g = 0; g < ngroups && e == hipSuccess; ++g) {
    const int64_t p0 = planes * g / ngroups, p1 = planes * (g + 1) / ngroups;
    if (p1 > p0) e = fn(p0, p1 - p0, streams[g]);
  }
  // join whatever was forked, also after an error
  for (int g = 1; g < ngroups; ++g) {
    if (!join[g]) continue;
    hipError_t e2 = hipEventRecord(join[g], streams[g]);
    if (e2 == hipSuccess) e2 = hipStreamWaitEvent(stream, join[g], 0);
    if (e == hipSuccess) e = e2;
  }
  if (fork) (void)hipEventDestroy(fork);
  for (int g = 1; g < ngroups; ++g)
    if (join[g]) (void)hipEventDestroy(join[g]);
  return e;
}

}  // namespace gspn

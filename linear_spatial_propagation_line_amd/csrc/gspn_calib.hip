// Plain HBM stream kernels: the measured bandwidth ceiling the propagation
// kernels are compared with. Each thread moves 16-byte vectors, four in flight
// per loop trip, over a grid-stride loop on a grid that fills every compute
// unit several times over; the accesses are ordinary or non-temporal (a
// streaming hint to the caches). Nothing here is part of the propagation.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gspn_bench.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kUnroll = 4;

template <bool NT> __device__ __forceinline__ u32x4 ld(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  return *p;
}
template <bool NT> __device__ __forceinline__ void st(u32x4* p, u32x4 v) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// read: XOR of every word; a lane stores only if its XOR hits one chosen
// value, which keeps the loads live
template <bool NT>
__global__ __launch_bounds__(kThreads) void stream_read(const u32x4* __restrict__ src, size_t n,
                                                        uint32_t* __restrict__ sink) {
  const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
  size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) v[k] = ld<NT>(src + i + k * stride);
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) acc ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < n; i += stride) {
    const u32x4 v = ld<NT>(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9e3779b9u) sink[threadIdx.x] = acc;
}

template <bool NT>
__global__ __launch_bounds__(kThreads) void stream_write(u32x4* __restrict__ dst, size_t n) {
  const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
  size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
  const u32x4 v = {0u, 0u, 0u, 0u};
  for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) st<NT>(dst + i + k * stride, v);
  }
  for (; i < n; i += stride) st<NT>(dst + i, v);
}

template <bool NT>
__global__ __launch_bounds__(kThreads) void stream_copy(const u32x4* __restrict__ src,
                                                        u32x4* __restrict__ dst, size_t n) {
  const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
  size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) v[k] = ld<NT>(src + i + k * stride);
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) st<NT>(dst + i + k * stride, v[k]);
  }
  for (; i < n; i += stride) st<NT>(dst + i, ld<NT>(src + i));
}

template <bool NT>
void launch(int kind, dim3 grid, const u32x4* s, void* dst, size_t n, hipStream_t stream) {
  if (kind == 0)
    hipLaunchKernelGGL(stream_read<NT>, grid, dim3(kThreads), 0, stream, s, n,
                       static_cast<uint32_t*>(dst));
  else if (kind == 1)
    hipLaunchKernelGGL(stream_write<NT>, grid, dim3(kThreads), 0, stream,
                       static_cast<u32x4*>(dst), n);
  else
    hipLaunchKernelGGL(stream_copy<NT>, grid, dim3(kThreads), 0, stream, s,
                       static_cast<u32x4*>(dst), n);
}

}  // namespace

extern "C" int gspn_bench_stream(int kind, int nontemporal, const void* src, void* dst,
                                 size_t bytes, int blocks_per_cu, hipStream_t stream) {
  if (kind < 0 || kind > 2 || bytes == 0 || bytes % 16 || blocks_per_cu < 1 ||
      blocks_per_cu > 64)
    return 1;
  if ((kind != 1 && (!src || reinterpret_cast<uintptr_t>(src) % 16)) ||
      !dst || reinterpret_cast<uintptr_t>(dst) % 16)
    return 1;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return 2;
  const size_t n = bytes / 16;
  const dim3 grid(static_cast<unsigned>(cus * blocks_per_cu));
  const u32x4* s = static_cast<const u32x4*>(src);
  if (nontemporal)
    launch<true>(kind, grid, s, dst, n, stream);
  else
    launch<false>(kind, grid, s, dst, n, stream);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// ---------------------------------------------------------------------------
// Cross-workgroup handshake: the latency of one flag exchange between two
// workgroups through device memory, the step any schedule that splits a
// scan line over several workgroups has to take between blocks of steps.
// Workgroup 0 and workgroup `partner` (one lane each) take turns: A stores
// round k into its flag (release, device scope), B waits for it (acquire)
// and answers in its own flag, A waits for the answer. Every wait is bounded
// by spin_max polls and also ends when the host sets *abort (host memory),
// so the kernel always exits; out[0] = A's elapsed wall-clock ticks, out[1] =
// waits that gave up, out[2] = polls in total.
// ---------------------------------------------------------------------------
namespace {

__device__ __forceinline__ bool wait_for(uint32_t* flag, uint32_t want, const uint32_t* abort_flag,
                                         int spin_max, uint64_t* polls) {
  for (int i = 0; i < spin_max; ++i) {
    ++*polls;
    if (__hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) == want) return true;
    if ((i & 255) == 255 &&
        __hip_atomic_load(abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) != 0u)
      return false;
  }
  return false;
}

__global__ __launch_bounds__(64) void handshake(uint32_t* flags, const uint32_t* abort_flag,
                                                int rounds, int spin_max, int partner,
                                                uint64_t* out) {
  const int b = static_cast<int>(blockIdx.x);
  if (threadIdx.x != 0 || (b != 0 && b != partner)) return;
  uint32_t* mine = flags + (b == 0 ? 0 : 64);     // 256 bytes apart
  uint32_t* theirs = flags + (b == 0 ? 64 : 0);
  uint64_t polls = 0, missed = 0;
  const uint64_t t0 = wall_clock64();
  for (int k = 1; k <= rounds; ++k) {
    const uint32_t v = static_cast<uint32_t>(k);
    if (b == 0) {
      __hip_atomic_store(mine, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      if (!wait_for(theirs, v, abort_flag, spin_max, &polls)) { ++missed; break; }
    } else {
      if (!wait_for(theirs, v, abort_flag, spin_max, &polls)) { ++missed; break; }
      __hip_atomic_store(mine, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  const uint64_t t1 = wall_clock64();
  if (b == 0) {
    out[0] = t1 - t0;
    out[1] = missed;
    out[2] = polls;
  } else {
    out[3] = missed;
  }
}

}  // namespace

extern "C" int gspn_bench_handshake(void* flags, const uint32_t* abort_flag, int rounds,
                                    int spin_max, int partner, uint64_t* out,
                                    hipStream_t stream) {
  if (!flags || !abort_flag || !out || rounds < 1 || spin_max < 1 || partner < 1 ||
      partner > 4095 || reinterpret_cast<uintptr_t>(flags) % 256 ||
      reinterpret_cast<uintptr_t>(out) % 8)
    return 1;
  hipLaunchKernelGGL(handshake, dim3(static_cast<unsigned>(partner + 1)), dim3(64), 0, stream,
                     static_cast<uint32_t*>(flags), abort_flag, rounds, spin_max, partner, out);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int gspn_bench_wall_clock_khz(void) {
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
    return 0;
  return khz;
}

// Measured prototype of the other schedule for large planes: a scan line
// split over several workgroups. It is not a plan of the library (nothing
// calls it but the benchmark); it exists so that the one-workgroup-per-plane
// pipeline can be compared with a measured alternative rather than an
// estimate.
//
// One direction (top->bottom, global, bf16 storage, fp32 state), out = u h.
// A plane of width W is split into S strips of Ws = W / S columns. One
// wavefront owns a strip plus a halo of K columns on each side (Ws + 2K <= 64
// lanes, neighbours by DPP), and walks the rows in blocks of K. A block
// starts from exact states of all its lanes; a lane's state stays exact while
// its neighbours' are, so after K rows the exact region has shrunk to the
// strip itself. Between blocks each strip hands the states of its K leftmost
// and K rightmost columns to its neighbours through device memory (relaxed
// agent-scope atomics for the values, a release flag per strip) and takes
// theirs as its new halo. P planes are in flight at once (pf), so the inputs
// of a slab of planes are what the caches must hold.
//
// Every wait is bounded (spin_max polls) and also ends when the host sets
// *abort_flag or another workgroup has given up (*fail), so the kernel
// always exits; a give-up is reported and the output is then not valid. The
// whole grid (pf * S one-wavefront workgroups) must be resident at once,
// which the host checks before the launch.
//
// Line recurrence and output gate: CSDN page on GSPN, section 方法;
// tridiagonal row-normalised sigmoid weights: section 如何设计一个高效的传播层.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gspn_bench.h"
#include "gspn_device.hpp"

namespace gspn {
namespace {

constexpr int kStripLanes = 64;
constexpr int kFlagStride = 64;   // uint32 between two strips' flags: 256 bytes

struct StripArgs {
  const bf16_t* x;
  const bf16_t* lam;
  const bf16_t* l0;
  const bf16_t* l1;
  const bf16_t* l2;
  const bf16_t* u;
  bf16_t* out;
  int64_t planes;
  int H, W, S, pf, spin_max;
  uint32_t* flags;            // [pf * S][kFlagStride]: last epoch a strip published
  uint32_t* fail;             // set by a workgroup whose wait gave up
  float* pub;                 // [pf * S][2 parities][2 sides][K] published states
  const uint32_t* abort_flag;
};

// Polls are relaxed: an acquire at agent scope invalidates the XCD's L2, and
// every poll of thousands of waiting workgroups doing that would flush the
// caches the scans read from. One acquire fence follows a successful poll.
__device__ __forceinline__ bool strip_wait(const uint32_t* flag, uint32_t want, const StripArgs& a) {
  for (int i = 0; i < a.spin_max; ++i) {
    if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= want) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      return true;
    }
    if ((i & 255) == 255 &&
        (__hip_atomic_load(a.fail, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u ||
         __hip_atomic_load(a.abort_flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) != 0u))
      return false;
  }
  return false;
}

template <int K>
__global__ __launch_bounds__(kStripLanes) void strip_t2b(StripArgs a) {
  const int S = a.S, W = a.W, H = a.H;
  const int Ws = W / S;
  const int lane = threadIdx.x;
  const int slot = static_cast<int>(blockIdx.x) / S, s = static_cast<int>(blockIdx.x) % S;
  const int c = s * Ws - K + lane;                 // this lane's column
  const int cc = min(max(c, 0), W - 1);            // in-bounds column for loads
  const bool own = lane >= K && lane < K + Ws;     // the strip's own columns
  const float m0 = c > 0 ? 1.f : 0.f, m2 = c < W - 1 ? 1.f : 0.f;
  const int nb = (H + K - 1) / K;
  uint32_t* myflag = a.flags + static_cast<int64_t>(slot * S + s) * kFlagStride;
  const uint32_t* lflag = a.flags + static_cast<int64_t>(slot * S + max(s - 1, 0)) * kFlagStride;
  const uint32_t* rflag = a.flags + static_cast<int64_t>(slot * S + min(s + 1, S - 1)) * kFlagStride;
  auto pub = [&](int strip, uint32_t epoch, int side) {
    return a.pub + ((static_cast<int64_t>(slot * S + strip) * 2 + (epoch & 1)) * 2 + side) * K;
  };
  uint32_t iter = 0;
  for (int64_t p = slot; p < a.planes; p += a.pf, ++iter) {
    const int64_t base = p * static_cast<int64_t>(H) * W;
    float h = 0.f;
    for (int b = 0; b < nb; ++b) {
      // epoch e: the number of blocks every strip of this slot has published.
      // Every block after the very first waits for both neighbours to have
      // published e, so no strip runs two epochs ahead of a neighbour and a
      // parity slot is never overwritten before it is read.
      const uint32_t e = iter * static_cast<uint32_t>(nb) + static_cast<uint32_t>(b);
      if (e > 0) {
        bool ok = true;
        if (s > 0) ok = strip_wait(lflag, e, a);
        if (ok && s < S - 1) ok = strip_wait(rflag, e, a);
        if (!ok) {
          if (lane == 0) __hip_atomic_store(a.fail, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          return;
        }
        if (b > 0) {   // the halo: the neighbours' edge columns at the row before this block
          if (lane < K && s > 0)
            h = __hip_atomic_load(pub(s - 1, e, 1) + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (lane >= K + Ws && lane < 2 * K + Ws && s < S - 1)
            h = __hip_atomic_load(pub(s + 1, e, 0) + (lane - K - Ws), __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      const int r0 = b * K, r1 = min(r0 + K, H);
      for (int r = r0; r < r1; ++r) {
        const int64_t i = base + static_cast<int64_t>(r) * W + cc;
        const float lx = to_f32(a.lam[i]) * to_f32(a.x[i]);
        const Weights w = make_weights(to_f32(a.l0[i]), to_f32(a.l1[i]), to_f32(a.l2[i]), m0, m2);
        const float hl = from_left<64>(h), hr = from_right<64>(h);
        const float hn = __builtin_fmaf(w.w0, hl, __builtin_fmaf(w.w1, h, __builtin_fmaf(w.w2, hr, lx)));
        h = r == 0 ? lx : hn;
        if (own) a.out[i].bits = static_cast<uint16_t>(f32_to_bf16_bits(to_f32(a.u[i]) * h));
      }
      // publish the K leftmost and K rightmost own columns, then the epoch
      const uint32_t e1 = e + 1;
      if (lane >= K && lane < 2 * K)
        __hip_atomic_store(pub(s, e1, 0) + (lane - K), h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (lane >= Ws && lane < Ws + K)
        __hip_atomic_store(pub(s, e1, 1) + (lane - Ws), h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // the release store orders the wavefront's stores before the flag (the
      // wait for outstanding stores it implies covers every lane)
      if (lane == 0) __hip_atomic_store(myflag, e1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace
}  // namespace gspn

extern "C" size_t gspn_bench_strip_fail_offset(int S, int pf) {
  return static_cast<size_t>(pf < 1 ? 0 : pf) * (S < 1 ? 0 : S) * gspn::kFlagStride * 4;
}

extern "C" size_t gspn_bench_strip_work_bytes(int S, int K, int pf) {
  if (S < 1 || K < 1 || pf < 1) return 0;
  const size_t flags = static_cast<size_t>(pf) * S * gspn::kFlagStride * 4;
  return flags + 256 + static_cast<size_t>(pf) * S * 4 * K * 4;
}

extern "C" int gspn_bench_strip_t2b(const void* x, const void* lam, const void* const logits[3],
                                    const void* u, void* out, int64_t planes, int H, int W,
                                    int S, int K, int pf, void* work, size_t work_bytes,
                                    const uint32_t* abort_flag, int spin_max, hipStream_t stream) {
  using namespace gspn;
  if (!x || !lam || !logits || !logits[0] || !logits[1] || !logits[2] || !u || !out || !work ||
      !abort_flag || planes < 1 || H < 1 || W < 2 || S < 2 || (K != 8 && K != 16) || pf < 1 ||
      spin_max < 1 || W % S != 0 || W / S + 2 * K > kStripLanes || W / S < K ||
      work_bytes < gspn_bench_strip_work_bytes(S, K, pf) ||
      reinterpret_cast<uintptr_t>(work) % 256)
    return 1;
  // the whole grid must be resident at once: its workgroups wait on each other
  auto kern = K == 8 ? strip_t2b<8> : strip_t2b<16>;
  int per_cu = 0, dev = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern),
                                                   kStripLanes, 0) != hipSuccess ||
      hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 2;
  if (static_cast<int64_t>(pf) * S > static_cast<int64_t>(per_cu) * cus) return 1;
  StripArgs a;
  a.x = static_cast<const bf16_t*>(x);
  a.lam = static_cast<const bf16_t*>(lam);
  a.l0 = static_cast<const bf16_t*>(logits[0]);
  a.l1 = static_cast<const bf16_t*>(logits[1]);
  a.l2 = static_cast<const bf16_t*>(logits[2]);
  a.u = static_cast<const bf16_t*>(u);
  a.out = static_cast<bf16_t*>(out);
  a.planes = planes;
  a.H = H;
  a.W = W;
  a.S = S;
  a.pf = static_cast<int>(pf < planes ? pf : planes);
  a.spin_max = spin_max;
  char* w = static_cast<char*>(work);
  a.flags = reinterpret_cast<uint32_t*>(w);
  a.fail = reinterpret_cast<uint32_t*>(w + static_cast<size_t>(pf) * S * kFlagStride * 4);
  a.pub = reinterpret_cast<float*>(w + static_cast<size_t>(pf) * S * kFlagStride * 4 + 256);
  a.abort_flag = abort_flag;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(a.pf * S)), dim3(kStripLanes), 0, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

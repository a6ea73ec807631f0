// Streaming GSPN propagation for planes of any size: one launch per scan
// direction, one workgroup per plane.
//
// The workgroup owns the whole orthogonal axis of its plane (the scan couples
// neighbouring lines at every step, so a line cannot be split across
// workgroups). Thread t owns orthogonal indices t, t + 256, t + 512, ...;
// every step it reads x, lambda and the three logits of its pixels from HBM,
// builds the normalised weights inline, takes the previous line's states from
// a double-buffered LDS line and writes the new states back, with one barrier
// per step. Directions are combined through an fp32 accumulator in the
// workspace: the first selected direction writes it, the following ones add
// to it, the last one writes out = u * (acc + h) in the storage type.
//
// Line recurrence and output gate: CSDN page on GSPN, section 方法;
// tridiagonal weights, sigmoid + row normalisation, four directions: section
// 如何设计一个高效的传播层; local groups: section GSPN模块的设计.
#include "gspn_device.hpp"
#include "gspn_launch.hpp"

namespace gspn {

enum StreamMode { kFirst = 0, kMid = 1, kLast = 2, kOnly = 3 };

template <typename T>
struct StreamArgs {
  const T* x;
  const T* l0;
  const T* l1;
  const T* l2;
  const T* lam;
  const T* u;
  T* out;
  float* acc;
  int H, W, G;
  int dir;
  int mode;
  int64_t C, Cl;    // channels and logit channels (shared logits when Cl < C)
};

__device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld(const bf16_t* p, int64_t i) { return to_f32(p[i]); }

template <typename T>
__global__ __launch_bounds__(256) void stream_kernel(StreamArgs<T> a) {
  extern __shared__ float line[];   // [2][n_o]
  const int H = a.H, W = a.W, G = a.G, d = a.dir;
  const bool vert = d < 2, fwd = (d == 0 || d == 2);
  const int n_s = vert ? H : W, n_o = vert ? W : H;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * H * W;
  const int64_t ls = logit_shift(blockIdx.x, a.C, a.Cl, static_cast<int64_t>(H) * W);
  int next_restart = n_s;
  if (G > 0) next_restart = fwd ? G : n_s - ((n_s - 1) / G) * G;

  for (int s = 0; s < n_s; ++s) {
    bool restart = (s == 0);
    if (s == next_restart) { restart = true; next_restart += G; }
    const int pos = fwd ? s : n_s - 1 - s;
    float* cur = line + (s & 1) * n_o;
    const float* prev = line + ((s & 1) ^ 1) * n_o;
    for (int o = threadIdx.x; o < n_o; o += 256) {
      const int r = vert ? pos : o, c = vert ? o : pos;
      const int64_t idx = base + static_cast<int64_t>(r) * W + c;
      float h = ld(a.lam, idx) * ld(a.x, idx);
      if (!restart) {
        const Weights w = make_weights(ld(a.l0, idx + ls), ld(a.l1, idx + ls), ld(a.l2, idx + ls),
                                       o > 0 ? 1.f : 0.f, o < n_o - 1 ? 1.f : 0.f);
        const float hl = prev[o > 0 ? o - 1 : 0];
        const float hr = prev[o < n_o - 1 ? o + 1 : o];
        h = __builtin_fmaf(w.w0, hl, __builtin_fmaf(w.w1, prev[o], __builtin_fmaf(w.w2, hr, h)));
      }
      cur[o] = h;
      if (a.mode == kFirst) {
        a.acc[idx] = h;
      } else if (a.mode == kMid) {
        a.acc[idx] += h;
      } else if (a.mode == kLast) {
        Store<T>::put(a.out, idx, ld(a.u, idx) * (a.acc[idx] + h));
      } else {
        Store<T>::put(a.out, idx, ld(a.u, idx) * h);
      }
    }
    __syncthreads();
  }
}

int64_t stream_max_orth() { return 16384; }

template <typename T>
static hipError_t launch_stream_dt(const Problem& pr, float* acc, hipStream_t stream,
                                   Tracer* tr) {
  const int64_t planes = pr.B * pr.C;
  int dirs[4], nd = 0;
  for (int d = 0; d < 4; ++d)
    if ((pr.mask >> d) & 1u) dirs[nd++] = d;
  for (int i = 0; i < nd; ++i) {
    StreamArgs<T> a;
    a.x = static_cast<const T*>(pr.x);
    a.l0 = static_cast<const T*>(pr.l[0]);
    a.l1 = static_cast<const T*>(pr.l[1]);
    a.l2 = static_cast<const T*>(pr.l[2]);
    a.lam = static_cast<const T*>(pr.lam);
    a.u = static_cast<const T*>(pr.u);
    a.out = static_cast<T*>(pr.out);
    a.acc = acc;
    a.H = static_cast<int>(pr.H);
    a.W = static_cast<int>(pr.W);
    a.G = static_cast<int>(pr.G);
    a.dir = dirs[i];
    a.C = pr.C;
    a.Cl = pr.Cl;
    a.mode = nd == 1 ? kOnly : (i == 0 ? kFirst : (i == nd - 1 ? kLast : kMid));
    const int64_t n_o = dirs[i] < 2 ? pr.W : pr.H;
    const size_t lds = static_cast<size_t>(2 * n_o) * sizeof(float);
    auto kern = stream_kernel<T>;
    if (lds > 65536) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         static_cast<int>(lds));
      if (e != hipSuccess) return e;
    }
    tr->before(stream, "stream_kernel", planes);
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(planes)), dim3(256), lds, stream, a);
    tr->after(stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_stream(const Problem& pr, float* acc, hipStream_t stream, Tracer* tr) {
  if (pr.dtype == GSPN_F32) return launch_stream_dt<float>(pr, acc, stream, tr);
  return launch_stream_dt<bf16_t>(pr, acc, stream, tr);
}

}  // namespace gspn

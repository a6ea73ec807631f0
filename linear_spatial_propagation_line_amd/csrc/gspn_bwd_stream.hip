// Backward pass of the GSPN propagation, streaming path for planes of any
// size (orthogonal length up to 16384): two launches per scan direction, one
// workgroup per plane each.
//
// For one direction (CSDN page on GSPN, section 反向传播: the hidden-state
// gradient of a line collects what later lines send back; the input gradient
// goes through lambda; the gate gradients pair the error term with the
// previous hidden state):
//   bwd_fwd  runs the forward scan and stores every state h_s in an fp32
//            plane of the workspace (and adds h into the running sum that
//            becomes grad_u = grad_out * sum_d h_d);
//   bwd_adj  runs the reverse scan of the error term
//              e_s[o] = u gy + w_{s+1,0}[o+1] e_{s+1}[o+1]
//                            + w_{s+1,1}[o]   e_{s+1}[o]
//                            + w_{s+1,2}[o-1] e_{s+1}[o-1]
//            (the transposed tridiagonal; nothing from a line that restarts),
//            and from it and the stored h_{s-1} the logit gradients
//              dl_k = e w_k (1 - sigmoid(l_k)) (h_{s-1}[o+k-1] - p),
//              p = sum_j w_j h_{s-1}[o+j-1],
//            which is the chain rule through w_k = sigmoid(l_k) / sum_j
//            sigmoid(l_j). h_{s-1}[o+k-1] - p is formed from differences of
//            neighbouring states (sum_j w_j = 1), so it is exactly 0 wherever
//            the neighbours agree.
// Directions combine through fp32 accumulators in the workspace (d(lambda x),
// three logit gradients, sum of h): the first direction writes them, later
// ones add, the last one writes the six gradients in the storage type.
//
// Horizontal scans read the row-major tensors with a stride of W; this path
// is the general one, not the fast one.
#include "gspn_device.hpp"
#include "gspn_launch.hpp"

namespace gspn {

namespace {
constexpr int kBwThreads = 1024;
enum : int { kBwFirst = 1, kBwLast = 2 };

__device__ __forceinline__ float bl(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float bl(const bf16_t* p, int64_t i) { return to_f32(p[i]); }

// restart test of scan step s (first step, or first position of a group in
// this scan order)
__device__ __forceinline__ bool restarts(int s, int n_s, int G, bool fwd) {
  if (s == 0) return true;
  if (G <= 0) return false;
  return fwd ? (s % G) == 0 : ((n_s - 1 - s) % G) == G - 1;
}
}  // namespace

template <typename T>
struct BwArgs {
  const T* x;
  const T* l0;
  const T* l1;
  const T* l2;
  const T* lam;
  const T* u;
  const T* gy;
  T* dx;
  T* dl0;
  T* dl1;
  T* dl2;
  T* dlam;
  T* du;
  float* hbuf;      // states of the current direction, [planes][H][W]
  float* acc;       // [5][planes][H][W]: d(lambda x), dl0, dl1, dl2, sum of h
  int64_t pstride;  // planes * H * W
  int H, W, G, dir, mode;
};

// forward scan of one direction: h into hbuf, and into the running sum of h
template <typename T>
__global__ __launch_bounds__(kBwThreads) void bwd_fwd(BwArgs<T> a) {
  extern __shared__ float line[];   // [2][n_o]
  const int H = a.H, W = a.W, G = a.G, d = a.dir;
  const bool vert = d < 2, fwd = (d == 0 || d == 2);
  const int n_s = vert ? H : W, n_o = vert ? W : H;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * H * W;
  float* hsum = a.acc + 4 * a.pstride;
  for (int s = 0; s < n_s; ++s) {
    const bool restart = restarts(s, n_s, G, fwd);
    const int pos = fwd ? s : n_s - 1 - s;
    float* cur = line + (s & 1) * n_o;
    const float* prev = line + ((s & 1) ^ 1) * n_o;
    for (int o = threadIdx.x; o < n_o; o += kBwThreads) {
      const int r = vert ? pos : o, c = vert ? o : pos;
      const int64_t idx = base + static_cast<int64_t>(r) * W + c;
      float h = bl(a.lam, idx) * bl(a.x, idx);
      if (!restart) {
        const Weights w = make_weights(bl(a.l0, idx), bl(a.l1, idx), bl(a.l2, idx),
                                       o > 0 ? 1.f : 0.f, o < n_o - 1 ? 1.f : 0.f);
        const float hl = prev[o > 0 ? o - 1 : 0];
        const float hr = prev[o < n_o - 1 ? o + 1 : o];
        h = __builtin_fmaf(w.w0, hl, __builtin_fmaf(w.w1, prev[o], __builtin_fmaf(w.w2, hr, h)));
      }
      cur[o] = h;
      a.hbuf[idx] = h;
      if (a.mode & kBwFirst) {
        if (!(a.mode & kBwLast)) hsum[idx] = h;
      } else {
        hsum[idx] += h;
      }
    }
    __syncthreads();
  }
}

// reverse scan of the error term and the gradients of one direction.
// MAXP = bound on orthogonal positions per thread (n_o <= MAXP * 1024).
template <typename T, int MAXP>
__global__ __launch_bounds__(kBwThreads) void bwd_adj(BwArgs<T> a) {
  extern __shared__ float sm[];   // [2][n_o]: w_0 e and w_2 e of the line below
  const int H = a.H, W = a.W, G = a.G, d = a.dir;
  const bool vert = d < 2, fwd = (d == 0 || d == 2);
  const int n_s = vert ? H : W, n_o = vert ? W : H;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * H * W;
  const int64_t ps = a.pstride;
  const bool first = a.mode & kBwFirst, last = a.mode & kBwLast;
  float* A0 = sm;
  float* A2 = sm + n_o;
  // previous line in scan order sits one position back along the scan axis
  const int back = fwd ? -1 : 1;
  const int64_t back_off = vert ? static_cast<int64_t>(back) * W : back;

  float a1[MAXP], b0[MAXP], b2[MAXP];
#pragma unroll
  for (int i = 0; i < MAXP; ++i) a1[i] = 0.f;
  for (int o = threadIdx.x; o < n_o; o += kBwThreads) { A0[o] = 0.f; A2[o] = 0.f; }
  __syncthreads();

  for (int s = n_s - 1; s >= 0; --s) {
    const bool restart = restarts(s, n_s, G, fwd);
    const int pos = fwd ? s : n_s - 1 - s;
#pragma unroll
    for (int i = 0; i < MAXP; ++i) {
      const int o = threadIdx.x + i * kBwThreads;
      b0[i] = 0.f;
      b2[i] = 0.f;
      if (o < n_o) {
        const int r = vert ? pos : o, c = vert ? o : pos;
        const int64_t idx = base + static_cast<int64_t>(r) * W + c;
        const float gyv = bl(a.gy, idx);
        float e = bl(a.u, idx) * gyv + a1[i];
        if (o + 1 < n_o) e += A0[o + 1];
        if (o > 0) e += A2[o - 1];
        float dl0 = 0.f, dl1 = 0.f, dl2 = 0.f;
        float w1e = 0.f;
        if (!restart) {
          const float m0 = o > 0 ? 1.f : 0.f, m2 = o < n_o - 1 ? 1.f : 0.f;
          const WeightSlopes q = make_weight_slopes(bl(a.l0, idx), bl(a.l1, idx), bl(a.l2, idx), m0, m2);
          const int64_t pidx = idx + back_off;
          const int64_t oo = vert ? 1 : W;   // orthogonal stride
          const float hc = a.hbuf[pidx];
          const float hl = o > 0 ? a.hbuf[pidx - oo] : hc;
          const float hr = o < n_o - 1 ? a.hbuf[pidx + oo] : hc;
          // h_k - p = sum_j w_j (h_k - h_j)
          const float d01 = hl - hc, d12 = hc - hr, d02 = hl - hr;
          const float dev0 = q.w1 * d01 + q.w2 * d02;
          const float dev1 = q.w2 * d12 - q.w0 * d01;
          const float dev2 = -(q.w0 * d02 + q.w1 * d12);
          dl0 = e * q.q0 * dev0;
          dl1 = e * q.q1 * dev1;
          dl2 = e * q.q2 * dev2;
          b0[i] = q.w0 * e;
          b2[i] = q.w2 * e;
          w1e = q.w1 * e;
        }
        a1[i] = w1e;
        float dphi = e;
        if (!first) {
          dphi += a.acc[idx];
          dl0 += a.acc[ps + idx];
          dl1 += a.acc[2 * ps + idx];
          dl2 += a.acc[3 * ps + idx];
        }
        if (last) {
          Store<T>::put(a.dx, idx, bl(a.lam, idx) * dphi);
          Store<T>::put(a.dlam, idx, bl(a.x, idx) * dphi);
          Store<T>::put(a.dl0, idx, dl0);
          Store<T>::put(a.dl1, idx, dl1);
          Store<T>::put(a.dl2, idx, dl2);
          const float hs = first ? a.hbuf[idx] : a.acc[4 * ps + idx];
          Store<T>::put(a.du, idx, gyv * hs);
        } else {
          a.acc[idx] = dphi;
          a.acc[ps + idx] = dl0;
          a.acc[2 * ps + idx] = dl1;
          a.acc[3 * ps + idx] = dl2;
        }
      }
    }
    __syncthreads();   // every thread has read the line below
#pragma unroll
    for (int i = 0; i < MAXP; ++i) {
      const int o = threadIdx.x + i * kBwThreads;
      if (o < n_o) { A0[o] = b0[i]; A2[o] = b2[i]; }
    }
    __syncthreads();
  }
}

size_t bwd_stream_workspace_bytes(int64_t planes, int64_t H, int64_t W, uint32_t mask) {
  const size_t px = static_cast<size_t>(planes * H * W);
  return (__builtin_popcount(mask) > 1 ? 6 : 1) * px * sizeof(float);
}

template <typename T, int MAXP>
static hipError_t launch_adj(const BwArgs<T>& a, int64_t planes, int64_t n_o, hipStream_t stream,
                             Tracer* tr) {
  auto kern = bwd_adj<T, MAXP>;
  const size_t lds = static_cast<size_t>(2 * n_o) * sizeof(float);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  tr->before(stream, "bwd_adj", planes);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(planes)), dim3(kBwThreads), lds, stream, a);
  tr->after(stream);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_bwd_stream_dt(const BwdProblem& pr, void* ws, hipStream_t stream,
                                       Tracer* tr) {
  const int64_t planes = pr.B * pr.C;
  int dirs[4], nd = 0;
  for (int d = 0; d < 4; ++d)
    if ((pr.mask >> d) & 1u) dirs[nd++] = d;
  BwArgs<T> a;
  a.x = static_cast<const T*>(pr.x);
  a.l0 = static_cast<const T*>(pr.l[0]);
  a.l1 = static_cast<const T*>(pr.l[1]);
  a.l2 = static_cast<const T*>(pr.l[2]);
  a.lam = static_cast<const T*>(pr.lam);
  a.u = static_cast<const T*>(pr.u);
  a.gy = static_cast<const T*>(pr.gy);
  a.dx = static_cast<T*>(pr.dx);
  a.dl0 = static_cast<T*>(pr.dl[0]);
  a.dl1 = static_cast<T*>(pr.dl[1]);
  a.dl2 = static_cast<T*>(pr.dl[2]);
  a.dlam = static_cast<T*>(pr.dlam);
  a.du = static_cast<T*>(pr.du);
  a.pstride = planes * pr.H * pr.W;
  a.hbuf = static_cast<float*>(ws);
  a.acc = a.hbuf + a.pstride;
  a.H = static_cast<int>(pr.H);
  a.W = static_cast<int>(pr.W);
  a.G = static_cast<int>(pr.G);
  for (int i = 0; i < nd; ++i) {
    a.dir = dirs[i];
    a.mode = (i == 0 ? kBwFirst : 0) | (i == nd - 1 ? kBwLast : 0);
    const int64_t n_o = dirs[i] < 2 ? pr.W : pr.H;
    {
      auto kern = bwd_fwd<T>;
      const size_t lds = static_cast<size_t>(2 * n_o) * sizeof(float);
      if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(lds));
        if (e != hipSuccess) return e;
      }
      tr->before(stream, "bwd_fwd", planes);
      hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(planes)), dim3(kBwThreads), lds,
                         stream, a);
      tr->after(stream);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    hipError_t e;
    if (n_o <= kBwThreads)
      e = launch_adj<T, 1>(a, planes, n_o, stream, tr);
    else if (n_o <= 4 * kBwThreads)
      e = launch_adj<T, 4>(a, planes, n_o, stream, tr);
    else
      e = launch_adj<T, 16>(a, planes, n_o, stream, tr);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_bwd_stream(const BwdProblem& pr, void* ws, hipStream_t stream, Tracer* tr) {
  if (pr.dtype == GSPN_F32) return launch_bwd_stream_dt<float>(pr, ws, stream, tr);
  return launch_bwd_stream_dt<bf16_t>(pr, ws, stream, tr);
}

}  // namespace gspn

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
// Horizontal directions run in a transposed copy of the plane, where they are
// vertical scans and every access is coalesced: the seven inputs are
// transposed once (64 x 64 LDS tiles), left->right and right->left run as
// top->bottom and bottom->top there into transposed accumulators, and those
// are transposed back before the vertical directions add to them (or, with
// no vertical direction, a pointwise pass writes the gradients).
#include <cstring>

#include "gspn_device.hpp"
#include "gspn_launch.hpp"

namespace gspn {

namespace {
constexpr int kBwThreads = 1024;   // upper bound; a launch uses n_o rounded up to 64
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
  int64_t C, Cl;    // channels and logit channels (shared logits when Cl < C)
  float* dlw;       // shared logits: per-plane fp32 logit gradients [3][planes*H*W]
  // per-direction parameters: the output gate of this direction is scaled
  // per channel (merge weights; null: 1), and dx sums lambda d(lambda x)
  // over the directions in dxacc (fp32): the first direction writes it, the
  // last writes dx, the others add (dxacc null: dx = lambda d(lambda x))
  const float* gscale;
  float* dxacc;
  bool dxfirst, dxlast;
  // per-plane merge-gradient partials, sum over the plane of u gy h in fp64
  // (null: not wanted); only with first and last set
  double* dmpart;
  int64_t plane0;   // first plane of this launch (blockIdx.x counts from it)
};

// logit gradients of pixel idx: to the storage type, or per plane in fp32
// when logits are shared (summed over each group afterwards)
template <typename T>
__device__ __forceinline__ void put_dl(const BwArgs<T>& a, int64_t idx, float g0, float g1,
                                       float g2) {
  if (a.dlw) {
    a.dlw[idx] = g0;
    a.dlw[a.pstride + idx] = g1;
    a.dlw[2 * a.pstride + idx] = g2;
  } else {
    Store<T>::put(a.dl0, idx, g0);
    Store<T>::put(a.dl1, idx, g1);
    Store<T>::put(a.dl2, idx, g2);
  }
}

// Both scans keep every position's loads for D consecutive steps in flight
// together: all loads of a batch are issued first, unconditionally, at
// clamped in-bounds addresses, then the D steps are computed with one
// barrier each. (One workgroup per plane leaves few wavefronts per CU, so
// loads issued step by step would expose the full memory latency at every
// step.) MAXP bounds the orthogonal positions per thread
// (n_o <= MAXP * blockDim.x); MAXP * D stays small to fit the registers.

// forward scan of one direction: h into hbuf, and into the running sum of h
template <typename T, int MAXP, int D>
__global__ __launch_bounds__(kBwThreads) void bwd_fwd(BwArgs<T> a) {
  extern __shared__ float line[];   // [2][n_o]
  const int H = a.H, W = a.W, G = a.G, d = a.dir;
  const bool vert = d < 2, fwd = (d == 0 || d == 2);
  const int n_s = vert ? H : W, n_o = vert ? W : H;
  const int64_t plane = a.plane0 + blockIdx.x;
  const int64_t base = plane * H * W;
  const bool first = a.mode & kBwFirst, last = a.mode & kBwLast;
  const bool keep_sum = !(first && last);   // a single direction needs no running sum
  float* hsum = a.acc + 4 * a.pstride;
  const int64_t ls = logit_shift(plane, a.C, a.Cl, static_cast<int64_t>(H) * W);
  for (int s0 = 0; s0 < n_s; s0 += D) {
    float lx[D][MAXP], g0[D][MAXP], g1[D][MAXP], g2[D][MAXP], hs[D][MAXP];
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int s = min(s0 + j, n_s - 1);
      const int pos = fwd ? s : n_s - 1 - s;
#pragma unroll
      for (int i = 0; i < MAXP; ++i) {
        const int o = min(static_cast<int>(threadIdx.x + i * blockDim.x), n_o - 1);
        const int r = vert ? pos : o, c = vert ? o : pos;
        const int64_t idx = base + static_cast<int64_t>(r) * W + c;
        lx[j][i] = bl(a.lam, idx) * bl(a.x, idx);
        g0[j][i] = bl(a.l0, idx + ls);
        g1[j][i] = bl(a.l1, idx + ls);
        g2[j][i] = bl(a.l2, idx + ls);
        hs[j][i] = (keep_sum && !first) ? hsum[idx] : 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int s = s0 + j;
      if (s >= n_s) break;   // uniform
      const bool restart = restarts(s, n_s, G, fwd);
      const int pos = fwd ? s : n_s - 1 - s;
      float* cur = line + (s & 1) * n_o;
      const float* prev = line + ((s & 1) ^ 1) * n_o;
#pragma unroll
      for (int i = 0; i < MAXP; ++i) {
        const int o = threadIdx.x + i * blockDim.x;
        if (o < n_o) {
          const int r = vert ? pos : o, c = vert ? o : pos;
          const int64_t idx = base + static_cast<int64_t>(r) * W + c;
          float h = lx[j][i];
          if (!restart) {
            const Weights w = make_weights(g0[j][i], g1[j][i], g2[j][i], o > 0 ? 1.f : 0.f,
                                           o < n_o - 1 ? 1.f : 0.f);
            const float hl = prev[o > 0 ? o - 1 : 0];
            const float hr = prev[o < n_o - 1 ? o + 1 : o];
            h = __builtin_fmaf(w.w0, hl, __builtin_fmaf(w.w1, prev[o], __builtin_fmaf(w.w2, hr, h)));
          }
          cur[o] = h;
          a.hbuf[idx] = h;
          if (keep_sum) hsum[idx] = hs[j][i] + h;
        }
      }
      __syncthreads();
    }
  }
}

// reverse scan of the error term and the gradients of one direction.
// DB: the w_0 e / w_2 e line is double-buffered (one barrier per step);
// lines above 8192 positions use one buffer and two barriers per step.
template <typename T, int MAXP, int D, bool DB>
__global__ __launch_bounds__(kBwThreads) void bwd_adj(BwArgs<T> a) {
  // w_0 e and w_2 e of the line after this one in scan order,
  // [parity (DB only)][2][n_o]
  extern __shared__ float sm[];
  const int H = a.H, W = a.W, G = a.G, d = a.dir;
  const bool vert = d < 2, fwd = (d == 0 || d == 2);
  const int n_s = vert ? H : W, n_o = vert ? W : H;
  const int64_t plane = a.plane0 + blockIdx.x;
  const int64_t base = plane * H * W;
  const int64_t ps = a.pstride;
  const bool first = a.mode & kBwFirst, last = a.mode & kBwLast;
  // previous line in scan order sits one position back along the scan axis
  const int back = fwd ? -1 : 1;
  const int64_t back_off = vert ? static_cast<int64_t>(back) * W : back;
  const int64_t oo = vert ? 1 : W;   // orthogonal stride
  const int64_t lsh = logit_shift(plane, a.C, a.Cl, static_cast<int64_t>(H) * W);
  const float gsc = a.gscale ? a.gscale[plane % a.C] : 1.f;

  float a1[MAXP];
#pragma unroll
  for (int i = 0; i < MAXP; ++i) a1[i] = 0.f;
  double dm = 0.0;   // this thread's share of the merge-gradient partial
  for (int o = threadIdx.x; o < (DB ? 4 : 2) * n_o; o += blockDim.x) sm[o] = 0.f;
  __syncthreads();

  int par = 0;
  for (int s0 = n_s - 1; s0 >= 0; s0 -= D) {
    // ---- loads of D steps
    float gy[D][MAXP], ugp[D][MAXP], g0[D][MAXP], g1[D][MAXP], g2[D][MAXP];
    float hc[D][MAXP], hl[D][MAXP], hr[D][MAXP];
    float c0[D][MAXP], c1[D][MAXP], c2[D][MAXP], c3[D][MAXP];
    float xs[D][MAXP], ls[D][MAXP], hs[D][MAXP], dxa[D][MAXP];
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int s = max(s0 - j, 0);
      const bool restart = restarts(s, n_s, G, fwd);
      const int pos = fwd ? s : n_s - 1 - s;
#pragma unroll
      for (int i = 0; i < MAXP; ++i) {
        const int ot = static_cast<int>(threadIdx.x + i * blockDim.x);
        const int o = min(ot, n_o - 1);
        const int r = vert ? pos : o, c = vert ? o : pos;
        const int64_t idx = base + static_cast<int64_t>(r) * W + c;
        // a restart line has no previous line: its own position stands in
        const int64_t pidx = restart ? idx : idx + back_off;
        gy[j][i] = bl(a.gy, idx);
        ugp[j][i] = bl(a.u, idx) * gy[j][i];   // u gy
        g0[j][i] = bl(a.l0, idx + lsh);
        g1[j][i] = bl(a.l1, idx + lsh);
        g2[j][i] = bl(a.l2, idx + lsh);
        hc[j][i] = a.hbuf[pidx];
        hl[j][i] = a.hbuf[o > 0 ? pidx - oo : pidx];
        hr[j][i] = a.hbuf[o < n_o - 1 ? pidx + oo : pidx];
        if (!first) {
          c0[j][i] = a.acc[idx];
          c1[j][i] = a.acc[ps + idx];
          c2[j][i] = a.acc[2 * ps + idx];
          c3[j][i] = a.acc[3 * ps + idx];
        } else {
          c0[j][i] = 0.f; c1[j][i] = 0.f; c2[j][i] = 0.f; c3[j][i] = 0.f;
        }
        if (last) {
          xs[j][i] = bl(a.x, idx);
          ls[j][i] = bl(a.lam, idx);
          hs[j][i] = first ? a.hbuf[idx] : a.acc[4 * ps + idx];
          dxa[j][i] = (a.dxacc && !a.dxfirst) ? a.dxacc[idx] : 0.f;
        } else {
          xs[j][i] = 0.f; ls[j][i] = 0.f; hs[j][i] = 0.f; dxa[j][i] = 0.f;
        }
      }
    }
    // ---- D steps
    // merge-gradient products of this batch: at most D terms per position
    // summed in fp32, then added once to the fp64 total (fp64 arithmetic in
    // every step would lengthen each step, which the block waits for)
    float pm[MAXP];
#pragma unroll
    for (int i = 0; i < MAXP; ++i) pm[i] = 0.f;
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int s = s0 - j;
      if (s < 0) break;   // uniform
      const bool restart = restarts(s, n_s, G, fwd);
      const int pos = fwd ? s : n_s - 1 - s;
      const float* A0 = sm + (DB ? par * 2 * n_o : 0);
      const float* A2 = A0 + n_o;
      float* B0 = sm + (DB ? (par ^ 1) * 2 * n_o : 0);
      float* B2 = B0 + n_o;
      float st0[MAXP], st2[MAXP];
#pragma unroll
      for (int i = 0; i < MAXP; ++i) {
        const int o = threadIdx.x + i * blockDim.x;
        if (o < n_o) {
          const int r = vert ? pos : o, c = vert ? o : pos;
          const int64_t idx = base + static_cast<int64_t>(r) * W + c;
          float e = gsc * ugp[j][i] + a1[i];
          if (o + 1 < n_o) e += A0[o + 1];
          if (o > 0) e += A2[o - 1];
          float dl0 = 0.f, dl1 = 0.f, dl2 = 0.f, s0v = 0.f, s2v = 0.f, w1e = 0.f;
          if (!restart) {
            const float m0 = o > 0 ? 1.f : 0.f, m2 = o < n_o - 1 ? 1.f : 0.f;
            const WeightSlopes q = make_weight_slopes(g0[j][i], g1[j][i], g2[j][i], m0, m2);
            // h_k - p = sum_j w_j (h_k - h_j)
            const float d01 = hl[j][i] - hc[j][i], d12 = hc[j][i] - hr[j][i];
            const float d02 = hl[j][i] - hr[j][i];
            const float dev0 = q.w1 * d01 + q.w2 * d02;
            const float dev1 = q.w2 * d12 - q.w0 * d01;
            const float dev2 = -(q.w0 * d02 + q.w1 * d12);
            dl0 = e * q.q0 * dev0;
            dl1 = e * q.q1 * dev1;
            dl2 = e * q.q2 * dev2;
            s0v = q.w0 * e;
            s2v = q.w2 * e;
            w1e = q.w1 * e;
          }
          a1[i] = w1e;
          st0[i] = s0v;
          st2[i] = s2v;
          const float dphi = e + c0[j][i];
          dl0 += c1[j][i];
          dl1 += c2[j][i];
          dl2 += c3[j][i];
          if (last) {
            const float dxv = dxa[j][i] + ls[j][i] * dphi;
            if (!a.dxacc || a.dxlast)
              Store<T>::put(a.dx, idx, dxv);
            else
              a.dxacc[idx] = dxv;
            Store<T>::put(a.dlam, idx, xs[j][i] * dphi);
            put_dl(a, idx, dl0, dl1, dl2);
            Store<T>::put(a.du, idx, gsc * gy[j][i] * hs[j][i]);
            pm[i] = __builtin_fmaf(ugp[j][i], hs[j][i], pm[i]);
          } else {
            a.acc[idx] = dphi;
            a.acc[ps + idx] = dl0;
            a.acc[2 * ps + idx] = dl1;
            a.acc[3 * ps + idx] = dl2;
          }
        }
      }
      if (!DB) __syncthreads();   // every thread has read the line after
#pragma unroll
      for (int i = 0; i < MAXP; ++i) {
        const int o = threadIdx.x + i * blockDim.x;
        if (o < n_o) { B0[o] = st0[i]; B2[o] = st2[i]; }
      }
      par ^= 1;
      __syncthreads();
    }
    if (a.dmpart) {
#pragma unroll
      for (int i = 0; i < MAXP; ++i) dm += static_cast<double>(pm[i]);
    }
  }
  if (a.dmpart) {
    // a fixed tree: butterfly inside each wavefront, then the wavefronts in
    // order, so the partial does not depend on timing
    __shared__ double red[kBwThreads / 64];
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) dm += __shfl_xor(dm, m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = dm;
    __syncthreads();
    if (threadIdx.x == 0) {
      double t = 0.0;
      for (int k = 0; k < static_cast<int>(blockDim.x >> 6); ++k) t += red[k];
      a.dmpart[plane] = t;
    }
  }
}

// [n][R][C] -> [n][C][R] for up to seven tensors at once (blockIdx.y picks
// the tensor), through 64 x 64 LDS tiles; grid-stride over tiles
template <typename E>
struct TrArgs {
  const E* src[7];
  E* dst[7];
  int64_t n;
  int R, C;
};

template <typename E>
__global__ __launch_bounds__(256) void bwd_transpose(TrArgs<E> a) {
  __shared__ E tile[64][65];
  const E* src = a.src[blockIdx.y];
  E* dst = a.dst[blockIdx.y];
  const int R = a.R, C = a.C;
  const int tr = (R + 63) / 64, tc = (C + 63) / 64;
  const int64_t ntiles = a.n * tr * tc;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int64_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
    const int64_t p = t / (tr * tc);
    const int rem = static_cast<int>(t - p * tr * tc);
    const int r0 = (rem / tc) * 64, c0 = (rem % tc) * 64;
    const int64_t base = p * R * C;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int r = r0 + ty + 4 * k, c = c0 + tx;
      if (r < R && c < C) tile[ty + 4 * k][tx] = src[base + static_cast<int64_t>(r) * C + c];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int c = c0 + ty + 4 * k, r = r0 + tx;
      if (c < C && r < R) dst[base + static_cast<int64_t>(c) * R + r] = tile[tx][ty + 4 * k];
    }
    __syncthreads();
  }
}

// gradients from complete accumulators (no direction left to run)
template <typename T>
__global__ __launch_bounds__(256) void bwd_finish(BwArgs<T> a) {
  const int64_t ps = a.pstride;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < ps;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const float dphi = a.acc[i];
    Store<T>::put(a.dx, i, bl(a.lam, i) * dphi);
    Store<T>::put(a.dlam, i, bl(a.x, i) * dphi);
    put_dl(a, i, a.acc[ps + i], a.acc[2 * ps + i], a.acc[3 * ps + i]);
    Store<T>::put(a.du, i, bl(a.gy, i) * a.acc[4 * ps + i]);
  }
}

namespace {
size_t al256(size_t v) { return (v + 255) & ~size_t(255); }

// workspace regions (bytes from the start): forward states, accumulators,
// and for horizontal directions the transposed inputs and accumulators
struct BwLayout {
  size_t hbuf, acc, in_t, acc_t, total;
};

BwLayout bw_layout(int64_t planes, int64_t H, int64_t W, uint32_t mask, size_t es) {
  const size_t px = static_cast<size_t>(planes * H * W);
  const bool hz = mask & 12u;
  const bool accs = hz || __builtin_popcount(mask) > 1;
  BwLayout L;
  size_t o = 0;
  L.hbuf = o; o = al256(o + px * 4);
  L.acc = o; o = al256(o + (accs ? 5 * px * 4 : 0));
  L.in_t = o; o = al256(o + (hz ? 7 * px * es : 0));
  L.acc_t = o; o = al256(o + (hz ? 5 * px * 4 : 0));
  L.total = o;
  return L;
}
}  // namespace

size_t bwd_stream_workspace_bytes(int64_t planes, int64_t H, int64_t W, uint32_t mask,
                                  gspn_dtype dt) {
  return bw_layout(planes, H, W, mask, dt == GSPN_F32 ? 4 : 2).total;
}

static int bw_block(int64_t n_o) {
  const int64_t r = (n_o + 63) / 64 * 64;
  return static_cast<int>(r < kBwThreads ? r : kBwThreads);
}

template <typename T, int MAXP, int D, bool DB>
static hipError_t launch_pair(const BwArgs<T>& a, int64_t planes, int64_t n_o, hipStream_t stream,
                              Tracer* tr) {
  const int nb = bw_block(n_o);
  {
    auto kern = bwd_fwd<T, MAXP, D>;
    const size_t lds = static_cast<size_t>(2 * n_o) * sizeof(float);
    if (lds > 65536) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         static_cast<int>(lds));
      if (e != hipSuccess) return e;
    }
    tr->before(stream, "bwd_fwd", planes);
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(planes)), dim3(nb), lds, stream, a);
    tr->after(stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  auto kern = bwd_adj<T, MAXP, D, DB>;
  const size_t lds = static_cast<size_t>((DB ? 4 : 2) * n_o) * sizeof(float);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  tr->before(stream, "bwd_adj", planes);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(planes)), dim3(nb), lds, stream, a);
  tr->after(stream);
  return hipGetLastError();
}

// forward scan + reverse scan of scan direction d (0 top->bottom, 1
// bottom->top) over planes of a.H x a.W
template <typename T>
static hipError_t run_direction(BwArgs<T> a, int d, int mode, int64_t planes, hipStream_t stream,
                                Tracer* tr) {
  a.dir = d;
  a.mode = mode;
  const int64_t n_o = d < 2 ? a.W : a.H;
  const int nb = bw_block(n_o);
  if (n_o <= nb) return launch_pair<T, 1, 4, true>(a, planes, n_o, stream, tr);
  if (n_o <= 2 * nb) return launch_pair<T, 2, 2, true>(a, planes, n_o, stream, tr);
  if (n_o <= 4 * nb) return launch_pair<T, 4, 1, true>(a, planes, n_o, stream, tr);
  if (n_o <= 8 * nb) return launch_pair<T, 8, 1, true>(a, planes, n_o, stream, tr);
  return launch_pair<T, 16, 1, false>(a, planes, n_o, stream, tr);
}

template <typename E>
static hipError_t transpose(const E* const* src, E* const* dst, int count, int64_t n, int R, int C,
                            hipStream_t stream, Tracer* tr) {
  TrArgs<E> t;
  for (int i = 0; i < count; ++i) { t.src[i] = src[i]; t.dst[i] = dst[i]; }
  for (int i = count; i < 7; ++i) { t.src[i] = nullptr; t.dst[i] = nullptr; }
  t.n = n;
  t.R = R;
  t.C = C;
  const int64_t tiles = n * ((R + 63) / 64) * ((C + 63) / 64);
  const int64_t grid = tiles < (int64_t(1) << 20) ? tiles : (int64_t(1) << 20);
  tr->before(stream, "bwd_transpose", n);
  hipLaunchKernelGGL(bwd_transpose<E>, dim3(static_cast<unsigned>(grid), count), dim3(256), 0,
                     stream, t);
  tr->after(stream);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_bwd_stream_dt(const BwdProblem& pr, void* ws, hipStream_t stream,
                                       Tracer* tr) {
  const int64_t planes = pr.B * pr.C;
  const BwLayout lay = bw_layout(planes, pr.H, pr.W, pr.mask, sizeof(T));
  char* wsb = static_cast<char*>(ws);
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
  a.hbuf = reinterpret_cast<float*>(wsb + lay.hbuf);
  a.acc = reinterpret_cast<float*>(wsb + lay.acc);
  a.H = static_cast<int>(pr.H);
  a.W = static_cast<int>(pr.W);
  a.G = static_cast<int>(pr.G);
  a.C = pr.C;
  a.Cl = pr.Cl;
  a.dlw = pr.dlw;
  a.gscale = nullptr;
  a.dxacc = nullptr;
  a.dxfirst = a.dxlast = false;
  a.dmpart = nullptr;
  a.plane0 = 0;
  const bool t2b = pr.mask & 1u, b2t = pr.mask & 2u, l2r = pr.mask & 4u, r2l = pr.mask & 8u;
  hipError_t e;
  bool acc_written = false;
  if (l2r || r2l) {
    // transposed copies: left->right is top->bottom there, right->left is
    // bottom->top, and "up-left, up, up-right" keeps meaning rows r-1, r, r+1
    const T* src[7] = {a.x, a.l0, a.l1, a.l2, a.lam, a.u, a.gy};
    T* dst[7];
    T* in_t = reinterpret_cast<T*>(wsb + lay.in_t);
    for (int i = 0; i < 7; ++i) dst[i] = in_t + i * a.pstride;
    if (pr.Cl == pr.C) {
      if ((e = transpose<T>(src, dst, 7, planes, a.H, a.W, stream, tr)) != hipSuccess) return e;
    } else {
      // shared logits have B * Cl planes of their own
      const T* s4[4] = {a.x, a.lam, a.u, a.gy};
      T* d4[4] = {dst[0], dst[4], dst[5], dst[6]};
      if ((e = transpose<T>(s4, d4, 4, planes, a.H, a.W, stream, tr)) != hipSuccess) return e;
      if ((e = transpose<T>(src + 1, dst + 1, 3, pr.B * pr.Cl, a.H, a.W, stream, tr)) != hipSuccess)
        return e;
    }
    BwArgs<T> t = a;
    t.x = dst[0]; t.l0 = dst[1]; t.l1 = dst[2]; t.l2 = dst[3]; t.lam = dst[4]; t.u = dst[5];
    t.gy = dst[6];
    t.acc = reinterpret_cast<float*>(wsb + lay.acc_t);
    t.H = a.W;
    t.W = a.H;
    if (l2r && (e = run_direction(t, 0, kBwFirst, planes, stream, tr)) != hipSuccess) return e;
    if (r2l && (e = run_direction(t, 1, l2r ? 0 : kBwFirst, planes, stream, tr)) != hipSuccess)
      return e;
    // the five accumulators back to row-major ([5 planes][W][H] -> [H][W])
    const float* fs[1] = {t.acc};
    float* fd[1] = {a.acc};
    if ((e = transpose<float>(fs, fd, 1, 5 * planes, a.W, a.H, stream, tr)) != hipSuccess)
      return e;
    acc_written = true;
    if (!t2b && !b2t) {
      tr->before(stream, "bwd_finish", planes);
      const int64_t blocks = (a.pstride + 255) / 256;
      hipLaunchKernelGGL(bwd_finish<T>, dim3(static_cast<unsigned>(blocks < 65536 * 16 ? blocks : 65536 * 16)),
                         dim3(256), 0, stream, a);
      tr->after(stream);
      return hipGetLastError();
    }
  }
  if (t2b) {
    const int mode = (acc_written ? 0 : kBwFirst) | (b2t ? 0 : kBwLast);
    if ((e = run_direction(a, 0, mode, planes, stream, tr)) != hipSuccess) return e;
  }
  if (b2t) {
    const int mode = (acc_written || t2b ? 0 : kBwFirst) | kBwLast;
    if ((e = run_direction(a, 1, mode, planes, stream, tr)) != hipSuccess) return e;
  }
  return hipSuccess;
}

// shared logits: the gradient of logit plane (b, cl) at a pixel is the sum,
// in channel order, of the per-plane gradients of the C / Cl channels that
// read it
template <typename T>
__global__ __launch_bounds__(256) void bwd_reduce_logits(const float* dlw, T* d0, T* d1, T* d2,
                                                         int64_t B, int64_t C, int64_t Cl,
                                                         int64_t HW) {
  const int64_t n = B * Cl * HW, P = B * C * HW, g = C / Cl;
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t lp = i / HW, pix = i - lp * HW;
    const int64_t b = lp / Cl, cl = lp - b * Cl;
    const int64_t first = (b * C + cl * g) * HW + pix;
    float s0 = 0.f, s1 = 0.f, s2 = 0.f;
    for (int64_t c = 0; c < g; ++c) {
      const int64_t q = first + c * HW;
      s0 += dlw[q];
      s1 += dlw[P + q];
      s2 += dlw[2 * P + q];
    }
    Store<T>::put(d0, i, s0);
    Store<T>::put(d1, i, s1);
    Store<T>::put(d2, i, s2);
  }
}

template <typename T>
static hipError_t launch_reduce_dt(const BwdProblem& pr, hipStream_t stream, Tracer* tr) {
  const int64_t n = pr.B * pr.Cl * pr.H * pr.W;
  const int64_t blocks = (n + 255) / 256;
  const int64_t grid = blocks < 65536 * 16 ? blocks : 65536 * 16;
  tr->before(stream, "bwd_reduce_logits", pr.B * pr.Cl);
  hipLaunchKernelGGL(bwd_reduce_logits<T>, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream,
                     pr.dlw, static_cast<T*>(pr.dl[0]), static_cast<T*>(pr.dl[1]),
                     static_cast<T*>(pr.dl[2]), pr.B, pr.C, pr.Cl, pr.H * pr.W);
  tr->after(stream);
  return hipGetLastError();
}

hipError_t launch_bwd_reduce_logits(const BwdProblem& pr, hipStream_t stream, Tracer* tr) {
  if (pr.dtype == GSPN_F32) return launch_reduce_dt<float>(pr, stream, tr);
  return launch_reduce_dt<bf16_t>(pr, stream, tr);
}

hipError_t launch_bwd_stream(const BwdProblem& pr, void* ws, hipStream_t stream, Tracer* tr) {
  if (pr.dtype == GSPN_F32) return launch_bwd_stream_dt<float>(pr, ws, stream, tr);
  return launch_bwd_stream_dt<bf16_t>(pr, ws, stream, tr);
}

// ===========================================================================
// Per-direction parameters with a per-channel merger, backward. Direction d
// is one scan with its own lambda, logits and u (at element offset d *
// dir_stride), whose error term starts from merge[d][c] u gy; each direction
// runs the two launches above as a single direction (first and last), with
// its gradients written straight to its slice of the outputs, and
//   dx        = sum_d lambda_d d(lambda x)_d   (fp32 accumulator),
//   du_d      = merge[d][c] gy h_d,
//   dmerge[d][c] = sum over images and pixels of u_d gy h_d
// (the reverse scan, which holds u_d, gy and h_d at every pixel, leaves one
// fp64 partial per plane; a last launch sums the images in order).
// Horizontal directions run on transposed copies (x, gy and the direction's
// five tensors), their five gradients are transposed back, and their share
// of dx travels in a transposed accumulator; the transposes are the
// per-direction forward's (bf16 element pairs where the shapes allow).
// ===========================================================================
template <typename T>
__global__ __launch_bounds__(256) void bwd_dirs_zero(T* p, int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    Store<T>::put(p, i, 0.f);
}

template <typename T>
__global__ __launch_bounds__(256) void bwd_dirs_store_dx(const float* acc, T* dx, int64_t n) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    Store<T>::put(dx, i, acc[i]);
}

// merge gradients from the per-plane partials of each direction
// ([4][planes], fp64): one thread per (direction, channel) sums the images in
// order; directions outside the mask (and an empty batch) get zeros
__global__ __launch_bounds__(256) void bwd_dirs_merge(const double* part, int64_t B, int64_t C,
                                                      uint32_t mask, float* dmerge) {
  const int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x;
  if (i >= 4 * C) return;
  const int d = static_cast<int>(i / C);
  const int64_t c = i - d * C;
  double sum = 0.0;
  if (mask & (1u << d))
    for (int64_t b = 0; b < B; ++b) sum += part[d * B * C + b * C + c];
  dmerge[i] = static_cast<float>(sum);
}

namespace {
struct DirsLayout {
  size_t hbuf, dxacc, x_t, gy_t, par_t, out_t, dxacc_t, dmpart, total;
};

DirsLayout dirs_layout(int64_t planes, int64_t H, int64_t W, uint32_t mask, size_t es) {
  const size_t px = static_cast<size_t>(planes * H * W);
  const bool hz = mask & 12u;
  DirsLayout L;
  size_t o = 0;
  L.hbuf = o; o = al256(o + px * 4);
  L.dxacc = o; o = al256(o + px * 4);
  L.x_t = o; o = al256(o + (hz ? px * es : 0));
  L.gy_t = o; o = al256(o + (hz ? px * es : 0));
  L.par_t = o; o = al256(o + (hz ? 5 * px * es : 0));
  L.out_t = o; o = al256(o + (hz ? 5 * px * es : 0));
  L.dxacc_t = o; o = al256(o + (hz ? px * 4 : 0));
  L.dmpart = o; o = al256(o + static_cast<size_t>(4 * planes) * sizeof(double));
  L.total = o;
  return L;
}

int64_t fill_grid(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return b < 65536 * 16 ? (b > 0 ? b : 1) : 65536 * 16;
}
}  // namespace

size_t bwd_dirs_workspace_bytes(int64_t planes, int64_t H, int64_t W, uint32_t mask,
                                gspn_dtype dt) {
  return dirs_layout(planes, H, W, mask, dt == GSPN_F32 ? 4 : 2).total;
}

template <typename T>
static hipError_t launch_bwd_dirs_dt(const BwdProblem& pr, const BwdDirsExtra& ex, void* ws,
                                     hipStream_t stream, Tracer* tr) {
  const int64_t planes = pr.B * pr.C;
  const int64_t P = planes * pr.H * pr.W;
  const DirsLayout lay = dirs_layout(planes, pr.H, pr.W, pr.mask, sizeof(T));
  char* wsb = static_cast<char*>(ws);
  const int64_t ds = ex.dir_stride;
  const T* x = static_cast<const T*>(pr.x);
  const T* gy = static_cast<const T*>(pr.gy);
  const T* lam = static_cast<const T*>(pr.lam);
  const T* u = static_cast<const T*>(pr.u);
  const T* lg[3] = {static_cast<const T*>(pr.l[0]), static_cast<const T*>(pr.l[1]),
                    static_cast<const T*>(pr.l[2])};
  T* dx = static_cast<T*>(pr.dx);
  T* dlam = static_cast<T*>(pr.dlam);
  T* du = static_cast<T*>(pr.du);
  T* dl[3] = {static_cast<T*>(pr.dl[0]), static_cast<T*>(pr.dl[1]), static_cast<T*>(pr.dl[2])};
  float* hbuf = reinterpret_cast<float*>(wsb + lay.hbuf);
  float* dxacc = reinterpret_cast<float*>(wsb + lay.dxacc);
  hipError_t e;

  double* dmpart = reinterpret_cast<double*>(wsb + lay.dmpart);
  // the merge gradients from the partials of the selected directions (zeros
  // for the others and for an empty batch)
  auto merge_grad = [&]() -> hipError_t {
    if (!ex.dmerge || pr.C == 0) return hipSuccess;
    tr->before(stream, "bwd_dirs_merge", planes);
    hipLaunchKernelGGL(bwd_dirs_merge, dim3(static_cast<unsigned>((4 * pr.C + 255) / 256)),
                       dim3(256), 0, stream, dmpart, pr.B, pr.C, pr.mask, ex.dmerge);
    tr->after(stream);
    return hipGetLastError();
  };
  if (planes == 0) return merge_grad();

  // the order of the passes: horizontal first (their share of dx is
  // transposed back), then vertical
  const int order[4] = {2, 3, 0, 1};
  int first = -1, last = -1;
  for (int i = 0; i < 4; ++i)
    if (pr.mask & (1u << order[i])) {
      if (first < 0) first = order[i];
      last = order[i];
    }
  const bool vert_last = last == 0 || last == 1;

  // directions outside the mask: zero gradients
  for (int d = 0; d < 4; ++d) {
    if (pr.mask & (1u << d)) continue;
    T* outs[5] = {dlam + d * P, dl[0] + d * P, dl[1] + d * P, dl[2] + d * P, du + d * P};
    for (T* o : outs) {
      tr->before(stream, "bwd_dirs_zero", planes);
      hipLaunchKernelGGL(bwd_dirs_zero<T>, dim3(static_cast<unsigned>(fill_grid(P))), dim3(256), 0,
                         stream, o, P);
      tr->after(stream);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }

  BwArgs<T> base;
  std::memset(&base, 0, sizeof(base));
  base.pstride = P;
  base.hbuf = hbuf;
  base.acc = nullptr;
  base.G = static_cast<int>(pr.G);
  base.C = pr.C;
  base.Cl = pr.C;
  base.dlw = nullptr;

  const int64_t HW = pr.H * pr.W;
  const int H = static_cast<int>(pr.H), W = static_cast<int>(pr.W);
  T* x_t = reinterpret_cast<T*>(wsb + lay.x_t);
  T* gy_t = reinterpret_cast<T*>(wsb + lay.gy_t);
  T* par_t = reinterpret_cast<T*>(wsb + lay.par_t);
  T* out_t = reinterpret_cast<T*>(wsb + lay.out_t);
  float* dxacc_t = reinterpret_cast<float*>(wsb + lay.dxacc_t);

  // every launch of the chain for planes [p0, p0 + np) on stream st; planes
  // are independent throughout (their own slices of every buffer)
  auto run_group = [&](int64_t p0, int64_t np, hipStream_t st) -> hipError_t {
    hipError_t e;
    const int64_t o = p0 * HW;   // element offset of the group in a [planes][H][W] tensor
    if (pr.mask & 12u) {
      {
        const T* src[2] = {x + o, gy + o};
        T* dst[2] = {x_t + o, gy_t + o};
        if ((e = transpose_planes<T>(src, dst, 2, np, H, W, "bwd_dirs_tr", st, tr)) != hipSuccess)
          return e;
      }
      for (int d = 2; d < 4; ++d) {
        if (!(pr.mask & (1u << d))) continue;
        const T* src[5] = {lam + d * ds + o, lg[0] + d * ds + o, lg[1] + d * ds + o,
                           lg[2] + d * ds + o, u + d * ds + o};
        T* dst[5];
        for (int i = 0; i < 5; ++i) dst[i] = par_t + i * P + o;
        if ((e = transpose_planes<T>(src, dst, 5, np, H, W, "bwd_dirs_tr", st, tr)) != hipSuccess)
          return e;
        BwArgs<T> t = base;
        t.x = x_t;
        t.gy = gy_t;
        t.lam = par_t; t.l0 = par_t + P; t.l1 = par_t + 2 * P; t.l2 = par_t + 3 * P;
        t.u = par_t + 4 * P;
        t.dlam = out_t; t.dl0 = out_t + P; t.dl1 = out_t + 2 * P; t.dl2 = out_t + 3 * P;
        t.du = out_t + 4 * P;
        t.dx = nullptr;
        t.dxacc = dxacc_t;
        t.dxfirst = d == first;
        t.dxlast = false;
        t.gscale = ex.merge ? ex.merge + d * pr.C : nullptr;
        t.dmpart = ex.dmerge ? dmpart + d * planes : nullptr;
        t.plane0 = p0;
        t.H = W;
        t.W = H;
        if ((e = run_direction(t, d == 2 ? 0 : 1, kBwFirst | kBwLast, np, st, tr)) != hipSuccess)
          return e;
        // the five gradients back to row-major, into direction d's slices
        const T* bs[5] = {out_t + o, out_t + P + o, out_t + 2 * P + o, out_t + 3 * P + o,
                          out_t + 4 * P + o};
        T* bd[5] = {dlam + d * P + o, dl[0] + d * P + o, dl[1] + d * P + o, dl[2] + d * P + o,
                    du + d * P + o};
        if ((e = transpose_planes<T>(bs, bd, 5, np, W, H, "bwd_dirs_tr", st, tr)) != hipSuccess)
          return e;
      }
      const float* fs[1] = {dxacc_t + o};
      float* fd[1] = {dxacc + o};
      if ((e = transpose_planes<float>(fs, fd, 1, np, W, H, "bwd_dirs_tr_acc", st, tr)) !=
          hipSuccess)
        return e;
    }
    for (int d = 0; d < 2; ++d) {
      if (!(pr.mask & (1u << d))) continue;
      BwArgs<T> a = base;
      a.x = x;
      a.gy = gy;
      a.lam = lam + d * ds; a.l0 = lg[0] + d * ds; a.l1 = lg[1] + d * ds; a.l2 = lg[2] + d * ds;
      a.u = u + d * ds;
      a.dlam = dlam + d * P; a.dl0 = dl[0] + d * P; a.dl1 = dl[1] + d * P; a.dl2 = dl[2] + d * P;
      a.du = du + d * P;
      a.dx = dx;
      a.dxacc = dxacc;
      a.dxfirst = d == first;
      a.dxlast = d == last;
      a.gscale = ex.merge ? ex.merge + d * pr.C : nullptr;
      a.dmpart = ex.dmerge ? dmpart + d * planes : nullptr;
      a.plane0 = p0;
      a.H = H;
      a.W = W;
      if ((e = run_direction(a, d, kBwFirst | kBwLast, np, st, tr)) != hipSuccess) return e;
    }
    if (!vert_last) {
      tr->before(st, "bwd_dirs_store_dx", np);
      hipLaunchKernelGGL(bwd_dirs_store_dx<T>, dim3(static_cast<unsigned>(fill_grid(np * HW))),
                         dim3(256), 0, st, dxacc + o, dx + o, np * HW);
      tr->after(st);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
  };

  // A scan launch gives each plane one compute unit: plane groups on their
  // own streams let one group's tail overlap another group's next launch.
  if ((e = run_plane_groups(planes, stream, run_group)) != hipSuccess) return e;
  return merge_grad();
}

hipError_t launch_bwd_dirs(const BwdProblem& pr, const BwdDirsExtra& ex, void* ws,
                           hipStream_t stream, Tracer* tr) {
  if (pr.dtype == GSPN_F32) return launch_bwd_dirs_dt<float>(pr, ex, ws, stream, tr);
  return launch_bwd_dirs_dt<bf16_t>(pr, ex, ws, stream, tr);
}

}  // namespace gspn

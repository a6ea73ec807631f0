// Band-resident GSPN propagation for the local variant with small groups
// (1 <= G <= 16) on planes up to 512 x 512 whose vertical partial sum fits
// in LDS (H * W * 4 bytes <= 96 KiB).
//
// With local groups the scan restarts at every block of G positions, so each
// band of G rows is an independent problem for the two vertical directions,
// and each band of G columns for the two horizontal ones (CSDN page on GSPN,
// section GSPN模块的设计). One workgroup owns one plane:
//   phase V -- chain = (row band, column): the G rows of the chain are loaded
//              once (coalesced across columns), turned into records in
//              registers, scanned top->bottom and bottom->top with the
//              neighbour columns exchanged through a double-buffered LDS line;
//              y_V = h_T2B + h_B2T goes to an LDS plane;
//   phase H -- chain = (row, column band): the G columns of the chain are
//              loaded as one contiguous run (the plane was read moments ago,
//              so this mostly hits the last-level cache), scanned left->right
//              and right->left with neighbour rows through the LDS line, and
//              out = u * (y_V + h_L2R + h_R2L) is written once.
// Chains are processed in rounds of whole bands so that every chain's
// neighbours are in the same round.
//
// Line recurrence and output gate: same page, section 方法; tridiagonal
// row-normalised sigmoid weights and the four directions: section
// 如何设计一个高效的传播层.
#include "gspn_device.hpp"
#include "gspn_launch.hpp"

namespace gspn {

namespace {
constexpr int kBandMaxG = 16;
constexpr int kBandThreads = 512;
constexpr size_t kBandMaxYv = 96 * 1024;   // bytes of the vertical partial sum

__device__ __forceinline__ float bld(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float bld(const bf16_t* p, int64_t i) { return to_f32(p[i]); }
__device__ __forceinline__ void bst(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void bst(bf16_t* p, int64_t i, float v) {
  p[i].bits = static_cast<uint16_t>(f32_to_bf16_bits(v));
}
}  // namespace

template <typename T>
struct BandArgs {
  const T* x;
  const T* lam;
  const T* l0;
  const T* l1;
  const T* l2;
  const T* u;
  T* out;
  int64_t planes;
  int H, W, G;
  unsigned mask;
  int64_t C, Cl;    // channels and logit channels (shared logits when Cl < C)
};

// GM = compile-time bound on G (8 or 16); chains have min(G, rest) steps.
// VH: G == GM, W a multiple of GM and every tensor 16-byte aligned, so a
// horizontal chain's G columns are read and written as whole 16-byte vectors.
// The grid is persistent: a workgroup walks a list of rounds -- for each of
// its planes, the vertical rounds then the horizontal rounds -- and issues
// the loads of the next round as soon as the current one is done. With
// G <= 8 the register budget allows two workgroups per CU, whose rounds
// interleave and hide each other's load latency.
template <typename T, int GM, bool VH>
__global__ __launch_bounds__(kBandThreads, GM <= 8 ? 4 : 2) void band_kernel(BandArgs<T> a) {
  extern __shared__ float sm[];
  const int H = a.H, W = a.W, G = a.G;
  const int t = threadIdx.x;
  const bool tb = a.mask & 1u, bt = a.mask & 2u, lr = a.mask & 4u, rl = a.mask & 8u;
  const bool vert = tb || bt;
  const int nbv = (H + G - 1) / G, nbh = (W + G - 1) / G;
  const int pv = min(kBandThreads / W, nbv);   // row bands per vertical round
  const int ph = min(kBandThreads / H, nbh);   // column bands per horizontal round
  const int nrv = vert ? (nbv + pv - 1) / pv : 0;
  const int nrh = (nbh + ph - 1) / ph;
  // vertical partial sum [H][W + 1] (odd pitch: the horizontal phase reads it
  // with rows spread over the lanes), then the double-buffered line
  const int yp = W + 1;
  float* yv = sm;
  float* line = sm + H * yp;
  const int lw = W + 2;
  // line row per column band, padded to 8 (mod 32) words so that the eight
  // bands of a wavefront fall on different banks
  const int lh = H + 2 + ((8 - (H + 2) % 32) + 32) % 32;

  // this thread's chain in a vertical round (row band, column) ...
  const int vbl = t / W, vc = t % W;
  // ... and in a horizontal round (row, column band), column band fastest
  // across lanes so that the lanes of a row read adjacent runs
  const int hr = t / ph, hbl = t % ph;

  struct Loads {   // raw inputs of one chain, kept until the records are built
    float g0[GM], g1[GM], g2[GM], x[GM], l[GM];
  };
  struct Recs {
    float w0[GM], w1[GM], w2[GM], lx[GM];
  };
  // loads of round rd of plane p at clamped, always in-bounds addresses
  auto issue = [&](int64_t p, int rd, Loads& L) {
    const int64_t base = p * H * W;
    const int64_t ls = logit_shift(p, a.C, a.Cl, static_cast<int64_t>(H) * W);
    if (rd < nrv) {
      const int b = rd * pv + vbl;
      const int r0 = min(b, nbv - 1) * G;
#pragma unroll
      for (int s = 0; s < GM; ++s) {
        const int64_t i = base + static_cast<int64_t>(min(r0 + s, H - 1)) * W + vc;
        L.g0[s] = bld(a.l0, i + ls); L.g1[s] = bld(a.l1, i + ls); L.g2[s] = bld(a.l2, i + ls);
        L.x[s] = bld(a.x, i); L.l[s] = bld(a.lam, i);
      }
    } else {
      const int cb = (rd - nrv) * ph + hbl;
      const int c0 = min(cb, nbh - 1) * G;
      const int r = min(hr, H - 1);
      if constexpr (VH) {
        const int64_t i = base + static_cast<int64_t>(r) * W + c0;
        run_ld<GM>(a.l0, i + ls, L.g0); run_ld<GM>(a.l1, i + ls, L.g1); run_ld<GM>(a.l2, i + ls, L.g2);
        run_ld<GM>(a.x, i, L.x); run_ld<GM>(a.lam, i, L.l);
      } else {
#pragma unroll
        for (int s = 0; s < GM; ++s) {
          const int64_t i = base + static_cast<int64_t>(r) * W + min(c0 + s, W - 1);
          L.g0[s] = bld(a.l0, i + ls); L.g1[s] = bld(a.l1, i + ls); L.g2[s] = bld(a.l2, i + ls);
          L.x[s] = bld(a.x, i); L.l[s] = bld(a.lam, i);
        }
      }
    }
  };
  auto build = [&](const Loads& L, float m0, float m2, int len, Recs& R) {
#pragma unroll
    for (int s = 0; s < GM; ++s) {
      const Weights w = make_weights(L.g0[s], L.g1[s], L.g2[s], m0, m2);
      const bool in = s < len;
      R.w0[s] = in ? w.w0 : 0.f; R.w1[s] = in ? w.w1 : 0.f; R.w2[s] = in ? w.w2 : 0.f;
      R.lx[s] = in ? L.l[s] * L.x[s] : 0.f;
    }
  };

  // one chain of up to GM steps in both directions through the line buffer
  // (row stride `ls` words, position `li`); returns the per-step sums
  auto pair_scan = [&](const Recs& R, int len, bool act, int ls, int nb, int li, bool fwd_on,
                       bool rev_on, float hs[GM]) {
#pragma unroll
    for (int s = 0; s < GM; ++s) hs[s] = 0.f;
    for (int i = t; i < 2 * nb * ls; i += kBandThreads) line[i] = 0.f;
    __syncthreads();
    int par = 0;
    float h = 0.f;
    if (fwd_on) {   // restart at the band start
#pragma unroll
      for (int s = 0; s < GM; ++s) {
        if (s < G) {
          const float* pvv = line + par * nb * ls;
          h = s == 0 ? R.lx[s]
                     : __builtin_fmaf(R.w0[s], pvv[li - 1],
                           __builtin_fmaf(R.w1[s], h, __builtin_fmaf(R.w2[s], pvv[li + 1], R.lx[s])));
          if (act) line[(par ^ 1) * nb * ls + li] = h;
          par ^= 1;
          hs[s] = h;
          __syncthreads();
        }
      }
    }
    if (rev_on) {   // restart at the last position of the band
      h = 0.f;
#pragma unroll
      for (int s = GM - 1; s >= 0; --s) {
        if (s < G) {
          const float* pvv = line + par * nb * ls;
          const float nh = s == len - 1 ? R.lx[s]
                                        : __builtin_fmaf(R.w0[s], pvv[li - 1],
                                              __builtin_fmaf(R.w1[s], h,
                                                  __builtin_fmaf(R.w2[s], pvv[li + 1], R.lx[s])));
          // positions past the end of a short last band keep the state at 0
          h = s < len ? nh : 0.f;
          if (act) line[(par ^ 1) * nb * ls + li] = h;
          par ^= 1;
          hs[s] += h;
          __syncthreads();
        }
      }
    }
  };

  const int64_t planes = a.planes;
  const int nrounds = nrv + nrh;
  int64_t p = blockIdx.x;
  int rd = 0;
  Loads L;
  if (p < planes) issue(p, 0, L);
  while (p < planes) {
    int rd2 = rd + 1;
    int64_t p2 = p;
    if (rd2 == nrounds) { rd2 = 0; p2 += gridDim.x; }
    const int64_t base = p * H * W;
    float hs[GM];
    Recs R;
    if (rd < nrv) {
      // vertical round: chains (row band, column)
      const int b = rd * pv + vbl;
      const bool act = vbl < pv && b < nbv;
      const int r0 = min(b, nbv - 1) * G;
      const int len = act ? min(G, H - r0) : 0;
      build(L, vc > 0 ? 1.f : 0.f, vc < W - 1 ? 1.f : 0.f, len, R);
      // idle threads read a pad slot of band 0 and write nothing
      pair_scan(R, len, act, lw, pv, act ? vbl * lw + vc + 1 : 1, tb, bt, hs);
#pragma unroll
      for (int s = 0; s < GM; ++s)
        if (act && s < len) yv[(r0 + s) * yp + vc] = hs[s];
    } else {
      // horizontal round: chains (row, column band); writes out
      const int cb = (rd - nrv) * ph + hbl;
      const bool act = hr < H && cb < nbh && hbl < ph;
      const int c0 = min(cb, nbh - 1) * G;
      const int len = act ? min(G, W - c0) : 0;
      const int r = min(hr, H - 1);
      build(L, r > 0 ? 1.f : 0.f, r < H - 1 ? 1.f : 0.f, len, R);
      // u is needed only after the scans: its loads fly during them
      const int64_t row = base + static_cast<int64_t>(r) * W;
      float uu[GM];
      if constexpr (VH) {
        run_ld<GM>(a.u, row + c0, uu);
      } else {
#pragma unroll
        for (int s = 0; s < GM; ++s) uu[s] = bld(a.u, row + min(c0 + s, W - 1));
      }
      pair_scan(R, len, act, lh, ph, act ? hbl * lh + r + 1 : 1, lr, rl, hs);
      if constexpr (VH) {
        if (act) {
#pragma unroll
          for (int s = 0; s < GM; ++s) hs[s] = uu[s] * ((vert ? yv[r * yp + c0 + s] : 0.f) + hs[s]);
          run_st<GM>(a.out, row + c0, hs);
        }
      } else {
#pragma unroll
        for (int s = 0; s < GM; ++s) {
          if (act && s < len) {
            const int c = c0 + s;
            const float yvv = vert ? yv[r * yp + c] : 0.f;
            bst(a.out, row + c, uu[s] * (yvv + hs[s]));
          }
        }
      }
    }
    if (p2 < planes) issue(p2, rd2, L);
    __syncthreads();   // line and y_V are rewritten by the next round
    p = p2;
    rd = rd2;
  }
}

size_t band_lds_bytes(int64_t H, int64_t W, int64_t G) {
  // y_V plane (row pitch W + 1) plus the double-buffered line: per round at
  // most min(1024 / W, row bands) bands of W + 2 words, or
  // min(1024 / H, column bands) bands of at most H + 33 words
  const int64_t nbv = (H + G - 1) / G, nbh = (W + G - 1) / G;
  const int64_t pv = kBandThreads / W < nbv ? kBandThreads / W : nbv;
  const int64_t ph = kBandThreads / H < nbh ? kBandThreads / H : nbh;
  const int64_t lv = pv * (W + 2), lhz = ph * (H + 33);
  const int64_t line = 2 * (lv > lhz ? lv : lhz);
  return static_cast<size_t>(H * (W + 1) + line) * sizeof(float);
}

bool band_fits(int64_t H, int64_t W, int64_t G) {
  return G >= 1 && G <= kBandMaxG && G < (H > W ? H : W) && H <= kBandThreads && W <= kBandThreads &&
         static_cast<size_t>(H * (W + 1)) * 4 <= kBandMaxYv &&
         band_lds_bytes(H, W, G) <= 160 * 1024;
}

template <typename T, int GM, bool VH>
static hipError_t launch_band_t(const Problem& pr, hipStream_t stream, Tracer* tr) {
  BandArgs<T> a;
  a.x = static_cast<const T*>(pr.x);
  a.lam = static_cast<const T*>(pr.lam);
  a.l0 = static_cast<const T*>(pr.l[0]);
  a.l1 = static_cast<const T*>(pr.l[1]);
  a.l2 = static_cast<const T*>(pr.l[2]);
  a.u = static_cast<const T*>(pr.u);
  a.out = static_cast<T*>(pr.out);
  a.H = static_cast<int>(pr.H);
  a.W = static_cast<int>(pr.W);
  a.G = static_cast<int>(pr.G);
  a.mask = pr.mask;
  a.C = pr.C;
  a.Cl = pr.Cl;
  const size_t lds = band_lds_bytes(pr.H, pr.W, pr.G);
  auto kern = band_kernel<T, GM, VH>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  const int64_t planes = pr.B * pr.C;
  a.planes = planes;
  // persistent grid: as many workgroups as are resident at once
  int per_cu = 0, dev = 0, cus = 0;
  hipError_t e;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern),
                                                        kBandThreads, lds)) != hipSuccess)
    return e;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
    return e;
  const int64_t resident = static_cast<int64_t>(per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
  const int64_t grid = planes < resident ? planes : resident;
  tr->before(stream, "band_kernel", planes);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(kBandThreads), lds, stream, a);
  tr->after(stream);
  return hipGetLastError();
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <typename T>
static hipError_t launch_band_dt(const Problem& pr, hipStream_t stream, Tracer* tr) {
  const int gm = pr.G <= 8 ? 8 : 16;
  const bool vh = pr.G == gm && pr.W % gm == 0 && aligned16(pr.x) && aligned16(pr.lam) &&
                  aligned16(pr.l[0]) && aligned16(pr.l[1]) && aligned16(pr.l[2]) &&
                  aligned16(pr.u) && aligned16(pr.out);
  if (gm == 8)
    return vh ? launch_band_t<T, 8, true>(pr, stream, tr) : launch_band_t<T, 8, false>(pr, stream, tr);
  return vh ? launch_band_t<T, 16, true>(pr, stream, tr) : launch_band_t<T, 16, false>(pr, stream, tr);
}

hipError_t launch_band(const Problem& pr, hipStream_t stream, Tracer* tr) {
  return pr.dtype == GSPN_F32 ? launch_band_dt<float>(pr, stream, tr)
                              : launch_band_dt<bf16_t>(pr, stream, tr);
}

}  // namespace gspn

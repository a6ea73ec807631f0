// Backward pass for the local variant with small groups (1 <= G <= 8) on
// planes up to 512 x 512: the counterpart of the band-resident forward plan.
//
// With local groups every band of G rows is an independent problem for the
// vertical directions and every band of G columns for the horizontal ones
// (CSDN page on GSPN, section GSPN模块的设计), so a chain is at most 8 steps
// long and lives in registers. One workgroup walks a plane's rounds:
//   vertical rounds   -- chain = (row band, column): load the chain's seven
//     inputs, build its weights, run the forward scan of one direction
//     (recording each step's state and the two neighbours' previous states,
//     which the scan reads from the LDS line anyway), run the reverse scan of
//     the error term (section 反向传播):
//        e_s[o] = u gy + w_{s+1,0}[o+1] e_{s+1}[o+1] + w_{s+1,1}[o] e_{s+1}[o]
//                      + w_{s+1,2}[o-1] e_{s+1}[o-1]
//     with the next line's w_0 e and w_2 e through the LDS line, and form the
//     logit gradients e w_k (1 - sigmoid(l_k)) (h_prev[o+k-1] - p); then the
//     same for the other vertical direction. The vertical sums of e, of the
//     three logit gradients and of h go to an fp32 workspace;
//   horizontal rounds -- chain = (row, column band): the same for the two
//     horizontal directions, then the six gradients
//        grad_x = lambda sum e, grad_lambda = x sum e, grad_l_k = sum dl_k,
//        grad_u = gy sum h
//     are written once. Without horizontal directions the vertical rounds
//     write the gradients themselves; without vertical ones the workspace is
//     not used.
#include "gspn_device.hpp"
#include "gspn_launch.hpp"

namespace gspn {

namespace {
constexpr int kBbThreads = 512;
constexpr int kBbG = 8;   // chain bound

__host__ __device__ constexpr int bband_row(int64_t n) {
  return static_cast<int>(n + 2 + ((8 - (n + 2) % 32) + 32) % 32);
}

__device__ __forceinline__ float bb_ld(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float bb_ld(const bf16_t* p, int64_t i) { return to_f32(p[i]); }
}  // namespace

template <typename T>
struct BBandArgs {
  const T* x;
  const T* lam;
  const T* l0;
  const T* l1;
  const T* l2;
  const T* u;
  const T* gy;
  T* dx;
  T* dl0;
  T* dl1;
  T* dl2;
  T* dlam;
  T* du;
  float* part;      // [5][planes][H][W]: vertical sums of e, dl0, dl1, dl2, h
  int64_t pstride;  // planes * H * W
  int64_t planes;
  int H, W, G;
  unsigned mask;
  int64_t C, Cl;    // channels and logit channels (shared logits when Cl < C)
  float* dlw;       // shared logits: per-plane fp32 logit gradients [3][planes*H*W]
};

// VH: G == 8, W a multiple of 8 and every tensor 16-byte aligned, so a
// horizontal chain's eight columns move as whole 16-byte vectors (one
// instruction covers a row's cache line; scalar column accesses spread over
// eight instructions lose their lines from L2 in between).
template <typename T, bool VH>
__global__ __launch_bounds__(kBbThreads) void bband_kernel(BBandArgs<T> a) {
  constexpr int GM = kBbG;
  extern __shared__ float line[];
  const int H = a.H, W = a.W, G = a.G;
  const int t = threadIdx.x;
  const bool tb = a.mask & 1u, bt = a.mask & 2u, lr = a.mask & 4u, rl = a.mask & 8u;
  const bool vert = tb || bt, horz = lr || rl;
  const int nbv = (H + G - 1) / G, nbh = (W + G - 1) / G;
  const int pv = min(kBbThreads / W, nbv);   // row bands per vertical round
  const int ph = min(kBbThreads / H, nbh);   // column bands per horizontal round
  const int nrv = vert ? (nbv + pv - 1) / pv : 0;
  const int nrh = horz ? (nbh + ph - 1) / ph : 0;
  const int64_t ps = a.pstride;

  // line buffers: [2 parities][2 arrays][bands][row stride]; a band row holds
  // the orthogonal positions with one zero pad on each side
  // (horizontal band rows padded to 8 mod 32 words so that the bands a
  // wavefront spans fall on different LDS banks)
  const int lw = W + 2, lh = bband_row(H);
  const int vbl = t / W, vc = t % W;           // vertical chain (row band, column)
  const int hr = t / ph, hbl = t % ph;         // horizontal chain (row, column band)

  for (int64_t p = blockIdx.x; p < a.planes; p += gridDim.x) {
    const int64_t base = p * H * W;
    const int64_t lsh = logit_shift(p, a.C, a.Cl, static_cast<int64_t>(H) * W);
    for (int rd = 0; rd < nrv + nrh; ++rd) {
      const bool vround = rd < nrv;
      int len, ls, nb, li, o, n_o;
      bool act;
      int64_t gi0, gstride;   // global index of chain position 0, step stride
      if (vround) {
        const int b = rd * pv + vbl;
        act = vbl < pv && b < nbv;
        const int r0 = min(b, nbv - 1) * G;
        len = act ? min(G, H - r0) : 0;
        ls = lw; nb = pv; li = vbl * lw + vc + 1; o = vc; n_o = W;
        gi0 = base + static_cast<int64_t>(r0) * W + vc;
        gstride = W;
      } else {
        const int cb = (rd - nrv) * ph + hbl;
        act = hr < H && cb < nbh && hbl < ph;
        const int c0 = min(cb, nbh - 1) * G;
        const int r = min(hr, H - 1);
        len = act ? min(G, W - c0) : 0;
        ls = lh; nb = ph; li = hbl * lh + r + 1; o = r; n_o = H;
        gi0 = base + static_cast<int64_t>(r) * W + c0;
        gstride = 1;
      }
      const int lsz = nb * ls;
      if (!act) li = 1;   // idle threads read a pad slot and write nothing
      // inputs of the chain: every load unconditional at a clamped, in-bounds
      // address (a guarded load would make the compiler drain the memory
      // queue at each guard); positions past the chain are masked afterwards
      float w0[GM], w1[GM], w2[GM], q0[GM], q1[GM], q2[GM], lx[GM], ug[GM];
      const float m0 = o > 0 ? 1.f : 0.f, m2 = o < n_o - 1 ? 1.f : 0.f;
      {
        float vl0[GM], vl1[GM], vl2[GM], vlam[GM], vx[GM], vu[GM], vgy[GM];
        if (VH && !vround) {
          run_ld<GM>(a.l0, gi0 + lsh, vl0); run_ld<GM>(a.l1, gi0 + lsh, vl1);
          run_ld<GM>(a.l2, gi0 + lsh, vl2);
          run_ld<GM>(a.lam, gi0, vlam); run_ld<GM>(a.x, gi0, vx);
          run_ld<GM>(a.u, gi0, vu); run_ld<GM>(a.gy, gi0, vgy);
        } else {
#pragma unroll
          for (int s = 0; s < GM; ++s) {
            const int64_t i = gi0 + min(s, max(len - 1, 0)) * gstride;
            vl0[s] = bb_ld(a.l0, i + lsh); vl1[s] = bb_ld(a.l1, i + lsh); vl2[s] = bb_ld(a.l2, i + lsh);
            vlam[s] = bb_ld(a.lam, i); vx[s] = bb_ld(a.x, i);
            vu[s] = bb_ld(a.u, i); vgy[s] = bb_ld(a.gy, i);
          }
        }
#pragma unroll
        for (int s = 0; s < GM; ++s) {
          const WeightSlopes q = make_weight_slopes(vl0[s], vl1[s], vl2[s], m0, m2);
          const bool in = s < len;
          w0[s] = in ? q.w0 : 0.f; w1[s] = in ? q.w1 : 0.f; w2[s] = in ? q.w2 : 0.f;
          q0[s] = q.q0; q1[s] = q.q1; q2[s] = q.q2;
          lx[s] = in ? vlam[s] * vx[s] : 0.f;
          ug[s] = in ? vu[s] * vgy[s] : 0.f;
        }
      }
      // sums over this round's two directions
      float se[GM], sh[GM], g0[GM], g1[GM], g2[GM];
#pragma unroll
      for (int s = 0; s < GM; ++s) { se[s] = 0.f; sh[s] = 0.f; g0[s] = 0.f; g1[s] = 0.f; g2[s] = 0.f; }

      for (int dir = 0; dir < 2; ++dir) {
        const bool on = vround ? (dir == 0 ? tb : bt) : (dir == 0 ? lr : rl);
        if (!on) continue;
        const bool asc = dir == 0;   // top->bottom / left->right walk s upwards
        float h[GM], hl[GM], hr_[GM];
        // ---- forward scan: restart at the band's first position in scan order
        for (int i = t; i < 4 * lsz; i += kBbThreads) line[i] = 0.f;
        __syncthreads();
        {
          int par = 0;
          float hc = 0.f;
#pragma unroll
          for (int k = 0; k < GM; ++k) {
            const int s = asc ? k : GM - 1 - k;
            if (s < G) {   // uniform: positions past G are never part of a chain
              const float* pv_ = line + par * lsz;
              const bool first = asc ? s == 0 : s == len - 1;
              const float l_ = pv_[li - 1], r_ = pv_[li + 1];
              const float hn = __builtin_fmaf(w0[s], l_, __builtin_fmaf(w1[s], hc,
                                   __builtin_fmaf(w2[s], r_, lx[s])));
              // positions past the end of a short band keep state 0
              const float hv = s < len ? (first ? lx[s] : hn) : 0.f;
              hl[s] = l_; hr_[s] = r_;
              h[s] = hv;
              hc = hv;
              if (act) line[(par ^ 1) * lsz + li] = hv;
              par ^= 1;
              __syncthreads();
            }
          }
        }
        // ---- reverse scan of the error term, with this direction's gradients
        // formed at each step (e, the step's weights and the recorded
        // previous states are all at hand there)
        for (int i = t; i < 4 * lsz; i += kBbThreads) line[i] = 0.f;
        __syncthreads();
        {
          int par = 0;
          float p1 = 0.f;   // w_1 e of the line after this one (same position)
#pragma unroll
          for (int k = 0; k < GM; ++k) {
            const int s = asc ? GM - 1 - k : k;
            if (s < G) {
              const float* A0 = line + par * 2 * lsz;
              const float* A2 = A0 + lsz;
              const float ev = s < len ? ug[s] + A0[li + 1] + p1 + A2[li - 1] : 0.f;
              // the band's first line in scan order reads nothing before it
              const bool first = asc ? s == 0 : s == len - 1;
              const float s0 = first ? 0.f : w0[s] * ev, s2 = first ? 0.f : w2[s] * ev;
              p1 = first ? 0.f : w1[s] * ev;
              if (act) {
                float* B0 = line + (par ^ 1) * 2 * lsz;
                B0[li] = s0;
                B0[lsz + li] = s2;
              }
              se[s] += ev;
              sh[s] += h[s];
              if (!first) {
                // previous line in scan order: s - 1 (ascending) or s + 1
                const int sp = asc ? (s > 0 ? s - 1 : 0) : (s + 1 < GM ? s + 1 : GM - 1);
                const float hc = h[sp];
                // h_k - p = sum_j w_j (h_k - h_j); q_k = w_k (1 - sigmoid(l_k))
                const float d01 = hl[s] - hc, d12 = hc - hr_[s], d02 = hl[s] - hr_[s];
                const float dev0 = w1[s] * d01 + w2[s] * d02;
                const float dev1 = w2[s] * d12 - w0[s] * d01;
                const float dev2 = -(w0[s] * d02 + w1[s] * d12);
                g0[s] = __builtin_fmaf(ev * q0[s], dev0, g0[s]);
                g1[s] = __builtin_fmaf(ev * q1[s], dev1, g1[s]);
                g2[s] = __builtin_fmaf(ev * q2[s], dev2, g2[s]);
              }
              par ^= 1;
              __syncthreads();
            }
          }
        }
      }

      // ---- hand over or write
      const bool final_round = !vround || !horz;
      // loads of this step, all unconditional at clamped addresses (after the
      // last barrier of the scans, so they do not stay live through them)
      float xs[GM], lams[GM], gys[GM];
      float pe[GM], p0[GM], p1_[GM], p2[GM], psum[GM];
      const bool take_part = !vround && vert;   // uniform
      if (VH && !vround) {
        // horizontal round: final, and every chain has G = 8 positions
        run_ld<GM>(a.x, gi0, xs); run_ld<GM>(a.lam, gi0, lams); run_ld<GM>(a.gy, gi0, gys);
        if (take_part) {
          run_ld<GM>(a.part, gi0, pe); run_ld<GM>(a.part + ps, gi0, p0);
          run_ld<GM>(a.part + 2 * ps, gi0, p1_); run_ld<GM>(a.part + 3 * ps, gi0, p2);
          run_ld<GM>(a.part + 4 * ps, gi0, psum);
        } else {
#pragma unroll
          for (int s = 0; s < GM; ++s) { pe[s] = 0.f; p0[s] = 0.f; p1_[s] = 0.f; p2[s] = 0.f; psum[s] = 0.f; }
        }
      } else {
#pragma unroll
        for (int s = 0; s < GM; ++s) {
          const int64_t i = gi0 + min(s, max(len - 1, 0)) * gstride;
          if (final_round) {
            xs[s] = bb_ld(a.x, i);
            lams[s] = bb_ld(a.lam, i);
            gys[s] = bb_ld(a.gy, i);
          }
          if (take_part) {
            pe[s] = a.part[i];
            p0[s] = a.part[ps + i];
            p1_[s] = a.part[2 * ps + i];
            p2[s] = a.part[3 * ps + i];
            psum[s] = a.part[4 * ps + i];
          } else {
            pe[s] = 0.f; p0[s] = 0.f; p1_[s] = 0.f; p2[s] = 0.f; psum[s] = 0.f;
          }
        }
      }
      if (VH && !vround) {
        if (act) {
          float o6[6][GM];
#pragma unroll
          for (int s = 0; s < GM; ++s) {
            const float te = se[s] + pe[s], th = sh[s] + psum[s];
            o6[0][s] = lams[s] * te;
            o6[1][s] = g0[s] + p0[s];
            o6[2][s] = g1[s] + p1_[s];
            o6[3][s] = g2[s] + p2[s];
            o6[4][s] = xs[s] * te;
            o6[5][s] = gys[s] * th;
          }
          run_st<GM>(a.dx, gi0, o6[0]);
          if (a.dlw) {
            run_st<GM>(a.dlw, gi0, o6[1]); run_st<GM>(a.dlw + ps, gi0, o6[2]);
            run_st<GM>(a.dlw + 2 * ps, gi0, o6[3]);
          } else {
            run_st<GM>(a.dl0, gi0, o6[1]); run_st<GM>(a.dl1, gi0, o6[2]);
            run_st<GM>(a.dl2, gi0, o6[3]);
          }
          run_st<GM>(a.dlam, gi0, o6[4]); run_st<GM>(a.du, gi0, o6[5]);
        }
        __syncthreads();   // the line is cleared by the next round
        continue;
      }
#pragma unroll
      for (int s = 0; s < GM; ++s) {
        if (act && s < len) {
          const int64_t i = gi0 + s * gstride;
          const float te = se[s] + pe[s], th = sh[s] + psum[s];
          const float t0 = g0[s] + p0[s], t1 = g1[s] + p1_[s], t2 = g2[s] + p2[s];
          if (final_round) {
            Store<T>::put(a.dx, i, lams[s] * te);
            Store<T>::put(a.dlam, i, xs[s] * te);
            if (a.dlw) {
              a.dlw[i] = t0;
              a.dlw[ps + i] = t1;
              a.dlw[2 * ps + i] = t2;
            } else {
              Store<T>::put(a.dl0, i, t0);
              Store<T>::put(a.dl1, i, t1);
              Store<T>::put(a.dl2, i, t2);
            }
            Store<T>::put(a.du, i, gys[s] * th);
          } else {
            a.part[i] = te;
            a.part[ps + i] = t0;
            a.part[2 * ps + i] = t1;
            a.part[3 * ps + i] = t2;
            a.part[4 * ps + i] = th;
          }
        }
      }
      __syncthreads();   // the line is cleared by the next round
    }
  }
}

bool bband_fits(int64_t H, int64_t W, int64_t G) {
  return G >= 1 && G <= kBbG && G < (H > W ? H : W) && H <= kBbThreads && W <= kBbThreads;
}

size_t bband_workspace_bytes(int64_t planes, int64_t H, int64_t W, uint32_t mask) {
  const bool both = (mask & 3u) && (mask & 12u);
  return both ? static_cast<size_t>(5 * planes * H * W) * sizeof(float) : 0;
}

template <typename T, bool VH>
static hipError_t launch_bband_t(const BwdProblem& pr, void* ws, hipStream_t stream, Tracer* tr) {
  BBandArgs<T> a;
  a.x = static_cast<const T*>(pr.x);
  a.lam = static_cast<const T*>(pr.lam);
  a.l0 = static_cast<const T*>(pr.l[0]);
  a.l1 = static_cast<const T*>(pr.l[1]);
  a.l2 = static_cast<const T*>(pr.l[2]);
  a.u = static_cast<const T*>(pr.u);
  a.gy = static_cast<const T*>(pr.gy);
  a.dx = static_cast<T*>(pr.dx);
  a.dl0 = static_cast<T*>(pr.dl[0]);
  a.dl1 = static_cast<T*>(pr.dl[1]);
  a.dl2 = static_cast<T*>(pr.dl[2]);
  a.dlam = static_cast<T*>(pr.dlam);
  a.du = static_cast<T*>(pr.du);
  a.part = static_cast<float*>(ws);
  a.planes = pr.B * pr.C;
  a.pstride = a.planes * pr.H * pr.W;
  a.H = static_cast<int>(pr.H);
  a.W = static_cast<int>(pr.W);
  a.G = static_cast<int>(pr.G);
  a.mask = pr.mask;
  a.C = pr.C;
  a.Cl = pr.Cl;
  a.dlw = pr.dlw;
  // four line arrays per round: at most kBbThreads / n_o bands of n_o + 2
  const int64_t nbv = (pr.H + pr.G - 1) / pr.G, nbh = (pr.W + pr.G - 1) / pr.G;
  const int64_t pv = kBbThreads / pr.W < nbv ? kBbThreads / pr.W : nbv;
  const int64_t ph = kBbThreads / pr.H < nbh ? kBbThreads / pr.H : nbh;
  const int64_t lv = pv * (pr.W + 2), lhz = ph * bband_row(pr.H);
  const size_t lds = static_cast<size_t>(4 * (lv > lhz ? lv : lhz)) * sizeof(float);
  auto kern = bband_kernel<T, VH>;
  int per_cu = 0, dev = 0, cus = 0;
  hipError_t e;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern),
                                                        kBbThreads, lds)) != hipSuccess)
    return e;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
    return e;
  const int64_t resident = static_cast<int64_t>(per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
  const int64_t grid = a.planes < resident ? a.planes : resident;
  tr->before(stream, "bband_kernel", a.planes);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(kBbThreads), lds, stream, a);
  tr->after(stream);
  return hipGetLastError();
}

static bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

template <typename T>
static hipError_t launch_bband_dt(const BwdProblem& pr, void* ws, hipStream_t stream, Tracer* tr) {
  const bool vh = pr.G == kBbG && pr.W % kBbG == 0 && al16(pr.x) && al16(pr.lam) &&
                  al16(pr.l[0]) && al16(pr.l[1]) && al16(pr.l[2]) && al16(pr.u) &&
                  al16(pr.gy) && al16(pr.dx) && al16(pr.dl[0]) && al16(pr.dl[1]) &&
                  al16(pr.dl[2]) && al16(pr.dlam) && al16(pr.du) && al16(ws) && al16(pr.dlw);
  return vh ? launch_bband_t<T, true>(pr, ws, stream, tr) : launch_bband_t<T, false>(pr, ws, stream, tr);
}

hipError_t launch_bband(const BwdProblem& pr, void* ws, hipStream_t stream, Tracer* tr) {
  if (pr.dtype == GSPN_F32) return launch_bband_dt<float>(pr, ws, stream, tr);
  return launch_bband_dt<bf16_t>(pr, ws, stream, tr);
}

}  // namespace gspn

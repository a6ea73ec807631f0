// Backward pass of the GSPN propagation for planes with H, W <= 64, whole
// plane in LDS (the counterpart of the plane-resident forward kernel).
//
// A workgroup of four wavefronts owns PPB = 64 / SEG planes at a time and
// loops over plane groups (persistent grid). Per plane group:
//   1. records (w0, w1, w2, lambda x) per pixel in LDS, and the edge-lane
//      records whose missing neighbour changes the normalisation (their
//      inputs were loaded while the previous group ran);
//   2. wavefront d runs the forward scan of direction d (lane = orthogonal
//      index, neighbours by DPP) and keeps its states in registers;
//   3. the record's fourth component becomes u * grad_out;
//   4. wavefront d runs the reverse scan of the error term (CSDN page on GSPN,
//      section 反向传播):
//        e_s[o] = u gy + w_{s+1,0}[o+1] e_{s+1}[o+1] + w_{s+1,1}[o] e_{s+1}[o]
//                      + w_{s+1,2}[o-1] e_{s+1}[o-1]
//      -- the products w_k e of line s+1 come from lanes o+1 / o / o-1 by DPP,
//      a restart line sends nothing back -- and parks e_d in LDS;
//   5. the records are dead: each wavefront parks its forward states there;
//   6. every thread takes whole pixels and forms, in the fixed direction order
//      T2B, B2T, L2R, R2L,
//        grad_x = lambda sum_d e_d,  grad_lambda = x sum_d e_d,
//        grad_u = gy sum_d h_d,
//        grad_l_k = sum_d e_d w_k (1 - sigmoid(l_k)) (h_d,prev[o+k-1] - p_d),
//      with p_d = sum_j w_j h_d,prev[o+j-1] written as differences of
//      neighbouring states (sum_j w_j = 1) and the weights recomputed from
//      the logits for the scan axis of d (edge masks differ between axes).
// LDS holds 32 bytes per pixel (records, later the parked states, plus the
// parked error terms). HBM traffic: seven inputs read, six gradients
// written; step 6 reads the logits, x, lambda and grad_out once more (from
// L2), except on fixed 16 x 16 planes, which keep them in registers.
#include "gspn_device.hpp"
#include "gspn_launch.hpp"

#ifndef BP_NT16
#define BP_NT16 256
#endif
#ifndef BP_NT64
#define BP_NT64 512
#endif

namespace gspn {

namespace {
__device__ __forceinline__ float pl1(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float pl1(const bf16_t* p, int64_t i) { return to_f32(p[i]); }

// normalised weights from a_k = 1 + exp(-l_k) and the edge masks
__device__ __forceinline__ Weights weights_of(float a0, float a1, float a2, float m0, float m2) {
  const float p12 = (m0 * a1) * a2;
  const float p02 = a0 * a2;
  const float p01 = (m2 * a0) * a1;
  const float r = recip(p12 + p02 + p01);
  return Weights{p12 * r, p02 * r, p01 * r};
}

// e * w_k (1 - sigmoid_k) * (h_k - sum_j w_j h_j) for the three links, added
// into g[0..2]; hl, hc, hr are the previous line's states at o-1, o, o+1
__device__ __forceinline__ void add_logit_grads(float e, const Weights& w, const float s[3],
                                                float hl, float hc, float hr, float g[3]) {
  const float d01 = hl - hc, d12 = hc - hr, d02 = hl - hr;
  const float dev0 = w.w1 * d01 + w.w2 * d02;
  const float dev1 = w.w2 * d12 - w.w0 * d01;
  const float dev2 = -(w.w0 * d02 + w.w1 * d12);
  g[0] = __builtin_fmaf(e * (w.w0 * s[0]), dev0, g[0]);
  g[1] = __builtin_fmaf(e * (w.w1 * s[1]), dev1, g[1]);
  g[2] = __builtin_fmaf(e * (w.w2 * s[2]), dev2, g[2]);
}
}  // namespace

template <typename T>
struct BPlaneArgs {
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
  int64_t nplanes;
  int64_t ngroups;
  int H, W, G;
  unsigned mask;
  int pitch;        // LDS row pitch in pixels (W rounded up to odd)
  float inv_W, inv_HW;
  int64_t C, Cl;    // channels and logit channels (shared logits when Cl < C)
  float* dlw;       // shared logits: per-plane fp32 logit gradients [3][planes*H*W]
};

// Pixel i of a plane group is handled by thread i % NT in every per-pixel
// phase (consecutive lanes take consecutive pixels: coalesced global access
// and conflict-free LDS access). The gradient phase reads x, lambda, the
// logits and grad_out again; they were read moments before, so from L2.
// The first four wavefronts run the scans (one direction each); all NT
// threads share the per-pixel phases.
// HS, WS > 0: the plane's height and width fixed at compile time (common
// shapes), so index arithmetic folds to constants and the scans unroll to
// exactly their length; 0: taken from the arguments. LOCAL: local groups
// (G > 0); without them a scan restarts only at its first step.
template <typename T, int SEG, int NT, int HS = 0, int WS = 0, bool LOCAL = true>
__global__ __launch_bounds__(NT, SEG == 16 ? 3 : 1) void bplane_kernel(BPlaneArgs<T> a) {
  constexpr int PPB = 64 / SEG;
  constexpr bool FIX = HS > 0;
  // pixels per thread at most
  constexpr int KMAX = ((FIX ? PPB * HS * WS : PPB * SEG * SEG) + NT - 1) / NT;
  // longest scan: SEG, or the plane's longer side when it is fixed
  constexpr int NS = FIX ? (HS > WS ? HS : WS) : SEG;
  extern __shared__ float4 smem[];
  float* smf = reinterpret_cast<float*>(smem);

  const int H = FIX ? HS : a.H, W = FIX ? WS : a.W, pitch = FIX ? (WS | 1) : a.pitch;
  const int G = LOCAL ? a.G : 0;
  const int HW = H * W;
  // pixel index -> (plane, remainder) within a plane group
  auto split_plane = [&](int i, int* rem) {
    if constexpr (FIX) {
      const int pp = i / (HS * WS);
      *rem = i - pp * (HS * WS);
      return pp;
    } else {
      return div_small(i, HW, a.inv_HW, rem);
    }
  };
  const int rec_sz = PPB * H * pitch;          // pixels (with pitch padding)
  // float4 records [0, rec_sz) -> later parked states, floats [0, 4 rec_sz)
  float* hpark = smf;
  // parked error terms, floats [4 rec_sz, 8 rec_sz)
  float* epark = smf + 4 * rec_sz;
  const int ev_off = 2 * rec_sz;               // float4 [PPB][2][H]
  const int eh_off = ev_off + PPB * 2 * H;     // float4 [PPB][2][W]
  const int zero_off = eh_off + PPB * 2 * W;   // one zero record
  const int tid = threadIdx.x;

  // The inputs of the records (x, lambda, logits) are held raw in registers
  // one plane group ahead; the next group's loads are issued right after
  // this group's records are built, so they stay in flight through the
  // scans. 16-wide planes hold u and grad_out ahead as well.
  constexpr bool kAheadUg = SEG == 16;
  T px[KMAX], plm[KMAX], pq0[KMAX], pq1[KMAX], pq2[KMAX];
  T pu[kAheadUg ? KMAX : 1], pg[kAheadUg ? KMAX : 1];
  auto group_pixel = [&](int64_t grp, int k, int64_t* gi, int64_t* lgi) {
    const int64_t pl0 = grp * PPB;
    const int npx = static_cast<int>(min<int64_t>(PPB, a.nplanes - pl0)) * HW;
    const int i = tid + NT * k;
    const int ic = i < npx ? i : 0;   // always in bounds
    *gi = pl0 * HW + ic;
    *lgi = *gi;
    if (a.Cl != a.C) {
      int rem;
      const int pin = PPB == 1 ? 0 : split_plane(ic, &rem);
      *lgi += logit_shift(pl0 + pin, a.C, a.Cl, HW);
    }
  };
  auto fetch_records = [&](int64_t grp) {
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      int64_t gi, lgi;
      group_pixel(grp, k, &gi, &lgi);
      px[k] = a.x[gi];
      plm[k] = a.lam[gi];
      pq0[k] = a.l0[lgi];
      pq1[k] = a.l1[lgi];
      pq2[k] = a.l2[lgi];
      if constexpr (kAheadUg) {
        pu[k] = a.u[gi];
        pg[k] = a.gy[gi];
      }
    }
  };
  if (static_cast<int64_t>(blockIdx.x) < a.ngroups) fetch_records(blockIdx.x);

  for (int64_t grp = blockIdx.x; grp < a.ngroups; grp += gridDim.x) {
    const int64_t plane0 = grp * PPB;
    const int np = static_cast<int>(min<int64_t>(PPB, a.nplanes - plane0));
    const int64_t gbase = plane0 * HW;
    const int npix = np * HW;
    const bool more = grp + gridDim.x < a.ngroups;

    // ---- 1. records ---------------------------------------------------------
    // LDS index of pixel i of the group (and its plane within the group)
    auto lds_index = [&](int i, int* r, int* c, int* pp_out = nullptr) {
      int rem;
      const int pp = split_plane(i, &rem);
      if constexpr (FIX) {
        *r = rem / WS;
        *c = rem - *r * WS;
      } else {
        *r = div_small(rem, W, a.inv_W, c);
      }
      if (pp_out) *pp_out = pp;
      return (pp * H + *r) * pitch + *c;
    };
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      const int i = tid + NT * k;
      if (i < npix) {
        int r, c;
        const int li = lds_index(i, &r, &c);
        const Weights w = make_weights(to_f32(pq0[k]), to_f32(pq1[k]), to_f32(pq2[k]), 1.f, 1.f);
        smem[li] = make_float4(w.w0, w.w1, w.w2, to_f32(plm[k]) * to_f32(px[k]));
      }
    }
    // this group's inputs, before the next group's loads replace them: u and
    // grad_out for step 3, and (fixed 16 x 16 shapes) all seven for step 6.
    // Fixed 64-wide shapes load u and grad_out here, for step 3, so that the
    // forward scans hide their latency (the general kernel has no registers
    // left for them and loads them in step 3).
    constexpr bool kKeep = kAheadUg && FIX;
    constexpr bool kEarlyUg = !kAheadUg && FIX;
    constexpr int KC = kAheadUg || kEarlyUg ? KMAX : 1;
    T ug_u[KC], ug_g[KC], cx[kKeep ? KMAX : 1], clm[kKeep ? KMAX : 1], cq0[kKeep ? KMAX : 1],
        cq1[kKeep ? KMAX : 1], cq2[kKeep ? KMAX : 1];
    if constexpr (kEarlyUg) {
#pragma unroll
      for (int k = 0; k < KMAX; ++k) {
        const int i = tid + NT * k;
        const int64_t gi = gbase + (i < npix ? i : 0);
        ug_u[k] = a.u[gi];
        ug_g[k] = a.gy[gi];
      }
    }
    if constexpr (kAheadUg) {
#pragma unroll
      for (int k = 0; k < KMAX; ++k) {
        ug_u[k] = pu[k];
        ug_g[k] = pg[k];
        if constexpr (kKeep) {
          cx[k] = px[k];
          clm[k] = plm[k];
          cq0[k] = pq0[k];
          cq1[k] = pq1[k];
          cq2[k] = pq2[k];
        }
      }
    }
    if (more) fetch_records(grp + gridDim.x);
    if (tid == 0) smem[zero_off] = make_float4(0.f, 0.f, 0.f, 0.f);
    __syncthreads();

    // edge-lane records: vertical scans use lanes c = 0 / W-1 (masks on c),
    // horizontal scans lanes r = 0 / H-1 (masks on r)
    const int n_ev = np * 2 * H, n_eh = np * 2 * W;
    for (int k = tid; k < n_ev + n_eh; k += NT) {
      int p, e, pos, r, c, idx, n_o, o;
      if (k < n_ev) {
        p = k / (2 * H); e = (k / H) & 1; pos = k % H;
        r = pos; c = e ? W - 1 : 0; o = c; n_o = W; idx = ev_off + (p * 2 + e) * H + pos;
      } else {
        const int k2 = k - n_ev;
        p = k2 / (2 * W); e = (k2 / W) & 1; pos = k2 % W;
        c = pos; r = e ? H - 1 : 0; o = r; n_o = H; idx = eh_off + (p * 2 + e) * W + pos;
      }
      const float4 m = smem[(p * H + r) * pitch + c];
      const Weights w = edge_weights(m.x, m.y, m.z, o > 0 ? 1.f : 0.f, o < n_o - 1 ? 1.f : 0.f);
      smem[idx] = make_float4(w.w0, w.w1, w.w2, m.w);
    }
    __syncthreads();

    // ---- 2. forward scan, one direction per wavefront ------------------------
    const int d = tid >> 6;
    const int lane = tid & 63;
    const int p = lane / SEG, o = lane % SEG;
    const bool on = d < 4 && ((a.mask >> d) & 1u);
    const bool vert = d < 2, fwd = (d == 0 || d == 2);
    const int n_s = vert ? H : W, n_o = vert ? W : H;
    const bool active = on && o < n_o && p < np;
    int mbase, mstride;
    if (vert) { mbase = (p * H + (fwd ? 0 : H - 1)) * pitch + o; mstride = fwd ? pitch : -pitch; }
    else      { mbase = (p * H + o) * pitch + (fwd ? 0 : W - 1); mstride = fwd ? 1 : -1; }
    int addr0 = mbase, stride = mstride;
    if (!active) { addr0 = zero_off; stride = 0; }
    else if (o == 0 || o == n_o - 1) {
      const int e = (o == 0) ? 0 : 1;
      if (vert) addr0 = ev_off + (p * 2 + e) * H + (fwd ? 0 : H - 1);
      else      addr0 = eh_off + (p * 2 + e) * W + (fwd ? 0 : W - 1);
      stride = fwd ? 1 : -1;
    }
    // restart at step s: the first step, or the first position of a group
    auto restarts = [&](int s) {
      if (s == 0) return true;
      if (G <= 0) return false;
      return fwd ? (s % G) == 0 : ((n_s - 1 - s) % G) == G - 1;
    };

    float hist[NS];
    if (on) {
      float h = 0.0f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (s < n_s) {
          const float4 rc = smem[addr0 + s * stride];
          const float hn = line_step<SEG>(h, rc.x, rc.y, rc.z, rc.w);
          h = restarts(s) ? rc.w : hn;
          hist[s] = h;
        }
      }
    }
    __syncthreads();

    // ---- 3. u * grad_out into the records ------------------------------------
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      const int i = tid + NT * k;
      if (i < npix) {
        int r, c;
        smf[4 * lds_index(i, &r, &c) + 3] =
            KC > 1 ? to_f32(ug_u[k]) * to_f32(ug_g[k]) : pl1(a.u, gbase + i) * pl1(a.gy, gbase + i);
      }
    }
    __syncthreads();
    for (int k = tid; k < n_ev + n_eh; k += NT) {
      int pp, e, pos, r, c, idx;
      if (k < n_ev) {
        pp = k / (2 * H); e = (k / H) & 1; pos = k % H;
        r = pos; c = e ? W - 1 : 0; idx = ev_off + (pp * 2 + e) * H + pos;
      } else {
        const int k2 = k - n_ev;
        pp = k2 / (2 * W); e = (k2 / W) & 1; pos = k2 % W;
        c = pos; r = e ? H - 1 : 0; idx = eh_off + (pp * 2 + e) * W + pos;
      }
      smf[4 * idx + 3] = smf[4 * ((pp * H + r) * pitch + c) + 3];
    }
    __syncthreads();

    // ---- 4. reverse scan of the error term -----------------------------------
    if (on) {
      float p0 = 0.f, p1 = 0.f, p2 = 0.f;   // w_k e of the line after this one
#pragma unroll
      for (int s = NS - 1; s >= 0; --s) {
        if (s < n_s) {
          const float4 rc = smem[addr0 + s * stride];
          const float e = rc.w + from_right<SEG>(p0) + p1 + from_left<SEG>(p2);
          const bool rs = restarts(s);
          p0 = rs ? 0.f : rc.x * e;
          p1 = rs ? 0.f : rc.y * e;
          p2 = rs ? 0.f : rc.z * e;
          if (active) epark[d * rec_sz + mbase + s * mstride] = e;
        }
      }
    }
    __syncthreads();   // every wavefront is done with the records

    // ---- 5. park the forward states over the records --------------------------
    if (active) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
        if (s < n_s) hpark[d * rec_sz + mbase + s * mstride] = hist[s];
    }
    __syncthreads();

    // ---- 6. gradients per pixel ----------------------------------------------
    const unsigned mask = a.mask;
#pragma unroll (SEG == 16 && FIX ? KMAX : 2)
    for (int k = 0; k < KMAX; ++k) {
      const int i = tid + NT * k;
      if (i >= npix) continue;
      int r, c, pp;
      const int li = lds_index(i, &r, &c, &pp);
      const int64_t gi = gbase + i;
      const int64_t lgi = gi + logit_shift(plane0 + pp, a.C, a.Cl, HW);
      // (the fixed-shape kernels unroll this loop, so k indexes registers)
      const float xv = kKeep ? to_f32(cx[k]) : pl1(a.x, gi);
      const float lv = kKeep ? to_f32(clm[k]) : pl1(a.lam, gi);
      const float gyv = kKeep ? to_f32(ug_g[k]) : pl1(a.gy, gi);
      const float g0 = kKeep ? to_f32(cq0[k]) : pl1(a.l0, lgi);
      const float g1 = kKeep ? to_f32(cq1[k]) : pl1(a.l1, lgi);
      const float g2 = kKeep ? to_f32(cq2[k]) : pl1(a.l2, lgi);
      float se = 0.f, sh = 0.f;
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) {
        if ((mask >> dd) & 1u) {
          se += epark[dd * rec_sz + li];
          sh += hpark[dd * rec_sz + li];
        }
      }
      const float e0 = exp_neg(g0), e1 = exp_neg(g1), e2 = exp_neg(g2);
      const float a0 = 1.f + e0, a1 = 1.f + e1, a2 = 1.f + e2;
      const float sl[3] = {e0 * recip(a0), e1 * recip(a1), e2 * recip(a2)};
      float gl[3] = {0.f, 0.f, 0.f};
      const bool cl = c > 0, cr = c < W - 1, ru = r > 0, rd = r < H - 1;
      if (mask & 3u) {
        const Weights wv = weights_of(a0, a1, a2, cl ? 1.f : 0.f, cr ? 1.f : 0.f);
        // top->bottom: previous line is row r-1
        if ((mask & 1u) && !(r == 0 || (G > 0 && r % G == 0))) {
          const float* hp = hpark + li - pitch;
          const float hc = hp[0];
          add_logit_grads(epark[li], wv, sl, cl ? hp[-1] : hc, hc, cr ? hp[1] : hc, gl);
        }
        // bottom->top: previous line is row r+1
        if ((mask & 2u) && !(r == H - 1 || (G > 0 && r % G == G - 1))) {
          const float* hp = hpark + rec_sz + li + pitch;
          const float hc = hp[0];
          add_logit_grads(epark[rec_sz + li], wv, sl, cl ? hp[-1] : hc, hc, cr ? hp[1] : hc, gl);
        }
      }
      if (mask & 12u) {
        const Weights wh = weights_of(a0, a1, a2, ru ? 1.f : 0.f, rd ? 1.f : 0.f);
        // left->right: previous line is column c-1 (orthogonal neighbours are rows)
        if ((mask & 4u) && !(c == 0 || (G > 0 && c % G == 0))) {
          const float* hp = hpark + 2 * rec_sz + li - 1;
          const float hc = hp[0];
          add_logit_grads(epark[2 * rec_sz + li], wh, sl, ru ? hp[-pitch] : hc, hc,
                          rd ? hp[pitch] : hc, gl);
        }
        // right->left: previous line is column c+1
        if ((mask & 8u) && !(c == W - 1 || (G > 0 && c % G == G - 1))) {
          const float* hp = hpark + 3 * rec_sz + li + 1;
          const float hc = hp[0];
          add_logit_grads(epark[3 * rec_sz + li], wh, sl, ru ? hp[-pitch] : hc, hc,
                          rd ? hp[pitch] : hc, gl);
        }
      }
      Store<T>::put(a.dx, gi, lv * se);
      if (a.dlw) {
        const int64_t P = a.nplanes * HW;
        a.dlw[gi] = gl[0];
        a.dlw[P + gi] = gl[1];
        a.dlw[2 * P + gi] = gl[2];
      } else {
        Store<T>::put(a.dl0, gi, gl[0]);
        Store<T>::put(a.dl1, gi, gl[1]);
        Store<T>::put(a.dl2, gi, gl[2]);
      }
      Store<T>::put(a.dlam, gi, xv * se);
      Store<T>::put(a.du, gi, gyv * sh);
    }
    __syncthreads();   // LDS is rewritten by the next plane group
  }
}

size_t bplane_lds_bytes(int64_t H, int64_t W) {
  const int seg = plane_seg(H, W);
  const int64_t ppb = 64 / seg;
  const int64_t pitch = W | 1;
  const int64_t rec = ppb * H * pitch;
  return static_cast<size_t>(8 * rec) * sizeof(float) +
         static_cast<size_t>(ppb * (2 * H + 2 * W) + 1) * sizeof(float4);
}

// the kernel for a plane shape: compile-time shapes for common sizes (the
// 16 x 16 DiT latents, the 56 x 56 first classification stage, and the
// square planes of later stages), the general kernel otherwise
template <typename T, int SEG, int NT>
static void (*pick_bplane_kernel(int H, int W, bool local))(BPlaneArgs<T>) {
  if (H == W) {
    if constexpr (SEG == 16) {
      if (H == 16) return local ? bplane_kernel<T, 16, NT, 16, 16, true>
                                : bplane_kernel<T, 16, NT, 16, 16, false>;
    } else {
      switch (H) {
        case 28: return local ? bplane_kernel<T, 64, NT, 28, 28, true>
                              : bplane_kernel<T, 64, NT, 28, 28, false>;
        case 32: return local ? bplane_kernel<T, 64, NT, 32, 32, true>
                              : bplane_kernel<T, 64, NT, 32, 32, false>;
        case 56: return local ? bplane_kernel<T, 64, NT, 56, 56, true>
                              : bplane_kernel<T, 64, NT, 56, 56, false>;
        case 64: return local ? bplane_kernel<T, 64, NT, 64, 64, true>
                              : bplane_kernel<T, 64, NT, 64, 64, false>;
        default: break;
      }
    }
  }
  return local ? bplane_kernel<T, SEG, NT, 0, 0, true> : bplane_kernel<T, SEG, NT, 0, 0, false>;
}

template <typename T, int SEG, int NT>
static hipError_t launch_bplane_t(const BwdProblem& pr, hipStream_t stream, Tracer* tr) {
  BPlaneArgs<T> a;
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
  a.nplanes = pr.B * pr.C;
  constexpr int PPB = 64 / SEG;
  a.ngroups = (a.nplanes + PPB - 1) / PPB;
  a.H = static_cast<int>(pr.H);
  a.W = static_cast<int>(pr.W);
  a.G = static_cast<int>(pr.G >= pr.H && pr.G >= pr.W ? 0 : pr.G);
  a.mask = pr.mask;
  a.pitch = static_cast<int>(pr.W | 1);
  a.inv_W = 1.0f / static_cast<float>(pr.W);
  a.inv_HW = 1.0f / static_cast<float>(pr.H * pr.W);
  a.C = pr.C;
  a.Cl = pr.Cl;
  a.dlw = pr.dlw;
  const size_t lds = bplane_lds_bytes(pr.H, pr.W);
  auto kern = pick_bplane_kernel<T, SEG, NT>(a.H, a.W, a.G > 0);
  hipError_t e;
  if (lds > 65536) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  int per_cu = 0, dev = 0, cus = 0;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern),
                                                        NT, lds)) != hipSuccess)
    return e;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
    return e;
  const int64_t resident = static_cast<int64_t>(per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
  const int64_t grid = a.ngroups < resident ? a.ngroups : resident;
  tr->before(stream, SEG == 16 ? "bplane_kernel16" : "bplane_kernel64", a.nplanes);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(NT), lds, stream, a);
  tr->after(stream);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_bplane_dt(const BwdProblem& pr, hipStream_t stream, Tracer* tr) {
  // LDS (32 bytes per pixel) keeps large planes at one workgroup per CU:
  // those get more wavefronts for the per-pixel phases
  if (plane_seg(pr.H, pr.W) == 16) return launch_bplane_t<T, 16, BP_NT16>(pr, stream, tr);
  return launch_bplane_t<T, 64, BP_NT64>(pr, stream, tr);
}

hipError_t launch_bplane(const BwdProblem& pr, hipStream_t stream, Tracer* tr) {
  if (pr.dtype == GSPN_F32) return launch_bplane_dt<float>(pr, stream, tr);
  return launch_bplane_dt<bf16_t>(pr, stream, tr);
}

}  // namespace gspn

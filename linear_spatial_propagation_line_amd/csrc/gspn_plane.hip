// Plane-resident GSPN propagation for planes with H, W <= 64.
//
// A workgroup of four wavefronts owns PPB = 64 / SEG whole planes at a time
// and loops over plane groups (a persistent grid sized to what fits on the
// GPU at once):
//   1. records: every pixel becomes (w0, w1, w2, lambda*x) in LDS -- sigmoid
//      and normalisation computed once per pixel and shared by all four
//      directions. The inputs come from registers filled by the previous
//      iteration, and right after the records are built the loads of the next
//      plane group are issued, so HBM transfers overlap steps 2-4;
//   2. records for the edge lanes (orthogonal index 0 and n_o - 1, whose
//      missing neighbour changes the normalisation) go to small side arrays;
//   3. wavefront d runs scan direction d: lane o of a SEG-lane segment is
//      orthogonal index o, it walks the scan axis reading one record per step
//      and takes its two neighbours' previous states by DPP (wave_shr/shl for
//      SEG = 64, row_shr/shl inside 16-lane rows for SEG = 16, four planes
//      per wavefront); its states stay in registers;
//   4. the states are parked in LDS (over the now dead records), and all
//      threads form out = u * (h_T2B + h_B2T + h_L2R + h_R2L) in that fixed
//      order with one rounding to the storage type.
// HBM traffic is the compulsory one: five inputs and u read once, out
// written once.
//
// Line recurrence, output gate and unrolled form: CSDN page on GSPN, section
// 方法; three-neighbour tridiagonal weights with sigmoid + row normalisation
// and four scan directions: same page, section 如何设计一个高效的传播层;
// local groups: section GSPN模块的设计.
#include <cstdlib>

#include "gspn_device.hpp"
#include "gspn_launch.hpp"

namespace gspn {

template <typename T>
struct PlaneArgs {
  const T* x;
  const T* l0;
  const T* l1;
  const T* l2;
  const T* lam;
  const T* u;
  T* out;
  int64_t nplanes;
  int64_t ngroups;  // plane groups of PPB planes
  int H, W, G;
  unsigned mask;
  int pitch;        // records per LDS row (W rounded up to odd)
  float inv_W, inv_HW;
  int64_t C, Cl;    // channels and logit channels (shared logits when Cl < C)
};

__device__ __forceinline__ float ld1(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld1(const bf16_t* p, int64_t i) { return to_f32(p[i]); }
__device__ __forceinline__ void st1(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st1(bf16_t* p, int64_t i, float v) {
  p[i].bits = static_cast<uint16_t>(f32_to_bf16_bits(v));
}

// HS, WS > 0: the plane's height and width fixed at compile time (common
// shapes), so index arithmetic folds to constants and the scans unroll to
// exactly their length; 0: taken from the arguments. LOCAL: local groups
// (G > 0); without them a scan restarts only at its first step.
template <typename T, int SEG, int VEC, int HS = 0, int WS = 0, bool LOCAL = true>
__global__ __launch_bounds__(256, SEG == 64 ? 2 : 1) void plane_kernel(PlaneArgs<T> a) {
  constexpr int PPB = 64 / SEG;
  // pixels per thread handled in 4-wide vectors: up to 4096 (SEG 64) or 1024
  // (SEG 16) pixels per plane group over 256 threads
  constexpr int NIT = VEC == 4 ? (SEG == 64 ? 4 : 1) : 1;
  using V = V4<T>;
  extern __shared__ float4 smem[];
  float* smem_f = reinterpret_cast<float*>(smem);

  constexpr bool FIX = HS > 0;
  const int H = FIX ? HS : a.H, W = FIX ? WS : a.W, pitch = FIX ? (WS | 1) : a.pitch;
  // pixel index -> (plane, row, column) within a plane group
  auto split = [&](int i, int* pp, int* rr, int* cc) {
    if constexpr (FIX) {
      *pp = i / (HS * WS);
      const int rem = i - *pp * (HS * WS);
      *rr = rem / WS;
      *cc = rem - *rr * WS;
    } else {
      int rem;
      *pp = div_small(i, H * W, a.inv_HW, &rem);
      *rr = div_small(rem, W, a.inv_W, cc);
    }
  };
  const int HW = H * W;
  const int rec_sz = PPB * H * pitch;          // records (float4 units)
  const int ev_off = rec_sz;                   // [PPB][2][H]
  const int eh_off = ev_off + PPB * 2 * H;     // [PPB][2][W]
  const int zero_off = eh_off + PPB * 2 * W;   // one zero record
  const int tid = threadIdx.x;

  // registers filled one plane group ahead (VEC == 4 only); u only on
  // 16-wide planes, 64-wide ones load it for the group at hand
  typename V::raw rx[NIT], rl[NIT], r0[NIT], r1[NIT], r2[NIT], ru[SEG == 16 ? NIT : 1];
  // loads of 4-pixel vectors lo .. hi - 1 of plane group grp
  auto issue = [&](int64_t grp, int lo, int hi) {
    const int64_t gb = grp * PPB * HW;
    const int npx = static_cast<int>(min<int64_t>(PPB, a.nplanes - grp * PPB)) * HW;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      if (it < lo || it >= hi) continue;
      const int i0 = tid * 4 + it * 1024;
      const int ic = i0 < npx ? i0 : 0;                // always in bounds
      const int64_t gi = gb + ic;
      int64_t lgi = gi;
      if (a.Cl != a.C) {
        int rem;
        const int pin = PPB == 1 ? 0 : div_small(ic, HW, a.inv_HW, &rem);
        lgi += logit_shift(grp * PPB + pin, a.C, a.Cl, HW);
      }
      rx[it] = V::load(a.x, gi);
      rl[it] = V::load(a.lam, gi);
      r0[it] = V::load(a.l0, lgi);
      r1[it] = V::load(a.l1, lgi);
      r2[it] = V::load(a.l2, lgi);
      if constexpr (SEG == 16) ru[it] = V::load(a.u, gi);
    }
  };
  if constexpr (VEC == 4)
    if (static_cast<int64_t>(blockIdx.x) < a.ngroups) issue(blockIdx.x, 0, NIT);

  for (int64_t grp = blockIdx.x; grp < a.ngroups; grp += gridDim.x) {
    const int64_t plane0 = grp * PPB;
    const int np = static_cast<int>(min<int64_t>(PPB, a.nplanes - plane0));
    const int64_t gbase = plane0 * HW;
    const int npix = np * HW;

    // ---- 1. records --------------------------------------------------------
    typename V::raw uu[NIT];
    if constexpr (VEC == 4) {
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        if constexpr (SEG == 16) uu[it] = ru[it];
        const int i0 = tid * 4 + it * 1024;
        if (i0 < npix) {
          int p, r, c;
          split(i0, &p, &r, &c);
          // W % 4 == 0 on this path, so the four pixels share row r
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const Weights w = make_weights(V::get(r0[it], e), V::get(r1[it], e),
                                           V::get(r2[it], e), 1.0f, 1.0f);
            smem[(p * H + r) * pitch + c + e] =
                make_float4(w.w0, w.w1, w.w2, V::get(rl[it], e) * V::get(rx[it], e));
          }
        }
      }
      // 64-wide planes load this group's u now, for the merge: holding it a
      // group ahead as well would not fit the registers
      if constexpr (SEG == 64) {
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
          const int i0 = tid * 4 + it * 1024;
          uu[it] = V::load(a.u, gbase + (i0 < npix ? i0 : 0));
        }
      }
      // the next plane group's loads fly during steps 2-4; on 64-wide planes
      // they are issued a part per phase, so the memory stays busy
      if (grp + gridDim.x < a.ngroups) issue(grp + gridDim.x, 0, SEG == 64 ? 2 : NIT);
    } else {
      for (int i0 = tid; i0 < npix; i0 += 256) {
        int p, r, c;
        split(i0, &p, &r, &c);
        const int64_t gi = gbase + i0;
        const int64_t lgi = gi + logit_shift(plane0 + p, a.C, a.Cl, HW);
        const Weights w = make_weights(ld1(a.l0, lgi), ld1(a.l1, lgi), ld1(a.l2, lgi), 1.0f, 1.0f);
        smem[(p * H + r) * pitch + c] = make_float4(w.w0, w.w1, w.w2, ld1(a.lam, gi) * ld1(a.x, gi));
      }
    }
    if (tid == 0) smem[zero_off] = make_float4(0.f, 0.f, 0.f, 0.f);
    __syncthreads();

    // ---- 2. edge-lane records ----------------------------------------------
    // vertical scans: lanes c = 0 (e = 0) and c = W-1 (e = 1), masks on c;
    // horizontal scans: lanes r = 0 and r = H-1, masks on r.
    // Slot k of [horizontal][plane][side][SEG positions] (2 * PPB * 2 * SEG =
    // 256 slots: one per thread, index arithmetic by shifts); positions past
    // the line's end have nothing to do.
    {
      const int k = tid;
      const int hz = k / (PPB * 2 * SEG), p = (k / (2 * SEG)) % PPB, e = (k / SEG) & 1;
      const int pos = k % SEG;
      int r, c, idx, n_o, o;
      if (!hz) {
        r = pos; c = e ? W - 1 : 0; o = c; n_o = W; idx = ev_off + (p * 2 + e) * H + pos;
      } else {
        c = pos; r = e ? H - 1 : 0; o = r; n_o = H; idx = eh_off + (p * 2 + e) * W + pos;
      }
      if (p < np && pos < (hz ? W : H)) {
        const float4 m = smem[(p * H + r) * pitch + c];
        const Weights w = edge_weights(m.x, m.y, m.z, o > 0 ? 1.f : 0.f, o < n_o - 1 ? 1.f : 0.f);
        smem[idx] = make_float4(w.w0, w.w1, w.w2, m.w);
      }
    }
    __syncthreads();
    if constexpr (VEC == 4 && SEG == 64)
      if (grp + gridDim.x < a.ngroups) issue(grp + gridDim.x, 2, 3);

    // ---- 3. one scan direction per wavefront -------------------------------
    const int d = tid >> 6;
    const int lane = tid & 63;
    const int p = lane / SEG, o = lane % SEG;
    const bool on = (a.mask >> d) & 1u;
    const bool vert = d < 2, fwd = (d == 0 || d == 2);
    const int n_s = vert ? H : W, n_o = vert ? W : H;
    const bool active = on && o < n_o && p < np;
    // main-record position of step 0 and its per-step stride
    int mbase, mstride;
    if (vert) { mbase = (p * H + (fwd ? 0 : H - 1)) * pitch + o; mstride = fwd ? pitch : -pitch; }
    else      { mbase = (p * H + o) * pitch + (fwd ? 0 : W - 1); mstride = fwd ? 1 : -1; }
    int addr = mbase, stride = mstride;
    if (!active) { addr = zero_off; stride = 0; }
    else if (o == 0 || o == n_o - 1) {
      const int e = (o == 0) ? 0 : 1;
      if (vert) { addr = ev_off + (p * 2 + e) * H + (fwd ? 0 : H - 1); }
      else      { addr = eh_off + (p * 2 + e) * W + (fwd ? 0 : W - 1); }
      stride = fwd ? 1 : -1;
    }
    // steps at which the state restarts: 0, then every G from the first
    // block edge met
    const int G = LOCAL ? a.G : 0;
    int next_restart = n_s;
    if (G > 0) next_restart = fwd ? G : n_s - ((n_s - 1) / G) * G;

    // longest scan: SEG, or the plane's longer side when it is fixed
    constexpr int NS = FIX ? (HS > WS ? HS : WS) : SEG;
    float hist[NS];
    if (on) {
      float h = 0.0f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (s < n_s) {
          const float4 rc = smem[addr];
          addr += stride;
          const float hn = line_step<SEG>(h, rc.x, rc.y, rc.z, rc.w);
          bool restart = (s == 0);
          if (s == next_restart) { restart = true; next_restart += G; }
          h = restart ? rc.w : hn;
          hist[s] = h;
        }
      }
    }
    __syncthreads();   // every wavefront is done with the records
    if constexpr (VEC == 4 && SEG == 64)
      if (grp + gridDim.x < a.ngroups) issue(grp + gridDim.x, 3, NIT);

    // ---- 4. park states over the records, then merge ------------------------
    if (active) {
      int ya = d * rec_sz + mbase;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (s < n_s) { smem_f[ya] = hist[s]; ya += mstride; }
      }
    }
    __syncthreads();

    if constexpr (VEC == 4) {
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int i0 = tid * 4 + it * 1024;
        if (i0 < npix) {
          int pp, r, c;
          split(i0, &pp, &r, &c);
          const int li = (pp * H + r) * pitch + c;
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float sum = 0.0f;
#pragma unroll
            for (int dd = 0; dd < 4; ++dd)
              if ((a.mask >> dd) & 1u) sum += smem_f[dd * rec_sz + li + e];
            y[e] = V::get(uu[it], e) * sum;
          }
          V::store(a.out, gbase + i0, y);
        }
      }
    } else {
      for (int i0 = tid; i0 < npix; i0 += 256) {
        int pp, r, c;
        split(i0, &pp, &r, &c);
        const int li = (pp * H + r) * pitch + c;
        float sum = 0.0f;
#pragma unroll
        for (int dd = 0; dd < 4; ++dd)
          if ((a.mask >> dd) & 1u) sum += smem_f[dd * rec_sz + li];
        st1(a.out, gbase + i0, ld1(a.u, gbase + i0) * sum);
      }
    }
    __syncthreads();   // LDS is rewritten by the next plane group
  }
}

// ---------------------------------------------------------------------------
// Producer / consumer variant for one plane of fixed shape H x W (both at
// most 64, W % 4 == 0) per group. Eight wavefronts: wavefronts 0-3 produce
// (records and edge records of group k, from inputs loaded one group ahead),
// 4-7 consume (the four scans, the park and the merge of group
// k - 1), on two record buffers, so that the serial scans of one group
// overlap the weights of the next. Three workgroup barriers per group
// separate the phases that share a buffer. The producers' raw inputs and the
// consumers' scan states live in different wavefronts, which is what keeps
// 64 x 64 fp32 planes out of scratch. Same arithmetic as plane_kernel, in
// the same order: the two give the same bits.
template <typename T, int HS, int WS, bool LOCAL>
__global__ __launch_bounds__(512, 1) void plane_pc_kernel(PlaneArgs<T> a) {
  constexpr int H = HS, W = WS, HW = HS * WS, pitch = WS | 1;
  constexpr int NIT = (HW + 1023) / 1024;      // 4-pixel vectors per producer thread
  constexpr int NS = HS > WS ? HS : WS;
  constexpr int rec_sz = H * pitch;
  constexpr int ev_off = rec_sz, eh_off = ev_off + 2 * H, zero_off = eh_off + 2 * W;
  constexpr int buf_sz = zero_off + 1;          // float4 units per buffer
  using V = V4<T>;
  extern __shared__ float4 smem[];
  const int tid = threadIdx.x;
  const bool prod = tid < 256;
  const int rt = tid & 255;
  const int64_t ngroups = a.nplanes;            // one plane per group
  // groups of this workgroup: blockIdx.x + k gridDim.x, k < n
  const int64_t n = blockIdx.x < ngroups ? (ngroups - 1 - blockIdx.x) / gridDim.x + 1 : 0;
  auto group_of = [&](int64_t k) { return blockIdx.x + k * static_cast<int64_t>(gridDim.x); };

  // producers: the raw inputs of the next group in registers
  typename V::raw xA[NIT], lA[NIT], gA0[NIT], gA1[NIT], gA2[NIT];
  auto issue = [&](int64_t k, auto& rx, auto& rl, auto& r0, auto& r1, auto& r2) {
    const int64_t g = group_of(min(k, n - 1));  // past the last group: reload it
    const int64_t gb = g * HW;
    const int64_t ls = logit_shift(g, a.C, a.Cl, HW);
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int i0 = rt * 4 + it * 1024;
      const int64_t gi = gb + (i0 < HW ? i0 : 0);
      rx[it] = V::load(a.x, gi);
      rl[it] = V::load(a.lam, gi);
      r0[it] = V::load(a.l0, gi + ls);
      r1[it] = V::load(a.l1, gi + ls);
      r2[it] = V::load(a.l2, gi + ls);
    }
  };
  auto records = [&](float4* buf, const auto& rx, const auto& rl, const auto& r0, const auto& r1,
                     const auto& r2) {
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int i0 = rt * 4 + it * 1024;
      if (i0 < HW) {
        const int r = i0 / WS, c = i0 - r * WS;   // W % 4 == 0: four pixels of row r
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const Weights w = make_weights(V::get(r0[it], e), V::get(r1[it], e), V::get(r2[it], e),
                                         1.0f, 1.0f);
          buf[r * pitch + c + e] = make_float4(w.w0, w.w1, w.w2, V::get(rl[it], e) * V::get(rx[it], e));
        }
      }
    }
  };
  // edge-lane records: one slot per producer thread, [horizontal][side][64 positions]
  auto edges = [&](float4* buf) {
    const int k = rt;
    const int hz = k >> 7, e = (k >> 6) & 1, pos = k & 63;
    int r, c, idx, n_o, o;
    if (!hz) { r = pos; c = e ? W - 1 : 0; o = c; n_o = W; idx = ev_off + e * H + pos; }
    else     { c = pos; r = e ? H - 1 : 0; o = r; n_o = H; idx = eh_off + e * W + pos; }
    if (pos < (hz ? W : H)) {
      const float4 m = buf[r * pitch + c];
      const Weights w = edge_weights(m.x, m.y, m.z, o > 0 ? 1.f : 0.f, o < n_o - 1 ? 1.f : 0.f);
      buf[idx] = make_float4(w.w0, w.w1, w.w2, m.w);
    }
    if (k == 0) buf[zero_off] = make_float4(0.f, 0.f, 0.f, 0.f);
  };

  // consumers: wavefront d of 4..7 scans direction d - 4, lane o
  const int d = (tid >> 6) & 3, o = tid & 63;
  const bool on = (a.mask >> d) & 1u;
  const bool vert = d < 2, fwd = (d == 0 || d == 2);
  const int n_s = vert ? H : W, n_o = vert ? W : H;
  const bool active = on && o < n_o;
  int mbase, mstride;
  if (vert) { mbase = (fwd ? 0 : H - 1) * pitch + o; mstride = fwd ? pitch : -pitch; }
  else      { mbase = o * pitch + (fwd ? 0 : W - 1); mstride = fwd ? 1 : -1; }
  int addr0 = mbase, stride = mstride;
  if (!active) { addr0 = zero_off; stride = 0; }
  else if (o == 0 || o == n_o - 1) {
    const int e = (o == 0) ? 0 : 1;
    if (vert) addr0 = ev_off + e * H + (fwd ? 0 : H - 1);
    else      addr0 = eh_off + e * W + (fwd ? 0 : W - 1);
    stride = fwd ? 1 : -1;
  }
  const int G = LOCAL ? a.G : 0;
  int first_restart = n_s;
  if (G > 0) first_restart = fwd ? G : n_s - ((n_s - 1) / G) * G;
  float hist[NS];
  typename V::raw uu[NIT];
  auto load_u = [&](int64_t k, typename V::raw (&ru)[NIT]) {
    const int64_t gb = group_of(k) * HW;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int i0 = rt * 4 + it * 1024;
      ru[it] = V::load(a.u, gb + (i0 < HW ? i0 : 0));
    }
  };

  auto merge = [&](const float4* buf, int64_t cg, const typename V::raw (&ru)[NIT]) {
    const float* pf = reinterpret_cast<const float*>(buf);
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int i0 = rt * 4 + it * 1024;
      if (i0 < HW) {
        const int r = i0 / WS, c = i0 - r * WS;
        const int li = r * pitch + c;
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float sum = 0.0f;
#pragma unroll
          for (int dd = 0; dd < 4; ++dd)
            if ((a.mask >> dd) & 1u) sum += pf[dd * rec_sz + li + e];
          y[e] = V::get(ru[it], e) * sum;
        }
        V::store(a.out, cg * HW + i0, y);
      }
    }
  };

  if (prod && n > 0) issue(0, xA, lA, gA0, gA1, gA2);
  for (int64_t k = 0; k <= n; ++k) {
    float4* pbuf = smem + (k & 1) * buf_sz;          // producers: group k
    float4* cbuf = smem + ((k + 1) & 1) * buf_sz;    // consumers: group k - 1
    // ---- A: records of group k | scans of group k - 1 ----------------------
    if (prod) {
      if (k < n) {
        records(pbuf, xA, lA, gA0, gA1, gA2);
        issue(k + 1, xA, lA, gA0, gA1, gA2);
      }
    } else if (k > 0) {
      load_u(k - 1, uu);                 // u of the group, for the merge
      if (on) {
        int addr = addr0, next_restart = first_restart;
        float h = 0.0f;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          if (s < n_s) {
            const float4 rc = cbuf[addr];
            addr += stride;
            const float hn = line_step<64>(h, rc.x, rc.y, rc.z, rc.w);
            bool restart = (s == 0);
            if (s == next_restart) { restart = true; next_restart += G; }
            h = restart ? rc.w : hn;
            hist[s] = h;
          }
        }
      }
    }
    __syncthreads();
    // ---- B: edge records of group k | park the states of group k - 1 -------
    if (prod) {
      if (k < n) edges(pbuf);
    } else if (k > 0 && active) {
      float* pf = reinterpret_cast<float*>(cbuf);
      int ya = d * rec_sz + mbase;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (s < n_s) { pf[ya] = hist[s]; ya += mstride; }
      }
    }
    __syncthreads();
    // ---- C: merge of group k - 1 -------------------------------------------
    if (!prod && k > 0) merge(cbuf, group_of(k - 1), uu);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
bool plane_fits(int64_t H, int64_t W) { return H >= 1 && W >= 1 && H <= 64 && W <= 64; }

int plane_seg(int64_t H, int64_t W) { return (H <= 16 && W <= 16) ? 16 : 64; }

size_t plane_lds_bytes(int64_t H, int64_t W) {
  const int seg = plane_seg(H, W);
  const int ppb = 64 / seg;
  const int pitch = static_cast<int>(W | 1);
  const size_t recs = static_cast<size_t>(ppb) * (H * pitch + 2 * H + 2 * W) + 1;
  return recs * sizeof(float4);
}

// the kernel for a plane shape: compile-time shapes for common sizes (the
// 16 x 16 DiT latents, the 56 x 56 first classification stage, and the
// square planes of later stages), the general kernel otherwise
template <typename T, int SEG, int VEC>
static void (*pick_plane_kernel(int H, int W, bool local))(PlaneArgs<T>) {
  if constexpr (VEC == 4) {
    if (H == W) {
      if constexpr (SEG == 16) {
        if (H == 16) return local ? plane_kernel<T, 16, 4, 16, 16, true>
                                  : plane_kernel<T, 16, 4, 16, 16, false>;
      } else {
        switch (H) {
          case 28: return local ? plane_kernel<T, 64, 4, 28, 28, true>
                                : plane_kernel<T, 64, 4, 28, 28, false>;
          case 32: return local ? plane_kernel<T, 64, 4, 32, 32, true>
                                : plane_kernel<T, 64, 4, 32, 32, false>;
          case 56: return local ? plane_kernel<T, 64, 4, 56, 56, true>
                                : plane_kernel<T, 64, 4, 56, 56, false>;
          case 64: return local ? plane_kernel<T, 64, 4, 64, 64, true>
                                : plane_kernel<T, 64, 4, 64, 64, false>;
          default: break;
        }
      }
    }
  }
  return local ? plane_kernel<T, SEG, VEC, 0, 0, true> : plane_kernel<T, SEG, VEC, 0, 0, false>;
}

// the producer / consumer kernel where it is the faster one, else null:
// fp32 planes of 64 x 64, where the one-role kernel runs out of registers
// (about 0.15 against 0.21 ms for 64 x 96 such planes; at 56 x 56 and below,
// and in bf16, the one-role kernel with two workgroups per CU is as fast or
// faster). GSPN_PLANE_PC=0 turns it off, for comparisons.
template <typename T>
static void (*pick_plane_pc_kernel(int H, int W, bool local))(PlaneArgs<T>) {
  const char* env = std::getenv("GSPN_PLANE_PC");
  if (env && env[0] == '0') return nullptr;
  if constexpr (sizeof(T) == 4) {
    if (H == 64 && W == 64)
      return local ? plane_pc_kernel<T, 64, 64, true> : plane_pc_kernel<T, 64, 64, false>;
  }
  return nullptr;
}

template <typename T, int SEG, int VEC>
static hipError_t launch_plane_t(const Problem& pr, hipStream_t stream, Tracer* tr) {
  PlaneArgs<T> a;
  a.x = static_cast<const T*>(pr.x);
  a.l0 = static_cast<const T*>(pr.l[0]);
  a.l1 = static_cast<const T*>(pr.l[1]);
  a.l2 = static_cast<const T*>(pr.l[2]);
  a.lam = static_cast<const T*>(pr.lam);
  a.u = static_cast<const T*>(pr.u);
  a.out = static_cast<T*>(pr.out);
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
  const size_t lds = plane_lds_bytes(pr.H, pr.W);
  const bool local = a.G > 0;
  auto kern = pick_plane_kernel<T, SEG, VEC>(a.H, a.W, local);
  hipError_t e;
  if constexpr (SEG == 64 && VEC == 4) {
    if (auto pk = pick_plane_pc_kernel<T>(a.H, a.W, local)) {
      // two buffers of records, edge records and the zero record
      const size_t pl = 2 * (static_cast<size_t>(pr.H) * (pr.W | 1) + 2 * pr.H + 2 * pr.W + 1) *
                        sizeof(float4);
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(pk),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(pl));
      if (e != hipSuccess) return e;
      const int64_t grid = a.nplanes < cu_count() ? a.nplanes : cu_count();
      tr->before(stream, "plane_pc_kernel", a.nplanes);
      hipLaunchKernelGGL(pk, dim3(static_cast<unsigned>(grid)), dim3(512), pl, stream, a);
      tr->after(stream);
      return hipGetLastError();
    }
  }
  if (lds > 65536) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  // SEG 64 (one large plane per workgroup): persistent grid of as many
  // workgroups as are resident at once, each prefetching its next plane.
  // SEG 16 (four tiny planes per workgroup): one plane group per workgroup.
  int per_cu = 0;
  if (SEG == 64 &&
      (e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern),
                                                        256, lds)) != hipSuccess)
    return e;
  const int64_t resident = static_cast<int64_t>(per_cu > 0 ? per_cu : 1) * cu_count();
  const int64_t grid = (SEG == 16 || a.ngroups < resident) ? a.ngroups : resident;
  tr->before(stream, SEG == 16 ? "plane_kernel16" : "plane_kernel64", a.nplanes);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(256), lds, stream, a);
  tr->after(stream);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_plane_dt(const Problem& pr, hipStream_t stream, Tracer* tr) {
  // 4-wide vectors need whole rows of 4 (W % 4 == 0) and aligned pointers
  const bool vec = pr.W % 4 == 0 && pr.aligned_vec4;
  if (plane_seg(pr.H, pr.W) == 16)
    return vec ? launch_plane_t<T, 16, 4>(pr, stream, tr) : launch_plane_t<T, 16, 1>(pr, stream, tr);
  return vec ? launch_plane_t<T, 64, 4>(pr, stream, tr) : launch_plane_t<T, 64, 1>(pr, stream, tr);
}

hipError_t launch_plane(const Problem& pr, hipStream_t stream, Tracer* tr) {
  if (pr.dtype == GSPN_F32) return launch_plane_dt<float>(pr, stream, tr);
  return launch_plane_dt<bf16_t>(pr, stream, tr);
}

}  // namespace gspn

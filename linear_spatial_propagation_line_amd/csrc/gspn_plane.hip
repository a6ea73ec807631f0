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

template <typename T, int SEG, int VEC>
__global__ __launch_bounds__(256) void plane_kernel(PlaneArgs<T> a) {
  constexpr int PPB = 64 / SEG;
  // pixels per thread handled in 4-wide vectors: up to 4096 (SEG 64) or 1024
  // (SEG 16) pixels per plane group over 256 threads
  constexpr int NIT = VEC == 4 ? (SEG == 64 ? 4 : 1) : 1;
  using V = V4<T>;
  extern __shared__ float4 smem[];
  float* smem_f = reinterpret_cast<float*>(smem);

  const int H = a.H, W = a.W, pitch = a.pitch;
  const int HW = H * W;
  const int rec_sz = PPB * H * pitch;          // records (float4 units)
  const int ev_off = rec_sz;                   // [PPB][2][H]
  const int eh_off = ev_off + PPB * 2 * H;     // [PPB][2][W]
  const int zero_off = eh_off + PPB * 2 * W;   // one zero record
  const int tid = threadIdx.x;

  // registers filled one iteration ahead (VEC == 4 only)
  typename V::raw rx[NIT], rl[NIT], r0[NIT], r1[NIT], r2[NIT], ru[NIT];
  auto issue = [&](int64_t grp) {
    const int64_t gb = grp * PPB * HW;
    const int npx = static_cast<int>(min<int64_t>(PPB, a.nplanes - grp * PPB)) * HW;
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
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
      ru[it] = V::load(a.u, gi);
    }
  };
  if constexpr (VEC == 4)
    if (static_cast<int64_t>(blockIdx.x) < a.ngroups) issue(blockIdx.x);

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
        uu[it] = ru[it];
        const int i0 = tid * 4 + it * 1024;
        if (i0 < npix) {
          int rem, c;
          const int p = div_small(i0, HW, a.inv_HW, &rem);
          const int r = div_small(rem, W, a.inv_W, &c);
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
      // the next plane group's loads fly during steps 2-4
      if (grp + gridDim.x < a.ngroups) issue(grp + gridDim.x);
    } else {
      for (int i0 = tid; i0 < npix; i0 += 256) {
        int rem, c;
        const int p = div_small(i0, HW, a.inv_HW, &rem);
        const int r = div_small(rem, W, a.inv_W, &c);
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
    const int n_ev = np * 2 * H, n_eh = np * 2 * W;
    for (int k = tid; k < n_ev + n_eh; k += 256) {
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
    const int G = a.G;
    int next_restart = n_s;
    if (G > 0) next_restart = fwd ? G : n_s - ((n_s - 1) / G) * G;

    float hist[SEG];
    if (on) {
      float h = 0.0f;
#pragma unroll
      for (int s = 0; s < SEG; ++s) {
        if (s < n_s) {
          const float4 rc = smem[addr];
          addr += stride;
          const float hl = from_left<SEG>(h);
          const float hr = from_right<SEG>(h);
          const float hn = __builtin_fmaf(rc.x, hl, __builtin_fmaf(rc.y, h, __builtin_fmaf(rc.z, hr, rc.w)));
          bool restart = (s == 0);
          if (s == next_restart) { restart = true; next_restart += G; }
          h = restart ? rc.w : hn;
          hist[s] = h;
        }
      }
    }
    __syncthreads();   // every wavefront is done with the records

    // ---- 4. park states over the records, then merge ------------------------
    if (active) {
      int ya = d * rec_sz + mbase;
#pragma unroll
      for (int s = 0; s < SEG; ++s) {
        if (s < n_s) { smem_f[ya] = hist[s]; ya += mstride; }
      }
    }
    __syncthreads();

    if constexpr (VEC == 4) {
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int i0 = tid * 4 + it * 1024;
        if (i0 < npix) {
          int rem, c;
          const int pp = div_small(i0, HW, a.inv_HW, &rem);
          const int r = div_small(rem, W, a.inv_W, &c);
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
        int rem, c;
        const int pp = div_small(i0, HW, a.inv_HW, &rem);
        const int r = div_small(rem, W, a.inv_W, &c);
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
bool plane_fits(int64_t H, int64_t W) { return H >= 1 && W >= 1 && H <= 64 && W <= 64; }

int plane_seg(int64_t H, int64_t W) { return (H <= 16 && W <= 16) ? 16 : 64; }

size_t plane_lds_bytes(int64_t H, int64_t W) {
  const int seg = plane_seg(H, W);
  const int ppb = 64 / seg;
  const int pitch = static_cast<int>(W | 1);
  const size_t recs = static_cast<size_t>(ppb) * (H * pitch + 2 * H + 2 * W) + 1;
  return recs * sizeof(float4);
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
  auto kern = plane_kernel<T, SEG, VEC>;
  hipError_t e;
  if (lds > 65536) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  // SEG 64 (one large plane per workgroup): persistent grid of as many
  // workgroups as are resident at once, each prefetching its next plane.
  // SEG 16 (four tiny planes per workgroup): one plane group per workgroup.
  int per_cu = 0, dev = 0, cus = 0;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern),
                                                        256, lds)) != hipSuccess)
    return e;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if ((e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
    return e;
  const int64_t resident = static_cast<int64_t>(per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
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

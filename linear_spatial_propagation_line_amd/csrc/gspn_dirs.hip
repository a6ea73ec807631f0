// GSPN propagation with per-direction parameters and a per-channel merger:
// every scan direction d has its own lambda_d, logits l_{d,k} and gate u_d
// (x is shared), and the directions are merged with learnable per-channel
// weights, out = sum_d m[d][c] u_d (.) h_d (aitntnews page, sections
// 二维线性传播 and GSPN架构; CSDN page, section GSPN模块的设计, where a linear
// layer merges the scan directions).
//
// With separate parameters the directions share only x, so nothing is gained
// by running two directions from one read of the inputs: each direction is a
// pass of its own over the plane, in its own scan order.
//
// Planes up to 64 x 64 take dir_plane (below): one wavefront per plane, the
// four directions in turn, their sum in LDS, no workspace.
//
// Larger planes: one workgroup owns a plane (the scan couples a whole line at
// every step); the line is exchanged through a double-buffered LDS line with
// one barrier per step, and every load is a coalesced run along a row.
//
//   dir_vert       one top->bottom or bottom->top pass: thread = CPT adjacent
//                  columns, a row of every tensor is one coalesced run across
//                  the workgroup, and the loads of D rows are issued at once
//                  (clamped in-bounds addresses) before those D steps run.
//   dir_transpose  64 x 64 tiles through LDS, full 128-byte lines read and
//                  written. A left->right or right->left scan reads a column
//                  per step; read from row-major memory as short runs of
//                  every row, each run drags a whole cache line through the
//                  cache hierarchy and the lines do not survive until the
//                  next run (a 2048-row plane keeps 1.5 MB of lines open).
//                  So x and the horizontal directions' five tensors are
//                  transposed once, and left->right / right->left run as
//                  top->bottom / bottom->top passes of dir_vert over the
//                  transposed planes.
//
// Passes are chained through an fp32 accumulator: the horizontal passes
// first (in transposed layout), whose sum is transposed back; then the
// vertical passes; the first pass writes the accumulator, the middle ones add
// to it, the last one writes out = acc + m u h in the storage type. So the
// sum runs in the fixed order left->right, right->left, top->bottom,
// bottom->top, rounded once.
//
// Line recurrence and output gate: CSDN page on GSPN, section 方法;
// tridiagonal weights with sigmoid + row normalisation: section
// 如何设计一个高效的传播层; local groups: section GSPN模块的设计.
#include "gspn_device.hpp"
#include "gspn_launch.hpp"

namespace gspn {

namespace {
constexpr int kDirFirst = 1, kDirLast = 2;   // pass writes the accumulator / the output

// restart test of scan step s: the first step, or the first position of a
// local group in this scan order
__device__ __forceinline__ bool dir_restart(int s, int n_s, int G, bool fwd) {
  if (s == 0) return true;
  if (G <= 0) return false;
  return fwd ? (s % G) == 0 : ((n_s - 1 - s) % G) == G - 1;
}

// N consecutive elements of a row, kept in storage form until used
template <typename T, int N> struct Run;
template <int N> struct Run<float, N> {
  float v[N];
  // aligned vector load at element index i (i a multiple of N)
  __device__ __forceinline__ void load_vec(const float* p, int64_t i) {
    if constexpr (N % 4 == 0) {
#pragma unroll
      for (int k = 0; k < N / 4; ++k) {
        const float4 q = reinterpret_cast<const float4*>(p + i)[k];
        v[4 * k] = q.x; v[4 * k + 1] = q.y; v[4 * k + 2] = q.z; v[4 * k + 3] = q.w;
      }
    } else if constexpr (N == 2) {
      const float2 q = *reinterpret_cast<const float2*>(p + i);
      v[0] = q.x; v[1] = q.y;
    } else {
      v[0] = p[i];
    }
  }
  // elements lo .. lo+N-1 of the row starting at index row, each clamped
  // into [0, n)
  __device__ __forceinline__ void load_clamped(const float* p, int64_t row, int lo, int n) {
#pragma unroll
    for (int e = 0; e < N; ++e) v[e] = p[row + min(max(lo + e, 0), n - 1)];
  }
  __device__ __forceinline__ float get(int e) const { return v[e]; }
};
template <int N> struct Run<bf16_t, N> {
  uint32_t v[(N + 1) / 2];   // bf16 pairs, element 2k in the low half
  __device__ __forceinline__ void load_vec(const bf16_t* p, int64_t i) {
    if constexpr (N % 8 == 0) {
#pragma unroll
      for (int k = 0; k < N / 8; ++k) {
        const uint4 q = reinterpret_cast<const uint4*>(p + i)[k];
        v[4 * k] = q.x; v[4 * k + 1] = q.y; v[4 * k + 2] = q.z; v[4 * k + 3] = q.w;
      }
    } else if constexpr (N == 4) {
      const uint2 q = *reinterpret_cast<const uint2*>(p + i);
      v[0] = q.x; v[1] = q.y;
    } else if constexpr (N == 2) {
      v[0] = *reinterpret_cast<const uint32_t*>(p + i);
    } else {
      v[0] = p[i].bits;
    }
  }
  __device__ __forceinline__ void load_clamped(const bf16_t* p, int64_t row, int lo, int n) {
#pragma unroll
    for (int k = 0; k < (N + 1) / 2; ++k) v[k] = 0u;
#pragma unroll
    for (int e = 0; e < N; ++e)
      v[e >> 1] |= static_cast<uint32_t>(p[row + min(max(lo + e, 0), n - 1)].bits) << (16 * (e & 1));
  }
  __device__ __forceinline__ float get(int e) const {
    return (e & 1) ? bf16_hi(v[e >> 1]) : bf16_lo(v[e >> 1]);
  }
};

// N consecutive values to an aligned run (bf16 rounded to nearest even)
template <int N> __device__ __forceinline__ void put_run(float* p, int64_t i, const float* d) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int k = 0; k < N / 4; ++k)
      reinterpret_cast<float4*>(p + i)[k] = make_float4(d[4 * k], d[4 * k + 1], d[4 * k + 2], d[4 * k + 3]);
  } else if constexpr (N == 2) {
    *reinterpret_cast<float2*>(p + i) = make_float2(d[0], d[1]);
  } else {
    p[i] = d[0];
  }
}
template <int N> __device__ __forceinline__ void put_run(bf16_t* p, int64_t i, const float* d) {
  uint32_t w[(N + 1) / 2];
#pragma unroll
  for (int k = 0; k < N / 2; ++k)
    w[k] = pack_bf16x2(d[2 * k], d[2 * k + 1]);
  if constexpr (N % 8 == 0) {
#pragma unroll
    for (int k = 0; k < N / 8; ++k)
      reinterpret_cast<uint4*>(p + i)[k] = make_uint4(w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]);
  } else if constexpr (N == 4) {
    *reinterpret_cast<uint2*>(p + i) = make_uint2(w[0], w[1]);
  } else if constexpr (N == 2) {
    *reinterpret_cast<uint32_t*>(p + i) = w[0];
  } else {
    p[i].bits = static_cast<uint16_t>(f32_to_bf16_bits(d[0]));
  }
}
}  // namespace

template <typename T>
struct DirArgs {
  const T* x;
  const T* l0;      // this direction's logits, lambda and gate
  const T* l1;
  const T* l2;
  const T* lam;
  const T* u;
  const float* merge;   // this direction's merge weights [C], or null (all 1)
  T* out;
  float* acc;           // [planes][H][W] running sum over directions
  int64_t C;
  int64_t plane0;       // first plane of this launch
  int H, W, G;
  int mode;             // kDirFirst | kDirLast bits
};

// top->bottom (FWD) or bottom->top over row-major planes
template <typename T, int CPT, int D, bool VEC, bool FWD>
__global__ __launch_bounds__(1024) void dir_vert(DirArgs<T> a) {
  extern __shared__ float line[];   // [2][W]
  const int H = a.H, W = a.W;
  const int64_t plane = a.plane0 + blockIdx.x;
  const int64_t base = plane * H * W;
  const float m = a.merge ? a.merge[plane % a.C] : 1.f;
  const bool first = a.mode & kDirFirst, last = a.mode & kDirLast;
  const int o0 = threadIdx.x * CPT;
  const int lo = VEC ? min(o0, W - CPT) : o0;   // in-bounds run start
  float hp[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) hp[k] = 0.f;

  for (int s0 = 0; s0 < H; s0 += D) {
    Run<T, CPT> rx[D], rl[D], r0[D], r1[D], r2[D], ru[D];
    Run<float, CPT> ra[D];
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int s = min(s0 + j, H - 1);
      const int64_t row = base + static_cast<int64_t>(FWD ? s : H - 1 - s) * W;
      if constexpr (VEC) {
        rx[j].load_vec(a.x, row + lo);
        rl[j].load_vec(a.lam, row + lo);
        r0[j].load_vec(a.l0, row + lo);
        r1[j].load_vec(a.l1, row + lo);
        r2[j].load_vec(a.l2, row + lo);
        ru[j].load_vec(a.u, row + lo);
        if (!first) ra[j].load_vec(a.acc, row + lo);
      } else {
        rx[j].load_clamped(a.x, row, lo, W);
        rl[j].load_clamped(a.lam, row, lo, W);
        r0[j].load_clamped(a.l0, row, lo, W);
        r1[j].load_clamped(a.l1, row, lo, W);
        r2[j].load_clamped(a.l2, row, lo, W);
        ru[j].load_clamped(a.u, row, lo, W);
        if (!first) ra[j].load_clamped(a.acc, row, lo, W);
      }
    }
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int s = s0 + j;
      if (s >= H) break;   // uniform
      const bool restart = dir_restart(s, H, a.G, FWD);
      const int64_t row = base + static_cast<int64_t>(FWD ? s : H - 1 - s) * W;
      float* cur = line + (s & 1) * W;
      const float* prev = line + ((s & 1) ^ 1) * W;
      const float left = prev[min(max(o0 - 1, 0), W - 1)];
      const float right = prev[min(o0 + CPT, W - 1)];
      float hn[CPT], yv[CPT];
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        const int o = o0 + k;
        float h = rl[j].get(k) * rx[j].get(k);
        if (!restart) {
          const Weights w = make_weights(r0[j].get(k), r1[j].get(k), r2[j].get(k),
                                         o > 0 ? 1.f : 0.f, o < W - 1 ? 1.f : 0.f);
          const float hl = k > 0 ? hp[k - 1] : left;
          const float hr = k < CPT - 1 ? hp[k + 1] : right;
          h = __builtin_fmaf(w.w0, hl, __builtin_fmaf(w.w1, hp[k], __builtin_fmaf(w.w2, hr, h)));
        }
        hn[k] = h;
        const float y = (m * ru[j].get(k)) * h;
        yv[k] = first ? y : ra[j].get(k) + y;
      }
#pragma unroll
      for (int k = 0; k < CPT; ++k) {
        hp[k] = hn[k];
        if (o0 + k < W) cur[o0 + k] = hn[k];
      }
      if constexpr (VEC) {
        if (o0 < W) {
          if (last) put_run<CPT>(a.out, row + o0, yv);
          else put_run<CPT>(a.acc, row + o0, yv);
        }
      } else {
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
          if (o0 + k < W) {
            if (last) Store<T>::put(a.out, row + o0 + k, yv[k]);
            else a.acc[row + o0 + k] = yv[k];
          }
        }
      }
      __syncthreads();
    }
  }
}

// dst[k] = src[k] transposed plane by plane ([planes][R][C] -> [planes][C][R])
// for the tensors k = blockIdx.y, converting the element type on the way
template <typename S, typename Dt>
struct TrArgs {
  const S* src[11];
  Dt* dst[11];
  int64_t planes;
  int R, C;
};

namespace {
__device__ __forceinline__ float tr_ld(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float tr_ld(const bf16_t* p, int64_t i) { return to_f32(p[i]); }
}  // namespace

template <typename S, typename Dt>
__global__ __launch_bounds__(256) void dir_transpose(TrArgs<S, Dt> a) {
  __shared__ float tile[64][65];
  const int R = a.R, C = a.C;
  const int tr = (R + 63) / 64, tc = (C + 63) / 64;
  const int64_t tiles = a.planes * tr * tc;
  const S* src0 = a.src[blockIdx.y];
  Dt* dst0 = a.dst[blockIdx.y];
  const int cx = threadIdx.x & 63, ry = threadIdx.x >> 6;
  for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const int64_t p = t / (tr * tc);
    const int rem = static_cast<int>(t - p * tr * tc);
    const int r0 = (rem / tc) * 64, c0 = (rem % tc) * 64;
    const S* src = src0 + p * R * C;
    Dt* dst = dst0 + p * R * C;
#pragma unroll
    for (int i = 0; i < 64; i += 4) {
      const int r = r0 + ry + i, c = c0 + cx;
      if (r < R && c < C) tile[ry + i][cx] = tr_ld(src, static_cast<int64_t>(r) * C + c);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 64; i += 4) {
      const int c = c0 + ry + i, r = r0 + cx;
      if (c < C && r < R) Store<Dt>::put(dst, static_cast<int64_t>(c) * R + r, tile[cx][ry + i]);
    }
    __syncthreads();
  }
}

// The same for bf16 planes with even sides and 4-byte aligned tensors, two
// adjacent elements per lane on both sides (4-byte accesses, 256-byte rows)
// over tiles of 64 rows x 128 columns: a lane loads a column pair of one
// source row and stores a pair of adjacent source rows into one destination
// row.
__global__ __launch_bounds__(256) void dir_transpose_pairs(TrArgs<bf16_t, bf16_t> a) {
  __shared__ uint16_t tile[64][130];
  const int R = a.R, C = a.C;
  const int tr = (R + 63) / 64, tc = (C + 127) / 128;
  const int64_t tiles = a.planes * tr * tc;
  const uint16_t* src0 = reinterpret_cast<const uint16_t*>(a.src[blockIdx.y]);
  uint16_t* dst0 = reinterpret_cast<uint16_t*>(a.dst[blockIdx.y]);
  const int cp = threadIdx.x & 63, ry = threadIdx.x >> 6;   // load: column pair, row
  const int rp = threadIdx.x & 31, cy = threadIdx.x >> 5;   // store: row pair, column
  for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const int64_t p = t / (tr * tc);
    const int rem = static_cast<int>(t - p * tr * tc);
    const int r0 = (rem / tc) * 64, c0 = (rem % tc) * 128;
    const uint16_t* src = src0 + p * R * C;
    uint16_t* dst = dst0 + p * R * C;
#pragma unroll
    for (int i = 0; i < 64; i += 4) {
      const int r = r0 + ry + i, c = c0 + 2 * cp;
      if (r < R && c < C)
        *reinterpret_cast<uint32_t*>(&tile[ry + i][2 * cp]) =
            *reinterpret_cast<const uint32_t*>(src + static_cast<int64_t>(r) * C + c);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 128; i += 8) {
      const int c = c0 + cy + i, r = r0 + 2 * rp;
      if (c < C && r < R) {
        const uint32_t v = static_cast<uint32_t>(tile[2 * rp][cy + i]) |
                           (static_cast<uint32_t>(tile[2 * rp + 1][cy + i]) << 16);
        *reinterpret_cast<uint32_t*>(dst + static_cast<int64_t>(c) * R + r) = v;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Small planes (H, W <= 64): one wavefront per plane, no line in LDS and no
// barrier. Lane o is orthogonal index o of every scan of the plane; it walks
// the scan axis with its state in a register and takes its neighbours'
// previous states by DPP (lane o - 1 holds offset -1 for all four directions).
// Each direction streams its own five tensors: a vertical scan loads one row
// per step, a coalesced run across the lanes; a horizontal scan loads four
// consecutive columns of its row per lane at once (16 or 8 bytes) when the
// row length and every pointer allow, else one element per step. The sum over
// the directions, m[d][c] u_d h_d, stays in LDS ([H][W + 1] fp32 per plane:
// rows and columns of it are both conflict-free) and is written once, in the
// direction order T2B, B2T, L2R, R2L, with one rounding to the storage type.
// Every input is read from HBM once, out written once.
template <typename T>
struct DpArgs {
  const T* x;
  const T* l0;
  const T* l1;
  const T* l2;
  const T* lam;
  const T* u;
  int64_t dir_stride;   // elements between two directions' parameter sets
  const float* merge;   // [4][C] merge weights, or null (all 1)
  T* out;
  int64_t nplanes, C;
  int H, W, G;
  unsigned mask;
};

template <typename T, bool VEC>
__global__ __launch_bounds__(256) void dir_plane(DpArgs<T> a) {
  extern __shared__ float ysum[];   // [4 wavefronts][H][W + 1]
  constexpr int D = 8;              // steps per batch of loads
  const int wave = threadIdx.x >> 6, o = threadIdx.x & 63;
  const int64_t plane = static_cast<int64_t>(blockIdx.x) * 4 + wave;
  if (plane >= a.nplanes) return;   // the whole wavefront
  const int H = a.H, W = a.W, P = W + 1, G = a.G;
  float* acc = ysum + wave * H * P;
  const int64_t base = plane * H * W;
  const int64_t ch = plane % a.C;
  bool first = true;
  for (int d = 0; d < 4; ++d) {
    if (!((a.mask >> d) & 1u)) continue;
    const int64_t off = d * a.dir_stride;
    const T* lam = a.lam + off;
    const T* l0 = a.l0 + off;
    const T* l1 = a.l1 + off;
    const T* l2 = a.l2 + off;
    const T* u = a.u + off;
    const float m = a.merge ? a.merge[d * a.C + ch] : 1.f;
    const bool vert = d < 2, fwd = (d == 0 || d == 2);
    const int n_s = vert ? H : W, n_o = vert ? W : H;
    const bool act = o < n_o;
    const int oc = act ? o : n_o - 1;   // clamped, for loads only
    const float m0 = o > 0 ? 1.f : 0.f, m2 = o < n_o - 1 ? 1.f : 0.f;
    // restarts after step 0: every G steps from the first block edge met
    int next = n_s;
    if (G > 0) next = fwd ? G : n_s - ((n_s - 1) / G) * G;
    float h = 0.f;
    // one step at scan position pos (row of a vertical scan, column of a
    // horizontal one) from its lambda x, logits and u
    auto step = [&](int s, int pos, float lx, float g0, float g1, float g2, float uv) {
      const Weights w = make_weights(g0, g1, g2, m0, m2);
      const float hn = line_step<64>(h, w.w0, w.w1, w.w2, lx);
      bool restart = s == 0;
      if (s == next) { restart = true; next += G; }
      h = act ? (restart ? lx : hn) : 0.f;
      if (act) {
        float* q = acc + (vert ? pos * P + o : o * P + pos);
        const float v = m * uv * h;
        *q = first ? v : *q + v;
      }
    };
    if (vert || !VEC) {
      for (int s0 = 0; s0 < n_s; s0 += D) {
        float lx[D], g0[D], g1[D], g2[D], uv[D];
#pragma unroll
        for (int j = 0; j < D; ++j) {
          const int s = min(s0 + j, n_s - 1);
          const int pos = fwd ? s : n_s - 1 - s;
          const int64_t i = base + (vert ? static_cast<int64_t>(pos) * W + oc
                                         : static_cast<int64_t>(oc) * W + pos);
          lx[j] = tr_ld(lam, i) * tr_ld(a.x, i);
          g0[j] = tr_ld(l0, i);
          g1[j] = tr_ld(l1, i);
          g2[j] = tr_ld(l2, i);
          uv[j] = tr_ld(u, i);
        }
#pragma unroll
        for (int j = 0; j < D; ++j) {
          const int s = s0 + j;
          if (s >= n_s) break;   // uniform
          step(s, fwd ? s : n_s - 1 - s, lx[j], g0[j], g1[j], g2[j], uv[j]);
        }
      }
    } else {
      // horizontal, W % 4 == 0: each lane loads 64 bytes of its row per
      // tensor at once (NQ runs of 4 columns), so that a 64-byte sector is
      // fetched whole; partial sectors refetched run by run cost several
      // times the bytes, since the rows of all the wavefronts in flight do
      // not stay in L2 between runs. Left->right takes columns s0 .. in
      // order; right->left the runs from the right end, used from the top.
      using V = V4<T>;
      constexpr int NQ = 64 / (4 * static_cast<int>(sizeof(T)));
      const int64_t row = base + static_cast<int64_t>(oc) * W;
      for (int s0 = 0; s0 < n_s; s0 += 4 * NQ) {
        typename V::raw vx[NQ], vl[NQ], v0[NQ], v1[NQ], v2[NQ], vu[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          // runs past the end of the row repeat its last run (in bounds)
          const int c4 = min(s0 + 4 * q, n_s - 4);
          const int64_t i = row + (fwd ? c4 : n_s - 4 - c4);
          vx[q] = V::load(a.x, i);
          vl[q] = V::load(lam, i);
          v0[q] = V::load(l0, i);
          v1[q] = V::load(l1, i);
          v2[q] = V::load(l2, i);
          vu[q] = V::load(u, i);
        }
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int s = s0 + 4 * q + j;
            if (s < n_s) {   // uniform
              const int e = fwd ? j : 3 - j;
              step(s, fwd ? s : n_s - 1 - s, V::get(vl[q], e) * V::get(vx[q], e),
                   V::get(v0[q], e), V::get(v1[q], e), V::get(v2[q], e), V::get(vu[q], e));
            }
          }
        }
      }
    }
    first = false;
  }
  // the plane's sum, row by row
  if (o < W)
    for (int r = 0; r < H; ++r) Store<T>::put(a.out, base + static_cast<int64_t>(r) * W + o, acc[r * P + o]);
}

int64_t dirs_max_orth() { return 8192; }

size_t dirs_workspace_bytes(int64_t planes, int64_t H, int64_t W, uint32_t mask,
                            gspn_dtype dt) {
  if (plane_fits(H, W)) return 0;   // one wavefront per plane, no workspace
  const size_t P = static_cast<size_t>(planes * H * W);
  const size_t es = dt == GSPN_F32 ? 4 : 2;
  auto al = [](size_t v) { return (v + 255) & ~size_t(255); };
  const int nh = __builtin_popcount(mask & 12u), nv = __builtin_popcount(mask & 3u);
  if (nh == 0) return nv > 1 ? P * sizeof(float) : 0;
  // transposed accumulator, row-major accumulator (vertical passes after the
  // horizontal ones), transposed x and five tensors per horizontal direction
  return al(P * sizeof(float)) + (nv > 0 ? al(P * sizeof(float)) : 0) +
         static_cast<size_t>(1 + 5 * nh) * al(P * es);
}

namespace {
int round64(int64_t n) { return static_cast<int>((n + 63) / 64 * 64); }

bool aligned_to(const void* const* p, int n, size_t bytes) {
  for (int i = 0; i < n; ++i)
    if (reinterpret_cast<uintptr_t>(p[i]) % bytes) return false;
  return true;
}

template <typename T, int CPT, int D, bool FWD>
hipError_t vert_pass(const DirArgs<T>& a, bool vec, int64_t planes, hipStream_t stream,
                     Tracer* tr) {
  const int threads = round64((a.W + CPT - 1) / CPT);
  const size_t lds = static_cast<size_t>(2 * a.W) * sizeof(float);
  auto kern = vec ? dir_vert<T, CPT, D, true, FWD> : dir_vert<T, CPT, D, false, FWD>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  tr->before(stream, "dir_vert", planes);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(planes)), dim3(threads), lds, stream, a);
  tr->after(stream);
  return hipGetLastError();
}

// one pass over planes of a.H rows x a.W columns: CPT columns per thread so
// that a workgroup has at most 1024 threads, D rows per load batch
template <typename T>
hipError_t vert_dispatch(const DirArgs<T>& a, bool fwd, int64_t planes, hipStream_t stream,
                         Tracer* tr) {
  const int W = a.W;
  const int cpt = W <= 1024 ? 1 : (W <= 2048 ? 2 : (W <= 4096 ? 4 : 8));
  const void* ptrs[7] = {a.x, a.l0, a.l1, a.l2, a.lam, a.u, a.out};
  const bool vec = cpt > 1 && W % cpt == 0 && aligned_to(ptrs, 7, cpt * sizeof(T)) &&
                   reinterpret_cast<uintptr_t>(a.acc) % (cpt * sizeof(float)) == 0;
  if (fwd) {
    switch (cpt) {
      case 1: return vert_pass<T, 1, 8, true>(a, false, planes, stream, tr);
      case 2: return vert_pass<T, 2, 4, true>(a, vec, planes, stream, tr);
      case 4: return vert_pass<T, 4, 2, true>(a, vec, planes, stream, tr);
      default: return vert_pass<T, 8, 1, true>(a, vec, planes, stream, tr);
    }
  }
  switch (cpt) {
    case 1: return vert_pass<T, 1, 8, false>(a, false, planes, stream, tr);
    case 2: return vert_pass<T, 2, 4, false>(a, vec, planes, stream, tr);
    case 4: return vert_pass<T, 4, 2, false>(a, vec, planes, stream, tr);
    default: return vert_pass<T, 8, 1, false>(a, vec, planes, stream, tr);
  }
}

template <typename S, typename Dt>
hipError_t transpose(const S* const* src, Dt* const* dst, int n, int64_t planes, int R, int C,
                     const char* name, hipStream_t stream, Tracer* tr) {
  TrArgs<S, Dt> t;
  for (int i = 0; i < 11; ++i) {
    t.src[i] = i < n ? src[i] : nullptr;
    t.dst[i] = i < n ? dst[i] : nullptr;
  }
  t.planes = planes;
  t.R = R;
  t.C = C;
  bool pairs = false;
  if constexpr (sizeof(S) == 2 && sizeof(Dt) == 2) {
    pairs = R % 2 == 0 && C % 2 == 0;
    for (int i = 0; i < n; ++i)
      pairs = pairs && reinterpret_cast<uintptr_t>(src[i]) % 4 == 0 &&
              reinterpret_cast<uintptr_t>(dst[i]) % 4 == 0;
  }
  const int64_t tiles = planes * ((R + 63) / 64) * ((C + (pairs ? 127 : 63)) / (pairs ? 128 : 64));
  const int64_t grid = tiles < 65536 ? tiles : 65536;
  tr->before(stream, name, planes * n);
  if constexpr (sizeof(S) == 2 && sizeof(Dt) == 2) {
    if (pairs) {
      hipLaunchKernelGGL(dir_transpose_pairs, dim3(static_cast<unsigned>(grid), n), dim3(256), 0,
                         stream, t);
      tr->after(stream);
      return hipGetLastError();
    }
  }
  auto kern = dir_transpose<S, Dt>;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid), n), dim3(256), 0, stream, t);
  tr->after(stream);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dir_plane(const Problem& pr, hipStream_t stream, Tracer* tr) {
  DpArgs<T> a;
  a.x = static_cast<const T*>(pr.x);
  a.l0 = static_cast<const T*>(pr.l[0]);
  a.l1 = static_cast<const T*>(pr.l[1]);
  a.l2 = static_cast<const T*>(pr.l[2]);
  a.lam = static_cast<const T*>(pr.lam);
  a.u = static_cast<const T*>(pr.u);
  a.dir_stride = pr.dir_stride;
  a.merge = pr.merge;
  a.out = static_cast<T*>(pr.out);
  a.nplanes = pr.B * pr.C;
  a.C = pr.C;
  a.H = static_cast<int>(pr.H);
  a.W = static_cast<int>(pr.W);
  a.G = static_cast<int>(pr.G >= pr.H && pr.G >= pr.W ? 0 : pr.G);
  a.mask = pr.mask;
  // four-column loads for the horizontal scans: whole runs of 4 in a row and
  // every tensor they read aligned to 4 elements
  bool vec = pr.W % 4 == 0 && reinterpret_cast<uintptr_t>(a.x) % (4 * sizeof(T)) == 0;
  for (int d = 2; d < 4; ++d) {
    if (!((pr.mask >> d) & 1u)) continue;
    const void* p[5] = {a.lam + d * a.dir_stride, a.l0 + d * a.dir_stride,
                        a.l1 + d * a.dir_stride, a.l2 + d * a.dir_stride, a.u + d * a.dir_stride};
    vec = vec && aligned_to(p, 5, 4 * sizeof(T));
  }
  const size_t lds = static_cast<size_t>(4 * pr.H * (pr.W + 1)) * sizeof(float);
  auto kern = vec ? dir_plane<T, true> : dir_plane<T, false>;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(lds));
    if (e != hipSuccess) return e;
  }
  tr->before(stream, "dir_plane", a.nplanes);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>((a.nplanes + 3) / 4)), dim3(256), lds, stream,
                     a);
  tr->after(stream);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_dirs_dt(const Problem& pr, void* ws, hipStream_t stream, Tracer* tr) {
  if (plane_fits(pr.H, pr.W)) return launch_dir_plane<T>(pr, stream, tr);
  const int64_t planes = pr.B * pr.C;
  const int64_t P = planes * pr.H * pr.W;
  const int H = static_cast<int>(pr.H), W = static_cast<int>(pr.W);
  auto al = [](size_t v) { return (v + 255) & ~size_t(255); };
  const int nh = __builtin_popcount(pr.mask & 12u), nv = __builtin_popcount(pr.mask & 3u);
  const T* xs = static_cast<const T*>(pr.x);
  auto param = [&](const void* base, int d) {
    return static_cast<const T*>(base) + d * pr.dir_stride;
  };
  DirArgs<T> a;
  a.merge = nullptr;
  a.out = static_cast<T*>(pr.out);
  a.C = pr.C;
  a.plane0 = 0;
  a.G = static_cast<int>(pr.G);
  char* wsb = static_cast<char*>(ws);
  const int64_t HW = pr.H * pr.W;

  // every launch for planes [p0, p0 + np) on stream st; planes are
  // independent throughout (their own slices of every buffer)
  auto run_group = [&](int64_t p0, int64_t np, hipStream_t st) -> hipError_t {
    const int64_t o = p0 * HW;   // element offset of the group in a [planes][H][W] tensor
    DirArgs<T> ag = a;
    ag.plane0 = p0;
    float* acc = static_cast<float*>(ws);   // row-major sum (vertical passes)
    int pass = 0;                           // passes run so far
    hipError_t e;
    if (nh > 0) {
      // workspace: [transposed sum][row-major sum][x^T][5 tensors^T per direction]
      float* acc_t = reinterpret_cast<float*>(wsb);
      size_t off = al(P * sizeof(float));
      if (nv > 0) {
        acc = reinterpret_cast<float*>(wsb + off);
        off += al(P * sizeof(float));
      }
      // whole tensors (the kernels address planes from plane0), and the
      // group's slices for the transposes
      const T* src[11];
      T* dst[11];
      const T* gsrc[11];
      T* gdst[11];
      int n = 0;
      src[n] = xs;
      dst[n++] = reinterpret_cast<T*>(wsb + off);
      off += al(P * sizeof(T));
      // with dir_stride 0 both horizontal directions read the same five
      // tensors: they are transposed once
      const bool shared_h = pr.dir_stride == 0;
      for (int d = 2; d < 4; ++d) {
        if (!((pr.mask >> d) & 1u)) continue;
        if (shared_h && n > 1) break;
        const void* bases[5] = {pr.lam, pr.l[0], pr.l[1], pr.l[2], pr.u};
        for (int k = 0; k < 5; ++k) {
          src[n] = param(bases[k], d);
          dst[n++] = reinterpret_cast<T*>(wsb + off);
          off += al(P * sizeof(T));
        }
      }
      for (int k = 0; k < n; ++k) {
        gsrc[k] = src[k] + o;
        gdst[k] = dst[k] + o;
      }
      e = transpose<T, T>(gsrc, gdst, n, np, H, W, "dir_tr_in", st, tr);
      if (e != hipSuccess) return e;
      // left->right and right->left as top->bottom and bottom->top passes over
      // the transposed planes (W rows of H), into the transposed sum
      int t = 1;
      for (int d = 2; d < 4; ++d) {
        if (!((pr.mask >> d) & 1u)) continue;
        ag.x = dst[0];
        ag.lam = dst[t];
        ag.l0 = dst[t + 1];
        ag.l1 = dst[t + 2];
        ag.l2 = dst[t + 3];
        ag.u = dst[t + 4];
        if (!shared_h) t += 5;
        ag.merge = pr.merge ? pr.merge + d * pr.C : nullptr;
        ag.acc = acc_t;
        ag.H = W;
        ag.W = H;
        ag.mode = (pass == 0 ? kDirFirst : 0);
        e = vert_dispatch<T>(ag, d == 2, np, st, tr);
        if (e != hipSuccess) return e;
        ++pass;
      }
      // back to row-major: into the sum the vertical passes continue, or, with
      // no vertical direction, straight into out
      const float* s1[1] = {acc_t + o};
      if (nv > 0) {
        float* d1[1] = {acc + o};
        e = transpose<float, float>(s1, d1, 1, np, W, H, "dir_tr_acc", st, tr);
      } else {
        T* d1[1] = {static_cast<T*>(pr.out) + o};
        e = transpose<float, T>(s1, d1, 1, np, W, H, "dir_tr_acc", st, tr);
      }
      if (e != hipSuccess) return e;
    }
    int done_v = 0;
    for (int d = 0; d < 2; ++d) {
      if (!((pr.mask >> d) & 1u)) continue;
      ag.x = xs;
      ag.lam = param(pr.lam, d);
      ag.l0 = param(pr.l[0], d);
      ag.l1 = param(pr.l[1], d);
      ag.l2 = param(pr.l[2], d);
      ag.u = param(pr.u, d);
      ag.merge = pr.merge ? pr.merge + d * pr.C : nullptr;
      ag.acc = acc;
      ag.H = H;
      ag.W = W;
      ++done_v;
      ag.mode = (pass == 0 ? kDirFirst : 0) | (done_v == nv ? kDirLast : 0);
      e = vert_dispatch<T>(ag, d == 0, np, st, tr);
      if (e != hipSuccess) return e;
      ++pass;
    }
    return hipSuccess;
  };
  // A pass gives each plane one compute unit: plane groups on their own
  // streams let one group's tail overlap another group's next launch.
  return run_plane_groups(planes, stream, run_group);
}
}  // namespace

template <typename E>
hipError_t transpose_planes(const E* const* src, E* const* dst, int n, int64_t planes, int R, int C,
                            const char* name, hipStream_t stream, Tracer* tr) {
  return transpose<E, E>(src, dst, n, planes, R, C, name, stream, tr);
}
template hipError_t transpose_planes<float>(const float* const*, float* const*, int, int64_t, int,
                                            int, const char*, hipStream_t, Tracer*);
template hipError_t transpose_planes<bf16_t>(const bf16_t* const*, bf16_t* const*, int, int64_t,
                                             int, int, const char*, hipStream_t, Tracer*);

hipError_t launch_dirs(const Problem& pr, void* ws, hipStream_t stream, Tracer* tr) {
  if (pr.dtype == GSPN_F32) return launch_dirs_dt<float>(pr, ws, stream, tr);
  return launch_dirs_dt<bf16_t>(pr, ws, stream, tr);
}

}  // namespace gspn

// Backward pass of the GSPN propagation for large planes (both sides even,
// W <= 1024, H <= 2048): the counterpart of the forward transpose pipeline.
//
// Per scan direction (CSDN page on GSPN, section 反向传播) the error term of
// a line collects what the next line in scan order sends back through the
// transposed tridiagonal weights,
//   e_s[o] = u gy + w_{s+1,0}[o+1] e_{s+1}[o+1] + w_{s+1,1}[o] e_{s+1}[o]
//                 + w_{s+1,2}[o-1] e_{s+1}[o-1],
// and, summed over the directions, d(lambda x) = sum_d e_d, du = gy sum_d h_d,
//   dl_k = sum_d e_d w_k (1 - sigmoid(l_k)) (h_{s-1}[o+k-1] - sum_j w_j h_{s-1}[o+j-1]).
//
// The two scans of one axis pair up. A sweep in one order runs the forward
// recurrence of the direction that scans that way together with the
// error-term recurrence of the opposite direction, which walks the same way.
// Both use the weights of the same pixels, and a line that restarts the
// first is exactly a line after which the second receives nothing, so one
// restart test serves both. The sweep in the other order then has, at every
// pixel, both states and both error terms the gradients need:
//
//   bt_vA  top->bottom over the row-major inputs: h of top->bottom and e of
//          bottom->top, stored per pixel; writes the column-major copy
//          (lambda x and u gy in fp32, the logits in the storage type, in
//          column quads written as whole lines by lane pairs) that the
//          horizontal sweeps read as contiguous lines.
//   bt_hA  left->right over the copy: h of left->right and e of right->left,
//          stored per pixel.
//   bt_hB  right->left over the copy: h of right->left and e of left->right;
//          with bt_hA's values it forms the horizontal parts of d(lambda x),
//          the three logit gradients and sum h, written in fp32 in tiles of
//          4 rows x 4 columns; the right column pair of a tile waits in LDS
//          for its left pair, so each thread writes 32 contiguous bytes.
//   bt_vB  bottom->top over the row-major inputs: h of bottom->top and e of
//          top->bottom; with bt_vA's values and the horizontal parts it
//          writes the six gradients once.
//
// One workgroup per plane in every launch: a thread owns two adjacent
// positions of the line (the orthogonal axis), neighbours exchange their
// states and w e products through a double-buffered LDS line with one
// barrier per step, and each thread keeps the loads of several steps in
// flight at clamped, unconditional addresses.
#include <algorithm>
#include <type_traits>

#include "gspn_device.hpp"
#include "gspn_quad.hpp"
#include "gspn_launch.hpp"

namespace gspn {

namespace {

// The horizontal parts are stored in tiles of 4 rows x 4 columns (64 bytes,
// row-major inside): bt_hB writes a thread's two rows of a tile as 32
// contiguous bytes, and bt_vB reads a tile's rows on consecutive steps, so
// each tile is used while it is still in L2.
constexpr int kGrp = 4;          // rows per tile
constexpr int kTc = 4;           // columns per tile
constexpr int kNone = 1 << 30;

// two adjacent elements in their storage form
template <typename T> struct Two;
template <> struct Two<float> {
  using raw = float2;
  __device__ static raw load(const float* p, int64_t i) {
    return *reinterpret_cast<const float2*>(p + i);
  }
  __device__ static float lo(raw v) { return v.x; }
  __device__ static float hi(raw v) { return v.y; }
  __device__ static void store(float* p, int64_t i, float a, float b) {
    *reinterpret_cast<float2*>(p + i) = make_float2(a, b);
  }
};
template <> struct Two<bf16_t> {
  using raw = uint32_t;
  __device__ static raw load(const bf16_t* p, int64_t i) {
    return *reinterpret_cast<const uint32_t*>(p + i);
  }
  __device__ static float lo(raw v) { return bf16_lo(v); }
  __device__ static float hi(raw v) { return bf16_hi(v); }
  __device__ static void store(bf16_t* p, int64_t i, float a, float b) {
    *reinterpret_cast<uint32_t*>(p + i) = pack_bf16x2(a, b);
  }
};

// Rows o, o+1 of a column pair, as (o, even), (o, odd), (o+1, even),
// (o+1, odd): the pair's half of two rows of a quad of the copy.
template <typename T> struct Four;
template <> struct Four<float> {
  using raw = float4;
  // the pair's values in two rows of a quad copy (rows 4 elements apart)
  __device__ static raw load_rows(const float* p, int64_t i) {
    const float2 r0 = *reinterpret_cast<const float2*>(p + i);
    const float2 r1 = *reinterpret_cast<const float2*>(p + i + 4);
    return make_float4(r0.x, r0.y, r1.x, r1.y);
  }
  __device__ static float get(const raw& v, int row, int odd) {
    return row ? (odd ? v.w : v.z) : (odd ? v.y : v.x);
  }
};
template <> struct Four<bf16_t> {
  using raw = uint2;
  __device__ static raw load_rows(const bf16_t* p, int64_t i) {
    return make_uint2(*reinterpret_cast<const uint32_t*>(p + i),
                      *reinterpret_cast<const uint32_t*>(p + i + 4));
  }
  __device__ static float get(const raw& v, int row, int odd) {
    const uint32_t w = row ? v.y : v.x;
    return odd ? bf16_hi(w) : bf16_lo(w);
  }
};
__device__ __forceinline__ float quad(const float4& v, int row, int odd) {
  return row ? (odd ? v.w : v.z) : (odd ? v.y : v.x);
}

// Barrier for the LDS line alone: global loads and stores of the thread stay
// in flight (a full __syncthreads would wait for all of them).
__device__ __forceinline__ void line_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Restart tests without a division per step. A scan in increasing position
// restarts at 0 and at every multiple of G; one in decreasing position at
// n - 1 and at every mG - 1 (G = 0: global).
struct StartsUp {     // walking up: p == 0 or p % G == 0
  int next, G;
  __device__ bool at(int p) {
    const bool r = p == next;
    next = r ? (G > 0 ? p + G : kNone) : next;
    return r;
  }
};
struct StartsDown {   // walking down: p == 0 or p % G == 0
  int next, G;
  __device__ bool at(int p) {
    const bool r = p == next;
    next = r ? (G > 0 ? p - G : -kNone) : next;
    return r;
  }
};
__device__ __forceinline__ StartsDown starts_down(int n, int G) {
  return StartsDown{G > 0 ? (n - 1) / G * G : 0, G};
}
struct EndsDown {     // walking down: p == n - 1 or p % G == G - 1
  int next, G, last, after_last;
  __device__ bool at(int p) {
    const bool r = p == next;
    next = r ? (p == last ? after_last : p - G) : next;
    return r;
  }
};
__device__ __forceinline__ EndsDown ends_down(int n, int G) {
  // below n - 1 the next end is the largest mG - 1 < n - 1
  return EndsDown{n - 1, G, n - 1, G > 0 ? (n - 1) / G * G - 1 : -kNone};
}

// Line exchange: slot t + 1 holds thread t's (h_A, h_B, w_0 e_A, w_2 e_B) of
// the last line; slots 0 and n + 1, and those of threads without positions,
// stay zero, which is what a missing neighbour contributes.
struct Line {
  float4* buf;   // [2][slots]
  int slots, par;
};

__device__ __forceinline__ void line_clear(float4* buf, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) buf[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  line_barrier();
}

// Running values of a sweep for the thread's positions A = o0, B = o0 + 1.
struct Sweep {
  float hA, hB;             // forward state of the direction scanning this way
  float eA, eB;             // error term of the opposite direction
  float k0, k1A, k1B, k2;   // own w e products of the last line that the next
                            // line's error terms take: w0(B) eB, w1(A) eA,
                            // w1(B) eB, w2(A) eA
};

// One step: the neighbours' last line (L = left thread, R = right thread),
// this line's weights, lambda x and u gy. A restart line takes lambda x as
// its state and u gy as its error term.
__device__ __forceinline__ void advance(Sweep& s, const float4& L, const float4& R,
                                        const Weights& wa, const Weights& wb, float lxa,
                                        float lxb, float uga, float ugb, bool restart) {
  const float hA = __builtin_fmaf(wa.w0, L.y, __builtin_fmaf(wa.w1, s.hA, __builtin_fmaf(wa.w2, s.hB, lxa)));
  const float hB = __builtin_fmaf(wb.w0, s.hA, __builtin_fmaf(wb.w1, s.hB, __builtin_fmaf(wb.w2, R.x, lxb)));
  const float eA = uga + (s.k1A + (s.k0 + L.w));
  const float eB = ugb + (s.k1B + (s.k2 + R.z));
  s.hA = restart ? lxa : hA;
  s.hB = restart ? lxb : hB;
  s.eA = restart ? uga : eA;
  s.eB = restart ? ugb : eB;
  s.k0 = wb.w0 * s.eB;
  s.k1A = wa.w1 * s.eA;
  s.k1B = wb.w1 * s.eB;
  s.k2 = wa.w2 * s.eA;
}

// Writes the thread's slot of the next line (and, when `side` is given, its
// slot of a second double-buffered float2 line that travels with it), then
// waits for the whole line.
__device__ __forceinline__ void publish(const Sweep& s, Line& ln, int t, bool act, float wa0,
                                        float wb2, float2* side = nullptr,
                                        float2 sv = float2{0.f, 0.f}) {
  if (act) {
    ln.buf[(ln.par ^ 1) * ln.slots + t + 1] = make_float4(s.hA, s.hB, wa0 * s.eA, wb2 * s.eB);
    if (side) side[(ln.par ^ 1) * ln.slots + t + 1] = sv;
  }
  ln.par ^= 1;
  line_barrier();
}

__device__ __forceinline__ Weights weights_of(const WeightSlopes& q) {
  return Weights{q.w0, q.w1, q.w2};
}

// Logit gradients of one pixel for one direction: error term e, the previous
// line's states at offsets -1, 0, +1. h_k - sum_j w_j h_j is formed from
// differences of neighbouring states (sum_j w_j = 1), so it is exactly zero
// where the neighbours agree.
struct G3 {
  float g0, g1, g2;
};
__device__ __forceinline__ G3 logit_grads(const WeightSlopes& q, float e, float hl, float hc,
                                          float hr) {
  const float d01 = hl - hc, d12 = hc - hr, d02 = hl - hr;
  G3 g;
  g.g0 = e * q.q0 * (q.w1 * d01 + q.w2 * d02);
  g.g1 = e * q.q1 * (q.w2 * d12 - q.w0 * d01);
  g.g2 = -(e * q.q2 * (q.w0 * d02 + q.w1 * d12));
  return g;
}

// Gradient sums of one pixel: d(lambda x), three logit gradients, sum h.
struct Grad {
  float dphi, d0, d1, d2, hs;
};

// One step of a sweep in the opposite order: the forward direction here is
// the one whose error term the first sweep stored (st.z / st.w), and the
// error term here belongs to the direction whose states the first sweep
// stored (st.x / st.y at this line, `up*` at the line before in its order).
// rb: this line restarts the forward direction here; ra: it restarts the
// other one. fd: the other direction is selected; fu: this one is.
// side: when given, the neighbours' stored previous-line states (upl, upr)
// are not passed in but exchanged through this second line in the same step.
__device__ __forceinline__ void sweep_b(Sweep& s, Line& ln, int t, bool act,
                                        const WeightSlopes& qa, const WeightSlopes& qb, float lxa,
                                        float lxb, float uga, float ugb, bool rb, bool ra,
                                        const float4& st, float upl, float upA, float upB,
                                        float upr, float fd, float fu, Grad& ga, Grad& gb,
                                        float2* side = nullptr) {
  const float4* cur = ln.buf + ln.par * ln.slots;
  const float4 L = cur[t], R = cur[t + 2];
  // this direction's logit gradients: its stored error term with its own
  // previous line, which is this sweep's state before the step
  const G3 fa = logit_grads(qa, st.z, L.y, s.hA, s.hB);
  const G3 fb = logit_grads(qb, st.w, s.hA, s.hB, R.x);
  advance(s, L, R, weights_of(qa), weights_of(qb), lxa, lxb, uga, ugb, rb);
  publish(s, ln, t, act, qa.w0, qb.w2, side, make_float2(upA, upB));
  if (side) {
    upl = side[ln.par * ln.slots + t].y;
    upr = side[ln.par * ln.slots + t + 2].x;
  }
  // the other direction's: the new error term with its stored previous line
  const G3 ba = logit_grads(qa, s.eA, upl, upA, upB);
  const G3 bb = logit_grads(qb, s.eB, upA, upB, upr);
  const float cf = rb ? 0.f : fu, cb = ra ? 0.f : fd;
  ga.dphi = fd * s.eA + fu * st.z;
  gb.dphi = fd * s.eB + fu * st.w;
  ga.d0 = cb * ba.g0 + cf * fa.g0;
  ga.d1 = cb * ba.g1 + cf * fa.g1;
  ga.d2 = cb * ba.g2 + cf * fa.g2;
  gb.d0 = cb * bb.g0 + cf * fb.g0;
  gb.d1 = cb * bb.g1 + cf * fb.g1;
  gb.d2 = cb * bb.g2 + cf * fb.g2;
  ga.hs = fu * s.hA + fd * st.x;
  gb.hs = fu * s.hB + fd * st.y;
}

}  // namespace

template <typename T>
struct BtArgs {
  const T* x;
  const T* lam;
  const T* l0;
  const T* l1;
  const T* l2;
  const T* u;
  const T* gy;
  T* dx;
  T* dlam;
  T* dl0;
  T* dl1;
  T* dl2;
  T* du;
  float* dlw;        // shared logits: fp32 per-plane logit gradients [3][pstride]
  float4* hv;        // [planes][H][W/2]: (h_T2B A, B, e_B2T A, B) per column pair
  float* lxt;        // [planes][Wq][Hp][4] lambda x in column quads, four columns per row
  float* ugt;        // same layout, u gy
  T* lgt;            // [3][planes][Wq][Hp][4] logits
  float4* hh;        // [planes][W][H/2]: (h_L2R A, B, e_R2L A, B) per row pair
  float* part;       // [5][planes][ng][ceil(W/4)][kGrp][kTc]: horizontal
                     // d(lambda x), dl0, dl1, dl2, sum h in 4 x 4 tiles
  int H, W, G, Hp, ng;
  int Wq;                 // column quads of the copy, ceil(W / 4)
  float fT, fB, fL, fR;   // 1 for the directions in the mask, else 0
  int64_t lg_stride;      // elements between the three logit copies
  int64_t part_stride;    // elements between the five horizontal parts
  int64_t pstride;        // planes * H * W
  int64_t plane0;         // first plane of this launch (blockIdx.x is relative)
  int64_t C, Cl;          // channels and logit channels (shared when Cl < C)
};

// ===========================================================================
// bt_vA: top->bottom, h of top->bottom and e of bottom->top, column-major copy
// ===========================================================================
template <typename T, bool COPY>
__global__ __launch_bounds__(512) void bt_vA(BtArgs<T> a) {
  __shared__ float4 lbuf[2 * (512 + 2)];
  constexpr bool BF = sizeof(T) == 2;
  constexpr int PF = BF ? 8 : 4;    // rows in flight
  constexpr int XP = 8;             // rows per 128-byte line of lambda x / u gy quads
  constexpr int GP = BF ? 16 : 8;   // rows per 128-byte line of logit quads
  constexpr int U = 16;             // unroll: a multiple of both periods
  using P = Two<T>;
  const int H = a.H, W = a.W, W2 = W / 2;
  const int t = threadIdx.x, c0 = 2 * t;
  const bool act = c0 < W;
  const int cl = act ? c0 : 0;
  const int64_t plane = a.plane0 + blockIdx.x;
  const int64_t base = plane * H * W;
  const int64_t ls = logit_shift(plane, a.C, a.Cl, static_cast<int64_t>(H) * W);
  Line ln{lbuf, static_cast<int>(blockDim.x) + 2, 0};
  line_clear(lbuf, 2 * ln.slots);
  const float mA0 = c0 > 0 ? 1.f : 0.f;
  const float mB2 = c0 + 1 < W - 1 ? 1.f : 0.f;

  struct Raw {
    typename P::raw x, lam, l0, l1, l2, u, gy;
  };
  auto load_row = [&](int r) {
    const int64_t i = base + static_cast<int64_t>(min(r, H - 1)) * W + cl;
    Raw v;
    v.x = P::load(a.x, i);
    v.lam = P::load(a.lam, i);
    v.l0 = P::load(a.l0, i + ls);
    v.l1 = P::load(a.l1, i + ls);
    v.l2 = P::load(a.l2, i + ls);
    v.u = P::load(a.u, i);
    v.gy = P::load(a.gy, i);
    return v;
  };
  Raw ring[PF];
#pragma unroll
  for (int j = 0; j < PF; ++j) ring[j] = load_row(j);

  Sweep s{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  StartsUp rst{0, a.G};
  float2 lxP[XP], ugP[XP];
  typename P::raw lgP[3][GP];
#pragma unroll
  for (int k = 0; k < XP; ++k) lxP[k] = ugP[k] = make_float2(0.f, 0.f);   // rows past H: padding
#pragma unroll
  for (int k = 0; k < GP; ++k) lgP[0][k] = lgP[1][k] = lgP[2][k] = typename P::raw{};
  // this thread's quad of the copy: the lane pair that owns it swaps half its
  // buffered rows, and the odd lane writes the second half of each line
  const bool odd = t & 1;
  const bool qact = 2 * (t & ~1) < W;
  const int64_t qbase = ((plane * a.Wq + t / 2) * a.Hp) * 4;
  float4* hv = a.hv + plane * H * W2 + t;

  auto block = [&](int r0, auto tail) {
    constexpr bool TAIL = decltype(tail)::value;
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int r = r0 + j;
      if (!TAIL || r < H) {
        const Raw v = ring[j % PF];
        ring[j % PF] = load_row(r + PF);
        const float lxa = P::lo(v.lam) * P::lo(v.x), lxb = P::hi(v.lam) * P::hi(v.x);
        const float uga = P::lo(v.u) * P::lo(v.gy), ugb = P::hi(v.u) * P::hi(v.gy);
        const Weights wa = make_weights(P::lo(v.l0), P::lo(v.l1), P::lo(v.l2), mA0, 1.f);
        const Weights wb = make_weights(P::hi(v.l0), P::hi(v.l1), P::hi(v.l2), 1.f, mB2);
        const float4* cur = ln.buf + ln.par * ln.slots;
        advance(s, cur[t], cur[t + 2], wa, wb, lxa, lxb, uga, ugb, rst.at(r));
        publish(s, ln, t, act, wa.w0, wb.w2);
        if (act) hv[static_cast<int64_t>(r) * W2] = make_float4(s.hA, s.hB, s.eA, s.eB);
        if constexpr (COPY) {
          lxP[j % XP] = make_float2(lxa, lxb);
          ugP[j % XP] = make_float2(uga, ugb);
          lgP[0][j % GP] = v.l0;
          lgP[1][j % GP] = v.l1;
          lgP[2][j % GP] = v.l2;
        }
      }
      if constexpr (COPY) {
        // whole 128-byte lines per lane pair (every lane takes part in the
        // swap); the copy's row pitch Hp is a multiple of U, so a line that
        // passes H lands in the padding
        if ((j % XP) == XP - 1 && (!TAIL || r0 + j - (XP - 1) < H)) {
          const int rs = r0 + j - (XP - 1);
          float4 ol[XP / 2], ou[XP / 2];
#pragma unroll
          for (int k = 0; k < XP / 2; ++k) {
            float2 lo, hi;
            quad_rows(lxP, XP, k, odd, &lo, &hi);
            ol[k] = make_float4(lo.x, lo.y, hi.x, hi.y);
            quad_rows(ugP, XP, k, odd, &lo, &hi);
            ou[k] = make_float4(lo.x, lo.y, hi.x, hi.y);
          }
          if (qact) {
            const int64_t o = qbase + 4 * (rs + (odd ? XP / 2 : 0));
            float4* dl = reinterpret_cast<float4*>(a.lxt + o);
            float4* du = reinterpret_cast<float4*>(a.ugt + o);
#pragma unroll
            for (int k = 0; k < XP / 2; ++k) {
              dl[k] = ol[k];
              du[k] = ou[k];
            }
          }
        }
        if ((j % GP) == GP - 1 && (!TAIL || r0 + j - (GP - 1) < H)) {
          const int rs = r0 + j - (GP - 1);
#pragma unroll
          for (int z = 0; z < 3; ++z) {
            T* g = a.lgt + z * a.lg_stride + qbase + 4 * (rs + (odd ? GP / 2 : 0));
            if constexpr (BF) {
              uint32_t o[GP];   // per row: columns 4q, 4q+1 then 4q+2, 4q+3
#pragma unroll
              for (int k = 0; k < GP / 2; ++k) quad_rows(lgP[z], GP, k, odd, &o[2 * k], &o[2 * k + 1]);
              if (qact) {
                uint4* d = reinterpret_cast<uint4*>(g);
#pragma unroll
                for (int k = 0; k < GP / 4; ++k) d[k] = make_uint4(o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]);
              }
            } else {
              float4 o[GP / 2];
#pragma unroll
              for (int k = 0; k < GP / 2; ++k) {
                float2 lo, hi;
                quad_rows(lgP[z], GP, k, odd, &lo, &hi);
                o[k] = make_float4(lo.x, lo.y, hi.x, hi.y);
              }
              if (qact) {
                float4* d = reinterpret_cast<float4*>(reinterpret_cast<float*>(g));
#pragma unroll
                for (int k = 0; k < GP / 2; ++k) d[k] = o[k];
              }
            }
          }
        }
      }
    }
  };
  int r0 = 0;
  for (; r0 + U <= H; r0 += U) block(r0, std::false_type{});
  if (r0 < H) block(r0, std::true_type{});
}

// ===========================================================================
// Horizontal sweeps over the copy: a thread owns image rows o0, o0 + 1;
// bt_hA loads both rows of a whole column quad at once, bt_hB (no registers
// for a quad) its column pair's half of them.
// ===========================================================================
template <typename T>
struct CopyIn {
  float4 lx, ug;
  typename Four<T>::raw g0, g1, g2;
};

// one column pair: its half of the quad in rows o0 and o0 + 1 (two loads per
// tensor, 8 bytes of lambda x apart by 16)
template <typename T>
__device__ __forceinline__ CopyIn<T> load_copy(const BtArgs<T>& a, int64_t plane, int cp, int ol) {
  using Q = Four<T>;
  const int64_t cc = min(max(cp, 0), a.W / 2 - 1);
  const int64_t i = ((plane * a.Wq + cc / 2) * a.Hp + ol) * 4 + 2 * (cc % 2);
  auto f4 = [](const float* p) {
    const float2 r0 = *reinterpret_cast<const float2*>(p);
    const float2 r1 = *reinterpret_cast<const float2*>(p + 4);
    return make_float4(r0.x, r0.y, r1.x, r1.y);
  };
  CopyIn<T> v;
  v.lx = f4(a.lxt + i);
  v.ug = f4(a.ugt + i);
  v.g0 = Q::load_rows(a.lgt, i);
  v.g1 = Q::load_rows(a.lgt + a.lg_stride, i);
  v.g2 = Q::load_rows(a.lgt + 2 * a.lg_stride, i);
  return v;
}

// a whole column quad: rows o0, o0 + 1 of four columns, one contiguous run
// per tensor (32 bytes of lambda x)
template <typename T>
struct CopyQ {
  Quad<float>::raw lx, ug;
  typename Quad<T>::raw g0, g1, g2;
};

template <typename T>
__device__ __forceinline__ CopyQ<T> load_copy_quad(const BtArgs<T>& a, int64_t plane, int q, int ol) {
  const int64_t qq = min(max(q, 0), a.Wq - 1);
  const int64_t i = ((plane * a.Wq + qq) * a.Hp + ol) * 4;
  CopyQ<T> v;
  v.lx = Quad<float>::load(a.lxt, i);
  v.ug = Quad<float>::load(a.ugt, i);
  v.g0 = Quad<T>::load(a.lgt, i);
  v.g1 = Quad<T>::load(a.lgt + a.lg_stride, i);
  v.g2 = Quad<T>::load(a.lgt + 2 * a.lg_stride, i);
  return v;
}

// bt_hA: left->right, h of left->right and e of right->left, stored per pixel
template <typename T>
__global__ __launch_bounds__(1024) void bt_hA(BtArgs<T> a) {
  __shared__ float4 lbuf[2 * (1024 + 2)];
  constexpr int PQ = sizeof(T) == 2 ? 2 : 1;   // column quads in flight (fp32: registers)
  const int H = a.H, W = a.W, H2 = H / 2;
  const int t = threadIdx.x, o0 = 2 * t;
  const bool act = o0 < H;
  const int ol = act ? o0 : 0;
  const int64_t plane = a.plane0 + blockIdx.x;
  Line ln{lbuf, static_cast<int>(blockDim.x) + 2, 0};
  line_clear(lbuf, 2 * ln.slots);
  const float mA0 = o0 > 0 ? 1.f : 0.f;
  const float mB2 = o0 + 1 < H - 1 ? 1.f : 0.f;
  float4* hh = a.hh + plane * W * H2 + t;

  CopyQ<T> ring[PQ];
#pragma unroll
  for (int j = 0; j < PQ; ++j) ring[j] = load_copy_quad(a, plane, j, ol);
  Sweep s{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  StartsUp rst{0, a.G};
  // columns cb .. cb + 4 PQ - 1 (a partial last block: only those below W)
  auto block = [&](int cb, auto tail) {
    constexpr bool TAIL = decltype(tail)::value;
#pragma unroll
    for (int j = 0; j < PQ; ++j) {
      const int q = cb / 4 + j;
      if (!TAIL || 4 * q < W) {
        const CopyQ<T> v = ring[j];
        ring[j] = load_copy_quad(a, plane, q + PQ, ol);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int c = 4 * q + i;
          if (!TAIL || c < W) {   // the last quad of W % 4 == 2 holds two columns
            float g0[2], g1[2], g2[2], lx[2], ug[2];
            Quad<T>::col(v.g0, i, g0);
            Quad<T>::col(v.g1, i, g1);
            Quad<T>::col(v.g2, i, g2);
            Quad<float>::col(v.lx, i, lx);
            Quad<float>::col(v.ug, i, ug);
            const Weights wa = make_weights(g0[0], g1[0], g2[0], mA0, 1.f);
            const Weights wb = make_weights(g0[1], g1[1], g2[1], 1.f, mB2);
            const float4* cur = ln.buf + ln.par * ln.slots;
            advance(s, cur[t], cur[t + 2], wa, wb, lx[0], lx[1], ug[0], ug[1], rst.at(c));
            publish(s, ln, t, act, wa.w0, wb.w2);
            if (act) hh[static_cast<int64_t>(c) * H2] = make_float4(s.hA, s.hB, s.eA, s.eB);
          }
        }
      }
    }
  };
  int cb = 0;
  for (; cb + 4 * PQ <= W; cb += 4 * PQ) block(cb, std::false_type{});
  if (cb < W) block(cb, std::true_type{});
}

// bt_hB: right->left, h of right->left and e of left->right; writes the
// horizontal parts of the gradients
size_t bt_hb_lds_bytes(unsigned threads) {
  const size_t slots = threads + 2;
  return 2 * slots * sizeof(float4) + 2 * slots * sizeof(float2) + 20 * threads * sizeof(float);
}

template <typename T>
__global__ __launch_bounds__(1024) void bt_hB(BtArgs<T> a) {
  // the line, the left->right states of the previous column (in that
  // direction's order) of the neighbouring rows, and each thread's outputs
  // of the right column pair of a tile until its left pair is done
  extern __shared__ float4 dyn[];
  const int nt = blockDim.x, slots = nt + 2;
  float4* lbuf = dyn;
  float2* nbuf = reinterpret_cast<float2*>(dyn + 2 * slots);
  float* stash = reinterpret_cast<float*>(nbuf + 2 * slots);   // [20][nt]
  using Q = Four<T>;
  const int H = a.H, W = a.W, H2 = H / 2, W2 = W / 2, nq = (W2 + 1) / 2;
  const int t = threadIdx.x, o0 = 2 * t;
  const bool act = o0 < H;
  const int tl = act ? t : 0, ol = 2 * tl;
  const int64_t plane = a.plane0 + blockIdx.x;
  Line ln{lbuf, slots, 0};
  for (int i = t; i < 2 * slots; i += nt) nbuf[i] = make_float2(0.f, 0.f);
  for (int i = 0; i < 20; ++i) stash[i * nt + t] = 0.f;
  line_clear(lbuf, 2 * slots);
  const float mA0 = o0 > 0 ? 1.f : 0.f;
  const float mB2 = o0 + 1 < H - 1 ? 1.f : 0.f;
  const float4* hh = a.hh + plane * W * H2 + tl;

  // a column pair: the copy, and bt_hA's values of this row pair in columns
  // 2 cp + 1, 2 cp and 2 cp - 1 (the last is the previous column of 2 cp in
  // left->right order)
  // (every load fetches exactly what is used: a wider load whose unused
  // part the compiler recycles as scratch registers must land first)
  struct In {
    CopyIn<T> c;
    float4 st[2];
    float2 sp;
  };
  auto load_pair = [&](int cp) {
    In v;
    v.c = load_copy(a, plane, cp, ol);
    const int cc = min(max(cp, 0), W2 - 1);
    v.st[0] = hh[static_cast<int64_t>(2 * cc + 1) * H2];
    v.st[1] = hh[static_cast<int64_t>(2 * cc) * H2];
    v.sp = *reinterpret_cast<const float2*>(hh + static_cast<int64_t>(max(2 * cc - 1, 0)) * H2);
    return v;
  };
  // rows o0, o0 + 1 of this thread in tile 0 of its row group
  float* part = a.part + (plane * a.ng + ol / kGrp) * nq * (kGrp * kTc) + (ol % kGrp) * kTc;

  // one pair in flight: registers
  In ring = load_pair(W2 - 1);
  Sweep s{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  EndsDown rb = ends_down(W, a.G);     // right->left restarts
  StartsDown ra = starts_down(W, a.G); // left->right restarts
  // columns 2 cp + 1, 2 cp: the outputs of rows o0, o0 + 1 (index: even / odd column)
  auto pair = [&](int cp, Grad (&gA)[2], Grad (&gB)[2]) {
    const In v = ring;
    ring = load_pair(cp - 1);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int odd = 1 - k;
      const int c = 2 * cp + odd;
      const WeightSlopes qa = make_weight_slopes(Q::get(v.c.g0, 0, odd), Q::get(v.c.g1, 0, odd),
                                                 Q::get(v.c.g2, 0, odd), mA0, 1.f);
      const WeightSlopes qb = make_weight_slopes(Q::get(v.c.g0, 1, odd), Q::get(v.c.g1, 1, odd),
                                                 Q::get(v.c.g2, 1, odd), 1.f, mB2);
      const bool rbc = rb.at(c), rac = ra.at(c);
      const float2 up = k ? v.sp : make_float2(v.st[1].x, v.st[1].y);
      sweep_b(s, ln, t, act, qa, qb, quad(v.c.lx, 0, odd), quad(v.c.lx, 1, odd),
              quad(v.c.ug, 0, odd), quad(v.c.ug, 1, odd), rbc, rac, v.st[k], 0.f, up.x, up.y,
              0.f, a.fL, a.fR, gA[odd], gB[odd], nbuf);
    }
  };
  auto field = [](const Grad& g, int p) {
    return p == 0 ? g.dphi : (p == 1 ? g.d0 : (p == 2 ? g.d1 : (p == 3 ? g.d2 : g.hs)));
  };
  // the right pair of a tile: parked in the thread's own LDS slots
  auto park = [&](const Grad (&gA)[2], const Grad (&gB)[2]) {
#pragma unroll
    for (int p = 0; p < 5; ++p) {
      stash[(4 * p) * nt + t] = field(gA[0], p);
      stash[(4 * p + 1) * nt + t] = field(gA[1], p);
      stash[(4 * p + 2) * nt + t] = field(gB[0], p);
      stash[(4 * p + 3) * nt + t] = field(gB[1], p);
    }
  };
  // the left pair: the whole tile row pair, 32 contiguous bytes per part
  auto put_tile = [&](int q, const Grad (&gA)[2], const Grad (&gB)[2]) {
    if (!act) return;
    float* d = part + static_cast<int64_t>(q) * (kGrp * kTc);
#pragma unroll
    for (int p = 0; p < 5; ++p) {
      float4* dp = reinterpret_cast<float4*>(d + p * a.part_stride);
      dp[0] = make_float4(field(gA[0], p), field(gA[1], p), stash[(4 * p) * nt + t],
                          stash[(4 * p + 1) * nt + t]);
      dp[1] = make_float4(field(gB[0], p), field(gB[1], p), stash[(4 * p + 2) * nt + t],
                          stash[(4 * p + 3) * nt + t]);
    }
  };
  int cp = W2 - 1;
  Grad gA[2], gB[2];
  if (!(cp & 1)) {
    // an odd number of pairs: the last tile has no right pair (its half is
    // padding and takes the zeroed slots)
    pair(cp, gA, gB);
    put_tile(cp / 2, gA, gB);
    --cp;
  }
  for (; cp >= 1; cp -= 2) {
    pair(cp, gA, gB);
    park(gA, gB);
    pair(cp - 1, gA, gB);
    put_tile(cp / 2, gA, gB);
  }
}

// ===========================================================================
// bt_vB: bottom->top, h of bottom->top and e of top->bottom, the gradients
// ===========================================================================
template <typename T, bool HZ>
__global__ __launch_bounds__(512) void bt_vB(BtArgs<T> a) {
  __shared__ float4 lbuf[2 * (512 + 2)];
  constexpr int RP = sizeof(T) == 2 ? 4 : 3;   // row pairs in flight
  using P = Two<T>;
  const int H = a.H, W = a.W, W2 = W / 2;
  const int t = threadIdx.x, c0 = 2 * t;
  const bool act = c0 < W;
  const int tl = act ? t : 0, cl = 2 * tl;
  const int tm = max(tl - 1, 0), tp = min(tl + 1, W2 - 1);
  const int64_t plane = a.plane0 + blockIdx.x;
  const int64_t base = plane * H * W;
  const int64_t ls = logit_shift(plane, a.C, a.Cl, static_cast<int64_t>(H) * W);
  Line ln{lbuf, static_cast<int>(blockDim.x) + 2, 0};
  line_clear(lbuf, 2 * ln.slots);
  const float mA0 = c0 > 0 ? 1.f : 0.f;
  const float mB2 = c0 + 1 < W - 1 ? 1.f : 0.f;
  const float4* hv = a.hv + plane * H * W2;

  struct Row {
    typename P::raw x, lam, l0, l1, l2, u, gy;
    float4 st;         // bt_vA's values of this row
    float nl, nr;      // top->bottom states of the row above at c0 - 1, c0 + 2
  };
  struct RowPair {
    Row r[2];          // rows 2k, 2k + 1
    float2 up0;        // top->bottom states of row 2k - 1 (the row above 2k)
    float2 hz[5][2];   // horizontal parts of rows 2k, 2k + 1 at columns c0, c0 + 1
  };
  auto load_pair = [&](int k) {
    RowPair v;
    k = max(k, 0);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 2 * k + i;
      const int64_t idx = base + static_cast<int64_t>(r) * W + cl;
      Row& q = v.r[i];
      q.x = P::load(a.x, idx);
      q.lam = P::load(a.lam, idx);
      q.l0 = P::load(a.l0, idx + ls);
      q.l1 = P::load(a.l1, idx + ls);
      q.l2 = P::load(a.l2, idx + ls);
      q.u = P::load(a.u, idx);
      q.gy = P::load(a.gy, idx);
      q.st = hv[static_cast<int64_t>(r) * W2 + tl];
      // (scalar and pair loads of exactly what is used: a wider load whose
      // unused part the compiler recycles as scratch registers must land first)
      const float* up = reinterpret_cast<const float*>(hv + static_cast<int64_t>(max(r - 1, 0)) * W2);
      q.nl = up[4 * tm + 1];
      q.nr = up[4 * tp];
    }
    v.up0 = *reinterpret_cast<const float2*>(hv + static_cast<int64_t>(max(2 * k - 1, 0)) * W2 + tl);
    if constexpr (HZ) {
      const int nq = (W2 + 1) / 2;
      const float* pp = a.part + ((plane * a.ng + (2 * k) / kGrp) * nq + tl / 2) * (kGrp * kTc) +
                        ((2 * k) % kGrp) * kTc + (tl % 2) * 2;
#pragma unroll
      for (int q = 0; q < 5; ++q) {
        v.hz[q][0] = *reinterpret_cast<const float2*>(pp + q * a.part_stride);
        v.hz[q][1] = *reinterpret_cast<const float2*>(pp + q * a.part_stride + kTc);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 5; ++q) v.hz[q][0] = v.hz[q][1] = make_float2(0.f, 0.f);
    }
    return v;
  };

  Sweep s{0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  EndsDown rb = ends_down(H, a.G);      // bottom->top restarts
  StartsDown ra = starts_down(H, a.G);  // top->bottom restarts
  auto row_step = [&](const RowPair& v, int i, int r) {
    const Row& q = v.r[i];
    const float2 up = i ? make_float2(v.r[0].st.x, v.r[0].st.y) : v.up0;
    const WeightSlopes qa = make_weight_slopes(P::lo(q.l0), P::lo(q.l1), P::lo(q.l2), mA0, 1.f);
    const WeightSlopes qb = make_weight_slopes(P::hi(q.l0), P::hi(q.l1), P::hi(q.l2), 1.f, mB2);
    const float lxa = P::lo(q.lam) * P::lo(q.x), lxb = P::hi(q.lam) * P::hi(q.x);
    const float uga = P::lo(q.u) * P::lo(q.gy), ugb = P::hi(q.u) * P::hi(q.gy);
    const bool rbr = rb.at(r), rar = ra.at(r);
    Grad ga, gb;
    sweep_b(s, ln, t, act, qa, qb, lxa, lxb, uga, ugb, rbr, rar, q.st, q.nl, up.x, up.y, q.nr,
            a.fT, a.fB, ga, gb);
    auto hzv = [&](int q, int col) { return col ? v.hz[q][i].y : v.hz[q][i].x; };
    ga.dphi += hzv(0, 0);
    gb.dphi += hzv(0, 1);
    ga.d0 += hzv(1, 0);
    gb.d0 += hzv(1, 1);
    ga.d1 += hzv(2, 0);
    gb.d1 += hzv(2, 1);
    ga.d2 += hzv(3, 0);
    gb.d2 += hzv(3, 1);
    ga.hs += hzv(4, 0);
    gb.hs += hzv(4, 1);
    if (act) {
      const int64_t o = base + static_cast<int64_t>(r) * W + c0;
      P::store(a.dx, o, P::lo(q.lam) * ga.dphi, P::hi(q.lam) * gb.dphi);
      P::store(a.dlam, o, P::lo(q.x) * ga.dphi, P::hi(q.x) * gb.dphi);
      P::store(a.du, o, P::lo(q.gy) * ga.hs, P::hi(q.gy) * gb.hs);
      if (a.dlw) {
        *reinterpret_cast<float2*>(a.dlw + o) = make_float2(ga.d0, gb.d0);
        *reinterpret_cast<float2*>(a.dlw + a.pstride + o) = make_float2(ga.d1, gb.d1);
        *reinterpret_cast<float2*>(a.dlw + 2 * a.pstride + o) = make_float2(ga.d2, gb.d2);
      } else {
        P::store(a.dl0, o, ga.d0, gb.d0);
        P::store(a.dl1, o, ga.d1, gb.d1);
        P::store(a.dl2, o, ga.d2, gb.d2);
      }
    }
  };

  const int np = H / 2;
  RowPair ring[RP];
#pragma unroll
  for (int j = 0; j < RP; ++j) ring[j] = load_pair(np - 1 - j);
  auto block = [&](int kb, auto tail) {
    constexpr bool TAIL = decltype(tail)::value;
#pragma unroll
    for (int j = 0; j < RP; ++j) {
      const int k = kb - j;
      if (!TAIL || k >= 0) {
        // the slot is used in place and refilled after its two rows (a copy
        // of it taken before the refill made the compiler rotate the ring
        // through register moves that wait for every load in flight)
        row_step(ring[j], 1, 2 * k + 1);
        row_step(ring[j], 0, 2 * k);
        ring[j] = load_pair(k - RP);
      }
    }
  };
  int kb = np - 1;
  for (; kb - (RP - 1) >= 0; kb -= RP) block(kb, std::false_type{});
  if (kb >= 0) block(kb, std::true_type{});
}

// ---------------------------------------------------------------------------
// a column pair per thread of the 512-thread row sweeps: W <= 1024
bool btpipe_fits(int64_t H, int64_t W) { return tpipe_fits(H, W) && W <= 1024; }

namespace {
size_t al256(size_t v) { return (v + 255) & ~size_t(255); }

struct BtLayout {
  int64_t Hp, Wq, ng;
  size_t hv, lxt, ugt, lgt, hh, part, total;
};

BtLayout bt_layout(int64_t planes, int64_t H, int64_t W, size_t es, bool hz) {
  BtLayout L;
  L.Hp = (H + 15) / 16 * 16;
  L.Wq = (W + 3) / 4;
  L.ng = (H + kGrp - 1) / kGrp;
  const size_t px = static_cast<size_t>(planes * H * W);
  const size_t cp = static_cast<size_t>(planes * 4 * L.Wq * L.Hp);   // elements of one copy
  const size_t np = static_cast<size_t>(planes * L.ng * ((W / 2 + 1) / 2) * kGrp * kTc);
  size_t o = 0;
  L.hv = o; o = al256(o + px * 8);
  L.lxt = o; o = al256(o + (hz ? cp * 4 : 0));
  L.ugt = o; o = al256(o + (hz ? cp * 4 : 0));
  L.lgt = o; o = al256(o + (hz ? 3 * cp * es : 0));
  L.hh = o; o = al256(o + (hz ? px * 8 : 0));
  L.part = o; o = al256(o + (hz ? 5 * np * 4 : 0));
  L.total = o;
  return L;
}
}  // namespace

size_t bwd_tpipe_workspace_bytes(int64_t planes, int64_t H, int64_t W, uint32_t mask,
                                 gspn_dtype dt) {
  const size_t es = dt == GSPN_F32 ? 4 : 2;
  // at least the streaming path's: calls whose tensors start at an odd
  // element offset take that path with the same workspace
  return std::max(bt_layout(planes, H, W, es, mask & 12u).total,
                  bwd_stream_workspace_bytes(planes, H, W, mask, dt));
}

template <typename T>
static hipError_t launch_bt_dt(const BwdProblem& pr, void* ws, hipStream_t stream, Tracer* tr) {
  const int64_t planes = pr.B * pr.C;
  const uint32_t m = pr.mask;
  const bool hz = m & 12u;
  const BtLayout L = bt_layout(planes, pr.H, pr.W, sizeof(T), hz);
  char* w = static_cast<char*>(ws);
  BtArgs<T> a;
  a.x = static_cast<const T*>(pr.x);
  a.lam = static_cast<const T*>(pr.lam);
  a.l0 = static_cast<const T*>(pr.l[0]);
  a.l1 = static_cast<const T*>(pr.l[1]);
  a.l2 = static_cast<const T*>(pr.l[2]);
  a.u = static_cast<const T*>(pr.u);
  a.gy = static_cast<const T*>(pr.gy);
  a.dx = static_cast<T*>(pr.dx);
  a.dlam = static_cast<T*>(pr.dlam);
  a.dl0 = static_cast<T*>(pr.dl[0]);
  a.dl1 = static_cast<T*>(pr.dl[1]);
  a.dl2 = static_cast<T*>(pr.dl[2]);
  a.du = static_cast<T*>(pr.du);
  a.dlw = pr.dlw;
  a.hv = reinterpret_cast<float4*>(w + L.hv);
  a.lxt = reinterpret_cast<float*>(w + L.lxt);
  a.ugt = reinterpret_cast<float*>(w + L.ugt);
  a.lgt = reinterpret_cast<T*>(w + L.lgt);
  a.hh = reinterpret_cast<float4*>(w + L.hh);
  a.part = reinterpret_cast<float*>(w + L.part);
  a.H = static_cast<int>(pr.H);
  a.W = static_cast<int>(pr.W);
  a.G = static_cast<int>(pr.G >= pr.H && pr.G >= pr.W ? 0 : pr.G);
  a.Hp = static_cast<int>(L.Hp);
  a.Wq = static_cast<int>(L.Wq);
  a.ng = static_cast<int>(L.ng);
  a.fT = (m & 1u) ? 1.f : 0.f;
  a.fB = (m & 2u) ? 1.f : 0.f;
  a.fL = (m & 4u) ? 1.f : 0.f;
  a.fR = (m & 8u) ? 1.f : 0.f;
  a.lg_stride = planes * 4 * L.Wq * L.Hp;
  a.part_stride = planes * L.ng * ((pr.W / 2 + 1) / 2) * kGrp * kTc;
  a.pstride = planes * pr.H * pr.W;
  a.plane0 = 0;
  a.C = pr.C;
  a.Cl = pr.Cl;
  const unsigned tv = static_cast<unsigned>((pr.W / 2 + 63) / 64 * 64);
  const unsigned th = static_cast<unsigned>((pr.H / 2 + 63) / 64 * 64);
  using K = void (*)(BtArgs<T>);
  const K kva = hz ? bt_vA<T, true> : bt_vA<T, false>;
  const K kvb = hz ? bt_vB<T, true> : bt_vB<T, false>;
  const K kha = bt_hA<T>, khb = bt_hB<T>;

  // one compute unit per plane in every launch: plane groups on their own
  // streams let one group's tail overlap another group's next launch
  const int ngroups = tpipe_groups(planes);
  hipStream_t streams[kMaxGroups] = {stream, stream, stream, stream};
  hipEvent_t fork = nullptr, join[kMaxGroups] = {};
  hipError_t e = hipSuccess;
  auto release = [&]() {
    if (fork) (void)hipEventDestroy(fork);
    for (int g = 1; g < ngroups; ++g)
      if (join[g]) (void)hipEventDestroy(join[g]);
  };
  if (ngroups > 1) {
    if ((e = hipEventCreateWithFlags(&fork, hipEventDisableTiming)) != hipSuccess) return e;
    for (int g = 1; g < ngroups && e == hipSuccess; ++g) {
      streams[g] = aux_stream(g - 1);
      if (!streams[g]) e = hipErrorOutOfMemory;
      if (e == hipSuccess) e = hipEventCreateWithFlags(&join[g], hipEventDisableTiming);
    }
    if (e == hipSuccess) e = hipEventRecord(fork, stream);
    for (int g = 1; g < ngroups && e == hipSuccess; ++g) e = hipStreamWaitEvent(streams[g], fork, 0);
    if (e != hipSuccess) {
      release();
      return e;
    }
  }
  int64_t g0[kMaxGroups], gn[kMaxGroups];
  for (int g = 0; g < ngroups; ++g) {
    g0[g] = planes * g / ngroups;
    gn[g] = planes * (g + 1) / ngroups - g0[g];
  }
  const size_t hb_lds = bt_hb_lds_bytes(th);
  if (hz && hb_lds > 65536) {
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(khb),
                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                 static_cast<int>(hb_lds))) != hipSuccess) {
      release();
      return e;
    }
  }
  auto launch = [&](K k, unsigned threads, const char* name, int g) -> hipError_t {
    if (gn[g] == 0) return hipSuccess;
    BtArgs<T> ag = a;
    ag.plane0 = g0[g];
    tr->before(streams[g], name, gn[g]);
    const size_t lds = k == khb ? hb_lds : 0;
    hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(gn[g])), dim3(threads), lds, streams[g], ag);
    tr->after(streams[g]);
    return hipGetLastError();
  };
  for (int g = 0; g < ngroups && e == hipSuccess; ++g) e = launch(kva, tv, "bt_vA", g);
  for (int g = 0; g < ngroups && e == hipSuccess; ++g)
    if (hz) e = launch(kha, th, "bt_hA", g);
  for (int g = 0; g < ngroups && e == hipSuccess; ++g)
    if (hz) e = launch(khb, th, "bt_hB", g);
  for (int g = 0; g < ngroups && e == hipSuccess; ++g) e = launch(kvb, tv, "bt_vB", g);
  for (int g = 1; g < ngroups; ++g) {
    hipError_t e2 = hipEventRecord(join[g], streams[g]);
    if (e2 == hipSuccess) e2 = hipStreamWaitEvent(stream, join[g], 0);
    if (e == hipSuccess) e = e2;
  }
  release();
  return e;
}

hipError_t launch_bwd_tpipe(const BwdProblem& pr, void* ws, hipStream_t stream, Tracer* tr) {
  if (pr.dtype == GSPN_F32) return launch_bt_dt<float>(pr, ws, stream, tr);
  return launch_bt_dt<bf16_t>(pr, ws, stream, tr);
}

}  // namespace gspn

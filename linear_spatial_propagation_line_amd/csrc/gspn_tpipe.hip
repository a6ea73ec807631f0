// Large-plane GSPN propagation ("transpose pipeline"), for planes above 64x64
// with W <= 2048 and H <= 2048, both even. Planes up to 1024 wide run the row
// sweeps (K1, K3) with 512 threads; wider ones with 1024 threads, smaller
// per-thread buffers and 4-row chunks, so that the same pipeline serves the
// portrait form of a latent without transposing it.
//
// A plane is too large for on-chip memory, and every scan step couples a whole
// line (each pixel mixes its three predecessors), so one workgroup must own a
// whole line of a plane. Three launches, one workgroup per plane each:
//
//   K1 vfwd  -- top->bottom sweep over the row-major inputs (a thread owns
//               two adjacent columns, coalesced 4-byte loads prefetched 8 rows
//               ahead). Saves the state every 8 rows (checkpoints) and writes a
//               column-major copy of lambda*x (fp32) and the three logits in
//               column quads: per-thread register buffers, then a swap within
//               the lane pair that owns a quad, so that the pair's stores
//               complete whole 128-byte lines.
//   K2 hpair -- left->right and right->left on the column-major copy, where a
//               horizontal scan reads whole contiguous lines (a thread loads
//               two rows of a column quad at once). The right->left
//               pass walks 4-column chunks from the right; for each chunk it
//               recomputes left->right from the checkpoint before it, so one
//               pass over the copy serves both directions. Writes
//               h_L2R + h_R2L column-major (fp32).
//   K3 vbwd  -- bottom->top over the row-major inputs in 8-row chunks, with
//               top->bottom recomputed per chunk from K1's checkpoints; reads
//               the horizontal sum of the chunk as one 32-byte column segment
//               per column and writes out = u * (h_T2B + h_B2T + h_H) once,
//               row-major.
//
// The normalised weights of a pixel are the same for both scans of one axis
// (same logits, same in-range neighbours), so each chunk computes them once
// for its recompute and its reverse pass.
//
// Line recurrence, output gate: CSDN page on GSPN, section 方法; tridiagonal
// row-normalised sigmoid weights and four scan directions: section
// 如何设计一个高效的传播层; local groups: section GSPN模块的设计.
#include <algorithm>
#include <cstring>
#include <type_traits>

#include "gspn_device.hpp"
#include "gspn_quad.hpp"
#include "gspn_launch.hpp"

namespace gspn {

namespace {

constexpr int kCkH = 4;    // columns per horizontal chunk / checkpoint interval

// The column-major copy K1 writes and K2 reads holds the columns of a plane
// in quads: [plane][ceil(W / 4)][Hp][4], so a 128-byte line is 8 rows of
// four lambda*x values (16 rows of four bf16 logits). The two threads that
// own a quad's column pairs swap half their buffered rows (a DPP move within
// the lane pair) and then each writes 64 contiguous bytes: together one
// whole line in the same four stores.
//
// Shapes of the row sweeps (K1, K3) by workgroup size NT: 512 threads own up
// to 1024 columns, 1024 threads up to 2048. At 1024 threads a thread has 128
// registers, so the prefetch ring is 4 rows deep and the vertical chunks 4
// rows high (which is also the checkpoint interval of K1 and the chunk height
// of the horizontal sum).
template <typename T, int NT> struct RowShape {
  static constexpr bool kWide = NT > 512;
  static constexpr int CKV = kWide ? 4 : 8;                          // rows per vertical chunk
  static constexpr int PF = kWide ? 4 : (sizeof(T) == 2 ? 8 : 4);    // K1 prefetch distance
  static constexpr int LXP = 8;                                      // lambda*x rows per line
  static constexpr int LGP = 128 / (4 * static_cast<int>(sizeof(T)));   // logit rows per line
  static constexpr int MAXW = 2 * NT;                                // widest plane
};

// vertical chunk height for a plane of width W (the launcher's choice of NT)
inline int row_chunk(int64_t W) { return W > 1024 ? 4 : 8; }

// ---- storage access: pairs of adjacent elements --------------------------
template <typename T> struct Pair;
template <> struct Pair<float> {
  using raw = float2;
  __device__ static raw load(const float* p, int64_t i) {
    return *reinterpret_cast<const float2*>(p + i);
  }
  __device__ static float lo(raw v) { return v.x; }
  __device__ static float hi(raw v) { return v.y; }
};
template <> struct Pair<bf16_t> {
  using raw = uint32_t;
  __device__ static raw load(const bf16_t* p, int64_t i) {
    return *reinterpret_cast<const uint32_t*>(p + i);
  }
  __device__ static float lo(raw v) { return bf16_lo(v); }
  __device__ static float hi(raw v) { return bf16_hi(v); }
};

__device__ __forceinline__ void store_pair(float* p, int64_t i, float a, float b) {
  *reinterpret_cast<float2*>(p + i) = make_float2(a, b);
}
__device__ __forceinline__ void store_pair(bf16_t* p, int64_t i, float a, float b) {
  *reinterpret_cast<uint32_t*>(p + i) = pack_bf16x2(a, b);
}

// raw inputs of two adjacent pixels
template <typename T>
struct Raw2 {
  typename Pair<T>::raw x, lam, l0, l1, l2;
};

// (the logits of pixel i sit at i + ls: ls = 0 unless logits are shared)
template <typename T>
__device__ __forceinline__ Raw2<T> load_raw2(const T* x, const T* lam, const T* l0, const T* l1,
                                             const T* l2, int64_t i, int64_t ls) {
  Raw2<T> r;
  r.x = Pair<T>::load(x, i);
  r.lam = Pair<T>::load(lam, i);
  r.l0 = Pair<T>::load(l0, i + ls);
  r.l1 = Pair<T>::load(l1, i + ls);
  r.l2 = Pair<T>::load(l2, i + ls);
  return r;
}

// record of one pixel: normalised weights and lambda*x
struct Rec {
  float w0, w1, w2, lx;
};

__device__ __forceinline__ Rec make_rec(float l0, float l1, float l2, float lx, float m0,
                                        float m2) {
  const Weights w = make_weights(l0, l1, l2, m0, m2);
  return Rec{w.w0, w.w1, w.w2, lx};
}

__device__ __forceinline__ float mix(const Rec& r, float hl, float hc, float hr) {
  return __builtin_fmaf(r.w0, hl, __builtin_fmaf(r.w1, hc, __builtin_fmaf(r.w2, hr, r.lx)));
}

// Restart bookkeeping without a division per step. A forward scan restarts
// at position 0 and at every multiple of G (G > 0); a reverse scan (positions
// decreasing) at n - 1 and at every mG - 1. These give the first restart
// position met from p on; later ones follow by adding / subtracting G.
constexpr int kNone = 1 << 30;
__device__ __forceinline__ int fwd_restart_from(int p, int G) {
  if (p <= 0) return 0;
  if (G <= 0) return kNone;
  return (p + G - 1) / G * G;
}
__device__ __forceinline__ int rev_restart_from(int p, int n, int G) {
  if (p >= n - 1) return n - 1;
  if (G <= 0) return -kNone;
  return (p + 1) / G * G - 1;
}
// state of a forward restart counter: next restart position
struct FwdRestart {
  int next, G;
  __device__ bool at(int p) {
    const bool r = (p == next);
    next = r ? (G > 0 ? p + G : kNone) : next;
    return r;
  }
};
// reverse counter: after position n - 1 the next one is not n - 1 - G in
// general, so it is precomputed
struct RevRestart {
  int next, after_last, G, last;
  __device__ bool at(int p) {
    const bool r = (p == next);
    next = r ? (p == last ? after_last : p - G) : next;
    return r;
  }
};
__device__ __forceinline__ RevRestart rev_counter(int p, int n, int G) {
  return RevRestart{rev_restart_from(p, n, G), rev_restart_from(n - 2, n, G), G, n - 1};
}

// Line exchange: the states of one line, two per thread, in LDS with two
// zero pads on each side (index = position + 2); double-buffered so that one
// barrier per step suffices. Only threads that own positions of the line
// write it; the pads stay zero from the initial clear.
struct LineX {
  float* buf;     // [2][n + 4]
  int n4;         // n + 4
  int par;
  __device__ float* cur() { return buf + par * n4; }
  __device__ float* nxt() { return buf + (par ^ 1) * n4; }
};

}  // namespace

template <typename T>
struct TpArgs {
  const T* x;
  const T* lam;
  const T* l0;
  const T* l1;
  const T* l2;
  const T* u;
  T* out;
  float* lxt;     // [planes][Wq][Hp][4] lambda*x, column-major by column quads
  T* lgt;         // [3][planes][Wq][Hp][4] logits, same layout
  float* yht;     // [planes][nckv][W][ckr] h_L2R + h_R2L, in ckr-row chunks
  float* ckv;     // [planes][nckv][W] top->bottom states after rows ckr k + ckr - 1
  float* ckh;     // [planes][nckh][H] left->right states after columns 4k+3
  int H, W, G, Hp, nckv, nckh;
  int Wq;         // column quads of the copy, ceil(W / 4)
  int ckr;        // rows per vertical chunk (8, or 4 for planes wider than 1024)
  unsigned mask;
  int64_t lg_stride;   // elements between the three logit copies
  int64_t plane0;      // first plane of this launch (blockIdx.x is relative)
  int64_t C, Cl;       // channels and logit channels (shared logits when Cl < C)
};

// ===========================================================================
// K1: top->bottom forward sweep, checkpoints, column-major copy
// ===========================================================================
// SCAN: run top->bottom and save checkpoints; COPY: write lambda*x into the
// column-major copy; COPYLG: write the logits into it. With shared logits
// the logit copy is made once per logit plane by tp_lgcopy and this kernel
// writes lambda*x only.
// The main loop covers full 32-row blocks with straight-line code and
// unconditional (row-clamped) loads so that the prefetch ring stays in flight;
// a partial last block runs the same body with per-row guards.
template <typename T, int NT, bool SCAN, bool COPY, bool COPYLG = COPY>
__global__ __launch_bounds__(NT) void tp_vfwd(TpArgs<T> a) {
  using S = RowShape<T, NT>;
  __shared__ float lbuf[2 * (S::MAXW + 4)];
  constexpr int LGP = S::LGP;                     // logit flush period (rows)
  constexpr int LXP = S::LXP;                     // lambda*x flush period (rows)
  constexpr int U = 32;                           // unroll (multiple of both periods)
  constexpr int PF = S::PF;                       // prefetch distance (rows)
  constexpr int CKV = S::CKV;                     // checkpoint interval (rows)
  using P = Pair<T>;
  const int H = a.H, W = a.W, G = a.G;
  const int t = threadIdx.x;
  const int c0 = 2 * t;
  const bool act = c0 < W;
  const int cl = act ? c0 : 0;                    // in-bounds column for idle threads
  const int64_t plane = a.plane0 + blockIdx.x;
  const int64_t base = plane * H * W;
  const int n4 = W + 4;
  for (int i = t; i < 2 * n4; i += blockDim.x) lbuf[i] = 0.0f;
  __syncthreads();
  LineX lx{lbuf, n4, 0};
  const float mA0 = c0 > 0 ? 1.f : 0.f;              // column c0 has a left neighbour
  const float mB2 = c0 + 1 < W - 1 ? 1.f : 0.f;      // column c0+1 has a right neighbour
  const int64_t ls = logit_shift(plane, a.C, a.Cl, static_cast<int64_t>(H) * W);
  auto load_row = [&](int r) {
    return load_raw2(a.x, a.lam, a.l0, a.l1, a.l2, base + (int64_t)min(r, H - 1) * W + cl, ls);
  };

  Raw2<T> ring[PF];
#pragma unroll
  for (int j = 0; j < PF; ++j) ring[j] = load_row(j);

  float hA = 0.f, hB = 0.f;
  FwdRestart rst{0, G};
  // copy buffers: per row, the values of columns c0 and c0 + 1
  float2 lxP[LXP];
  typename P::raw lgP[3][LGP];
#pragma unroll
  for (int k = 0; k < LXP; ++k) lxP[k] = make_float2(0.f, 0.f);   // rows past H: padding
#pragma unroll
  for (int k = 0; k < LGP; ++k) lgP[0][k] = lgP[1][k] = lgP[2][k] = typename P::raw{};
  // this thread's quad in the copy; the odd lane of the pair writes the
  // second half of each line
  const bool odd = t & 1;
  const bool qact = 2 * (t & ~1) < W;             // the quad holds a column of the plane
  const int64_t qbase = ((plane * a.Wq + t / 2) * a.Hp) * 4;

  auto block = [&](int r0, auto tail) {
    constexpr bool TAIL = decltype(tail)::value;
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int r = r0 + j;
      if (!TAIL || r < H) {
        const Raw2<T> v = ring[j % PF];
        ring[j % PF] = load_row(r + PF);
        const float lxa = P::lo(v.lam) * P::lo(v.x);
        const float lxb = P::hi(v.lam) * P::hi(v.x);
        if constexpr (SCAN) {
          const bool restart = rst.at(r);
          const float* pv = lx.cur();
          const Rec ra = make_rec(P::lo(v.l0), P::lo(v.l1), P::lo(v.l2), lxa, mA0, 1.f);
          const Rec rb = make_rec(P::hi(v.l0), P::hi(v.l1), P::hi(v.l2), lxb, 1.f, mB2);
          const float na = mix(ra, pv[c0 + 1], hA, hB);
          const float nb = mix(rb, hA, hB, pv[c0 + 4]);
          hA = restart ? lxa : na;
          hB = restart ? lxb : nb;
          if (act) *reinterpret_cast<float2*>(lx.nxt() + c0 + 2) = make_float2(hA, hB);
          lx.par ^= 1;
          if ((j + 1) % CKV == 0 && act)
            store_pair(a.ckv, (plane * a.nckv + r / CKV) * W + c0, hA, hB);
          __syncthreads();
        }
        if constexpr (COPY) lxP[j % LXP] = make_float2(lxa, lxb);
        if constexpr (COPYLG) {
          lgP[0][j % LGP] = v.l0;
          lgP[1][j % LGP] = v.l1;
          lgP[2][j % LGP] = v.l2;
        }
      }
      if constexpr (COPY) {
        // a whole line of lambda*x quads (8 rows) per lane pair; every lane
        // takes part in the swap, and a line that passes H lands in the
        // padding (Hp is a multiple of 32)
        if ((j % LXP) == LXP - 1 && (!TAIL || r0 + j - (LXP - 1) < H)) {
          const int rs = r0 + j - (LXP - 1);
          float4 o[LXP / 2];
#pragma unroll
          for (int k = 0; k < LXP / 2; ++k) {
            float2 lo, hi;
            quad_rows(lxP, LXP, k, odd, &lo, &hi);
            o[k] = make_float4(lo.x, lo.y, hi.x, hi.y);
          }
          if (qact) {
            float4* d = reinterpret_cast<float4*>(a.lxt + qbase + 4 * (rs + (odd ? LXP / 2 : 0)));
#pragma unroll
            for (int k = 0; k < LXP / 2; ++k) d[k] = o[k];
          }
        }
      }
      if constexpr (COPYLG) {
        if ((j % LGP) == LGP - 1 && (!TAIL || r0 + j - (LGP - 1) < H)) {
          const int rs = r0 + j - (LGP - 1);
#pragma unroll
          for (int z = 0; z < 3; ++z) {
            T* g = a.lgt + z * a.lg_stride + qbase + 4 * (rs + (odd ? LGP / 2 : 0));
            if constexpr (sizeof(T) == 2) {
              uint32_t o[LGP];   // per row: columns 4q, 4q+1 then 4q+2, 4q+3
#pragma unroll
              for (int k = 0; k < LGP / 2; ++k) quad_rows(lgP[z], LGP, k, odd, &o[2 * k], &o[2 * k + 1]);
              if (qact) {
                uint4* d = reinterpret_cast<uint4*>(g);
#pragma unroll
                for (int k = 0; k < LGP / 4; ++k) d[k] = make_uint4(o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]);
              }
            } else {
              float4 o[LGP / 2];
#pragma unroll
              for (int k = 0; k < LGP / 2; ++k) {
                float2 lo, hi;
                quad_rows(lgP[z], LGP, k, odd, &lo, &hi);
                o[k] = make_float4(lo.x, lo.y, hi.x, hi.y);
              }
              if (qact) {
                float4* d = reinterpret_cast<float4*>(reinterpret_cast<float*>(g));
#pragma unroll
                for (int k = 0; k < LGP / 2; ++k) d[k] = o[k];
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

// Shared logits: the column-major logit copy of the B * Cl logit planes, one
// thread per (logit plane, 16-row block, column quad), quad fastest so that
// the row loads coalesce; each thread writes whole 16-row runs of its quad.
template <typename T>
__global__ __launch_bounds__(256) void tp_lgcopy(TpArgs<T> a, int64_t nlp) {
  using P = Pair<T>;
  constexpr int RB = 16;                    // rows per thread
  const int H = a.H, W = a.W, Hp = a.Hp, Wq = a.Wq;
  const int nblk = Hp / RB;
  const int64_t total = nlp * Wq * nblk;
  for (int64_t t = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; t < total;
       t += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int qd = static_cast<int>(t % Wq);
    const int64_t rest = t / Wq;
    const int blk = static_cast<int>(rest % nblk);
    const int64_t lp = rest / nblk;
    const int r0 = blk * RB;
    // the quad's two column pairs (the second one clamped: with W % 4 == 2
    // the last quad's second pair is padding)
    const int64_t srcA = lp * H * W + 4 * qd;
    const int64_t srcB = lp * H * W + min(4 * qd + 2, W - 2);
    const int64_t dst = ((lp * Wq + qd) * Hp + r0) * 4;
    const T* ls[3] = {a.l0, a.l1, a.l2};
#pragma unroll
    for (int z = 0; z < 3; ++z) {
      typename P::raw va[RB], vb[RB];
#pragma unroll
      for (int j = 0; j < RB; ++j) {   // rows past H land in the copy's padding
        const int64_t ro = static_cast<int64_t>(min(r0 + j, H - 1)) * W;
        va[j] = P::load(ls[z], srcA + ro);
        vb[j] = P::load(ls[z], srcB + ro);
      }
      T* g = a.lgt + z * a.lg_stride + dst;
      if constexpr (sizeof(T) == 2) {
        uint4* d = reinterpret_cast<uint4*>(g);
#pragma unroll
        for (int q = 0; q < RB / 2; ++q) d[q] = make_uint4(va[2 * q], vb[2 * q], va[2 * q + 1], vb[2 * q + 1]);
      } else {
        float4* d = reinterpret_cast<float4*>(reinterpret_cast<float*>(g));
#pragma unroll
        for (int q = 0; q < RB; ++q) d[q] = make_float4(va[q].x, va[q].y, vb[q].x, vb[q].y);
      }
    }
  }
}

// ===========================================================================
// K2: left->right and right->left on the column-major copy
// ===========================================================================
template <typename T, bool LR, bool RL>
__global__ __launch_bounds__(1024) void tp_hpair(TpArgs<T> a) {
  // two double-buffered lines: left->right (the first pass and the
  // recomputes) and right->left, whose states then stay in LDS across chunks
  __shared__ float lbuf[4 * (2048 + 4)];
  constexpr int PF = 8;
  using P = Pair<T>;
  const int H = a.H, W = a.W, G = a.G, Hp = a.Hp;
  const int t = threadIdx.x;
  const int o0 = 2 * t;                 // image rows o0, o0 + 1
  const bool act = o0 < H;
  const int ol = act ? o0 : 0;
  const int64_t plane = a.plane0 + blockIdx.x;
  const int n4 = H + 4;
  for (int i = t; i < 4 * n4; i += blockDim.x) lbuf[i] = 0.0f;
  __syncthreads();
  LineX lx{lbuf, n4, 0};
  LineX lr{lbuf + 2 * n4, n4, 0};
  const float mA0 = o0 > 0 ? 1.f : 0.f;
  const float mB2 = o0 + 1 < H - 1 ? 1.f : 0.f;

  // One load covers rows o0, o0 + 1 of a column quad (columns 4 qd ..
  // 4 qd + 3): 32 contiguous bytes of lambda*x, 16 (bf16) or 32 of each logit.
  using Q = Quad<T>;
  struct In4 {
    Quad<float>::raw lx;
    typename Q::raw g0, g1, g2;
  };
  const int Wq = a.Wq;
  // the logit copy of this plane (shared logits: of its logit plane)
  const int64_t lgpl = plane + logit_shift(plane, a.C, a.Cl, 1);
  auto load_quad = [&](int qd) {
    In4 v;
    const int64_t qq = min(max(qd, 0), Wq - 1);
    const int64_t i = ((plane * Wq + qq) * Hp + ol) * 4;
    const int64_t il = ((lgpl * Wq + qq) * Hp + ol) * 4;
    v.lx = Quad<float>::load(a.lxt, i);
    v.g0 = Q::load(a.lgt, il);
    v.g1 = Q::load(a.lgt + a.lg_stride, il);
    v.g2 = Q::load(a.lgt + 2 * a.lg_stride, il);
    return v;
  };
  // column c (0..3) of the quad as a per-row view
  struct In {
    float2 lx;
    float g0[2], g1[2], g2[2];
  };
  auto column = [&](const In4& v, int c) {
    In cc;
    float l[2];
    Quad<float>::col(v.lx, c, l);
    cc.lx = make_float2(l[0], l[1]);
    Q::col(v.g0, c, cc.g0);
    Q::col(v.g1, c, cc.g1);
    Q::col(v.g2, c, cc.g2);
    return cc;
  };
  // the horizontal sum is stored in chunks of ckr rows,
  // [plane][row / ckr][column][ckr], so that the bottom->top kernel reads
  // whole chunks contiguously
  const int ckr = a.ckr;
  const int64_t ychunk = plane * a.nckv + o0 / ckr, yoff = o0 % ckr;
  auto yidx = [&](int c) { return (ychunk * W + c) * ckr + yoff; };
  auto recs = [&](const In& v, Rec& ra, Rec& rb) {
    ra = make_rec(v.g0[0], v.g1[0], v.g2[0], v.lx.x, mA0, 1.f);
    rb = make_rec(v.g0[1], v.g1[1], v.g2[1], v.lx.y, 1.f, mB2);
  };
  // one scan step on line ln given the previous states of the neighbouring
  // rows (o0 - 1, o0 + 2): the new pair is the mix of the previous line (or
  // the restart value); publishes it and waits for the whole line
  auto step_nb = [&](LineX& ln, const Rec& ra, const Rec& rb, bool restart, float& hA,
                     float& hB, float nl, float nr) {
    const float na = mix(ra, nl, hA, hB);
    const float nb = mix(rb, hA, hB, nr);
    hA = restart ? ra.lx : na;
    hB = restart ? rb.lx : nb;
    if (act) *reinterpret_cast<float2*>(ln.nxt() + o0 + 2) = make_float2(hA, hB);
    ln.par ^= 1;
    __syncthreads();
  };
  // ... with the neighbours' previous states taken from the line
  auto step = [&](LineX& ln, const Rec& ra, const Rec& rb, bool restart, float& hA, float& hB) {
    const float* pv = ln.cur();
    step_nb(ln, ra, rb, restart, hA, hB, pv[o0 + 1], pv[o0 + 4]);
  };

  // ---- left->right: checkpoints, or the final sum when there is no reverse
  if constexpr (LR) {
    constexpr int PQ = PF / 4;            // column quads in flight
    In4 ring[PQ];
#pragma unroll
    for (int j = 0; j < PQ; ++j) ring[j] = load_quad(j);
    float hA = 0.f, hB = 0.f;
    FwdRestart rst{0, G};
    auto block = [&](int cb, auto tail) {
      constexpr bool TAIL = decltype(tail)::value;
#pragma unroll
      for (int j = 0; j < PQ; ++j) {
        const int qd = cb / 4 + j;
        if (!TAIL || 4 * qd < W) {
          const In4 v4 = ring[j];
          ring[j] = load_quad(qd + PQ);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int c = 4 * qd + i;
            if (!TAIL || c < W) {   // the last quad of W % 4 == 2 holds two columns
              Rec ra, rb;
              recs(column(v4, i), ra, rb);
              step(lx, ra, rb, rst.at(c), hA, hB);
              if (act) {
                if constexpr (RL) {
                  if ((c + 1) % kCkH == 0) store_pair(a.ckh, (plane * a.nckh + c / kCkH) * H + o0, hA, hB);
                } else {
                  store_pair(a.yht, yidx(c), hA, hB);
                }
              }
            }
          }
        }
      }
    };
    int cb = 0;
    for (; cb + PF <= W; cb += PF) block(cb, std::false_type{});
    if (cb < W) block(cb, std::true_type{});
  }

  // ---- right->left in chunks of kCkH columns, recomputing left->right -----
  if constexpr (RL) {
    static_assert(kCkH == 4, "a right->left chunk is one column quad of the copy");
    struct Chunk {
      In4 in;
      float2 ck;      // left->right states of rows o0, o0 + 1 before the chunk
      float2 nb;      // ... and of the neighbouring rows o0 - 1, o0 + 2 (0 past the edge)
    };
    auto load_chunk = [&](int k) {
      Chunk ch;
      ch.in = load_quad(k);
      ch.ck = make_float2(0.f, 0.f);
      ch.nb = make_float2(0.f, 0.f);
      if constexpr (LR) {
        const float* ck = a.ckh + (plane * a.nckh + max(k - 1, 0)) * H;
        ch.ck = *reinterpret_cast<const float2*>(ck + ol);
        ch.nb = make_float2(ck[max(ol - 1, 0)], ck[min(ol + 2, H - 1)]);
      }
      return ch;
    };
    float hrA = 0.f, hrB = 0.f;   // right->left state, carried across chunks
    auto chunk = [&](const Chunk& ch, int k, auto tail) {
      constexpr bool TAIL = decltype(tail)::value;
      const int cs = k * kCkH;
      Rec ra[kCkH], rb[kCkH];
#pragma unroll
      for (int i = 0; i < kCkH; ++i) recs(column(ch.in, i), ra[i], rb[i]);
      float hlA[kCkH], hlB[kCkH];
#pragma unroll
      for (int i = 0; i < kCkH; ++i) { hlA[i] = 0.f; hlB[i] = 0.f; }
      if constexpr (LR) {
        // the first step takes the neighbours' checkpoint states from memory,
        // so the line needs no seeding barrier
        const bool in = k > 0;
        float hA = in ? ch.ck.x : 0.f, hB = in ? ch.ck.y : 0.f;
        const float nl = in && o0 > 0 ? ch.nb.x : 0.f, nr = in && o0 + 2 < H ? ch.nb.y : 0.f;
        FwdRestart rst{fwd_restart_from(cs, G), G};
#pragma unroll
        for (int i = 0; i < kCkH; ++i) {
          if (!TAIL || cs + i < W) {
            if (i == 0) step_nb(lx, ra[i], rb[i], rst.at(cs), hA, hB, nl, nr);
            else step(lx, ra[i], rb[i], rst.at(cs + i), hA, hB);
          }
          hlA[i] = hA;
          hlB[i] = hB;
        }
      }
      // right->left continues on its own line from the previous chunk
      RevRestart rst = rev_counter(min(cs + kCkH - 1, W - 1), W, G);
#pragma unroll
      for (int i = kCkH - 1; i >= 0; --i) {
        const int c = cs + i;
        if (!TAIL || c < W) {
          step(lr, ra[i], rb[i], rst.at(c), hrA, hrB);
          if (act) store_pair(a.yht, yidx(c), hlA[i] + hrA, hlB[i] + hrB);
        }
      }
    };
    int k = (W + kCkH - 1) / kCkH - 1;
    Chunk nxt = load_chunk(k);
    if (W % kCkH) {
      const Chunk cur = nxt;
      nxt = load_chunk(max(k - 1, 0));
      chunk(cur, k, std::true_type{});
      --k;
    }
    for (; k >= 0; --k) {
      const Chunk cur = nxt;
      nxt = load_chunk(max(k - 1, 0));
      chunk(cur, k, std::false_type{});
    }
  }
}

// ===========================================================================
// K3: bottom->top with top->bottom recomputed per chunk, merge, output
// ===========================================================================
template <typename T, int NT, bool TB, bool BT, bool HZ>
__global__ __launch_bounds__(NT) void tp_vbwd(TpArgs<T> a) {
  using S = RowShape<T, NT>;
  constexpr int kCkV = S::CKV;
  __shared__ float lbuf[2 * (S::MAXW + 4)];
  using P = Pair<T>;
  const int H = a.H, W = a.W, G = a.G, Hp = a.Hp;
  const int t = threadIdx.x;
  const int c0 = 2 * t;
  const bool act = c0 < W;
  const int cl = act ? c0 : 0;
  const int64_t plane = a.plane0 + blockIdx.x;
  const int64_t base = plane * H * W;
  const int64_t ls = logit_shift(plane, a.C, a.Cl, static_cast<int64_t>(H) * W);
  const int n4 = W + 4;
  for (int i = t; i < 2 * n4; i += blockDim.x) lbuf[i] = 0.0f;
  __syncthreads();
  LineX lx{lbuf, n4, 0};
  const float mA0 = c0 > 0 ? 1.f : 0.f;
  const float mB2 = c0 + 1 < W - 1 ? 1.f : 0.f;

  struct Chunk {
    Raw2<T> in[kCkV];
    typename P::raw u[kCkV];
    float4 yA[kCkV / 4], yB[kCkV / 4];
    float2 ck;
  };
  auto load_chunk = [&](int k) {
    Chunk ch;
    const int rs = k * kCkV;
#pragma unroll
    for (int i = 0; i < kCkV; ++i) {
      const int64_t idx = base + (int64_t)min(rs + i, H - 1) * W + cl;
      ch.in[i] = load_raw2(a.x, a.lam, a.l0, a.l1, a.l2, idx, ls);
      ch.u[i] = P::load(a.u, idx);
    }
#pragma unroll
    for (int q = 0; q < kCkV / 4; ++q) {
      if constexpr (HZ) {
        // the chunk's rows of columns c0, c0+1: 8 kCkV contiguous bytes
        const float4* y =
            reinterpret_cast<const float4*>(a.yht + ((plane * a.nckv + k) * W + cl) * kCkV);
        ch.yA[q] = y[q];
        ch.yB[q] = y[kCkV / 4 + q];
      } else {
        ch.yA[q] = ch.yB[q] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    ch.ck = make_float2(0.f, 0.f);
    if constexpr (TB)
      ch.ck = *reinterpret_cast<const float2*>(a.ckv + (plane * a.nckv + max(k - 1, 0)) * W + cl);
    return ch;
  };
  auto step = [&](const Rec& ra, const Rec& rb, bool restart, float& hA, float& hB) {
    const float* pv = lx.cur();
    const float na = mix(ra, pv[c0 + 1], hA, hB);
    const float nb = mix(rb, hA, hB, pv[c0 + 4]);
    hA = restart ? ra.lx : na;
    hB = restart ? rb.lx : nb;
    if (act) *reinterpret_cast<float2*>(lx.nxt() + c0 + 2) = make_float2(hA, hB);
    lx.par ^= 1;
    __syncthreads();
  };
  auto seed = [&](float hA, float hB) {
    if (act) *reinterpret_cast<float2*>(lx.nxt() + c0 + 2) = make_float2(hA, hB);
    lx.par ^= 1;
    __syncthreads();
  };
  auto pick = [](const float4* y, int i) {
    const float4 q = y[i / 4];
    const int m = i % 4;
    return m == 0 ? q.x : (m == 1 ? q.y : (m == 2 ? q.z : q.w));
  };

  float hbA = 0.f, hbB = 0.f;   // bottom->top state, carried across chunks
  auto chunk = [&](const Chunk& ch, int k, auto tail) {
    constexpr bool TAIL = decltype(tail)::value;
    const int rs = k * kCkV;
    Rec ra[kCkV], rb[kCkV];
#pragma unroll
    for (int i = 0; i < kCkV; ++i) {
      const Raw2<T>& v = ch.in[i];
      ra[i] = make_rec(P::lo(v.l0), P::lo(v.l1), P::lo(v.l2), P::lo(v.lam) * P::lo(v.x), mA0, 1.f);
      rb[i] = make_rec(P::hi(v.l0), P::hi(v.l1), P::hi(v.l2), P::hi(v.lam) * P::hi(v.x), 1.f, mB2);
    }
    float htA[kCkV], htB[kCkV];
#pragma unroll
    for (int i = 0; i < kCkV; ++i) { htA[i] = 0.f; htB[i] = 0.f; }
    if constexpr (TB) {
      float hA = k > 0 ? ch.ck.x : 0.f, hB = k > 0 ? ch.ck.y : 0.f;
      seed(hA, hB);
      FwdRestart rst{fwd_restart_from(rs, G), G};
#pragma unroll
      for (int i = 0; i < kCkV; ++i) {
        if (!TAIL || rs + i < H) step(ra[i], rb[i], rst.at(rs + i), hA, hB);
        htA[i] = hA;
        htB[i] = hB;
      }
    }
    if constexpr (BT) seed(hbA, hbB);
    RevRestart rst = rev_counter(min(rs + kCkV - 1, H - 1), H, G);
#pragma unroll
    for (int i = kCkV - 1; i >= 0; --i) {
      const int r = rs + i;
      if (!TAIL || r < H) {
        float sA = htA[i] + pick(ch.yA, i), sB = htB[i] + pick(ch.yB, i);
        if constexpr (BT) {
          step(ra[i], rb[i], rst.at(r), hbA, hbB);
          sA += hbA;
          sB += hbB;
        }
        if (act)
          store_pair(a.out, base + (int64_t)r * W + c0, P::lo(ch.u[i]) * sA, P::hi(ch.u[i]) * sB);
      }
    }
  };
  int k = (H + kCkV - 1) / kCkV - 1;
  Chunk nxt = load_chunk(k);
  if (H % kCkV) {
    const Chunk cur = nxt;
    nxt = load_chunk(max(k - 1, 0));
    chunk(cur, k, std::true_type{});
    --k;
  }
  for (; k >= 0; --k) {
    const Chunk cur = nxt;
    nxt = load_chunk(max(k - 1, 0));
    chunk(cur, k, std::false_type{});
  }
}

// ---------------------------------------------------------------------------
bool tpipe_fits(int64_t H, int64_t W) {
  return H >= 2 && W >= 2 && H % 2 == 0 && W % 2 == 0 && W <= 2048 && H <= 2048;
}

namespace {
struct TpLayout {
  int64_t Hp, Wq, nckv, nckh;
  size_t off_lxt, off_lgt, off_yht, off_ckv, off_ckh, total;
};

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

TpLayout tp_layout(int64_t planes, int64_t H, int64_t W, size_t es) {
  TpLayout L;
  const int ckr = row_chunk(W);
  L.Hp = (H + 31) / 32 * 32;
  L.Wq = (W + 3) / 4;
  L.nckv = (H + ckr - 1) / ckr;
  L.nckh = (W + kCkH - 1) / kCkH;
  const size_t cp = static_cast<size_t>(planes * 4 * L.Wq * L.Hp);   // elements of one copy
  size_t o = 0;
  L.off_lxt = o; o = align256(o + cp * 4);
  L.off_lgt = o; o = align256(o + 3 * cp * es);
  L.off_yht = o; o = align256(o + static_cast<size_t>(planes * L.nckv * W) * ckr * 4);
  L.off_ckv = o; o = align256(o + static_cast<size_t>(planes * L.nckv * W) * 4);
  L.off_ckh = o; o = align256(o + static_cast<size_t>(planes * L.nckh * H) * 4);
  L.total = o;
  return L;
}
}  // namespace

size_t tpipe_workspace_bytes(int64_t planes, int64_t H, int64_t W, gspn_dtype dt) {
  return tp_layout(planes, H, W, dt == GSPN_F32 ? 4 : 2).total;
}

template <typename T, int NT>
static hipError_t launch_tpipe_nt(const Problem& pr, void* ws, hipStream_t stream, Tracer* tr) {
  const int64_t planes = pr.B * pr.C;
  const TpLayout L = tp_layout(planes, pr.H, pr.W, sizeof(T));
  char* w = static_cast<char*>(ws);
  TpArgs<T> a;
  a.x = static_cast<const T*>(pr.x);
  a.lam = static_cast<const T*>(pr.lam);
  a.l0 = static_cast<const T*>(pr.l[0]);
  a.l1 = static_cast<const T*>(pr.l[1]);
  a.l2 = static_cast<const T*>(pr.l[2]);
  a.u = static_cast<const T*>(pr.u);
  a.out = static_cast<T*>(pr.out);
  a.lxt = reinterpret_cast<float*>(w + L.off_lxt);
  a.lgt = reinterpret_cast<T*>(w + L.off_lgt);
  a.yht = reinterpret_cast<float*>(w + L.off_yht);
  a.ckv = reinterpret_cast<float*>(w + L.off_ckv);
  a.ckh = reinterpret_cast<float*>(w + L.off_ckh);
  a.H = static_cast<int>(pr.H);
  a.W = static_cast<int>(pr.W);
  a.G = static_cast<int>(pr.G >= pr.H && pr.G >= pr.W ? 0 : pr.G);
  a.Hp = static_cast<int>(L.Hp);
  a.nckv = static_cast<int>(L.nckv);
  a.nckh = static_cast<int>(L.nckh);
  a.Wq = static_cast<int>(L.Wq);
  a.ckr = RowShape<T, NT>::CKV;
  a.mask = pr.mask;
  a.C = pr.C;
  a.Cl = pr.Cl;
  a.lg_stride = planes * 4 * L.Wq * L.Hp;
  a.plane0 = 0;
  const unsigned tv = static_cast<unsigned>((pr.W / 2 + 63) / 64 * 64);
  const unsigned th = static_cast<unsigned>((pr.H / 2 + 63) / 64 * 64);
  const unsigned m = pr.mask;
  const bool tb = m & 1u, bt = m & 2u, lr = m & 4u, rl = m & 8u, hz = lr || rl;
  using K = void (*)(TpArgs<T>);
  const bool shared = pr.Cl < pr.C;
  const K k1 = shared ? (tb ? (hz ? tp_vfwd<T, NT, true, true, false> : tp_vfwd<T, NT, true, false, false>)
                            : tp_vfwd<T, NT, false, true, false>)
                      : (tb ? (hz ? tp_vfwd<T, NT, true, true> : tp_vfwd<T, NT, true, false>)
                            : tp_vfwd<T, NT, false, true>);
  const K k2 = lr ? (rl ? tp_hpair<T, true, true> : tp_hpair<T, true, false>) : tp_hpair<T, false, true>;
  static const K k3s[8] = {tp_vbwd<T, NT, false, false, false>, tp_vbwd<T, NT, true, false, false>,
                           tp_vbwd<T, NT, false, true, false>, tp_vbwd<T, NT, true, true, false>,
                           tp_vbwd<T, NT, false, false, true>, tp_vbwd<T, NT, true, false, true>,
                           tp_vbwd<T, NT, false, true, true>, tp_vbwd<T, NT, true, true, true>};
  const K k3 = k3s[(tb ? 1 : 0) | (bt ? 2 : 0) | (hz ? 4 : 0)];

  // Every kernel needs one whole compute unit per plane, so a plane count a
  // little above the CU count leaves a latency-bound second round. Two plane
  // groups on two streams let one group's K2/K3 overlap the other's tail.
  const int ngroups = pr.one_stream ? 1 : tpipe_groups(planes);
  hipStream_t streams[kMaxGroups] = {stream, stream, stream, stream};
  hipEvent_t fork = nullptr, join[kMaxGroups] = {};
  hipError_t e = hipSuccess;
  if (shared && hz) {
    // the logit copy of each of the B * Cl logit planes, before any K2
    const int64_t nlp = pr.B * pr.Cl;
    const int64_t work = nlp * L.Wq * (L.Hp / 16);
    const int64_t blocks = (work + 255) / 256;
    tr->before(stream, "tp_lgcopy", nlp);
    hipLaunchKernelGGL(tp_lgcopy<T>, dim3(static_cast<unsigned>(blocks < 65536 ? blocks : 65536)),
                       dim3(256), 0, stream, a, nlp);
    tr->after(stream);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
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
  auto launch = [&](K k, unsigned threads, const char* name, int g) -> hipError_t {
    if (gn[g] == 0) return hipSuccess;
    TpArgs<T> ag = a;
    ag.plane0 = g0[g];
    tr->before(streams[g], name, gn[g]);
    hipLaunchKernelGGL(k, dim3(static_cast<unsigned>(gn[g])), dim3(threads), 0, streams[g], ag);
    tr->after(streams[g]);
    return hipGetLastError();
  };
  for (int g = 0; g < ngroups && e == hipSuccess; ++g)
    if (tb || hz) e = launch(k1, tv, "tp_vfwd", g);
  for (int g = 0; g < ngroups && e == hipSuccess; ++g)
    if (hz) e = launch(k2, th, "tp_hpair", g);
  for (int g = 0; g < ngroups && e == hipSuccess; ++g) e = launch(k3, tv, "tp_vbwd", g);
  for (int g = 1; g < ngroups; ++g) {
    hipError_t e2 = hipEventRecord(join[g], streams[g]);
    if (e2 == hipSuccess) e2 = hipStreamWaitEvent(stream, join[g], 0);
    if (e == hipSuccess) e = e2;
  }
  release();
  return e;
}

template <typename T>
static hipError_t launch_tpipe_dt(const Problem& pr, void* ws, hipStream_t stream, Tracer* tr) {
  // the row sweeps take a column pair per thread: 512 threads up to 1024
  // columns, 1024 threads beyond (row_chunk() gives the matching chunk height)
  return pr.W > 1024 ? launch_tpipe_nt<T, 1024>(pr, ws, stream, tr)
                     : launch_tpipe_nt<T, 512>(pr, ws, stream, tr);
}

hipError_t launch_tpipe(const Problem& pr, void* ws, hipStream_t stream, Tracer* tr) {
  if (pr.dtype == GSPN_F32) return launch_tpipe_dt<float>(pr, ws, stream, tr);
  return launch_tpipe_dt<bf16_t>(pr, ws, stream, tr);
}

}  // namespace gspn

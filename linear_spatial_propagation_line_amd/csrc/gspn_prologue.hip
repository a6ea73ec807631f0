// The module prologue: the 1x1 convolutions that produce the propagation's
// inputs (aitntnews page, section GSPN架构: a shared 1x1 convolution reduces
// the channels, three independent 1x1 convolutions produce the logits, lambda
// and u). In [B, C, H, W] layout a 1x1 convolution of image b is a matrix
// product over channels,
//     Y[b] (M x N) = A (M x K) X[b] (K x N) + bias,   N = H * W pixels,
// so the prologue is two launches of one MFMA GEMM kernel:
//     x      = W_r (C x Cin)  X_in[b]          (rounded to the storage type)
//     params = W_p (5C x C)   x[b]             rows t*C .. t*C+C-1 go to the
//                                              t-th of l0, l1, l2, lambda, u
// The second launch reads x as stored, so it sees exactly the rounded x the
// propagation reads.
//
// Why not one kernel with the scan: the scan needs a whole plane of one
// channel, while a 1x1 convolution produces all channels of a pixel tile;
// for the channel counts of the pages' models (320 to 1152) neither the
// plane's parameters nor the image's x fit on chip at once, so the prologue
// writes the scan's inputs once and the scan reads them.
//
// Tiling (gfx950, 64-wide wavefronts): a workgroup of four wavefronts owns a
// 128 x 128 output tile; each wavefront a 64 x 64 quarter, 4 x 4 MFMA tiles
// of 16 x 16 with fp32 accumulators (v_mfma_f32_16x16x32_bf16 for bf16,
// v_mfma_f32_16x16x4_f32 for fp32). K advances one 128-byte row at a time
// (64 bf16 or 32 fp32) through LDS, the next tile's loads in flight while the
// current one is multiplied: the weight tile as [m][k]; the bf16 pixel tile
// transposed to [n][k] (an MFMA operand is 8 consecutive k), written as
// 8-byte runs of four k; the fp32 pixel tile as loaded. The finished tile is staged in LDS
// (64 rows at a time) and written as 16-byte row runs. The linear block index
// walks M fastest, so the M tiles that share a pixel tile run together and
// find it in L2.
#include <cstdlib>

#include "gspn_device.hpp"
#include "gspn_launch.hpp"
#include "gspn_mfma.hpp"

namespace gspn {

namespace {
constexpr int kMT = 128, kNT = 128;
constexpr size_t kXsMaxLds = 150 * 1024;   // pixel-stationary variant up to this LDS size
constexpr int kOP = kNT + 8;     // LDS pitch of the staged output tile

__device__ __forceinline__ float g_ld(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float g_ld(const bf16_t* p, int64_t i) { return to_f32(p[i]); }

// output tensor t of the kernel arguments, picked without indexing them (an
// indexed kernel argument is a memory load the store would have to wait for)
template <typename T>
__device__ __forceinline__ T* pick_out(T* const (&out)[5], int t) {
  return t == 0 ? out[0] : t == 1 ? out[1] : t == 2 ? out[2] : t == 3 ? out[3] : out[4];
}

// one element kept in storage form in LDS
__device__ __forceinline__ uint16_t raw(bf16_t v) { return v.bits; }
__device__ __forceinline__ float raw(float v) { return v; }
}  // namespace

template <typename T>
struct GemmArgs {
  const T* A;       // [M][K]
  const T* bias;    // [M] or null
  const T* X;       // [B][K][N]
  T* out[5];        // output tensor t holds rows t*Mt .. t*Mt+Mt-1: [B][Mt][N]
  int M, K, N, Mt;
  int64_t B;        // images
  int vec_a, vec_x, vec_o;   // 16-byte runs allowed for A rows, X rows, output rows
};

// 16 bytes of consecutive elements p[i .. ], the first `avail` of them real
// and the rest zero (a whole vector load when allowed)
template <typename T>
__device__ __forceinline__ uint4 run16(const T* p, int64_t i, int avail, bool vec) {
  constexpr int E = 16 / sizeof(T);
  if (vec && avail >= E) return *reinterpret_cast<const uint4*>(p + i);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (e < avail) {
      if constexpr (sizeof(T) == 2)
        w[e >> 1] |= static_cast<uint32_t>(reinterpret_cast<const uint16_t*>(p)[i + e])
                     << (16 * (e & 1));
      else
        w[e] = __float_as_uint(reinterpret_cast<const float*>(p)[i + e]);
    }
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ uint32_t half16(const uint4& v, int e) {
  const uint32_t w = e < 2 ? v.x : (e < 4 ? v.y : (e < 6 ? v.z : v.w));
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

__device__ __forceinline__ u32x4 vec4(const uint4& v) { return u32x4{v.x, v.y, v.z, v.w}; }
__device__ __forceinline__ uint32_t half16(const u32x4& v, int e) {
  const uint32_t w = v[e >> 1];
  return (e & 1) ? (w >> 16) : (w & 0xffffu);
}

// The finished M x 128 tile: bias, rounding to the storage type, staging
// half a tile (MT / 2 rows, the two wavefronts of one row half) at a time in
// LDS, then 16-byte row runs to the output tensors.
template <typename T, bool FULL, int MT>
__device__ __forceinline__ void store_tile(const GemmArgs<T>& a, const f32x4 (&acc)[MT / 32][4],
                                           decltype(raw(T{}))* Os, int m0, int n0, int64_t b,
                                           int tid, int wave) {
  using R = decltype(raw(T{}));
  constexpr int MI = MT / 32;
  constexpr int E = 16 / sizeof(T);
  const int M = a.M, N = a.N;
  const int lane = tid & 63, wn = (wave & 1) * 64;
  // lane l holds rows 4 (l / 16) + e, column l % 16 of each 16 x 16 tile
  const int col = lane & 15, rq = (lane >> 4) * 4;
  for (int h = 0; h < 2; ++h) {
    if ((wave >> 1) == h) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * i + rq + e;          // row within the half
          const int m = m0 + h * (MT / 2) + r;
          const float bv = (a.bias && m < M) ? g_ld(a.bias, m) : 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float v = acc[i][j][e] + bv;
            if constexpr (sizeof(T) == 2)
              Os[r * kOP + wn + 16 * j + col] = static_cast<uint16_t>(f32_to_bf16_bits(v));
            else
              Os[r * kOP + wn + 16 * j + col] = v;
          }
        }
    }
    lds_barrier();
    // the half's rows to their output tensors, 16-byte runs
    for (int c = tid; c < (MT / 2) * kNT / E; c += 256) {
      const int r = c / (kNT / E), nn = (c % (kNT / E)) * E;
      const int m = m0 + h * (MT / 2) + r, n = n0 + nn;
      if (!FULL && (m >= M || n >= N)) continue;
      const int t = m / a.Mt, mr = m - t * a.Mt;
      T* dst = pick_out(a.out, t) + (b * a.Mt + mr) * static_cast<int64_t>(N);
      const R* src = Os + r * kOP + nn;
      if (FULL || (a.vec_o && n + E <= N)) {
        *reinterpret_cast<uint4*>(dst + n) = *reinterpret_cast<const uint4*>(src);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          if (n + e >= N) break;
          if constexpr (sizeof(T) == 2) dst[n + e].bits = src[e];
          else dst[n + e] = src[e];
        }
      }
    }
    lds_barrier();
  }
}

// FULL: M and N multiples of 128, K a multiple of the K tile, every tensor in
// 16-byte runs. Then no access needs a bounds check, and the code between
// memory waits is straight-line, so the compiler can count what is in
// flight instead of draining the in-order memory counter at every check.
template <typename T, bool FULL, int MT>
__global__ __launch_bounds__(256, 1) void prologue_gemm(GemmArgs<T> a) {
  static_assert(MT == 128 || MT == 96, "M tile: 4 or 3 MFMA tiles per wavefront");
  constexpr int MI = MT / 32;                // 16-row MFMA tiles per wavefront
  constexpr int QA = MT * 8 / 256;           // 16-byte weight runs per thread per K tile
  using R = decltype(raw(T{}));   // uint16_t (bf16 bits) or float
  constexpr bool BF = sizeof(T) == 2;
  constexpr int E = 16 / sizeof(T);          // elements in 16 bytes
  constexpr int KT = 128 / sizeof(T);        // K per tile: 128-byte rows
  constexpr int AP = KT + 16 / sizeof(T);    // pitch of the weight tile [m][k]
  // pixel tile as loaded, [k][n]: an fp32 operand is one value, a bf16
  // operand (8 consecutive k of one n) comes from two transposing reads. The
  // bf16 pitch of 144 elements puts the four rows a 16-lane group reads 8
  // banks apart.
  constexpr int BP = BF ? kNT + 16 : kNT + 4;
  constexpr int kABytes = MT * AP * sizeof(R);
  constexpr int kBBytes = KT * BP * sizeof(R);
  constexpr int kOutBytes = (MT / 2) * kOP * sizeof(R);
  constexpr int kSmem = kABytes + kBBytes > kOutBytes ? kABytes + kBBytes : kOutBytes;
  __shared__ __align__(16) unsigned char smem[kSmem];
  R* As = reinterpret_cast<R*>(smem);
  R* Bs = reinterpret_cast<R*>(smem + kABytes);
  R* Os = reinterpret_cast<R*>(smem);        // [MT / 2][kOP], after the K loop

  const int M = a.M, K = a.K, N = a.N;
  const int nmt = (M + MT - 1) / MT;
  // Workgroups are dealt to the 8 XCDs in turn, each with its own L2. Over
  // all images' tiles, tile t runs on XCD t / per, so consecutive tiles --
  // the M tiles that share a pixel tile, then the next pixel tiles and
  // images -- meet in one L2, and every XCD gets a share.
  const int tiles = nmt * ((N + kNT - 1) / kNT);
  const int64_t all = static_cast<int64_t>(tiles) * a.B;
  const int64_t per = (all + 7) / 8;
  const int64_t t = static_cast<int64_t>(blockIdx.x % 8) * per + blockIdx.x / 8;
  if (t >= all) return;
  const int64_t b = t / tiles;
  const int tile = static_cast<int>(t - b * tiles);
  const int m0 = (tile % nmt) * MT;
  const int n0 = (tile / nmt) * kNT;
  const T* X = a.X + b * static_cast<int64_t>(K) * N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = (wave >> 1) * (MT / 2), wn = (wave & 1) * 64;   // this wavefront's quarter

  f32x4 acc[MI][4];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Each thread moves four 16-byte runs of the weight tile and four of the
  // pixel tile per K tile; the next tile's runs are loaded into registers
  // while the current one is multiplied.
  //   weights: run c = tid + 256 q is row c / 8, k offset (c % 8) * E
  //   pixels, bf16: rows 4 g .. 4 g + 3 (g = tid / 16), pixels 8 (tid % 16) ..
  //   pixels, fp32: run c = tid + 256 q is k row c / 32, pixels (c % 32) * 4 ..
  // two register sets: the straight-line variant for whole tiles keeps the
  // loads of two K tiles in flight (one K tile of products, about 0.2 us, is
  // shorter than a memory latency); the general one uses the first only
  u32x4 pa[QA], px[4], pb[QA], py[4];
  auto fetch_to = [&](int k0, u32x4 (&pa)[QA], u32x4 (&px)[4]) {
#pragma unroll
    for (int q = 0; q < QA; ++q) {
      const int c = tid + 256 * q, r = c / (KT / E), kk = (c % (KT / E)) * E;
      const int m = m0 + r, k = k0 + kk;
      if constexpr (FULL)
        pa[q] = *reinterpret_cast<const u32x4*>(a.A + static_cast<int64_t>(m) * K + k);
      else
        pa[q] = vec4(run16(a.A, static_cast<int64_t>(m) * K + k, m < M ? K - k : 0, a.vec_a));
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int k, n;
      if constexpr (BF) {
        k = k0 + 4 * (tid >> 4) + q;
        n = n0 + 8 * (tid & 15);
      } else {
        const int c = tid + 256 * q;
        k = k0 + c / (kNT / E);
        n = n0 + (c % (kNT / E)) * E;
      }
      if constexpr (FULL)
        px[q] = *reinterpret_cast<const u32x4*>(X + static_cast<int64_t>(k) * N + n);
      else
        px[q] = vec4(run16(X, static_cast<int64_t>(k) * N + n, k < K ? N - n : 0, a.vec_x));
    }
  };
  auto fetch = [&](int k0) { fetch_to(k0, pa, px); };
  auto stash_from = [&](const u32x4 (&pa)[QA], const u32x4 (&px)[4]) {
#pragma unroll
    for (int q = 0; q < QA; ++q) {
      const int c = tid + 256 * q, r = c / (KT / E), kk = (c % (KT / E)) * E;
      *reinterpret_cast<u32x4*>(As + r * AP + kk) = pa[q];
    }
    if constexpr (BF) {
      // four k rows of eight pixels, as loaded
      const int kr = 4 * (tid >> 4), nl = 8 * (tid & 15);
#pragma unroll
      for (int q = 0; q < 4; ++q) *reinterpret_cast<u32x4*>(Bs + (kr + q) * BP + nl) = px[q];
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = tid + 256 * q, kr = c / (kNT / E), nn = (c % (kNT / E)) * E;
        *reinterpret_cast<u32x4*>(Bs + kr * BP + nn) = px[q];
      }
    }
  };

  auto stash = [&]() { stash_from(pa, px); };

  // the products of the K tile in LDS
  auto multiply = [&]() {
    if constexpr (BF) {
      // v_mfma_f32_16x16x32_bf16: lane l holds A[l % 16][8 (l / 16) .. +7]
      // and B[8 (l / 16) .. +7][l % 16]; two of them cover K = 64
      const int r = lane & 15, kq = (lane >> 4) * 8;
      // transposing reads: lane c of each 16-lane group points at row c / 4,
      // columns 4 (c % 4) .. of its group's 4 x 16 block
      const int tr_off = (kq + (r >> 2)) * BP + 4 * (r & 3);
#pragma unroll
      for (int kh = 0; kh < KT; kh += 32) {
        bf16x8 fa[MI], fb[4];
#pragma unroll
        for (int i = 0; i < MI; ++i)
          fa[i] = *reinterpret_cast<const bf16x8*>(As + (wm + 16 * i + r) * AP + kh + kq);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint16_t* bp = reinterpret_cast<const uint16_t*>(Bs) + kh * BP + wn + 16 * j + tr_off;
          const v4i16 lo = lds_read_tr(bp), hi = lds_read_tr(bp + 4 * BP);
          fb[j] = __builtin_bit_cast(bf16x8, v8i16{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w});
        }
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
    } else {
      // v_mfma_f32_16x16x4_f32: lane l holds A[l % 16][l / 16] and
      // B[l / 16][l % 16]; eight of them cover K = 32
      const int r = lane & 15, kq = lane >> 4;
#pragma unroll
      for (int ks = 0; ks < KT; ks += 4) {
        float fa[MI], fb[4];
#pragma unroll
        for (int i = 0; i < MI; ++i) fa[i] = As[(wm + 16 * i + r) * AP + ks + kq];
#pragma unroll
        for (int j = 0; j < 4; ++j) fb[j] = Bs[(ks + kq) * BP + wn + 16 * j + r];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
    }
  };

  if constexpr (FULL) {
    // whole tiles and an even number of K tiles: set a holds the even K
    // tiles, set b the odd ones, each refilled two K tiles ahead right after
    // it is stored (the last refills fetch the last tile again). The first
    // tile is peeled, so that the loop is entered with the loads in flight
    // in the same order as at its back edge: set b's, then set a's.
    fetch_to(0, pa, px);
    fetch_to(KT, pb, py);
    stash_from(pa, px);
    fetch_to(min(2 * KT, K - KT), pa, px);
    lds_barrier();
    multiply();
    lds_barrier();
    for (int k0 = KT; k0 < K - KT; k0 += 2 * KT) {
      stash_from(pb, py);
      fetch_to(min(k0 + 2 * KT, K - KT), pb, py);
      lds_barrier();
      multiply();
      lds_barrier();
      stash_from(pa, px);
      fetch_to(min(k0 + 3 * KT, K - KT), pa, px);
      lds_barrier();
      multiply();
      lds_barrier();
    }
    stash_from(pb, py);   // the last K tile
    lds_barrier();
    multiply();
    lds_barrier();
  } else {
    fetch(0);
    for (int k0 = 0; k0 < K; k0 += KT) {
      stash();
      lds_barrier();
      if (k0 + KT < K) fetch(k0 + KT);
      multiply();
      lds_barrier();
    }
  }

  store_tile<T, FULL, MT>(a, acc, Os, m0, n0, b, tid, wave);
}

// bf16, whole tiles (the FULL conditions): the same tiling, with the K loop's
// stages (K = 32) moved from global memory straight into LDS by
// global_load_lds_dwordx4, NS stages in a ring, loads NS - 1 stages ahead of
// the multiply. Two stages (one ahead) measured best: 28-32 KB of LDS leave
// room for four workgroups per CU, where three stages (three workgroups) and
// four (two) were 10% and 20% slower on the DiT-width products. Each instruction writes 64 lanes x 16 bytes as one
// contiguous 1 KB block (lane i at 16 i), so each lane's source is chosen to
// give the block the layout the fragment reads want:
//   weight block t (rows 16 t .. 16 t + 15 of the M tile, 64 bytes each):
//     lane i fills row i / 4, slot i % 4 with the row's 16-byte unit
//     (i % 4) ^ sw(i / 4), sw(r) = ((r >> 1) ^ (r >> 2)) & 3, so the 16 rows
//     a fragment read takes hit distinct banks;
//   pixel block j (k rows 4 j .. 4 j + 3, 128 pixels each): lane i fills row
//     4 j + i / 16 at stored pixels 8 (i % 16) .. + 7, the row's 16-pixel
//     blocks stored at block ^ tsw(row), so the four rows a transposing read
//     takes are in different banks.
// Same products in the same order as prologue_gemm: the same bits.
template <int MT, int NS>
__global__ __launch_bounds__(256, 2) void prologue_gemm_lds(GemmArgs<bf16_t> a) {
  constexpr int MI = MT / 32;                // 16-row MFMA tiles per wavefront
  constexpr int KS = 32;                     // K per stage
  constexpr int ABLK = MT / 16, BBLK = KS * kNT * 2 / 1024, NBLK = ABLK + BBLK;
  constexpr int STAGE = NBLK * 1024;
  constexpr int kOutBytes = (MT / 2) * kOP * 2;
  constexpr int kSmem = NS * STAGE > kOutBytes ? NS * STAGE : kOutBytes;
  __shared__ __align__(16) unsigned char smem[kSmem];
  uint16_t* Os = reinterpret_cast<uint16_t*>(smem);   // [MT / 2][kOP], after the K loop

  const int M = a.M, K = a.K, N = a.N;
  const int nmt = M / MT;
  // the tile order of prologue_gemm: XCD t / per runs tile t
  const int tiles = nmt * (N / kNT);
  const int64_t all = static_cast<int64_t>(tiles) * a.B;
  const int64_t per = (all + 7) / 8;
  const int64_t t = static_cast<int64_t>(blockIdx.x % 8) * per + blockIdx.x / 8;
  if (t >= all) return;
  const int64_t b = t / tiles;
  const int tile = static_cast<int>(t - b * tiles);
  const int m0 = (tile % nmt) * MT;
  const int n0 = (tile / nmt) * kNT;
  const bf16_t* X = a.X + b * static_cast<int64_t>(K) * N;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS bases in SGPRs
  const int wm = (wave >> 1) * (MT / 2), wn = (wave & 1) * 64;   // this wavefront's quarter
  const int r16 = lane & 15, g = lane >> 4;

  f32x4 acc[MI][4];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto sw = [](int r) { return ((r >> 1) ^ (r >> 2)) & 3; };
  auto tsw = [](int k) { return (k & 3) | ((k >> 1) & 4); };
  // wave w loads blocks w, w + 4, w + 8, w + 12 of each stage (those below
  // NBLK): its source pointers at stage 0 and their step per stage
  const int nld = (NBLK - wave + 3) / 4;
  const bf16_t* src[4];
  int64_t step[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int blk = wave + 4 * q < NBLK ? wave + 4 * q : wave;
    if (blk < ABLK) {
      const int r = lane >> 2;
      src[q] = a.A + static_cast<int64_t>(m0 + 16 * blk + r) * K + 8 * ((lane & 3) ^ sw(r));
      step[q] = KS;
    } else {
      const int row = 4 * (blk - ABLK) + (lane >> 4), pos = 8 * (lane & 15);
      const int n = n0 + ((((pos >> 4) ^ tsw(row)) << 4) | (pos & 15));
      src[q] = X + static_cast<int64_t>(row) * N + n;
      step[q] = static_cast<int64_t>(KS) * N;
    }
  }
  auto issue = [&](int st) {
    unsigned char* base = smem + (st % NS) * STAGE;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (q < nld)
        __builtin_amdgcn_global_load_lds(src[q] + st * step[q], base + (wave + 4 * q) * 1024,
                                         16, 0, 0);
  };
  // LDS byte addresses of this lane's transposing reads in stage 0: rows
  // 8 (l / 16) + (l % 16) / 4 (+ 4: 1 KB further, rows k + 4 share k's
  // swizzle), pixels wn + 16 j + 4 (l % 4) ..
  const uint32_t lds_base = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) unsigned char*)smem));
  uint32_t tr_addr[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 8 * g + (r16 >> 2), n = wn + 16 * j + 4 * (r16 & 3);
    tr_addr[j] = lds_base + ABLK * 1024 +
                 2 * (row * kNT + ((((n >> 4) ^ tsw(row)) << 4) | (n & 15)));
  }
  auto multiply = [&](int st) {
    const unsigned char* base = smem + (st % NS) * STAGE;
    bf16x8 fa[MI], fb[4];
#pragma unroll
    for (int i = 0; i < MI; ++i)
      fa[i] = *reinterpret_cast<const bf16x8*>(base + (wm / 16 + i) * 1024 + r16 * 64 +
                                               16 * (g ^ sw(r16)));
    // the transposing reads (rows + 4 are 1 KB further)
    const uint32_t so = static_cast<uint32_t>((st % NS) * STAGE);
    const uint32_t q[4] = {tr_addr[0] + so, tr_addr[1] + so, tr_addr[2] + so, tr_addr[3] + so};
    lds_read_tr_b4<1024>(q, fb);
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  };

  const int S = K / KS;
  constexpr int AH = NS - 1;                 // stages loaded ahead
  for (int st = 0; st < AH && st < S; ++st) issue(st);
  for (int st = 0; st < S; ++st) {
    // this wave's loads of stage st are done when at most the later stages'
    // are in flight (vector memory loads complete in order)
    wait_vmcnt_of((AH - 1 < S - 1 - st ? AH - 1 : S - 1 - st) * nld);
    // every wave's loads of stage st are in, and stage st - 1 is no longer read
    bare_barrier();
    if (st + AH < S) issue(st + AH);
    multiply(st);
  }
  lds_barrier();   // the output staging overwrites the stages
  store_tile<bf16_t, true, MT>(a, acc, Os, m0, n0, b, tid, wave);
}

// Pixel-stationary variant for small K (all K rows of a 64-pixel tile fit
// in LDS). A block owns one pixel tile, loads it once and loops over every M
// tile; each wavefront owns 32 rows x 64 pixels of an M tile (2 x 4 MFMA
// tiles). Weight fragments come straight from global memory (a few hundred
// KB, resident in L2) into registers a whole M tile ahead; the pixel
// operands come from the LDS tile. Each finished strip is staged in the
// wavefront's own LDS slice and written as 16-byte row runs halfway through
// the next tile.
//
// The memory counter the hardware waits on is in-order, and the compiler
// can only count what is in flight on straight-line code: a conditional or
// variable-length load or store anywhere makes it wait for everything,
// prefetches included. So this kernel has none: K is a compile-time multiple
// of the step, every load is an unconditional 16-byte run at a clamped
// address, the prefetch of the next M tile always runs (the last tile
// reloads itself), the bias is staged in LDS once, and each store is one
// masked 16-byte run. The host takes this path only when K, M and every
// tensor allow it.
constexpr int kXsMaxSteps = 12;   // K steps of one M tile held in registers

template <typename T>
__host__ __device__ constexpr int xs_kstep() { return sizeof(T) == 2 ? 32 : 16; }

// pixel tile width and output slice pitch of this variant: 64 pixels keep
// its LDS near 67 KB, so two blocks share a CU and one block's loads and
// waits overlap the other's products
constexpr int kNX = 64;
constexpr int kOX = kNX + 8;

// LDS bytes: pixel tile (bf16 [n][k] with 8 spare k, fp32 [k][n]), four
// 32-row output slices, the bias of all M rows in fp32
template <typename T>
__host__ __device__ constexpr size_t xs_lds_bytes(int K, int M) {
  return (sizeof(T) == 2 ? static_cast<size_t>(kNX) * (K + 8) * 2
                         : static_cast<size_t>(K) * (kNX + 4) * 4) +
         static_cast<size_t>(4 * 32 * kOX) * sizeof(T) + static_cast<size_t>(M) * 4;
}

// The XCD-aware tile order pays on planes of many tiles (a 2048 x 1024
// plane has 32768); on small planes (a 56 x 56 plane has 49) the padding
// to a multiple of 8 costs more than the pages save.
__host__ __device__ constexpr bool xs_xcd_order(int ntiles) { return ntiles >= 1024; }

// two blocks per CU (LDS), two wavefronts per SIMD
template <typename T, int NKS>
__global__ __launch_bounds__(256, 2) void prologue_xs(GemmArgs<T> a) {
  extern __shared__ __align__(16) unsigned char dsm[];
  using R = decltype(raw(T{}));
  constexpr bool BF = sizeof(T) == 2;
  constexpr int E = 16 / sizeof(T);
  constexpr int KS = xs_kstep<T>();
  constexpr int K = NKS * KS;
  constexpr int KP = BF ? K + 8 : kNX + 4;   // bf16 [kNX][KP]; fp32 [K][KP]
  const int M = a.M, N = a.N;
  R* Xs = reinterpret_cast<R*>(dsm);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  R* Os = Xs + (BF ? kNX * KP : K * KP) + wave * 32 * kOX;   // this wavefront's [32][kOX]
  float* Bsh = reinterpret_cast<float*>(Xs + (BF ? kNX * KP : K * KP) + 4 * 32 * kOX);   // [M]
  // XCD-aware tile order on large planes: workgroups are dealt to the 8
  // XCDs in turn, so XCD x takes the contiguous pixel tiles [x per,
  // (x + 1) per) and the tiles running at once on an XCD write neighbouring
  // pieces of every output row (the same pages, one translation each in the
  // XCD's caches)
  const int ntiles = (N + kNX - 1) / kNX;
  int tile = static_cast<int>(blockIdx.x);
  if (xs_xcd_order(ntiles)) {
    const int per = (ntiles + 7) / 8;
    tile = static_cast<int>(blockIdx.x % 8) * per + static_cast<int>(blockIdx.x / 8);
    if (tile >= ntiles) return;
  }
  const int n0 = tile * kNX;
  const int64_t b = blockIdx.y;
  const T* X = a.X + b * static_cast<int64_t>(K) * N;

  // the pixel tile (pixels past N read a clamped, valid run; their outputs
  // are not stored)
  if constexpr (BF) {
    const int nl = 8 * (tid & 7);
    const int n = min(n0 + nl, N - E);
#pragma unroll
    for (int g0 = 0; g0 < K / 4; g0 += 32) {
      const int g = g0 + (tid >> 3);
      if (g < K / 4) {
        uint4 v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          v[q] = *reinterpret_cast<const uint4*>(X + static_cast<int64_t>(4 * g + q) * N + n);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          *reinterpret_cast<uint2*>(Xs + (nl + e) * KP + 4 * g) =
              make_uint2(half16(v[0], e) | (half16(v[1], e) << 16),
                         half16(v[2], e) | (half16(v[3], e) << 16));
      }
    }
  } else {
#pragma unroll
    for (int c0 = 0; c0 < K * (kNX / E); c0 += 256) {
      const int c = c0 + tid;
      if (c < K * (kNX / E)) {
        const int k = c / (kNX / E), nn = (c % (kNX / E)) * E;
        const int n = min(n0 + nn, N - E);
        *reinterpret_cast<uint4*>(Xs + k * KP + nn) =
            *reinterpret_cast<const uint4*>(X + static_cast<int64_t>(k) * N + n);
      }
    }
  }
  // the bias, once (the loop below then has no load it must wait for at once)
  for (int i = tid; i < M; i += 256) Bsh[i] = a.bias ? g_ld(a.bias, i) : 0.f;
  lds_barrier();

  // the weight fragments of K step ks sit in slot ks; right after step ks of
  // M tile mt is multiplied, slot ks is refilled with step ks of M tile
  // mt + 1 (of mt itself on the last tile)
  const int nmt = (M + kMT - 1) / kMT;
  const int r16 = lane & 15, q = lane >> 4;
  // bf16: lane holds k = 8q .. 8q+7 of the step; fp32: four consecutive k
  // 4q .. 4q+3, used one per MFMA (any k order works if both operands agree)
  auto wload = [&](int mt, int ks, int i) {
    const int m = min(mt * kMT + 32 * wave + 16 * i + r16, M - 1);
    return *reinterpret_cast<const uint4*>(a.A + static_cast<int64_t>(m) * K + ks * KS +
                                           (BF ? 8 : 4) * q);
  };
  uint4 fa0[NKS], fa1[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    fa0[ks] = wload(0, ks, 0);
    fa1[ks] = wload(0, ks, 1);
  }
  const int col = lane & 15, rq = (lane >> 4) * 4;
  // the staged strip of M tile mt to its output rows (mt = -1: nothing);
  // called halfway through the next tile's K loop, so that the stores are
  // not still in flight at the next wait on the in-order memory counter
  auto store_tile = [&](int mt) {
#pragma unroll
    for (int c0 = 0; c0 < 32 * kNX / E; c0 += 64) {
      const int c = c0 + lane;
      const int r = c / (kNX / E), nn = (c % (kNX / E)) * E;
      const int m = mt * kMT + 32 * wave + r, n = n0 + nn;
      const uint4 v = *reinterpret_cast<const uint4*>(Os + r * kOX + nn);
      if (mt >= 0 && m < M && n < N) {
        const int t = m / a.Mt, mr = m - t * a.Mt;
        T* dst = pick_out(a.out, t) + (b * a.Mt + mr) * static_cast<int64_t>(N) + n;
        *reinterpret_cast<uint4*>(dst) = v;
      }
    }
  };
  for (int mt = 0; mt < nmt; ++mt) {
    const int mn = min(mt + 1, nmt - 1);
    f32x4 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int kb = ks * KS;
      if constexpr (BF) {
        const bf16x8 A0 = __builtin_bit_cast(bf16x8, fa0[ks]);
        const bf16x8 A1 = __builtin_bit_cast(bf16x8, fa1[ks]);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x8 fb = *reinterpret_cast<const bf16x8*>(Xs + (16 * j + r16) * KP + kb + 8 * q);
          acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, fb, acc[0][j], 0, 0, 0);
          acc[1][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, fb, acc[1][j], 0, 0, 0);
        }
      } else {
        const float a0[4] = {__uint_as_float(fa0[ks].x), __uint_as_float(fa0[ks].y),
                             __uint_as_float(fa0[ks].z), __uint_as_float(fa0[ks].w)};
        const float a1[4] = {__uint_as_float(fa1[ks].x), __uint_as_float(fa1[ks].y),
                             __uint_as_float(fa1[ks].z), __uint_as_float(fa1[ks].w)};
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float fb = Xs[(kb + 4 * q + s4) * KP + 16 * j + r16];
            acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0[s4], fb, acc[0][j], 0, 0, 0);
            acc[1][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1[s4], fb, acc[1][j], 0, 0, 0);
          }
        }
      }
      fa0[ks] = wload(mn, ks, 0);
      fa1[ks] = wload(mn, ks, 1);
      if (ks == NKS / 2) store_tile(mt - 1);
    }
    lds_wave_sync();   // the slice's reads by store_tile precede the staging below
    // bias, rounding, staging (lane holds rows 4 (l / 16) + e, column l % 16
    // of each 16 x 16 tile) in this wavefront's own LDS slice
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 16 * i + rq + e;
        const float bv = Bsh[min(mt * kMT + 32 * wave + r, M - 1)];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float v = acc[i][j][e] + bv;
          if constexpr (BF)
            Os[r * kOX + 16 * j + col] = static_cast<uint16_t>(f32_to_bf16_bits(v));
          else
            Os[r * kOX + 16 * j + col] = v;
        }
      }
    lds_wave_sync();
  }
  store_tile(nmt - 1);
}

template <typename T, int NKS>
hipError_t launch_xs(const GemmArgs<T>& g, int64_t B, const char* name, hipStream_t stream,
                     Tracer* tr) {
  auto kern = prologue_xs<T, NKS>;
  const size_t lds = xs_lds_bytes<T>(NKS * xs_kstep<T>(), g.M);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  // with the XCD-aware order, 8 x ceil(tiles / 8) workgroups, so that every
  // tile has one
  const int ntiles = (g.N + kNX - 1) / kNX;
  const int gx = xs_xcd_order(ntiles) ? (ntiles + 7) / 8 * 8 : ntiles;
  const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(B));
  tr->before(stream, name, B);
  hipLaunchKernelGGL(kern, grid, dim3(256), lds, stream, g);
  tr->after(stream);
  return hipGetLastError();
}

// the pixel-stationary kernel for this K, or hipErrorInvalidValue when K is
// not a multiple of the step up to kXsMaxSteps steps
template <typename T>
hipError_t launch_xs_k(const GemmArgs<T>& g, int64_t B, const char* name, hipStream_t stream,
                       Tracer* tr) {
  switch (g.K / xs_kstep<T>()) {
    case 1: return launch_xs<T, 1>(g, B, name, stream, tr);
    case 2: return launch_xs<T, 2>(g, B, name, stream, tr);
    case 3: return launch_xs<T, 3>(g, B, name, stream, tr);
    case 4: return launch_xs<T, 4>(g, B, name, stream, tr);
    case 5: return launch_xs<T, 5>(g, B, name, stream, tr);
    case 6: return launch_xs<T, 6>(g, B, name, stream, tr);
    case 7: return launch_xs<T, 7>(g, B, name, stream, tr);
    case 8: return launch_xs<T, 8>(g, B, name, stream, tr);
    case 9: return launch_xs<T, 9>(g, B, name, stream, tr);
    case 10: return launch_xs<T, 10>(g, B, name, stream, tr);
    case 11: return launch_xs<T, 11>(g, B, name, stream, tr);
    case 12: return launch_xs<T, 12>(g, B, name, stream, tr);
    default: return hipErrorInvalidValue;
  }
}

namespace {
bool al16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

template <typename T>
hipError_t gemm(const T* A, const T* bias, const T* X, T* const* outs, int nout, int64_t B,
                int M, int K, int N, const char* name, hipStream_t stream, Tracer* tr) {
  GemmArgs<T> g;
  g.A = A;
  g.bias = bias;
  g.X = X;
  for (int t = 0; t < 5; ++t) g.out[t] = t < nout ? outs[t] : nullptr;
  g.M = M;
  g.K = K;
  g.N = N;
  g.Mt = M / nout;
  g.B = B;
  constexpr int E = 16 / sizeof(T);
  g.vec_a = K % E == 0 && al16(A);
  g.vec_x = N % E == 0 && al16(X);
  bool vo = N % E == 0;
  for (int t = 0; t < nout; ++t) vo = vo && al16(outs[t]);
  g.vec_o = vo;
  // the pixel-stationary kernel where its straight-line conditions hold
  const int ks = xs_kstep<T>();
  if (K % ks == 0 && K / ks <= kXsMaxSteps && xs_lds_bytes<T>(K, M) <= kXsMaxLds &&
      M % 32 == 0 && g.vec_a && g.vec_x && g.vec_o)
    return launch_xs_k<T>(g, B, name, stream, tr);
  // M tile height: the one that leaves the least work on the busiest compute
  // unit (tiles spread evenly, each unit's time proportional to its tiles'
  // rows), the taller one on a tie
  const int64_t ntn = (N + kNT - 1) / kNT;
  auto load = [&](int mt) {
    const int64_t t = (M + mt - 1) / mt * ntn * B;
    return (t + cu_count() - 1) / cu_count() * mt;
  };
  int mt = load(96) < load(128) ? 96 : 128;
  // whole bf16 tiles load their stages straight into LDS (below); with four
  // workgroups per CU the taller tile measured 5% faster whatever the tile
  // count, so it is taken whenever M allows
  const int kt = 128 / static_cast<int>(sizeof(T));
  const bool whole_nk = N % kNT == 0 && K % (2 * kt) == 0 && g.vec_a && g.vec_x && g.vec_o;
  const char* lds_env = std::getenv("GSPN_GEMM_LDS");
  const bool lds = sizeof(T) == 2 && whole_nk && K % 32 == 0 && !(lds_env && lds_env[0] == '0');
  if (lds && M % 128 == 0) mt = 128;
  else if (lds && M % 96 == 0) mt = 96;
  const int64_t tiles = (M + mt - 1) / mt * ntn * B;
  const dim3 grid(static_cast<unsigned>((tiles + 7) / 8 * 8));
  // the straight-line variant: whole tiles, an even number of K tiles
  const bool full = M % mt == 0 && whole_nk;
  auto kern = mt == 96 ? (full ? prologue_gemm<T, true, 96> : prologue_gemm<T, false, 96>)
                       : (full ? prologue_gemm<T, true, 128> : prologue_gemm<T, false, 128>);
  if constexpr (sizeof(T) == 2) {
    // whole bf16 tiles, K a multiple of the stage: stages straight into LDS
    if (full && lds) kern = mt == 96 ? prologue_gemm_lds<96, 2> : prologue_gemm_lds<128, 2>;
  }
  tr->before(stream, name, B);
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, g);
  tr->after(stream);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_prologue_dt(const PrologueProblem& pr, hipStream_t stream, Tracer* tr) {
  const int N = static_cast<int>(pr.H * pr.W);
  const int C = static_cast<int>(pr.C), Cin = static_cast<int>(pr.Cin);
  T* x = static_cast<T*>(pr.x_out);
  hipError_t e = gemm<T>(static_cast<const T*>(pr.w_r), static_cast<const T*>(pr.b_r),
                         static_cast<const T*>(pr.x_in), &x, 1, pr.B, C, Cin, N,
                         "prologue_reduce", stream, tr);
  if (e != hipSuccess) return e;
  T* outs[5];
  for (int t = 0; t < 5; ++t) outs[t] = static_cast<T*>(pr.p_out[t]);
  return gemm<T>(static_cast<const T*>(pr.w_p), static_cast<const T*>(pr.b_p), x, outs, 5, pr.B,
                 5 * C, C, N, "prologue_params", stream, tr);
}
}  // namespace

hipError_t launch_prologue(const PrologueProblem& pr, hipStream_t stream, Tracer* tr) {
  if (pr.dtype == GSPN_F32) return launch_prologue_dt<float>(pr, stream, tr);
  return launch_prologue_dt<bf16_t>(pr, stream, tr);
}

namespace {
template <typename T>
hipError_t launch_reduce_dt(const PrologueProblem& pr, hipStream_t stream, Tracer* tr) {
  T* x = static_cast<T*>(pr.x_out);
  return gemm<T>(static_cast<const T*>(pr.w_r), static_cast<const T*>(pr.b_r),
                 static_cast<const T*>(pr.x_in), &x, 1, pr.B, static_cast<int>(pr.C),
                 static_cast<int>(pr.Cin), static_cast<int>(pr.H * pr.W), "prologue_reduce",
                 stream, tr);
}
}  // namespace

hipError_t launch_prologue_reduce(const PrologueProblem& pr, hipStream_t stream, Tracer* tr) {
  if (pr.dtype == GSPN_F32) return launch_reduce_dt<float>(pr, stream, tr);
  return launch_reduce_dt<bf16_t>(pr, stream, tr);
}

}  // namespace gspn

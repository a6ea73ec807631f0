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
// v_mfma_f32_16x16x4_f32 for fp32). K advances 32 at a time through LDS: the
// weight tile as [m][k] and the pixel tile transposed to [n][k], so every
// MFMA operand is a run of consecutive k. The finished tile is staged in LDS
// (64 rows at a time) and written as 16-byte row runs. The linear block index
// walks M fastest, so the M tiles that share a pixel tile run together and
// find it in L2.
#include "gspn_device.hpp"
#include "gspn_launch.hpp"

namespace gspn {

namespace {
constexpr int kMT = 128, kNT = 128, kKT = 32;
constexpr int kAP = kKT + 8;     // LDS pitch (elements) of the [m][k] and [n][k] tiles
constexpr int kOP = kNT + 8;     // LDS pitch of the staged output tile

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float g_ld(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float g_ld(const bf16_t* p, int64_t i) { return to_f32(p[i]); }

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
  int vec_a, vec_x, vec_o;   // 16-byte runs allowed for A rows, X rows, output rows
};

template <typename T>
__global__ __launch_bounds__(256) void prologue_gemm(GemmArgs<T> a) {
  using R = decltype(raw(T{}));   // uint16_t (bf16 bits) or float
  constexpr int E = 16 / sizeof(T);   // elements in 16 bytes
  constexpr int kTileBytes = 2 * kMT * kAP * sizeof(R);
  constexpr int kOutBytes = (kMT / 2) * kOP * sizeof(R);
  __shared__ __align__(16) unsigned char smem[kTileBytes > kOutBytes ? kTileBytes : kOutBytes];
  R* As = reinterpret_cast<R*>(smem);                 // [kMT][kAP]
  R* Bs = As + kMT * kAP;                             // [kNT][kAP], transposed pixel tile
  R* Os = reinterpret_cast<R*>(smem);                 // [kMT / 2][kOP], after the K loop

  const int M = a.M, K = a.K, N = a.N;
  const int nmt = (M + kMT - 1) / kMT;
  const int m0 = static_cast<int>(blockIdx.x % nmt) * kMT;
  const int n0 = static_cast<int>(blockIdx.x / nmt) * kNT;
  const int64_t b = blockIdx.y;
  const T* X = a.X + b * static_cast<int64_t>(K) * N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;   // this wavefront's quarter

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < K; k0 += kKT) {
    // weight tile [kMT][kKT]: kMT * kKT / E runs of E elements
#pragma unroll
    for (int c = tid; c < kMT * kKT / E; c += 256) {
      const int r = c / (kKT / E), kk = (c % (kKT / E)) * E;
      const int m = m0 + r, k = k0 + kk;
      R* dst = As + r * kAP + kk;
      if (a.vec_a && m < M && k + E <= K) {
        *reinterpret_cast<uint4*>(dst) =
            *reinterpret_cast<const uint4*>(a.A + static_cast<int64_t>(m) * K + k);
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e)
          dst[e] = (m < M && k + e < K) ? raw(a.A[static_cast<int64_t>(m) * K + k + e]) : R(0);
      }
    }
    // pixel tile [kKT][kNT] from X, stored transposed as [n][k]
#pragma unroll
    for (int c = tid; c < kKT * kNT / E; c += 256) {
      const int kr = c / (kNT / E), nn = (c % (kNT / E)) * E;
      const int k = k0 + kr, n = n0 + nn;
      R v[E];
      if (a.vec_x && k < K && n + E <= N) {
        const uint4 q = *reinterpret_cast<const uint4*>(X + static_cast<int64_t>(k) * N + n);
        *reinterpret_cast<uint4*>(v) = q;
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e)
          v[e] = (k < K && n + e < N) ? raw(X[static_cast<int64_t>(k) * N + n + e]) : R(0);
      }
#pragma unroll
      for (int e = 0; e < E; ++e) Bs[(nn + e) * kAP + kr] = v[e];
    }
    __syncthreads();
    if constexpr (sizeof(T) == 2) {
      // v_mfma_f32_16x16x32_bf16: lane l holds A[l % 16][8 (l / 16) .. +7]
      // and B[8 (l / 16) .. +7][l % 16]
      const int r = lane & 15, kq = (lane >> 4) * 8;
      bf16x8 fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[i] = *reinterpret_cast<const bf16x8*>(As + (wm + 16 * i + r) * kAP + kq);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        fb[j] = *reinterpret_cast<const bf16x8*>(Bs + (wn + 16 * j + r) * kAP + kq);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    } else {
      // v_mfma_f32_16x16x4_f32: lane l holds A[l % 16][l / 16] and
      // B[l / 16][l % 16]; eight of them cover K = 32
      const int r = lane & 15, kq = lane >> 4;
#pragma unroll
      for (int ks = 0; ks < kKT; ks += 4) {
        float fa[4], fb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[i] = As[(wm + 16 * i + r) * kAP + ks + kq];
#pragma unroll
        for (int j = 0; j < 4; ++j) fb[j] = Bs[(wn + 16 * j + r) * kAP + ks + kq];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[i], fb[j], acc[i][j], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // bias, rounding to the storage type, staging half a tile (64 rows, the
  // two wavefronts of one row half) at a time: lane l holds rows
  // 4 (l / 16) + e, column l % 16 of each 16 x 16 tile
  const int col = lane & 15, rq = (lane >> 4) * 4;
  for (int h = 0; h < 2; ++h) {
    if ((wave >> 1) == h) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 16 * i + rq + e;          // row within the half
          const int m = m0 + h * 64 + r;
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
    __syncthreads();
    // the half's rows to their output tensors, 16-byte runs
    for (int c = tid; c < 64 * kNT / E; c += 256) {
      const int r = c / (kNT / E), nn = (c % (kNT / E)) * E;
      const int m = m0 + h * 64 + r, n = n0 + nn;
      if (m >= M || n >= N) continue;
      const int t = m / a.Mt, mr = m - t * a.Mt;
      T* dst = a.out[t] + (b * a.Mt + mr) * static_cast<int64_t>(N);
      const R* src = Os + r * kOP + nn;
      if (a.vec_o && n + E <= N) {
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
    __syncthreads();
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
  constexpr int E = 16 / sizeof(T);
  g.vec_a = K % E == 0 && al16(A);
  g.vec_x = N % E == 0 && al16(X);
  bool vo = N % E == 0;
  for (int t = 0; t < nout; ++t) vo = vo && al16(outs[t]);
  g.vec_o = vo;
  const int64_t tiles = static_cast<int64_t>((M + kMT - 1) / kMT) * ((N + kNT - 1) / kNT);
  const dim3 grid(static_cast<unsigned>(tiles), static_cast<unsigned>(B));
  tr->before(stream, name, B);
  hipLaunchKernelGGL(prologue_gemm<T>, grid, dim3(256), 0, stream, g);
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

}  // namespace gspn

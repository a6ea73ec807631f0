// The GSPN unit's parameter product fused with the propagation, for small
// planes (H, W <= 16, bf16): the logits, lambda and u of a group of 16
// channels go from MFMA accumulators into LDS records and are scanned there,
// so the five parameter tensors never reach HBM.
//
// The unit (aitntnews page, section GSPN架构; CSDN page, section
// GSPN模块的设计, Fig. 3c) is a shared 1x1 convolution x = W_r X_in + b_r,
// three 1x1 convolutions producing the logits, lambda and u from x, and the
// four-direction propagation of x with them. In [B, C, H, W] layout a 1x1
// convolution of image b is a matrix product over channels with N = H W
// pixels as columns. The first product runs as before (x is needed in full by
// every channel group, so it is stored once); this kernel does the second
// and the propagation. One workgroup owns channels c0 .. c0 + 15 of image b:
//
//   1. product: the 80 rows of W_p that produce the group's l0, l1, l2,
//      lambda and u (rows t C + c0 + i, t = 0..4) times x[b] (C x N). Wave w
//      owns pixel tiles w, w + 4, w + 8, w + 12 (16 pixels each) for all 80
//      rows: 5 x 4 MFMA tiles of 16 x 16 (v_mfma_f32_16x16x32_bf16), K in
//      steps of 64 through LDS (the pixel operand by transposing reads of the
//      tile as loaded), the next step's operands in registers while the
//      current one is multiplied. Lane l then holds, for channels
//      4 (l / 16) + e of the group and pixel 16 tile + l % 16, all five
//      parameters, so a pixel's record needs no exchange between lanes;
//   2. records: bias added, each parameter rounded to bf16 (the unit's
//      parameters are tensors of the storage type, exactly as the unfused
//      path stores and rereads them), then (w0, w1, w2, lambda x) with the
//      sigmoid + row normalisation of the three logits; x of the group's
//      channels is taken from the product's own LDS tile;
//   3. scans: wave w scans planes 4w .. 4w + 3 (one per 16-lane row,
//      neighbours by DPP row shifts) in each selected direction, edge lanes
//      renormalising over their in-range neighbours;
//   4. merge: out = u (h_T2B + h_B2T + h_L2R + h_R2L) in that order, one
//      rounding, the group's 16 output planes written as one contiguous run.
//
// Line recurrence and output gate: CSDN page, section 方法; tridiagonal
// row-normalised sigmoid weights, four directions: section
// 如何设计一个高效的传播层; local groups: section GSPN模块的设计.
#include "gspn_device.hpp"
#include "gspn_launch.hpp"
#include "gspn_mfma.hpp"

namespace gspn {

namespace {

constexpr int kCg = 16;            // channels per workgroup
constexpr int kIB = 4;             // images per block of the tile order
constexpr int kMR = 5 * kCg;       // rows of W_p per workgroup
constexpr int kKT = 32;            // K per stage: 64-byte rows of the weight tile
constexpr int kStages = 3;         // stages in flight: loads run two stages ahead
constexpr int kNmax = 256;         // pixels of one image
constexpr int kRP = 17;            // records per plane row (odd: no bank conflicts
                                   // on horizontal scans)
constexpr int kABytes = kMR * kKT * 2;              // weight tile [80][32], 5 blocks of 1 KB
constexpr int kStageBytes = kABytes + kKT * kNmax * 2;   // + pixel tile [32][256], 16 blocks
constexpr int kRecBytes = kCg * (16 * kRP + 1) * 16;
constexpr int kOutOff = kRecBytes;                  // output staging [16][N] bf16
constexpr int kZeroOff = kRecBytes + kCg * kNmax * 2;
constexpr int kLdsBytes = kZeroOff + 16;
static_assert(kStages * kStageBytes <= kRecBytes, "the product's stages live in the record area");

struct FusedArgs {
  const bf16_t* wp;    // [5C][C]
  const bf16_t* bp;    // [5C] or null
  const bf16_t* x;     // [B][C][N], as the first product stored it
  bf16_t* out;         // [B][C][N]
  int B, C, H, W, N, G;
  unsigned mask;
  int tiles, per;      // (image, channel group) tiles; tiles per XCD
};

// The pixel tile sits in LDS as [k][256] with its 32-byte blocks (16
// pixels) swizzled per row: block b of row k is stored at block b ^ bswz(k).
// The transposing reads of an MFMA operand take 4 consecutive rows from each
// 16-lane group (rows k0 + 8 g + i, i < 4, for the four groups g), and the
// swizzle puts rows i and 8 + i in different banks, where an unswizzled
// 512-byte row would put all of them in the same ones.
__device__ __forceinline__ int bswz(int k) { return (k & 3) | ((k >> 1) & 4); }
__device__ __forceinline__ int bpos(int k, int n) {
  return k * kNmax + ((((n >> 4) ^ bswz(k)) << 4) | (n & 15));
}

// HS, WS > 0: the plane's sides fixed at compile time (the 16 x 16 latents),
// so pixel indices split by constants and the scans unroll to their length.
// (A variant without local groups runs out of registers.)
template <int HS, int WS>
__global__ __launch_bounds__(256, 2) void fused_unit(FusedArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  float4* recs = reinterpret_cast<float4*>(smem);
  float* recf = reinterpret_cast<float*>(smem);
  uint16_t* ost = reinterpret_cast<uint16_t*>(smem + kOutOff);

  // Workgroups are dealt to the 8 XCDs in turn; tile t runs on XCD t / per.
  // Tiles are ordered by blocks of kIB images, channel group, then image, so
  // the workgroups one XCD runs at once (about 64) are some 16 channel
  // groups of 4 images: each weight slice is shared by 4 of them and each
  // image's x by 16, and the K step they all read meets in that L2.
  const int tile = static_cast<int>(blockIdx.x % 8) * a.per + static_cast<int>(blockIdx.x / 8);
  if (tile >= a.tiles) return;
  const int C = a.C, H = HS > 0 ? HS : a.H, W = WS > 0 ? WS : a.W, N = HS > 0 ? HS * WS : a.N;
  const int ps = H * kRP + 1;
  const int ng = C / kCg;
  const int blk = tile / (kIB * ng);
  const int ibe = min(kIB, a.B - blk * kIB);
  const int rem = tile - blk * kIB * ng;
  const int64_t b = blk * kIB + rem % ibe;
  const int c0 = (rem / ibe) * kCg;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: LDS bases in SGPRs
  const int r16 = lane & 15, rq = (lane >> 4) * 4;
  const bf16_t* X = a.x + b * static_cast<int64_t>(C) * N;

  // the bias of the group's rows, loaded now so that the product hides it
  // (without a bias, the weights stand in as a valid address, unused)
  const bf16_t* bsrc = a.bp ? a.bp : a.wp;
  bf16_t braw[5][4];
#pragma unroll
  for (int t = 0; t < 5; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) braw[t][e] = bsrc[t * C + c0 + rq + e];

  // ---- 1. the product -------------------------------------------------------
  f32x4 acc[5][4];
#pragma unroll
  for (int t = 0; t < 5; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Stages of K = 32 go from global memory straight into LDS
  // (global_load_lds_dwordx4: each instruction writes 64 lanes x 16 bytes
  // as one contiguous 1 KB block, lane i at 16 i), three stages in a ring,
  // loads two stages ahead of the multiply. The block layouts are fixed by
  // choosing each lane's source:
  //   weight block t (rows 16 t .. 16 t + 15 of the 80, 64 bytes each): lane
  //     i fills row r = i / 4, slot i % 4 with the row's 16-byte unit
  //     (i % 4) ^ sw(r), sw(r) = ((r >> 1) ^ (r >> 2)) & 3, so that the
  //     fragment reads (16 rows, one unit each) hit distinct banks;
  //   pixel block j (k rows 2 j, 2 j + 1, 256 pixels each): lane i fills
  //     row 2 j + i / 32 at pixels 8 (i % 32) .. + 7 of the stored order,
  //     which holds the swizzled 16-pixel blocks of bpos.
  // Wave w loads pixel blocks 4 w .. 4 w + 3 and weight block w, wave 0
  // weight block 4 as well: 5 or 6 loads per stage.
  auto sw = [](int r) { return ((r >> 1) ^ (r >> 2)) & 3; };
  const int64_t a_row = (static_cast<int64_t>(wave) * C + c0 + (lane >> 2)) * C;
  const int64_t a_row4 = (static_cast<int64_t>(4) * C + c0 + (lane >> 2)) * C;
  const int a_unit = 8 * ((lane & 3) ^ sw(lane >> 2));
  const bf16_t* a_src = a.wp + a_row + a_unit;     // weight block `wave`
  const bf16_t* a_src4 = a.wp + a_row4 + a_unit;   // weight block 4 (wave 0)
  // (pixels past N, when N < 256, load pixel 0 again: every lane loads, so
  // every wave issues the same number of loads per stage)
  const bf16_t* b_src[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int blk = 4 * wave + q;
    const int row = 2 * blk + (lane >> 5), pos = 8 * (lane & 31);
    const int n = (((pos >> 4) ^ bswz(row)) << 4) | (pos & 15);
    b_src[q] = X + static_cast<int64_t>(row) * N + (n < N ? n : 0);
  }
  auto issue = [&](int st) {
    unsigned char* base = smem + (st % kStages) * kStageBytes;
    const int k0 = st * kKT;
    __builtin_amdgcn_global_load_lds(a_src + k0, base + wave * 1024, 16, 0, 0);
    if (wave == 0) __builtin_amdgcn_global_load_lds(a_src4 + k0, base + 4 * 1024, 16, 0, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_amdgcn_global_load_lds(b_src[q] + static_cast<int64_t>(k0) * N,
                                       base + kABytes + (4 * wave + q) * 1024, 16, 0, 0);
  };
  // LDS byte addresses of this lane's transposing reads in stage 0 (row
  // 8 (l / 16) + (l % 16) / 4, pixels 16 (4 j + w) + 4 (l % 4) ..; the
  // second half, rows + 4, is 2 KB further: rows k + 4 share k's swizzle)
  const uint32_t lds_base = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) unsigned char*)smem));
  uint32_t tr_addr[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 8 * (lane >> 4) + (r16 >> 2);
    tr_addr[j] = lds_base + kABytes + 2 * bpos(row, 16 * (4 * j + wave) + 4 * (r16 & 3));
  }
  auto multiply = [&](int st) {
    const unsigned char* base = smem + (st % kStages) * kStageBytes;
    // lane l: A[l % 16][8 (l / 16) .. +7] of each M tile, unit l / 16 stored
    // at slot (l / 16) ^ sw(l % 16) of its row
    const int g = lane >> 4;
    bf16x8 fa[5], fb[4];
#pragma unroll
    for (int t = 0; t < 5; ++t)
      fa[t] = *reinterpret_cast<const bf16x8*>(base + t * 1024 + r16 * 64 + 16 * (g ^ sw(r16)));
    // B by transposing reads (rows + 4 are 2 KB further)
    const uint32_t so = static_cast<uint32_t>((st % kStages) * kStageBytes);
    const uint32_t q[4] = {tr_addr[0] + so, tr_addr[1] + so, tr_addr[2] + so, tr_addr[3] + so};
    lds_read_tr_b4<2048>(q, fb);
#pragma unroll
    for (int t = 0; t < 5; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[t], fb[j], acc[t][j], 0, 0, 0);
  };

  // x of the group's channels, for lambda x: rows c0 - kx0 .. of the pixel
  // tile of the stage at kx0, taken while it is in LDS
  const int kx0 = c0 & ~(kKT - 1);
  uint16_t xv[4][4];
  const int S = C / kKT;
  issue(0);
  if (S > 1) issue(1);
  for (int st = 0; st < S; ++st) {
    // this wave's loads of stage st are done when at most the next stage's
    // are in flight (vector memory loads complete in order)
    if (st + 1 < S) {
      if (wave == 0) wait_vmcnt<6>();
      else           wait_vmcnt<5>();
    } else {
      wait_vmcnt<0>();
    }
    bare_barrier();   // ... and every wave's; stage st - 1 is no longer read
    if (st + 2 < S) issue(st + 2);
    multiply(st);
    if (st * kKT == kx0) {
      const uint16_t* Bst = reinterpret_cast<const uint16_t*>(smem + (st % kStages) * kStageBytes +
                                                              kABytes);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          xv[e][j] = Bst[bpos(c0 - kx0 + rq + e, 16 * (4 * j + wave) + r16)];
    }
  }
  lds_barrier();   // the records overwrite the stages

  // ---- 2. records -------------------------------------------------------------
  // plane p's records start at p ps: one spare record per plane moves each
  // plane's LDS banks by four, so the lanes of different planes that read
  // or write the same pixel together do not collide
  float bias[5][4];
#pragma unroll
  for (int t = 0; t < 5; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      bias[t][e] = a.bp ? to_f32(braw[t][e]) : 0.0f;
  float uu[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = 16 * (4 * j + wave) + r16;
    const int row = n / W, col = n - row * W;
    // the parameters as the unfused path stores them: rounded to bf16
    float pr[5][4];
#pragma unroll
    for (int t = 0; t < 5; ++t)
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        pr[t][e] = acc[t][j][e] + bias[t][e];
        pr[t][e + 1] = acc[t][j][e + 1] + bias[t][e + 1];
        round_bf16x2(pr[t][e], pr[t][e + 1]);
      }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float l0 = pr[0][e], l1 = pr[1][e], l2 = pr[2][e], lam = pr[3][e];
      uu[e][j] = pr[4][e];
      if (n < N) {
        const Weights w = make_weights(l0, l1, l2, 1.0f, 1.0f);
        const float xx = __uint_as_float(static_cast<uint32_t>(xv[e][j]) << 16);
        recs[(rq + e) * ps + row * kRP + col] = make_float4(w.w0, w.w1, w.w2, lam * xx);
      }
    }
  }
  if (tid == 0) recs[kZeroOff / 16] = make_float4(0.f, 0.f, 0.f, 0.f);
  lds_barrier();

  // ---- 3. scans: wave w owns planes 4w .. 4w + 3 ------------------------------
  const int pl = 4 * wave + (lane >> 4), o = r16;
  const int G = a.G;
  float hist[4][16];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    if (!((a.mask >> d) & 1u)) continue;
    const bool vert = d < 2, fwd = (d == 0 || d == 2);
    const int n_s = vert ? H : W, n_o = vert ? W : H;
    const bool active = o < n_o;
    const float m0 = o > 0 ? 1.f : 0.f, m2 = o < n_o - 1 ? 1.f : 0.f;
    const bool edge = active && (o == 0 || o == n_o - 1);
    const int p0 = fwd ? 0 : n_s - 1;
    int addr = vert ? pl * ps + p0 * kRP + o : pl * ps + o * kRP + p0;
    int stride = (vert ? kRP : 1) * (fwd ? 1 : -1);
    if (!active) { addr = kZeroOff / 16; stride = 0; }
    int next_restart = n_s;
    if (G > 0) next_restart = fwd ? G : n_s - ((n_s - 1) / G) * G;
    float h = 0.0f;
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      if (s < n_s) {
        float4 rc = recs[addr];
        addr += stride;
        if (edge) {
          const Weights we = edge_weights(rc.x, rc.y, rc.z, m0, m2);
          rc.x = we.w0; rc.y = we.w1; rc.z = we.w2;
        }
        const float hn = line_step<16>(h, rc.x, rc.y, rc.z, rc.w);
        bool restart = (s == 0);
        if (s == next_restart) { restart = true; next_restart += G; }
        h = restart ? rc.w : hn;
        hist[d][s] = h;
      }
    }
  }
  // park each direction's states in its slot of the records of this wave's
  // own planes (no other wave reads them)
  lds_wave_sync();
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    if (!((a.mask >> d) & 1u)) continue;
    const bool vert = d < 2, fwd = (d == 0 || d == 2);
    const int n_s = vert ? H : W, n_o = vert ? W : H;
    if (o >= n_o) continue;
    const int p0 = fwd ? 0 : n_s - 1;
    int addr = vert ? pl * ps + p0 * kRP + o : pl * ps + o * kRP + p0;
    const int stride = (vert ? kRP : 1) * (fwd ? 1 : -1);
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      if (s < n_s) {
        recf[4 * addr + d] = hist[d][s];
        addr += stride;
      }
    }
  }
  lds_barrier();

  // ---- 4. merge and store -------------------------------------------------------
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = 16 * (4 * j + wave) + r16;
    if (n >= N) continue;
    const int row = n / W, col = n - row * W;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float4 st = recs[(rq + e) * ps + row * kRP + col];
      float sum = 0.0f;
      if (a.mask & 1u) sum += st.x;
      if (a.mask & 2u) sum += st.y;
      if (a.mask & 4u) sum += st.z;
      if (a.mask & 8u) sum += st.w;
      ost[(rq + e) * N + n] = static_cast<uint16_t>(f32_to_bf16_bits(uu[e][j] * sum));
    }
  }
  lds_barrier();
  // the group's planes are one contiguous run of 16 N elements
  uint4* dst = reinterpret_cast<uint4*>(a.out + (b * C + c0) * static_cast<int64_t>(N));
  const uint4* src = reinterpret_cast<const uint4*>(ost);
  for (int c = tid; c < 2 * N; c += 256) dst[c] = src[c];
}

bool al16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

}  // namespace

bool fused_unit_fits(const PrologueProblem& pr) {
  return pr.dtype == GSPN_BF16 && pr.H >= 1 && pr.W >= 1 && pr.H <= 16 && pr.W <= 16 &&
         (pr.H * pr.W) % 8 == 0 && pr.C % 64 == 0 && pr.C >= 64 && pr.C <= 20000 &&
         al16(pr.w_p);
}

hipError_t launch_fused_unit(const PrologueProblem& pr, const void* x, void* out, uint32_t mask,
                             int64_t G, hipStream_t stream, Tracer* tr) {
  FusedArgs a;
  a.wp = static_cast<const bf16_t*>(pr.w_p);
  a.bp = static_cast<const bf16_t*>(pr.b_p);
  a.x = static_cast<const bf16_t*>(x);
  a.out = static_cast<bf16_t*>(out);
  a.B = static_cast<int>(pr.B);
  a.C = static_cast<int>(pr.C);
  a.H = static_cast<int>(pr.H);
  a.W = static_cast<int>(pr.W);
  a.N = static_cast<int>(pr.H * pr.W);
  a.G = static_cast<int>(G >= pr.H && G >= pr.W ? 0 : G);
  a.mask = mask;
  const int64_t tiles = pr.B * (pr.C / kCg);
  a.tiles = static_cast<int>(tiles);
  a.per = static_cast<int>((tiles + 7) / 8);
  auto kern = (a.H == 16 && a.W == 16) ? fused_unit<16, 16> : fused_unit<0, 0>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  if (e != hipSuccess) return e;
  tr->before(stream, "fused_unit", pr.B * pr.C);
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(a.per * 8)), dim3(256), kLdsBytes, stream,
                     a);
  tr->after(stream);
  return hipGetLastError();
}

}  // namespace gspn

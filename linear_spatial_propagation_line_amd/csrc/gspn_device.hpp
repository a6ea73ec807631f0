// Device helpers shared by the gfx950 GSPN kernels: storage decode/encode,
// the fused sigmoid + row normalisation of the three neighbour logits, and
// cross-lane neighbour exchange.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gspn {

// ---------------------------------------------------------------------------
// storage types
// ---------------------------------------------------------------------------
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) {
  return __uint_as_float(static_cast<uint32_t>(v.bits) << 16);
}
// bf16 is the upper half of binary32: widening is exact
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }

// binary32 -> bf16, round to nearest, ties to even (NaN stays a NaN), by
// gfx950's packed conversion, one instruction per pair: `a` in the low half
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return pack_bf16x2(f, 0.0f) & 0xffffu;
}
// two values replaced by their nearest bf16 values, kept as binary32
__device__ __forceinline__ void round_bf16x2(float& a, float& b) {
  const uint32_t p = pack_bf16x2(a, b);
  a = __uint_as_float(p << 16);
  b = __uint_as_float(p & 0xffff0000u);
}

template <typename T> struct Store;
template <> struct Store<float> {
  __device__ static __forceinline__ void put(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Store<bf16_t> {
  __device__ static __forceinline__ void put(bf16_t* p, int64_t i, float v) {
    p[i].bits = static_cast<uint16_t>(f32_to_bf16_bits(v));
  }
};

// four consecutive elements, kept in their storage form until used
template <typename T> struct V4;
template <> struct V4<float> {
  using raw = float4;
  __device__ static raw load(const float* p, int64_t i) {
    return *reinterpret_cast<const float4*>(p + i);
  }
  __device__ static float get(const raw& v, int e) {
    return e == 0 ? v.x : (e == 1 ? v.y : (e == 2 ? v.z : v.w));
  }
  __device__ static void store(float* p, int64_t i, const float v[4]) {
    *reinterpret_cast<float4*>(p + i) = make_float4(v[0], v[1], v[2], v[3]);
  }
};
template <> struct V4<bf16_t> {
  using raw = uint2;
  __device__ static raw load(const bf16_t* p, int64_t i) {
    return *reinterpret_cast<const uint2*>(p + i);
  }
  __device__ static float get(const raw& v, int e) {
    const uint32_t w = e < 2 ? v.x : v.y;
    return (e & 1) ? bf16_hi(w) : bf16_lo(w);
  }
  __device__ static void store(bf16_t* p, int64_t i, const float v[4]) {
    uint2 q;
    q.x = pack_bf16x2(v[0], v[1]);
    q.y = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<uint2*>(p + i) = q;
  }
};

// N contiguous elements at a 16-byte aligned index, widened to fp32 ...
template <int N> __device__ __forceinline__ void run_ld(const float* p, int64_t i, float* d) {
  const float4* q = reinterpret_cast<const float4*>(p + i);
#pragma unroll
  for (int k = 0; k < N / 4; ++k) {
    const float4 v = q[k];
    d[4 * k] = v.x; d[4 * k + 1] = v.y; d[4 * k + 2] = v.z; d[4 * k + 3] = v.w;
  }
}
template <int N> __device__ __forceinline__ void run_ld(const bf16_t* p, int64_t i, float* d) {
  const uint4* q = reinterpret_cast<const uint4*>(p + i);
#pragma unroll
  for (int k = 0; k < N / 8; ++k) {
    const uint4 v = q[k];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) { d[8 * k + 2 * j] = bf16_lo(w[j]); d[8 * k + 2 * j + 1] = bf16_hi(w[j]); }
  }
}
// ... and stored back the same way (bf16 rounded to nearest even)
template <int N> __device__ __forceinline__ void run_st(float* p, int64_t i, const float* d) {
  float4* q = reinterpret_cast<float4*>(p + i);
#pragma unroll
  for (int k = 0; k < N / 4; ++k) q[k] = make_float4(d[4 * k], d[4 * k + 1], d[4 * k + 2], d[4 * k + 3]);
}
template <int N> __device__ __forceinline__ void run_st(bf16_t* p, int64_t i, const float* d) {
  uint4* q = reinterpret_cast<uint4*>(p + i);
#pragma unroll
  for (int k = 0; k < N / 8; ++k) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = pack_bf16x2(d[8 * k + 2 * j], d[8 * k + 2 * j + 1]);
    q[k] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// ---------------------------------------------------------------------------
// weights of one pixel
// ---------------------------------------------------------------------------
// With a_k = 1 + exp(-l_k) (so sigmoid(l_k) = 1 / a_k), the normalised
// weights are
//     w_0 = a_1 a_2 / D,  w_1 = a_0 a_2 / D,  w_2 = a_0 a_1 / D,
//     D   = a_1 a_2 + a_0 a_2 + a_0 a_1,
// which needs three exponentials and one reciprocal per pixel instead of
// three reciprocals more. Out-of-range neighbours get mask m = 0 (their
// product term is dropped from both numerator and D). The centre neighbour
// always exists. Logits are clamped below at -40 (sigmoid < 4.3e-18) so the
// products stay finite in fp32; +inf gives a = 1 exactly.
struct Weights {
  float w0, w1, w2;
};

// exp(-max(l, -40)), as exp2 of -l log2(e) capped at the exponent of -40.
// The cap is applied after the multiply: rounding is monotonic, so the cap
// gives the same bits as clamping l first, NaN and -inf included (both go
// to the cap), and a cap on a product needs no NaN quieting of its input,
// where a clamp of the raw logit costs one more instruction.
__device__ __forceinline__ float exp_neg(float l) {
  constexpr float kNegLog2e = -1.4426950408889634f;
  constexpr float kCap = -40.0f * kNegLog2e;
  return __builtin_amdgcn_exp2f(fminf(l * kNegLog2e, kCap));
}

// Reciprocal: hardware estimate refined by one Newton-Raphson step
// (r' = r + r (1 - d r)), which brings it to about half an ulp.
__device__ __forceinline__ float recip(float d) {
  float r = __builtin_amdgcn_rcpf(d);
  float e = __builtin_fmaf(-d, r, 1.0f);
  return __builtin_fmaf(r, e, r);
}

__device__ __forceinline__ Weights make_weights(float l0, float l1, float l2,
                                                float m0, float m2) {
  const float a0 = 1.0f + exp_neg(l0);
  const float a1 = 1.0f + exp_neg(l1);
  const float a2 = 1.0f + exp_neg(l2);
  const float p12 = (m0 * a1) * a2;
  const float p02 = a0 * a2;
  const float p01 = (m2 * a0) * a1;
  const float r = recip(p12 + p02 + p01);
  return Weights{p12 * r, p02 * r, p01 * r};
}

// Weights and their sigmoid slopes for the backward pass: q_k = w_k (1 -
// sigmoid(l_k)), with 1 - sigmoid(l) = exp(-l) / (1 + exp(-l)) taken from the
// same exponentials (no cancellation as sigmoid -> 1). Out-of-range links
// have w_k = q_k = 0.
struct WeightSlopes {
  float w0, w1, w2, q0, q1, q2;
};

__device__ __forceinline__ WeightSlopes make_weight_slopes(float l0, float l1, float l2,
                                                           float m0, float m2) {
  const float e0 = exp_neg(l0), e1 = exp_neg(l1), e2 = exp_neg(l2);
  const float a0 = 1.0f + e0, a1 = 1.0f + e1, a2 = 1.0f + e2;
  const float p12 = (m0 * a1) * a2;
  const float p02 = a0 * a2;
  const float p01 = (m2 * a0) * a1;
  const float r = recip(p12 + p02 + p01);
  WeightSlopes q;
  q.w0 = p12 * r;
  q.w1 = p02 * r;
  q.w2 = p01 * r;
  q.q0 = q.w0 * (e0 * recip(a0));
  q.q1 = q.w1 * (e1 * recip(a1));
  q.q2 = q.w2 * (e2 * recip(a2));
  return q;
}

// Renormalise already normalised interior weights for an edge pixel whose
// side neighbours may be missing: w_k' = m_k w_k / sum_j m_j w_j.
__device__ __forceinline__ Weights edge_weights(float w0, float w1, float w2,
                                                float m0, float m2) {
  const float v0 = m0 * w0, v2 = m2 * w2;
  const float r = recip(v0 + w1 + v2);
  return Weights{v0 * r, w1 * r, v2 * r};
}

// ---------------------------------------------------------------------------
// cross-lane neighbour values (DPP); lanes with no source read 0
// ---------------------------------------------------------------------------
// SEG = 64: the orthogonal axis spans the whole wave (wave_shr:1 / wave_shl:1).
// SEG = 16: four independent 16-lane segments (row_shr:1 / row_shl:1).
template <int SEG> __device__ __forceinline__ float from_left(float v);
template <int SEG> __device__ __forceinline__ float from_right(float v);

template <> __device__ __forceinline__ float from_left<64>(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x138, 0xf, 0xf, true));
}
template <> __device__ __forceinline__ float from_right<64>(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x130, 0xf, 0xf, true));
}
template <> __device__ __forceinline__ float from_left<16>(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xf, 0xf, true));
}
template <> __device__ __forceinline__ float from_right<16>(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x101, 0xf, 0xf, true));
}

// One step of the line recurrence, lx + w1 h[o] + w2 h[o+1] + w0 h[o-1] (in
// that order), the neighbours' states taken from the adjacent lanes. The
// lane's own term comes first: it needs no cross-lane move, so it overlaps
// the two DPP moves instead of waiting behind them.
template <int SEG>
__device__ __forceinline__ float line_step(float h, float w0, float w1, float w2, float lx) {
  float acc = __builtin_fmaf(w1, h, lx);
  acc = __builtin_fmaf(from_right<SEG>(h), w2, acc);
  return __builtin_fmaf(from_left<SEG>(h), w0, acc);
}

// ---------------------------------------------------------------------------
// channel-shared logits: plane p = (b, c) of a [B, C] batch reads logit
// channel c / (C / Cl) of batch entry b. Returns how many elements the
// plane's logits sit after (or before) its own offset: add it to a pixel
// index of the plane to get the pixel's logit index. 0 when Cl == C.
// ---------------------------------------------------------------------------
__host__ __device__ __forceinline__ int64_t logit_shift(int64_t p, int64_t C, int64_t Cl,
                                                        int64_t HW) {
  if (Cl == C) return 0;
  const int64_t b = p / C, c = p - b * C;
  return (b * Cl + c / (C / Cl) - p) * HW;
}

// ---------------------------------------------------------------------------
// small exact integer division for n < 2^24 (plane-local pixel indices)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int div_small(int n, int d, float inv_d, int* rem) {
  int q = static_cast<int>(static_cast<float>(n) * inv_d);
  int r = n - q * d;
  if (r < 0) { q -= 1; r += d; }
  if (r >= d) { q += 1; r -= d; }
  *rem = r;
  return q;
}

}  // namespace gspn

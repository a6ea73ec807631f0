// Column-quad copies of a plane for the large-plane pipelines: the layout
// [plane][ceil(W / 4)][Hp][4] keeps four columns per row and rows
// contiguous, so a 128-byte line holds 8 rows of four fp32 values or 16 rows
// of four bf16 values. The two lanes that own a quad's column pairs swap half
// of their buffered rows (one DPP move per value) and then each writes 64
// contiguous bytes: a whole line in the same stores. Readers take two rows
// of a quad at a time.
#pragma once

#include "gspn_device.hpp"

namespace gspn {

// the value held by the other lane of an adjacent lane pair (2i, 2i + 1)
__device__ __forceinline__ uint32_t pair_swap(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_mov_dpp(static_cast<int>(v), 0xB1 /* quad_perm [1,0,3,2] */, 0xf, 0xf, false));
}
__device__ __forceinline__ float pair_swap(float v) {
  return __uint_as_float(pair_swap(__float_as_uint(v)));
}
__device__ __forceinline__ float2 pair_swap(float2 v) {
  return make_float2(pair_swap(v.x), pair_swap(v.y));
}
// rows k of the even lane and k + n / 2 of the odd lane, both as the quad's
// four values: the even lane's pair first
template <typename R>
__device__ __forceinline__ void quad_rows(const R* buf, int n, int k, bool odd, R* lo, R* hi) {
  const R keep = odd ? buf[k + n / 2] : buf[k];
  const R got = pair_swap(odd ? buf[k] : buf[k + n / 2]);
  *lo = odd ? got : keep;
  *hi = odd ? keep : got;
}
// rows o, o + 1 of a column quad of the copy: 4 values per row
template <typename T> struct Quad;
template <> struct Quad<float> {
  struct raw {
    float4 r0, r1;
  };
  __device__ static raw load(const float* p, int64_t i) {
    const float4* q = reinterpret_cast<const float4*>(p + i);
    return raw{q[0], q[1]};
  }
  // column c (0..3) of the quad for the two rows
  __device__ static void col(const raw& v, int c, float out[2]) {
    out[0] = c == 0 ? v.r0.x : (c == 1 ? v.r0.y : (c == 2 ? v.r0.z : v.r0.w));
    out[1] = c == 0 ? v.r1.x : (c == 1 ? v.r1.y : (c == 2 ? v.r1.z : v.r1.w));
  }
};
template <> struct Quad<bf16_t> {
  using raw = uint4;   // row o: x (columns 0, 1), y (2, 3); row o + 1: z, w
  __device__ static raw load(const bf16_t* p, int64_t i) {
    return *reinterpret_cast<const uint4*>(p + i);
  }
  __device__ static void col(const raw& v, int c, float out[2]) {
    const uint32_t a = c < 2 ? v.x : v.y, b = c < 2 ? v.z : v.w;
    out[0] = (c & 1) ? bf16_hi(a) : bf16_lo(a);
    out[1] = (c & 1) ? bf16_hi(b) : bf16_lo(b);
  }
};

}  // namespace gspn

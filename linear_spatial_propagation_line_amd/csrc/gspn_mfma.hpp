// MFMA operand types and LDS helpers shared by the kernels that multiply on
// matrix cores (the module prologue and the fused parameter product + scan).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gspn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// 16 bytes as a plain vector of four words (arrays of these stay in
// registers; arrays of the uint4 struct copied whole may not)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Barriers that order LDS only. A plain __syncthreads() also fences global
// memory, which on this GPU waits for every outstanding global load and
// store: prefetched operands and output runs just written would be drained
// at each barrier. These wait for LDS traffic alone.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// the same within one wavefront (its lanes read what its other lanes wrote)
__device__ __forceinline__ void lds_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// gfx950 transposing LDS read of 16-bit data: within each group of 16 lanes
// the lanes' 8-byte chunks, taken in lane order, form a run of 64 elements,
// and lane j receives elements j, j + 16, j + 32, j + 48 of it. When lane c
// of a group points at row r0 + c / 4, columns n0 + 4 (c % 4) of a [k][n]
// tile, lane j therefore gets rows r0 .. r0 + 3 of column n0 + j: four
// consecutive k of one n, half of an MFMA B operand (checked on the GPU with
// a one-wavefront probe).
__device__ __forceinline__ v4i16 lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
}

// The B operand of v_mfma_f32_16x16x32_bf16 (lane l: 8 consecutive k,
// 8 (l / 16) .. +7, of column l % 16) from a bf16 [k][n] tile with row pitch
// `pitch` elements: `p` points at row k0, column n0 of the 32 x 16 block.
__device__ __forceinline__ bf16x8 mfma_b_from_kn(const uint16_t* p, int pitch, int lane) {
  const int r = lane & 15, kq = (lane >> 4) * 8;
  const uint16_t* q = p + (kq + (r >> 2)) * pitch + 4 * (r & 3);
  const v4i16 lo = lds_read_tr(q), hi = lds_read_tr(q + 4 * pitch);
  return __builtin_bit_cast(bf16x8, v8i16{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w});
}

}  // namespace gspn

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

// For K loops that load their stages straight into LDS
// (global_load_lds_dwordx4). Those loads count in the vector memory counter
// and write LDS, so a fenced barrier would wait for every stage in flight;
// instead each wavefront waits for its own loads of the stage it needs, then
// all meet at a bare barrier.
//
// Wait until at most n of this wavefront's vector memory operations are
// outstanding, leaving the other counters alone (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// the same for a count known at run time among those the loops use
__device__ __forceinline__ void wait_vmcnt_of(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 12: wait_vmcnt<12>(); break;
    default: wait_vmcnt<0>(); break;   // any other count: wait for all
  }
}
// A workgroup barrier that orders no memory by itself; the empty asm keeps
// the compiler from moving LDS accesses across it.
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
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

// Four B operands of v_mfma_f32_16x16x32_bf16 by eight transposing reads:
// lane addresses q[j] (LDS byte addresses) for the first four k rows and
// q[j] + HALF for the next four. Written as one asm block with its own wait,
// because before the builtin form the compiler waits for every load into
// LDS in flight (the stages ahead of a direct-to-LDS K loop included).
template <int HALF>
__device__ __forceinline__ void lds_read_tr_b4(const uint32_t (&q)[4], bf16x8 (&b)[4]) {
  v4i16 t[8];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:%c12\n\t"
      "ds_read_b64_tr_b16 %2, %9\n\t"
      "ds_read_b64_tr_b16 %3, %9 offset:%c12\n\t"
      "ds_read_b64_tr_b16 %4, %10\n\t"
      "ds_read_b64_tr_b16 %5, %10 offset:%c12\n\t"
      "ds_read_b64_tr_b16 %6, %11\n\t"
      "ds_read_b64_tr_b16 %7, %11 offset:%c12\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(t[0]), "=&v"(t[1]), "=&v"(t[2]), "=&v"(t[3]), "=&v"(t[4]), "=&v"(t[5]),
        "=&v"(t[6]), "=&v"(t[7])
      : "v"(q[0]), "v"(q[1]), "v"(q[2]), "v"(q[3]), "i"(HALF)
      : "memory");
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const v4i16 lo = t[2 * j], hi = t[2 * j + 1];
    b[j] = __builtin_bit_cast(bf16x8, v8i16{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w});
  }
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

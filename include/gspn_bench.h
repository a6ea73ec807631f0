/*
 * Measurement kernels that ship with the GSPN library: plain HBM streams that
 * give the bandwidth ceiling the propagation is compared with. They compute
 * nothing of the propagation.
 */
#ifndef GSPN_BENCH_H
#define GSPN_BENCH_H

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * gspn_bench_stream -- enqueue one pass over `bytes` bytes on `stream`:
 *   kind 0  read `src` (16-byte loads); `dst` receives at most 1 KiB of
 *           noise that keeps the loads live;
 *   kind 1  write `dst` (16-byte stores of zero);
 *   kind 2  copy `src` to `dst`.
 * nontemporal != 0 marks every access non-temporal (a streaming hint to the
 * caches). The grid has blocks_per_cu (1..64) workgroups of 256 threads per
 * compute unit and walks the buffer grid-stride, four 16-byte accesses in
 * flight per thread. Pointers are caller-owned device memory, 16-byte aligned, and must
 * not overlap; bytes is a positive multiple of 16. Returns 0 when enqueued, 1
 * for a bad argument (nothing enqueued), 2 for a HIP error.
 */
int gspn_bench_stream(int kind, int nontemporal, const void* src, void* dst, size_t bytes,
                      int blocks_per_cu, hipStream_t stream);

/*
 * gspn_bench_handshake -- enqueue a kernel in which workgroup 0 and workgroup
 * `partner` (1..4095; the grid has partner + 1 workgroups, the others exit at
 * once) pass a counter back and forth `rounds` times through two flags in
 * device memory: a release store by one, acquire loads by the other until it
 * sees the value. This is the latency a schedule pays each time it hands a
 * scan line's state from one workgroup to another.
 *   flags       device memory, 512 bytes, 256-byte aligned, zeroed by the
 *               caller before the launch;
 *   abort_flag  host-visible memory (hipHostMalloc); setting it non-zero ends
 *               every wait;
 *   spin_max    polls after which a wait gives up (so the kernel always
 *               exits, whether or not the two workgroups run at once);
 *   out         device memory, 4 uint64: workgroup 0's elapsed wall-clock
 *               ticks (hipDeviceAttributeWallClockRate kHz), its waits that
 *               gave up, its polls, and the partner's waits that gave up.
 * Returns 0 when enqueued, 1 for a bad argument, 2 for a HIP error.
 */
int gspn_bench_handshake(void* flags, const uint32_t* abort_flag, int rounds, int spin_max,
                         int partner, uint64_t* out, hipStream_t stream);

/* gspn_bench_wall_clock_khz -- rate of the current device's wall clock
 * (the one gspn_bench_handshake reads) in kHz, or 0 on a HIP error. */
int gspn_bench_wall_clock_khz(void);

/*
 * gspn_bench_strip_t2b -- a measured prototype of the schedule that splits a
 * scan line over several workgroups (not a plan of the library): the
 * top->bottom scan of the propagation (CSDN page on GSPN, section 方法; the
 * weights of section 如何设计一个高效的传播层), global, bf16 storage, fp32
 * state, out = u * h_T2B, for `planes` contiguous row-major H x W planes.
 * Each plane is split into S strips of W / S columns; one 64-lane workgroup
 * owns a strip plus K halo columns on each side (W / S + 2K <= 64, W / S >= K,
 * K 8 or 16) and hands its edge states to its neighbours through device
 * memory every K rows. pf planes are in flight at once; the pf * S
 * workgroups must all be resident (checked: returns 1 otherwise).
 *   x, lam, logits[3], u, out  device bf16 tensors of planes * H * W elements;
 *   work        device memory, 256-byte aligned, at least
 *               gspn_bench_strip_work_bytes(S, K, pf) bytes, zeroed by the
 *               caller before every launch (flags, give-up word, halo states);
 *   abort_flag  host-visible memory; setting it non-zero ends every wait;
 *   spin_max    polls after which a wait gives up; a give-up sets the word
 *               at work + gspn_bench_strip_fail_offset(S, pf) (uint32), every
 *               workgroup then exits, and out is not valid.
 * Returns 0 when enqueued, 1 for a bad argument (nothing enqueued), 2 for a
 * HIP error.
 */
size_t gspn_bench_strip_work_bytes(int S, int K, int pf);
size_t gspn_bench_strip_fail_offset(int S, int pf);
int gspn_bench_strip_t2b(const void* x, const void* lam, const void* const logits[3],
                         const void* u, void* out, int64_t planes, int H, int W, int S, int K,
                         int pf, void* work, size_t work_bytes, const uint32_t* abort_flag,
                         int spin_max, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif  /* GSPN_BENCH_H */

/*
 * GSPN 2D line-scan propagation: fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may include, link or
 * call this library; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it. It shares no code, header or constant with the HIP
 * library under linear_spatial_propagation_line_amd/.
 *
 * What it computes ("Parallel Sequence Modeling via Generalized Spatial
 * Propagation Network", summarised on the CSDN page "GSPN——在convolution基础上
 * 并行序列建模", section 方法 (method) and section 如何设计一个高效的传播层):
 *
 *   for each scan direction d in dir_mask, each plane (b, c):
 *     h_s = w_s h_{s-1} + lambda_s (.) x_s          (recurrence, section 方法)
 *     w_s tridiagonal: pixel o of line s links to o-1, o, o+1 of line s-1
 *         (up-left, up, up-right; section 如何设计一个高效的传播层)
 *     w_s[o][o+k-1] = sigmoid(l_k) / sum over in-range k' of sigmoid(l_k')
 *         (row-wise normalisation, same section, the w_{tau,i,k} formula)
 *   y = sum_d u (.) h_d                              (output gate y_i = u_i h_i,
 *                                                     four-direction merge)
 *
 * Readings of points the pages leave open are listed in the source file.
 */
#ifndef GSPN_ORACLE_H
#define GSPN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element type of the oracle's inputs */
enum { ORC_F64 = 0, ORC_F32 = 1, ORC_BF16 = 2 };

/* direction bits: top->bottom, bottom->top, left->right, right->left */
enum { ORC_T2B = 1, ORC_B2T = 2, ORC_L2R = 4, ORC_R2L = 8 };

/*
 * x, l0, l1, l2, lam, u: host arrays, contiguous [B, C, H, W], element type
 * in_dtype (bf16 given as raw uint16 bit patterns). l0/l1/l2 hold the logit of
 * the neighbour at orthogonal offset -1 / 0 / +1 (image coordinates).
 * group_rows: 0 = global scan; G >= 1 = the scan restarts at every block of G
 * positions [mG, (m+1)G) along the scan axis.
 * out: host array of B*C*H*W doubles, overwritten with y.
 * nthreads: worker threads over planes (<= 0 means 1).
 * Returns 0, or -1 on a bad argument (nothing written).
 */
int gspn_oracle_propagate(const void* x, const void* l0, const void* l1,
                          const void* l2, const void* lam, const void* u,
                          int in_dtype, int64_t B, int64_t C, int64_t H,
                          int64_t W, uint32_t dir_mask, int64_t group_rows,
                          double* out, int nthreads);

/*
 * Backward pass (CSDN page, section 反向传播): given gy = dL/dy (same layout
 * and element type as the inputs), writes dL/dx, dL/dl0, dL/dl1, dL/dl2,
 * dL/dlambda and dL/du as B*C*H*W doubles each (the logit gradients go
 * through the sigmoid and the normalisation). Same arguments and return
 * value as gspn_oracle_propagate otherwise.
 */
int gspn_oracle_backward(const void* x, const void* l0, const void* l1, const void* l2,
                         const void* lam, const void* u, const void* gy, int in_dtype,
                         int64_t B, int64_t C, int64_t H, int64_t W, uint32_t dir_mask,
                         int64_t group_rows, double* dx, double* dl0, double* dl1,
                         double* dl2, double* dlam, double* du, int nthreads);

/*
 * Channel-shared logits (CSDN page, section 局限性: the speed test sets the
 * weights' feature dimension to 1): l0, l1, l2 are [B, logit_channels, H, W]
 * with logit_channels dividing C; channel c uses logit channel
 * c / (C / logit_channels). The backward's dl0..dl2 then have that shape too,
 * each the sum over the channels that share it. logit_channels = C is the
 * plain call. Returns -1 when logit_channels is < 1 or does not divide C.
 */
int gspn_oracle_propagate_shared(const void* x, const void* l0, const void* l1,
                                 const void* l2, const void* lam, const void* u,
                                 int in_dtype, int64_t B, int64_t C, int64_t H,
                                 int64_t W, int64_t logit_channels, uint32_t dir_mask,
                                 int64_t group_rows, double* out, int nthreads);
int gspn_oracle_backward_shared(const void* x, const void* l0, const void* l1,
                                const void* l2, const void* lam, const void* u,
                                const void* gy, int in_dtype, int64_t B, int64_t C,
                                int64_t H, int64_t W, int64_t logit_channels,
                                uint32_t dir_mask, int64_t group_rows, double* dx,
                                double* dl0, double* dl1, double* dl2, double* dlam,
                                double* du, int nthreads);

/*
 * Per-direction parameters and a per-channel merger (aitntnews page, sections
 * 二维线性传播 and GSPN架构; CSDN page, section GSPN模块的设计): direction d
 * (0 top->bottom, 1 bottom->top, 2 left->right, 3 right->left) reads lam, l0,
 * l1, l2 and u at element offset d * dir_stride (x is shared), and
 *   y = sum over d in dir_mask of merge[d * C + c] * u_d (.) h_d.
 * merge: host array of 4 * C doubles, or NULL for all ones. dir_stride = 0
 * with merge = NULL is gspn_oracle_propagate. Returns -1 on a bad argument.
 */
int gspn_oracle_propagate_dirs(const void* x, const void* l0, const void* l1,
                               const void* l2, const void* lam, const void* u,
                               int in_dtype, int64_t B, int64_t C, int64_t H,
                               int64_t W, int64_t dir_stride, const double* merge,
                               uint32_t dir_mask, int64_t group_rows, double* out,
                               int nthreads);

/*
 * Backward pass of the per-direction layer (R15; CSDN page, section 反向传播):
 * inputs as gspn_oracle_propagate_dirs plus gy = dL/dy [B, C, H, W]. Outputs
 * (host, float64): dx [B, C, H, W]; dl0, dl1, dl2, dlam, du [4, B, C, H, W]
 * (slice d = direction d; zero for directions outside dir_mask); dmerge
 * [4, C], the gradient of the merge weights (of an all-ones merger when
 * merge is NULL). Returns 0, or -1 on a bad argument.
 */
int gspn_oracle_backward_dirs(const void* x, const void* l0, const void* l1, const void* l2,
                              const void* lam, const void* u, const void* gy, int in_dtype,
                              int64_t B, int64_t C, int64_t H, int64_t W, int64_t dir_stride,
                              const double* merge, uint32_t dir_mask, int64_t group_rows,
                              double* dx, double* dl0, double* dl1, double* dl2,
                              double* dlam, double* du, double* dmerge, int nthreads);

/*
 * Module prologue (aitntnews page, section GSPN架构; reading R16 in the
 * source): x_in [B, Cin, H, W]; w_r [C, Cin], b_r [C]; w_p [5C, C], b_p [5C]
 * with output channel q = t * C + c for t = 0..4 (l0, l1, l2, lambda, u), all
 * of element type in_dtype; b_r / b_p may be NULL (zero bias).
 *   x_out  [B, C, H, W]     = b_r + w_r x_in per pixel, exact (fp64)
 *   xr_out [B, C, H, W]     = x_out rounded to in_dtype (nearest, ties even)
 *   p_out  [5, B, C, H, W]  = b_p + w_p xr_out per pixel, exact (fp64)
 * Returns 0, or -1 on a bad argument.
 */
int gspn_oracle_prologue(const void* x_in, int in_dtype, int64_t B, int64_t Cin, int64_t C,
                         int64_t H, int64_t W, const void* w_r, const void* b_r,
                         const void* w_p, const void* b_p, double* x_out, double* xr_out,
                         double* p_out, int nthreads);

/* out[i] = in[i] rounded to the element type dt (nearest, ties to even), the
 * rounding gspn_oracle_prologue applies to x. Returns 0, or -1. */
int gspn_oracle_round(const double* in, int dt, int64_t n, double* out);

#ifdef __cplusplus
}
#endif

#endif

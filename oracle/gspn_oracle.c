/*
 * GSPN 2D line-scan propagation: fp64 CPU oracle (test infrastructure only;
 * see gspn_oracle.h). Plain loops, written for reading, not for speed.
 *
 * Sources (cited by page title and section):
 *  [P2] CSDN page "GSPN——在convolution基础上并行序列建模":
 *       section 方法 -- the line recurrence h_i = w_i h_{i-1} + lambda_i x_i,
 *           the output gate y_i = u_i h_i, and the unrolled lower-triangular
 *           form G;
 *       section 稳定性-上下文条件 -- Theorems 1 and 2: row-stochastic w_tau
 *           keep the propagation stable and every h a weighted average;
 *       section 如何设计一个高效的传播层 -- three-neighbour (up-left, up,
 *           up-right) tridiagonal w; sigmoid of every non-zero, normalised
 *           over the m_i non-zeros of its row; line scans in four directions;
 *       section GSPN模块的设计 -- local GSPN splits one spatial dimension into
 *           non-overlapping groups and scans inside each group;
 *       section 前向传播 / 算法1 -- the width-axis scan combines the
 *           diagonal-up, horizontal and diagonal-down neighbours.
 *  [P1] aitntnews page on GSPN, section 传播层的关键实现 -- three-neighbour
 *       links, global and local variants, four-direction integration, sigmoid
 *       plus normalisation for every propagation direction.
 *
 * Readings where the pages are silent or ambiguous (R11 concerns only how
 * the test inputs are drawn and has no part here):
 *  R1 The first line of a scan (and of every local group) has no predecessor:
 *     h = lambda x there (the recurrence starts at i = 1 and G_ii = lambda_i).
 *  R2 The weights of line s, orthogonal index o, come from the logits stored
 *     at that pixel; normalising over its in-range neighbours makes each row
 *     of w_s sum to one (row-stochastic, as Theorem 1 requires).
 *  R3 Edge pixels have only the in-range neighbours (m_i = 2, or 1 when the
 *     orthogonal length is 1); links that would leave the image do not exist.
 *     No epsilon in the denominator.
 *  R4 Logit k belongs to the neighbour at orthogonal offset k-1 in image
 *     coordinates (column offset for vertical scans, row offset for
 *     horizontal ones), the same three logit tensors for all four directions.
 *     This follows the listed order up-left, up, up-right and the algorithm's
 *     diagonal-up, horizontal, diagonal-down order.
 *  R5 Unrolling the recurrence multiplies the weight matrices in scan order,
 *     G_ij = w_i w_{i-1} ... w_{j+1} lambda_j; the loops below apply them one
 *     line at a time in that order.
 *  R6 Local groups are blocks of G consecutive positions along the scan axis,
 *     fixed in absolute image coordinates ([mG, (m+1)G), the last one may be
 *     partial); the hidden state restarts whenever the scan enters a new
 *     block, in either scan order, on both axes.
 *  R7 The group size is an argument; the default of 2 that one passage
 *     names is not used (it contradicts the g-fold cost stated beside it).
 *  R8 One set of (logits, lambda, u) is shared by all directions and the
 *     direction outputs are summed (u (.) sum_d h_d).
 *  R9 sigmoid(+inf) = 1, sigmoid(-inf) = 0. A pixel whose in-range logits
 *     all give sigmoid 0 has no defined weights (0/0) and yields NaN.
 *  R10 Everything here is fp64 from exactly decoded fp32 or bf16 inputs.
 *  R12 Backward pass (CSDN page, section 反向传播): the gradients are taken
 *     with respect to this layer's own inputs -- x, lambda, the three logits
 *     before the sigmoid and the normalisation, and u -- for a scalar loss
 *     whose gradient dL/dy is given. The page's version stops at the gates
 *     G1..G3; here the chain rule continues through the normalisation and
 *     the sigmoid, since the gates are built from the logits inside the
 *     layer.
 *  R13 A line that restarts reads nothing from the line before it, so in the
 *     backward pass it sends no error term back to that line (R1, R6).
 *  R14 Channel-shared logits (CSDN page, section 局限性: the speed test sets
 *     the feature dimension of the weights to 1): the logits may have Cl
 *     channels, Cl dividing C, and channel c then uses logit channel
 *     c / (C / Cl) of the same batch entry. Cl = C is the unshared layer. A
 *     shared logit's gradient is the sum over the channels that use it.
 *  R15 Per-direction parameters and the learnable merger (aitntnews page,
 *     sections 二维线性传播 and GSPN架构; CSDN page, section GSPN模块的设计:
 *     every direction has its own normalised weight matrices, and a linear
 *     layer merges the directions): direction d reads its own lambda, logits
 *     and u, stored dir_stride elements after direction d-1's (x is shared),
 *     and the directions are merged by per-channel weights m[d][c],
 *     y = sum_d m[d][c] u_d (.) h_d. A merger that mixes channels as well
 *     would be a dense matrix product and is not part of this layer.
 *  R16 The module's prologue (aitntnews page, section GSPN架构: a shared 1x1
 *     convolution reduces the channels, then three independent 1x1
 *     convolutions produce the input-dependent propagation parameters): a 1x1
 *     convolution is a per-pixel affine map over channels. x = W_r X_in + b_r
 *     (Cin -> C channels); the logit convolution maps x to the three logit
 *     tensors (3C channels), the other two map x to lambda and to u (C
 *     channels each). Every convolution output is a tensor of the storage
 *     type, so x is rounded to it (to nearest, ties to even) before the three
 *     parameter convolutions read it. No activation is applied: the sigmoid
 *     and normalisation of the logits belong to the propagation.
 *  R17 The backward pass of the per-direction layer (CSDN page, section
 *     反向传播, with R15): the gradients of x, of every selected direction's
 *     lambda, logits and u, and of the merge weights. Direction d's error
 *     term starts from m[d][c] u_d gy; dx = sum_d lambda_d e_d,
 *     dlambda_d = x e_d, du_d = m[d][c] gy h_d, and dm[d][c] is the sum over
 *     the batch and the pixels of u_d gy h_d. Directions outside the mask get
 *     zero gradients.
 */
#include "gspn_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ---- input decoding: exact conversion of every storage type to double ---- */
static double load_value(const void* p, int dt, int64_t i) {
  if (dt == ORC_F64) return ((const double*)p)[i];
  if (dt == ORC_F32) return (double)((const float*)p)[i];
  /* bf16: the upper 16 bits of an IEEE binary32 */
  uint32_t bits = (uint32_t)((const uint16_t*)p)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static double sigmoid(double v) { return 1.0 / (1.0 + exp(-v)); }

/* ---- scan geometry of one direction ------------------------------------ */
/* d = 0 top->bottom, 1 bottom->top, 2 left->right, 3 right->left.
 * Scan step s walks the scan axis; o indexes the orthogonal axis. */
static int64_t scan_len(int d, int64_t H, int64_t W) { return d < 2 ? H : W; }
static int64_t orth_len(int d, int64_t H, int64_t W) { return d < 2 ? W : H; }

/* position along the scan axis (image row for vertical, column for
 * horizontal scans) visited at step s */
static int64_t scan_pos(int d, int64_t n_s, int64_t s) {
  return (d == 0 || d == 2) ? s : n_s - 1 - s;
}

static void pixel_of(int d, int64_t p, int64_t o, int64_t* r, int64_t* c) {
  if (d < 2) { *r = p; *c = o; }   /* vertical: rows are lines */
  else       { *r = o; *c = p; }   /* horizontal: columns are lines */
}

/* R1, R6: the state restarts at the first step and whenever the previous
 * position in scan order lies in another group of G positions. */
static int restarts(int d, int64_t n_s, int64_t s, int64_t G) {
  if (s == 0) return 1;
  if (G <= 0) return 0;
  int64_t p = scan_pos(d, n_s, s);
  int64_t prev = scan_pos(d, n_s, s - 1);
  return (p / G) != (prev / G);
}

typedef struct {
  const void *x, *l[3], *lam, *u;
  int dt;
  int64_t B, C, H, W, G, Cl;
  int64_t dstride;      /* R15: elements between two directions' parameters */
  const double* merge;  /* R15: [4][C] merge weights, or NULL for all ones */
  uint32_t mask;
  double* out;
  int64_t next_plane;   /* shared work counter */
  pthread_mutex_t lock;
} job_t;

/* R14: the logit plane that plane (b, c) = plane uses */
static int64_t logit_plane(int64_t plane, int64_t C, int64_t Cl) {
  const int64_t b = plane / C, c = plane % C;
  return b * Cl + c / (C / Cl);
}

/* one direction over one plane; adds u * h into y (this plane's slice) */
static void scan_plane(const job_t* j, int d, int64_t plane, double* y,
                       double* h_prev, double* h_cur) {
  const int64_t H = j->H, W = j->W;
  const int64_t n_s = scan_len(d, H, W), n_o = orth_len(d, H, W);
  const int64_t doff = d * j->dstride;   /* R15: this direction's parameters */
  const int64_t base = plane * H * W;
  const int64_t lbase = logit_plane(plane, j->C, j->Cl) * H * W + doff;
  const double m = j->merge ? j->merge[d * j->C + plane % j->C] : 1.0;
  for (int64_t o = 0; o < n_o; ++o) h_prev[o] = 0.0;

  for (int64_t s = 0; s < n_s; ++s) {
    const int64_t p = scan_pos(d, n_s, s);
    const int first = restarts(d, n_s, s, j->G);
    for (int64_t o = 0; o < n_o; ++o) {
      int64_t r, c;
      pixel_of(d, p, o, &r, &c);
      const int64_t idx = base + r * W + c;
      double acc = 0.0;
      if (!first) {
        /* R2-R4: normalise the sigmoids of the in-range neighbours */
        double sig[3] = {0.0, 0.0, 0.0}, S = 0.0;
        for (int k = 0; k < 3; ++k) {
          const int64_t q = o + k - 1;
          if (q < 0 || q >= n_o) continue;
          sig[k] = sigmoid(load_value(j->l[k], j->dt, lbase + r * W + c));
          S += sig[k];
        }
        for (int k = 0; k < 3; ++k) {
          const int64_t q = o + k - 1;
          if (q < 0 || q >= n_o) continue;
          acc += (sig[k] / S) * h_prev[q];
        }
      }
      h_cur[o] = acc + load_value(j->lam, j->dt, idx + doff) *
                           load_value(j->x, j->dt, idx);
      y[r * W + c] += m * load_value(j->u, j->dt, idx + doff) * h_cur[o];
    }
    double* t = h_prev; h_prev = h_cur; h_cur = t;
  }
}

static void* worker(void* arg) {
  job_t* j = (job_t*)arg;
  const int64_t n_max = j->H > j->W ? j->H : j->W;
  double* h_prev = (double*)malloc(sizeof(double) * (size_t)n_max);
  double* h_cur = (double*)malloc(sizeof(double) * (size_t)n_max);
  if (!h_prev || !h_cur) { free(h_prev); free(h_cur); return (void*)1; }
  for (;;) {
    pthread_mutex_lock(&j->lock);
    const int64_t plane = j->next_plane++;
    pthread_mutex_unlock(&j->lock);
    if (plane >= j->B * j->C) break;
    double* y = j->out + plane * j->H * j->W;
    for (int64_t i = 0; i < j->H * j->W; ++i) y[i] = 0.0;
    /* R8: directions in the fixed order T->B, B->T, L->R, R->L, summed */
    for (int d = 0; d < 4; ++d)
      if (j->mask & (1u << d)) scan_plane(j, d, plane, y, h_prev, h_cur);
  }
  free(h_prev);
  free(h_cur);
  return NULL;
}

/* the forward pass over all planes, on nthreads workers */
static int run_forward(job_t* j, int nthreads) {
  j->next_plane = 0;
  pthread_mutex_init(&j->lock, NULL);
  int nt = nthreads <= 0 ? 1 : nthreads;
  if ((int64_t)nt > j->B * j->C) nt = (int)(j->B * j->C);
  int rc = 0;
  if (nt == 1) {
    if (worker(j) != NULL) rc = -1;
  } else {
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nt);
    if (!th) { pthread_mutex_destroy(&j->lock); return -1; }
    for (int t = 0; t < nt; ++t) pthread_create(&th[t], NULL, worker, j);
    for (int t = 0; t < nt; ++t) {
      void* ret = NULL;
      pthread_join(th[t], &ret);
      if (ret != NULL) rc = -1;
    }
    free(th);
  }
  pthread_mutex_destroy(&j->lock);
  return rc;
}

int gspn_oracle_propagate_shared(const void* x, const void* l0, const void* l1,
                                 const void* l2, const void* lam, const void* u,
                                 int in_dtype, int64_t B, int64_t C, int64_t H,
                                 int64_t W, int64_t logit_channels, uint32_t dir_mask,
                                 int64_t group_rows, double* out, int nthreads) {
  if (!x || !l0 || !l1 || !l2 || !lam || !u || !out) return -1;
  if (B < 0 || C < 0 || H <= 0 || W <= 0) return -1;
  if (dir_mask == 0 || dir_mask > 15) return -1;
  if (group_rows < 0) return -1;
  if (in_dtype != ORC_F64 && in_dtype != ORC_F32 && in_dtype != ORC_BF16)
    return -1;
  if (logit_channels < 1 || (C > 0 && C % logit_channels != 0)) return -1;
  if (B * C == 0) return 0;

  job_t j;
  j.x = x; j.l[0] = l0; j.l[1] = l1; j.l[2] = l2; j.lam = lam; j.u = u;
  j.dt = in_dtype; j.B = B; j.C = C; j.H = H; j.W = W; j.G = group_rows;
  j.Cl = logit_channels; j.dstride = 0; j.merge = NULL;
  j.mask = dir_mask; j.out = out;
  return run_forward(&j, nthreads);
}

int gspn_oracle_propagate_dirs(const void* x, const void* l0, const void* l1,
                               const void* l2, const void* lam, const void* u,
                               int in_dtype, int64_t B, int64_t C, int64_t H,
                               int64_t W, int64_t dir_stride, const double* merge,
                               uint32_t dir_mask, int64_t group_rows, double* out,
                               int nthreads) {
  if (!x || !l0 || !l1 || !l2 || !lam || !u || !out) return -1;
  if (B < 0 || C < 0 || H <= 0 || W <= 0) return -1;
  if (dir_mask == 0 || dir_mask > 15) return -1;
  if (group_rows < 0 || dir_stride < 0) return -1;
  if (in_dtype != ORC_F64 && in_dtype != ORC_F32 && in_dtype != ORC_BF16)
    return -1;
  if (B * C == 0) return 0;

  job_t j;
  j.x = x; j.l[0] = l0; j.l[1] = l1; j.l[2] = l2; j.lam = lam; j.u = u;
  j.dt = in_dtype; j.B = B; j.C = C; j.H = H; j.W = W; j.G = group_rows;
  j.Cl = C; j.dstride = dir_stride; j.merge = merge;
  j.mask = dir_mask; j.out = out;
  return run_forward(&j, nthreads);
}

int gspn_oracle_propagate(const void* x, const void* l0, const void* l1,
                          const void* l2, const void* lam, const void* u,
                          int in_dtype, int64_t B, int64_t C, int64_t H,
                          int64_t W, uint32_t dir_mask, int64_t group_rows,
                          double* out, int nthreads) {
  return gspn_oracle_propagate_shared(x, l0, l1, l2, lam, u, in_dtype, B, C, H, W,
                                      C > 0 ? C : 1, dir_mask, group_rows, out, nthreads);
}

/* ========================================================================
 * Module prologue (R16)
 * ======================================================================== */

/* v rounded to the nearest value of the storage type, ties to even */
static double round_to_type(double v, int dt) {
  if (dt == ORC_F64) return v;
  if (dt == ORC_F32) return (double)(float)v;
  if (v == 0.0 || !isfinite(v)) return v;
  /* bf16 keeps 8 significant bits: v = m 2^e with 0.5 <= |m| < 1 */
  int e;
  const double m = frexp(v, &e);
  return ldexp(nearbyint(ldexp(m, 8)), e - 8);
}

int gspn_oracle_round(const double* in, int dt, int64_t n, double* out) {
  if (!in || !out || n < 0) return -1;
  if (dt != ORC_F64 && dt != ORC_F32 && dt != ORC_BF16) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = round_to_type(in[i], dt);
  return 0;
}

typedef struct {
  const void *x_in, *w_r, *b_r, *w_p, *b_p;
  int dt;
  int64_t B, Cin, C, HW;
  double *x_out, *xr_out, *p_out;
  int64_t next;          /* shared work counter over (b, pixel) */
  pthread_mutex_t lock;
} pjob_t;

static void* prologue_worker(void* arg) {
  pjob_t* j = (pjob_t*)arg;
  const int64_t B = j->B, Cin = j->Cin, C = j->C, HW = j->HW;
  double* xr = (double*)malloc(sizeof(double) * (size_t)(C > 0 ? C : 1));
  if (!xr) return (void*)1;
  for (;;) {
    pthread_mutex_lock(&j->lock);
    const int64_t item = j->next++;
    pthread_mutex_unlock(&j->lock);
    if (item >= B * HW) break;
    const int64_t b = item / HW, px = item % HW;
    /* x[c] = b_r[c] + sum_k w_r[c][k] x_in[k] at this pixel */
    for (int64_t c = 0; c < C; ++c) {
      double acc = j->b_r ? load_value(j->b_r, j->dt, c) : 0.0;
      for (int64_t k = 0; k < Cin; ++k)
        acc += load_value(j->w_r, j->dt, c * Cin + k) *
               load_value(j->x_in, j->dt, (b * Cin + k) * HW + px);
      j->x_out[(b * C + c) * HW + px] = acc;
      xr[c] = round_to_type(acc, j->dt);
      j->xr_out[(b * C + c) * HW + px] = xr[c];
    }
    /* parameter channels q = t * C + c (t: l0, l1, l2, lambda, u) read the
     * rounded x */
    for (int64_t q = 0; q < 5 * C; ++q) {
      double acc = j->b_p ? load_value(j->b_p, j->dt, q) : 0.0;
      for (int64_t c = 0; c < C; ++c) acc += load_value(j->w_p, j->dt, q * C + c) * xr[c];
      const int64_t t = q / C, c = q % C;
      j->p_out[((t * B + b) * C + c) * HW + px] = acc;
    }
  }
  free(xr);
  return NULL;
}

int gspn_oracle_prologue(const void* x_in, int in_dtype, int64_t B, int64_t Cin, int64_t C,
                         int64_t H, int64_t W, const void* w_r, const void* b_r,
                         const void* w_p, const void* b_p, double* x_out, double* xr_out,
                         double* p_out, int nthreads) {
  if (!x_in || !w_r || !w_p || !x_out || !xr_out || !p_out) return -1;
  if (B < 0 || Cin < 1 || C < 1 || H <= 0 || W <= 0) return -1;
  if (in_dtype != ORC_F64 && in_dtype != ORC_F32 && in_dtype != ORC_BF16) return -1;
  if (B == 0) return 0;
  pjob_t j;
  j.x_in = x_in; j.w_r = w_r; j.b_r = b_r; j.w_p = w_p; j.b_p = b_p;
  j.dt = in_dtype; j.B = B; j.Cin = Cin; j.C = C; j.HW = H * W;
  j.x_out = x_out; j.xr_out = xr_out; j.p_out = p_out; j.next = 0;
  pthread_mutex_init(&j.lock, NULL);
  int nt = nthreads <= 0 ? 1 : nthreads;
  if ((int64_t)nt > B * H * W) nt = (int)(B * H * W);
  int rc = 0;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nt);
  if (!th) { pthread_mutex_destroy(&j.lock); return -1; }
  for (int t = 0; t < nt; ++t) pthread_create(&th[t], NULL, prologue_worker, &j);
  for (int t = 0; t < nt; ++t) {
    void* ret = NULL;
    pthread_join(th[t], &ret);
    if (ret != NULL) rc = -1;
  }
  free(th);
  pthread_mutex_destroy(&j.lock);
  return rc;
}

/* ========================================================================
 * Backward pass (CSDN page, section 反向传播 (backward pass): every input
 * gets a gradient; the gradient of a hidden state collects what the later
 * steps of the scan send back; the input gradient goes through the lambda
 * (there: B) factor; the gate gradients combine the error term with the
 * previous hidden state). Reading R12 for the logits.
 *
 * For one direction, with e_s = dL/dh_s (the "error term"):
 *   e_s[o] = u gy at pixel (s, o)
 *            + sum over the pixels o' of line s+1 that link to o (link k of
 *              o' points at o = o' + k - 1) of w_{s+1,k}[o'] e_{s+1}[o'],
 *              unless line s+1 restarts (then it reads nothing from line s);
 *   d(lambda x) at (s, o) += e_s[o];
 *   d w_{s,k}[o] = e_s[o] h_{s-1}[o+k-1] for the in-range links of a line that
 *              does not restart;
 *   w_k = sig_k / S, S = sum_j sig_j  =>  d sig_j = d w_j / S
 *              - (sum_k d w_k sig_k) / S^2;
 *   d l_j = d sig_j sig_j (1 - sig_j);
 *   du += gy h_s (summed over directions), and finally
 *   dx = lambda d(lambda x), dlambda = x d(lambda x).
 * ====================================================================== */

typedef struct {
  const void *x, *l[3], *lam, *u, *gy;
  int dt;
  int64_t B, C, H, W, G, Cl;
  uint32_t mask;
  double *dx, *dl[3], *dlam, *du;
  int64_t next_group;   /* shared work counter over logit planes (or channels) */
  pthread_mutex_t lock;
  /* per-direction parameters (R15): direction d reads lam, the logits and u
   * at element offset d * dstride, its output is scaled by merge[d * C + c],
   * and its gradients go to slice d of dl, dlam and du ([4][B*C*H*W]) */
  int64_t dstride;
  const double* merge;
  double* dmerge;       /* [4][C]: gradient of the merge weights */
} bjob_t;

/* sigmoids of the in-range links of the pixel at plane offset idx, which sits
 * at orthogonal index o of a line of n_o pixels; returns their sum S */
static double link_sigmoids(const bjob_t* j, int64_t idx, int64_t o, int64_t n_o,
                            double sig[3], int in_range[3]) {
  double S = 0.0;
  for (int k = 0; k < 3; ++k) {
    const int64_t q = o + k - 1;
    in_range[k] = q >= 0 && q < n_o;
    sig[k] = in_range[k] ? sigmoid(load_value(j->l[k], j->dt, idx)) : 0.0;
    S += sig[k];
  }
  return S;
}

/* plane offset of the pixel at step s, orthogonal index o of direction d */
static int64_t pixel_offset(const bjob_t* j, int d, int64_t s, int64_t o) {
  const int64_t n_s = scan_len(d, j->H, j->W);
  int64_t r, c;
  pixel_of(d, scan_pos(d, n_s, s), o, &r, &c);
  return r * j->W + c;
}

/* one direction over one plane: adds this direction's share of
 * d(lambda x) into dphi, of du / gy into hsum and of the logit gradients
 * into dl (at the plane's logit plane, R14). The direction's lambda, logits
 * and u sit at element offset doff (R15); its output gate is scaled by m, so
 * its error term starts from m u gy. */
static void backward_plane(const bjob_t* j, int d, int64_t plane, int64_t doff, double m,
                           double* const dl[3], double* h, double* e_cur, double* e_next,
                           double* dphi, double* hsum) {
  const int64_t H = j->H, W = j->W;
  const int64_t n_s = scan_len(d, H, W), n_o = orth_len(d, H, W);
  const int64_t base = plane * H * W;
  const int64_t lbase = logit_plane(plane, j->C, j->Cl) * H * W;
  const int64_t lin = lbase + doff;   /* where the direction's logits are read */

  /* forward: every hidden state of the scan, h[s * n_o + o] */
  for (int64_t s = 0; s < n_s; ++s) {
    const int first = restarts(d, n_s, s, j->G);
    for (int64_t o = 0; o < n_o; ++o) {
      const int64_t pix = pixel_offset(j, d, s, o);
      const int64_t idx = base + pix;
      double acc = 0.0;
      if (!first) {
        double sig[3];
        int in_range[3];
        const double S = link_sigmoids(j, lin + pix, o, n_o, sig, in_range);
        for (int k = 0; k < 3; ++k)
          if (in_range[k]) acc += (sig[k] / S) * h[(s - 1) * n_o + o + k - 1];
      }
      h[s * n_o + o] =
          acc + load_value(j->lam, j->dt, doff + idx) * load_value(j->x, j->dt, idx);
      hsum[pix] += h[s * n_o + o];
    }
  }

  /* adjoint, last step first */
  for (int64_t o = 0; o < n_o; ++o) e_next[o] = 0.0;
  for (int64_t s = n_s - 1; s >= 0; --s) {
    const int next_reads = s + 1 < n_s && !restarts(d, n_s, s + 1, j->G);
    for (int64_t o = 0; o < n_o; ++o) {
      const int64_t pix = pixel_offset(j, d, s, o);
      const int64_t idx = base + pix;
      double e = m * load_value(j->u, j->dt, doff + idx) * load_value(j->gy, j->dt, idx);
      if (next_reads) {
        for (int k = 0; k < 3; ++k) {
          const int64_t op = o - k + 1;   /* o' with o' + k - 1 == o */
          if (op < 0 || op >= n_o) continue;
          double sig[3];
          int in_range[3];
          const double S = link_sigmoids(j, lin + pixel_offset(j, d, s + 1, op), op, n_o,
                                         sig, in_range);
          e += (sig[k] / S) * e_next[op];
        }
      }
      e_cur[o] = e;
      dphi[pix] += e;
      if (!restarts(d, n_s, s, j->G)) {
        double sig[3], dw[3] = {0.0, 0.0, 0.0};
        int in_range[3];
        const double S = link_sigmoids(j, lin + pix, o, n_o, sig, in_range);
        double t = 0.0;   /* sum_k dw_k sig_k */
        for (int k = 0; k < 3; ++k) {
          if (!in_range[k]) continue;
          dw[k] = e * h[(s - 1) * n_o + o + k - 1];
          t += dw[k] * sig[k];
        }
        for (int k = 0; k < 3; ++k) {
          if (!in_range[k]) continue;
          const double dsig = dw[k] / S - t / (S * S);
          dl[k][lbase + pix] += dsig * sig[k] * (1.0 - sig[k]);
        }
      }
    }
    double* tmp = e_next; e_next = e_cur; e_cur = tmp;
  }
}

static void* bworker(void* arg) {
  bjob_t* j = (bjob_t*)arg;
  const int64_t H = j->H, W = j->W;
  const int64_t n_max = H > W ? H : W;
  double* h = (double*)malloc(sizeof(double) * (size_t)(H * W));
  double* dphi = (double*)malloc(sizeof(double) * (size_t)(H * W));
  double* hsum = (double*)malloc(sizeof(double) * (size_t)(H * W));
  double* e_cur = (double*)malloc(sizeof(double) * (size_t)n_max);
  double* e_next = (double*)malloc(sizeof(double) * (size_t)n_max);
  void* ret = NULL;
  if (!h || !dphi || !hsum || !e_cur || !e_next) { ret = (void*)1; goto done; }
  /* one unit of work = one logit plane and, in channel order, the planes
   * that share it, so every shared gradient is summed in a fixed order */
  const int64_t per = j->C / j->Cl;
  for (;;) {
    pthread_mutex_lock(&j->lock);
    const int64_t grp = j->next_group++;
    pthread_mutex_unlock(&j->lock);
    if (grp >= j->B * j->Cl) break;
    for (int k = 0; k < 3; ++k)
      for (int64_t i = 0; i < H * W; ++i) j->dl[k][grp * H * W + i] = 0.0;
    const int64_t b = grp / j->Cl, cl = grp % j->Cl;
    for (int64_t c = cl * per; c < (cl + 1) * per; ++c) {
      const int64_t plane = b * j->C + c;
      const int64_t base = plane * H * W;
      for (int64_t i = 0; i < H * W; ++i) {
        dphi[i] = 0.0;
        hsum[i] = 0.0;
      }
      for (int d = 0; d < 4; ++d)
        if (j->mask & (1u << d))
          backward_plane(j, d, plane, 0, 1.0, j->dl, h, e_cur, e_next, dphi, hsum);
      for (int64_t i = 0; i < H * W; ++i) {
        j->dx[base + i] = load_value(j->lam, j->dt, base + i) * dphi[i];
        j->dlam[base + i] = load_value(j->x, j->dt, base + i) * dphi[i];
        j->du[base + i] = load_value(j->gy, j->dt, base + i) * hsum[i];
      }
    }
  }
done:
  free(h); free(dphi); free(hsum); free(e_cur); free(e_next);
  return ret;
}

int gspn_oracle_backward_shared(const void* x, const void* l0, const void* l1,
                                const void* l2, const void* lam, const void* u,
                                const void* gy, int in_dtype, int64_t B, int64_t C,
                                int64_t H, int64_t W, int64_t logit_channels,
                                uint32_t dir_mask, int64_t group_rows, double* dx,
                                double* dl0, double* dl1, double* dl2, double* dlam,
                                double* du, int nthreads) {
  if (!x || !l0 || !l1 || !l2 || !lam || !u || !gy) return -1;
  if (!dx || !dl0 || !dl1 || !dl2 || !dlam || !du) return -1;
  if (B < 0 || C < 0 || H <= 0 || W <= 0) return -1;
  if (dir_mask == 0 || dir_mask > 15) return -1;
  if (group_rows < 0) return -1;
  if (in_dtype != ORC_F64 && in_dtype != ORC_F32 && in_dtype != ORC_BF16)
    return -1;
  if (logit_channels < 1 || (C > 0 && C % logit_channels != 0)) return -1;
  if (B * C == 0) return 0;

  bjob_t j;
  j.x = x; j.l[0] = l0; j.l[1] = l1; j.l[2] = l2; j.lam = lam; j.u = u; j.gy = gy;
  j.dt = in_dtype; j.B = B; j.C = C; j.H = H; j.W = W; j.G = group_rows;
  j.Cl = logit_channels;
  j.mask = dir_mask;
  j.dx = dx; j.dl[0] = dl0; j.dl[1] = dl1; j.dl[2] = dl2; j.dlam = dlam; j.du = du;
  j.next_group = 0;
  j.dstride = 0; j.merge = NULL; j.dmerge = NULL;
  pthread_mutex_init(&j.lock, NULL);

  int nt = nthreads <= 0 ? 1 : nthreads;
  if ((int64_t)nt > B * logit_channels) nt = (int)(B * logit_channels);
  int rc = 0;
  if (nt == 1) {
    if (bworker(&j) != NULL) rc = -1;
  } else {
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nt);
    if (!th) { pthread_mutex_destroy(&j.lock); return -1; }
    for (int t = 0; t < nt; ++t) pthread_create(&th[t], NULL, bworker, &j);
    for (int t = 0; t < nt; ++t) {
      void* r = NULL;
      pthread_join(th[t], &r);
      if (r != NULL) rc = -1;
    }
    free(th);
  }
  pthread_mutex_destroy(&j.lock);
  return rc;
}

int gspn_oracle_backward(const void* x, const void* l0, const void* l1, const void* l2,
                         const void* lam, const void* u, const void* gy, int in_dtype,
                         int64_t B, int64_t C, int64_t H, int64_t W, uint32_t dir_mask,
                         int64_t group_rows, double* dx, double* dl0, double* dl1,
                         double* dl2, double* dlam, double* du, int nthreads) {
  return gspn_oracle_backward_shared(x, l0, l1, l2, lam, u, gy, in_dtype, B, C, H, W,
                                     C > 0 ? C : 1, dir_mask, group_rows, dx, dl0, dl1,
                                     dl2, dlam, du, nthreads);
}

/* Per-direction parameters (R15), backward (R17). With y = sum_d m_d u_d (.) h_d
 * (m_d = merge[d * C + c]), direction d is one scan with its own lambda,
 * logits and u whose error term starts from m_d u_d gy; then
 *   dx       = sum_d lambda_d d(lambda x)_d,   dlambda_d = x d(lambda x)_d,
 *   du_d     = m_d gy h_d,
 *   dmerge_d = sum over the batch and the pixels of u_d gy h_d,
 * and the logit gradients of direction d are the single-direction ones. One
 * unit of work is one channel (all of its images, in batch order), so each
 * merge gradient is summed by one thread in a fixed order. */
static void* bworker_dirs(void* arg) {
  bjob_t* j = (bjob_t*)arg;
  const int64_t H = j->H, W = j->W, HW = H * W, P = j->B * j->C * HW;
  const int64_t n_max = H > W ? H : W;
  double* h = (double*)malloc(sizeof(double) * (size_t)HW);
  double* dphi = (double*)malloc(sizeof(double) * (size_t)HW);
  double* hsum = (double*)malloc(sizeof(double) * (size_t)HW);
  double* e_cur = (double*)malloc(sizeof(double) * (size_t)n_max);
  double* e_next = (double*)malloc(sizeof(double) * (size_t)n_max);
  void* ret = NULL;
  if (!h || !dphi || !hsum || !e_cur || !e_next) { ret = (void*)1; goto done; }
  for (;;) {
    pthread_mutex_lock(&j->lock);
    const int64_t c = j->next_group++;
    pthread_mutex_unlock(&j->lock);
    if (c >= j->C) break;
    for (int d = 0; d < 4; ++d) j->dmerge[d * j->C + c] = 0.0;
    for (int64_t b = 0; b < j->B; ++b) {
      const int64_t plane = b * j->C + c;
      const int64_t base = plane * HW;
      for (int64_t i = 0; i < HW; ++i) j->dx[base + i] = 0.0;
      for (int d = 0; d < 4; ++d) {
        const int64_t go = d * P;   /* this direction's gradient slice */
        double* const dl[3] = {j->dl[0] + go, j->dl[1] + go, j->dl[2] + go};
        for (int k = 0; k < 3; ++k)
          for (int64_t i = 0; i < HW; ++i) dl[k][base + i] = 0.0;
        for (int64_t i = 0; i < HW; ++i) j->dlam[go + base + i] = j->du[go + base + i] = 0.0;
        if (!(j->mask & (1u << d))) continue;
        const int64_t doff = d * j->dstride;
        const double m = j->merge ? j->merge[d * j->C + c] : 1.0;
        for (int64_t i = 0; i < HW; ++i) dphi[i] = hsum[i] = 0.0;
        backward_plane(j, d, plane, doff, m, dl, h, e_cur, e_next, dphi, hsum);
        for (int64_t i = 0; i < HW; ++i) {
          const double g = load_value(j->gy, j->dt, base + i);
          j->dx[base + i] += load_value(j->lam, j->dt, doff + base + i) * dphi[i];
          j->dlam[go + base + i] = load_value(j->x, j->dt, base + i) * dphi[i];
          j->du[go + base + i] = m * g * hsum[i];
          j->dmerge[d * j->C + c] += load_value(j->u, j->dt, doff + base + i) * g * hsum[i];
        }
      }
    }
  }
done:
  free(h); free(dphi); free(hsum); free(e_cur); free(e_next);
  return ret;
}

int gspn_oracle_backward_dirs(const void* x, const void* l0, const void* l1, const void* l2,
                              const void* lam, const void* u, const void* gy, int in_dtype,
                              int64_t B, int64_t C, int64_t H, int64_t W, int64_t dir_stride,
                              const double* merge, uint32_t dir_mask, int64_t group_rows,
                              double* dx, double* dl0, double* dl1, double* dl2,
                              double* dlam, double* du, double* dmerge, int nthreads) {
  if (!x || !l0 || !l1 || !l2 || !lam || !u || !gy) return -1;
  if (!dx || !dl0 || !dl1 || !dl2 || !dlam || !du || !dmerge) return -1;
  if (B < 0 || C < 0 || H <= 0 || W <= 0) return -1;
  if (dir_mask == 0 || dir_mask > 15) return -1;
  if (group_rows < 0 || dir_stride < 0) return -1;
  if (in_dtype != ORC_F64 && in_dtype != ORC_F32 && in_dtype != ORC_BF16)
    return -1;
  if (C == 0) return 0;

  bjob_t j;
  j.x = x; j.l[0] = l0; j.l[1] = l1; j.l[2] = l2; j.lam = lam; j.u = u; j.gy = gy;
  j.dt = in_dtype; j.B = B; j.C = C; j.H = H; j.W = W; j.G = group_rows;
  j.Cl = C;
  j.mask = dir_mask;
  j.dx = dx; j.dl[0] = dl0; j.dl[1] = dl1; j.dl[2] = dl2; j.dlam = dlam; j.du = du;
  j.next_group = 0;
  j.dstride = dir_stride; j.merge = merge; j.dmerge = dmerge;
  pthread_mutex_init(&j.lock, NULL);

  int nt = nthreads <= 0 ? 1 : nthreads;
  if ((int64_t)nt > C) nt = (int)C;
  int rc = 0;
  if (nt == 1) {
    if (bworker_dirs(&j) != NULL) rc = -1;
  } else {
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nt);
    if (!th) { pthread_mutex_destroy(&j.lock); return -1; }
    for (int t = 0; t < nt; ++t) pthread_create(&th[t], NULL, bworker_dirs, &j);
    for (int t = 0; t < nt; ++t) {
      void* r = NULL;
      pthread_join(th[t], &r);
      if (r != NULL) rc = -1;
    }
    free(th);
  }
  pthread_mutex_destroy(&j.lock);
  return rc;
}

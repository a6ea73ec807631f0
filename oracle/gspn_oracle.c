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
 * Readings where the pages are silent or ambiguous:
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
 *  R5 One set of (logits, lambda, u) is shared by all directions and the
 *     direction outputs are summed (u (.) sum_d h_d).
 *  R6 Local groups are blocks of G consecutive positions along the scan axis,
 *     fixed in absolute image coordinates ([mG, (m+1)G), the last one may be
 *     partial); the hidden state restarts whenever the scan enters a new
 *     block, in either scan order, on both axes.
 *  R7 sigmoid(+inf) = 1, sigmoid(-inf) = 0. A pixel whose in-range logits
 *     all give sigmoid 0 has no defined weights (0/0) and yields NaN.
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
  int64_t B, C, H, W, G;
  uint32_t mask;
  double* out;
  int64_t next_plane;   /* shared work counter */
  pthread_mutex_t lock;
} job_t;

/* one direction over one plane; adds u * h into y (this plane's slice) */
static void scan_plane(const job_t* j, int d, int64_t plane, double* y,
                       double* h_prev, double* h_cur) {
  const int64_t H = j->H, W = j->W;
  const int64_t n_s = scan_len(d, H, W), n_o = orth_len(d, H, W);
  const int64_t base = plane * H * W;
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
          sig[k] = sigmoid(load_value(j->l[k], j->dt, idx));
          S += sig[k];
        }
        for (int k = 0; k < 3; ++k) {
          const int64_t q = o + k - 1;
          if (q < 0 || q >= n_o) continue;
          acc += (sig[k] / S) * h_prev[q];
        }
      }
      h_cur[o] = acc + load_value(j->lam, j->dt, idx) *
                           load_value(j->x, j->dt, idx);
      y[r * W + c] += load_value(j->u, j->dt, idx) * h_cur[o];
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
    /* R5: directions in the fixed order T->B, B->T, L->R, R->L, summed */
    for (int d = 0; d < 4; ++d)
      if (j->mask & (1u << d)) scan_plane(j, d, plane, y, h_prev, h_cur);
  }
  free(h_prev);
  free(h_cur);
  return NULL;
}

int gspn_oracle_propagate(const void* x, const void* l0, const void* l1,
                          const void* l2, const void* lam, const void* u,
                          int in_dtype, int64_t B, int64_t C, int64_t H,
                          int64_t W, uint32_t dir_mask, int64_t group_rows,
                          double* out, int nthreads) {
  if (!x || !l0 || !l1 || !l2 || !lam || !u || !out) return -1;
  if (B < 0 || C < 0 || H <= 0 || W <= 0) return -1;
  if (dir_mask == 0 || dir_mask > 15) return -1;
  if (group_rows < 0) return -1;
  if (in_dtype != ORC_F64 && in_dtype != ORC_F32 && in_dtype != ORC_BF16)
    return -1;
  if (B * C == 0) return 0;

  job_t j;
  j.x = x; j.l[0] = l0; j.l[1] = l1; j.l[2] = l2; j.lam = lam; j.u = u;
  j.dt = in_dtype; j.B = B; j.C = C; j.H = H; j.W = W; j.G = group_rows;
  j.mask = dir_mask; j.out = out; j.next_plane = 0;
  pthread_mutex_init(&j.lock, NULL);

  int nt = nthreads <= 0 ? 1 : nthreads;
  if ((int64_t)nt > B * C) nt = (int)(B * C);
  int rc = 0;
  if (nt == 1) {
    if (worker(&j) != NULL) rc = -1;
  } else {
    pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nt);
    if (!th) { pthread_mutex_destroy(&j.lock); return -1; }
    for (int t = 0; t < nt; ++t) pthread_create(&th[t], NULL, worker, &j);
    for (int t = 0; t < nt; ++t) {
      void* ret = NULL;
      pthread_join(th[t], &ret);
      if (ret != NULL) rc = -1;
    }
    free(th);
  }
  pthread_mutex_destroy(&j.lock);
  return rc;
}

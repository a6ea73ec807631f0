/* Drives every oracle entry point over small, ragged problems (edge sizes,
 * local groups, shared logits, per-direction parameters, the prologue, and
 * rejected arguments) so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer checks its memory accesses and arithmetic.
 * Exit status 0 when every call returned what it should. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "gspn_oracle.h"

static uint64_t rng = 88172645463325252ull;
static double unif(void) {            /* xorshift64, in [-1, 1) */
  rng ^= rng << 13; rng ^= rng >> 7; rng ^= rng << 17;
  return (double)(rng >> 11) / 4503599627370496.0 - 1.0;
}

static void* fill(int dt, size_t n) {
  size_t es = dt == ORC_F64 ? 8 : (dt == ORC_F32 ? 4 : 2);
  unsigned char* p = malloc(n * es ? n * es : 1);
  for (size_t i = 0; i < n; ++i) {
    double v = 2.0 * unif();
    if (dt == ORC_F64) ((double*)p)[i] = v;
    else if (dt == ORC_F32) ((float*)p)[i] = (float)v;
    else { float f = (float)v; uint32_t b; memcpy(&b, &f, 4); ((uint16_t*)p)[i] = (uint16_t)(b >> 16); }
  }
  return p;
}

static int fails = 0;
#define EXPECT(cond) do { if (!(cond)) { fprintf(stderr, "failed: %s (line %d)\n", #cond, __LINE__); ++fails; } } while (0)

int main(void) {
  const int64_t shapes[][4] = {{1, 1, 1, 1}, {1, 2, 1, 7}, {2, 1, 6, 1}, {1, 3, 5, 4},
                               {2, 2, 17, 9}, {1, 1, 33, 64}};
  const int dts[3] = {ORC_F64, ORC_F32, ORC_BF16};
  for (size_t si = 0; si < sizeof shapes / sizeof shapes[0]; ++si) {
    const int64_t B = shapes[si][0], C = shapes[si][1], H = shapes[si][2], W = shapes[si][3];
    const size_t n = (size_t)(B * C * H * W);
    for (int di = 0; di < 3; ++di) {
      const int dt = dts[di];
      void* in[7];
      for (int k = 0; k < 7; ++k) in[k] = fill(dt, 4 * n);   /* room for 4 directions */
      double* o[7];
      for (int k = 0; k < 7; ++k) o[k] = malloc(4 * n * sizeof(double) + 4 * C * sizeof(double));
      for (uint32_t mask = 1; mask <= 15; mask += 7) {
        for (int64_t G = 0; G <= 3; G += 3) {
          EXPECT(gspn_oracle_propagate(in[0], in[1], in[2], in[3], in[4], in[5], dt, B, C, H,
                                       W, mask, G, o[0], 2) == 0);
          EXPECT(gspn_oracle_backward(in[0], in[1], in[2], in[3], in[4], in[5], in[6], dt, B,
                                      C, H, W, mask, G, o[0], o[1], o[2], o[3], o[4], o[5],
                                      3) == 0);
          EXPECT(gspn_oracle_propagate_shared(in[0], in[1], in[2], in[3], in[4], in[5], dt, B,
                                              C, H, W, 1, mask, G, o[0], 1) == 0);
          EXPECT(gspn_oracle_backward_shared(in[0], in[1], in[2], in[3], in[4], in[5], in[6],
                                             dt, B, C, H, W, 1, mask, G, o[0], o[1], o[2],
                                             o[3], o[4], o[5], 2) == 0);
          double merge[4 * 8];
          for (int k = 0; k < 4 * 8; ++k) merge[k] = unif();
          EXPECT(gspn_oracle_propagate_dirs(in[0], in[1], in[2], in[3], in[4], in[5], dt, B,
                                            C, H, W, (int64_t)n, merge, mask, G, o[0],
                                            2) == 0);
          EXPECT(gspn_oracle_backward_dirs(in[0], in[1], in[2], in[3], in[4], in[5], in[6], dt,
                                           B, C, H, W, (int64_t)n, merge, mask, G, o[0], o[1],
                                           o[2], o[3], o[4], o[5], o[6], 3) == 0);
        }
      }
      /* rejected arguments write nothing and return -1 */
      EXPECT(gspn_oracle_propagate(in[0], in[1], in[2], in[3], in[4], in[5], dt, B, C, H, W,
                                   0, 0, o[0], 1) == -1);
      EXPECT(gspn_oracle_propagate(in[0], in[1], in[2], in[3], in[4], in[5], 7, B, C, H, W,
                                   15, 0, o[0], 1) == -1);
      if (C > 1)
        EXPECT(gspn_oracle_propagate_shared(in[0], in[1], in[2], in[3], in[4], in[5], dt, B, C,
                                            H, W, C + 1, 15, 0, o[0], 1) == -1);
      /* prologue: Cin = 3 channels in, C out */
      if (dt != ORC_F64 || si < 3) {
        void* xin = fill(dt, (size_t)(B * 3 * H * W));
        void* wr = fill(dt, (size_t)(C * 3));
        void* br = fill(dt, (size_t)C);
        void* wp = fill(dt, (size_t)(5 * C * C));
        double* xo = malloc(n * sizeof(double));
        double* xr = malloc(n * sizeof(double));
        double* po = malloc(5 * n * sizeof(double));
        EXPECT(gspn_oracle_prologue(xin, dt, B, 3, C, H, W, wr, br, wp, NULL, xo, xr, po,
                                    2) == 0);
        EXPECT(gspn_oracle_round(xo, dt, (int64_t)n, xr) == 0);
        free(xin); free(wr); free(br); free(wp); free(xo); free(xr); free(po);
      }
      for (int k = 0; k < 7; ++k) { free(in[k]); free(o[k]); }
    }
  }
  if (fails) fprintf(stderr, "%d checks failed\n", fails);
  else printf("oracle driver: all calls clean\n");
  return fails ? 1 : 0;
}

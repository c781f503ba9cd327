/*
 * Host driver for the oracle under AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_oracle_sanitizers.py
 * builds it with oracle/sdm_oracle.c). It checks nothing about the oracle's values: it only runs every entry point
 * over small shapes (two and three factors, W != R, float32 and bfloat16 banks and activations, bank rows beyond
 * the slot count, every snapshot mode, both bank-gradient precisions, several threads) so that an out-of-bounds
 * access, a use of freed memory, a leak or undefined arithmetic in the oracle stops the run with a report.
 * Inputs come from a fixed linear congruential sequence; exit status 0 means every call ran and returned 0.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_topk(int B, int T, int H, int F, const int* widths, int dk, const float* queries, const float* subkeys,
                int k, int32_t* ids, float* scores, int nthreads);
int oracle_write_read(int B, int T, int H, int F, const int* widths, int dk, int d, int W, int R, int bank_bf16,
                      int act_bf16, const float* wkeys, const float* rq, const float* values, const float* alpha,
                      const float* beta, const float* subkeys, float* bank, int64_t bank_rows, float* out,
                      int32_t* widx, int32_t* ridx, float* wsc, float* rsc, int nthreads);
int oracle_write_read_backward(int B, int T, int H, int F, const int* widths, int dk, int d, int W, int R,
                               int bank_bf16, int exact, int snap_bf16, int grad_bank_bf16, const float* wkeys,
                               const float* rq, const float* values, const float* alpha, const float* beta,
                               const float* subkeys, const float* bank, int64_t bank_rows, const float* dout,
                               const float* dbank, double* d_wkeys, double* d_rq, double* d_values, double* d_alpha,
                               double* d_beta, double* d_subkeys, double* d_bank, double* out64, double* bank64,
                               int nthreads);
int oracle_write_read_backward_bounds(int B, int T, int H, int F, const int* widths, int dk, int d, int W, int R,
                                      int bank_bf16, int snap_bf16, int grad_bank_bf16, const float* wkeys,
                                      const float* rq, const float* values, const float* alpha, const float* beta,
                                      const float* subkeys, const float* bank, int64_t bank_rows, const float* dout,
                                      const float* dbank, double* d_wkeys, double* d_rq, double* d_values,
                                      double* d_alpha, double* d_beta, double* d_subkeys, double* d_bank,
                                      double* out64, double* bank64, float* snap_out, const double* par,
                                      double* e_wkeys, double* e_rq, double* e_values, double* e_alpha,
                                      double* e_beta, double* e_subkeys, double* e_bank, int nthreads);
void oracle_snap_rows(const double* in, double* out, int64_t n, int d, int mode);
void oracle_factor_scores(int n, int dk, const float* q, const float* C, float* s);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;

static float next_uniform(void) { /* in (-1, 1) */
  g_state = g_state * 6364136223846793005ull + 1442695040888963407ull;
  return (float)((double)(g_state >> 11) * (2.0 / 9007199254740992.0) - 1.0);
}

static float* randf(size_t n, float lo, float hi) {
  float* p = malloc((n ? n : 1) * sizeof(float));
  if (!p) exit(3);
  for (size_t i = 0; i < n; ++i) p[i] = lo + (hi - lo) * 0.5f * (next_uniform() + 1.0f);
  return p;
}

static void* zalloc(size_t n) {
  void* p = calloc(n ? n : 1, 1);
  if (!p) exit(3);
  return p;
}

static int failures = 0;

static void expect(int rc, const char* what) {
  if (rc != 0) {
    fprintf(stderr, "%s returned %d\n", what, rc);
    ++failures;
  }
}

typedef struct {
  int B, T, H, F, widths[3], dk, d, W, R, extra_rows;
} shape_t;

static void run_shape(const shape_t* s, int bank_bf16, int act_bf16) {
  const int B = s->B, T = s->T, H = s->H, F = s->F, dk = s->dk, d = s->d, W = s->W, R = s->R;
  int64_t N = 1, sumn = 0;
  for (int f = 0; f < F; ++f) { N *= s->widths[f]; sumn += s->widths[f]; }
  const int64_t rows = N + s->extra_rows;
  const size_t tok = (size_t)B * T * H;
  float* wk = randf(tok * F * dk, -1.0f, 1.0f);
  float* rq = randf(tok * F * dk, -1.0f, 1.0f);
  float* v = randf(tok * d, -1.0f, 1.0f);
  float* al = randf(tok, 0.05f, 0.95f);
  float* be = randf(tok, 0.05f, 0.95f);
  float* sub = randf((size_t)H * sumn * dk, -1.0f, 1.0f);
  const size_t nb = (size_t)B * H * rows * d;
  float* bank = randf(nb, -0.05f, 0.05f);
  float* dout = randf(tok * d, -1.0f, 1.0f);
  float* dbank = randf(nb, -0.1f, 0.1f);

  int32_t* ids = zalloc(tok * W * sizeof(int32_t));
  float* sc = zalloc(tok * W * sizeof(float));
  expect(oracle_topk(B, T, H, F, s->widths, dk, wk, sub, W, ids, sc, 3), "oracle_topk");

  float* bank2 = zalloc(nb * sizeof(float));
  for (size_t i = 0; i < nb; ++i) bank2[i] = bank[i];
  float* out = zalloc(tok * d * sizeof(float));
  int32_t* widx = zalloc(tok * W * sizeof(int32_t));
  int32_t* ridx = zalloc(tok * R * sizeof(int32_t));
  float* wsc = zalloc(tok * W * sizeof(float));
  float* rsc = zalloc(tok * R * sizeof(float));
  expect(oracle_write_read(B, T, H, F, s->widths, dk, d, W, R, bank_bf16, act_bf16, wk, rq, v, al, be, sub, bank2,
                           rows, out, widx, ridx, wsc, rsc, 2),
         "oracle_write_read");
  expect(oracle_write_read(B, T, H, F, s->widths, dk, d, W, R, bank_bf16, act_bf16, wk, rq, v, al, be, sub, bank2,
                           rows, out, NULL, NULL, NULL, NULL, 1),
         "oracle_write_read without ids");

  double* g[7];
  double* e[7];
  const size_t gn[7] = {tok * F * dk, tok * F * dk, tok * d, tok, tok, (size_t)H * sumn * dk, nb};
  for (int i = 0; i < 7; ++i) {
    g[i] = zalloc(gn[i] * sizeof(double));
    e[i] = zalloc(gn[i] * sizeof(double));
  }
  double* out64 = zalloc(tok * d * sizeof(double));
  double* bank64 = zalloc(nb * sizeof(double));
  float* snap = zalloc((size_t)B * H * T * W * d * sizeof(float));
  for (int exact = 0; exact <= 1; ++exact)
    expect(oracle_write_read_backward(B, T, H, F, s->widths, dk, d, W, R, bank_bf16, exact, 0, 0, wk, rq, v, al, be,
                                      sub, bank, rows, dout, exact ? NULL : dbank, g[0], g[1], g[2], g[3], g[4], g[5],
                                      g[6], exact ? NULL : out64, exact ? NULL : bank64, 2),
           "oracle_write_read_backward");
  const double par[6] = {ldexp(1.0, -24), 1e-6, ldexp(1.0, -23), 0.0, 0.0, ldexp(1.0, -7)};
  for (int mode = 0; mode <= 3; ++mode) {
    if (bank_bf16 && mode != 0) continue;            /* quantized snapshots are of float32 banks */
    if (mode >= 2 && d % 16 != 0) continue;          /* 16-column groups */
    for (int gb = 0; gb <= bank_bf16; ++gb)
      expect(oracle_write_read_backward_bounds(B, T, H, F, s->widths, dk, d, W, R, bank_bf16, mode, gb, wk, rq, v, al,
                                               be, sub, bank, rows, dout, dbank, g[0], g[1], g[2], g[3], g[4], g[5],
                                               g[6], out64, bank64, snap, par, e[0], e[1], e[2], e[3], e[4], e[5],
                                               e[6], 3),
             "oracle_write_read_backward_bounds");
  }
  for (int i = 0; i < 7; ++i) {
    free(g[i]);
    free(e[i]);
  }
  free(out64); free(bank64); free(snap);
  free(out); free(widx); free(ridx); free(wsc); free(rsc); free(bank2);
  free(ids); free(sc);
  free(wk); free(rq); free(v); free(al); free(be); free(sub); free(bank); free(dout); free(dbank);
}

int main(void) {
  const shape_t shapes[] = {
      {2, 9, 2, 2, {8, 8, 0}, 4, 16, 5, 3, 3},   /* two factors, W != R, bank rows beyond the slots */
      {1, 7, 1, 3, {4, 4, 2}, 2, 32, 6, 9, 0},   /* three factors, R > W */
  };
  for (int i = 0; i < 2; ++i)
    for (int bb = 0; bb <= 1; ++bb)
      for (int ab = 0; ab <= 1; ++ab) run_shape(&shapes[i], bb, ab);
  /* the snapshot row formats on their own: a row with zeros, tiny and large values */
  double in[32], outq[32];
  for (int c = 0; c < 32; ++c) in[c] = c % 5 == 0 ? 0.0 : ldexp((double)next_uniform(), (c % 7) * 9 - 30);
  for (int mode = 0; mode <= 3; ++mode) oracle_snap_rows(in, outq, 1, 32, mode);
  float q[8], C[3 * 8], s3[3];
  for (int c = 0; c < 8; ++c) q[c] = next_uniform();
  for (int c = 0; c < 24; ++c) C[c] = next_uniform();
  oracle_factor_scores(3, 8, q, C, s3);
  if (failures) return 1;
  printf("oracle sanitizer driver: all calls returned 0\n");
  return 0;
}

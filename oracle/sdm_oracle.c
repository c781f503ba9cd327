/*
 * Sparse Delta Memory: CPU oracle. TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, sequential per-token implementation of what the SDM write/read computes, in fp64 arithmetic.
 * It shares no code with the HIP library (no common headers, helpers or tables). Only the test-suite, the smoke
 * check and the bench's cpu_baseline leg load it. Build: gcc -O2 -fPIC -shared -ffp-contract=off -pthread
 * (no fast-math: the factor score and the float32 slot-score additions must be IEEE round-to-nearest-even).
 *
 * Sources (web pages):
 *  [CL]  facebookresearch/sparse-delta-memory, CHANGELOG.md, 2.0.0: "Upgrading from v1" (slot score is the float32
 *        sum of the factor scores; exact top-k; tie order), "New" (any number of factors of any widths; exact top-k),
 *        "Deterministic", "Behavior changes".
 *  [RM]  facebookresearch/sparse-delta-memory, README.md: summary (product keys + gated forget/input delta-rule
 *        updates of a sparse memory), ideas (product-key memory of Lample et al. 2019; the gated delta rule of
 *        Yang et al. 2025).
 *  [PR]  latticedynamics/lumen PR #29 "0.8.0 - a state holds only itself, and a step can give it up": cost model
 *        (per-token arithmetic is O((W+R) d_v), independent of the slot count).
 *
 * Readings taken where the pages are silent:
 *  - factor score: float32 rounding of an fp64 fused-multiply-add chain over the sub-key coordinates, in order,
 *    starting from +0. Factor f uses query columns [f*dk, (f+1)*dk).
 *  - slot score: float32 sum of the factor scores, left to right, each partial rounded to float32 [CL].
 *  - slot id: mixed radix of the per-factor sub-key indices, factor 0 most significant.
 *  - per-factor rank: sub-keys ordered by (score descending, index ascending); position p_f = 0 is the best, so the
 *    pages' "rank" is n_f - 1 - p_f and "larger rank sum, then larger first rank" [CL] is "smaller sum of
 *    positions, then smaller first position"; equal first positions fall through to the next factor's position.
 *  - exact top-k = the k best slots over ALL N slots under that total order (brute force here, by definition).
 *  - address weights: softmax over the k selected slot scores (no temperature), as in product-key memory [RM].
 *  - gated delta rule restricted to the selected rows [RM][PR]: with w the write weights, alpha the forget gate and
 *    beta the input gate, r = sum_i w_i M[S_i];  delta = beta (v - alpha r);  M[S_i] <- alpha M[S_i] + w_i delta.
 *    Rows outside the write set are untouched (per-token work independent of N [PR]).
 *  - the read happens after the token's write: out = sum_i rho_i M[R_i].
 *  - the bank is stored in its dtype: every written row is rounded (round-to-nearest-even) to float32 or bfloat16
 *    after each token; the output is rounded to the activation dtype.
 *
 * Parity pins: the factor score against exact rational arithmetic; brute force top-k against an independent Python
 * enumeration; tie closed forms; F = 1 textbook top-k; no-op gates; single-write closed form; the dense Gated
 * DeltaNet limit (W = R = N); linearity. See tests/test_oracle_pins.py. The backward (oracle_write_read_backward) is
 * pinned by central finite differences of its fp64-state forward along random directions in every input, on banks
 * small enough that slots collide across tokens; see tests/test_oracle_backward_pins.py.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_MAX_F 4

/* ---------------------------------------------------------------------------------------------------------------
 * Rounding helpers (IEEE round-to-nearest-even).
 * ------------------------------------------------------------------------------------------------------------- */

/* Round an fp64 value to the nearest bfloat16 (8 significant bits, float32 exponent range), ties to even, returned
 * as a float (exactly representable). Done directly from fp64 so there is no double rounding through float32. */
double oracle_round_bf16(double x) {
  if (x == 0.0 || !isfinite(x)) return (double)(float)x;
  int e;
  frexp(x, &e);                            /* |x| = m * 2^e, m in [0.5, 1) */
  int lsb_exp = e - 8;                     /* 8 significant bits */
  if (lsb_exp < -133) lsb_exp = -133;      /* bfloat16 subnormal spacing = 2^-133 */
  double q = nearbyint(ldexp(x, -lsb_exp)); /* exact scaling, then RNE to an integer */
  double r = ldexp(q, lsb_exp);
  if (fabs(r) > 3.3895313892515355e38) r = copysign(INFINITY, x); /* above the largest finite bfloat16 */
  return r;
}

static inline float round_to(double x, int bf16) { return bf16 ? (float)oracle_round_bf16(x) : (float)x; }

/* ---------------------------------------------------------------------------------------------------------------
 * Quantized backward snapshots (fp8, int4). The pages name the modes but not their formats; the reading taken:
 * a snapshot row (float32) is stored in groups of 16 consecutive columns, each group with a power-of-two scale
 * s = 2^e, the smallest with (the group's largest magnitude) / s <= qmax, where qmax is the largest finite value of
 * the element format: 448 for OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals
 * spaced 2^-9, no infinities) and 7 for int4 (integers in [-7, 7]). Each element x is stored as the format's
 * nearest value to x / s (exact: s is a power of two), ties to even, and read back as that value times s.
 * ------------------------------------------------------------------------------------------------------------- */
#define SNAP_GROUP 16

/* Nearest OCP E4M3 value to v, ties to even (|v| <= 448, so no saturation is needed). */
double oracle_e4m3_round(double v) {
  const double a = fabs(v);
  if (a == 0.0) return 0.0;
  int ex;
  (void)frexp(a, &ex);                  /* a in [2^(ex-1), 2^ex) */
  int E = ex - 1;                       /* binade exponent */
  if (E < -6) E = -6;                   /* below 2^-6 the spacing stays 2^-9 (subnormals) */
  const double step = ldexp(1.0, E - 3); /* 3 mantissa bits */
  return copysign(nearbyint(a / step) * step, v);
}

/* Scale exponent e of a group whose largest magnitude is amax: the smallest e with amax / 2^e <= qmax. */
int oracle_snap_scale_exp(double amax, double qmax) {
  int ex;
  (void)frexp(amax, &ex);
  int e = ex - 40;
  while (ldexp(amax, -e) > qmax) ++e;
  return e;
}

/* A float32 row of d columns as a snapshot of the given mode stores it: 1 bfloat16, 2 fp8, 3 int4 (d % 16 == 0 for
 * the last two); other modes leave it unchanged. */
static void snap_row(const double* src, double* dst, int d, int mode) {
  if (mode == 1) {
    for (int c = 0; c < d; ++c) dst[c] = (double)round_to(src[c], 1);
    return;
  }
  if (mode != 2 && mode != 3) {
    for (int c = 0; c < d; ++c) dst[c] = src[c];
    return;
  }
  const double qmax = mode == 2 ? 448.0 : 7.0;
  for (int g = 0; g < d; g += SNAP_GROUP) {
    double amax = 0.0;
    for (int c = g; c < g + SNAP_GROUP; ++c) amax = fmax(amax, fabs(src[c]));
    if (amax == 0.0) {
      for (int c = g; c < g + SNAP_GROUP; ++c) dst[c] = 0.0;
      continue;
    }
    const int e = oracle_snap_scale_exp(amax, qmax);
    for (int c = g; c < g + SNAP_GROUP; ++c) {
      const double x = ldexp(src[c], -e);
      const double q = mode == 2 ? oracle_e4m3_round(x) : nearbyint(x);
      dst[c] = ldexp(q, e);
    }
  }
}

/* Python-facing: rows [n, d] through snap_row (out may equal in). */
void oracle_snap_rows(const double* in, double* out, int64_t n, int d, int mode) {
  for (int64_t i = 0; i < n; ++i) snap_row(in + i * d, out + i * d, d, mode);
}

/* ---------------------------------------------------------------------------------------------------------------
 * Factor scores.
 * ------------------------------------------------------------------------------------------------------------- */

/* s[i] = fl32( fma chain over c of q[c] * C[i][c], starting from +0, in coordinate order ). */
void oracle_factor_scores(int n, int dk, const float* q, const float* C, float* s) {
  for (int i = 0; i < n; ++i) {
    double acc = 0.0;
    for (int c = 0; c < dk; ++c) acc = fma((double)q[c], (double)C[(size_t)i * dk + c], acc);
    s[i] = (float)acc;
  }
}

/* ---------------------------------------------------------------------------------------------------------------
 * Exact product-key top-k, by brute force over every slot.
 * ------------------------------------------------------------------------------------------------------------- */

typedef struct {
  float S;               /* float32 slot score */
  int psum;              /* sum of per-factor positions */
  int p[ORACLE_MAX_F];   /* per-factor positions (0 = best) */
  int64_t id;
} cand_t;

/* Total order: larger slot score first; then smaller position sum (= larger rank sum); then smaller position in
 * factor 0 (= larger first rank), then factor 1, ... Returns <0 if a precedes b. */
static int cand_cmp(const cand_t* a, const cand_t* b, int F) {
  if (a->S > b->S) return -1;
  if (a->S < b->S) return 1;
  if (a->psum != b->psum) return a->psum < b->psum ? -1 : 1;
  for (int f = 0; f < F; ++f)
    if (a->p[f] != b->p[f]) return a->p[f] < b->p[f] ? -1 : 1;
  return 0;
}

typedef struct { float s; int i; } fs_t;
static int fs_cmp(const void* x, const void* y) {
  const fs_t* a = (const fs_t*)x; const fs_t* b = (const fs_t*)y;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return a->i < b->i ? -1 : (a->i > b->i ? 1 : 0);
}

/* One query of one head. q: [F*dk]; sub: [sum_f n_f, dk] (factor tables stacked in factor order).
 * Outputs the k best slots, best first: ids (int32) and float32 slot scores. Scratch is allocated here.
 * Returns 0, or -1 on allocation failure / bad arguments. */
int oracle_topk_one(int F, const int* widths, int dk, const float* q, const float* sub, int k, int32_t* ids,
                    float* scores) {
  if (F < 1 || F > ORACLE_MAX_F || k < 1) return -1;
  int64_t N = 1;
  for (int f = 0; f < F; ++f) N *= widths[f];
  if (k > N) return -1;
  float* fsc[ORACLE_MAX_F];
  int* pos[ORACLE_MAX_F];
  fs_t* tmp = NULL;
  int maxw = 0;
  for (int f = 0; f < F; ++f) if (widths[f] > maxw) maxw = widths[f];
  tmp = (fs_t*)malloc(sizeof(fs_t) * (size_t)maxw);
  cand_t* best = (cand_t*)malloc(sizeof(cand_t) * (size_t)k);
  int ok = tmp && best;
  for (int f = 0; f < F; ++f) { fsc[f] = NULL; pos[f] = NULL; }
  size_t off = 0;
  for (int f = 0; f < F && ok; ++f) {
    fsc[f] = (float*)malloc(sizeof(float) * (size_t)widths[f]);
    pos[f] = (int*)malloc(sizeof(int) * (size_t)widths[f]);
    if (!fsc[f] || !pos[f]) { ok = 0; break; }
    oracle_factor_scores(widths[f], dk, q + (size_t)f * dk, sub + off * dk, fsc[f]);
    off += widths[f];
    for (int i = 0; i < widths[f]; ++i) { tmp[i].s = fsc[f][i]; tmp[i].i = i; }
    qsort(tmp, (size_t)widths[f], sizeof(fs_t), fs_cmp);
    for (int p = 0; p < widths[f]; ++p) pos[f][tmp[p].i] = p;
  }
  if (ok) {
    int nbest = 0;
    int dig[ORACLE_MAX_F] = {0, 0, 0, 0};
    for (int64_t id = 0; id < N; ++id) {
      /* digits of id in mixed radix (factor 0 most significant), kept incrementally */
      if (id > 0) {
        for (int f = F - 1; f >= 0; --f) {
          if (++dig[f] < widths[f]) break;
          dig[f] = 0;
        }
      }
      cand_t c;
      float S = fsc[0][dig[0]];
      for (int f = 1; f < F; ++f) S = S + fsc[f][dig[f]]; /* float32 addition, left to right */
      c.S = S;
      c.psum = 0;
      for (int f = 0; f < ORACLE_MAX_F; ++f) c.p[f] = 0;
      for (int f = 0; f < F; ++f) { c.p[f] = pos[f][dig[f]]; c.psum += c.p[f]; }
      c.id = id;
      if (nbest == k && cand_cmp(&c, &best[k - 1], F) >= 0) continue;
      /* insert into the sorted list */
      int j = nbest < k ? nbest : k - 1;
      while (j > 0 && cand_cmp(&c, &best[j - 1], F) < 0) { best[j] = best[j - 1]; --j; }
      best[j] = c;
      if (nbest < k) ++nbest;
    }
    for (int i = 0; i < k; ++i) { ids[i] = (int32_t)best[i].id; scores[i] = best[i].S; }
  }
  for (int f = 0; f < F; ++f) { free(fsc[f]); free(pos[f]); }
  free(tmp);
  free(best);
  return ok ? 0 : -1;
}

/* Softmax over k float32 scores, in fp64, max-subtracted. */
static void softmax64(int k, const float* s, double* w) {
  double m = s[0];
  for (int i = 1; i < k; ++i) if (s[i] > m) m = s[i];
  double z = 0.0;
  for (int i = 0; i < k; ++i) { w[i] = exp((double)s[i] - m); z += w[i]; }
  for (int i = 0; i < k; ++i) w[i] /= z;
}

void oracle_softmax(int k, const float* s, double* w) { softmax64(k, s, w); }

/* ---------------------------------------------------------------------------------------------------------------
 * Top-k over a [B, T, H, F*dk] query tensor (per-head sub-key tables [H, sum n_f, dk]).
 * ------------------------------------------------------------------------------------------------------------- */

typedef struct {
  int B, T, H, F, dk, k;
  const int* widths;
  const float* q;
  const float* sub;
  int32_t* ids;
  float* scores;
  int64_t sumn;
  int64_t begin, end; /* row range [begin, end) over B*T*H rows */
  int err;
} topk_job_t;

static void* topk_worker(void* arg) {
  topk_job_t* j = (topk_job_t*)arg;
  for (int64_t row = j->begin; row < j->end; ++row) {
    int h = (int)(row % j->H);
    if (oracle_topk_one(j->F, j->widths, j->dk, j->q + row * (int64_t)j->F * j->dk, j->sub + (int64_t)h * j->sumn * j->dk,
                        j->k, j->ids + row * j->k, j->scores + row * j->k) != 0)
      j->err = 1;
  }
  return NULL;
}

int oracle_topk(int B, int T, int H, int F, const int* widths, int dk, const float* queries, const float* subkeys,
                int k, int32_t* ids, float* scores, int nthreads) {
  int64_t rows = (int64_t)B * T * H;
  int64_t sumn = 0;
  for (int f = 0; f < F; ++f) sumn += widths[f];
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  int started[256];
  topk_job_t jobs[256];
  int err = 0;
  for (int i = 0; i < nthreads; ++i) {
    topk_job_t* j = &jobs[i];
    j->B = B; j->T = T; j->H = H; j->F = F; j->dk = dk; j->k = k; j->widths = widths; j->q = queries;
    j->sub = subkeys; j->ids = ids; j->scores = scores; j->sumn = sumn; j->err = 0;
    j->begin = rows * i / nthreads; j->end = rows * (i + 1) / nthreads;
    started[i] = pthread_create(&th[i], NULL, topk_worker, j) == 0;
    if (!started[i]) topk_worker(j);
  }
  for (int i = 0; i < nthreads; ++i) { if (started[i]) pthread_join(th[i], NULL); err |= jobs[i].err; }
  return err ? -1 : 0;
}

/* ---------------------------------------------------------------------------------------------------------------
 * The write/read: sequential per token, one stream (b, h) at a time.
 * ------------------------------------------------------------------------------------------------------------- */

typedef struct {
  int B, T, H, F, dk, d, W, R, bank_bf16, act_bf16;
  const int* widths;
  const float *wkeys, *rq, *values, *alpha, *beta, *sub;
  float* bank;
  int64_t bank_rows;
  float* out;
  int32_t *widx, *ridx;
  float *wsc, *rsc;
  int64_t sumn;
  int s_begin, s_end; /* stream range over B*H streams, stream = b*H + h */
  int err;
} wr_job_t;

static void* wr_worker(void* arg) {
  wr_job_t* j = (wr_job_t*)arg;
  const int F = j->F, dk = j->dk, d = j->d, W = j->W, R = j->R, H = j->H, T = j->T;
  int32_t* S = (int32_t*)malloc(sizeof(int32_t) * (size_t)W);
  int32_t* Rd = (int32_t*)malloc(sizeof(int32_t) * (size_t)R);
  float* sS = (float*)malloc(sizeof(float) * (size_t)W);
  float* sR = (float*)malloc(sizeof(float) * (size_t)R);
  double* w = (double*)malloc(sizeof(double) * (size_t)W);
  double* rho = (double*)malloc(sizeof(double) * (size_t)R);
  double* r = (double*)malloc(sizeof(double) * (size_t)d);
  double* delta = (double*)malloc(sizeof(double) * (size_t)d);
  double* o = (double*)malloc(sizeof(double) * (size_t)d);
  if (!S || !Rd || !sS || !sR || !w || !rho || !r || !delta || !o) { j->err = 1; goto done; }
  for (int st = j->s_begin; st < j->s_end; ++st) {
    int b = st / H, h = st % H;
    float* M = j->bank + (int64_t)st * j->bank_rows * d;
    const float* sub = j->sub + (int64_t)h * j->sumn * dk;
    for (int t = 0; t < T; ++t) {
      int64_t row = ((int64_t)b * T + t) * H + h; /* [B, T, H] row */
      if (oracle_topk_one(F, j->widths, dk, j->wkeys + row * F * dk, sub, W, S, sS) != 0 ||
          oracle_topk_one(F, j->widths, dk, j->rq + row * F * dk, sub, R, Rd, sR) != 0) { j->err = 1; goto done; }
      softmax64(W, sS, w);
      softmax64(R, sR, rho);
      const double a = j->alpha[row], be = j->beta[row];
      const float* v = j->values + row * d;
      /* prediction at the write address, from the rows before this token's write */
      for (int c = 0; c < d; ++c) r[c] = 0.0;
      for (int i = 0; i < W; ++i) {
        const float* m = M + (int64_t)S[i] * d;
        for (int c = 0; c < d; ++c) r[c] += w[i] * (double)m[c];
      }
      for (int c = 0; c < d; ++c) delta[c] = be * ((double)v[c] - a * r[c]);
      /* gated delta-rule update of the W selected rows; stored in the bank dtype */
      for (int i = 0; i < W; ++i) {
        float* m = M + (int64_t)S[i] * d;
        for (int c = 0; c < d; ++c) m[c] = round_to(a * (double)m[c] + w[i] * delta[c], j->bank_bf16);
      }
      /* read after the write */
      for (int c = 0; c < d; ++c) o[c] = 0.0;
      for (int i = 0; i < R; ++i) {
        const float* m = M + (int64_t)Rd[i] * d;
        for (int c = 0; c < d; ++c) o[c] += rho[i] * (double)m[c];
      }
      float* out = j->out + row * d;
      for (int c = 0; c < d; ++c) out[c] = round_to(o[c], j->act_bf16);
      if (j->widx) memcpy(j->widx + row * W, S, sizeof(int32_t) * (size_t)W);
      if (j->ridx) memcpy(j->ridx + row * R, Rd, sizeof(int32_t) * (size_t)R);
      if (j->wsc) memcpy(j->wsc + row * W, sS, sizeof(float) * (size_t)W);
      if (j->rsc) memcpy(j->rsc + row * R, sR, sizeof(float) * (size_t)R);
    }
  }
done:
  free(S); free(Rd); free(sS); free(sR); free(w); free(rho); free(r); free(delta); free(o);
  return NULL;
}

/* Tensors (all float32 arrays holding values already rounded to their dtype; bfloat16 values are exact in float32):
 *   wkeys, rq  [B, T, H, F*dk]   write keys / read queries
 *   values     [B, T, H, d]
 *   alpha,beta [B, T, H]         forget / input gates
 *   subkeys    [H, sum n_f, dk]
 *   bank       [B, H, bank_rows, d]  advanced in place (rows >= N untouched)
 *   out        [B, T, H, d]
 *   widx/ridx  [B, T, H, W|R] int32 and wsc/rsc float32 slot scores: optional (NULL to skip)
 * Streams (b, h) are independent and are spread over nthreads threads. Returns 0 or -1. */
int oracle_write_read(int B, int T, int H, int F, const int* widths, int dk, int d, int W, int R, int bank_bf16,
                      int act_bf16, const float* wkeys, const float* rq, const float* values, const float* alpha,
                      const float* beta, const float* subkeys, float* bank, int64_t bank_rows, float* out,
                      int32_t* widx, int32_t* ridx, float* wsc, float* rsc, int nthreads) {
  int64_t sumn = 0, N = 1;
  for (int f = 0; f < F; ++f) { sumn += widths[f]; N *= widths[f]; }
  if (F < 1 || F > ORACLE_MAX_F || W < 1 || R < 1 || W > N || R > N || bank_rows < N) return -1;
  int streams = B * H;
  if (nthreads < 1) nthreads = 1;
  if (nthreads > streams) nthreads = streams > 0 ? streams : 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  int started[256];
  wr_job_t jobs[256];
  int err = 0;
  for (int i = 0; i < nthreads; ++i) {
    wr_job_t* j = &jobs[i];
    j->B = B; j->T = T; j->H = H; j->F = F; j->dk = dk; j->d = d; j->W = W; j->R = R;
    j->bank_bf16 = bank_bf16; j->act_bf16 = act_bf16; j->widths = widths; j->wkeys = wkeys; j->rq = rq;
    j->values = values; j->alpha = alpha; j->beta = beta; j->sub = subkeys; j->bank = bank;
    j->bank_rows = bank_rows; j->out = out; j->widx = widx; j->ridx = ridx; j->wsc = wsc; j->rsc = rsc;
    j->sumn = sumn; j->err = 0;
    j->s_begin = (int)((int64_t)streams * i / nthreads);
    j->s_end = (int)((int64_t)streams * (i + 1) / nthreads);
    started[i] = pthread_create(&th[i], NULL, wr_worker, j) == 0;
    if (!started[i]) wr_worker(j);
  }
  for (int i = 0; i < nthreads; ++i) { if (started[i]) pthread_join(th[i], NULL); err |= jobs[i].err; }
  return err ? -1 : 0;
}

/* ---------------------------------------------------------------------------------------------------------------
 * Backward of the write/read: the reverse-mode derivative of the per-token recurrence above, one stream at a time.
 *
 * The pages ask for gradients of every input, computed deterministically, with the bank restored in place by the
 * backward ([CL] 2.0.0, "Deterministic", "New", "Known limitations"); they print no formula. This is the plain
 * chain rule applied to the recurrence of oracle_write_read, token by token in reverse. With P_i = M[S_i] before
 * the token's write, r = sum_i w_i P_i, delta = beta (v - alpha r), M[S_i] <- alpha P_i + w_i delta and
 * out = sum_j rho_j M[R_j] after the write, and G the adjoint of the bank after the token:
 *   reads:   d rho_j = <dout, M[R_j]>,  G[R_j] += rho_j dout
 *   writes:  g_i = G[S_i];  D = sum_i w_i g_i (the adjoint of delta);  dv = beta D;
 *            d beta = <D, v - alpha r>;  d alpha = sum_i <g_i, P_i> - beta <D, r>;
 *            d w_i = <g_i, delta> - alpha beta <D, P_i>;  G[S_i] <- alpha g_i - alpha beta w_i D
 *   weights: softmax derivative, d s_i = w_i (d w_i - sum_k w_k d w_k)
 *   scores:  a slot score is the sum of its factor scores <x^(f), C_f[i_f]>, so d x^(f) += d s C_f[i_f] and
 *            d C_f[i_f] += d s x^(f) (rounding of the float32 scores is taken as exact: it has no derivative).
 * After the first token G is the gradient of the bank before the call. Every sum is fp64 in a fixed order.
 * exact = 1 keeps the bank states in fp64 (no rounding to the bank dtype): the smooth function that the finite-
 * difference pins differentiate. exact = 0 rounds them after every token exactly as oracle_write_read does.
 * grad_bank_bf16 = 1 accumulates the bank gradient in bfloat16, the bank dtype of a bfloat16 bank ([CL] 2.0.0,
 * "Deterministic": float32 accumulation of the bank gradient, grad_bank_fp32, is the opt-in; the default keeps it in
 * the bank dtype): every update of G (the read's and the write's) is rounded to bfloat16 (nearest, ties to even).
 *
 * Error bounds (optional, for comparing another evaluation of this backward with it). For an evaluation that
 *   (i)  reads pre-write rows P and read rows M[R_j] within eps_row * (that row's largest magnitude) of these, plus
 *        q_rel * |element| + q_grp * (the largest magnitude of the element's 16-column group) for rows it reads
 *        from a rounded or quantized snapshot (a rounding that falls the other way: one bfloat16 spacing is at most
 *        2^-7 of the element; one fp8 spacing at most 2^-3 of it; one int4 step at most 2/7 of the group),
 *   (ii) has softmax weights within eps_w of these (relative), and
 *   (iii) does every other sum, product and difference in an arithmetic with unit roundoff u, in any order,
 * first-order running error analysis bounds the difference of every gradient element from this fp64 one:
 *   a sum of n terms computed in any order is off by at most gamma(n) = n u / (1 - n u) times the sum of the terms'
 *   magnitudes, plus the propagated errors of its terms; a product or difference adds u times its magnitude; and the
 *   error of every quantity carries into the quantities computed from it with the magnitude of its coefficient
 *   (the adjoint G carries its error from token to token like its value). The bound is that propagation, evaluated
 *   alongside the backward with the magnitudes of this backward's own values (first order: products of two errors
 *   are left out, and the caller allows a small relative slack for them).
 * ------------------------------------------------------------------------------------------------------------- */

/* Parameters of the error bounds: u, eps_row, eps_w, q_rel (see above). */
typedef struct {
  double u, eps_row, eps_w, q_rel, q_grp;
  double g_rel;  /* with a bfloat16-accumulated bank gradient: an update's rounding falling the other way */
} bound_par_t;

/* Largest magnitude of the 16-column snapshot group of row element c (d % 16 == 0 where it is used). */
static double group_max(const double* row, int c) {
  const int g = c - c % SNAP_GROUP;
  double m = 0.0;
  for (int k = g; k < g + SNAP_GROUP; ++k) m = fmax(m, fabs(row[k]));
  return m;
}

static inline double gam(double n, double u) { return n * u / (1.0 - n * u); }

typedef struct {
  int B, T, H, F, dk, d, W, R, bank_bf16, exact, snap_bf16; /* snap_bf16: the snapshot mode (0, 1 bf16, 2 fp8, 3 int4) */
  int gacc_bf16;  /* the bank gradient accumulated in bfloat16: every update of G rounded to bfloat16 */
  const int* widths;
  const float *wkeys, *rq, *values, *alpha, *beta, *sub, *bank, *dout, *dbank;
  int64_t bank_rows, sumn;
  double *d_wkeys, *d_rq, *d_values, *d_alpha, *d_beta, *d_sub_stream, *d_bank, *out64, *bank64;
  float* snap_out;                  /* optional [B, H, T, W, d]: the pre-write rows as the backward reads them */
  const bound_par_t* bp;            /* NULL: no error bounds */
  double *e_wkeys, *e_rq, *e_values, *e_alpha, *e_beta, *e_bank;
  double *esub_stream, *msub_stream; /* per stream and sub-key element: propagated error, sum of term magnitudes */
  int64_t* nsub_stream;             /* per stream and sub-key row: number of terms */
  int s_begin, s_end;
  int err;
} bwd_job_t;

static void score_backward(int F, const int* widths, int dk, int64_t id, double ds, const float* x, const float* sub,
                           double* dx, double* dsub) {
  int dig[ORACLE_MAX_F];
  for (int f = F - 1; f >= 0; --f) { dig[f] = (int)(id % widths[f]); id /= widths[f]; }
  int64_t off = 0;
  for (int f = 0; f < F; ++f) {
    const float* c = sub + (off + dig[f]) * dk;
    double* dc = dsub + (off + dig[f]) * dk;
    for (int e = 0; e < dk; ++e) {
      dx[(int64_t)f * dk + e] += ds * (double)c[e];
      dc[e] += ds * (double)x[(int64_t)f * dk + e];
    }
    off += widths[f];
  }
}

/* Error bound of score_backward's updates: the slot-score gradient ds (error eds) times sub-key and query values.
 * Accumulates the propagated error into ex/esub and the term magnitudes into mx/msub, and counts a term per
 * sub-key row in nsub. */
static void score_bound(int F, const int* widths, int dk, int64_t id, double ds, double eds, const float* x,
                        const float* sub, double* ex, double* mx, double* esub, double* msub, int64_t* nsub) {
  int dig[ORACLE_MAX_F];
  for (int f = F - 1; f >= 0; --f) { dig[f] = (int)(id % widths[f]); id /= widths[f]; }
  int64_t off = 0;
  for (int f = 0; f < F; ++f) {
    const int64_t srow = off + dig[f];
    const float* c = sub + srow * dk;
    for (int e = 0; e < dk; ++e) {
      const double xe = fabs((double)x[(int64_t)f * dk + e]), ce = fabs((double)c[e]);
      ex[(int64_t)f * dk + e] += eds * ce;
      mx[(int64_t)f * dk + e] += fabs(ds) * ce;
      esub[srow * dk + e] += eds * xe;
      msub[srow * dk + e] += fabs(ds) * xe;
    }
    nsub[srow] += 1;
    off += widths[f];
  }
}

static void* bwd_worker(void* arg) {
  bwd_job_t* j = (bwd_job_t*)arg;
  const int F = j->F, dk = j->dk, d = j->d, W = j->W, R = j->R, H = j->H, T = j->T;
  const int64_t rows = j->bank_rows;
  int32_t* S = (int32_t*)malloc(sizeof(int32_t) * (size_t)T * W);
  int32_t* Rd = (int32_t*)malloc(sizeof(int32_t) * (size_t)T * R);
  float* sc = (float*)malloc(sizeof(float) * (size_t)(W > R ? W : R));
  double* w = (double*)malloc(sizeof(double) * (size_t)T * W);
  double* rho = (double*)malloc(sizeof(double) * (size_t)T * R);
  double* P = (double*)malloc(sizeof(double) * (size_t)T * W * d);
  double* Vr = (double*)malloc(sizeof(double) * (size_t)T * R * d);
  double* rr = (double*)malloc(sizeof(double) * (size_t)T * d);
  double* del = (double*)malloc(sizeof(double) * (size_t)T * d);
  double* M = (double*)malloc(sizeof(double) * (size_t)rows * d);
  double* G = (double*)malloc(sizeof(double) * (size_t)rows * d);
  double* g = (double*)malloc(sizeof(double) * (size_t)W * d);
  double* D = (double*)malloc(sizeof(double) * (size_t)d);
  double* dw = (double*)malloc(sizeof(double) * (size_t)(W > R ? W : R));
  unsigned char* later = (unsigned char*)malloc((size_t)rows);
  /* error-bound state (bound mode only): EG the bound on the adjoint bank, the rest per token */
  const bound_par_t* bp = j->bp;
  const int KM = W > R ? W : R;
  double* qrow = (double*)malloc(sizeof(double) * (size_t)d); /* a read row as a snapshot restore left it */
  double *EG = NULL, *Eg = NULL, *Er = NULL, *Mr = NULL, *Edl = NULL, *ED = NULL, *Edw = NULL, *Ex = NULL;
  double* Mx = NULL;
  if (bp) {
    Mr = (double*)malloc(sizeof(double) * (size_t)d);
    EG = (double*)malloc(sizeof(double) * (size_t)rows * d);
    Eg = (double*)malloc(sizeof(double) * (size_t)W * d);
    Er = (double*)malloc(sizeof(double) * (size_t)d);
    Edl = (double*)malloc(sizeof(double) * (size_t)d);
    ED = (double*)malloc(sizeof(double) * (size_t)d);
    Edw = (double*)malloc(sizeof(double) * (size_t)KM);
    Ex = (double*)malloc(sizeof(double) * (size_t)F * dk);
    Mx = (double*)malloc(sizeof(double) * (size_t)F * dk);
  }
  if (!S || !Rd || !sc || !w || !rho || !P || !Vr || !rr || !del || !M || !G || !g || !D || !dw || !later || !qrow ||
      (bp && (!EG || !Eg || !Er || !Mr || !Edl || !ED || !Edw || !Ex || !Mx))) {
    j->err = 1;
    goto done;
  }
  for (int st = j->s_begin; st < j->s_end; ++st) {
    const int b = st / H, h = st % H;
    const float* sub = j->sub + (int64_t)h * j->sumn * dk;
    double* dsub = j->d_sub_stream + (int64_t)st * j->sumn * dk;
    for (int64_t i = 0; i < rows * d; ++i) M[i] = (double)j->bank[(int64_t)st * rows * d + i];
    /* forward, keeping what the backward reads */
    for (int t = 0; t < T; ++t) {
      const int64_t row = ((int64_t)b * T + t) * H + h;
      int32_t* St = S + (int64_t)t * W;
      int32_t* Rt = Rd + (int64_t)t * R;
      if (oracle_topk_one(F, j->widths, dk, j->wkeys + row * F * dk, sub, W, St, sc) != 0) { j->err = 1; goto done; }
      softmax64(W, sc, w + (int64_t)t * W);
      if (oracle_topk_one(F, j->widths, dk, j->rq + row * F * dk, sub, R, Rt, sc) != 0) { j->err = 1; goto done; }
      softmax64(R, sc, rho + (int64_t)t * R);
      const double a = j->alpha[row], be = j->beta[row];
      const float* v = j->values + row * d;
      double* r = rr + (int64_t)t * d;
      double* dl = del + (int64_t)t * d;
      for (int c = 0; c < d; ++c) r[c] = 0.0;
      for (int i = 0; i < W; ++i) {
        const double* m = M + (int64_t)St[i] * d;
        double* p = P + ((int64_t)t * W + i) * d;
        for (int c = 0; c < d; ++c) { p[c] = m[c]; r[c] += w[(int64_t)t * W + i] * m[c]; }
      }
      for (int c = 0; c < d; ++c) dl[c] = be * ((double)v[c] - a * r[c]);
      for (int i = 0; i < W; ++i) {
        double* m = M + (int64_t)St[i] * d;
        const double wi = w[(int64_t)t * W + i];
        for (int c = 0; c < d; ++c) {
          const double x = a * m[c] + wi * dl[c];
          m[c] = j->exact ? x : (double)round_to(x, j->bank_bf16);
        }
      }
      for (int i = 0; i < R; ++i) {
        const double* m = M + (int64_t)Rt[i] * d;
        double* q = Vr + ((int64_t)t * R + i) * d;
        for (int c = 0; c < d; ++c) q[c] = m[c];
      }
      if (j->out64) {
        double* o = j->out64 + row * d;
        for (int c = 0; c < d; ++c) o[c] = 0.0;
        for (int i = 0; i < R; ++i)
          for (int c = 0; c < d; ++c) o[c] += rho[(int64_t)t * R + i] * Vr[((int64_t)t * R + i) * d + c];
      }
    }
    if (j->bank64)
      for (int64_t i = 0; i < rows * d; ++i) j->bank64[(int64_t)st * rows * d + i] = M[i];
    /* bfloat16 / fp8 / int4 snapshot (CHANGELOG 2.0.0, "New"): the backward sees every pre-write row as the snapshot
     * stores it, and r and delta rebuilt from those rows; a row read at token t whose slot a later token writes was
     * restored in place from such a row, so it is stored that way too (marked in `later` as the sweep goes back) */
    if (j->snap_bf16) {
      for (int64_t i = 0; i < (int64_t)T * W; ++i) snap_row(P + i * d, P + i * d, d, j->snap_bf16);
      for (int t = 0; t < T; ++t) {
        const int64_t row = ((int64_t)b * T + t) * H + h;
        const double a = j->alpha[row], be = j->beta[row];
        const float* v = j->values + row * d;
        double* r = rr + (int64_t)t * d;
        double* dl = del + (int64_t)t * d;
        for (int c = 0; c < d; ++c) {
          double acc = 0.0;
          for (int i = 0; i < W; ++i) acc += w[(int64_t)t * W + i] * P[((int64_t)t * W + i) * d + c];
          r[c] = acc;
          dl[c] = be * ((double)v[c] - a * acc);
        }
      }
    }
    if (j->snap_out)
      for (int64_t i = 0; i < (int64_t)T * W * d; ++i) j->snap_out[(int64_t)st * T * W * d + i] = (float)P[i];
    for (int64_t i = 0; i < rows; ++i) later[i] = 0;
    /* reverse sweep */
    for (int64_t i = 0; i < rows * d; ++i) G[i] = j->dbank ? (double)j->dbank[(int64_t)st * rows * d + i] : 0.0;
    if (bp) for (int64_t i = 0; i < rows * d; ++i) EG[i] = 0.0;
    double* esub = bp ? j->esub_stream + (int64_t)st * j->sumn * dk : NULL;
    double* msub = bp ? j->msub_stream + (int64_t)st * j->sumn * dk : NULL;
    int64_t* nsub = bp ? j->nsub_stream + (int64_t)st * j->sumn : NULL;
    for (int t = T - 1; t >= 0; --t) {
      const int64_t row = ((int64_t)b * T + t) * H + h;
      const int32_t* St = S + (int64_t)t * W;
      const int32_t* Rt = Rd + (int64_t)t * R;
      const double* wt = w + (int64_t)t * W;
      const double* rt = rho + (int64_t)t * R;
      const float* dout = j->dout + row * d;
      const double a = j->alpha[row], be = j->beta[row];
      const float* v = j->values + row * d;
      const double* r = rr + (int64_t)t * d;
      const double* dl = del + (int64_t)t * d;
      /* the read */
      double sum = 0.0;
      for (int i = 0; i < R; ++i) {
        const int rounded = j->snap_bf16 && later[Rt[i]];
        const double* q = Vr + ((int64_t)t * R + i) * d;
        if (rounded) { /* the row as the restore left it */
          snap_row(q, qrow, d, j->snap_bf16);
          q = qrow;
        }
        double acc = 0.0;
        for (int c = 0; c < d; ++c) acc += (double)dout[c] * q[c];
        dw[i] = acc;
        double* Gr = G + (int64_t)Rt[i] * d;
        if (bp) { /* d rho_i from the read row (error eps_row of its largest magnitude, plus q_rel if rounded) */
          const double u = bp->u;
          double vmax = 0.0, e = 0.0, m = 0.0;
          for (int c = 0; c < d; ++c) vmax = fmax(vmax, fabs(q[c]));
          double* EGr = EG + (int64_t)Rt[i] * d;
          for (int c = 0; c < d; ++c) {
            const double qc = fabs(q[c]);
            const double ev = bp->eps_row * vmax;
            const double eq = ev + (rounded ? bp->q_rel * (qc + ev) + bp->q_grp * (group_max(q, c) + ev) : 0.0);
            const double go = fabs((double)dout[c]);
            e += go * eq;
            m += go * qc;
            EGr[c] += go * bp->eps_w * rt[i] + gam(2, u) * (fabs(Gr[c]) + rt[i] * go); /* G += rho dout */
          }
          Edw[i] = e + gam(d, u) * m;
          if (j->gacc_bf16) /* a bfloat16 rounding of the updated entry, which may fall the other way */
            for (int c = 0; c < d; ++c) EGr[c] += bp->g_rel * (fabs(Gr[c] + rt[i] * (double)dout[c]) + EGr[c]);
        }
        for (int c = 0; c < d; ++c) Gr[c] += rt[i] * (double)dout[c];
        if (j->gacc_bf16)
          for (int c = 0; c < d; ++c) Gr[c] = (double)round_to(Gr[c], 1);
      }
      for (int i = 0; i < R; ++i) sum += rt[i] * dw[i];
      for (int i = 0; i < R; ++i)
        score_backward(F, j->widths, dk, Rt[i], rt[i] * (dw[i] - sum), j->rq + row * F * dk, sub,
                       j->d_rq + row * F * dk, dsub);
      if (bp) { /* softmax derivative and the read query / sub-key updates */
        const double u = bp->u;
        double es = 0.0, ms = 0.0;
        for (int i = 0; i < R; ++i) { es += rt[i] * Edw[i] + fabs(dw[i]) * bp->eps_w * rt[i]; ms += rt[i] * fabs(dw[i]); }
        es += gam(R + 1, u) * ms;
        for (int e = 0; e < F * dk; ++e) Ex[e] = Mx[e] = 0.0;
        for (int i = 0; i < R; ++i) {
          const double ds = rt[i] * (dw[i] - sum);
          const double eds = rt[i] * (Edw[i] + es) + bp->eps_w * rt[i] * fabs(dw[i] - sum) +
                             gam(2, u) * rt[i] * (fabs(dw[i]) + fabs(sum));
          score_bound(F, j->widths, dk, Rt[i], ds, eds, j->rq + row * F * dk, sub, Ex, Mx, esub, msub, nsub);
        }
        for (int e = 0; e < F * dk; ++e) j->e_rq[row * F * dk + e] = Ex[e] + gam(R + 1, u) * Mx[e];
      }
      /* the write */
      for (int i = 0; i < W; ++i)
        for (int c = 0; c < d; ++c) g[(int64_t)i * d + c] = G[(int64_t)St[i] * d + c];
      for (int c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int i = 0; i < W; ++i) acc += wt[i] * g[(int64_t)i * d + c];
        D[c] = acc;
      }
      double dbe = 0.0, dal = 0.0, rD = 0.0;
      for (int c = 0; c < d; ++c) {
        j->d_values[row * d + c] = be * D[c];
        dbe += D[c] * ((double)v[c] - a * r[c]);
        rD += D[c] * r[c];
      }
      for (int i = 0; i < W; ++i) {
        const double* p = P + ((int64_t)t * W + i) * d;
        const double* gi = g + (int64_t)i * d;
        double gp = 0.0, gd = 0.0, Dp = 0.0;
        for (int c = 0; c < d; ++c) { gp += gi[c] * p[c]; gd += gi[c] * dl[c]; Dp += D[c] * p[c]; }
        dal += gp;
        dw[i] = gd - a * be * Dp;
      }
      dal -= be * rD;
      j->d_alpha[row] = dal;
      j->d_beta[row] = dbe;
      if (bp) { /* bounds of r, delta, D, d values, d beta, d alpha, d w_i; then of the adjoint update below */
        const double u = bp->u, qP = j->snap_bf16 ? bp->q_rel : 0.0, qG = j->snap_bf16 ? bp->q_grp : 0.0;
        /* r = sum_i w_i P_i (the rows within eps_row of their largest magnitude, plus qP if rounded) */
        for (int c = 0; c < d; ++c) Er[c] = Mr[c] = 0.0;
        for (int i = 0; i < W; ++i) {
          const double* p = P + ((int64_t)t * W + i) * d;
          double pmax = 0.0;
          for (int c = 0; c < d; ++c) pmax = fmax(pmax, fabs(p[c]));
          for (int c = 0; c < d; ++c) {
            const double ev = bp->eps_row * pmax;
            const double ep = ev + qP * (fabs(p[c]) + ev) + qG * (group_max(p, c) + ev);
            Er[c] += wt[i] * ep + fabs(p[c]) * bp->eps_w * wt[i];
            Mr[c] += wt[i] * fabs(p[c]);
          }
        }
        /* delta = beta (v - alpha r) */
        for (int c = 0; c < d; ++c) {
          Er[c] += gam(W + 1, u) * Mr[c];
          Edl[c] = be * a * Er[c] + gam(3, u) * be * (fabs((double)v[c]) + a * fabs(r[c]));
        }
        for (int c = 0; c < d; ++c) {
          double e = 0.0, m = 0.0;
          for (int i = 0; i < W; ++i) {
            Eg[(int64_t)i * d + c] = EG[(int64_t)St[i] * d + c];
            e += wt[i] * Eg[(int64_t)i * d + c] + fabs(g[(int64_t)i * d + c]) * bp->eps_w * wt[i];
            m += wt[i] * fabs(g[(int64_t)i * d + c]);
          }
          ED[c] = e + gam(W + 1, u) * m;
          j->e_values[row * d + c] = be * ED[c] + u * be * fabs(D[c]);
        }
        double ebe = 0.0, mbe = 0.0, eal = 0.0, mal = 0.0;
        for (int c = 0; c < d; ++c) {
          const double y = (double)v[c] - a * r[c];
          const double ey = a * Er[c] + gam(2, u) * (fabs((double)v[c]) + a * fabs(r[c]));
          ebe += fabs(D[c]) * ey + fabs(y) * ED[c];
          mbe += fabs(D[c] * y);
          eal += be * (fabs(D[c]) * Er[c] + fabs(r[c]) * ED[c]);
          mal += be * fabs(D[c] * r[c]);
        }
        for (int i = 0; i < W; ++i) {
          const double* p = P + ((int64_t)t * W + i) * d;
          const double* gi = g + (int64_t)i * d;
          const double* egi = Eg + (int64_t)i * d;
          double pmax = 0.0;
          for (int c = 0; c < d; ++c) pmax = fmax(pmax, fabs(p[c]));
          double ew = 0.0, mw = 0.0;
          for (int c = 0; c < d; ++c) {
            const double ev = bp->eps_row * pmax;
            const double ep = ev + qP * (fabs(p[c]) + ev) + qG * (group_max(p, c) + ev);
            eal += fabs(gi[c]) * ep + fabs(p[c]) * egi[c];
            mal += fabs(gi[c] * p[c]);
            ew += fabs(gi[c]) * Edl[c] + fabs(dl[c]) * egi[c] + a * be * (fabs(D[c]) * ep + fabs(p[c]) * ED[c]);
            mw += fabs(gi[c] * dl[c]) + a * be * fabs(D[c] * p[c]);
          }
          Edw[i] = ew + gam(d + 3, u) * mw;
        }
        j->e_beta[row] = ebe + gam(d + 1, u) * mbe;
        j->e_alpha[row] = eal + gam((double)W * d + 2, u) * mal;
      }
      for (int i = 0; i < W; ++i) {
        double* Gw = G + (int64_t)St[i] * d;
        const double* gi = g + (int64_t)i * d;
        for (int c = 0; c < d; ++c) Gw[c] = a * gi[c] - a * be * wt[i] * D[c];
        if (bp) {
          double* EGw = EG + (int64_t)St[i] * d;
          const double* egi = Eg + (int64_t)i * d;
          for (int c = 0; c < d; ++c) {
            EGw[c] = a * egi[c] + a * be * (wt[i] * ED[c] + fabs(D[c]) * bp->eps_w * wt[i]) +
                     gam(4, bp->u) * (a * fabs(gi[c]) + a * be * wt[i] * fabs(D[c]));
            if (j->gacc_bf16) EGw[c] += bp->g_rel * (fabs(Gw[c]) + EGw[c]);
          }
        }
        if (j->gacc_bf16)
          for (int c = 0; c < d; ++c) Gw[c] = (double)round_to(Gw[c], 1);
        later[St[i]] = 1;
      }
      sum = 0.0;
      for (int i = 0; i < W; ++i) sum += wt[i] * dw[i];
      for (int i = 0; i < W; ++i)
        score_backward(F, j->widths, dk, St[i], wt[i] * (dw[i] - sum), j->wkeys + row * F * dk, sub,
                       j->d_wkeys + row * F * dk, dsub);
      if (bp) { /* softmax derivative and the write key / sub-key updates */
        const double u = bp->u;
        double es = 0.0, ms = 0.0;
        for (int i = 0; i < W; ++i) { es += wt[i] * Edw[i] + fabs(dw[i]) * bp->eps_w * wt[i]; ms += wt[i] * fabs(dw[i]); }
        es += gam(W + 1, u) * ms;
        for (int e = 0; e < F * dk; ++e) Ex[e] = Mx[e] = 0.0;
        for (int i = 0; i < W; ++i) {
          const double ds = wt[i] * (dw[i] - sum);
          const double eds = wt[i] * (Edw[i] + es) + bp->eps_w * wt[i] * fabs(dw[i] - sum) +
                             gam(2, u) * wt[i] * (fabs(dw[i]) + fabs(sum));
          score_bound(F, j->widths, dk, St[i], ds, eds, j->wkeys + row * F * dk, sub, Ex, Mx, esub, msub, nsub);
        }
        for (int e = 0; e < F * dk; ++e) j->e_wkeys[row * F * dk + e] = Ex[e] + gam(W + 1, u) * Mx[e];
      }
    }
    for (int64_t i = 0; i < rows * d; ++i) j->d_bank[(int64_t)st * rows * d + i] = G[i];
    if (bp) for (int64_t i = 0; i < rows * d; ++i) j->e_bank[(int64_t)st * rows * d + i] = EG[i];
  }
done:
  free(S); free(Rd); free(sc); free(w); free(rho); free(P); free(Vr); free(rr); free(del); free(M); free(G);
  free(g); free(D); free(dw); free(later);
  free(EG); free(Eg); free(Er); free(Mr); free(Edl); free(ED); free(Edw); free(Ex); free(Mx); free(qrow);
  return NULL;
}

/* Inputs as for oracle_write_read (bank = the bank BEFORE the call, not modified), plus
 *   dout  [B, T, H, d]            gradient of the loss with respect to out
 *   dbank [B, H, bank_rows, d]    gradient with respect to the bank after the call (NULL = zero)
 * Outputs (fp64, zero-initialised here): d_wkeys, d_rq [B, T, H, F*dk], d_values [B, T, H, d], d_alpha, d_beta
 * [B, T, H], d_subkeys [H, sum n_f, dk] (summed over the batch in order b = 0, 1, ...), d_bank [B, H, bank_rows, d]
 * (the gradient with respect to the bank before the call); optional out64 [B, T, H, d] and bank64 (the forward's
 * outputs in fp64, unrounded, NULL to skip). Returns 0 or -1. */
static int backward_impl(int B, int T, int H, int F, const int* widths, int dk, int d, int W, int R, int bank_bf16,
                         int exact, int snap_bf16, int gacc_bf16, const float* wkeys, const float* rq, const float* values,
                         const float* alpha, const float* beta, const float* subkeys, const float* bank,
                         int64_t bank_rows, const float* dout, const float* dbank, double* d_wkeys, double* d_rq,
                         double* d_values, double* d_alpha, double* d_beta, double* d_subkeys, double* d_bank,
                         double* out64, double* bank64, float* snap_out, const bound_par_t* bp, double* e_wkeys,
                         double* e_rq, double* e_values, double* e_alpha, double* e_beta, double* e_subkeys,
                         double* e_bank, int nthreads) {
  int64_t sumn = 0, N = 1;
  for (int f = 0; f < F; ++f) { sumn += widths[f]; N *= widths[f]; }
  if (F < 1 || F > ORACLE_MAX_F || W < 1 || R < 1 || W > N || R > N || bank_rows < N) return -1;
  if (snap_bf16 < 0 || snap_bf16 > 3 || (snap_bf16 >= 2 && d % SNAP_GROUP != 0)) return -1;
  const int streams = B * H;
  memset(d_wkeys, 0, sizeof(double) * (size_t)B * T * H * F * dk);
  memset(d_rq, 0, sizeof(double) * (size_t)B * T * H * F * dk);
  memset(d_subkeys, 0, sizeof(double) * (size_t)H * sumn * dk);
  double* dsub_stream = (double*)calloc((size_t)(streams > 0 ? streams : 1) * sumn * dk, sizeof(double));
  if (!dsub_stream) return -1;
  double *esub = NULL, *msub = NULL;
  int64_t* nsub = NULL;
  if (bp) {
    esub = (double*)calloc((size_t)(streams > 0 ? streams : 1) * sumn * dk, sizeof(double));
    msub = (double*)calloc((size_t)(streams > 0 ? streams : 1) * sumn * dk, sizeof(double));
    nsub = (int64_t*)calloc((size_t)(streams > 0 ? streams : 1) * sumn, sizeof(int64_t));
    if (!esub || !msub || !nsub) { free(dsub_stream); free(esub); free(msub); free(nsub); return -1; }
  }
  if (nthreads < 1) nthreads = 1;
  if (nthreads > streams) nthreads = streams > 0 ? streams : 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  int started[256];
  bwd_job_t jobs[256];
  int err = 0;
  for (int i = 0; i < nthreads; ++i) {
    bwd_job_t* j = &jobs[i];
    j->B = B; j->T = T; j->H = H; j->F = F; j->dk = dk; j->d = d; j->W = W; j->R = R;
    j->bank_bf16 = bank_bf16; j->exact = exact; j->snap_bf16 = snap_bf16; j->gacc_bf16 = gacc_bf16; j->widths = widths; j->wkeys = wkeys; j->rq = rq;
    j->values = values; j->alpha = alpha; j->beta = beta; j->sub = subkeys; j->bank = bank; j->dout = dout;
    j->dbank = dbank; j->bank_rows = bank_rows; j->sumn = sumn; j->d_wkeys = d_wkeys; j->d_rq = d_rq;
    j->d_values = d_values; j->d_alpha = d_alpha; j->d_beta = d_beta; j->d_sub_stream = dsub_stream;
    j->d_bank = d_bank; j->out64 = out64; j->bank64 = bank64; j->err = 0;
    j->snap_out = snap_out; j->bp = bp; j->e_wkeys = e_wkeys; j->e_rq = e_rq; j->e_values = e_values;
    j->e_alpha = e_alpha; j->e_beta = e_beta; j->e_bank = e_bank; j->esub_stream = esub; j->msub_stream = msub;
    j->nsub_stream = nsub;
    j->s_begin = (int)((int64_t)streams * i / nthreads);
    j->s_end = (int)((int64_t)streams * (i + 1) / nthreads);
    started[i] = pthread_create(&th[i], NULL, bwd_worker, j) == 0;
    if (!started[i]) bwd_worker(j);
  }
  for (int i = 0; i < nthreads; ++i) { if (started[i]) pthread_join(th[i], NULL); err |= jobs[i].err; }
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      const double* src = dsub_stream + ((int64_t)b * H + h) * sumn * dk;
      double* dst = d_subkeys + (int64_t)h * sumn * dk;
      for (int64_t i = 0; i < sumn * dk; ++i) dst[i] += src[i];
    }
  if (bp) { /* sub-key gradients: the sum over every term of every stream of the head, in any order */
    for (int h = 0; h < H; ++h)
      for (int64_t rr = 0; rr < sumn; ++rr) {
        int64_t n = 0;
        for (int b = 0; b < B; ++b) n += nsub[((int64_t)b * H + h) * sumn + rr];
        for (int e = 0; e < dk; ++e) {
          double ee = 0.0, mm = 0.0;
          for (int b = 0; b < B; ++b) {
            ee += esub[(((int64_t)b * H + h) * sumn + rr) * dk + e];
            mm += msub[(((int64_t)b * H + h) * sumn + rr) * dk + e];
          }
          e_subkeys[((int64_t)h * sumn + rr) * dk + e] = ee + gam((double)n + 1, bp->u) * mm;
        }
      }
  }
  free(dsub_stream); free(esub); free(msub); free(nsub);
  return err ? -1 : 0;
}

int oracle_write_read_backward(int B, int T, int H, int F, const int* widths, int dk, int d, int W, int R,
                               int bank_bf16, int exact, int snap_bf16, int grad_bank_bf16, const float* wkeys,
                               const float* rq,
                               const float* values,
                               const float* alpha, const float* beta, const float* subkeys, const float* bank,
                               int64_t bank_rows, const float* dout, const float* dbank, double* d_wkeys,
                               double* d_rq, double* d_values, double* d_alpha, double* d_beta, double* d_subkeys,
                               double* d_bank, double* out64, double* bank64, int nthreads) {
  return backward_impl(B, T, H, F, widths, dk, d, W, R, bank_bf16, exact, snap_bf16, grad_bank_bf16, wkeys, rq, values,
                       alpha, beta, subkeys, bank, bank_rows, dout, dbank, d_wkeys, d_rq, d_values, d_alpha, d_beta,
                       d_subkeys, d_bank, out64, bank64, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                       nthreads);
}

/* oracle_write_read_backward with error bounds (see the comment above bound_par_t): par = {u, eps_row, eps_w,
 * q_rel, q_grp}; e_* receive, per gradient element, the bound on the difference from this backward of an evaluation
 * that meets the stated conditions (same shapes as the gradients; fp64). snap_out (optional, float32
 * [B, H, T, W, d]) receives the pre-write rows of every write event as the backward reads them (rounded to
 * bfloat16 with snap_bf16). The gradients and the other outputs are those of oracle_write_read_backward. */
int oracle_write_read_backward_bounds(int B, int T, int H, int F, const int* widths, int dk, int d, int W, int R,
                                      int bank_bf16, int snap_bf16, int grad_bank_bf16, const float* wkeys,
                                      const float* rq,
                                      const float* values, const float* alpha, const float* beta,
                                      const float* subkeys, const float* bank, int64_t bank_rows, const float* dout,
                                      const float* dbank, double* d_wkeys, double* d_rq, double* d_values,
                                      double* d_alpha, double* d_beta, double* d_subkeys, double* d_bank,
                                      double* out64, double* bank64, float* snap_out, const double* par,
                                      double* e_wkeys, double* e_rq, double* e_values, double* e_alpha,
                                      double* e_beta, double* e_subkeys, double* e_bank, int nthreads) {
  if (!par || !e_wkeys || !e_rq || !e_values || !e_alpha || !e_beta || !e_subkeys || !e_bank) return -1;
  bound_par_t bp = {par[0], par[1], par[2], par[3], par[4], par[5]};
  return backward_impl(B, T, H, F, widths, dk, d, W, R, bank_bf16, 0, snap_bf16, grad_bank_bf16, wkeys, rq, values,
                       alpha, beta,
                       subkeys, bank, bank_rows, dout, dbank, d_wkeys, d_rq, d_values, d_alpha, d_beta, d_subkeys,
                       d_bank, out64, bank64, snap_out, &bp, e_wkeys, e_rq, e_values, e_alpha, e_beta, e_subkeys,
                       e_bank, nthreads);
}

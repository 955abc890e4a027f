/*
 * Driver for the AddressSanitizer / UndefinedBehaviorSanitizer build of the
 * CPU oracle (oracle/tc_oracle.c), run by tests/test_sanitizers.py on the
 * host only.  It calls every oracle entry point on small seeded inputs that
 * cover the edge cases of the recurrence (no eviction, one eviction, W = 1,
 * W >= T, T = 1, a ring that wraps) and checks that every output is finite;
 * the sanitizers check every memory access and every arithmetic operation
 * on the way.  Exit status 0 and the line "ok" on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void tco_forward(int B, int H, int T, int D, int W, double tau, const double* q, const double* k, const double* v,
                 const double* lam, const double* eta, const double* gate, double* y, double* A_final, double* lse);
void tco_decode_step(int S, int H, int D, int W, double tau, const double* q, const double* k, const double* v,
                     double* k_ring, double* v_ring, double* A, int64_t* pos, const double* lam, const double* eta,
                     const double* gate, double* y);
void tco_backward(int B, int H, int T, int D, int W, double tau, const double* q, const double* k, const double* v,
                  const double* dy, const double* lam, const double* eta, const double* gate, double* dq, double* dk,
                  double* dv, double* dlam, double* deta, double* dgate);
void tco_forward_chunk_mean(int B, int H, int T, int D, int W, int C, double tau, const double* q, const double* k,
                            const double* v, const double* lam, const double* eta, const double* gate, double* y,
                            double* A_final, double* lse);
void tco_memory_f32_sequential(int T, int D, int W, float lam, float eta, const float* q, const float* k,
                               const float* v, float* m, float* A_final);
void tco_memory_f32_chunked(int T, int D, int W, int C, float lam, float eta, const float* q, const float* k,
                            const float* v, float* m, float* A_final);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double urand(void) { /* xorshift64*, uniform in [-1, 1) */
  rng ^= rng >> 12;
  rng ^= rng << 25;
  rng ^= rng >> 27;
  return (double)((rng * 0x2545F4914F6CDD1Dull) >> 11) / (double)(1ull << 52) - 1.0;
}
static double* dalloc(size_t n, int fill) {
  double* p = (double*)malloc(sizeof(double) * (n ? n : 1));
  for (size_t i = 0; i < n; ++i) p[i] = fill ? urand() : 0.0;
  return p;
}
static int finite_all(const double* p, size_t n) {
  for (size_t i = 0; i < n; ++i)
    if (!isfinite(p[i])) return 0;
  return 1;
}

static int check_forward_backward(int B, int H, int T, int D, int W) {
  const size_t n = (size_t)B * H * T * D, nh = (size_t)H;
  double *q = dalloc(n, 1), *k = dalloc(n, 1), *v = dalloc(n, 1), *dy = dalloc(n, 1);
  double *lam = dalloc(nh, 0), *eta = dalloc(nh, 0), *gate = dalloc(nh, 1);
  for (size_t h = 0; h < nh; ++h) {
    lam[h] = h % 3 == 0 ? 0.0 : (h % 3 == 1 ? 1.0 : 0.9);
    eta[h] = 0.5;
  }
  double *y = dalloc(n, 0), *A = dalloc((size_t)B * H * D * D, 0), *lse = dalloc((size_t)B * H * T, 0);
  double *dq = dalloc(n, 0), *dk = dalloc(n, 0), *dv = dalloc(n, 0);
  double *dl = dalloc(nh, 0), *de = dalloc(nh, 0), *dg = dalloc(nh, 0);
  tco_forward(B, H, T, D, W, 1.0 / sqrt((double)D), q, k, v, lam, eta, gate, y, A, lse);
  tco_backward(B, H, T, D, W, 1.0 / sqrt((double)D), q, k, v, dy, lam, eta, gate, dq, dk, dv, dl, de, dg);
  int ok = 1;
  for (int C = 1; C <= 5; C += 2) {  /* the chunk-mean shortcut, incomplete last chunks included */
    tco_forward_chunk_mean(B, H, T, D, W, C, 0.5, q, k, v, lam, eta, gate, dq, A, lse);
    ok = ok && finite_all(dq, n) && finite_all(A, (size_t)B * H * D * D);
  }
  tco_backward(B, H, T, D, W, 1.0 / sqrt((double)D), q, k, v, dy, lam, eta, gate, dq, dk, dv, dl, de, dg);
  ok = ok && finite_all(y, n) && finite_all(A, (size_t)B * H * D * D) && finite_all(lse, (size_t)B * H * T) &&
           finite_all(dq, n) && finite_all(dk, n) && finite_all(dv, n) && finite_all(dl, nh) &&
           finite_all(de, nh) && finite_all(dg, nh);
  free(q); free(k); free(v); free(dy); free(lam); free(eta); free(gate); free(y); free(A); free(lse);
  free(dq); free(dk); free(dv); free(dl); free(de); free(dg);
  return ok;
}

static int check_decode(int S, int H, int D, int W, int steps) {
  const size_t nt = (size_t)S * H * D, nr = (size_t)S * H * W * D;
  double *kr = dalloc(nr, 0), *vr = dalloc(nr, 0), *A = dalloc((size_t)S * H * D * D, 0), *y = dalloc(nt, 0);
  double *lam = dalloc(H, 0), *eta = dalloc(H, 0), *gate = dalloc(H, 1);
  int64_t* pos = (int64_t*)calloc((size_t)S, sizeof(int64_t));
  for (int h = 0; h < H; ++h) {
    lam[h] = 0.8;
    eta[h] = 0.3;
  }
  for (int s = 0; s < S; ++s) pos[s] = s * 3;  /* streams at different positions */
  int ok = 1;
  for (int t = 0; t < steps && ok; ++t) {
    double *q = dalloc(nt, 1), *k = dalloc(nt, 1), *v = dalloc(nt, 1);
    tco_decode_step(S, H, D, W, 0.25, q, k, v, kr, vr, A, pos, lam, eta, gate, y);
    ok = finite_all(y, nt);
    free(q); free(k); free(v);
  }
  ok = ok && finite_all(A, (size_t)S * H * D * D);
  free(kr); free(vr); free(A); free(y); free(lam); free(eta); free(gate); free(pos);
  return ok;
}

static int check_memory_models(int T, int D, int W, int C) {
  const size_t n = (size_t)T * D;
  float *q = (float*)malloc(sizeof(float) * n), *k = (float*)malloc(sizeof(float) * n),
        *v = (float*)malloc(sizeof(float) * n), *m1 = (float*)malloc(sizeof(float) * n),
        *m2 = (float*)malloc(sizeof(float) * n);
  float *A1 = (float*)malloc(sizeof(float) * D * D), *A2 = (float*)malloc(sizeof(float) * D * D);
  for (size_t i = 0; i < n; ++i) {
    q[i] = (float)urand();
    k[i] = (float)urand();
    v[i] = (float)urand();
  }
  tco_memory_f32_sequential(T, D, W, 0.95f, 0.5f, q, k, v, m1, A1);
  tco_memory_f32_chunked(T, D, W, C, 0.95f, 0.5f, q, k, v, m2, A2);
  int ok = 1;
  for (size_t i = 0; i < n; ++i) ok = ok && isfinite(m1[i]) && isfinite(m2[i]);
  free(q); free(k); free(v); free(m1); free(m2); free(A1); free(A2);
  return ok;
}

int main(void) {
  const int fb[][5] = {{1, 1, 64, 16, 8}, {2, 3, 37, 8, 5}, {1, 2, 10, 4, 1}, {1, 1, 9, 4, 20},
                       {1, 1, 1, 4, 1},   {1, 2, 33, 16, 32}};
  for (unsigned i = 0; i < sizeof(fb) / sizeof(fb[0]); ++i)
    if (!check_forward_backward(fb[i][0], fb[i][1], fb[i][2], fb[i][3], fb[i][4])) {
      printf("forward/backward case %u not finite\n", i);
      return 1;
    }
  if (!check_decode(3, 2, 8, 5, 17) || !check_decode(1, 1, 4, 1, 4)) {
    printf("decode not finite\n");
    return 1;
  }
  if (!check_memory_models(70, 8, 6, 8) || !check_memory_models(5, 4, 8, 3) || !check_memory_models(40, 4, 3, 7)) {
    printf("memory models not finite\n");
    return 1;
  }
  printf("ok\n");
  return 0;
}

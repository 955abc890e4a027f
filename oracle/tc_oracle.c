/*
 * Tensor Cache (TC) CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * This file is the slow, obviously-correct reference that the GPU library is
 * checked against.  Only tests/, the smoke check and the bench's CPU-baseline
 * leg load it.  It shares no code, header or table with the HIP path.
 *
 * Source of every formula: "Tensor Cache: Eviction-conditioned Associative
 * Memory for Transformers" (Swain, Han, Weidele, Martino, Torralba, 2026):
 *   - Section 3.1, Eq. (1): the local window K_win, V_win holds the most recent
 *     W key/value pairs; y_local = Attn(q_t, K_win, V_win) (exact causal
 *     softmax attention).
 *   - Section 3.2 and Figure 2 (one streaming step): A starts at zero; when the
 *     ring slot pos is overwritten the displaced pair (k_old, v_old) is written
 *     A <- lambda*A + eta*(k_old outer v_old) (step 3), then the new pair takes
 *     the slot (step 4), then the query reads m_t = q_t A and the output is
 *     y_t = y_local + sigma(g)*m_t (step 5).
 *   - Abstract: per-head decay lambda and write rate eta, a learned scalar
 *     gate g, all trained end to end (hence the backward pass below).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - softmax scale tau is an argument (standard choice 1/sqrt(D));
 *   - after inserting token t the window is max(0,t-W+1)..t (W tokens);
 *   - the eviction of token t-W is written before the read at step t;
 *   - nothing is written while t < W (no eviction event);
 *   - the memory read has no normaliser (the related-work section says TC
 *     uses no normaliser vector or feature map);
 *   - lambda, eta, g are taken as given values; gradients are with respect
 *     to those values.
 *
 * Arithmetic: IEEE double throughout, no fast-math, no BLAS, no intrinsics.
 * Layout: row-major, [B,H,T,D] for per-token vectors, [B,H,D,D] for A with
 * A[a][c] = sum eta*lambda^.. k[a] v[c]  (k outer v = k v^T).
 * Parallelism: OpenMP over independent (b,h) (or (stream,head)) pairs only.
 */
#include <math.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdlib.h>
#include <string.h>

static double sigmoid(double g) { return 1.0 / (1.0 + exp(-g)); }

static double dot(const double* a, const double* b, int n) {
  double s = 0.0;
  for (int i = 0; i < n; ++i) s += a[i] * b[i];
  return s;
}

/* Threads for the following calls (the CPU baseline also times one thread). */
void tco_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* Number of threads OpenMP will use (reported by the CPU baseline). */
int tco_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * One (b,h) sequence of the forward pass, literally per token
 * (Figure 2: evict -> write -> insert -> read -> fuse).
 */
static void forward_one(int T, int D, int W, double tau, const double* q,
                        const double* k, const double* v, double lam,
                        double eta, double g, double* y, double* A_out,
                        double* lse) {
  const double sg = sigmoid(g);
  double* A = (double*)calloc((size_t)D * D, sizeof(double));
  double* z = (double*)malloc(sizeof(double) * (size_t)(W > 0 ? W : 1));
  for (int t = 0; t < T; ++t) {
    const double* qt = q + (size_t)t * D;
    /* steps 2-3: token t-W leaves the window and is written into A */
    if (t >= W) {
      const double* ke = k + (size_t)(t - W) * D;
      const double* ve = v + (size_t)(t - W) * D;
      for (int a = 0; a < D; ++a)
        for (int c = 0; c < D; ++c)
          A[a * D + c] = lam * A[a * D + c] + eta * ke[a] * ve[c];
    }
    /* step 5, L1: exact softmax over the window {max(0,t-W+1) .. t} */
    int lo = t - W + 1;
    if (lo < 0) lo = 0;
    double mu = -INFINITY;
    for (int i = lo; i <= t; ++i) {
      z[i - lo] = tau * dot(qt, k + (size_t)i * D, D);
      if (z[i - lo] > mu) mu = z[i - lo];
    }
    double ell = 0.0;
    for (int i = lo; i <= t; ++i) ell += exp(z[i - lo] - mu);
    double* yt = y + (size_t)t * D;
    for (int c = 0; c < D; ++c) yt[c] = 0.0;
    for (int i = lo; i <= t; ++i) {
      const double p = exp(z[i - lo] - mu) / ell;
      const double* vi = v + (size_t)i * D;
      for (int c = 0; c < D; ++c) yt[c] += p * vi[c];
    }
    if (lse) lse[t] = mu + log(ell);
    /* step 5, L2: m_t = q_t A (no normaliser), fused through sigma(g) */
    for (int c = 0; c < D; ++c) {
      double m = 0.0;
      for (int a = 0; a < D; ++a) m += qt[a] * A[a * D + c];
      yt[c] += sg * m;
    }
  }
  if (A_out) memcpy(A_out, A, sizeof(double) * (size_t)D * D);
  free(A);
  free(z);
}

/*
 * tco_forward: y [B,H,T,D], A_final [B,H,D,D] (nullable), lse [B,H,T]
 * (nullable, natural log of the softmax normaliser of the scaled scores).
 */
void tco_forward(int B, int H, int T, int D, int W, double tau,
                 const double* q, const double* k, const double* v,
                 const double* lam, const double* eta, const double* gate,
                 double* y, double* A_final, double* lse) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int bh = 0; bh < B * H; ++bh) {
    const int h = bh % H;
    const size_t off = (size_t)bh * T * D;
    forward_one(T, D, W, tau, q + off, k + off, v + off, lam[h], eta[h],
                gate[h], y + off, A_final ? A_final + (size_t)bh * D * D : 0,
                lse ? lse + (size_t)bh * T : 0);
  }
}

/*
 * The chunk-mean shortcut that the abstract and Section 1 (contributions) and
 * Section 2 (training considerations) describe and that the parallel
 * weighted-sum scan replaces: a chunked scan that summarises each chunk of C
 * evicted pairs by its mean key and mean value and writes
 *     A <- lambda A + eta (kbar outer vbar)
 * once per chunk (lambda applied once per chunk).  The pages fix that write;
 * they do not say what a query reads between two writes.  Reading taken
 * (the inter-chunk state of a chunked scan): the evicted tokens form chunks
 * n = tokens nC .. nC+C-1 in eviction order; a query at step t >= W, whose
 * evicted token t-W lies in chunk n = (t-W)/C, reads the memory after the
 * writes of chunks 0 .. n-1; a query at t < W reads nothing.  The write of
 * chunk n is therefore made at the first step of chunk n+1, before its read,
 * and the returned A_final is the memory after every complete chunk (the
 * pairs of an incomplete last chunk are not written).  L1 is exactly as in
 * forward_one.
 */
static void chunk_mean_forward_one(int T, int D, int W, int C, double tau, const double* q, const double* k,
                                   const double* v, double lam, double eta, double g, double* y, double* A_out,
                                   double* lse) {
  const double sg = sigmoid(g);
  double* A = (double*)calloc((size_t)D * D, sizeof(double));
  double* ks = (double*)calloc((size_t)D, sizeof(double)); /* sums of the current chunk */
  double* vs = (double*)calloc((size_t)D, sizeof(double));
  double* z = (double*)malloc(sizeof(double) * (size_t)(W > 0 ? W : 1));
  for (int t = 0; t < T; ++t) {
    const double* qt = q + (size_t)t * D;
    if (t >= W) {
      const int e = t - W; /* the token leaving the window at this step */
      if (e > 0 && e % C == 0) {
        /* chunk e/C - 1 is complete: one write of its mean pair */
        for (int a = 0; a < D; ++a)
          for (int c = 0; c < D; ++c)
            A[a * D + c] = lam * A[a * D + c] + eta * (ks[a] / C) * (vs[c] / C);
        memset(ks, 0, sizeof(double) * (size_t)D);
        memset(vs, 0, sizeof(double) * (size_t)D);
      }
      for (int a = 0; a < D; ++a) {
        ks[a] += k[(size_t)e * D + a];
        vs[a] += v[(size_t)e * D + a];
      }
    }
    /* L1: exact softmax over the window {max(0,t-W+1) .. t} */
    int lo = t - W + 1;
    if (lo < 0) lo = 0;
    double mu = -INFINITY;
    for (int i = lo; i <= t; ++i) {
      z[i - lo] = tau * dot(qt, k + (size_t)i * D, D);
      if (z[i - lo] > mu) mu = z[i - lo];
    }
    double ell = 0.0;
    for (int i = lo; i <= t; ++i) ell += exp(z[i - lo] - mu);
    double* yt = y + (size_t)t * D;
    for (int c = 0; c < D; ++c) yt[c] = 0.0;
    for (int i = lo; i <= t; ++i) {
      const double p = exp(z[i - lo] - mu) / ell;
      const double* vi = v + (size_t)i * D;
      for (int c = 0; c < D; ++c) yt[c] += p * vi[c];
    }
    if (lse) lse[t] = mu + log(ell);
    /* L2: the read of the chunk writes made so far, fused through sigma(g) */
    for (int c = 0; c < D; ++c) {
      double m = 0.0;
      for (int a = 0; a < D; ++a) m += qt[a] * A[a * D + c];
      yt[c] += sg * m;
    }
  }
  if (T > W && (T - W) % C == 0) {
    /* the last chunk completed at the last step */
    for (int a = 0; a < D; ++a)
      for (int c = 0; c < D; ++c) A[a * D + c] = lam * A[a * D + c] + eta * (ks[a] / C) * (vs[c] / C);
  }
  if (A_out) memcpy(A_out, A, sizeof(double) * (size_t)D * D);
  free(A);
  free(ks);
  free(vs);
  free(z);
}

/* tco_forward_chunk_mean: the chunk-mean shortcut's forward, same layout as tco_forward. */
void tco_forward_chunk_mean(int B, int H, int T, int D, int W, int C, double tau, const double* q, const double* k,
                            const double* v, const double* lam, const double* eta, const double* gate, double* y,
                            double* A_final, double* lse) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int bh = 0; bh < B * H; ++bh) {
    const int h = bh % H;
    const size_t off = (size_t)bh * T * D;
    chunk_mean_forward_one(T, D, W, C, tau, q + off, k + off, v + off, lam[h], eta[h], gate[h], y + off,
                           A_final ? A_final + (size_t)bh * D * D : 0, lse ? lse + (size_t)bh * T : 0);
  }
}

/*
 * The delta-rule write that Figure 2 (step 3) names as the optional
 * alternative to the outer-product write.  The pages give no formula for it;
 * the related-work section traces the delta rule to the Widrow-Hoff
 * error-correcting update.  Reading taken: the evicted key first reads the
 * memory as it stands before this write, and only the error of that
 * prediction is written, with the same decay and write rate,
 *     u     = v_old - k_old A            (row vector: u[c] = v[c] - sum_a k[a] A[a][c])
 *     A    <- lambda A + eta (k_old outer u).
 * Everything else (the eviction schedule, the window, the read m_t = q_t A
 * and the gated fusion) is exactly as in forward_one.
 */
static void delta_forward_one(int T, int D, int W, double tau, const double* q, const double* k, const double* v,
                              double lam, double eta, double g, double* y, double* A_out, double* lse) {
  const double sg = sigmoid(g);
  double* A = (double*)calloc((size_t)D * D, sizeof(double));
  double* u = (double*)malloc(sizeof(double) * (size_t)D);
  double* z = (double*)malloc(sizeof(double) * (size_t)(W > 0 ? W : 1));
  for (int t = 0; t < T; ++t) {
    const double* qt = q + (size_t)t * D;
    if (t >= W) {
      const double* ke = k + (size_t)(t - W) * D;
      const double* ve = v + (size_t)(t - W) * D;
      for (int c = 0; c < D; ++c) {
        double pred = 0.0; /* what the memory returns for the evicted key */
        for (int a = 0; a < D; ++a) pred += ke[a] * A[a * D + c];
        u[c] = ve[c] - pred;
      }
      for (int a = 0; a < D; ++a)
        for (int c = 0; c < D; ++c) A[a * D + c] = lam * A[a * D + c] + eta * ke[a] * u[c];
    }
    int lo = t - W + 1;
    if (lo < 0) lo = 0;
    double mu = -INFINITY;
    for (int i = lo; i <= t; ++i) {
      z[i - lo] = tau * dot(qt, k + (size_t)i * D, D);
      if (z[i - lo] > mu) mu = z[i - lo];
    }
    double ell = 0.0;
    for (int i = lo; i <= t; ++i) ell += exp(z[i - lo] - mu);
    double* yt = y + (size_t)t * D;
    for (int c = 0; c < D; ++c) yt[c] = 0.0;
    for (int i = lo; i <= t; ++i) {
      const double p = exp(z[i - lo] - mu) / ell;
      const double* vi = v + (size_t)i * D;
      for (int c = 0; c < D; ++c) yt[c] += p * vi[c];
    }
    if (lse) lse[t] = mu + log(ell);
    for (int c = 0; c < D; ++c) {
      double m = 0.0;
      for (int a = 0; a < D; ++a) m += qt[a] * A[a * D + c];
      yt[c] += sg * m;
    }
  }
  if (A_out) memcpy(A_out, A, sizeof(double) * (size_t)D * D);
  free(A);
  free(u);
  free(z);
}

/* tco_forward_delta: the delta-rule variant's forward, same layout as tco_forward. */
void tco_forward_delta(int B, int H, int T, int D, int W, double tau, const double* q, const double* k,
                       const double* v, const double* lam, const double* eta, const double* gate, double* y,
                       double* A_final, double* lse) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int bh = 0; bh < B * H; ++bh) {
    const int h = bh % H;
    const size_t off = (size_t)bh * T * D;
    delta_forward_one(T, D, W, tau, q + off, k + off, v + off, lam[h], eta[h], gate[h], y + off,
                      A_final ? A_final + (size_t)bh * D * D : 0, lse ? lse + (size_t)bh * T : 0);
  }
}

/*
 * tco_decode_step: one streaming step (Figure 2, steps 1-5) for S streams x
 * H heads.  Ring slot of token t is t mod W; pos[s] is the index of the
 * incoming token of stream s.  While pos < W the slots pos+1..W-1 hold no
 * token and nothing is evicted.  Updates k_ring, v_ring, A, pos in place.
 */
void tco_decode_step(int S, int H, int D, int W, double tau, const double* q,
                     const double* k, const double* v, double* k_ring,
                     double* v_ring, double* A, int64_t* pos,
                     const double* lam, const double* eta, const double* gate,
                     double* y) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int sh = 0; sh < S * H; ++sh) {
    const int s = sh / H, h = sh % H;
    const int64_t t = pos[s];
    const int slot = (int)(t % W);
    const double* qt = q + (size_t)sh * D;
    const double* kt = k + (size_t)sh * D;
    const double* vt = v + (size_t)sh * D;
    double* kr = k_ring + (size_t)sh * W * D;
    double* vr = v_ring + (size_t)sh * W * D;
    double* Ash = A + (size_t)sh * D * D;
    /* steps 2-3: evict the pair in the slot, write it into A */
    if (t >= W) {
      const double* ke = kr + (size_t)slot * D;
      const double* ve = vr + (size_t)slot * D;
      for (int a = 0; a < D; ++a)
        for (int c = 0; c < D; ++c)
          Ash[a * D + c] = lam[h] * Ash[a * D + c] + eta[h] * ke[a] * ve[c];
    }
    /* step 4: insert the new pair */
    memcpy(kr + (size_t)slot * D, kt, sizeof(double) * D);
    memcpy(vr + (size_t)slot * D, vt, sizeof(double) * D);
    /* step 5: read both paths */
    const int nvalid = t + 1 < W ? (int)(t + 1) : W;
    double mu = -INFINITY;
    for (int j = 0; j < nvalid; ++j) {
      const double zj = tau * dot(qt, kr + (size_t)j * D, D);
      if (zj > mu) mu = zj;
    }
    double ell = 0.0;
    double* yt = y + (size_t)sh * D;
    for (int c = 0; c < D; ++c) yt[c] = 0.0;
    for (int j = 0; j < nvalid; ++j) {
      const double p = exp(tau * dot(qt, kr + (size_t)j * D, D) - mu);
      ell += p;
      for (int c = 0; c < D; ++c) yt[c] += p * vr[(size_t)j * D + c];
    }
    const double sg = sigmoid(gate[h]);
    for (int c = 0; c < D; ++c) {
      double m = 0.0;
      for (int a = 0; a < D; ++a) m += qt[a] * Ash[a * D + c];
      yt[c] = yt[c] / ell + sg * m;
    }
  }
  for (int s = 0; s < S; ++s) pos[s] += 1;
}

/*
 * Backward of L = sum_t <dy_t, y_t> for one (b,h).
 *   L1 (softmax band): P = softmax weights, dP_i = <dy,v_i>,
 *     dZ_i = P_i (dP_i - sum_j P_j dP_j);  dq += tau sum dZ_i k_i,
 *     dk_i += tau dZ_i q_t,  dv_i += P_i dy_t.
 *   L2, forward sweep with forward-mode tangents of the state:
 *     A_t as in the forward, Bt = dA_t/dlambda, Et = dA_t/deta; with
 *     dm_t = sigma*dy_t:  dq_t += A_t dm_t,  dlambda += <dm_t, q_t Bt>,
 *     deta += <dm_t, q_t Et>,  dg += sigma(1-sigma) <dy_t, m_t>.
 *   L2, reverse sweep with the adjoint R_t = q_t^T dm_t + lambda R_{t+1}:
 *     for t >= W: dk_{t-W} += eta R_t v_{t-W},  dv_{t-W} += eta R_t^T k_{t-W}.
 * Outputs are accumulated into dq/dk/dv (zeroed by the caller) and the
 * three scalars.
 */
static void backward_one(int T, int D, int W, double tau, const double* q,
                         const double* k, const double* v, const double* dy,
                         double lam, double eta, double g, double* dq,
                         double* dk, double* dv, double* dlam, double* deta,
                         double* dg) {
  const double sg = sigmoid(g);
  double* z = (double*)malloc(sizeof(double) * (size_t)(W > 0 ? W : 1));
  double* dp = (double*)malloc(sizeof(double) * (size_t)(W > 0 ? W : 1));
  /* ---- L1 ---- */
  for (int t = 0; t < T; ++t) {
    const double* qt = q + (size_t)t * D;
    const double* dyt = dy + (size_t)t * D;
    int lo = t - W + 1;
    if (lo < 0) lo = 0;
    double mu = -INFINITY;
    for (int i = lo; i <= t; ++i) {
      z[i - lo] = tau * dot(qt, k + (size_t)i * D, D);
      if (z[i - lo] > mu) mu = z[i - lo];
    }
    double ell = 0.0;
    for (int i = lo; i <= t; ++i) ell += exp(z[i - lo] - mu);
    double pdp = 0.0;
    for (int i = lo; i <= t; ++i) {
      z[i - lo] = exp(z[i - lo] - mu) / ell; /* now P_i */
      dp[i - lo] = dot(dyt, v + (size_t)i * D, D);
      pdp += z[i - lo] * dp[i - lo];
    }
    for (int i = lo; i <= t; ++i) {
      const double P = z[i - lo];
      const double dZ = P * (dp[i - lo] - pdp);
      const double* ki = k + (size_t)i * D;
      for (int a = 0; a < D; ++a) {
        dq[(size_t)t * D + a] += tau * dZ * ki[a];
        dk[(size_t)i * D + a] += tau * dZ * qt[a];
        dv[(size_t)i * D + a] += P * dyt[a];
      }
    }
  }
  /* ---- L2 forward sweep ---- */
  const size_t DD = (size_t)D * D;
  double* A = (double*)calloc(DD, sizeof(double));
  double* Bt = (double*)calloc(DD, sizeof(double));
  double* Et = (double*)calloc(DD, sizeof(double));
  double sl = 0.0, se = 0.0, sgd = 0.0;
  for (int t = 0; t < T; ++t) {
    if (t >= W) {
      const double* ke = k + (size_t)(t - W) * D;
      const double* ve = v + (size_t)(t - W) * D;
      for (int a = 0; a < D; ++a)
        for (int c = 0; c < D; ++c) {
          const size_t ac = (size_t)a * D + c;
          const double kv = ke[a] * ve[c];
          Bt[ac] = A[ac] + lam * Bt[ac]; /* d(lam*A)/dlam uses the old A */
          Et[ac] = lam * Et[ac] + kv;
          A[ac] = lam * A[ac] + eta * kv;
        }
    }
    const double* qt = q + (size_t)t * D;
    const double* dyt = dy + (size_t)t * D;
    for (int c = 0; c < D; ++c) {
      double m = 0.0, mb = 0.0, me = 0.0;
      for (int a = 0; a < D; ++a) {
        m += qt[a] * A[(size_t)a * D + c];
        mb += qt[a] * Bt[(size_t)a * D + c];
        me += qt[a] * Et[(size_t)a * D + c];
      }
      const double dm = sg * dyt[c];
      sl += dm * mb;
      se += dm * me;
      sgd += dyt[c] * m;
    }
    for (int a = 0; a < D; ++a) {
      double acc = 0.0;
      for (int c = 0; c < D; ++c) acc += A[(size_t)a * D + c] * sg * dyt[c];
      dq[(size_t)t * D + a] += acc;
    }
  }
  *dlam += sl;
  *deta += se;
  *dg += sg * (1.0 - sg) * sgd;
  /* ---- L2 reverse sweep ---- */
  double* R = A; /* reuse storage */
  memset(R, 0, sizeof(double) * DD);
  for (int t = T - 1; t >= 0; --t) {
    const double* qt = q + (size_t)t * D;
    const double* dyt = dy + (size_t)t * D;
    for (int a = 0; a < D; ++a)
      for (int c = 0; c < D; ++c)
        R[(size_t)a * D + c] = lam * R[(size_t)a * D + c] + qt[a] * sg * dyt[c];
    if (t >= W) {
      const int i = t - W;
      const double* ki = k + (size_t)i * D;
      const double* vi = v + (size_t)i * D;
      for (int a = 0; a < D; ++a) {
        double acc = 0.0;
        for (int c = 0; c < D; ++c) acc += R[(size_t)a * D + c] * vi[c];
        dk[(size_t)i * D + a] += eta * acc;
      }
      for (int c = 0; c < D; ++c) {
        double acc = 0.0;
        for (int a = 0; a < D; ++a) acc += R[(size_t)a * D + c] * ki[a];
        dv[(size_t)i * D + c] += eta * acc;
      }
    }
  }
  free(A);
  free(Bt);
  free(Et);
  free(z);
  free(dp);
}

/*
 * tco_backward: dq, dk, dv [B,H,T,D] (overwritten); dlam, deta, dgate [H]
 * (overwritten, summed over the batch in b order).
 */
void tco_backward(int B, int H, int T, int D, int W, double tau,
                  const double* q, const double* k, const double* v,
                  const double* dy, const double* lam, const double* eta,
                  const double* gate, double* dq, double* dk, double* dv,
                  double* dlam, double* deta, double* dgate) {
  const size_t n = (size_t)B * H * T * D;
  memset(dq, 0, sizeof(double) * n);
  memset(dk, 0, sizeof(double) * n);
  memset(dv, 0, sizeof(double) * n);
  double* part = (double*)calloc((size_t)3 * B * H, sizeof(double));
#pragma omp parallel for schedule(dynamic, 1)
  for (int bh = 0; bh < B * H; ++bh) {
    const int h = bh % H;
    const size_t off = (size_t)bh * T * D;
    backward_one(T, D, W, tau, q + off, k + off, v + off, dy + off, lam[h],
                 eta[h], gate[h], dq + off, dk + off, dv + off,
                 &part[3 * bh + 0], &part[3 * bh + 1], &part[3 * bh + 2]);
  }
  for (int h = 0; h < H; ++h) {
    double a = 0.0, b = 0.0, c = 0.0;
    for (int bb = 0; bb < B; ++bb) {
      a += part[3 * (bb * H + h) + 0];
      b += part[3 * (bb * H + h) + 1];
      c += part[3 * (bb * H + h) + 2];
    }
    dlam[h] = a;
    deta[h] = b;
    dgate[h] = c;
  }
  free(part);
}

/* ------------------------------------------------------------------------
 * fp32 models of the memory path only (m_t = q_t A_t and the final A), used
 * to check the claim of the abstract and of the contributions list that the
 * parallel weighted-sum scan agrees with per-token writes to float32
 * rounding (the contributions list puts it below 1e-7 relative).  Both read
 * the same float inputs.
 * ---------------------------------------------------------------------- */

/* Per-token writes in float: A <- lam*A + eta*k v^T on each eviction. */
void tco_memory_f32_sequential(int T, int D, int W, float lam, float eta,
                               const float* q, const float* k, const float* v,
                               float* m, float* A_final) {
  float* A = (float*)calloc((size_t)D * D, sizeof(float));
  for (int t = 0; t < T; ++t) {
    if (t >= W) {
      const float* ke = k + (size_t)(t - W) * D;
      const float* ve = v + (size_t)(t - W) * D;
      for (int a = 0; a < D; ++a)
        for (int c = 0; c < D; ++c)
          A[a * D + c] = lam * A[a * D + c] + eta * ke[a] * ve[c];
    }
    for (int c = 0; c < D; ++c) {
      float acc = 0.0f;
      for (int a = 0; a < D; ++a) acc += q[(size_t)t * D + a] * A[a * D + c];
      m[(size_t)t * D + c] = acc;
    }
  }
  if (A_final) memcpy(A_final, A, sizeof(float) * (size_t)D * D);
  free(A);
}

static float powf_int(float x, int n) {
  float r = 1.0f;
  for (int i = 0; i < n; ++i) r *= x;
  return r;
}

/*
 * Chunked weighted-sum scan in float.  Eviction indices e = t - W are grouped
 * into chunks of C.  Per chunk n the weighted sum of its outer products
 *   U_n = sum_r eta*lam^(C-1-r) k_{nC+r} v_{nC+r}^T
 * replaces the chunk-mean write, and the carry is S_{n+1} = lam^C S_n + U_n
 * (S_0 = 0).  A query whose eviction index is s = nC + r reads
 *   m = lam^(r+1) q S_n + sum_{j<=r} eta*lam^(r-j) <q,k_{nC+j}> v_{nC+j}.
 * This is our reading of the parallel weighted-sum scan named in the
 * abstract: it equals the per-token writes exactly in real arithmetic.
 */
void tco_memory_f32_chunked(int T, int D, int W, int C, float lam, float eta,
                            const float* q, const float* k, const float* v,
                            float* m, float* A_final) {
  float* S = (float*)calloc((size_t)D * D, sizeof(float));
  float* U = (float*)calloc((size_t)D * D, sizeof(float));
  const int E = T - W; /* number of evictions */
  const int nchunks = E > 0 ? (E + C - 1) / C : 0;
  for (int t = 0; t < (W < T ? W : T); ++t)
    for (int c = 0; c < D; ++c) m[(size_t)t * D + c] = 0.0f;
  for (int n = 0; n < nchunks; ++n) {
    const int e0 = n * C;
    const int len = (E - e0) < C ? (E - e0) : C;
    /* reads of the queries whose eviction index falls in this chunk */
    for (int r = 0; r < len; ++r) {
      const int t = e0 + r + W;
      const float* qt = q + (size_t)t * D;
      const float f = powf_int(lam, r + 1);
      for (int c = 0; c < D; ++c) {
        float acc = 0.0f;
        for (int a = 0; a < D; ++a) acc += qt[a] * S[a * D + c];
        m[(size_t)t * D + c] = f * acc;
      }
      for (int j = 0; j <= r; ++j) {
        const float* kj = k + (size_t)(e0 + j) * D;
        const float* vj = v + (size_t)(e0 + j) * D;
        float s = 0.0f;
        for (int a = 0; a < D; ++a) s += qt[a] * kj[a];
        const float w = eta * powf_int(lam, r - j) * s;
        for (int c = 0; c < D; ++c) m[(size_t)t * D + c] += w * vj[c];
      }
    }
    /* carry: S <- lam^len S + sum_r eta*lam^(len-1-r) k v^T */
    memset(U, 0, sizeof(float) * (size_t)D * D);
    for (int r = 0; r < len; ++r) {
      const float w = eta * powf_int(lam, len - 1 - r);
      const float* kr = k + (size_t)(e0 + r) * D;
      const float* vr = v + (size_t)(e0 + r) * D;
      for (int a = 0; a < D; ++a)
        for (int c = 0; c < D; ++c) U[a * D + c] += w * kr[a] * vr[c];
    }
    const float decay = powf_int(lam, len);
    for (size_t x = 0; x < (size_t)D * D; ++x) S[x] = decay * S[x] + U[x];
  }
  if (A_final) memcpy(A_final, S, sizeof(float) * (size_t)D * D);
  free(S);
  free(U);
}

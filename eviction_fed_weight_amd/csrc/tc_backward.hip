// TC backward on gfx950: gradients of L = sum_t <dy_t, y_t> with respect to
// q, k, v and the per-head lambda, eta, g ("Tensor Cache: Eviction-conditioned
// Associative Memory for Transformers": the abstract states that the decay,
// write rate and gate are trained end to end; Section 3.1 Eq. (1) and
// Section 3.2 / Figure 2 define the layer).
//
// Notation (per (b,h), eta factored out of the state):
//   S(e) = sum_{i<e} lambda^(e-1-i) k_i v_i^T,   A_t = eta S(t-W+1),
//   m_t = eta mt_t,  mt_t = q_t S(t-W+1),  sigma = sigmoid(g),  dm_t = sigma dy_t.
// Query block j (rows t0 = 64j + r) reads, with e0 = t0 - W,
//   mt_t = lambda^(r+1) q_t S(e0) + sum_{c<=r} lambda^(r-c) <q_t,k_{e0+c}> v_{e0+c}.
// Gradients of the memory path (L2):
//   dq_t  = sigma eta [lambda^(r+1) S(e0) dy_t + sum_c lambda^(r-c) <dy_t,v_c> k_c]
//   dk_i  = sigma eta R(i) v_i,   dv_i = sigma eta R(i)^T k_i,
//   R(e)  = sum_{t : t-W >= e} lambda^(t-W-e) q_t^T dy_t          (reverse adjoint)
//   deta  = sigma sum_t <dy_t, mt_t>,   dg = sigma (1-sigma) eta sum_t <dy_t, mt_t>
//   dlam  = sigma eta sum_t <dy_t, d mt_t / d lambda>, where
//   d mt_t/d lambda = (r+1) lambda^r q_t S(e0) + lambda^(r+1) q_t B(e0)
//                     + sum_c (r-c) lambda^(r-c-1) <q_t,k_c> v_c,   B = dS/dlambda.
// The window softmax (L1) uses the usual recomputation from the saved
// log-normaliser and Delta_t = <dy_t, y_local,t> = <dy_t, y_t> - sigma eta <dy_t, mt_t>.
//
// Kernels (64-row blocks, G blocks per workgroup segment):
//   bseg_fwd_kernel / bchain_fwd_kernel : segment-start S and B
//   bseg_rev_kernel / bchain_rev_kernel : segment-end R
//   dq_kernel   : forward walk over query blocks (S, B carried in registers):
//                 memory-path dq and scalars, Delta, then the band dq loop
//   dkdv_kernel : reverse walk over key blocks (R carried in registers in
//                 both operand layouts): memory-path dk, dv, then band dk, dv
//   reduce_kernel : deterministic sums for dlambda, deta, dgate.
#ifndef TC_BWD_BF16
#error "compile with -DTC_BWD_BF16=1 (bf16 kernels) or -DTC_BWD_BF16=0 (float32 kernels)"
#endif
#include "tc_device.h"
#include "tc_launch.h"

namespace tck {

template <class E, int D>
struct BwdCfg {
  static constexpr int NT = D / 16;
  static constexpr int NKC = (D + 31) / 32;
  static constexpr int NOWN = (NT + 3) / 4;
  static constexpr int VE = 16 / (int)sizeof(E);
  static constexpr int LDK = D + VE;
  static constexpr int LDX = D + 4;
  static constexpr int TILE = 64 * LDK * (int)sizeof(E);
  static constexpr int XB = 64 * LDX * 4;
  static constexpr int U = (2 * TILE) > XB ? (2 * TILE) : XB;
};

// Fragment of two runs of four rows (rows r0..r0+3 at p0, r0'..r0'+3 at p1)
// of a row-major LDS tile, column l16 (contraction down the rows).
template <class E>
struct ColFrag2;
template <>
struct ColFrag2<bf16> {
  static __device__ __forceinline__ bf16x8 read(const bf16* p0, const bf16* p1, int ld, int l16) {
    const bf16* a0 = p0 + (l16 >> 2) * ld + 4 * (l16 & 3);
    const bf16* a1 = p1 + (l16 >> 2) * ld + 4 * (l16 & 3);
    const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(a0));
    const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(a1));
    bf16x8 r;
    const bf16* ea = (const bf16*)&a;
    const bf16* eb = (const bf16*)&b;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r[j] = ea[j];
      r[j + 4] = eb[j];
    }
    return r;
  }
};
template <>
struct ColFrag2<float> {
  static __device__ __forceinline__ f32x8 read(const float* p0, const float* p1, int ld, int l16) {
    f32x8 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r[j] = p0[j * ld + l16];
      r[j + 4] = p1[j * ld + l16];
    }
    return r;
  }
};

// Two runs of four consecutive LDS elements as one fragment.
template <class E>
__device__ __forceinline__ typename Mfma<E>::frag frag4x2(const E* p0, const E* p1, bool second);
template <>
__device__ __forceinline__ bf16x8 frag4x2<bf16>(const bf16* p0, const bf16* p1, bool second) {
  const bf16x4 a = *(const bf16x4*)p0;
  bf16x4 b = *(const bf16x4*)p1;
  if (!second) b = bf16x4{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
template <>
__device__ __forceinline__ f32x8 frag4x2<float>(const float* p0, const float* p1, bool second) {
  const f32x4 a = *(const f32x4*)p0;
  f32x4 b = *(const f32x4*)p1;
  if (!second) b = f32x4{0.f, 0.f, 0.f, 0.f};
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ void st4(bf16* dst, f32x4 x) {
  bf16x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = (bf16)x[i];
  *(bf16x4*)dst = r;
}
__device__ __forceinline__ void st4(float* dst, f32x4 x) { *(f32x4*)dst = x; }

// Tables pw[x] = lambda^x, dpw[x] = x lambda^(x-1) (dpw[0] = 0), x = 0..64.
__device__ __forceinline__ void fill_pow_tables(float lam, float* pw, float* dpw) {
  const int x = threadIdx.x;
  if (x <= 64) {
    pw[x] = powi(lam, x);
    dpw[x] = x == 0 ? 0.0f : (float)x * powi(lam, x - 1);
  }
}

// Load a D x D float state (row a, column c at g[a*D + c]) into tiles
// t[o][m] where the lane holds element [row = 16*m + 4lg + i][col = 16*n + l16]
// with n = wid + 4o (ROWS_BY_LG) -- the layout of an MFMA output out[m][n] --
// or its transpose (element [row = 16*n + l16][col = 16*m + 4lg + i]).
template <int D, bool TRANS>
__device__ __forceinline__ void load_tiles(f32x4 (&t)[(D / 16 + 3) / 4][D / 16], const float* g, int wid,
                                           int l16, int lg) {
  constexpr int NT = D / 16, NOWN = (NT + 3) / 4;
#pragma unroll
  for (int o = 0; o < NOWN; ++o) {
    const int n = wid + 4 * o;
#pragma unroll
    for (int m = 0; m < NT; ++m) {
      f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
      if (n < NT) {
        if (TRANS) {
          x = *(const f32x4*)(g + (n * 16 + l16) * D + m * 16 + lg * 4);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) x[i] = g[(m * 16 + lg * 4 + i) * D + n * 16 + l16];
        }
      }
      t[o][m] = x;
    }
  }
}

template <int D>
__device__ __forceinline__ void store_tiles(const f32x4 (&t)[(D / 16 + 3) / 4][D / 16], float* g, int wid,
                                            int l16, int lg) {
  constexpr int NT = D / 16, NOWN = (NT + 3) / 4;
#pragma unroll
  for (int o = 0; o < NOWN; ++o) {
    const int n = wid + 4 * o;
    if (n < NT) {
#pragma unroll
      for (int m = 0; m < NT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) g[(m * 16 + lg * 4 + i) * D + n * 16 + l16] = t[o][m][i];
    }
  }
}

template <int D>
__device__ __forceinline__ void zero_tiles(f32x4 (&t)[(D / 16 + 3) / 4][D / 16]) {
#pragma unroll
  for (int o = 0; o < (D / 16 + 3) / 4; ++o)
#pragma unroll
    for (int m = 0; m < D / 16; ++m) t[o][m] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// acc(o, m) <- scale*acc + sum_{c<64} A[c][16m + ..]^T (w_c B[c][16n + ..]),
// i.e. out[m-row][n-col] += sum_c A[c][row] w_c B[c][col], where A, B are 64-row
// row-major LDS tiles, all m tiles, owned n = wid + 4o.  Optionally a second
// accumulator gets the same product with weights w2 (no extra scale).
template <class E, int D, bool TWO>
__device__ __forceinline__ void rank64_update(f32x4 (&acc)[(D / 16 + 3) / 4][D / 16], float scale,
                                              f32x4 (&acc2)[(D / 16 + 3) / 4][D / 16], const E* A,
                                              const E* B, const float* w, const float* w2, int wid, int l16,
                                              int lg) {
  using M = Mfma<E>;
  using frag = typename M::frag;
  constexpr int NT = D / 16, NOWN = (NT + 3) / 4, LDK = BwdCfg<E, D>::LDK;
#pragma unroll
  for (int o = 0; o < NOWN; ++o) {
    const int n = wid + 4 * o;
    if (n < NT) {
#pragma unroll
      for (int m = 0; m < NT; ++m) acc[o][m] *= scale;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        float bv[8], bw[8], bw2[8];
        M::to_f32(ColFrag<E>::read(B + (kc * 32 + lg * 8) * LDK + n * 16, LDK, l16), bv);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          bw[j] = w[kc * 32 + lg * 8 + j] * bv[j];
          if (TWO) bw2[j] = w2[kc * 32 + lg * 8 + j] * bv[j];
        }
        frag hi, lo, hi2, lo2;
        M::split(bw, hi, lo);
        if (TWO) M::split(bw2, hi2, lo2);
#pragma unroll
        for (int m = 0; m < NT; ++m) {
          const frag af = ColFrag<E>::read(A + (kc * 32 + lg * 8) * LDK + m * 16, LDK, l16);
          acc[o][m] = M::mma(af, hi, acc[o][m]);
          if (M::kSplit) acc[o][m] = M::mma(af, lo, acc[o][m]);
          if (TWO) {
            acc2[o][m] = M::mma(af, hi2, acc2[o][m]);
            if (M::kSplit) acc2[o][m] = M::mma(af, lo2, acc2[o][m]);
          }
        }
      }
    }
  }
}

// out[m = x-row (16*o' tiles)][n = 64 rows of R (4 groups)] for one owned
// state tile column: acc[g] += sum_k St[k][x] * R[16g + l16][k], where the
// state tiles t[o][*] hold [k = 16*kt + 4lg + i][x = 16*n + l16] and R is a
// row-major LDS tile (4-element runs).  Used for q S, S dy, R v, R^T k.
template <class E, int D>
__device__ __forceinline__ void state_times_rows(const f32x4 (&t)[(D / 16 + 3) / 4][D / 16], int o,
                                                 const E* R, f32x4 (&acc)[4], int l16, int lg) {
  using M = Mfma<E>;
  using frag = typename M::frag;
  constexpr int NT = D / 16, LDK = BwdCfg<E, D>::LDK;
#pragma unroll
  for (int g = 0; g < 4; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int pp = 0; pp < (NT + 1) / 2; ++pp) {
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sv[i] = t[o][2 * pp][i];
      sv[4 + i] = (2 * pp + 1 < NT) ? t[o][(2 * pp + 1) % NT][i] : 0.0f;
    }
    frag hi, lo;
    M::split(sv, hi, lo);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const E* row = R + (g * 16 + l16) * LDK;
      const frag b = frag4x2<E>(row + 32 * pp + lg * 4, row + (32 * pp + 16 + lg * 4) % D, 32 * pp + 16 < D);
      acc[g] = M::mma(hi, b, acc[g]);
      if (M::kSplit) acc[g] = M::mma(lo, b, acc[g]);
    }
  }
}

// ===========================================================================
// Segment states for the backward.
// Forward: S and B = dS/dlambda over each segment's evictions (from zero);
// grid = BH * (nseg-1); writes fstate/tstate[bh][m+1].
template <class E, int D>
__global__ void __launch_bounds__(256, 2) bseg_fwd_kernel(BwdArgs a) {
  using C = BwdCfg<E, D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::TILE];
  __shared__ float pw[72], dpw[72], w1[64], w2[64];
  E* Ks = (E*)smem;
  E* Vs = (E*)(smem + C::TILE);
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int nm = a.nseg - 1;
  const int bh = blockIdx.x / nm, m = blockIdx.x - bh * nm;
  const int h = bh % a.H;
  const uint32_t nbytes = (uint32_t)a.T * D * sizeof(E);
  const size_t base = (size_t)bh * a.T * D;
  const auto Kg = make_rsrc((const E*)a.k + base, nbytes);
  const auto Vg = make_rsrc((const E*)a.v + base, nbytes);
  fill_pow_tables(a.lam[h], pw, dpw);
  f32x4 S[C::NOWN][C::NT], B[C::NOWN][C::NT];
  zero_tiles<D>(S);
  zero_tiles<D>(B);
  TileRegs<E, D, 64> kl, vl;
  for (int g = 0; g < a.G; ++g) {
    const int e0 = (m * a.G + g) * 64 - a.W;
    if (e0 + 63 < 0) continue;
    kl.load(Kg, e0);
    vl.load(Vg, e0);
    __syncthreads();
    kl.store(Ks, C::LDK);
    vl.store(Vs, C::LDK);
    if (tid < 64) {
      const bool ok = e0 + tid >= 0;
      w1[tid] = ok ? pw[63 - tid] : 0.0f;
      w2[tid] = ok ? dpw[63 - tid] : 0.0f;
    }
    __syncthreads();
    // B <- lam^64 B + 64 lam^63 S + sum w2 k v^T ; S <- lam^64 S + sum w1 k v^T
#pragma unroll
    for (int o = 0; o < C::NOWN; ++o)
#pragma unroll
      for (int mm = 0; mm < C::NT; ++mm) B[o][mm] = pw[64] * B[o][mm] + dpw[64] * S[o][mm];
    rank64_update<E, D, true>(S, pw[64], B, Ks, Vs, w1, w2, wid, l16, lg);
  }
  store_tiles<D>(S, a.fstate + ((size_t)bh * a.nseg + m + 1) * D * D, wid, l16, lg);
  store_tiles<D>(B, a.tstate + ((size_t)bh * a.nseg + m + 1) * D * D, wid, l16, lg);
}

// S[0] = B[0] = 0; S[m+1] = L S[m] + Ls_m; B[m+1] = L' S[m] + L B[m] + Lb_m
// with L = lambda^(64G), L' = 64G lambda^(64G-1).
template <int D>
__global__ void __launch_bounds__(256) bchain_fwd_kernel(BwdArgs a) {
  const int bh = blockIdx.y;
  const int x = blockIdx.x * 256 + threadIdx.x;
  if (x * 4 >= D * D) return;
  const float lam = a.lam[bh % a.H];
  const int n = 64 * a.G;
  const float L = powi(lam, n), Ld = (float)n * powi(lam, n - 1);
  float4* ps = (float4*)(a.fstate + (size_t)bh * a.nseg * D * D) + x;
  float4* pb = (float4*)(a.tstate + (size_t)bh * a.nseg * D * D) + x;
  const size_t stride = (size_t)D * D / 4;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f), b = s;
  ps[0] = s;
  pb[0] = b;
  for (int m = 1; m < a.nseg; ++m) {
    const float4 ls = ps[m * stride], lb = pb[m * stride];
    b.x = Ld * s.x + L * b.x + lb.x;
    b.y = Ld * s.y + L * b.y + lb.y;
    b.z = Ld * s.z + L * b.z + lb.z;
    b.w = Ld * s.w + L * b.w + lb.w;
    s.x = L * s.x + ls.x;
    s.y = L * s.y + ls.y;
    s.z = L * s.z + ls.z;
    s.w = L * s.w + ls.w;
    ps[m * stride] = s;
    pb[m * stride] = b;
  }
}

// Reverse: local adjoint of segment m (m >= 1) over the query rows whose
// eviction index lies in its key range, relative to its first key:
// Lr_m = sum_{jk in seg, descending} lambda^(64 (jk - jb)) U(jk),
// U(jk) = sum_{c<64} lambda^c q_{64jk+W+c}^T dy_{64jk+W+c};  writes rstate[bh][m-1].
template <class E, int D>
__global__ void __launch_bounds__(256, 2) bseg_rev_kernel(BwdArgs a) {
  using C = BwdCfg<E, D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::TILE];
  __shared__ float pw[72], dpw[72];
  E* Qs = (E*)smem;
  E* Ys = (E*)(smem + C::TILE);
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int nm = a.nseg - 1;
  const int bh = blockIdx.x / nm, m = blockIdx.x - bh * nm + 1;
  const int h = bh % a.H;
  const uint32_t nbytes = (uint32_t)a.T * D * sizeof(E);
  const size_t base = (size_t)bh * a.T * D;
  const auto Qg = make_rsrc((const E*)a.q + base, nbytes);
  const auto Yg = make_rsrc((const E*)a.dy + base, nbytes);
  fill_pow_tables(a.lam[h], pw, dpw);
  f32x4 R[C::NOWN][C::NT];
  zero_tiles<D>(R);
  const int jb = m * a.G, je = min(a.nblk, jb + a.G);
  TileRegs<E, D, 64> ql, yl;
  for (int jk = je - 1; jk >= jb; --jk) {
    const int q0 = jk * 64 + a.W;
    if (q0 >= a.T) continue;
    ql.load(Qg, q0);
    yl.load(Yg, q0);
    __syncthreads();
    ql.store(Qs, C::LDK);
    yl.store(Ys, C::LDK);
    __syncthreads();
    // R[a][c] <- lam^64 R + sum_c' Q[c'][a] lam^c' dY[c'][c]  (skipped blocks
    // contribute zero and need no decay: R is zero until the first block)
    rank64_update<E, D, false>(R, pw[64], R, Qs, Ys, pw, pw, wid, l16, lg);
  }
  // blocks skipped at the top (q0 >= T) would only scale a zero state;
  // blocks present below them were decayed correctly relative to jb.
  store_tiles<D>(R, a.rstate + ((size_t)bh * a.nseg + m - 1) * D * D, wid, l16, lg);
}

// R_end[nseg-1] = 0; R_end[m] = lambda^(64G) R_end[m+1] + Lr_{m+1} (in place).
template <int D>
__global__ void __launch_bounds__(256) bchain_rev_kernel(BwdArgs a) {
  const int bh = blockIdx.y;
  const int x = blockIdx.x * 256 + threadIdx.x;
  if (x * 4 >= D * D) return;
  const float L = powi(a.lam[bh % a.H], 64 * a.G);
  float4* p = (float4*)(a.rstate + (size_t)bh * a.nseg * D * D) + x;
  const size_t stride = (size_t)D * D / 4;
  float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
  p[(a.nseg - 1) * stride] = r;
  for (int m = a.nseg - 2; m >= 0; --m) {
    const float4 l = p[m * stride];
    r.x = L * r.x + l.x;
    r.y = L * r.y + l.y;
    r.z = L * r.z + l.z;
    r.w = L * r.w + l.w;
    p[m * stride] = r;
  }
}

// ===========================================================================
// dq kernel: grid = BH * nseg, 4 waves x 16 query rows per 64-row block.
template <class E, int D>
__global__ void __launch_bounds__(256, 1) dq_kernel(BwdArgs a) {
  using M = Mfma<E>;
  using frag = typename M::frag;
  using C = BwdCfg<E, D>;
  constexpr int NT = C::NT, NKC = C::NKC, NOWN = C::NOWN, LDK = C::LDK, LDX = C::LDX, VE = C::VE;
  __shared__ __attribute__((aligned(16))) char smem[C::U + 2 * C::TILE];
  __shared__ float pw[72], dpw[72], ypart[4][64], red[4][2];
  E* Ks = (E*)smem;
  E* Vs = (E*)(smem + C::TILE);
  float* X = (float*)smem;
  E* Qs = (E*)(smem + C::U);
  E* Ys = (E*)(smem + C::U + C::TILE);

  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int wgi = xcd_remap(blockIdx.x, gridDim.x);  // one head's segments on one XCD
  const int bh = wgi / a.nseg, seg = wgi - bh * a.nseg;
  const int h = bh % a.H;
  const int T = a.T, W = a.W;
  const size_t base = (size_t)bh * T * D;
  const uint32_t nbytes = (uint32_t)T * D * sizeof(E);
  const auto Qg = make_rsrc((const E*)a.q + base, nbytes);
  const auto Kg = make_rsrc((const E*)a.k + base, nbytes);
  const auto Vg = make_rsrc((const E*)a.v + base, nbytes);
  const auto dYg = make_rsrc((const E*)a.dy + base, nbytes);
  const auto Yg = make_rsrc((const E*)a.y + base, nbytes);
  E* dQg = (E*)a.dq + base;
  const float sg = sigmoidf(a.gate[h]);
  const float seta = sg * a.eta[h];
  const float tau = a.scale, sl2 = a.scale * kLog2e;
  fill_pow_tables(a.lam[h], pw, dpw);

  // S^T and B^T: tiles [o][ct] hold element [c = 16 ct + 4lg + i][a = 16 (wid+4o) + l16]
  f32x4 S[NOWN][NT], B[NOWN][NT];
  if (seg == 0) {
    zero_tiles<D>(S);
    zero_tiles<D>(B);
  } else {
    load_tiles<D, true>(S, a.fstate + ((size_t)bh * a.nseg + seg) * D * D, wid, l16, lg);
    load_tiles<D, true>(B, a.tstate + ((size_t)bh * a.nseg + seg) * D * D, wid, l16, lg);
  }
  vm_fence_loads();
  const int jb = seg * a.G, je = min(a.nblk, jb + a.G);
  const int r = wid * 16 + l16;
  float md_acc = 0.0f, dl_acc = 0.0f;
  TileRegs<E, D, 64> ql, yl, kl, vl;
  for (int j = jb; j < je; ++j) {
    const int t0 = j * 64, trow = t0 + r, e0 = t0 - W;
    const bool has_mem = t0 + 63 >= W;
    __syncthreads();
    ql.load(Qg, t0);
    yl.load(dYg, t0);
    kl.load(Kg, e0);
    vl.load(Vg, e0);
    ql.store(Qs, LDK);
    yl.store(Ys, LDK);
    __syncthreads();
    frag qf[NKC], yf[NKC];
#pragma unroll
    for (int dc = 0; dc < NKC; ++dc) {
      const bool in = dc * 32 + lg * 8 < D;
      qf[dc] = in ? M::lds8(Qs + r * LDK + dc * 32 + lg * 8) : M::zero();
      yf[dc] = in ? M::lds8(Ys + r * LDK + dc * 32 + lg * 8) : M::zero();
    }
    f32x4 dQ[NT];
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) dQ[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float md = 0.0f, dlr = 0.0f;  // <dy, mt> and <dy, d mt/dlam> of row r (all 4 lanes)

    if (has_mem) {
      if (e0 > 0) {
        // X = S dY (all rows, owned a-tiles) and partial <q, B dY>
        float yp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int o = 0; o < NOWN; ++o) {
          const int at = wid + 4 * o;
          if (at < NT) {
            f32x4 xa[4], ya[4];
            state_times_rows<E, D>(S, o, Ys, xa, l16, lg);
            state_times_rows<E, D>(B, o, Ys, ya, l16, lg);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              *(f32x4*)(X + (g * 16 + l16) * LDX + at * 16 + lg * 4) = xa[g];
              const E* qrow = Qs + (g * 16 + l16) * LDK + at * 16 + lg * 4;
#pragma unroll
              for (int i = 0; i < 4; ++i) yp[g] += (float)qrow[i] * ya[g][i];
            }
          }
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float v = xsum4(yp[g]);
          if (lg == 0) ypart[wid][g * 16 + l16] = v;
        }
        __syncthreads();
        const float f = pw[r + 1], df = dpw[r + 1];
        float qx = 0.0f;
#pragma unroll
        for (int dt = 0; dt < NT; ++dt) {
          const f32x4 xv = *(const f32x4*)(X + r * LDX + dt * 16 + lg * 4);
          const E* qrow = Qs + r * LDK + dt * 16 + lg * 4;
#pragma unroll
          for (int i = 0; i < 4; ++i) qx += (float)qrow[i] * xv[i];
          dQ[dt] += (seta * f) * xv;
        }
        qx = xsum4(qx);
        const float qy = ypart[0][r] + ypart[1][r] + ypart[2][r] + ypart[3][r];
        md += f * qx;
        dlr += df * qx + f * qy;
        __syncthreads();
      }
      kl.store(Ks, LDK);
      vl.store(Vs, LDK);
      __syncthreads();
      // intra-chunk decayed tile: Z = K q, P = V dy
      f32x4 Z[4], P[4];
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        Z[n] = f32x4{0.f, 0.f, 0.f, 0.f};
        P[n] = Z[n];
        const int kr = 32 * (n >> 1) + (l16 >> 2) * 8 + (n & 1) * 4 + (l16 & 3);
#pragma unroll
        for (int dc = 0; dc < NKC; ++dc) {
          const bool in = dc * 32 + lg * 8 < D;
          const frag ka = in ? M::lds8(Ks + kr * LDK + dc * 32 + lg * 8) : M::zero();
          const frag va = in ? M::lds8(Vs + kr * LDK + dc * 32 + lg * 8) : M::zero();
          Z[n] = M::mma(ka, qf[dc], Z[n]);
          P[n] = M::mma(va, yf[dc], P[n]);
        }
      }
      float mp = 0.0f, dp = 0.0f;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        float gv[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int c = 32 * p + lg * 8 + jj;
          const float z = Z[2 * p + (jj >> 2)][jj & 3];
          const float pv = P[2 * p + (jj >> 2)][jj & 3];
          const bool mem = c <= r && e0 + c >= 0;
          const float w = mem ? pw[r - c] : 0.0f;
          const float dw = mem ? dpw[r - c] : 0.0f;
          mp += w * z * pv;
          dp += dw * z * pv;
          gv[jj] = seta * w * pv;
        }
        const frag gf = M::pack(gv);
#pragma unroll
        for (int dt = 0; dt < NT; ++dt)
          dQ[dt] = M::mma(ColFrag<E>::read(Ks + (p * 32 + lg * 8) * LDK + dt * 16, LDK, l16), gf, dQ[dt]);
      }
      md += xsum4(mp);
      dlr += xsum4(dp);
      // carry S and B to the next block of this segment
      if (j + 1 < je) {
        __shared__ float w1[64], w2[64];
        if (tid < 64) {
          const bool ok = e0 + tid >= 0;
          w1[tid] = ok ? pw[63 - tid] : 0.0f;
          w2[tid] = ok ? dpw[63 - tid] : 0.0f;
        }
        __syncthreads();
#pragma unroll
        for (int o = 0; o < NOWN; ++o)
#pragma unroll
          for (int m = 0; m < NT; ++m) B[o][m] = pw[64] * B[o][m] + dpw[64] * S[o][m];
        // S^T[c][a] += sum_c' V[c'][c] w K[c'][a]
        rank64_update<E, D, true>(S, pw[64], B, Vs, Ks, w1, w2, wid, l16, lg);
      }
    }
    // Delta = <dy, y> - sigma eta <dy, mt>
    float yd = 0.0f;
    for (int vv = lg; vv < D / VE; vv += 4) {
      const uint4 yr = buf_load16(Yg, (trow * D + vv * VE) * (int)sizeof(E));
      const E* ye = (const E*)&yr;
      const E* dy = Ys + r * LDK + vv * VE;
#pragma unroll
      for (int x = 0; x < VE; ++x) yd += (float)ye[x] * (float)dy[x];
    }
    yd = xsum4(yd);
    const float delta = yd - seta * md;
    if (lg == 0 && trow < T) a.delta[(size_t)bh * T + trow] = delta;
    const float lse2 = (trow < T) ? a.lse[(size_t)bh * T + trow] * kLog2e : __builtin_huge_valf();

    // ---- L1 band: dq += tau sum dS k ----
    const int kt_lo = max(0, t0 - W + 1) >> 6;
    const int kt_hi = min(T - 1, t0 + 63) >> 6;
    kl.load(Kg, kt_lo * 64);
    vl.load(Vg, kt_lo * 64);
    for (int kt = kt_lo; kt <= kt_hi; ++kt) {
      const int k0 = kt * 64;
      __syncthreads();
      kl.store(Ks, LDK);
      vl.store(Vs, LDK);
      __syncthreads();
      kl.load(Kg, k0 + 64);
      vl.load(Vg, k0 + 64);
      f32x4 Z[4], P[4];
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        Z[n] = f32x4{0.f, 0.f, 0.f, 0.f};
        P[n] = Z[n];
        const int kr = 32 * (n >> 1) + (l16 >> 2) * 8 + (n & 1) * 4 + (l16 & 3);
#pragma unroll
        for (int dc = 0; dc < NKC; ++dc) {
          const bool in = dc * 32 + lg * 8 < D;
          const frag ka = in ? M::lds8(Ks + kr * LDK + dc * 32 + lg * 8) : M::zero();
          const frag va = in ? M::lds8(Vs + kr * LDK + dc * 32 + lg * 8) : M::zero();
          Z[n] = M::mma(ka, qf[dc], Z[n]);
          P[n] = M::mma(va, yf[dc], P[n]);
        }
      }
      const bool full = (k0 + 63 <= t0) && (k0 >= t0 + 64 - W);
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        float gv[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int key = k0 + 32 * p + lg * 8 + jj;
          const bool band = full || (key <= trow && key > trow - W);
          const float z = Z[2 * p + (jj >> 2)][jj & 3];
          const float dpv = P[2 * p + (jj >> 2)][jj & 3];
          const float pr = band ? fast_exp2(__builtin_fmaf(z, sl2, -lse2)) : 0.0f;
          gv[jj] = tau * pr * (dpv - delta);
        }
        const frag gf = M::pack(gv);
#pragma unroll
        for (int dt = 0; dt < NT; ++dt)
          dQ[dt] = M::mma(ColFrag<E>::read(Ks + (p * 32 + lg * 8) * LDK + dt * 16, LDK, l16), gf, dQ[dt]);
      }
    }
    if (trow < T) {
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) st4(dQg + (size_t)trow * D + dt * 16 + lg * 4, dQ[dt]);
    }
    if (lg == 0 && trow < T) {
      md_acc += md;
      dl_acc += dlr;
    }
  }
  // deterministic per-workgroup partial sums
  md_acc = wave_sum(md_acc);
  dl_acc = wave_sum(dl_acc);
  if (lane == 0) {
    red[wid][0] = md_acc;
    red[wid][1] = dl_acc;
  }
  __syncthreads();
  if (tid == 0) {
    float s0 = 0.0f, s1 = 0.0f;
    for (int w = 0; w < 4; ++w) {
      s0 += red[w][0];
      s1 += red[w][1];
    }
    a.part[((size_t)bh * a.nseg + seg) * 2 + 0] = s0;
    a.part[((size_t)bh * a.nseg + seg) * 2 + 1] = s1;
  }
}

// ===========================================================================
// dk/dv kernel: grid = BH * nseg, reverse walk over key blocks; wave w owns
// keys 16w .. 16w+15 of the 64-key block.
template <class E, int D>
__global__ void __launch_bounds__(256, 1) dkdv_kernel(BwdArgs a) {
  using M = Mfma<E>;
  using frag = typename M::frag;
  using C = BwdCfg<E, D>;
  constexpr int NT = C::NT, NKC = C::NKC, NOWN = C::NOWN, LDK = C::LDK, LDX = C::LDX;
  constexpr int QY = (2 * C::TILE) > C::XB ? (2 * C::TILE) : C::XB;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::TILE + QY];
  __shared__ float pw[72], dpw[72], lse_s[64], del_s[64];
  E* Ks = (E*)smem;
  E* Vs = (E*)(smem + C::TILE);
  E* Qs = (E*)(smem + 2 * C::TILE);
  E* Ys = (E*)(smem + 3 * C::TILE);
  float* X = (float*)(smem + 2 * C::TILE);

  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int wgi = xcd_remap(blockIdx.x, gridDim.x);  // one head's segments on one XCD
  const int bh = wgi / a.nseg, seg = wgi - bh * a.nseg;
  const int h = bh % a.H;
  const int T = a.T, W = a.W;
  const size_t base = (size_t)bh * T * D;
  const uint32_t nbytes = (uint32_t)T * D * sizeof(E);
  const auto Qg = make_rsrc((const E*)a.q + base, nbytes);
  const auto Kg = make_rsrc((const E*)a.k + base, nbytes);
  const auto Vg = make_rsrc((const E*)a.v + base, nbytes);
  const auto dYg = make_rsrc((const E*)a.dy + base, nbytes);
  E* dKg = (E*)a.dk + base;
  E* dVg = (E*)a.dv + base;
  const float seta = sigmoidf(a.gate[h]) * a.eta[h];
  const float tau = a.scale, sl2 = a.scale * kLog2e;
  fill_pow_tables(a.lam[h], pw, dpw);

  // RA tiles [o][at]: element R[a = 16 at + 4lg + i][c = 16 (wid+4o) + l16]
  // RB tiles [o][ct]: element R[a = 16 (wid+4o) + l16][c = 16 ct + 4lg + i]
  f32x4 RA[NOWN][NT], RB[NOWN][NT];
  if (seg == a.nseg - 1) {
    zero_tiles<D>(RA);
    zero_tiles<D>(RB);
  } else {
    const float* g = a.rstate + ((size_t)bh * a.nseg + seg) * D * D;
    load_tiles<D, false>(RA, g, wid, l16, lg);
    load_tiles<D, true>(RB, g, wid, l16, lg);
  }
  vm_fence_loads();
  const int jb = seg * a.G, je = min(a.nblk, jb + a.G);
  const int kidx = wid * 16 + l16;
  TileRegs<E, D, 64> kl, vl, ql, yl;
  for (int jk = je - 1; jk >= jb; --jk) {
    const int i0 = jk * 64, key = i0 + kidx;
    __syncthreads();
    kl.load(Kg, i0);
    vl.load(Vg, i0);
    kl.store(Ks, LDK);
    vl.store(Vs, LDK);
    __syncthreads();
    frag kf[NKC], vf[NKC];
#pragma unroll
    for (int dc = 0; dc < NKC; ++dc) {
      const bool in = dc * 32 + lg * 8 < D;
      kf[dc] = in ? M::lds8(Ks + kidx * LDK + dc * 32 + lg * 8) : M::zero();
      vf[dc] = in ? M::lds8(Vs + kidx * LDK + dc * 32 + lg * 8) : M::zero();
    }
    f32x4 dK[NT], dV[NT];
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) {
      dK[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      dV[dt] = dK[dt];
    }
    // ---- memory path, later queries: R(i0+64) v and R(i0+64)^T k ----
    if (i0 + 64 + W < T) {
      const float f = seta * pw[64 - kidx];
      // (R v)[a][key] with RB (lane-fixed a), exchanged through X[key][a]
#pragma unroll
      for (int o = 0; o < NOWN; ++o) {
        const int at = wid + 4 * o;
        if (at < NT) {
          f32x4 acc[4];
          state_times_rows<E, D>(RB, o, Vs, acc, l16, lg);
#pragma unroll
          for (int g = 0; g < 4; ++g) *(f32x4*)(X + (g * 16 + l16) * LDX + at * 16 + lg * 4) = acc[g];
        }
      }
      __syncthreads();
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) dK[dt] += f * *(const f32x4*)(X + kidx * LDX + dt * 16 + lg * 4);
      __syncthreads();
      // (R^T k)[c][key] with RA (lane-fixed c)
#pragma unroll
      for (int o = 0; o < NOWN; ++o) {
        const int ct = wid + 4 * o;
        if (ct < NT) {
          f32x4 acc[4];
          state_times_rows<E, D>(RA, o, Ks, acc, l16, lg);
#pragma unroll
          for (int g = 0; g < 4; ++g) *(f32x4*)(X + (g * 16 + l16) * LDX + ct * 16 + lg * 4) = acc[g];
        }
      }
      __syncthreads();
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) dV[dt] += f * *(const f32x4*)(X + kidx * LDX + dt * 16 + lg * 4);
      __syncthreads();
    }
    // ---- memory path, the queries whose eviction index is in this block ----
    const int q0m = i0 + W;
    if (q0m < T) {
      ql.load(Qg, q0m);
      yl.load(dYg, q0m);
      ql.store(Qs, LDK);
      yl.store(Ys, LDK);
      __syncthreads();
      f32x4 Z[4], P[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        Z[g] = f32x4{0.f, 0.f, 0.f, 0.f};
        P[g] = Z[g];
#pragma unroll
        for (int dc = 0; dc < NKC; ++dc) {
          const bool in = dc * 32 + lg * 8 < D;
          const frag qa = in ? M::lds8(Qs + (g * 16 + l16) * LDK + dc * 32 + lg * 8) : M::zero();
          const frag ya = in ? M::lds8(Ys + (g * 16 + l16) * LDK + dc * 32 + lg * 8) : M::zero();
          Z[g] = M::mma(qa, kf[dc], Z[g]);
          P[g] = M::mma(ya, vf[dc], P[g]);
        }
      }
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        float pv[8], gv[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int g = 2 * p + (jj >> 2);
          const int cq = g * 16 + lg * 4 + (jj & 3);  // query row in the tile
          const bool mem = cq >= kidx && q0m + cq < T;
          const float w = mem ? seta * pw[cq - kidx] : 0.0f;
          pv[jj] = w * Z[g][jj & 3];
          gv[jj] = w * P[g][jj & 3];
        }
        const frag pf = M::pack(pv), gf = M::pack(gv);
#pragma unroll
        for (int dt = 0; dt < NT; ++dt) {
          dV[dt] = M::mma(ColFrag2<E>::read(Ys + (32 * p + lg * 4) * LDK + dt * 16,
                                            Ys + (32 * p + 16 + lg * 4) * LDK + dt * 16, LDK, l16),
                          pf, dV[dt]);
          dK[dt] = M::mma(ColFrag2<E>::read(Qs + (32 * p + lg * 4) * LDK + dt * 16,
                                            Qs + (32 * p + 16 + lg * 4) * LDK + dt * 16, LDK, l16),
                          gf, dK[dt]);
        }
      }
      // R(i0) = lam^64 R(i0+64) + sum_c' lam^c' q^T dy  (both layouts)
      if (jk > jb) {
        rank64_update<E, D, false>(RA, pw[64], RA, Qs, Ys, pw, pw, wid, l16, lg);
        rank64_update<E, D, false>(RB, pw[64], RB, Ys, Qs, pw, pw, wid, l16, lg);
      }
      __syncthreads();
    }
    // ---- L1 band: query tiles covering rows key .. key + W - 1 ----
    // (each tile's Q, dY, lse and Delta rows are loaded one tile ahead)
    const int qt_lo = i0 >> 6;
    const int qt_hi = min(T - 1, i0 + 62 + W) >> 6;
    float lse_r = 0.0f, del_r = 0.0f;
    auto load_qtile = [&](int q0) {
      ql.load(Qg, q0);
      yl.load(dYg, q0);
      if (tid < 64) {
        const bool ok = q0 + tid < T;
        const size_t ix = (size_t)bh * T + (ok ? q0 + tid : 0);
        lse_r = a.lse[ix];
        del_r = a.delta[ix];
        if (!ok) {
          lse_r = __builtin_huge_valf();
          del_r = 0.0f;
        }
      }
    };
    load_qtile(qt_lo * 64);
    for (int qt = qt_lo; qt <= qt_hi; ++qt) {
      const int q0 = qt * 64;
      __syncthreads();
      if (tid < 64) {
        lse_s[tid] = lse_r * kLog2e;
        del_s[tid] = del_r;
      }
      ql.store(Qs, LDK);
      yl.store(Ys, LDK);
      __syncthreads();
      if (qt < qt_hi) load_qtile(q0 + 64);
      f32x4 Z[4], P[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        Z[g] = f32x4{0.f, 0.f, 0.f, 0.f};
        P[g] = Z[g];
#pragma unroll
        for (int dc = 0; dc < NKC; ++dc) {
          const bool in = dc * 32 + lg * 8 < D;
          const frag qa = in ? M::lds8(Qs + (g * 16 + l16) * LDK + dc * 32 + lg * 8) : M::zero();
          const frag ya = in ? M::lds8(Ys + (g * 16 + l16) * LDK + dc * 32 + lg * 8) : M::zero();
          Z[g] = M::mma(qa, kf[dc], Z[g]);
          P[g] = M::mma(ya, vf[dc], P[g]);
        }
      }
      const bool full = (i0 + 63 <= q0) && (i0 >= q0 + 64 - W) && (q0 + 63 < T);
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        float pv[8], gv[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int g = 2 * p + (jj >> 2);
          const int rr = g * 16 + lg * 4 + (jj & 3);
          const int t = q0 + rr;
          const bool band = full || (key <= t && key > t - W && t < T);
          const float pr = band ? fast_exp2(__builtin_fmaf(Z[g][jj & 3], sl2, -lse_s[rr])) : 0.0f;
          pv[jj] = pr;
          gv[jj] = tau * pr * (P[g][jj & 3] - del_s[rr]);
        }
        const frag pf = M::pack(pv), gf = M::pack(gv);
#pragma unroll
        for (int dt = 0; dt < NT; ++dt) {
          dV[dt] = M::mma(ColFrag2<E>::read(Ys + (32 * p + lg * 4) * LDK + dt * 16,
                                            Ys + (32 * p + 16 + lg * 4) * LDK + dt * 16, LDK, l16),
                          pf, dV[dt]);
          dK[dt] = M::mma(ColFrag2<E>::read(Qs + (32 * p + lg * 4) * LDK + dt * 16,
                                            Qs + (32 * p + 16 + lg * 4) * LDK + dt * 16, LDK, l16),
                          gf, dK[dt]);
        }
      }
    }
    if (key < T) {
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) {
        st4(dKg + (size_t)key * D + dt * 16 + lg * 4, dK[dt]);
        st4(dVg + (size_t)key * D + dt * 16 + lg * 4, dV[dt]);
      }
    }
  }
}

// dlambda[h] = sigma eta sum dl, deta[h] = sigma sum md,
// dgate[h] = sigma (1-sigma) eta sum md; sums over b then segments in order.
static __global__ void reduce_kernel(BwdArgs a) {
  const int h = blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= a.H) return;
  double smd = 0.0, sdl = 0.0;
  for (int b = 0; b < a.B; ++b) {
    const float* p = a.part + ((size_t)(b * a.H + h) * a.nseg) * 2;
    for (int s = 0; s < a.nseg; ++s) {
      smd += p[2 * s];
      sdl += p[2 * s + 1];
    }
  }
  const float sg = sigmoidf(a.gate[h]), eta = a.eta[h];
  a.dlam[h] = (float)(sg * eta * sdl);
  a.deta[h] = (float)(sg * smd);
  a.dgate[h] = (float)(sg * (1.0 - sg) * eta * smd);
}

template <class E, int D>
static hipError_t launch_bwd_impl(const BwdArgs& a, hipStream_t s) {
  const int BH = a.B * a.H;
  if (a.nseg > 1) {
    hipLaunchKernelGGL((bseg_fwd_kernel<E, D>), dim3(BH * (a.nseg - 1)), dim3(256), 0, s, a);
    hipLaunchKernelGGL((bchain_fwd_kernel<D>), dim3((D * D / 4 + 255) / 256, BH), dim3(256), 0, s, a);
    hipLaunchKernelGGL((bseg_rev_kernel<E, D>), dim3(BH * (a.nseg - 1)), dim3(256), 0, s, a);
    hipLaunchKernelGGL((bchain_rev_kernel<D>), dim3((D * D / 4 + 255) / 256, BH), dim3(256), 0, s, a);
  }
  hipLaunchKernelGGL((dq_kernel<E, D>), dim3(BH * a.nseg), dim3(256), 0, s, a);
  hipLaunchKernelGGL((dkdv_kernel<E, D>), dim3(BH * a.nseg), dim3(256), 0, s, a);
  hipLaunchKernelGGL(reduce_kernel, dim3((a.H + 63) / 64), dim3(64), 0, s, a);
  return hipGetLastError();
}

// This file is compiled twice: TC_BWD_BF16=1 builds the bf16 kernels (with
// matrix-core results kept in VGPRs, which removes most scratch spills of
// the D = 128 walks), TC_BWD_BF16=0 the float32 kernels (default register
// form: a float32 16x16x4 MFMA result copied between VGPR forms too early
// reads stale elements on gfx950).
#if TC_BWD_BF16
hipError_t launch_backward_bf16(const BwdArgs& a, int D, hipStream_t s) {
  switch (D) {
    case 16: return launch_bwd_impl<bf16, 16>(a, s);
    case 32: return launch_bwd_impl<bf16, 32>(a, s);
    case 64: return launch_bwd_impl<bf16, 64>(a, s);
    case 128: return launch_bwd_impl<bf16, 128>(a, s);
  }
  return hipErrorInvalidValue;
}
#else
hipError_t launch_backward_f32(const BwdArgs& a, int D, hipStream_t s) {
  switch (D) {
    case 16: return launch_bwd_impl<float, 16>(a, s);
    case 32: return launch_bwd_impl<float, 32>(a, s);
    case 64: return launch_bwd_impl<float, 64>(a, s);
    case 128: return launch_bwd_impl<float, 128>(a, s);
  }
  return hipErrorInvalidValue;
}
#endif

}  // namespace tck

// TC forward with the delta-rule write on gfx950.
//
// "Tensor Cache: Eviction-conditioned Associative Memory for Transformers",
// Figure 2, step 3: the evicted pair may update the memory with a delta rule
// instead of the plain outer product; the pages give no formula.  Reading
// (the Widrow-Hoff error correction that the related-work section names): the
// evicted key reads the memory before the write and only the error is stored,
//   u_e = v_e - k_e A,    A <- lambda A + eta k_e^T u_e      (A: D x D, eta inside).
// Everything else -- the window, the read m_t = q_t A_t, the gate -- is the
// layer of Sections 3.1-3.2.
//
// Chunked form (chunks of C = 64 consecutive evictions; A_c = memory before
// chunk c, n <= 64 writes, local index i, eviction e = 64 c + i):
//   u_i = v_i - lambda^i k_i A_c - eta sum_{j<i} lambda^(i-1-j) <k_i,k_j> u_j,
// i.e. (I + N) U = V - diag(lambda^i) K A_c with N strictly lower triangular,
// N_ij = eta lambda^(i-1-j) <k_i,k_j>.  With U' = (I+N)^-1 V and
// Wm = (I+N)^-1 diag(lambda^i) K (no dependence on A_c: every chunk at once),
//   U       = U' - Wm A_c,
//   A_{c+1} = lambda^n A_c + eta sum_i lambda^(n-1-i) k_i^T u_i,
// and the query at step t = W + e (e = 64 c + r) reads
//   m_t = lambda^(r+1) q_t A_c + eta sum_{j<=r} lambda^(r-j) <q_t,k_j> u_j
// (the exact scan's read with v replaced by u).  The transition between
// chunks is affine but not a scalar decay (the delta write projects the
// memory):  A_{c+1} = M_c A_c + B_c  with
//   M_c = lambda^n I - eta K^T diag(lambda^(n-1-i)) Wm,
//   B_c = eta K^T diag(lambda^(n-1-i)) U'.
// Affine maps compose, (M2,B2) o (M1,B1) = (M2 M1, M2 B1 + B2), so the states
// come from a two-level scan: groups of G chunks compose their maps (in
// parallel), a walk over the groups gives the group-start states, and each
// group then walks its own chunks from its start: a sequential depth of
// about 2 G + nch / G matrix products instead of nch.  With
// m = P U' + Qt A_c for P_rj = eta lambda^(r-j) <q_r,k_j> (j <= r) and
// Qt = diag(lambda^(r+1)) Q - P Wm, the read needs only A_c, U' and Wm.
//
// Kernels (float32 arithmetic throughout, the matrix products on the matrix
// cores in float32; D x D states kept transposed, A^T[c][a] = A[a][c]):
//   delta_chunk_kernel  : per chunk, U'^T and Wm^T (Gram matrix, forward
//                         substitution per column), M_c and B_c^T;
//   delta_group_kernel  : per group of G chunks, the composed map (M_g, B_g^T);
//   delta_walk_kernel   : per (b,h), the walk over the groups (and A_final);
//   delta_expand_kernel : per group, the walk over its chunks -> A_c^T;
//   delta_read_kernel   : sigma(g) m_t for every row (zero while t < W), the
//                         term the window-only forward adds before rounding y.
#include "tc_device.h"
#include "tc_launch.h"

namespace tck {

namespace {

constexpr int kDeltaC = 64;  // evictions per chunk

// 8 consecutive elements at p as floats.
__device__ __forceinline__ f32x8 ld8f(const float* p) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ f32x8 ld8f(const bf16* p) {
  const bf16x8 x = *(const bf16x8*)p;
  f32x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (float)x[j];
  return r;
}
__device__ __forceinline__ float ldf(const float* p) { return *p; }
__device__ __forceinline__ float ldf(const bf16* p) { return (float)*p; }

// Two runs of four floats (p0[0..3], p1[0..3]) as one fragment.
__device__ __forceinline__ f32x8 ld4x2f(const float* p0, const float* p1) {
  const f32x4 a = *(const f32x4*)p0, b = *(const f32x4*)p1;
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

}  // namespace

// Per chunk c of head bh: U'^T and Wm^T ([D][64]), M_c (row-major) and
// B_c^T.  grid = BH * nch, 256 threads.
template <class E, int D>
__global__ void __launch_bounds__(256) delta_chunk_kernel(DeltaArgs a) {
  using M = Mfma<float>;
  constexpr int C = kDeltaC, LDX = 2 * D + 4, LDN = C + 4, LDT = C + 4, NT = D / 16;
  constexpr int XN = C * LDX + C * LDN, XT_ = 2 * D * LDT;
  __shared__ __attribute__((aligned(16))) float KT[D * LDT];         // keys, rows d
  __shared__ __attribute__((aligned(16))) float big[XN > XT_ ? XN : XT_];
  __shared__ float pw[C + 1];  // lambda^n
  __shared__ float wv[C];      // eta lambda^(n-1-i), zero for i >= n
  float* const X = big;             // [V | lambda^i K] (rows i), solved in place into registers
  float* const N = big + C * LDX;   // N_ij, zero for j >= i
  float* const XT = big;            // after the solve: [U'^T ; Wm^T] (rows = columns of X)
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int bh = blockIdx.x / a.nch, c = blockIdx.x - bh * a.nch, h = bh % a.H;
  const int e0 = C * c, n = min(C, a.E - e0);
  const float lam = a.lam[h], eta = a.eta[h];
  if (tid <= C) pw[tid] = powi(lam, tid);
  if (tid < C) wv[tid] = tid < n ? eta * powi(lam, n - 1 - tid) : 0.0f;
  __syncthreads();
  // eviction e is token e of the sequence
  const E* kg = (const E*)a.k + ((size_t)bh * a.T + e0) * D;
  const E* vg = (const E*)a.v + ((size_t)bh * a.T + e0) * D;
  for (int x = tid; x < C * D; x += 256) {
    const int i = x / D, d = x - i * D;
    const float kv = i < n ? ldf(kg + (size_t)i * D + d) : 0.0f;
    const float vv = i < n ? ldf(vg + (size_t)i * D + d) : 0.0f;
    KT[d * LDT + i] = kv;
    X[i * LDX + d] = vv;
    X[i * LDX + D + d] = pw[i] * kv;
  }
  __syncthreads();
  // Gram matrix: wave w forms rows i of tile w; lane element ii of tile jt
  // is (j = 16 jt + 4 lg + ii, i = 16 w + l16).  (Operands read down the
  // columns of K^T: no row-major copy of the keys, so that two workgroups
  // fit a compute unit for D <= 64.)
  {
    const int i = 16 * wid + l16;
    auto kcol = [&](int row, int d0) {
      f32x8 f;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) f[jj] = KT[(d0 + jj) * LDT + row];
      return f;
    };
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      f32x4 g = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < (D + 31) / 32; ++kc) {
        const int d0 = 32 * kc + 8 * lg;
        const f32x8 ka = d0 < D ? kcol(16 * jt + l16, d0) : M::zero();
        const f32x8 kb = d0 < D ? kcol(i, d0) : M::zero();
        g = M::mma(ka, kb, g);
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int j = 16 * jt + 4 * lg + ii;
        N[i * LDN + j] = j < i ? eta * pw[i - 1 - j] * g[ii] : 0.0f;
      }
    }
  }
  __syncthreads();
  // (I + N) X = [V | lambda^i K] by forward substitution, one column per thread
  float x[C];
  const bool solver = tid < 2 * D;
  if (solver) {
#pragma unroll
    for (int i = 0; i < C; ++i) x[i] = X[i * LDX + tid];
#pragma unroll
    for (int i = 1; i < C; ++i) {
      float s = x[i];
#pragma unroll
      for (int j4 = 0; j4 < i; j4 += 4) {
        const f32x4 nv = *(const f32x4*)(N + i * LDN + j4);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          if (j4 + jj < i) s -= nv[jj] * x[j4 + jj];
      }
      x[i] = s;
    }
  }
  __syncthreads();  // X and N are read; XT reuses their space
  if (solver) {
#pragma unroll
    for (int i4 = 0; i4 < C; i4 += 4)
      *(f32x4*)(XT + tid * LDT + i4) = f32x4{x[i4], x[i4 + 1], x[i4 + 2], x[i4 + 3]};
  }
  __syncthreads();
  // U'^T and Wm^T to the workspace (rows of 64 floats, float4 stores)
  {
    float* up = a.UpT + ((size_t)bh * a.nch + c) * D * C;
    float* wm = a.WmT + ((size_t)bh * a.nch + c) * D * C;
    for (int x4 = tid; x4 < 2 * D * (C / 4); x4 += 256) {
      const int row = x4 / (C / 4), i4 = 4 * (x4 - row * (C / 4));
      const f32x4 val = *(const f32x4*)(XT + row * LDT + i4);
      *(f32x4*)((row < D ? up + (size_t)row * C : wm + (size_t)(row - D) * C) + i4) = val;
    }
  }
  // M_c[a][b] = lambda^n [a = b] - sum_i k_i[a] w_i Wm[i][b]   (tiles (at, bt))
  // B_c^T[q][p] = sum_i k_i[p] w_i U'[i][q]                    (tiles (pt, qt))
  // lane element ii is (row 16 t1 + 4 lg + ii, column 16 t2 + l16) of the product
  float* Mg = a.Mc + ((size_t)bh * a.nch + c) * D * D;
  float* Bg = a.BcT + ((size_t)bh * a.nch + c) * D * D;
  const float dn = pw[n];
  for (int t = wid; t < 2 * NT * NT; t += 4) {
    const bool isM = t < NT * NT;
    const int tt = isM ? t : t - NT * NT, t1 = tt / NT, t2 = tt - t1 * NT;
    const float* brow = XT + ((isM ? D : 0) + 16 * t2 + l16) * LDT;  // Wm^T or U'^T row
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const int i0 = 32 * kc + 8 * lg;
      f32x8 bf = ld8f(brow + i0);
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) bf[jj] *= wv[i0 + jj];
      acc = M::mma(ld8f(KT + (16 * t1 + l16) * LDT + i0), bf, acc);
    }
    if (isM) {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int ar = 16 * t1 + 4 * lg + ii, bc = 16 * t2 + l16;
        Mg[(size_t)ar * D + bc] = (ar == bc ? dn : 0.0f) - acc[ii];
      }
    } else {
      *(f32x4*)(Bg + (size_t)(16 * t2 + l16) * D + 16 * t1 + 4 * lg) = acc;
    }
  }
}

// One affine step on the matrix cores, X_out = M X_in (+ B), for the tiles of
// this wave (tile (pt, qt) = rows 16 pt.., columns 16 qt..; lane element ii
// is X_out[16 pt + 4 lg + ii][16 qt + l16]).  M row-major in global memory,
// X_in^T in LDS (row stride lda), B^T (nullable) in global memory.
template <int D, int NWV>
struct AffineStep {
  static constexpr int NT = D / 16, NKC = (D + 31) / 32, TPW = (NT * NT + NWV - 1) / NWV;
  f32x4 out[TPW];
  __device__ __forceinline__ void run(const float* Mrow, const float* XT, int lda, const float* BT, int wid, int l16,
                                      int lg) {
    using M = Mfma<float>;
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
      const int t = wid + NWV * m;
      if (t < NT * NT) {
        const int pt = t / NT, qt = t - pt * NT;
        f32x4 acc = BT ? *(const f32x4*)(BT + (size_t)(16 * qt + l16) * D + 16 * pt + 4 * lg)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
          const int d0 = 32 * kc + 8 * lg;
          if (d0 < D)
            acc = M::mma(ld8f(Mrow + (size_t)(16 * pt + l16) * D + d0), ld8f(XT + (16 * qt + l16) * lda + d0), acc);
        }
        out[m] = acc;
      }
    }
  }
  // X_out^T into LDS (and, if g, into global memory, row stride D)
  __device__ __forceinline__ void put(float* XT, int lda, float* g, int wid, int l16, int lg) const {
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
      const int t = wid + NWV * m;
      if (t < NT * NT) {
        const int pt = t / NT, qt = t - pt * NT, row = 16 * qt + l16, col = 16 * pt + 4 * lg;
        *(f32x4*)(XT + row * lda + col) = out[m];
        if (g) *(f32x4*)(g + (size_t)row * D + col) = out[m];
      }
    }
  }
};

constexpr int kDeltaWaves = 8;  // waves of the group, walk and expand kernels

// Per group g of head bh: the composed map of its chunks, M_g (row-major)
// and B_g^T.  grid = BH * ng, 512 threads.
template <int D>
__global__ void __launch_bounds__(64 * kDeltaWaves) delta_group_kernel(DeltaArgs a) {
  constexpr int LDA = D + 4;
  __shared__ __attribute__((aligned(16))) float PT[D * LDA];  // product of the maps so far (transposed)
  __shared__ __attribute__((aligned(16))) float QT[D * LDA];  // offset so far (transposed)
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int bh = blockIdx.x / a.ng, g = blockIdx.x - bh * a.ng;
  for (int x = tid; x < D * LDA; x += 64 * kDeltaWaves) {
    const int row = x / LDA, col = x - row * LDA;
    PT[x] = row == col ? 1.0f : 0.0f;
    QT[x] = 0.0f;
  }
  __syncthreads();
  const int c0 = g * a.G, c1 = min(a.nch, c0 + a.G);
  AffineStep<D, kDeltaWaves> st;  // (the two products one after the other: half the registers)
  for (int c = c0; c < c1; ++c) {
    const float* Mc = a.Mc + ((size_t)bh * a.nch + c) * D * D;
    st.run(Mc, PT, LDA, nullptr, wid, l16, lg);
    __syncthreads();
    st.put(PT, LDA, nullptr, wid, l16, lg);
    st.run(Mc, QT, LDA, a.BcT + ((size_t)bh * a.nch + c) * D * D, wid, l16, lg);
    __syncthreads();
    st.put(QT, LDA, nullptr, wid, l16, lg);
    __syncthreads();
  }
  float* Mg = a.Mg + ((size_t)bh * a.ng + g) * D * D;
  float* Bg = a.BgT + ((size_t)bh * a.ng + g) * D * D;
  for (int x = tid; x < D * D; x += 64 * kDeltaWaves) {
    const int row = x / D, col = x - row * D;
    Mg[x] = PT[col * LDA + row];
    Bg[x] = QT[row * LDA + col];
  }
}

// Per head: the walk over the groups, A^T at every group start, and the
// final memory.  grid = BH, 512 threads.
template <int D>
__global__ void __launch_bounds__(64 * kDeltaWaves) delta_walk_kernel(DeltaArgs a) {
  constexpr int LDA = D + 4;
  __shared__ __attribute__((aligned(16))) float AT[D * LDA];
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int bh = blockIdx.x;
  float* Ag = a.AgT + (size_t)bh * (a.ng + 1) * D * D;
  for (int x = tid; x < D * LDA; x += 64 * kDeltaWaves) AT[x] = 0.0f;
  for (int x = tid; x < D * D; x += 64 * kDeltaWaves) Ag[x] = 0.0f;
  __syncthreads();
  AffineStep<D, kDeltaWaves> st;
  for (int g = 0; g < a.ng; ++g) {
    st.run(a.Mg + ((size_t)bh * a.ng + g) * D * D, AT, LDA, a.BgT + ((size_t)bh * a.ng + g) * D * D, wid, l16, lg);
    __syncthreads();
    st.put(AT, LDA, Ag + (size_t)(g + 1) * D * D, wid, l16, lg);
    __syncthreads();
  }
  if (a.A_final) {
    float* Af = a.A_final + (size_t)bh * D * D;
    for (int x = tid; x < D * D; x += 64 * kDeltaWaves) {
      const int ar = x / D, col = x - ar * D;
      Af[x] = AT[col * LDA + ar];
    }
  }
}

// Per group: from its start state, the walk over its chunks, A^T at every
// chunk start.  grid = BH * ng, 512 threads.
template <int D>
__global__ void __launch_bounds__(64 * kDeltaWaves) delta_expand_kernel(DeltaArgs a) {
  constexpr int LDA = D + 4;
  __shared__ __attribute__((aligned(16))) float AT[D * LDA];
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int bh = blockIdx.x / a.ng, g = blockIdx.x - bh * a.ng;
  const float* Ag = a.AgT + ((size_t)bh * (a.ng + 1) + g) * D * D;
  const int c0 = g * a.G, c1 = min(a.nch, c0 + a.G);
  float* Ac0 = a.AcT + ((size_t)bh * a.nch + c0) * D * D;
  for (int x = tid; x < D * D; x += 64 * kDeltaWaves) {
    const int row = x / D, col = x - row * D;
    AT[row * LDA + col] = Ag[x];
    Ac0[x] = Ag[x];
  }
  __syncthreads();
  AffineStep<D, kDeltaWaves> st;
  for (int c = c0; c + 1 < c1; ++c) {
    st.run(a.Mc + ((size_t)bh * a.nch + c) * D * D, AT, LDA, a.BcT + ((size_t)bh * a.nch + c) * D * D, wid, l16,
           lg);
    __syncthreads();
    st.put(AT, LDA, a.AcT + ((size_t)bh * a.nch + c + 1) * D * D, wid, l16, lg);
    __syncthreads();
  }
}

// yadd_t = sigma(g) m_t for the rows of chunk c of head bh (rows t < W: zero,
// by the workgroups of chunk 0).  grid = BH * max(nch, 1), 256 threads; wave w
// takes rows 16 w .. 16 w + 15 of the chunk.  Everything in registers:
//   P_rj = eta lambda^(r-j) <q_r,k_j> (j <= r),  Qt = diag(lambda^(r+1)) Q - P Wm,
//   m = Qt A_c + P U'.
// The contraction slots of a fragment pair up two 16-wide tiles of the
// product before (index 32 kc + 4 lg + ii, then 32 kc + 16 + 4 lg + ii), and
// the other operand is read in the same order.
template <class E, int D>
__global__ void __launch_bounds__(256) delta_read_kernel(DeltaArgs a) {
  using M = Mfma<float>;
  constexpr int C = kDeltaC, NT = D / 16, NKC = (D + 31) / 32;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int nb = a.nch > 0 ? a.nch : 1;
  const int bh = blockIdx.x / nb, c = blockIdx.x - bh * nb, h = bh % a.H;
  float* yb = a.yadd + (size_t)bh * a.T * D;
  if (c == 0) {
    const int nz = min(a.W, a.T) * D;
    for (int x = tid; x < nz; x += 256) yb[x] = 0.0f;
  }
  if (c >= a.nch) return;
  const float lam = a.lam[h], eta = a.eta[h], sg = sigmoidf(a.gate[h]);
  const int e0 = C * c, n = min(C, a.E - e0);
  const int r = 16 * wid + l16;  // this lane's row of the chunk (query t = W + e0 + r)
  const E* qg = (const E*)a.q + ((size_t)bh * a.T + a.W + e0) * D;
  const E* kg = (const E*)a.k + ((size_t)bh * a.T + e0) * D;
  const float* AcT = a.AcT + ((size_t)bh * a.nch + c) * D * D;
  const float* UpT = a.UpT + ((size_t)bh * a.nch + c) * D * C;
  const float* WmT = a.WmT + ((size_t)bh * a.nch + c) * D * C;
  f32x8 qf[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) {
    const int d0 = 32 * kc + 8 * lg;
    qf[kc] = (r < n && d0 < D) ? ld8f(qg + (size_t)r * D + d0) : M::zero();
  }
  // P as two fragments (j slots as above)
  f32x8 pf[2];
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int jt = 2 * kc + half;
      f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < NKC; ++dc) {
        const int d0 = 32 * dc + 8 * lg;
        // (keys past the chunk's last eviction may lie past the sequence)
        const f32x8 kf = (d0 < D && 16 * jt + l16 < n) ? ld8f(kg + (size_t)(16 * jt + l16) * D + d0) : M::zero();
        s = M::mma(kf, qf[dc], s);
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int j = 16 * jt + 4 * lg + ii;
        pf[kc][4 * half + ii] = (j <= r && j < n) ? eta * powi(lam, r - j) * s[ii] : 0.0f;
      }
    }
  }
  // Qt^T tiles: element ii of tile at is Qt[r][16 at + 4 lg + ii]
  const float dr = powi(lam, r + 1);
  f32x4 qt[NT];
#pragma unroll
  for (int at = 0; at < NT; ++at) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const float* wr = WmT + (size_t)(16 * at + l16) * C + 32 * kc + 4 * lg;
      acc = M::mma(ld4x2f(wr, wr + 16), pf[kc], acc);
    }
    f32x4 q4;
    {
      const E* qp = qg + (size_t)r * D + 16 * at + 4 * lg;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) q4[ii] = r < n ? ldf(qp + ii) : 0.0f;
    }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) qt[at][ii] = dr * q4[ii] - acc[ii];
  }
  float* yrow = yb + (size_t)(a.W + e0 + r) * D;
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    f32x4 m = f32x4{0.f, 0.f, 0.f, 0.f};
    const int col = 16 * ct + l16;
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      if (32 * kc + 16 < D) {  // tiles 2 kc and 2 kc + 1 of Qt
        const f32x8 qq = f32x8{qt[2 * kc][0], qt[2 * kc][1], qt[2 * kc][2], qt[2 * kc][3],
                               qt[2 * kc + 1][0], qt[2 * kc + 1][1], qt[2 * kc + 1][2], qt[2 * kc + 1][3]};
        const float* ar = AcT + (size_t)col * D + 32 * kc + 4 * lg;
        m = M::mma(ld4x2f(ar, ar + 16), qq, m);
      } else {  // D = 16: one tile of Qt, the other half of the slots empty
        const f32x8 qq = f32x8{qt[2 * kc][0], qt[2 * kc][1], qt[2 * kc][2], qt[2 * kc][3], 0.f, 0.f, 0.f, 0.f};
        const float* ar = AcT + (size_t)col * D + 32 * kc + 4 * lg;
        const f32x4 a0 = *(const f32x4*)ar;
        m = M::mma(f32x8{a0[0], a0[1], a0[2], a0[3], 0.f, 0.f, 0.f, 0.f}, qq, m);
      }
    }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const float* ur = UpT + (size_t)col * C + 32 * kc + 4 * lg;
      m = M::mma(ld4x2f(ur, ur + 16), pf[kc], m);
    }
    if (r < n) {
      f32x4 o;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) o[ii] = sg * m[ii];
      *(f32x4*)(yrow + 16 * ct + 4 * lg) = o;
    }
  }
}

namespace {
template <class E, int D>
hipError_t launch_delta_impl(const DeltaArgs& a, hipStream_t s) {
  const int BH = a.B * a.H;
  const dim3 wide(64 * kDeltaWaves);
  if (a.nch > 0) {
    hipLaunchKernelGGL((delta_chunk_kernel<E, D>), dim3(BH * a.nch), dim3(256), 0, s, a);
    hipLaunchKernelGGL((delta_group_kernel<D>), dim3(BH * a.ng), wide, 0, s, a);
  }
  hipLaunchKernelGGL((delta_walk_kernel<D>), dim3(BH), wide, 0, s, a);
  if (a.nch > 0) hipLaunchKernelGGL((delta_expand_kernel<D>), dim3(BH * a.ng), wide, 0, s, a);
  hipLaunchKernelGGL((delta_read_kernel<E, D>), dim3(BH * (a.nch > 0 ? a.nch : 1)), dim3(256), 0, s, a);
  return hipGetLastError();
}
template <class E>
hipError_t launch_delta_e(const DeltaArgs& a, int D, hipStream_t s) {
  switch (D) {
    case 16: return launch_delta_impl<E, 16>(a, s);
    case 32: return launch_delta_impl<E, 32>(a, s);
    case 64: return launch_delta_impl<E, 64>(a, s);
    case 128: return launch_delta_impl<E, 128>(a, s);
  }
  return hipErrorInvalidValue;
}
}  // namespace

hipError_t launch_delta_memory(const DeltaArgs& a, int D, bool is_bf16, hipStream_t s) {
  return is_bf16 ? launch_delta_e<bf16>(a, D, s) : launch_delta_e<float>(a, D, s);
}

}  // namespace tck

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

// Eight (RawFrag8) or four (RawFrag4) consecutive elements loaded as raw
// bytes (zero when !ok) and converted to float only at their use.
template <class E>
struct RawFrag8;
template <>
struct RawFrag8<bf16> {
  uint4 v;
  __device__ __forceinline__ void load(const bf16* p, bool ok) { v = ok ? *(const uint4*)p : make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ f32x8 f32() const {
    const bf16x8 x = __builtin_bit_cast(bf16x8, v);
    f32x8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (float)x[j];
    return r;
  }
};
template <>
struct RawFrag8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p, bool ok) {
    a = ok ? *(const f32x4*)p : f32x4{0.f, 0.f, 0.f, 0.f};
    b = ok ? *(const f32x4*)(p + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __device__ __forceinline__ f32x8 f32() const { return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}; }
};
template <class E>
struct RawFrag4;
template <>
struct RawFrag4<bf16> {
  uint2 v;
  __device__ __forceinline__ void load(const bf16* p, bool ok) { v = ok ? *(const uint2*)p : make_uint2(0, 0); }
  __device__ __forceinline__ f32x4 f32() const {
    const bf16x4 x = __builtin_bit_cast(bf16x4, v);
    return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
  }
};
template <>
struct RawFrag4<float> {
  f32x4 v;
  __device__ __forceinline__ void load(const float* p, bool ok) { v = ok ? *(const f32x4*)p : f32x4{0.f, 0.f, 0.f, 0.f}; }
  __device__ __forceinline__ f32x4 f32() const { return v; }
};


}  // namespace

// Per chunk c of head bh: U'^T and Wm^T ([D][64]), M_c (row-major) and
// B_c^T.  grid = BH * nch, 256 threads.
template <class E, int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) delta_chunk_kernel(DeltaArgs a) {
  using M = Mfma<float>;
  constexpr int C = kDeltaC, LDN = C + 4, LDT = C + 4, NT = D / 16;
  constexpr int XN = D * LDT + C * LDN, XT_ = 2 * D * LDT;
  // (about 52 KB at D = 64: three workgroups per compute unit)
  __shared__ __attribute__((aligned(16))) float KT[D * LDT];         // keys, rows d
  __shared__ __attribute__((aligned(16))) float big[XN > XT_ ? XN : XT_];
  __shared__ float pw[C + 1];  // lambda^n
  __shared__ float wv[C];      // eta lambda^(n-1-i), zero for i >= n
  float* const VT = big;            // values, rows d (the right-hand sides V; the others are lambda^i K, from KT)
  float* const Nt = big + D * LDT;  // N^T: N_ij at j * LDN + i, zero for j >= i
  float* const XT = big;            // after the solve: [U'^T ; Wm^T] (rows = columns of the solution)
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
  {
    // the chunk's K and V rows as 16-byte vectors, every load in flight
    // before the first store (rows past the last eviction read as zero)
    constexpr int VE = 16 / (int)sizeof(E), VPR = D / VE, NV = C * VPR, PER = (NV + 255) / 256;
    uint4 kr[PER], vr[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int x = tid + 256 * p, i = x / VPR, d = (x - i * VPR) * VE;
      const bool ok = (NV % 256 == 0 || x < NV) && i < n;
      kr[p] = ok ? *(const uint4*)(kg + (size_t)i * D + d) : make_uint4(0, 0, 0, 0);
      vr[p] = ok ? *(const uint4*)(vg + (size_t)i * D + d) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int x = tid + 256 * p, i = x / VPR, d = (x - i * VPR) * VE;
      if (NV % 256 == 0 || x < NV) {
        const E* ke = (const E*)&kr[p];
        const E* ve = (const E*)&vr[p];
#pragma unroll
        for (int jj = 0; jj < VE; ++jj) {
          KT[(d + jj) * LDT + i] = (float)ke[jj];
          VT[(d + jj) * LDT + i] = (float)ve[jj];
        }
      }
    }
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
        if constexpr (sizeof(E) == 2) {
          // the keys are bf16 values: back to bf16 exactly, one bf16 op
          float xa[8], xb[8];
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            xa[jj] = ka[jj];
            xb[jj] = kb[jj];
          }
          g = Mfma<bf16>::mma(Mfma<bf16>::pack(xa), Mfma<bf16>::pack(xb), g);
        } else {
          g = M::mma(ka, kb, g);
        }
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int j = 16 * jt + 4 * lg + ii;
        Nt[j * LDN + i] = j < i ? eta * pw[i - 1 - j] * g[ii] : 0.0f;
      }
    }
  }
  __syncthreads();
  // (I + N) X = [V | lambda^i K] by forward substitution, one column per
  // thread, column-oriented: once x_j is final its term leaves every later
  // row (x_i -= N_ij x_j, i > j; each x_i receives its terms in the order
  // j = 0, 1, .. as in the row-oriented form).  The reads of column j of N
  // do not wait on the running sums, so they issue ahead of the arithmetic.
  float x[C];
  const bool solver = tid < 2 * D;
  if (solver) {
    // column tid of [V | lambda^i K]
    const bool isv = tid < D;
    const float* col0 = isv ? VT + tid * LDT : KT + (tid - D) * LDT;
#pragma unroll
    for (int i4 = 0; i4 < C; i4 += 4) {
      const f32x4 c4 = *(const f32x4*)(col0 + i4);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) x[i4 + ii] = isv ? c4[ii] : pw[i4 + ii] * c4[ii];
    }
    // (each 4-row slot of column j + 1 is loaded into the registers of the
    // same slot of column j as soon as that slot has been applied: one
    // column's registers instead of two, so that three workgroups fit a
    // compute unit, whose other waves cover the shorter lead)
    f32x4 col[C / 4];
#pragma unroll
    for (int i4 = 0; i4 < C; i4 += 4) col[i4 / 4] = *(const f32x4*)(Nt + i4);
#pragma unroll
    for (int j = 0; j < C - 1; ++j) {
#pragma unroll
      for (int i4 = (j + 1) & ~3; i4 < C; i4 += 4) {
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          if (i4 + ii > j) x[i4 + ii] -= col[i4 / 4][ii] * x[j];
        if (j + 2 < C && i4 + 3 > j + 1) col[i4 / 4] = *(const f32x4*)(Nt + (j + 1) * LDN + i4);
      }
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
  // (ldm, ldb: row strides of M and B^T, D in global memory)
  __device__ __forceinline__ void run(const float* Mrow, const float* XT, int lda, const float* BT, int wid, int l16,
                                      int lg, int ldm = D, int ldb = D) {
    using M = Mfma<float>;
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
      const int t = wid + NWV * m;
      if (t < NT * NT) {
        const int pt = t / NT, qt = t - pt * NT;
        f32x4 acc = BT ? *(const f32x4*)(BT + (size_t)(16 * qt + l16) * ldb + 16 * pt + 4 * lg)
                       : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
          const int d0 = 32 * kc + 8 * lg;
          if (d0 < D)
            acc = M::mma(ld8f(Mrow + (size_t)(16 * pt + l16) * ldm + d0), ld8f(XT + (16 * qt + l16) * lda + d0), acc);
        }
        out[m] = acc;
      }
    }
  }
  // The same step from operands fetched ahead into a StepOperands set
  // (below); only where they fit in registers (D <= 64), larger D uses run().
  static constexpr bool kFetch = TPW * NKC <= 8;
  struct Operands {
    f32x8 mf[kFetch ? TPW : 1][kFetch ? NKC : 1];
    f32x4 bf[kFetch ? TPW : 1];
    // M (row-major) and B^T (nullable) of one step
    __device__ __forceinline__ void fetch(const float* Mrow, const float* BT, int wid, int l16, int lg) {
      if constexpr (kFetch) {
#pragma unroll
        for (int m = 0; m < TPW; ++m) {
          const int t = wid + NWV * m;
          const int pt = t / NT, qt = t - pt * NT;
          const bool ok = t < NT * NT;
          bf[m] = (ok && BT) ? *(const f32x4*)(BT + (size_t)(16 * qt + l16) * D + 16 * pt + 4 * lg)
                             : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kc = 0; kc < NKC; ++kc) {
            const int d0 = 32 * kc + 8 * lg;
            mf[m][kc] = (ok && d0 < D) ? ld8f(Mrow + (size_t)(16 * pt + l16) * D + d0) : Mfma<float>::zero();
          }
        }
      }
    }
  };
  __device__ __forceinline__ void run_fetched(const Operands& o, const float* XT, int lda, bool addB, int wid,
                                              int l16, int lg) {
    using M = Mfma<float>;
    if constexpr (kFetch) {
#pragma unroll
      for (int m = 0; m < TPW; ++m) {
        const int t = wid + NWV * m;
        if (t < NT * NT) {
          const int qt = t % NT;
          f32x4 acc = addB ? o.bf[m] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kc = 0; kc < NKC; ++kc) {
            const int d0 = 32 * kc + 8 * lg;
            if (d0 < D) acc = M::mma(o.mf[m][kc], ld8f(XT + (16 * qt + l16) * lda + d0), acc);
          }
          out[m] = acc;
        }
      }
    }
  }
  // A step's X_out kept back (hold()) and written to global memory one step
  // later (store_held(), row stride D, transposed): a wait for the next
  // step's operand loads then never covers stores issued just before it.
  f32x4 held[TPW];
  __device__ __forceinline__ void hold() {
#pragma unroll
    for (int m = 0; m < TPW; ++m) held[m] = out[m];
  }
  __device__ __forceinline__ void store_held(float* g, int wid, int l16, int lg) const {
#pragma unroll
    for (int m = 0; m < TPW; ++m) {
      const int t = wid + NWV * m;
      if (t < NT * NT) {
        const int pt = t / NT, qt = t - pt * NT;
        *(f32x4*)(g + (size_t)(16 * qt + l16) * D + 16 * pt + 4 * lg) = held[m];
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

// One level of the scan over affine maps X <- M X + B, per head bh: n maps
// (M row-major at M + (bh n + i) D^2, B^T likewise), taken in groups of gs.
// The group kernel composes each group into Mo, BoT ([BH][ceil(n/gs)]); the
// walk runs the n maps from zero, storing the state before each map and after
// the last at AoT ([BH][n+1], transposed) and the last also at A_final; the
// expand kernel starts group g from A0T[bh][g] (a0_stride states per head)
// and stores the state before each of its maps at AoT[bh][i] (ao_stride).
struct ScanLevel {
  const float* M;
  const float* BT;
  int n, gs;
  float* Mo;
  float* BoT;
  const float* A0T;
  int a0_stride;
  float* AoT;
  int ao_stride;
  float* A_final;
};

// Steps s = 0 .. n-1 of a walk whose step operands come three steps ahead:
// fetch(o, s) loads step s into the operand set o, apply(o, s) runs step s
// from it.  Three sets rotate (the loop is unrolled by three so that each is
// addressed at compile time); a step's loads are issued when the set is free,
// two steps before their use, so their latency hides behind those steps.
template <class Ops, class Fetch, class Apply>
__device__ __forceinline__ void walk3(Ops (&o)[3], int n, Fetch fetch, Apply apply) {
#pragma unroll
  for (int u = 0; u < 3; ++u)
    if (u < n) fetch(o[u], u);
  for (int s0 = 0; s0 < n; s0 += 3) {
#pragma unroll
    for (int u = 0; u < 3; ++u) {
      const int s = s0 + u;
      if (s < n) {
        apply(o[u], s);
        if (s + 3 < n) fetch(o[u], s + 3);
      }
    }
  }
}

// Per group g of head bh: the composed map of its maps (row-major) and its
// offset (transposed).  grid = BH * ceil(n / gs), 512 threads.
template <int D>
__global__ void __launch_bounds__(64 * kDeltaWaves) delta_group_kernel(ScanLevel L) {
  constexpr int LDA = D + 4;
  __shared__ __attribute__((aligned(16))) float PT[D * LDA];  // product of the maps so far (transposed)
  __shared__ __attribute__((aligned(16))) float QT[D * LDA];  // offset so far (transposed)
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int ngo = (L.n + L.gs - 1) / L.gs;
  const int bh = blockIdx.x / ngo, g = blockIdx.x - bh * ngo;
  const int c0 = g * L.gs, c1 = min(L.n, c0 + L.gs);  // (c0 < c1: no group is empty)
  auto mc = [&](int c) { return L.M + ((size_t)bh * L.n + c) * D * D; };
  auto bc = [&](int c) { return L.BT + ((size_t)bh * L.n + c) * D * D; };
  {
    // the group's first map as it is (its product with the identity and the
    // zero offset would give the same values exactly)
    const float* m0 = mc(c0);
    const float* b0 = bc(c0);
    for (int x = tid; x < D * D; x += 64 * kDeltaWaves) {
      const int row = x / D, col = x - row * D;
      PT[col * LDA + row] = m0[x];
      QT[row * LDA + col] = b0[x];
    }
  }
  __syncthreads();
  AffineStep<D, kDeltaWaves> st;  // (the two products one after the other: half the registers)
  if constexpr (AffineStep<D, kDeltaWaves>::kFetch) {
    // (one set of operands, the next chunk's loaded during this one's second
    // product: here, unlike the walk, the registers of more sets would cost
    // resident workgroups)
    typename AffineStep<D, kDeltaWaves>::Operands o;
    if (c0 + 1 < c1) o.fetch(mc(c0 + 1), bc(c0 + 1), wid, l16, lg);
    for (int c = c0 + 1; c < c1; ++c) {
      st.run_fetched(o, PT, LDA, false, wid, l16, lg);
      __syncthreads();
      st.put(PT, LDA, nullptr, wid, l16, lg);
      st.run_fetched(o, QT, LDA, true, wid, l16, lg);
      if (c + 1 < c1) o.fetch(mc(c + 1), bc(c + 1), wid, l16, lg);
      __syncthreads();
      st.put(QT, LDA, nullptr, wid, l16, lg);
      __syncthreads();
    }
  } else {
    for (int c = c0 + 1; c < c1; ++c) {
      st.run(mc(c), PT, LDA, nullptr, wid, l16, lg);
      __syncthreads();
      st.put(PT, LDA, nullptr, wid, l16, lg);
      st.run(mc(c), QT, LDA, bc(c), wid, l16, lg);
      __syncthreads();
      st.put(QT, LDA, nullptr, wid, l16, lg);
      __syncthreads();
    }
  }
  float* Mg = L.Mo + ((size_t)bh * ngo + g) * D * D;
  float* Bg = L.BoT + ((size_t)bh * ngo + g) * D * D;
  for (int x = tid; x < D * D; x += 64 * kDeltaWaves) {
    const int row = x / D, col = x - row * D;
    Mg[x] = PT[col * LDA + row];
    Bg[x] = QT[row * LDA + col];
  }
}

// Per head: the walk over the level's maps from zero, A^T before every map
// (and after the last), and the final memory.  grid = BH, 512 threads.
template <int D>
__global__ void __launch_bounds__(64 * kDeltaWaves) delta_walk_kernel(ScanLevel L) {
  constexpr int LDA = D + 4;
  __shared__ __attribute__((aligned(16))) float AT[D * LDA];
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int bh = blockIdx.x;
  float* Ag = L.AoT + (size_t)bh * (L.n + 1) * D * D;
  auto mg = [&](int g) { return L.M + ((size_t)bh * L.n + g) * D * D; };
  auto bg = [&](int g) { return L.BT + ((size_t)bh * L.n + g) * D * D; };
  // A_0 = 0 and A_1 = M_0 A_0 + B_0 = B_0: the first map applied as it is
  for (int x = tid; x < D * D; x += 64 * kDeltaWaves) {
    const int q = x / D, p = x - q * D;  // (B_0^T row-major: B_0[p][q] at q D + p)
    const float b = L.n > 0 ? bg(0)[x] : 0.0f;
    AT[q * LDA + p] = b;
    Ag[x] = 0.0f;
    if (L.n > 0) Ag[(size_t)D * D + x] = b;
  }
  __syncthreads();
  AffineStep<D, kDeltaWaves> st;
  if constexpr (AffineStep<D, kDeltaWaves>::kFetch) {
    // (each step's state goes to global memory one step late, after the next
    // step's products: see hold(); step s applies map s + 1)
    using Ops = typename AffineStep<D, kDeltaWaves>::Operands;
    Ops ops[3];
    walk3(
        ops, L.n > 0 ? L.n - 1 : 0, [&](Ops& o, int s) { o.fetch(mg(s + 1), bg(s + 1), wid, l16, lg); },
        [&](Ops& o, int s) {
          const int g = s + 1;
          st.run_fetched(o, AT, LDA, true, wid, l16, lg);
          if (s > 0) st.store_held(Ag + (size_t)g * D * D, wid, l16, lg);
          __syncthreads();
          st.put(AT, LDA, nullptr, wid, l16, lg);
          st.hold();
          if (g + 1 == L.n) st.store_held(Ag + (size_t)L.n * D * D, wid, l16, lg);
          __syncthreads();
        });
  } else {
    for (int g = 1; g < L.n; ++g) {
      st.run(mg(g), AT, LDA, bg(g), wid, l16, lg);
      __syncthreads();
      st.put(AT, LDA, Ag + (size_t)(g + 1) * D * D, wid, l16, lg);
      __syncthreads();
    }
  }
  if (L.A_final) {
    float* Af = L.A_final + (size_t)bh * D * D;
    for (int x = tid; x < D * D; x += 64 * kDeltaWaves) {
      const int ar = x / D, col = x - ar * D;
      Af[x] = AT[col * LDA + ar];
    }
  }
}

// Per group: from its start state, the walk over its maps, A^T before each.
// grid = BH * ceil(n / gs), 512 threads.
template <int D>
__global__ void __launch_bounds__(64 * kDeltaWaves) delta_expand_kernel(ScanLevel L) {
  constexpr int LDA = D + 4;
  __shared__ __attribute__((aligned(16))) float AT[D * LDA];
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int ngo = (L.n + L.gs - 1) / L.gs;
  const int bh = blockIdx.x / ngo, g = blockIdx.x - bh * ngo;
  const float* Ag = L.A0T + ((size_t)bh * L.a0_stride + g) * D * D;
  const int c0 = g * L.gs, c1 = min(L.n, c0 + L.gs);
  auto aout = [&](int c) { return L.AoT + ((size_t)bh * L.ao_stride + c) * D * D; };
  float* Ac0 = aout(c0);
  {
    // the group's start state: every load in flight before the first store
    constexpr int NV = D * D / 4, PER = (NV + 64 * kDeltaWaves - 1) / (64 * kDeltaWaves);
    f32x4 v[PER];
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int x4 = tid + 64 * kDeltaWaves * p;
      if (NV % (64 * kDeltaWaves) == 0 || x4 < NV) v[p] = *(const f32x4*)(Ag + 4 * x4);
    }
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int x4 = tid + 64 * kDeltaWaves * p;
      if (NV % (64 * kDeltaWaves) == 0 || x4 < NV) {
        const int row = (4 * x4) / D, col = 4 * x4 - row * D;
        *(f32x4*)(AT + row * LDA + col) = v[p];
        *(f32x4*)(Ac0 + 4 * x4) = v[p];
      }
    }
  }
  __syncthreads();
  AffineStep<D, kDeltaWaves> st;
  auto mc = [&](int c) { return L.M + ((size_t)bh * L.n + c) * D * D; };
  auto bc = [&](int c) { return L.BT + ((size_t)bh * L.n + c) * D * D; };
  if constexpr (AffineStep<D, kDeltaWaves>::kFetch) {
    // (one set of operands, as in the group kernel; each state goes to
    // global memory one step late, as in the walk)
    typename AffineStep<D, kDeltaWaves>::Operands o;
    if (c0 + 1 < c1) o.fetch(mc(c0), bc(c0), wid, l16, lg);
    for (int c = c0; c + 1 < c1; ++c) {
      st.run_fetched(o, AT, LDA, true, wid, l16, lg);
      if (c > c0) st.store_held(aout(c), wid, l16, lg);
      __syncthreads();
      st.put(AT, LDA, nullptr, wid, l16, lg);
      st.hold();
      if (c + 2 < c1) o.fetch(mc(c + 1), bc(c + 1), wid, l16, lg);
      __syncthreads();
    }
    if (c0 + 1 < c1) st.store_held(aout(c1 - 1), wid, l16, lg);
  } else {
    for (int c = c0; c + 1 < c1; ++c) {
      st.run(mc(c), AT, LDA, bc(c), wid, l16, lg);
      __syncthreads();
      st.put(AT, LDA, aout(c + 1), wid, l16, lg);
      __syncthreads();
    }
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
// The read of chunk c of head bh by four waves (256 threads): A_c^T at AcT,
// row stride lda (global memory, or the expanding kernel's LDS copy).
template <class E, int D>
__device__ __forceinline__ void delta_read_chunk(const DeltaArgs& a, int bh, int c, const float* AcT, int lda) {
  using M = Mfma<float>;
  constexpr int C = kDeltaC, NT = D / 16, NKC = (D + 31) / 32;
  // The operands arrive in three rounds of loads, each issued as a whole
  // before any of it is used (a scheduling barrier keeps the compiler from
  // interleaving them with their uses): the query rows and keys; W_m^T and
  // the query's columns (for D <= 64 already with the first round); then A_c^T
  // and U'^T, two column tiles at a time.
  constexpr bool EARLY = D <= 64;
  constexpr int CTB = NT >= 2 ? 2 : 1;  // column tiles per round of A_c / U' loads
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  (void)tid;
  const int h = bh % a.H;
  float* yb = a.yadd + (size_t)bh * a.T * D;
  const float lam = a.lam[h], eta = a.eta[h], sg = sigmoidf(a.gate[h]);
  const int e0 = C * c, n = min(C, a.E - e0);
  const int r = 16 * wid + l16;  // this lane's row of the chunk (query t = W + e0 + r)
  const E* qg = (const E*)a.q + ((size_t)bh * a.T + a.W + e0) * D;
  const E* kg = (const E*)a.k + ((size_t)bh * a.T + e0) * D;
  const float* UpT = a.UpT + ((size_t)bh * a.nch + c) * D * C;
  const float* WmT = a.WmT + ((size_t)bh * a.nch + c) * D * C;

  RawFrag8<E> qr[NKC], kr[4][NKC];
  RawFrag4<E> q4r[NT];
  f32x4 wm[NT][2][2];
  auto load_wm = [&]() {
#pragma unroll
    for (int at = 0; at < NT; ++at) {
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const float* wr = WmT + (size_t)(16 * at + l16) * C + 32 * kc + 4 * lg;
        wm[at][kc][0] = *(const f32x4*)wr;
        wm[at][kc][1] = *(const f32x4*)(wr + 16);
      }
      q4r[at].load(qg + (size_t)r * D + 16 * at + 4 * lg, r < n);
    }
  };
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) {
    const int d0 = 32 * kc + 8 * lg;
    qr[kc].load(qg + (size_t)r * D + d0, r < n && d0 < D);
  }
#pragma unroll
  for (int jt = 0; jt < 4; ++jt)
#pragma unroll
    for (int dc = 0; dc < NKC; ++dc) {
      const int d0 = 32 * dc + 8 * lg;
      // (keys past the chunk's last eviction may lie past the sequence)
      kr[jt][dc].load(kg + (size_t)(16 * jt + l16) * D + d0, d0 < D && 16 * jt + l16 < n);
    }
  if constexpr (EARLY) load_wm();
  __builtin_amdgcn_sched_barrier(0);
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
        // bf16 inputs: one bf16 matrix-core op (exact products, float32 sums)
        // instead of eight float32 ones on the same values
        if constexpr (sizeof(E) == 2)
          s = Mfma<bf16>::mma(__builtin_bit_cast(bf16x8, kr[jt][dc].v), __builtin_bit_cast(bf16x8, qr[dc].v), s);
        else
          s = M::mma(kr[jt][dc].f32(), qr[dc].f32(), s);
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int j = 16 * jt + 4 * lg + ii;
        pf[kc][4 * half + ii] = (j <= r && j < n) ? eta * powi(lam, r - j) * s[ii] : 0.0f;
      }
    }
  }
  if constexpr (!EARLY) {
    load_wm();
    __builtin_amdgcn_sched_barrier(0);
  }
  // Qt^T tiles: element ii of tile at is Qt[r][16 at + 4 lg + ii]
  const float dr = powi(lam, r + 1);
  f32x4 qt[NT];
#pragma unroll
  for (int at = 0; at < NT; ++at) {
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const f32x4 w0 = wm[at][kc][0], w1 = wm[at][kc][1];
      acc = M::mma(f32x8{w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3]}, pf[kc], acc);
    }
    const f32x4 q4 = q4r[at].f32();
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) qt[at][ii] = dr * q4[ii] - acc[ii];
  }
  float* yrow = yb + (size_t)(a.W + e0 + r) * D;
#pragma unroll
  for (int cb = 0; cb < NT; cb += CTB) {
    f32x4 av[CTB][NKC][2], uv[CTB][2][2];
#pragma unroll
    for (int u = 0; u < CTB; ++u) {
      const int col = 16 * (cb + u) + l16;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const float* ar = AcT + (size_t)col * lda + 32 * kc + 4 * lg;
        av[u][kc][0] = *(const f32x4*)ar;
        // (D = 16: one tile of Qt, the other half of the slots empty)
        av[u][kc][1] = 32 * kc + 16 < D ? *(const f32x4*)(ar + 16) : f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const float* ur = UpT + (size_t)col * C + 32 * kc + 4 * lg;
        uv[u][kc][0] = *(const f32x4*)ur;
        uv[u][kc][1] = *(const f32x4*)(ur + 16);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < CTB; ++u) {
      const int ct = cb + u;
      f32x4 m = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const f32x4 x0 = qt[2 * kc], x1 = 32 * kc + 16 < D ? qt[2 * kc + 1] : f32x4{0.f, 0.f, 0.f, 0.f};
        const f32x8 qq = f32x8{x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
        const f32x4 a0 = av[u][kc][0], a1 = av[u][kc][1];
        m = M::mma(f32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]}, qq, m);
      }
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const f32x4 u0 = uv[u][kc][0], u1 = uv[u][kc][1];
        m = M::mma(f32x8{u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]}, pf[kc], m);
      }
      if (r < n) {
        f32x4 o;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) o[ii] = sg * m[ii];
        *(f32x4*)(yrow + 16 * ct + 4 * lg) = o;
      }
    }
  }
}

template <class E, int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 3))) delta_read_kernel(DeltaArgs a) {
  const int nb = a.nch > 0 ? a.nch : 1;
  const int bh = blockIdx.x / nb, c = blockIdx.x - bh * nb;
  if (c == 0) {
    float* yb = a.yadd + (size_t)bh * a.T * D;
    const int nz = min(a.W, a.T) * D;
    for (int x = threadIdx.x; x < nz; x += 256) yb[x] = 0.0f;
  }
  if (c >= a.nch) return;
  delta_read_chunk<E, D>(a, bh, c, a.AcT + ((size_t)bh * a.nch + c) * D * D, D);
}

// The last expansion fused with the read (D <= 64): per group of chunks,
// from the group's start state, the read of each chunk from A_c in LDS and
// the step to A_{c+1}; A_c never goes to global memory.  The four waves run
// the read of chunk c, then the step (both read A_c^T; a barrier before the
// new state replaces it).  The step's M_c and B_c^T are loaded before the
// read, which covers their latency, and parked in LDS after it.
// grid = BH * ceil(nch / gs), 256 threads.
template <class E, int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 3)))
    delta_expand_read_kernel(DeltaArgs a, ScanLevel L) {
  constexpr int LDA = D + 4;
  __shared__ __attribute__((aligned(16))) float AT[D * LDA];
  __shared__ __attribute__((aligned(16))) float MS[D * LDA];  // M_c, row stride LDA
  __shared__ __attribute__((aligned(16))) float BS[D * LDA];  // B_c^T, row stride LDA
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int ngo = (L.n + L.gs - 1) / L.gs;
  const int bh = blockIdx.x / ngo, g = blockIdx.x - bh * ngo;
  const int c0 = g * L.gs, c1 = min(L.n, c0 + L.gs);
  if (g == 0) {  // rows t < W read no memory
    float* yb = a.yadd + (size_t)bh * a.T * D;
    const int nz = min(a.W, a.T) * D;
    for (int x = tid; x < nz; x += 256) yb[x] = 0.0f;
  }
  {
    const float* A0 = L.A0T + ((size_t)bh * L.a0_stride + g) * D * D;
    for (int x4 = 4 * tid; x4 < D * D; x4 += 4 * 256) {
      const int q = x4 / D, p = x4 - q * D;
      *(f32x4*)(AT + q * LDA + p) = *(const f32x4*)(A0 + x4);
    }
  }
  __syncthreads();
  AffineStep<D, 4> st;
  constexpr int NV4 = D * D / 4, PER = (NV4 + 255) / 256;  // float4 vectors of one matrix; per thread
  for (int c = c0; c < c1; ++c) {
    const bool step = c + 1 < c1;
    f32x4 mreg[PER], breg[PER];
    if (step) {
      const f32x4* Mc = (const f32x4*)(L.M + ((size_t)bh * L.n + c) * D * D);
      const f32x4* Bc = (const f32x4*)(L.BT + ((size_t)bh * L.n + c) * D * D);
#pragma unroll
      for (int v = 0; v < PER; ++v) {
        const int x = tid + 256 * v;
        mreg[v] = (NV4 % 256 == 0 || x < NV4) ? Mc[x] : f32x4{0.f, 0.f, 0.f, 0.f};
        breg[v] = (NV4 % 256 == 0 || x < NV4) ? Bc[x] : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    delta_read_chunk<E, D>(a, bh, c, AT, LDA);
    if (step) {
#pragma unroll
      for (int v = 0; v < PER; ++v) {
        const int x = tid + 256 * v, row = 4 * x / D, col = 4 * x - row * D;
        if (NV4 % 256 == 0 || x < NV4) {
          *(f32x4*)(MS + row * LDA + col) = mreg[v];
          *(f32x4*)(BS + row * LDA + col) = breg[v];
        }
      }
      __syncthreads();
      st.run(MS, AT, LDA, BS, wid, l16, lg, LDA, LDA);
      __syncthreads();
      st.put(AT, LDA, nullptr, wid, l16, lg);
      __syncthreads();
    }
  }
}

namespace {
template <class E, int D>
hipError_t launch_delta_impl(const DeltaArgs& a, hipStream_t s) {
  const int BH = a.B * a.H;
  const dim3 wide(64 * kDeltaWaves);
  // levels: chunk maps -> groups of G (-> supergroups of G2 groups when nsg > 0)
  const ScanLevel chunks{a.Mc, a.BcT, a.nch, a.G, a.Mg, a.BgT, a.AgT, a.ng + 1, a.AcT, a.nch, nullptr};
  const ScanLevel groups{a.Mg, a.BgT, a.ng, a.G2, a.Ms, a.BsT, a.AsT, a.nsg + 1, a.AgT, a.ng + 1, nullptr};
  if (a.nch > 0) {
    hipLaunchKernelGGL((delta_chunk_kernel<E, D>), dim3(BH * a.nch), dim3(256), 0, s, a);
    hipLaunchKernelGGL((delta_group_kernel<D>), dim3(BH * a.ng), wide, 0, s, chunks);
    if (a.nsg > 0) hipLaunchKernelGGL((delta_group_kernel<D>), dim3(BH * a.nsg), wide, 0, s, groups);
  }
  // the walk over the top level's maps (none when there are no evictions)
  const ScanLevel top = a.nsg > 0 ? ScanLevel{a.Ms, a.BsT, a.nsg, 1, nullptr, nullptr, nullptr, 0, a.AsT, a.nsg + 1,
                                              a.A_final}
                                  : ScanLevel{a.Mg, a.BgT, a.ng, 1, nullptr, nullptr, nullptr, 0, a.AgT, a.ng + 1,
                                              a.A_final};
  hipLaunchKernelGGL((delta_walk_kernel<D>), dim3(BH), wide, 0, s, top);
  if (a.nch > 0) {
    if (a.nsg > 0) hipLaunchKernelGGL((delta_expand_kernel<D>), dim3(BH * a.nsg), wide, 0, s, groups);
    if constexpr (D <= 64) {
      // the expansion over the chunks and the read in one kernel (no A_c in global memory)
      hipLaunchKernelGGL((delta_expand_read_kernel<E, D>), dim3(BH * a.ng), dim3(256), 0, s, a, chunks);
      return hipGetLastError();
    }
    hipLaunchKernelGGL((delta_expand_kernel<D>), dim3(BH * a.ng), wide, 0, s, chunks);
  }
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

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
// chunks is not a scalar decay (the delta write projects the memory), so the
// states A_c come from a walk over the chunks, one workgroup per (b,h).
//
// Kernels (float32 arithmetic throughout, the matrix products on the matrix
// cores in float32):
//   delta_chunk_kernel : U' and Wm of every chunk (Gram matrix, then a
//                        forward substitution per column);
//   delta_chain_kernel : the walk A_c -> A_{c+1}, storing A_c^T and U^T;
//   delta_read_kernel  : sigma(g) m_t for every row (zero while t < W), the
//                        term the window-only forward adds before rounding y.
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

// U' and Wm of chunk c of head bh.  grid = BH * nch, 256 threads.
template <class E, int D>
__global__ void __launch_bounds__(256) delta_chunk_kernel(DeltaArgs a) {
  using M = Mfma<float>;
  constexpr int C = kDeltaC, LDKF = D + 4, LDX = 2 * D + 4, LDN = C + 4;
  __shared__ __attribute__((aligned(16))) float Kf[C * LDKF];  // the chunk's keys
  __shared__ __attribute__((aligned(16))) float X[C * LDX];    // [V | lambda^i K], then [U' | Wm]
  __shared__ __attribute__((aligned(16))) float N[C * LDN];    // N_ij, zero for j >= i
  __shared__ float pw[C + 1];                                  // lambda^n
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int bh = blockIdx.x / a.nch, c = blockIdx.x - bh * a.nch, h = bh % a.H;
  const int e0 = C * c, n = min(C, a.E - e0);
  const float lam = a.lam[h], eta = a.eta[h];
  if (tid <= C) pw[tid] = powi(lam, tid);
  __syncthreads();
  // eviction e is token e of the sequence
  const E* kg = (const E*)a.k + ((size_t)bh * a.T + e0) * D;
  const E* vg = (const E*)a.v + ((size_t)bh * a.T + e0) * D;
  for (int x = tid; x < C * D; x += 256) {
    const int i = x / D, d = x - i * D;
    const float kv = i < n ? ldf(kg + (size_t)i * D + d) : 0.0f;
    const float vv = i < n ? ldf(vg + (size_t)i * D + d) : 0.0f;
    Kf[i * LDKF + d] = kv;
    X[i * LDX + d] = vv;
    X[i * LDX + D + d] = pw[i] * kv;
  }
  __syncthreads();
  // Gram matrix on the matrix cores: wave w forms rows i of tile w, all j
  // tiles; lane element ii of tile (jt) is (j = 16 jt + 4 lg + ii, i = 16 w + l16)
  {
    const int i = 16 * wid + l16;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      f32x4 g = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < D / 32 + (D % 32 ? 1 : 0); ++kc) {
        const int d0 = 32 * kc + 8 * lg;
        const f32x8 ka = d0 < D ? ld8f(Kf + (16 * jt + l16) * LDKF + d0) : M::zero();
        const f32x8 kb = d0 < D ? ld8f(Kf + i * LDKF + d0) : M::zero();
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
  for (int col = tid; col < 2 * D; col += 256) {
    float x[C];
#pragma unroll
    for (int i = 0; i < C; ++i) x[i] = X[i * LDX + col];
#pragma unroll
    for (int i = 1; i < C; ++i) {
      float s = x[i];
#pragma unroll
      for (int j4 = 0; j4 < i; j4 += 4) {
        const f32x4 nv = *(const f32x4*)(N + i * LDN + j4);  // (zero at j >= i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          if (j4 + jj < i) s -= nv[jj] * x[j4 + jj];
      }
      x[i] = s;
    }
    float* dst = (col < D ? a.Up : a.Wm) + ((size_t)bh * a.nch + c) * C * D + (col < D ? col : col - D);
#pragma unroll
    for (int i = 0; i < C; ++i) dst[(size_t)i * D] = x[i];
  }
}

// The walk over the chunks of head bh: A_c^T (stored for the reads), U^T of
// every chunk, and the final memory.  grid = BH, 256 threads.
template <class E, int D>
__global__ void __launch_bounds__(256) delta_chain_kernel(DeltaArgs a) {
  using M = Mfma<float>;
  constexpr int C = kDeltaC, LDA = D + 4, LDU = C + 4, NT = D / 16;
  __shared__ __attribute__((aligned(16))) float At[D * LDA];  // A^T: At[c][a] = A[a][c]
  __shared__ __attribute__((aligned(16))) float Ut[D * LDU];  // U^T of the chunk, eta lambda^(n-1-i) applied
  __shared__ __attribute__((aligned(16))) float Kt[D * LDU];  // K^T of the chunk
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int bh = blockIdx.x, h = bh % a.H;
  const float lam = a.lam[h], eta = a.eta[h];
  for (int x = tid; x < D * LDA; x += 256) At[x] = 0.0f;  // A_0 = 0
  __syncthreads();
  float* AcT = a.AcT + (size_t)bh * (a.nch + 1) * D * D;
  for (int x = tid; x < D * D; x += 256) AcT[x] = 0.0f;
  for (int c = 0; c < a.nch; ++c) {
    const int e0 = C * c, n = min(C, a.E - e0);
    const E* kg = (const E*)a.k + ((size_t)bh * a.T + e0) * D;
    for (int x = tid; x < C * D; x += 256) {
      const int i = x / D, d = x - i * D;
      Kt[d * LDU + i] = i < n ? ldf(kg + (size_t)i * D + d) : 0.0f;
    }
    // (a) U^T = U'^T - (Wm A)^T: tile (ct, it), lane element ii is
    // (col = 16 ct + 4 lg + ii, i = 16 it + l16)
    const float* Up = a.Up + ((size_t)bh * a.nch + c) * C * D;
    const float* Wm = a.Wm + ((size_t)bh * a.nch + c) * C * D;
    float* Ug = a.Ut + ((size_t)bh * a.nch + c) * D * C;
    for (int t = wid; t < NT * 4; t += 4) {
      const int ct = t >> 2, it = t & 3, i = 16 * it + l16;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < (D + 31) / 32; ++kc) {
        const int d0 = 32 * kc + 8 * lg;
        const f32x8 af = d0 < D ? ld8f(At + (16 * ct + l16) * LDA + d0) : M::zero();
        const f32x8 bf = d0 < D ? ld8f(Wm + (size_t)i * D + d0) : M::zero();
        acc = M::mma(af, bf, acc);
      }
      const f32x4 up = *(const f32x4*)(Up + (size_t)i * D + 16 * ct + 4 * lg);
      const float wi = i < n ? eta * powi(lam, n - 1 - i) : 0.0f;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int col = 16 * ct + 4 * lg + ii;
        const float u = up[ii] - acc[ii];
        Ug[(size_t)col * C + i] = u;
        Ut[col * LDU + i] = wi * u;
      }
    }
    __syncthreads();  // every wave has read A_c; U^T and K^T are complete
    // (b) A_{c+1}^T[col][a] = lambda^n A_c^T[col][a] + sum_i (eta lambda^(n-1-i) u_i[col]) k_i[a]:
    // tile (ct, at), lane element ii is (col = 16 ct + 4 lg + ii, a = 16 at + l16)
    const float dn = powi(lam, n);
    f32x4 nxt[(NT * NT + 3) / 4];
#pragma unroll
    for (int m = 0; m < (NT * NT + 3) / 4; ++m) {
      const int t = wid + 4 * m;
      if (t < NT * NT) {
        const int ct = t / NT, at = t - ct * NT;
        f32x4 acc;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) acc[ii] = dn * At[(16 * ct + 4 * lg + ii) * LDA + 16 * at + l16];
#pragma unroll
        for (int kc = 0; kc < 2; ++kc) {
          const int i0 = 32 * kc + 8 * lg;
          acc = M::mma(ld8f(Ut + (16 * ct + l16) * LDU + i0), ld8f(Kt + (16 * at + l16) * LDU + i0), acc);
        }
        nxt[m] = acc;
      }
    }
    __syncthreads();  // every wave has read A_c (its own tiles) and the chunk's U^T, K^T
    float* An = AcT + (size_t)(c + 1) * D * D;
#pragma unroll
    for (int m = 0; m < (NT * NT + 3) / 4; ++m) {
      const int t = wid + 4 * m;
      if (t < NT * NT) {
        const int ct = t / NT, at = t - ct * NT;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int col = 16 * ct + 4 * lg + ii, ar = 16 * at + l16;
          At[col * LDA + ar] = nxt[m][ii];
          An[(size_t)col * D + ar] = nxt[m][ii];
        }
      }
    }
    __syncthreads();
  }
  if (a.A_final) {
    float* Af = a.A_final + (size_t)bh * D * D;
    for (int x = tid; x < D * D; x += 256) {
      const int ar = x / D, col = x - ar * D;
      Af[x] = At[col * LDA + ar];
    }
  }
}

// yadd_t = sigma(g) m_t for the rows of chunk c of head bh (rows t < W: zero,
// by the workgroups of chunk 0).  grid = BH * max(nch, 1), 256 threads; wave w
// takes rows 16 w .. 16 w + 15 of the chunk.
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
  const float* AcT = a.AcT + ((size_t)bh * (a.nch + 1) + c) * D * D;
  const float* Ug = a.Ut + ((size_t)bh * a.nch + c) * D * C;
  // query fragments of this lane's row (zero past the chunk's last eviction)
  f32x8 qf[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) {
    const int d0 = 32 * kc + 8 * lg;
    qf[kc] = (r < n && d0 < D) ? ld8f(qg + (size_t)r * D + d0) : M::zero();
  }
  // P[r][j] = eta lambda^(r-j) <q_r, k_j> for j <= r, as two fragments whose
  // contraction slots are (j = 32 kc + 4 lg + ii, then 32 kc + 16 + 4 lg + ii)
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
  const float dr = powi(lam, r + 1);
  float* yrow = yb + (size_t)(a.W + e0 + r) * D;
#pragma unroll
  for (int ct = 0; ct < NT; ++ct) {
    f32x4 m1 = f32x4{0.f, 0.f, 0.f, 0.f}, m2 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const int d0 = 32 * kc + 8 * lg;
      m1 = M::mma(d0 < D ? ld8f(AcT + (size_t)(16 * ct + l16) * D + d0) : M::zero(), qf[kc], m1);
    }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const float* ur = Ug + (size_t)(16 * ct + l16) * C + 32 * kc + 4 * lg;
      m2 = M::mma(ld4x2f(ur, ur + 16), pf[kc], m2);
    }
    if (r < n) {
      f32x4 o;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) o[ii] = sg * (dr * m1[ii] + m2[ii]);
      *(f32x4*)(yrow + 16 * ct + 4 * lg) = o;
    }
  }
}

namespace {
template <class E, int D>
hipError_t launch_delta_impl(const DeltaArgs& a, hipStream_t s) {
  const int BH = a.B * a.H;
  if (a.nch > 0) {
    hipLaunchKernelGGL((delta_chunk_kernel<E, D>), dim3(BH * a.nch), dim3(256), 0, s, a);
  }
  hipLaunchKernelGGL((delta_chain_kernel<E, D>), dim3(BH), dim3(256), 0, s, a);
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

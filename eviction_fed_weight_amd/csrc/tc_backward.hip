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
//   dq_kernel   : forward walk over query blocks (S, B carried in registers,
//                 eight waves): memory-path dq and scalars, then the band key
//                 tiles from the evicted chunk on (Delta fixed in the first)
//   dkdv_kernel : reverse walk over key blocks (R carried in registers in
//                 both operand layouts, eight waves): memory path of the later
//                 queries, then the band query tiles ending with the queries
//                 that evict the block
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
  static constexpr int VE = 16 / (int)sizeof(E);
  static constexpr int LDK = D + 2 * VE;  // 32 bytes of row padding: fewer LDS bank conflicts (measured)
  static constexpr int TILE = 64 * LDK * (int)sizeof(E);
};

// Waves per workgroup of the dq, dk/dv and forward segment-state kernels.
// In dq and dk/dv, waves w and w ^ 4 share one 16-row group (w & 3) and take
// one half (w >> 2) of each 64-row band tile each; the D x D states are split
// over all eight.  The pair's partial sums meet in LDS at the end of each block.
constexpr int kBwdWaves = 8;

// Compile-time variant tag for the per-tile element math.
template <int V>
struct Mode {
  static constexpr int value = V;
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

// A D x D float state split over NW waves: wave wid owns the 16-column tiles
// n = wid + NW*o of all 16-row tiles m.
template <int D, int NW>
using StateTiles = f32x4[(D / 16 + NW - 1) / NW][D / 16];

// Load a D x D float state (row a, column c at g[a*D + c]) into tiles
// t[o][m] where the lane holds element [row = 16*m + 4lg + i][col = 16*n + l16]
// with n = wid + NW*o -- the layout of an MFMA output out[m][n] -- or its
// transpose (element [row = 16*n + l16][col = 16*m + 4lg + i]).
template <int D, int NW, bool TRANS>
__device__ __forceinline__ void load_tiles(StateTiles<D, NW>& t, const float* g, int wid, int l16, int lg) {
  constexpr int NT = D / 16, NOWN = (NT + NW - 1) / NW;
#pragma unroll
  for (int o = 0; o < NOWN; ++o) {
    const int n = wid + NW * o;
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

template <int D, int NW>
__device__ __forceinline__ void store_tiles(const StateTiles<D, NW>& t, float* g, int wid, int l16, int lg) {
  constexpr int NT = D / 16, NOWN = (NT + NW - 1) / NW;
#pragma unroll
  for (int o = 0; o < NOWN; ++o) {
    const int n = wid + NW * o;
    if (n < NT) {
#pragma unroll
      for (int m = 0; m < NT; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) g[(m * 16 + lg * 4 + i) * D + n * 16 + l16] = t[o][m][i];
    }
  }
}

template <int D, int NW>
__device__ __forceinline__ void zero_tiles(StateTiles<D, NW>& t) {
#pragma unroll
  for (int o = 0; o < (D / 16 + NW - 1) / NW; ++o)
#pragma unroll
    for (int m = 0; m < D / 16; ++m) t[o][m] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// acc(o, m) <- scale*acc + sum_{c<64} A[c][16m + ..]^T (w_c B[c][16n + ..]),
// i.e. out[m-row][n-col] += sum_c A[c][row] w_c B[c][col], where A, B are 64-row
// row-major LDS tiles, all m tiles, owned n = wid + NW*o.  Optionally a second
// accumulator gets the same product with weights w2 (no extra scale).
template <class E, int D, int NW, bool TWO>
__device__ __forceinline__ void rank64_update(StateTiles<D, NW>& acc, float scale, StateTiles<D, NW>& acc2,
                                              const E* A, const E* B, const float* w, const float* w2, int wid,
                                              int l16, int lg) {
  using M = Mfma<E>;
  using frag = typename M::frag;
  constexpr int NT = D / 16, NOWN = (NT + NW - 1) / NW, LDK = BwdCfg<E, D>::LDK;
#pragma unroll
  for (int o = 0; o < NOWN; ++o) {
    const int n = wid + NW * o;
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

// Write the owned tiles of a state t[o][m] (element [row 16m + 4lg + i]
// [col 16n + l16]) to LDS transposed, dst[col][row] with leading dimension
// ld, as matrix-core operands: float32 as is, bf16 as a hi part and the
// rounding remainder lo (hi + lo carries about 16 significant bits).
template <int D, int NW>
__device__ __forceinline__ void put_state_t(const StateTiles<D, NW>& t, float* hi, float* lo, int ld, int wid,
                                            int l16, int lg) {
  constexpr int NT = D / 16, NOWN = (NT + NW - 1) / NW;
  (void)lo;
#pragma unroll
  for (int o = 0; o < NOWN; ++o) {
    const int n = wid + NW * o;
    if (n < NT) {
#pragma unroll
      for (int m = 0; m < NT; ++m) *(f32x4*)(hi + (16 * n + l16) * ld + 16 * m + 4 * lg) = t[o][m];
    }
  }
}
template <int D, int NW>
__device__ __forceinline__ void put_state_t(const StateTiles<D, NW>& t, bf16* hi, bf16* lo, int ld, int wid,
                                            int l16, int lg) {
  constexpr int NT = D / 16, NOWN = (NT + NW - 1) / NW;
#pragma unroll
  for (int o = 0; o < NOWN; ++o) {
    const int n = wid + NW * o;
    if (n < NT) {
#pragma unroll
      for (int m = 0; m < NT; ++m) {
        bf16x4 h, l;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          h[i] = (bf16)t[o][m][i];
          l[i] = (bf16)(t[o][m][i] - (float)h[i]);
        }
        *(bf16x4*)(hi + (16 * n + l16) * ld + 16 * m + 4 * lg) = h;
        *(bf16x4*)(lo + (16 * n + l16) * ld + 16 * m + 4 * lg) = l;
      }
    }
  }
}

// ===========================================================================
// Segment states for the backward.
// Forward: S and B = dS/dlambda over each segment's evictions (from zero);
// grid = BH * (nseg-1); writes fstate/tstate[bh][m+1].
template <class E, int D>
__global__ void __launch_bounds__(64 * kBwdWaves, 1) bseg_fwd_kernel(BwdArgs a) {
  using C = BwdCfg<E, D>;
  constexpr int NW = kBwdWaves, NTH = 64 * NW, NOWN = (C::NT + NW - 1) / NW;
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
  StateTiles<D, NW> S, B;
  zero_tiles<D, NW>(S);
  zero_tiles<D, NW>(B);
  TileRegs<E, D, 64, NTH> kl, vl;
  int g = 0;
  while (g < a.G && (m * a.G + g) * 64 - a.W + 63 < 0) ++g;  // blocks wholly before the first token
  kl.load(Kg, (m * a.G + g) * 64 - a.W);
  vl.load(Vg, (m * a.G + g) * 64 - a.W);
  for (; g < a.G; ++g) {
    const int e0 = (m * a.G + g) * 64 - a.W;
    __syncthreads();
    kl.store(Ks, C::LDK);
    vl.store(Vs, C::LDK);
    if (tid < 64) {
      const bool ok = e0 + tid >= 0;
      w1[tid] = ok ? pw[63 - tid] : 0.0f;
      w2[tid] = ok ? dpw[63 - tid] : 0.0f;
    }
    __syncthreads();
    if (g + 1 < a.G) {  // the next block's chunk, in flight during the update
      kl.load(Kg, e0 + 64);
      vl.load(Vg, e0 + 64);
    }
    // B <- lam^64 B + 64 lam^63 S + sum w2 k v^T ; S <- lam^64 S + sum w1 k v^T
#pragma unroll
    for (int o = 0; o < NOWN; ++o)
#pragma unroll
      for (int mm = 0; mm < C::NT; ++mm) B[o][mm] = pw[64] * B[o][mm] + dpw[64] * S[o][mm];
    rank64_update<E, D, NW, true>(S, pw[64], B, Ks, Vs, w1, w2, wid, l16, lg);
  }
  store_tiles<D, NW>(S, a.fstate + ((size_t)bh * a.nseg + m + 1) * D * D, wid, l16, lg);
  store_tiles<D, NW>(B, a.tstate + ((size_t)bh * a.nseg + m + 1) * D * D, wid, l16, lg);
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
  // (eight segments' local states loaded ahead of the dependent chain)
  for (int m0 = 1; m0 < a.nseg; m0 += 8) {
    float4 ls[8], lb[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (m0 + u < a.nseg) {
        ls[u] = ps[(m0 + u) * stride];
        lb[u] = pb[(m0 + u) * stride];
      }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (m0 + u < a.nseg) {
        b.x = Ld * s.x + L * b.x + lb[u].x;
        b.y = Ld * s.y + L * b.y + lb[u].y;
        b.z = Ld * s.z + L * b.z + lb[u].z;
        b.w = Ld * s.w + L * b.w + lb[u].w;
        s.x = L * s.x + ls[u].x;
        s.y = L * s.y + ls[u].y;
        s.z = L * s.z + ls[u].z;
        s.w = L * s.w + ls[u].w;
        ps[(m0 + u) * stride] = s;
        pb[(m0 + u) * stride] = b;
      }
  }
}

// Reverse: local adjoint of segment m (m >= 1) over the query rows whose
// eviction index lies in its key range, relative to its first key:
// Lr_m = sum_{jk in seg, descending} lambda^(64 (jk - jb)) U(jk),
// U(jk) = sum_{c<64} lambda^c q_{64jk+W+c}^T dy_{64jk+W+c};  writes rstate[bh][m-1].
template <class E, int D>
__global__ void __launch_bounds__(64 * kBwdWaves, 1) bseg_rev_kernel(BwdArgs a) {
  using C = BwdCfg<E, D>;
  constexpr int NW = kBwdWaves, NTH = 64 * NW;
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
  StateTiles<D, NW> R;
  zero_tiles<D, NW>(R);
  const int jb = m * a.G, je = min(a.nblk, jb + a.G);
  TileRegs<E, D, 64, NTH> ql, yl;
  int jk = je - 1;
  while (jk >= jb && jk * 64 + a.W >= a.T) --jk;  // blocks whose queries lie past the end
  ql.load(Qg, jk * 64 + a.W);
  yl.load(Yg, jk * 64 + a.W);
  for (; jk >= jb; --jk) {
    const int q0 = jk * 64 + a.W;
    __syncthreads();
    ql.store(Qs, C::LDK);
    yl.store(Ys, C::LDK);
    __syncthreads();
    if (jk > jb) {  // the next block's queries, in flight during the update
      ql.load(Qg, q0 - 64);
      yl.load(Yg, q0 - 64);
    }
    // R[a][c] <- lam^64 R + sum_c' Q[c'][a] lam^c' dY[c'][c]  (skipped blocks
    // contribute zero and need no decay: R is zero until the first block)
    rank64_update<E, D, NW, false>(R, pw[64], R, Qs, Ys, pw, pw, wid, l16, lg);
  }
  // blocks skipped at the top (q0 >= T) would only scale a zero state;
  // blocks present below them were decayed correctly relative to jb.
  store_tiles<D, NW>(R, a.rstate + ((size_t)bh * a.nseg + m - 1) * D * D, wid, l16, lg);
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
  // (eight segments' local adjoints loaded ahead of the dependent chain)
  for (int m0 = a.nseg - 2; m0 >= 0; m0 -= 8) {
    float4 l[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (m0 - u >= 0) l[u] = p[(m0 - u) * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (m0 - u >= 0) {
        r.x = L * r.x + l[u].x;
        r.y = L * r.y + l[u].y;
        r.z = L * r.z + l[u].z;
        r.w = L * r.w + l[u].w;
        p[(m0 - u) * stride] = r;
      }
  }
}

// ===========================================================================
// Band tiles of a 64-row block start at its evicted chunk.  For query block
// t0 the key tiles start at e0 + 64 m (e0 = t0 - W, m = 0 .. ceil(W/64)):
// tile 0 is the chunk that the block's rows evict, the last one holds the
// diagonal.  For key block i0 the query tiles start at i0 + W - 64 m: tile 0,
// taken last, holds the queries that evict the block.  The intra-chunk part
// of the memory path then reuses the scores of one band tile, and the band
// needs no tile of its own for it.  Streamed tiles go through two LDS buffers
// (one barrier per tile) when six 64-row tiles fit, else through one.
template <class E, int D>
struct BandBufs {
  static constexpr int N = 6 * BwdCfg<E, D>::TILE <= 150 * 1024 ? 2 : 1;
};

// dq kernel: grid = BH * nseg, one 64-row query block at a time.  Per block:
// the state part of the memory path (S(e0) dy, B(e0) dy), then the key tiles
// from the evicted chunk on (tile 0 adds the intra-chunk memory terms and
// fixes Delta before its band terms), then S and B carried past the chunk.
template <class E, int D>
__global__ void __launch_bounds__(64 * kBwdWaves, 1) dq_kernel(BwdArgs a) {
  using M = Mfma<E>;
  using frag = typename M::frag;
  using C = BwdCfg<E, D>;
  constexpr int NW = kBwdWaves, NTH = 64 * NW;
  constexpr int NT = C::NT, NKC = C::NKC, NOWN = (NT + NW - 1) / NW, LDK = C::LDK, VE = C::VE;
  constexpr int NB = BandBufs<E, D>::N;
  constexpr int NVR = D / VE / 2;  // 16-byte vectors in half a row
  constexpr int NYV = (NVR + 3) / 4;
  static_assert((M::kSplit ? 2 : 1) * D * LDK * (int)sizeof(E) <= 2 * NB * C::TILE,
                "a state copy must fit in the key buffers");
  static_assert(2 * NB * C::TILE >= ((NT + 1) / 2) * NW * 64 * 16, "the dq exchange must fit in the key buffers");
  __shared__ __attribute__((aligned(16))) char smem[(2 + 2 * NB) * C::TILE];
  __shared__ float pw[72], dpw[72], red[NW][2], w1[64], w2[64], dex[2][64];
  E* Qs = (E*)smem;
  E* Ys = (E*)(smem + C::TILE);
  // key buffer b: K at (2 + 2b) tiles, V after it.  Before the band they
  // hold S, then B, as matrix-core operands (SBh: [a][c], hi then lo); after
  // it XQ, the pair's dq exchange.
  auto Kb = [&](int b) { return (E*)(smem + (2 + 2 * b) * C::TILE); };
  auto Vb = [&](int b) { return (E*)(smem + (3 + 2 * b) * C::TILE); };
  E* SBh = (E*)(smem + 2 * C::TILE);
  f32x4* XQ = (f32x4*)(smem + 2 * C::TILE);

  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int half = wid >> 2;
  const int wgi = xcd_remap(blockIdx.x, gridDim.x);  // one head's segments on one XCD
  const int bh = wgi / a.nseg, seg = wgi - bh * a.nseg;
  const int h = bh % a.H;
  const int T = a.T, W = min(a.W, a.T);  // a window of T or more evicts nothing
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

  // S^T and B^T: tiles [o][ct] hold element [c = 16 ct + 4lg + i][a = 16 (wid+NW*o) + l16]
  StateTiles<D, NW> S, B;
  if (seg == 0) {
    zero_tiles<D, NW>(S);
    zero_tiles<D, NW>(B);
  } else {
    load_tiles<D, NW, true>(S, a.fstate + ((size_t)bh * a.nseg + seg) * D * D, wid, l16, lg);
    load_tiles<D, NW, true>(B, a.tstate + ((size_t)bh * a.nseg + seg) * D * D, wid, l16, lg);
  }
  vm_fence_loads();
  const int jb = seg * a.G, je = min(a.nblk, jb + a.G);
  const int r = (wid & 3) * 16 + l16;  // this lane's query row in the block
  const int mt = (W + 63) >> 6;        // key tiles e0 + 64 m, m = mlo .. mt
  // first tile with a key >= 0
  auto mlo_of = [](int e0) { return e0 + 63 >= 0 ? 0 : (-e0) >> 6; };
  float md_acc = 0.0f, dl_acc = 0.0f;
  TileRegs<E, D, 64, NTH> ql, yl, kl, vl;
  uint4 yv[NYV];  // this lane's part of this wave's half of row t0 + r of y
  float lse_r = 0.0f;
  auto load_rows = [&](int j) {  // Q, dY, y rows and lse of query block j
    const int t = j * 64 + r;
    ql.load(Qg, j * 64);
    yl.load(dYg, j * 64);
#pragma unroll
    for (int i = 0; i < NYV; ++i) {
      const int vv = lg + 4 * i;
      yv[i] = buf_load16(Yg, vv < NVR ? (t * D + (half * NVR + vv) * VE) * (int)sizeof(E) : -16);
    }
    lse_r = a.lse[(size_t)bh * T + min(t, T - 1)];
  };
  auto load_keys = [&](int k0) {
    kl.load(Kg, k0);
    vl.load(Vg, k0);
  };
  auto put_keys = [&](int b) {
    kl.store(Kb(b), LDK);
    vl.store(Vb(b), LDK);
  };
  load_rows(jb);
  load_keys(jb * 64 - W + 64 * mlo_of(jb * 64 - W));
  for (int j = jb; j < je; ++j) {
    const int t0 = j * 64, trow = t0 + r, e0 = t0 - W;
    const int mlo = mlo_of(e0);
    __syncthreads();
    ql.store(Qs, LDK);
    yl.store(Ys, LDK);
    if (tid < 64) {
      const bool ok = e0 + tid >= 0;
      w1[tid] = ok ? pw[63 - tid] : 0.0f;
      w2[tid] = ok ? dpw[63 - tid] : 0.0f;
    }
    __syncthreads();
    // <dy, y> of row trow over this wave's half of the columns
    float yd = 0.0f;
#pragma unroll
    for (int i = 0; i < NYV; ++i) {
      const int vv = lg + 4 * i;
      if (vv < NVR) {
        const E* ye = (const E*)&yv[i];
        const E* dy = Ys + r * LDK + (half * NVR + vv) * VE;
#pragma unroll
        for (int x = 0; x < VE; ++x) yd += (float)ye[x] * (float)dy[x];
      }
    }
    yd = xsum4(yd);
    const float lse2 = (trow < T) ? lse_r * kLog2e : __builtin_huge_valf();

    f32x4 dQ[NT];
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) dQ[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // this wave's shares of <dy, mt> and <dy, d mt/dlam> for row r (all 4 lanes)
    float md = 0.0f, dlr = 0.0f;

    if (mlo == 0 && e0 > 0) {
      // S(e0) dy and B(e0) dy for this lane's row over the column tiles dt
      // with dt % 2 == half, each state copied to LDS in turn: dq gains
      // sigma eta lambda^(r+1) S dy; <q, S dy> and <q, B dy> feed md and dlr.
      const float f = pw[r + 1], df = dpw[r + 1];
      float qx = 0.0f, qy = 0.0f;
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        put_state_t<D, NW>(pass == 0 ? S : B, SBh, SBh + D * LDK, LDK, wid, l16, lg);
        __syncthreads();
#pragma unroll
        for (int dt = 0; dt < NT; ++dt) {
          if ((dt & 1) == half) {
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int dc = 0; dc < NKC; ++dc) {
              const bool in = dc * 32 + lg * 8 < D;
              const frag yf = in ? M::lds8(Ys + r * LDK + dc * 32 + lg * 8) : M::zero();
              const E* sr = SBh + (dt * 16 + l16) * LDK + dc * 32 + lg * 8;
              acc = M::mma(in ? M::lds8(sr) : M::zero(), yf, acc);
              if (M::kSplit) acc = M::mma(in ? M::lds8(sr + D * LDK) : M::zero(), yf, acc);
            }
            const E* qrow = Qs + r * LDK + dt * 16 + lg * 4;
            float qd = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) qd += (float)qrow[i] * acc[i];
            if (pass == 0) {
              dQ[dt] += (seta * f) * acc;
              qx += qd;
            } else {
              qy += qd;
            }
          }
        }
        __syncthreads();  // the copy is read before the next one (or the first key tile) lands on it
      }
      qx = xsum4(qx);
      qy = xsum4(qy);
      md += f * qx;
      dlr += df * qx + f * qy;
    }
    put_keys(0);
    __syncthreads();
    // Tile order: the first tile (the evicted chunk when there is one) first,
    // then every other block walks the rest backwards, so that a block starts
    // on the key tiles its predecessor used last (still in L2).
    const int ntl = mt - mlo + 1;
    const bool rev = ((j - jb) & 1) != 0;
    auto m_at = [&](int i) { return (!rev || i == 0) ? mlo + i : mt + 1 - i; };
    // the tile at position i, or after the last one the next query block's rows and first key tile
    auto next_loads = [&](int i) {
      if (i < ntl) {
        load_keys(e0 + 64 * m_at(i));
      } else if (j + 1 < je) {
        load_rows(j + 1);
        load_keys(e0 + 64 + 64 * mlo_of(e0 + 64));
      }
    };
    next_loads(1);
    float delta = 0.0f;
    int buf = 0;
    for (int i = 0; i < ntl; ++i) {
      const int m = m_at(i);
      const int k0 = e0 + 64 * m;
      const E* Ks = Kb(buf);
      const E* Vs = Vb(buf);
      // Z = K q, P = V dy for this wave's 32 keys (rows) and this lane's query (column)
      // (the query row's fragments are re-read from LDS each tile: fewer live registers)
      f32x4 Z[2], P[2];
#pragma unroll
      for (int n2 = 0; n2 < 2; ++n2) {
        Z[n2] = f32x4{0.f, 0.f, 0.f, 0.f};
        P[n2] = Z[n2];
      }
      // (the matrix-product blocks run at raised wave priority: the waves
      // sharing a SIMD then spend less time in the same phase; measured)
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int dc = 0; dc < NKC; ++dc) {
        const bool in = dc * 32 + lg * 8 < D;
        const frag qf = in ? M::lds8(Qs + r * LDK + dc * 32 + lg * 8) : M::zero();
        const frag yf = in ? M::lds8(Ys + r * LDK + dc * 32 + lg * 8) : M::zero();
#pragma unroll
        for (int n2 = 0; n2 < 2; ++n2) {
          const int n = 2 * half + n2;
          const int kr = 32 * (n >> 1) + (l16 >> 2) * 8 + (n & 1) * 4 + (l16 & 3);
          const frag ka = in ? M::lds8(Ks + kr * LDK + dc * 32 + lg * 8) : M::zero();
          const frag va = in ? M::lds8(Vs + kr * LDK + dc * 32 + lg * 8) : M::zero();
          Z[n2] = M::mma(ka, qf, Z[n2]);
          P[n2] = M::mma(va, yf, P[n2]);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      if (m == 0) {
        // the evicted chunk: intra-chunk memory terms of <dy, mt> and its lambda derivative
        float mp = 0.0f, dp = 0.0f;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int c = 32 * half + lg * 8 + jj;
          const float zp = Z[jj >> 2][jj & 3] * P[jj >> 2][jj & 3];
          const float mem = ((c <= r) & (e0 + c >= 0)) ? zp : 0.0f;
          const int di = max(r - c, 0);
          mp = __builtin_fmaf(pw[di], mem, mp);
          dp = __builtin_fmaf(dpw[di], mem, dp);
        }
        md += xsum4(mp);
        dlr += xsum4(dp);
      }
      if (i == 0) {
        // Delta = <dy, y> - sigma eta <dy, mt>, the two halves' shares summed
        if (lg == 0) dex[half][r] = yd - seta * md;
        __syncthreads();
        delta = dex[0][r] + dex[1][r];
        if (half == 0 && lg == 0 && trow < T) a.delta[(size_t)bh * T + trow] = delta;
      }
      // dS for this lane's query and the wave's 32 keys, then dQ += dS K.
      // Variants: 0 = tile inside the band, 1 = band edge, 2 = band edge plus
      // the intra-chunk memory weights (the evicted chunk).  Masks enter as an
      // added -inf or a 0/1 factor, so that no operand load sits under a branch.
      auto tile_update = [&](auto mode_c) {
        constexpr int mode = decltype(mode_c)::value;
        float gv[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int c = 32 * half + lg * 8 + jj;
          const int key = k0 + c;
          const float z = Z[jj >> 2][jj & 3];
          const float dpv = P[jj >> 2][jj & 3];
          float x = __builtin_fmaf(z, sl2, -lse2);
          if (mode != 0) {
            const bool in = ((unsigned)(trow - key) < (unsigned)W) & (key >= 0);
            x += in ? 0.0f : -__builtin_huge_valf();
          }
          float g = tau * fast_exp2(x) * (dpv - delta);
          if (mode == 2) {
            const float w = seta * pw[max(r - c, 0)] * (((c <= r) & (key >= 0)) ? 1.0f : 0.0f);
            g = __builtin_fmaf(w, dpv, g);
          }
          gv[jj] = g;
        }
        const frag gf = M::pack(gv);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int dt = 0; dt < NT; ++dt)
          dQ[dt] = M::mma(ColFrag<E>::read(Ks + (half * 32 + lg * 8) * LDK + dt * 16, LDK, l16), gf, dQ[dt]);
        __builtin_amdgcn_s_setprio(0);
      };
      if (m == 0)
        tile_update(Mode<2>{});
      else if ((k0 >= 0) && (k0 + 63 <= t0) && (k0 >= t0 + 64 - W))
        tile_update(Mode<0>{});
      else
        tile_update(Mode<1>{});
      if (m == 0 && j + 1 < je) {
        // carry S and B past the evicted chunk
#pragma unroll
        for (int o = 0; o < NOWN; ++o)
#pragma unroll
          for (int mm = 0; mm < NT; ++mm) B[o][mm] = pw[64] * B[o][mm] + dpw[64] * S[o][mm];
        // S^T[c][a] += sum_c' V[c'][c] w K[c'][a]
        rank64_update<E, D, NW, true>(S, pw[64], B, Vs, Ks, w1, w2, wid, l16, lg);
      }
      if (i + 1 < ntl) {
        const int nb = NB == 2 ? buf ^ 1 : 0;
        if (NB == 1) __syncthreads();
        put_keys(nb);
        __syncthreads();
        buf = nb;
        next_loads(i + 2);
      }
    }
    // the pair's dq shares: half h keeps the tiles dt with dt % 2 == h
    __syncthreads();
#pragma unroll
    for (int dt = 0; dt < NT; ++dt)
      if ((dt & 1) != half) XQ[((dt >> 1) * NW + wid) * 64 + lane] = dQ[dt];
    __syncthreads();
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) {
      if ((dt & 1) == half) {
        const f32x4 o = dQ[dt] + XQ[((dt >> 1) * NW + (wid ^ 4)) * 64 + lane];
        if (trow < T) st4(dQg + (size_t)trow * D + dt * 16 + lg * 4, o);
      }
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
    for (int w = 0; w < NW; ++w) {
      s0 += red[w][0];
      s1 += red[w][1];
    }
    a.part[((size_t)bh * a.nseg + seg) * 2 + 0] = s0;
    a.part[((size_t)bh * a.nseg + seg) * 2 + 1] = s1;
  }
}

// ===========================================================================
// dk/dv kernel: grid = BH * nseg, reverse walk over 64-row key blocks.  Per
// key block: the memory path of the later queries (R(i0+64) v, R(i0+64)^T k),
// the query tiles of the band (the last one, the queries that evict the
// block, also carries the intra-chunk memory weights), then R(i0) from that
// last tile.
template <class E, int D>
__global__ void __launch_bounds__(64 * kBwdWaves, 1) dkdv_kernel(BwdArgs a) {
  using M = Mfma<E>;
  using frag = typename M::frag;
  using C = BwdCfg<E, D>;
  constexpr int NW = kBwdWaves, NTH = 64 * NW;
  constexpr int NT = C::NT, NKC = C::NKC, NOWN = (NT + NW - 1) / NW, LDK = C::LDK;
  constexpr int NB = BandBufs<E, D>::N;
  static_assert((M::kSplit ? 2 : 1) * D * LDK * (int)sizeof(E) <= 2 * NB * C::TILE,
                "the state copy must fit in the query buffers");
  static_assert(2 * NB * C::TILE >= NT * NW * 64 * 16, "the dk/dv exchange must fit in the query buffers");
  __shared__ __attribute__((aligned(16))) char smem[(2 + 2 * NB) * C::TILE];
  __shared__ float pw[72], dpw[72], lse_s[NB][64], del_s[NB][64];
  E* Ks = (E*)smem;
  E* Vs = (E*)(smem + C::TILE);
  // query buffer b: Q at (2 + 2b) tiles, dY after it.  Before the band
  // they hold R^T as matrix-core operands (RTh, RTl: [c][a]); after it XK,
  // the pair's dk/dv exchange.
  auto Qb = [&](int b) { return (E*)(smem + (2 + 2 * b) * C::TILE); };
  auto Yb = [&](int b) { return (E*)(smem + (3 + 2 * b) * C::TILE); };
  E* RTh = (E*)(smem + 2 * C::TILE);
  E* RTl = RTh + D * LDK;
  f32x4* XK = (f32x4*)(smem + 2 * C::TILE);

  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int half = wid >> 2;
  const int wgi = xcd_remap(blockIdx.x, gridDim.x);  // one head's segments on one XCD
  const int bh = wgi / a.nseg, seg = wgi - bh * a.nseg;
  const int h = bh % a.H;
  const int T = a.T, W = min(a.W, a.T);  // a window of T or more evicts nothing
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

  // R tiles [o][at]: element R[a = 16 at + 4lg + i][c = 16 (wid+NW*o) + l16]
  StateTiles<D, NW> RA;
  if (seg == a.nseg - 1)
    zero_tiles<D, NW>(RA);
  else
    load_tiles<D, NW, false>(RA, a.rstate + ((size_t)bh * a.nseg + seg) * D * D, wid, l16, lg);
  vm_fence_loads();
  const int jb = seg * a.G, je = min(a.nblk, jb + a.G);
  const int kidx = (wid & 3) * 16 + l16;  // this lane's key in the block
  const int mt = (W + 63) >> 6;           // query tiles i0 + W - 64 m, m = mt .. mlo
  // last tile index that starts before T
  auto mlo_of = [&](int i0) { return i0 + W < T ? 0 : ((i0 + W - T) >> 6) + 1; };
  TileRegs<E, D, 64, NTH> kl, vl, ql, yl;
  float lse_r = 0.0f, del_r = 0.0f;
  auto load_qtile = [&](int q0) {
    ql.load(Qg, q0);
    yl.load(dYg, q0);
    if (tid < 64) {
      const int t = q0 + tid;
      const bool ok = t >= 0 && t < T;
      const size_t ix = (size_t)bh * T + (ok ? t : 0);
      lse_r = a.lse[ix];
      del_r = a.delta[ix];
      if (!ok) {
        lse_r = __builtin_huge_valf();
        del_r = 0.0f;
      }
    }
  };
  auto put_qtile = [&](int b) {
    ql.store(Qb(b), LDK);
    yl.store(Yb(b), LDK);
    if (tid < 64) {
      lse_s[b][tid] = lse_r * kLog2e;
      del_s[b][tid] = del_r;
    }
  };
  kl.load(Kg, (je - 1) * 64);
  vl.load(Vg, (je - 1) * 64);
  load_qtile((je - 1) * 64 + W - 64 * mt);
  for (int jk = je - 1; jk >= jb; --jk) {
    const int i0 = jk * 64, key = i0 + kidx, q0m = i0 + W;
    const int mlo = mlo_of(i0);
    const bool later = i0 + 64 + W < T;  // queries evict keys past this block
    __syncthreads();
    kl.store(Ks, LDK);
    vl.store(Vs, LDK);
    if (later) put_state_t<D, NW>(RA, RTh, RTl, LDK, wid, l16, lg);
    __syncthreads();
    // this wave's shares of dK, dV for its 16 keys
    f32x4 dK[NT], dV[NT];
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) {
      dK[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
      dV[dt] = dK[dt];
    }
    // ---- memory path of the later queries: dk += f R(i0+64) v,
    // dv += f R(i0+64)^T k (the pair splits the column tiles dt by parity) ----
    if (later) {
      const float f = seta * pw[64 - kidx];
      frag kf[NKC], vf[NKC];
#pragma unroll
      for (int dc = 0; dc < NKC; ++dc) {
        const bool in = dc * 32 + lg * 8 < D;
        kf[dc] = in ? M::lds8(Ks + kidx * LDK + dc * 32 + lg * 8) : M::zero();
        vf[dc] = in ? M::lds8(Vs + kidx * LDK + dc * 32 + lg * 8) : M::zero();
      }
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) {
        if ((dt & 1) == half) {
          f32x4 ak = f32x4{0.f, 0.f, 0.f, 0.f}, av = ak;
#pragma unroll
          for (int dc = 0; dc < NKC; ++dc) {
            const bool in = dc * 32 + lg * 8 < D;
            // (R v)[a][key]: A = R rows a (columns of R^T), B = v.  The
            // transposing read runs on every lane; for D = 16 the lanes past
            // the contraction read written (finite) rows and meet v = 0.
            const E* rc = RTh + ((dc * 32 + lg * 8) & (D >= 32 ? ~0 : 15)) * LDK + dt * 16;
            ak = M::mma(ColFrag<E>::read(rc, LDK, l16), vf[dc], ak);
            if (M::kSplit) ak = M::mma(ColFrag<E>::read(rc + D * LDK, LDK, l16), vf[dc], ak);
            // (R^T k)[c][key]: A = R^T rows c, B = k
            const E* rr = RTh + (dt * 16 + l16) * LDK + dc * 32 + lg * 8;
            av = M::mma(in ? M::lds8(rr) : M::zero(), kf[dc], av);
            if (M::kSplit) av = M::mma(in ? M::lds8(rr + D * LDK) : M::zero(), kf[dc], av);
          }
          dK[dt] += f * ak;
          dV[dt] += f * av;
        }
      }
      __syncthreads();  // R^T read before the first query tile lands on it
    }
    // ---- band query tiles; the last one (m = 0) also carries the memory
    // weights of the queries that evict this block ----
    put_qtile(0);
    __syncthreads();
    // the next tile, or after the last one the next key block and its first tile
    auto next_loads = [&](int mn) {
      if (mn >= mlo) {
        load_qtile(q0m - 64 * mn);
      } else if (jk > jb) {
        kl.load(Kg, i0 - 64);
        vl.load(Vg, i0 - 64);
        load_qtile(i0 - 64 + W - 64 * mt);
      }
    };
    next_loads(mt - 1);
    int buf = 0;
    for (int m = mt; m >= mlo; --m) {
      const int q0 = q0m - 64 * m;
      const E* Qs = Qb(buf);
      const E* Ys = Yb(buf);
      const float* ls = lse_s[buf];
      const float* ds = del_s[buf];
      // Z = Q k, P = dY v for this wave's 32 queries (rows) and this lane's key (column)
      // (the key's fragments are re-read from LDS each tile: fewer live registers)
      f32x4 Z[2], P[2];
#pragma unroll
      for (int g2 = 0; g2 < 2; ++g2) {
        Z[g2] = f32x4{0.f, 0.f, 0.f, 0.f};
        P[g2] = Z[g2];
      }
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int dc = 0; dc < NKC; ++dc) {
        const bool in = dc * 32 + lg * 8 < D;
        const frag kf = in ? M::lds8(Ks + kidx * LDK + dc * 32 + lg * 8) : M::zero();
        const frag vf = in ? M::lds8(Vs + kidx * LDK + dc * 32 + lg * 8) : M::zero();
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
          const int g = 2 * half + g2;
          const frag qa = in ? M::lds8(Qs + (g * 16 + l16) * LDK + dc * 32 + lg * 8) : M::zero();
          const frag ya = in ? M::lds8(Ys + (g * 16 + l16) * LDK + dc * 32 + lg * 8) : M::zero();
          Z[g2] = M::mma(qa, kf, Z[g2]);
          P[g2] = M::mma(ya, vf, P[g2]);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      // P and dS^T for the wave's 32 queries, then dV += P^T dY, dK += dS^T Q.
      // Variants: 0 = tile inside the band, 1 = band edge, 2 = band edge plus
      // the memory weights of the evicting queries.  Masks enter as an added
      // -inf or a 0/1 factor, so that no operand load sits under a branch.
      auto tile_update = [&](auto mode_c) {
        constexpr int mode = decltype(mode_c)::value;
        float pv[8], gv[8];
        f32x4 lsv[2], dsv[2];
#pragma unroll
        for (int g2 = 0; g2 < 2; ++g2) {
          lsv[g2] = *(const f32x4*)(ls + (2 * half + g2) * 16 + lg * 4);
          dsv[g2] = *(const f32x4*)(ds + (2 * half + g2) * 16 + lg * 4);
        }
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int rr = 32 * half + (jj >> 2) * 16 + lg * 4 + (jj & 3);
          const int t = q0 + rr;
          const float z = Z[jj >> 2][jj & 3], dp = P[jj >> 2][jj & 3];
          float x = __builtin_fmaf(z, sl2, -lsv[jj >> 2][jj & 3]);
          if (mode != 0) {
            const bool in = ((unsigned)(t - key) < (unsigned)W) & (t < T);
            x += in ? 0.0f : -__builtin_huge_valf();
          }
          const float pr = fast_exp2(x);
          float pvv = pr, gvv = tau * pr * (dp - dsv[jj >> 2][jj & 3]);
          if (mode == 2) {
            // query t evicts key i0 + rr: weight sigma eta lambda^(rr - kidx) on keys up to it
            const int di = rr - kidx;
            const float w = seta * pw[max(di, 0)] * (((di >= 0) & (t < T)) ? 1.0f : 0.0f);
            pvv = __builtin_fmaf(w, z, pvv);
            gvv = __builtin_fmaf(w, dp, gvv);
          }
          pv[jj] = pvv;
          gv[jj] = gvv;
        }
        const frag pf = M::pack(pv), gf = M::pack(gv);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int dt = 0; dt < NT; ++dt) {
          dV[dt] = M::mma(ColFrag2<E>::read(Ys + (32 * half + lg * 4) * LDK + dt * 16,
                                            Ys + (32 * half + 16 + lg * 4) * LDK + dt * 16, LDK, l16),
                          pf, dV[dt]);
          dK[dt] = M::mma(ColFrag2<E>::read(Qs + (32 * half + lg * 4) * LDK + dt * 16,
                                            Qs + (32 * half + 16 + lg * 4) * LDK + dt * 16, LDK, l16),
                          gf, dK[dt]);
        }
        __builtin_amdgcn_s_setprio(0);
      };
      if (m == 0)
        tile_update(Mode<2>{});
      else if ((i0 + 63 <= q0) && (i0 >= q0 + 64 - W) && (q0 + 63 < T))
        tile_update(Mode<0>{});
      else
        tile_update(Mode<1>{});
      if (m > mlo) {
        const int nb = NB == 2 ? buf ^ 1 : 0;
        if (NB == 1) __syncthreads();
        put_qtile(nb);
        __syncthreads();
        buf = nb;
        next_loads(m - 2);
      }
    }
    // R(i0) = lam^64 R(i0+64) + sum_c lam^c q_{q0m+c}^T dy_{q0m+c}
    if (mlo == 0 && jk > jb) rank64_update<E, D, NW, false>(RA, pw[64], RA, Qb(buf), Yb(buf), pw, pw, wid, l16, lg);
    // the pair's shares: half 0 completes dK, half 1 dV
    __syncthreads();
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) XK[(dt * NW + wid) * 64 + lane] = half == 0 ? dV[dt] : dK[dt];
    __syncthreads();
    if (key < T) {
      E* dst = half == 0 ? dKg : dVg;
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) {
        const f32x4 o = (half == 0 ? dK[dt] : dV[dt]) + XK[(dt * NW + (wid ^ 4)) * 64 + lane];
        st4(dst + (size_t)key * D + dt * 16 + lg * 4, o);
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
    hipLaunchKernelGGL((bseg_fwd_kernel<E, D>), dim3(BH * (a.nseg - 1)), dim3(64 * kBwdWaves), 0, s, a);
    hipLaunchKernelGGL((bchain_fwd_kernel<D>), dim3((D * D / 4 + 255) / 256, BH), dim3(256), 0, s, a);
    hipLaunchKernelGGL((bseg_rev_kernel<E, D>), dim3(BH * (a.nseg - 1)), dim3(64 * kBwdWaves), 0, s, a);
    hipLaunchKernelGGL((bchain_rev_kernel<D>), dim3((D * D / 4 + 255) / 256, BH), dim3(256), 0, s, a);
  }
  hipLaunchKernelGGL((dq_kernel<E, D>), dim3(BH * a.nseg), dim3(64 * kBwdWaves), 0, s, a);
  hipLaunchKernelGGL((dkdv_kernel<E, D>), dim3(BH * a.nseg), dim3(64 * kBwdWaves), 0, s, a);
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

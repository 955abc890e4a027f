// TC forward on gfx950: window attention (L1) fused with the eviction-state
// read (L2) and the gate, plus the W-shifted weighted-sum scan of the state.
//
// Method ("Tensor Cache: Eviction-conditioned Associative Memory for
// Transformers"): Section 3.1 Eq. (1) window softmax; Section 3.2 and
// Figure 2 write-on-evict A <- lambda A + eta k v^T, read m = q A, fuse
// y = y_local + sigmoid(g) m; abstract: parallel weighted-sum scan.
//
// Scan used here.  Token i is evicted at step i + W.  Let S(e) be the state
// after the first e evictions with eta factored out,
//   S(e) = sum_{i<e} lambda^(e-1-i) k_i v_i^T,     A_t = eta * S(t-W+1).
// Query block j covers rows t0 = 64j .. t0+63 and its evicted chunk is
// e0 = t0 - W .. e0+63.  For row t = t0 + r (r < 64)
//   A_t = eta [ lambda^(r+1) S(e0) + sum_{c<=r} lambda^(r-c) k_{e0+c} v_{e0+c}^T ]
// so the read is one D x D product with S(e0) plus a lower-triangular,
// decay-weighted 64 x 64 tile against the chunk (read identity of the
// abstract: q (k outer v) = <q,k> v), and the carry is
//   S(e0 + 64) = lambda^64 S(e0) + sum_c lambda^(63-c) k_{e0+c} v_{e0+c}^T.
// A workgroup walks a segment of G consecutive blocks carrying S in float32
// MFMA accumulators; the segment-start states come from a per-segment pass
// (seg_state_kernel) and a short chain over segments (seg_chain_kernel).
#include "tc_device.h"
#include "tc_launch.h"

namespace tck {

// LDS plan of the fused forward kernel (elements / bytes).  K and V tiles
// are stored row-major; operands that contract down their rows are read with
// transpose reads (ColFrag).  X (float rows x D) aliases the K/V tiles: it is
// only live between the band loop and the store of the evicted chunk.
template <class E, int D>
struct FwdLds {
  static constexpr int VE = 16 / sizeof(E);
  static constexpr int LDK = D + VE;  // row stride of K, V, Q tiles
  static constexpr int LDX = D + 4;
  static constexpr int TILE = 64 * LDK * (int)sizeof(E);
  static constexpr int XB = 64 * LDX * 4;
  static constexpr int U = (2 * TILE) > XB ? (2 * TILE) : XB;
  static constexpr int TOTAL = U + TILE;  // + Q block
};

// S[o][at] holds rows a = 16*at + 4*lg + i, column c = 16*(wid + 4*o) + l16.
template <class E, int D>
struct State {
  static constexpr int NT = D / 16;
  static constexpr int NOWN = (NT + 3) / 4;
  f32x4 s[NOWN][NT];
};

// S <- lambda^len S + sum_{c<len, e0+c>=0} lambda^(len-1-c) K[c,:]^T V[c,:]
// with the chunk's K and V row-major in LDS (row stride LDK).
template <class E, int D>
__device__ __forceinline__ void state_update(State<E, D>& st, const E* Ks, const E* Vs, const float* pw,
                                             int len, int e0, int wid, int l16, int lg) {
  using M = Mfma<E>;
  using frag = typename M::frag;
  constexpr int NT = D / 16, NOWN = State<E, D>::NOWN, LDK = FwdLds<E, D>::LDK;
  const float decay = pw[len];
#pragma unroll
  for (int o = 0; o < NOWN; ++o) {
    const int ct = wid + 4 * o;
    if (ct < NT) {
#pragma unroll
      for (int at = 0; at < NT; ++at) st.s[o][at] *= decay;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        float wv[8];
        {
          float vv[8];
          M::to_f32(ColFrag<E>::read(Vs + (kc * 32 + lg * 8) * LDK + ct * 16, LDK, l16), vv);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int c = kc * 32 + lg * 8 + j;
            const float w = (c < len && e0 + c >= 0) ? pw[len - 1 - c] : 0.0f;
            wv[j] = w * vv[j];
          }
        }
        frag bhi, blo;
        M::split(wv, bhi, blo);
#pragma unroll
        for (int at = 0; at < NT; ++at) {
          const frag a = ColFrag<E>::read(Ks + (kc * 32 + lg * 8) * LDK + at * 16, LDK, l16);
          st.s[o][at] = M::mma(a, bhi, st.s[o][at]);
          if (M::kSplit) st.s[o][at] = M::mma(a, blo, st.s[o][at]);
        }
      }
    }
  }
}

template <class E, int D>
__device__ __forceinline__ void state_zero(State<E, D>& st) {
#pragma unroll
  for (int o = 0; o < State<E, D>::NOWN; ++o)
#pragma unroll
    for (int at = 0; at < D / 16; ++at) st.s[o][at] = f32x4{0.f, 0.f, 0.f, 0.f};
}

template <class E, int D>
__device__ __forceinline__ void state_load(State<E, D>& st, const float* g, int wid, int l16, int lg) {
  constexpr int NT = D / 16;
#pragma unroll
  for (int o = 0; o < State<E, D>::NOWN; ++o) {
    const int ct = wid + 4 * o;
#pragma unroll
    for (int at = 0; at < NT; ++at)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = 0.0f;
        if (ct < NT) x = g[(at * 16 + lg * 4 + i) * D + ct * 16 + l16];
        st.s[o][at][i] = x;
      }
  }
}

template <class E, int D>
__device__ __forceinline__ void state_store(const State<E, D>& st, float* g, float mult, int wid, int l16,
                                            int lg) {
  constexpr int NT = D / 16;
#pragma unroll
  for (int o = 0; o < State<E, D>::NOWN; ++o) {
    const int ct = wid + 4 * o;
    if (ct < NT) {
#pragma unroll
      for (int at = 0; at < NT; ++at)
#pragma unroll
        for (int i = 0; i < 4; ++i) g[(at * 16 + lg * 4 + i) * D + ct * 16 + l16] = mult * st.s[o][at][i];
    }
  }
}

// Fragment made of two runs of four consecutive LDS elements (the second
// run replaced by zeros when !second).
template <class E>
__device__ __forceinline__ typename Mfma<E>::frag lds4x2(const E* p0, const E* p1, bool second);
template <>
__device__ __forceinline__ bf16x8 lds4x2<bf16>(const bf16* p0, const bf16* p1, bool second) {
  const bf16x4 a = *(const bf16x4*)p0;
  bf16x4 b = *(const bf16x4*)p1;
  if (!second) b = bf16x4{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
template <>
__device__ __forceinline__ f32x8 lds4x2<float>(const float* p0, const float* p1, bool second) {
  const f32x4 a = *(const f32x4*)p0;
  f32x4 b = *(const f32x4*)p1;
  if (!second) b = f32x4{0.f, 0.f, 0.f, 0.f};
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Store four consecutive outputs of one row.
__device__ __forceinline__ void store4(bf16* dst, f32x4 x) {
  bf16x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = (bf16)x[i];
  *(bf16x4*)dst = r;
}
__device__ __forceinline__ void store4(float* dst, f32x4 x) { *(f32x4*)dst = x; }

// ---------------------------------------------------------------------------
// Per-segment local states: L_m = S over the evictions of segment m, from 0.
// grid = BH * (nseg - 1); writes ws[bh][m + 1].
template <class E, int D>
__global__ void __launch_bounds__(256, 2) seg_state_kernel(FwdArgs a) {
  using L = FwdLds<E, D>;
  __shared__ __attribute__((aligned(16))) char smem[2 * L::TILE];
  __shared__ float pw[72];
  E* Ks = (E*)smem;
  E* Vs = (E*)(smem + L::TILE);
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int nm = a.nseg - 1;
  const int bh = blockIdx.x / nm, m = blockIdx.x - bh * nm;
  const int h = bh % a.H;
  const size_t base = (size_t)bh * a.T * D;
  const uint32_t nbytes = (uint32_t)a.T * D * sizeof(E);
  const auto Kg = make_rsrc((const E*)a.k + base, nbytes);
  const auto Vg = make_rsrc((const E*)a.v + base, nbytes);
  if (tid <= 64) pw[tid] = powi(a.lam[h], tid);
  State<E, D> st;
  state_zero(st);
  TileRegs<E, D, 64> kl, vl;
  int g0 = 0;
  while (g0 < a.G && (m * a.G + g0) * 64 - a.W + 63 < 0) ++g0;
  if (g0 < a.G) {
    kl.load(Kg, (m * a.G + g0) * 64 - a.W);
    vl.load(Vg, (m * a.G + g0) * 64 - a.W);
  }
  for (int g = g0; g < a.G; ++g) {
    const int e0 = (m * a.G + g) * 64 - a.W;
    __syncthreads();
    kl.store(Ks, L::LDK);
    vl.store(Vs, L::LDK);
    __syncthreads();
    if (g + 1 < a.G) {
      kl.load(Kg, e0 + 64);
      vl.load(Vg, e0 + 64);
    }
    state_update(st, Ks, Vs, pw, 64, e0, wid, l16, lg);
  }
  state_store(st, a.seg_state + ((size_t)bh * a.nseg + m + 1) * D * D, 1.0f, wid, l16, lg);
}

// Chain over segments, in place: ws[0] = 0, ws[m+1] = lambda^(64G) ws[m] + L_m.
// grid = (D*D/4 + 255)/256 x BH; each thread owns four consecutive floats and
// loads eight segments ahead of the dependent chain.
template <int D>
__global__ void __launch_bounds__(256) seg_chain_kernel(FwdArgs a) {
  const int bh = blockIdx.y;
  const int x = blockIdx.x * 256 + threadIdx.x;
  if (x * 4 >= D * D) return;
  const float decay = powi(a.lam[bh % a.H], 64 * a.G);
  float4* p = (float4*)(a.seg_state + (size_t)bh * a.nseg * D * D) + x;
  const size_t stride = (size_t)D * D / 4;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  p[0] = s;
  for (int m0 = 1; m0 < a.nseg; m0 += 8) {
    float4 l[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (m0 + u < a.nseg) l[u] = p[(m0 + u) * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (m0 + u < a.nseg) {
        s.x = decay * s.x + l[u].x;
        s.y = decay * s.y + l[u].y;
        s.z = decay * s.z + l[u].z;
        s.w = decay * s.w + l[u].w;
        p[(m0 + u) * stride] = s;
      }
  }
}

// ---------------------------------------------------------------------------
// Fused forward: grid = BH * nseg, 256 threads (4 waves x 16 query rows).
template <class E, int D>
__global__ void __launch_bounds__(256, (D >= 128 ? 1 : 2)) fwd_kernel(FwdArgs a) {
  using M = Mfma<E>;
  using frag = typename M::frag;
  using L = FwdLds<E, D>;
  constexpr int NT = D / 16, NKC = (D + 31) / 32, NOWN = State<E, D>::NOWN;
  constexpr int LDK = L::LDK, LDX = L::LDX;
  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  __shared__ float pw[72];
  E* Ks = (E*)smem;
  E* Vs = (E*)(smem + L::TILE);
  float* X = (float*)smem;
  E* Qs = (E*)(smem + L::U);

  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int bh = blockIdx.x / a.nseg, seg = blockIdx.x - bh * a.nseg;
  const int h = bh % a.H;
  const int T = a.T, W = a.W;
  const size_t base = (size_t)bh * T * D;
  const uint32_t nbytes = (uint32_t)T * D * sizeof(E);
  const auto Qg = make_rsrc((const E*)a.q + base, nbytes);
  const auto Kg = make_rsrc((const E*)a.k + base, nbytes);
  const auto Vg = make_rsrc((const E*)a.v + base, nbytes);
  E* Yg = (E*)a.y + base;
  const float seta = sigmoidf(a.gate[h]) * a.eta[h];
  const float sl2 = a.scale * kLog2e;
  if (tid <= 64) pw[tid] = powi(a.lam[h], tid);

  State<E, D> st;
  if (seg == 0)
    state_zero(st);
  else
    state_load(st, a.seg_state + ((size_t)bh * a.nseg + seg) * D * D, wid, l16, lg);

  const int jb = seg * a.G;
  const int je = min(a.nblk, jb + a.G);
  const int r = wid * 16 + l16;  // this lane's row within the block
  TileRegs<E, D, 64> ql, kl, vl;
  ql.load(Qg, jb * 64);
  kl.load(Kg, (max(0, jb * 64 - W + 1) >> 6) * 64);
  vl.load(Vg, (max(0, jb * 64 - W + 1) >> 6) * 64);
  for (int j = jb; j < je; ++j) {
    const int t0 = j * 64;
    const int trow = t0 + r;
    const int e0 = t0 - W;
    const bool has_mem = t0 + 63 >= W;
    const bool more = j + 1 < je;
    const int next_k0 = (max(0, t0 + 64 - W + 1) >> 6) * 64;
    __syncthreads();
    ql.store(Qs, LDK);
    ql.load(Qg, t0 + 64);  // next block's queries, in flight during this block
    __syncthreads();
    frag qf[NKC];
#pragma unroll
    for (int dc = 0; dc < NKC; ++dc)
      qf[dc] = (dc * 32 + lg * 8 < D) ? M::lds8(Qs + r * LDK + dc * 32 + lg * 8) : M::zero();

    float mrow = kNegInf, lrow = 0.0f;
    f32x4 O[NT];
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) O[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // ---- L1: band tiles ----
    const int kt_lo = max(0, t0 - W + 1) >> 6;
    const int kt_hi = min(T - 1, t0 + 63) >> 6;
    for (int kt = kt_lo; kt <= kt_hi; ++kt) {
      const int k0 = kt * 64;
      if (kt > kt_lo) __syncthreads();
      kl.store(Ks, LDK);
      vl.store(Vs, LDK);
      __syncthreads();
      {
        // next tile of this block, else the evicted chunk, else the next block's first tile
        const int nr = (kt < kt_hi) ? k0 + 64 : (has_mem ? e0 : next_k0);
        kl.load(Kg, nr);
        vl.load(Vg, nr);
      }
      f32x4 Z[4];
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        Z[n] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int kr = 32 * (n >> 1) + (l16 >> 2) * 8 + (n & 1) * 4 + (l16 & 3);
#pragma unroll
        for (int dc = 0; dc < NKC; ++dc) {
          const frag ka = (dc * 32 + lg * 8 < D) ? M::lds8(Ks + kr * LDK + dc * 32 + lg * 8) : M::zero();
          Z[n] = M::mma(ka, qf[dc], Z[n]);
        }
      }
      const bool full = (k0 + 63 <= t0) && (k0 >= t0 + 64 - W);
      float zv[16];
      float mz = kNegInf;
#pragma unroll
      for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = k0 + 32 * (n >> 1) + lg * 8 + (n & 1) * 4 + i;
          float z = Z[n][i];
          if (!full && !(key <= trow && key > trow - W)) z = kNegInf;
          zv[(n >> 1) * 8 + (n & 1) * 4 + i] = z;
          mz = fmaxf(mz, z);
        }
      mz = max4(mz);
      const float mnew = fmaxf(mrow, mz * sl2);
      const float msafe = (mnew == kNegInf) ? 0.0f : mnew;
      const float alpha = exp2f(mrow - msafe);
      float ps = 0.0f;
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        zv[x] = exp2f(__builtin_fmaf(zv[x], sl2, -msafe));
        ps += zv[x];
      }
      ps = sum4(ps);
      lrow = lrow * alpha + ps;
      mrow = mnew;
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) O[dt] *= alpha;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        float pv[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) pv[jj] = zv[p * 8 + jj];
        const frag pf = M::pack(pv);
#pragma unroll
        for (int dt = 0; dt < NT; ++dt)
          O[dt] = M::mma(ColFrag<E>::read(Vs + (p * 32 + lg * 8) * LDK + dt * 16, LDK, l16), pf, O[dt]);
      }
    }
    {
      const float inv = 1.0f / lrow;
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) O[dt] *= inv;
      if (a.lse && lg == 0 && trow < T) a.lse[(size_t)bh * T + trow] = (mrow + __log2f(lrow)) * kLn2;
    }

    // ---- L2: read of the eviction state and the evicted chunk ----
    const bool last = (j == a.nblk - 1);
    if (has_mem) {
      __syncthreads();  // every wave is done with the last band tile
      if (e0 > 0) {
        // (QS)^T for this wave's state columns and all 64 rows -> X[row][c]
#pragma unroll
        for (int o = 0; o < NOWN; ++o) {
          const int ct = wid + 4 * o;
          if (ct < NT) {
            f32x4 acc[4];
#pragma unroll
            for (int rg = 0; rg < 4; ++rg) acc[rg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int pp = 0; pp < (NT + 1) / 2; ++pp) {
              float sv8[8];
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                sv8[i] = st.s[o][2 * pp][i];
                sv8[4 + i] = (2 * pp + 1 < NT) ? st.s[o][(2 * pp + 1) % NT][i] : 0.0f;
              }
              frag shi, slo;
              M::split(sv8, shi, slo);
#pragma unroll
              for (int rg = 0; rg < 4; ++rg) {
                const E* qrow = Qs + (rg * 16 + l16) * LDK;
                const frag qb = lds4x2<E>(qrow + 32 * pp + lg * 4, qrow + (32 * pp + 16 + lg * 4) % D,
                                          32 * pp + 16 < D);
                acc[rg] = M::mma(shi, qb, acc[rg]);
                if (M::kSplit) acc[rg] = M::mma(slo, qb, acc[rg]);
              }
            }
#pragma unroll
            for (int rg = 0; rg < 4; ++rg)
              *(f32x4*)(X + (rg * 16 + l16) * LDX + ct * 16 + lg * 4) = acc[rg];
          }
        }
        __syncthreads();
        const float f = seta * pw[r + 1];
#pragma unroll
        for (int dt = 0; dt < NT; ++dt) {
          const f32x4 xv = *(const f32x4*)(X + r * LDX + dt * 16 + lg * 4);
          O[dt] += f * xv;
        }
        __syncthreads();
      }
      // evicted chunk e0 .. e0+63 (prefetched during the last band tile)
      kl.store(Ks, LDK);
      vl.store(Vs, LDK);
      __syncthreads();
      kl.load(Kg, next_k0);
      vl.load(Vg, next_k0);
      f32x4 Z[4];
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        Z[n] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int kr = 32 * (n >> 1) + (l16 >> 2) * 8 + (n & 1) * 4 + (l16 & 3);
#pragma unroll
        for (int dc = 0; dc < NKC; ++dc) {
          const frag ka = (dc * 32 + lg * 8 < D) ? M::lds8(Ks + kr * LDK + dc * 32 + lg * 8) : M::zero();
          Z[n] = M::mma(ka, qf[dc], Z[n]);
        }
      }
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        float pv[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int c = 32 * p + lg * 8 + jj;  // chunk index of the key
          const float z = Z[2 * p + (jj >> 2)][jj & 3];
          pv[jj] = (c <= r && e0 + c >= 0) ? seta * pw[r - c] * z : 0.0f;
        }
        const frag pf = M::pack(pv);
#pragma unroll
        for (int dt = 0; dt < NT; ++dt)
          O[dt] = M::mma(ColFrag<E>::read(Vs + (p * 32 + lg * 8) * LDK + dt * 16, LDK, l16), pf, O[dt]);
      }
      // carry the state to the next block (or to step T-1 for A_final)
      if (more) {
        state_update(st, Ks, Vs, pw, 64, e0, wid, l16, lg);
      } else if (last && a.A_final) {
        state_update(st, Ks, Vs, pw, T - t0, e0, wid, l16, lg);
      }
    }
    // ---- store y ----
    if (trow < T) {
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) store4(Yg + (size_t)trow * D + dt * 16 + lg * 4, O[dt]);
    }
    if (last && a.A_final) {
      float* Af = a.A_final + (size_t)bh * D * D;
      if (has_mem)
        state_store(st, Af, a.eta[h], wid, l16, lg);
      else
        for (int x = tid; x < D * D; x += 256) Af[x] = 0.0f;
    }
  }
}

template <class E, int D>
static hipError_t launch_fwd_impl(const FwdArgs& a, hipStream_t s) {
  const int BH = a.B * a.H;
  if (a.nseg > 1) {
    hipLaunchKernelGGL((seg_state_kernel<E, D>), dim3(BH * (a.nseg - 1)), dim3(256), 0, s, a);
    hipLaunchKernelGGL((seg_chain_kernel<D>), dim3((D * D / 4 + 255) / 256, BH), dim3(256), 0, s, a);
  }
  hipLaunchKernelGGL((fwd_kernel<E, D>), dim3(BH * a.nseg), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_forward(const FwdArgs& a, int D, bool is_bf16, hipStream_t s) {
  if (is_bf16) {
    switch (D) {
      case 16: return launch_fwd_impl<bf16, 16>(a, s);
      case 32: return launch_fwd_impl<bf16, 32>(a, s);
      case 64: return launch_fwd_impl<bf16, 64>(a, s);
      case 128: return launch_fwd_impl<bf16, 128>(a, s);
    }
  } else {
    switch (D) {
      case 16: return launch_fwd_impl<float, 16>(a, s);
      case 32: return launch_fwd_impl<float, 32>(a, s);
      case 64: return launch_fwd_impl<float, 64>(a, s);
      case 128: return launch_fwd_impl<float, 128>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace tck

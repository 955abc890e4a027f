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
#include <type_traits>

#include "tc_device.h"
#include "tc_fwd_common.h"
#include "tc_launch.h"

namespace tck {

// LDS plan of the fused forward kernel (elements / bytes).  K and V tiles
// are stored row-major; operands that contract down their rows are read with
// transpose reads (ColFrag).  X (float rows x D) aliases the K/V tiles: it is
// only live between the band loop and the store of the evicted chunk.
//
// bf16 with D = 128 keeps the D x D state in LDS as float S^T (row stride
// LDSS, an odd number of 16-byte chunks: conflict-free 16-lane reads) instead
// of in registers, which leaves the band loop without register spills; the
// other instantiations keep it in MFMA accumulators (the float32 D = 128 state
// would not fit in LDS beside the tiles).
template <class E, int D>
struct FwdLds {
  static constexpr bool LS = std::is_same<E, bf16>::value && D == 128;  // state in LDS
  static constexpr int VE = 16 / sizeof(E);
  static constexpr int LDK = D + VE;  // row stride of K, V, Q tiles
  static constexpr int LDX = D + 4;
  static constexpr int LDSS = D + 4;
  static constexpr int TILE = 64 * LDK * (int)sizeof(E);
  static constexpr int XB = 64 * LDX * 4;
  static constexpr int U = (LS || (2 * TILE) > XB) ? (2 * TILE) : XB;
  static constexpr int SB = LS ? D * LDSS * 4 : 0;
  static constexpr int TOTAL = U + TILE + SB;  // + Q block (+ S^T)
};

// ---------------------------------------------------------------------------
// Note on float32 inputs.  On gfx950 a VALU read of a float32 16x16x4 MFMA
// result needs 10 wait states, and a v_accvgpr_mov_b32 copy of it more than
// 8 (measured).  Where a kernel runs at one workgroup per compute unit the
// compiler keeps accumulators in AGPRs and, at some control-flow joins, copies
// them with v_accvgpr_mov_b32 too soon, which reads a stale element.  This
// kernel at two workgroups per unit (D <= 64) keeps every accumulator in
// VGPRs, so the library runs float32 inputs of D <= 64 here.
//
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
  float* Sl = (float*)(smem + L::U + L::TILE);  // (LS only)
  constexpr bool LS = L::LS;
  constexpr int LDSS = L::LDSS;

  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int bh = blockIdx.x / a.nseg, seg = blockIdx.x - bh * a.nseg;
  const int h = bh % a.H;
  const int T = a.T, W = a.W;
  const size_t base = (size_t)bh * T * D;
  const uint32_t nbytes = (uint32_t)T * D * sizeof(E);
  const auto Qg = make_rsrc((const E*)a.q + base, nbytes);
  const auto Kg = make_rsrc((const E*)a.k + base, nbytes);
  const auto Vg = make_rsrc((const E*)a.v + base, nbytes);
  const int Tout = T - a.row0;  // stored rows
  E* Yg = (E*)a.y + (size_t)bh * Tout * D;
  const float seta = sigmoidf(a.gate[h]) * a.eta[h];
  const float sl2 = a.scale * kLog2e;
  if (tid <= 64) pw[tid] = powi(a.lam[h], tid);

  State<E, D> st;
  if (LS) {
    // S^T at the segment start -> LDS (read by every wave after the band loop's barriers)
    const float* g = a.seg_state + ((size_t)bh * a.nseg + seg) * D * D;
    for (int x = tid; x < D * D; x += 256) Sl[(x % D) * LDSS + x / D] = seg == 0 ? 0.0f : g[x];
  } else if (seg == 0) {
    state_zero(st);
  } else {
    state_load(st, a.seg_state + ((size_t)bh * a.nseg + seg) * D * D, wid, l16, lg);
  }
  vm_fence_loads();

  const int jb = seg_first_block(a, seg);
  const int je = seg_first_block(a, seg + 1);
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
      // scores, online softmax and P V for one 64-key tile; FULL: every key of
      // the tile is inside every row's window (no mask)
      auto tile = [&](auto full_c) {
        constexpr bool FULL = decltype(full_c)::value;
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
        float zv[16];
        float mz = kNegInf;
#pragma unroll
        for (int n = 0; n < 4; ++n)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float z = Z[n][i];
            if (!FULL) {
              const int key = k0 + 32 * (n >> 1) + lg * 8 + (n & 1) * 4 + i;
              if (!(key <= trow && key > trow - W)) z = kNegInf;
            }
            zv[(n >> 1) * 8 + (n & 1) * 4 + i] = z;
            mz = fmaxf(mz, z);
          }
        mz = xmax4(mz);
        const float mnew = fmaxf(mrow, mz * sl2);
        const float msafe = (mnew == kNegInf) ? 0.0f : mnew;
        const float alpha = fast_exp2(mrow - msafe);
        float ps = 0.0f;
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          zv[x] = fast_exp2(__builtin_fmaf(zv[x], sl2, -msafe));
          ps += zv[x];
        }
        lrow = lrow * alpha + ps;  // this lane's share of the row sum
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
      };
      if ((k0 + 63 <= t0) && (k0 >= t0 + 64 - W))
        tile(std::true_type{});
      else
        tile(std::false_type{});
    }
    {
      lrow = xsum4(lrow);
      const float inv = 1.0f / lrow;
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) O[dt] *= inv;
      if (a.lse && lg == 0 && trow >= a.row0 && trow < T)
        a.lse[(size_t)bh * Tout + trow - a.row0] = (mrow + __log2f(lrow)) * kLn2;
    }

    // ---- L2: read of the eviction state and the evicted chunk ----
    const bool last = (j == a.nblk - 1);
    if (has_mem) {
      __syncthreads();  // every wave is done with the last band tile
      if (LS && e0 > 0) {
        // O += sigma(g) eta lambda^(r+1) q S(e0), S^T read from LDS as hi/lo bf16
        const float f = seta * pw[r + 1];
#pragma unroll
        for (int dt = 0; dt < NT; ++dt) {
          f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int dc = 0; dc < NKC; ++dc) {
            float sv[8];
            const float* sp = Sl + (dt * 16 + l16) * LDSS + dc * 32 + lg * 8;
            const f32x4 x0 = *(const f32x4*)sp;
            const f32x4 x1 = *(const f32x4*)(sp + 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              sv[i] = x0[i];
              sv[4 + i] = x1[i];
            }
            frag shi, slo;
            M::split(sv, shi, slo);
            acc = M::mma(shi, qf[dc], acc);
            if (M::kSplit) acc = M::mma(slo, qf[dc], acc);
          }
          O[dt] += f * acc;
        }
      } else if (e0 > 0) {
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
      // carry the state to the next block (or to step T-1 for A_final); with
      // the state in LDS every wave has read it (the barrier after the chunk
      // tiles were stored) before the owners of its column tiles update it
      if (more || (last && a.A_final)) {
        const int len = more ? 64 : T - t0;
        if (LS)
          lds_state_update_cols<E, D, LDSS>(Sl, Ks, LDK, Vs, LDK, pw, len, e0, wid, l16, lg);
        else
          state_update(st, Ks, LDK, Vs, LDK, pw, len, e0, wid, l16, lg);
      }
    }
    // ---- store y ----
    if (trow >= a.row0 && trow < T) {
      const size_t o = (size_t)(trow - a.row0) * D + lg * 4;
      if (a.yadd) {
#pragma unroll
        for (int dt = 0; dt < NT; ++dt) O[dt] += *(const f32x4*)(a.yadd + (size_t)bh * Tout * D + o + dt * 16);
      }
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) store4(Yg + o + dt * 16, O[dt]);
    }
    if (last && a.A_final) {
      float* Af = a.A_final + (size_t)bh * D * D;
      if (LS) {
        __syncthreads();  // the state update above is done
        const float eta = a.eta[h];
        for (int x = tid; x < D * D; x += 256) Af[x] = has_mem ? eta * Sl[(x % D) * LDSS + x / D] : 0.0f;
      } else if (has_mem) {
        state_store(st, Af, a.eta[h], wid, l16, lg);
      } else {
        for (int x = tid; x < D * D; x += 256) Af[x] = 0.0f;
      }
    }
  }
}

template <class E, int D>
static hipError_t launch_fwd_impl(const FwdArgs& a, hipStream_t s) {
  const int BH = a.B * a.H;
  if (a.nseg > 1) {
    hipLaunchKernelGGL((seg_state_kernel<E, D, 64>), dim3(BH * (a.nseg - 1)), dim3(256), 0, s, a);
    hipLaunchKernelGGL((seg_chain_kernel<D, 64>), dim3((D * D / 4 + kChainThreads - 1) / kChainThreads, BH), dim3(kChainThreads), 0, s, a);
  }
  hipLaunchKernelGGL((fwd_kernel<E, D>), dim3(BH * a.nseg), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_forward(const FwdArgs& a, int D, bool is_bf16, hipStream_t s) {
  if (is_bf16) return D == 128 ? launch_fwd_impl<bf16, 128>(a, s) : hipErrorInvalidValue;
  switch (D) {
    case 16: return launch_fwd_impl<float, 16>(a, s);
    case 32: return launch_fwd_impl<float, 32>(a, s);
    case 64: return launch_fwd_impl<float, 64>(a, s);
    case 128: return launch_fwd_impl<float, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tck

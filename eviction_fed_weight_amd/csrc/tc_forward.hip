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

#ifndef TC_FWD_F32
#error "compile with -DTC_FWD_F32=0 (bf16 kernels) or -DTC_FWD_F32=1 (float32 kernels)"
#endif

#include "tc_device.h"
#include "tc_fwd_common.h"
#include "tc_launch.h"

namespace tck {

// LDS plan of the fused forward kernel (elements / bytes).  K and V tiles
// are stored row-major; operands that contract down their rows are read with
// transpose reads (ColFrag).  X (float rows x D) aliases the K/V tiles: it is
// only live between the band loop and the store of the evicted chunk.
//
// With D = 128 the D x D state lives in LDS as float S^T (row stride LDSS,
// an odd number of 16-byte chunks: conflict-free 16-lane reads) instead of in
// registers, which leaves the band loop without register spills; with D <= 64
// it is kept in MFMA accumulators.  For float32 with D = 128 the Q block is
// staged in the K tile's buffer (QA: it is read into registers once per block,
// before the first key tile is stored), so that the tiles and the float32
// state fit in the 160 KB of LDS.
//
// Blocks of BMR query rows, 16 per wave.  bf16 with D = 128 runs 128-row
// blocks on eight waves at one workgroup per compute unit (two waves per
// SIMD, and every key/value tile staged in LDS serves 128 rows); its evicted
// chunk is two 64-row tiles.  The other instances run 64-row blocks on four
// waves.
template <class E, int D>
struct FwdLds {
  static constexpr bool LS = D == 128;                                  // state in LDS
  static constexpr bool QA = LS && !std::is_same<E, bf16>::value;       // Q staged in the K buffer
  static constexpr int BMR = (std::is_same<E, bf16>::value && D == 128) ? 128 : 64;  // rows per block
  static constexpr int NWV = BMR / 16;                                  // waves
  static constexpr int NTH = 64 * NWV;                                  // threads
  static constexpr int MINB = NWV == 8 ? 1 : 2;                         // workgroups per unit (launch bound)
  static constexpr int NCH = BMR / 64;                                  // tiles of the evicted chunk
  static constexpr int VE = 16 / sizeof(E);
  static constexpr int LDK = D + VE;  // row stride of K, V, Q tiles
  static constexpr int LDX = D + 4;
  static constexpr int LDSS = D + 4;
  static constexpr int TILE = 64 * LDK * (int)sizeof(E);
  static constexpr int QB = BMR * LDK * (int)sizeof(E);
  static constexpr int XB = 64 * LDX * 4;
  static constexpr int U = (LS || (2 * TILE) > XB) ? (2 * TILE) : XB;
  static constexpr int SB = LS ? D * LDSS * 4 : 0;
  static constexpr int TOTAL = U + (QA ? 0 : QB) + SB;  // + Q block (+ S^T)
  static_assert(BMR == 64 || LS, "128-row blocks keep the state in LDS");
};

// ---------------------------------------------------------------------------
// Note on float32 inputs.  On gfx950 a VALU read of a float32 16x16x4 MFMA
// result needs 10 wait states, and a v_accvgpr_mov_b32 copy of it more than
// 8 (measured).  Where a kernel may use more than 256 registers per lane the
// compiler keeps accumulators in AGPRs and, at some control-flow joins, copies
// them with v_accvgpr_mov_b32 too soon, which reads a stale element.  Every
// float32 instantiation is therefore bounded to 256 registers (the launch
// bound of two workgroups per unit; with D = 128 the LDS still holds only
// one), which keeps every accumulator in VGPRs and uses no AGPR at all.
//
// Fused forward: grid = BH * nseg, NWV waves of 16 query rows each.
// RING: a continuation (row0 > 0) whose first row0 keys and values are read
// from the ring.
template <class E, int D, bool RING = false>
__global__ void __launch_bounds__((FwdLds<E, D>::NTH), (FwdLds<E, D>::MINB)) fwd_kernel(FwdArgs a) {
  using M = Mfma<E>;
  using frag = typename M::frag;
  using L = FwdLds<E, D>;
  constexpr int NT = D / 16, NKC = (D + 31) / 32, NOWN = State<E, D>::NOWN;
  constexpr int LDK = L::LDK, LDX = L::LDX;
  constexpr int BMR = L::BMR, NTH = L::NTH, NCH = L::NCH;
  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  __shared__ float pw[BMR + 8];  // pw[n] = lambda^n, 0 <= n <= BMR
  E* Ks = (E*)smem;
  E* Vs = (E*)(smem + L::TILE);
  float* X = (float*)smem;
  constexpr bool LS = L::LS, QA = L::QA;
  E* Qs = QA ? Ks : (E*)(smem + L::U);
  float* Sl = (float*)(smem + L::U + (QA ? 0 : L::QB));  // (LS only)
  constexpr int LDSS = L::LDSS;

  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int bh = blockIdx.x / a.nseg, seg = blockIdx.x - bh * a.nseg;
  const int h = bh % a.H;
  const int T = a.T, W = a.W;
  const auto Qg = query_rows<E, D>(a, bh);  // (query row t is row t - row0 of q)
  const SeqRows Kg = seq_rows<E, D>(a, a.k, a.k_ring, bh);
  const SeqRows Vg = seq_rows<E, D>(a, a.v, a.v_ring, bh);
  const int Tout = T - a.row0;  // stored rows
  E* Yg = (E*)a.y + (size_t)bh * Tout * D;
  const float seta = sigmoidf(a.gate[h]) * a.eta[h];
  const float sl2 = a.scale * kLog2e;
  for (int x = tid; x <= BMR; x += NTH) pw[x] = powi(a.lam[h], x);

  // S at the segment start: S(0) (zero, or A_in / eta) for the first segment
  State<E, D> st;
  const float ie = 1.0f / a.eta[h];
  const float* g0 = a.A_in ? a.A_in + (size_t)bh * D * D : nullptr;
  if (a.window_only) {
    state_zero(st);  // (no memory path: the state is never read)
  } else if (LS) {
    // S^T at the segment start -> LDS (read by every wave after the band loop's barriers)
    const float* g = a.seg_state + ((size_t)bh * a.nseg + seg) * D * D;
    for (int x = tid; x < D * D; x += NTH) Sl[(x % D) * LDSS + x / D] = seg > 0 ? g[x] : g0 ? ie * g0[x] : 0.0f;
  } else if (seg > 0) {
    state_load(st, a.seg_state + ((size_t)bh * a.nseg + seg) * D * D, wid, l16, lg);
  } else if (g0) {
    state_load(st, g0, wid, l16, lg);
    state_scale(st, ie);
  } else {
    state_zero(st);
  }
  vm_fence_loads();

  const int jb = seg_first_block(a, seg);
  const int je = seg_first_block(a, seg + 1);
  const int r = wid * 16 + l16;  // this lane's row within the block
  if (a.status && tid == 0) a.status[blockIdx.x] = a.gen;  // (no flag waits in this kernel)
  TileRegs<E, D, BMR, NTH> ql;
  KVRegs<RING, E, D, 64, NTH> kl, vl;
  if (!QA) ql.load(Qg, jb * BMR - a.row0);
  // Tiles are loaded one item ahead (in flight while the current one is
  // computed), except for float32 with D = 128 (QA), where the staging
  // registers of a prefetch would push the kernel past 256 registers: there
  // each tile is loaded right before it is stored.
  if (!QA) {
    load_seq<RING>(kl, Kg, (max(0, jb * BMR - W + 1) >> 6) * 64);
    load_seq<RING>(vl, Vg, (max(0, jb * BMR - W + 1) >> 6) * 64);
  }
  for (int j = jb; j < je; ++j) {
    const int t0 = j * BMR;
    const int trow = t0 + r;
    const int e0 = t0 - W;
    const bool has_mem = !a.window_only && t0 + BMR - 1 >= W;
    const bool more = j + 1 < je;
    const int next_k0 = (max(0, t0 + BMR - W + 1) >> 6) * 64;
    const int R0 = t0 + 16 * wid;  // first row of this wave
    __syncthreads();
    if (QA) ql.load(Qg, t0 - a.row0);  // (float32 D = 128: no registers to spare for a prefetch)
    ql.store(Qs, LDK);
    if (!QA) ql.load(Qg, t0 + BMR - a.row0);  // next block's queries, in flight during this block
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
    const int kt_hi = min(T - 1, t0 + BMR - 1) >> 6;
    for (int kt = kt_lo; kt <= kt_hi; ++kt) {
      const int k0 = kt * 64;
      if (kt > kt_lo || QA) __syncthreads();  // (QA: every wave has read its Q rows from the K buffer)
      if (QA) {
        load_seq<RING>(kl, Kg, k0);
        load_seq<RING>(vl, Vg, k0);
      }
      kl.store(Ks, LDK);
      vl.store(Vs, LDK);
      __syncthreads();
      if (!QA) {
        // next tile of this block, else the evicted chunk, else the next block's first tile
        const int nr = (kt < kt_hi) ? k0 + 64 : (has_mem ? e0 : next_k0);
        load_seq<RING>(kl, Kg, nr);
        load_seq<RING>(vl, Vg, nr);
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
        mz = xmax4(mz) * sl2;
        // move the reference max only when some row's maximum grew by more
        // than 2^8 (the probabilities stay below 256), so that most tiles
        // leave the accumulators unscaled
        if (__builtin_amdgcn_ballot_w64(mz > mrow + 8.0f)) {
          const float mnew = fmaxf(mrow, mz);
          const float alpha = fast_exp2(mrow - (mnew == kNegInf ? 0.0f : mnew));
          lrow *= alpha;
#pragma unroll
          for (int dt = 0; dt < NT; ++dt) O[dt] *= alpha;
          mrow = mnew;
        }
        const float msafe = (mrow == kNegInf) ? 0.0f : mrow;
        float ps = 0.0f;
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          zv[x] = fast_exp2(__builtin_fmaf(zv[x], sl2, -msafe));
          ps += zv[x];
        }
        lrow += ps;  // this lane's share of the row sum
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
      // (per wave: no key of the tile in any of its rows' windows -> nothing
      // to add; every key in every window -> no mask)
      if (!(k0 > R0 + 15 || k0 + 63 <= R0 - W)) {
        if ((k0 + 63 <= R0) && (k0 >= R0 + 16 - W))
          tile(std::true_type{});
        else
          tile(std::false_type{});
      }
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
      if (LS && (e0 > 0 || g0)) {
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
      } else if (e0 > 0 || g0) {
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
      // evicted chunk e0 .. e0+BMR-1, as NCH tiles of 64 (each prefetched
      // during the item before it): the intra-chunk terms of the read, then
      // the carry of the state (every wave has read S(e0) above, before the
      // barrier after the first chunk tile is stored)
      for (int c = 0; c < NCH; ++c) {
        const int ec = e0 + 64 * c;  // first eviction of chunk tile c
        if (c > 0) __syncthreads();  // tile c-1 and its state update are done
        if (QA) {
          load_seq<RING>(kl, Kg, ec);
          load_seq<RING>(vl, Vg, ec);
        }
        kl.store(Ks, LDK);
        vl.store(Vs, LDK);
        __syncthreads();
        if (!QA) {
          const int nr = c + 1 < NCH ? ec + 64 : next_k0;
          load_seq<RING>(kl, Kg, nr);
          load_seq<RING>(vl, Vg, nr);
        }
        if (16 * wid + 15 >= 64 * c) {  // (rows before the tile read none of its keys)
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
              const int cc = 64 * c + 32 * p + lg * 8 + jj;  // chunk index of the key
              const float z = Z[2 * p + (jj >> 2)][jj & 3];
              pv[jj] = (cc <= r && e0 + cc >= 0) ? seta * pw[r - cc] * z : 0.0f;
            }
            const frag pf = M::pack(pv);
#pragma unroll
            for (int dt = 0; dt < NT; ++dt)
              O[dt] = M::mma(ColFrag<E>::read(Vs + (p * 32 + lg * 8) * LDK + dt * 16, LDK, l16), pf, O[dt]);
          }
        }
        // carry the state to the next block (or to step T-1 for A_final)
        if (more || (last && a.A_final)) {
          const int len = more ? 64 : min(64, T - t0 - 64 * c);
          if (len > 0) {
            if (LS)
              lds_state_update_cols<E, D, LDSS, L::NWV>(Sl, Ks, LDK, Vs, LDK, pw, len, ec, wid, l16, lg);
            else
              state_update(st, Ks, LDK, Vs, LDK, pw, len, ec, wid, l16, lg);
          }
        }
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
        for (int x = tid; x < D * D; x += NTH) Af[x] = has_mem ? eta * Sl[(x % D) * LDSS + x / D] : 0.0f;
      } else if (has_mem) {
        state_store(st, Af, a.eta[h], wid, l16, lg);
      } else {
        for (int x = tid; x < D * D; x += NTH) Af[x] = 0.0f;
      }
    }
  }
}

template <class E, int D>
static hipError_t launch_fwd_impl(const FwdArgs& a0, hipStream_t s) {
  FwdArgs a = a0;
  if (a.mean_c != 0 || a.final_slot || a.nparts > kMaxStateParts)
    return hipErrorInvalidValue;  // (the chunk-mean shortcut and the final slot belong to the rows kernel)
  constexpr int BMR = FwdLds<E, D>::BMR, NTH = FwdLds<E, D>::NTH;
  a.blk_pow = BMR;  // exact scan: one decay per evicted token of a block
  const int BH = a.B * a.H;
  const bool ring = a.row0 > 0;
  if (a.nseg > 1 && !a.window_only) {
    const dim3 sg(BH * (a.nseg - 1) * (a.nparts > 1 ? a.nparts : 1));
    if (ring)
      hipLaunchKernelGGL((seg_state_kernel<E, D, BMR, 0, true>), sg, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((seg_state_kernel<E, D, BMR>), sg, dim3(256), 0, s, a);
    hipLaunchKernelGGL((seg_chain_kernel<D, BMR>), dim3((D * D + kChainThreads - 1) / kChainThreads, BH),
                       dim3(kChainThreads), 0, s, a);
  }
  if (ring)
    hipLaunchKernelGGL((fwd_kernel<E, D, true>), dim3(BH * a.nseg), dim3(NTH), 0, s, a);
  else
    hipLaunchKernelGGL((fwd_kernel<E, D>), dim3(BH * a.nseg), dim3(NTH), 0, s, a);
  return hipGetLastError();
}

// This file is compiled twice: TC_FWD_F32=0 builds the bf16 D = 128 kernels
// (default register form), TC_FWD_F32=1 the float32 kernels with matrix-core
// results in VGPRs (-mllvm -amdgpu-mfma-vgpr-form): the float32 D = 128
// kernel needs a few more than 256 registers, and in the default form the
// compiler would then keep its accumulators in AGPRs (see the note on
// float32 inputs above); in the VGPR form AGPRs hold only spilled integer
// indices, never a matrix-core result.
#if TC_FWD_F32
hipError_t launch_forward_f32(const FwdArgs& a, int D, hipStream_t s) {
  switch (D) {
    case 16: return launch_fwd_impl<float, 16>(a, s);
    case 32: return launch_fwd_impl<float, 32>(a, s);
    case 64: return launch_fwd_impl<float, 64>(a, s);
    case 128: return launch_fwd_impl<float, 128>(a, s);
  }
  return hipErrorInvalidValue;
}
#else
hipError_t launch_forward_bf16(const FwdArgs& a, int D, hipStream_t s) {
  return D == 128 ? launch_fwd_impl<bf16, 128>(a, s) : hipErrorInvalidValue;
}
#endif

}  // namespace tck

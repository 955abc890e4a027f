// TC forward for head dimensions up to 64 on gfx950: 128 query rows per
// block, four waves of 32 rows each.
//
// Method ("Tensor Cache: Eviction-conditioned Associative Memory for
// Transformers"): Section 3.1 Eq. (1) window softmax over the last W keys;
// Section 3.2 and Figure 2 write-on-evict A <- lambda A + eta k v^T, read
// m = q A, output y = y_local + sigmoid(g) m; abstract: the state is a
// weighted-sum scan of the evicted pairs.
//
// Scan.  S(e) = sum_{i<e} lambda^(e-1-i) k_i v_i^T and A_t = eta S(t-W+1).
// Block j holds rows t0 = 128 j .. t0+127 and evicts e0 = t0 - W .. e0+127;
// for row t = t0 + r
//   A_t = eta [ lambda^(r+1) S(e0) + sum_{c<=r} lambda^(r-c) k_{e0+c} v_{e0+c}^T ]
// so the read is q S(e0) plus a lower-triangular decay-weighted 128 x 128
// product with the evicted chunk (q (k outer v) = <q,k> v), and the state
// advances by two decayed rank-64 updates.
//
// Work of a workgroup: the blocks of one segment, each as a stream of 64-key
// items -- the window's key tiles, then the two tiles of the evicted chunk --
// through a two-buffer LDS pipeline with one barrier per item.  While an
// item is computed from one buffer, the next item (already in registers) is
// written to the other and the item after it is being loaded from HBM.
//
// Per wave and item: scores for 32 rows x 64 keys (16 MFMAs; every K
// fragment read from LDS feeds both 16-row groups), softmax on the
// transposed score layout (a lane holds one query row, so row statistics need
// only a four-lane exchange), and P V (16 MFMAs, V fragments shared by both
// groups).  The running max is only moved when a row's maximum grows by more
// than 2^8 (probabilities stay below 256), which leaves most tiles without
// the rescale of the accumulators.
#include <type_traits>

#include "tc_device.h"
#include "tc_fwd_common.h"
#include "tc_launch.h"

namespace tck {

template <class E, int D>
struct F128 {
  static constexpr int VE = 16 / (int)sizeof(E);
  // Row strides (elements).  K, Q and S^T are read 16 rows x 16 bytes at a
  // time (odd number of 16-byte chunks per row: no bank conflicts); V is read
  // with transpose reads of 8 rows x 32 bytes (stride 10 chunks for D = 64).
  static constexpr int LDK = D + VE;
  static constexpr int LDV = D + 2 * VE;
  static constexpr int KT = 64 * LDK * (int)sizeof(E);
  static constexpr int VT = 64 * LDV * (int)sizeof(E);
  static constexpr int BUF = KT + VT;
  static constexpr int QB = 128 * LDK * (int)sizeof(E);
  // The state lives in LDS as float S^T (S[a][c] at c * LDS + a; 17 chunks
  // per row for D = 64), so it costs no registers between its uses.
  static constexpr int LDS = D + 4;
  static constexpr int SB = D * LDS * 4;
  static constexpr int TOTAL = 2 * BUF + QB + SB;
  static constexpr int NT = D / 16;
  static constexpr int NKC = (D + 31) / 32;
};

// Rows rb..rb+3 and rb+16..rb+19 at column c0 + l16 of a row-major LDS tile:
// the 8 contraction values of the V operand for keys in the order the
// score layout produces them (key 16 n + 4 lg + i sits at contraction index
// 8 lg + 4 (n & 1) + i of the 32-key chunk n >> 1).
template <class E>
struct VFrag;
template <>
struct VFrag<bf16> {
  static __device__ __forceinline__ bf16x8 read(const bf16* tile, int ld, int rb, int c0, int l16) {
    const bf16* p0 = tile + (rb + (l16 >> 2)) * ld + c0 + 4 * (l16 & 3);
    const bf16* p1 = p0 + 16 * ld;
    const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p0));
    const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p1));
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
struct VFrag<float> {
  static __device__ __forceinline__ f32x8 read(const float* tile, int ld, int rb, int c0, int l16) {
    f32x8 r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r[j] = tile[(rb + j) * ld + c0 + l16];
      r[j + 4] = tile[(rb + 16 + j) * ld + c0 + l16];
    }
    return r;
  }
};

// S <- lambda^len S + (decayed rank-64 update) on the LDS copy of S: each of
// the first D/16 waves updates its 16 columns in registers.
template <class E, int D>
__device__ __forceinline__ void lds_state_update(float* Sl, const E* Kb, int ldk, const E* Vb, int ldv,
                                                 const float* pw, int len, int e0, int wid, int l16, int lg) {
  constexpr int NT = D / 16, LDS = F128<E, D>::LDS;
  if (wid < NT) {
    State<E, D> st;
    float* col = Sl + (16 * wid + l16) * LDS + 4 * lg;
#pragma unroll
    for (int at = 0; at < NT; ++at) st.s[0][at] = *(const f32x4*)(col + 16 * at);
    state_update(st, Kb, ldk, Vb, ldv, pw, len, e0, wid, l16, lg);
#pragma unroll
    for (int at = 0; at < NT; ++at) *(f32x4*)(col + 16 * at) = st.s[0][at];
  }
}

template <class E, int D>
__global__ void __launch_bounds__(256, (sizeof(E) == 2 ? 2 : 1)) fwd128_kernel(FwdArgs a) {
  using M = Mfma<E>;
  using frag = typename M::frag;
  using L = F128<E, D>;
  constexpr int NT = L::NT, NKC = L::NKC, LDK = L::LDK, LDV = L::LDV;
  static_assert(D <= 64, "one state column tile per wave");
  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  __shared__ float pw[132];
  E* Qs = (E*)(smem + 2 * L::BUF);
  float* Sl = (float*)(smem + 2 * L::BUF + L::QB);
  constexpr int LDS = L::LDS;

  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = wg / a.nseg, seg = wg - bh * a.nseg;
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
  if (tid <= 128) pw[tid] = powi(a.lam[h], tid);

  // S(e0) of the segment's first block -> LDS (transposed)
  if (seg == 0) {
    for (int x = tid; x < D * D; x += 256) Sl[(x % D) * LDS + x / D] = 0.0f;
  } else if (a.prefix_direct) {
    // S at the segment start from the local states L_m (stored at index m+1):
    // S = sum_{m < seg} lambda^((seg-1-m) 128 G) L_m, in chain order
    constexpr int PER = D * D / 256;
    const float dec = powi(a.lam[h], 128 * a.G);
    const float* g = a.seg_state + (size_t)bh * a.nseg * D * D;
    float acc[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] = 0.0f;
#pragma unroll 4
    for (int m = 1; m <= seg; ++m) {
#pragma unroll
      for (int k = 0; k < PER; ++k) acc[k] = dec * acc[k] + g[(size_t)m * D * D + tid + 256 * k];
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int x = tid + 256 * k;
      Sl[(x % D) * LDS + x / D] = acc[k];
    }
  } else {
    const float* g = a.seg_state + ((size_t)bh * a.nseg + seg) * D * D;
    for (int x = tid; x < D * D; x += 256) Sl[(x % D) * LDS + x / D] = g[x];
  }

  const int jb = seg * a.G;
  const int je = min(a.nblk, jb + a.G);

  // Item stream.  Block j contributes, in order: its Q block (item 0, two
  // 64-row halves written to the Q area), its window's key tiles (items
  // 1..nb) and, when it evicts, the two tiles of its evicted chunk.
  struct Blk {
    int t0, lo, nb, nit;
  };
  auto blk = [&](int j) {
    Blk b;
    b.t0 = j * 128;
    b.lo = max(0, b.t0 - W + 1) >> 6;
    const int hi = min(T - 1, b.t0 + 127) >> 6;
    b.nb = hi - b.lo + 1;
    b.nit = 1 + b.nb + ((b.t0 + 127 >= W) ? 2 : 0);
    return b;
  };
  // cursor of the item held in the staging registers
  int pj = jb, pidx = 0;
  Blk pb = blk(jb);
  int kv_stored = 0;  // key/value items written to LDS so far (buffer parity)
  TileRegs<E, D, 64> kr, vr;
  auto load_next = [&]() {
    const bool q = pidx == 0;
    int r0 = q ? pb.t0 : (pidx <= pb.nb ? (pb.lo + pidx - 1) * 64 : pb.t0 - W + 64 * (pidx - 1 - pb.nb));
    if (pj >= je) r0 = T + 64;  // past the end: reads zeros
    kr.load(q ? Qg : Kg, r0);
    vr.load(q ? Qg : Vg, q ? r0 + 64 : r0);
  };
  auto store_next = [&]() {
    if (pidx == 0) {
      kr.store(Qs, LDK);
      vr.store(Qs + 64 * LDK, LDK);
    } else {
      E* bp = (E*)(smem + (kv_stored & 1) * L::BUF);
      kr.store(bp, LDK);
      vr.store((E*)((char*)bp + L::KT), LDV);
      ++kv_stored;
    }
  };
  auto advance = [&]() {
    if (++pidx >= pb.nit) {
      ++pj;
      pidx = 0;
      pb = blk(pj);
    }
  };
  // publish the staged item, stage the next one, barrier
  auto step = [&]() {
    if (pj < je) store_next();
    advance();
    load_next();
    __syncthreads();
  };

  load_next();
  step();

  int kv_used = 0;  // key/value items consumed (buffer parity)
  const int rw = 32 * wid;  // first row of this wave within the block
  for (int j = jb; j < je; ++j) {
    const Blk cb = blk(j);
    const int t0 = cb.t0, e0 = t0 - W;
    const int nb = cb.nb, nkv = cb.nit - 1;
    const bool has_mem = nkv > nb;
    const bool last = (j == a.nblk - 1);
    const bool more = j + 1 < je;
    const int R0 = t0 + rw;  // first query row of this wave

    // item 0: the Q block
    frag qf[2][NKC];
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int dc = 0; dc < NKC; ++dc)
        qf[g][dc] = (dc * 32 + lg * 8 < D) ? M::lds8(Qs + (rw + 16 * g + l16) * LDK + dc * 32 + lg * 8) : M::zero();
    step();

    f32x4 O[2][NT];
    float mrow[2], lrow[2];
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      mrow[g] = kNegInf;
      lrow[g] = 0.0f;
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) O[g][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    for (int it = 0; it < nkv; ++it) {
      const E* Kb = (const E*)(smem + (kv_used & 1) * L::BUF);
      const E* Vb = (const E*)(smem + (kv_used & 1) * L::BUF + L::KT);

      // scores Z[g][n][i] = <q_row, k_key>, row = R0 + 16 g + l16,
      // key = tile row 16 n + 4 lg + i
      auto scores = [&](f32x4 (&Z)[2][4]) {
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          Z[0][n] = f32x4{0.f, 0.f, 0.f, 0.f};
          Z[1][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int dc = 0; dc < NKC; ++dc) {
            const frag ka =
                (dc * 32 + lg * 8 < D) ? M::lds8(Kb + (16 * n + l16) * LDK + dc * 32 + lg * 8) : M::zero();
            Z[0][n] = M::mma(ka, qf[0][dc], Z[0][n]);
            Z[1][n] = M::mma(ka, qf[1][dc], Z[1][n]);
          }
        }
      };
      // O[g] += P[g] V with P[g][8 p + 4 (n & 1) + i] the weight of key 16 n + 4 lg + i
      auto accum_pv = [&](const float (&P)[2][16]) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          float x0[8], x1[8];
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            x0[jj] = P[0][8 * p + jj];
            x1[jj] = P[1][8 * p + jj];
          }
          const frag p0 = M::pack(x0), p1 = M::pack(x1);
#pragma unroll
          for (int dt = 0; dt < NT; ++dt) {
            const frag vf = VFrag<E>::read(Vb, LDV, 32 * p + 4 * lg, dt * 16, l16);
            O[0][dt] = M::mma(vf, p0, O[0][dt]);
            O[1][dt] = M::mma(vf, p1, O[1][dt]);
          }
        }
      };

      if (it < nb) {
        // ---- window tile: keys k0 .. k0+63 ----
        const int k0 = (cb.lo + it) * 64;
        const bool skip = (k0 > R0 + 31) || (k0 + 63 <= R0 - W);
        const bool full = (k0 + 63 <= R0) && (k0 >= R0 + 32 - W);
        auto tile = [&](auto full_c) {
          constexpr bool FULL = decltype(full_c)::value;
          f32x4 Z[2][4];
          scores(Z);
          float P[2][16];
          float mz[2];
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const int trow = R0 + 16 * g + l16;
            float m = kNegInf;
#pragma unroll
            for (int n = 0; n < 4; ++n)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                float z = Z[g][n][i];
                if (!FULL) {
                  const int key = k0 + 16 * n + 4 * lg + i;
                  if (!(key <= trow && key > trow - W)) z = kNegInf;
                }
                P[g][8 * (n >> 1) + 4 * (n & 1) + i] = z;
                m = fmaxf(m, z);
              }
            mz[g] = xmax4(m) * sl2;
          }
          // move the reference max only when some row grew by more than 2^8
          const bool grow = (mz[0] > mrow[0] + 8.0f) || (mz[1] > mrow[1] + 8.0f);
          if (__builtin_amdgcn_ballot_w64(grow)) {
#pragma unroll
            for (int g = 0; g < 2; ++g) {
              const float mnew = fmaxf(mrow[g], mz[g]);
              const float alpha = fast_exp2(mrow[g] - (mnew == kNegInf ? 0.0f : mnew));
              lrow[g] *= alpha;
#pragma unroll
              for (int dt = 0; dt < NT; ++dt) O[g][dt] *= alpha;
              mrow[g] = mnew;
            }
          }
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const float ms = (mrow[g] == kNegInf) ? 0.0f : mrow[g];
            float ps = 0.0f;
#pragma unroll
            for (int x = 0; x < 16; ++x) {
              P[g][x] = fast_exp2(__builtin_fmaf(P[g][x], sl2, -ms));
              ps += P[g][x];
            }
            lrow[g] += ps;
          }
          accum_pv(P);
        };
        if (!skip) {
          if (full)
            tile(std::true_type{});
          else
            tile(std::false_type{});
        }
        if (it == nb - 1) {
          // softmax done: normalise, then add the read of S(e0)
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const float l = xsum4(lrow[g]);
            const float inv = 1.0f / l;
#pragma unroll
            for (int dt = 0; dt < NT; ++dt) O[g][dt] *= inv;
            const int trow = R0 + 16 * g + l16;
            if (a.lse && lg == 0 && trow < T) a.lse[(size_t)bh * T + trow] = (mrow[g] + __log2f(l)) * kLn2;
          }
          if (has_mem && e0 > 0) {
            // O += sigma(g) eta lambda^(r+1) q S(e0), S^T read from LDS as hi/lo bf16
#pragma unroll
            for (int dt = 0; dt < NT; ++dt) {
              f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
              for (int dc = 0; dc < NKC; ++dc) {
                const bool in = dc * 32 + lg * 8 < D;  // D = 16: upper half of the contraction is empty
                float sv[8];
                {
                  const float* p = Sl + (dt * 16 + l16) * LDS + dc * 32 + lg * 8;
                  const f32x4 x0 = in ? *(const f32x4*)p : f32x4{0.f, 0.f, 0.f, 0.f};
                  const f32x4 x1 = in ? *(const f32x4*)(p + 4) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                  for (int i = 0; i < 4; ++i) {
                    sv[i] = x0[i];
                    sv[4 + i] = x1[i];
                  }
                }
                frag shi, slo;
                M::split(sv, shi, slo);
                acc[0] = M::mma(shi, qf[0][dc], acc[0]);
                acc[1] = M::mma(shi, qf[1][dc], acc[1]);
                if (M::kSplit) {
                  acc[0] = M::mma(slo, qf[0][dc], acc[0]);
                  acc[1] = M::mma(slo, qf[1][dc], acc[1]);
                }
              }
#pragma unroll
              for (int g = 0; g < 2; ++g) O[g][dt] += (seta * pw[rw + 16 * g + l16 + 1]) * acc[g];
            }
          }
        }
      } else {
        // ---- tile c of the evicted chunk: keys e0 + 64 c .. +63 ----
        const int c = it - nb;
        const int ck0 = e0 + 64 * c;
        if (64 * c <= rw + 31) {
          f32x4 Z[2][4];
          scores(Z);
          float P[2][16];
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const int r = rw + 16 * g + l16;  // row within the block
#pragma unroll
            for (int n = 0; n < 4; ++n)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int ci = 64 * c + 16 * n + 4 * lg + i;  // index within the chunk
                const float w = (ci <= r && e0 + ci >= 0) ? seta * pw[r - ci] : 0.0f;
                P[g][8 * (n >> 1) + 4 * (n & 1) + i] = w * Z[g][n][i];
              }
          }
          accum_pv(P);
        }
        if (more || (last && a.A_final)) {
          const int len = more ? 64 : min(64, T - t0 - 64 * c);
          if (len > 0) lds_state_update<E, D>(Sl, Kb, LDK, Vb, LDV, pw, len, ck0, wid, l16, lg);
        }
      }

      ++kv_used;
      step();
    }

    // ---- store y ----
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int trow = R0 + 16 * g + l16;
      if (trow < T) {
#pragma unroll
        for (int dt = 0; dt < NT; ++dt) store4(Yg + (size_t)trow * D + dt * 16 + lg * 4, O[g][dt]);
      }
    }
    if (last && a.A_final) {
      float* Af = a.A_final + (size_t)bh * D * D;
      // the last item's barrier has published the final state
      const float eta = a.eta[h];
      for (int x = tid; x < D * D; x += 256) Af[x] = has_mem ? eta * Sl[(x % D) * LDS + x / D] : 0.0f;
    }
  }
}

// Segments up to which the fused kernel sums the local states itself (each
// workgroup reads at most this many D x D states, L2-resident) instead of a
// separate chain kernel.
constexpr int kDirectPrefixMaxSeg = 16;

template <class E, int D>
static hipError_t launch_fwd128_impl(const FwdArgs& a0, hipStream_t s) {
  FwdArgs a = a0;
  const int BH = a.B * a.H;
  a.prefix_direct = a.nseg <= kDirectPrefixMaxSeg ? 1 : 0;
  if (a.nseg > 1) {
    hipLaunchKernelGGL((seg_state_kernel<E, D, 128>), dim3(BH * (a.nseg - 1)), dim3(256), 0, s, a);
    if (!a.prefix_direct)
      hipLaunchKernelGGL((seg_chain_kernel<D, 128>), dim3((D * D / 4 + 255) / 256, BH), dim3(256), 0, s, a);
  }
  hipLaunchKernelGGL((fwd128_kernel<E, D>), dim3(BH * a.nseg), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_forward128(const FwdArgs& a, int D, bool is_bf16, hipStream_t s) {
  if (!is_bf16) return hipErrorInvalidValue;
  switch (D) {
    case 16: return launch_fwd128_impl<bf16, 16>(a, s);
    case 32: return launch_fwd128_impl<bf16, 32>(a, s);
    case 64: return launch_fwd128_impl<bf16, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tck

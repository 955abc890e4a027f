// Pieces shared by the forward kernels: the eviction state S held in
// matrix-core accumulators, its decayed rank-64 update, and small LDS and
// store helpers.
//
// Method ("Tensor Cache: Eviction-conditioned Associative Memory for
// Transformers", Section 3.2): A_t = lambda A_{t-1} + eta k_{t-W} v_{t-W}^T;
// the kernels carry S = A / eta so eta is applied once at the read.
#pragma once

#include "tc_device.h"
#include "tc_launch.h"

namespace tck {

// Keys (or values) of head bh: this call's rows from `cur` ([B,H,T-row0,D]),
// the re-read window of a continuation from the ring ([B,H,W,D]).
template <class E, int D>
__device__ __forceinline__ SeqRows seq_rows(const FwdArgs& a, const void* cur, const void* ring, int bh) {
  const int tn = a.T - a.row0;
  SeqRows r;
  r.cur = make_rsrc((const E*)cur + (size_t)bh * tn * D, (uint32_t)tn * D * sizeof(E));
  r.ring = a.row0 > 0 ? make_rsrc((const E*)ring + (size_t)bh * a.W * D, (uint32_t)a.W * D * sizeof(E)) : r.cur;
  r.p = a.row0;
  r.s0 = a.ring_s0;
  r.W = a.W;
  return r;
}
// Queries of head bh: row t of the sequence is row t - row0 of q (rows
// below row0 read as zeros).
template <class E, int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t query_rows(const FwdArgs& a, int bh) {
  const int tn = a.T - a.row0;
  return make_rsrc((const E*)a.q + (size_t)bh * tn * D, (uint32_t)tn * D * sizeof(E));
}

// S[o][at] holds rows a = 16*at + 4*lg + i, column c = 16*(wid + 4*o) + l16.
template <class E, int D>
struct State {
  static constexpr int NT = D / 16;
  static constexpr int NOWN = (NT + 3) / 4;
  f32x4 s[NOWN][NT];
};

// S <- lambda^len S + sum_{c<len, e0+c>=0} lambda^(len-1-c) K[c,:]^T V[c,:]
// for a 64-row chunk whose K and V are row-major in LDS (row strides ldk,
// ldv); pw[n] = lambda^n for n <= 64.
template <class E, int D>
__device__ __forceinline__ void state_update(State<E, D>& st, const E* Ks, int ldk, const E* Vs, int ldv,
                                             const float* pw, int len, int e0, int wid, int l16, int lg) {
  using M = Mfma<E>;
  using frag = typename M::frag;
  constexpr int NT = D / 16, NOWN = State<E, D>::NOWN;
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
          M::to_f32(ColFrag<E>::read(Vs + (kc * 32 + lg * 8) * ldv + ct * 16, ldv, l16), vv);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int c = kc * 32 + lg * 8 + j;
            // (branch-free: the LDS read is unconditional, at a clamped index)
        const float w = ((c < len && e0 + c >= 0) ? 1.0f : 0.0f) * pw[max(len - 1 - c, 0)];
            wv[j] = w * vv[j];
          }
        }
        frag bhi, blo;
        M::split(wv, bhi, blo);
#pragma unroll
        for (int at = 0; at < NT; ++at) {
          const frag a = ColFrag<E>::read(Ks + (kc * 32 + lg * 8) * ldk + at * 16, ldk, l16);
          st.s[o][at] = M::mma(a, bhi, st.s[o][at]);
          if (M::kSplit) st.s[o][at] = M::mma(a, blo, st.s[o][at]);
        }
      }
    }
  }
}

// state_update with the masks folded into the weight table: pwz[n] =
// lambda^n for 0 <= n <= 64 and 0 for -64 <= n < 0, so column c < 64 of the
// chunk gets weight pwz[len - 1 - c] (0 past len).  Rows of the chunk before
// token 0 need no mask: their K and V rows were loaded as zeros (buffer loads
// outside the sequence).
template <class E, int D>
__device__ __forceinline__ void state_update_z(State<E, D>& st, const E* Ks, int ldk, const E* Vs, int ldv,
                                               const float* pwz, int len, int wid, int l16, int lg) {
  using M = Mfma<E>;
  using frag = typename M::frag;
  constexpr int NT = D / 16, NOWN = State<E, D>::NOWN;
  const float decay = pwz[len];
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
          M::to_f32(ColFrag<E>::read(Vs + (kc * 32 + lg * 8) * ldv + ct * 16, ldv, l16), vv);
          const float* wp = pwz + (len - 1 - kc * 32 - lg * 8 - 7);  // weight of column c at wp[7 - (c % 8)]
#pragma unroll
          for (int j = 0; j < 8; ++j) wv[j] = wp[7 - j] * vv[j];
        }
        frag bhi, blo;
        M::split(wv, bhi, blo);
#pragma unroll
        for (int at = 0; at < NT; ++at) {
          const frag a = ColFrag<E>::read(Ks + (kc * 32 + lg * 8) * ldk + at * 16, ldk, l16);
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
__device__ __forceinline__ void state_scale(State<E, D>& st, float x) {
#pragma unroll
  for (int o = 0; o < State<E, D>::NOWN; ++o)
#pragma unroll
    for (int at = 0; at < D / 16; ++at) st.s[o][at] *= x;
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

// ---------------------------------------------------------------------------
// States exchanged between workgroups of one launch.  Buffer stores and loads
// with the sc1 cache policy are coherent across the whole device (they do not
// stop in a compute unit's or an XCD's cache), the same policy the compiler
// gives agent-scope atomics; a state is laid out in the accumulator order of
// State (256 contiguous bytes per wave and tile).
constexpr int kCoherentPolicy = 16;  // buffer cache-policy bits: sc1
// Default bound on the polls of one flag (a tenth of a second or more,
// against waits of microseconds): it guarantees that every wave ends.
constexpr int kPublishPolls = 1 << 16;

template <class E, int D>
__device__ __forceinline__ void state_publish(const State<E, D>& st, float* g, int wid, int lane) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  constexpr int NT = D / 16;
  const auto rs = make_rsrc(g, D * D * 4);
#pragma unroll
  for (int o = 0; o < State<E, D>::NOWN; ++o) {
    const int ct = wid + 4 * o;
    if (ct < NT) {
#pragma unroll
      for (int at = 0; at < NT; ++at)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i, st.s[o][at]), rs,
                                               (uint32_t)(((ct * NT + at) * 64 + lane) * 16), 0, kCoherentPolicy);
    }
  }
}

// acc = sum_{m0 <= m < m1} dec^(m1-1-m) (the state published at g + m D^2),
// the loads of up to four states in flight at once
template <class E, int D>
__device__ __forceinline__ void state_gather_all(State<E, D>& acc, float dec, const float* g, int m0, int m1,
                                                 int wid, int lane) {
  constexpr int NT = D / 16, NOWN = State<E, D>::NOWN;
  const auto rs = make_rsrc(g, (uint32_t)m1 * D * D * 4);
  for (int mb = m0; mb < m1; mb += 4) {
    f32x4 x[4][NOWN][NT];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int o = 0; o < NOWN; ++o)
#pragma unroll
        for (int at = 0; at < NT; ++at) {
          const int ct = wid + 4 * o;
          // (states past m1 and tiles past NT read zeros: offset outside the buffer)
          const uint32_t off = (mb + u < m1 && ct < NT)
                                   ? (uint32_t)((mb + u) * D * D * 4 + ((ct * NT + at) * 64 + lane) * 16)
                                   : 0x80000000u;
          x[u][o][at] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kCoherentPolicy));
        }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (mb + u < m1)
#pragma unroll
        for (int o = 0; o < NOWN; ++o)
#pragma unroll
          for (int at = 0; at < NT; ++at) acc.s[o][at] = dec * acc.s[o][at] + x[u][o][at];
  }
}

template <class E, int D>
__device__ __forceinline__ void state_fill(State<E, D>& st, float x) {
#pragma unroll
  for (int o = 0; o < State<E, D>::NOWN; ++o)
#pragma unroll
    for (int at = 0; at < D / 16; ++at) st.s[o][at] = f32x4{x, x, x, x};
}

// st <- dec * st + km vm^T (km, vm: D floats each, e.g. in LDS): one write
// of the chunk-mean shortcut in the accumulator layout of State.
template <class E, int D>
__device__ __forceinline__ void state_rank1(State<E, D>& st, float dec, const float* km, const float* vm, int wid,
                                            int l16, int lg) {
  constexpr int NT = D / 16;
#pragma unroll
  for (int o = 0; o < State<E, D>::NOWN; ++o) {
    const int ct = wid + 4 * o;
    if (ct < NT) {
      const float vc = vm[16 * ct + l16];
#pragma unroll
      for (int at = 0; at < NT; ++at)
#pragma unroll
        for (int i = 0; i < 4; ++i) st.s[o][at][i] = dec * st.s[o][at][i] + km[16 * at + 4 * lg + i] * vc;
    }
  }
}

// Sum of rows 0..63 of column c of a row-major LDS tile (row stride ld).
template <class E>
__device__ __forceinline__ float tile_col_sum(const E* tile, int ld, int c) {
  float s = 0.0f;
#pragma unroll 8
  for (int r = 0; r < 64; ++r) s += (float)tile[r * ld + c];
  return s;
}

// st <- mult * st + (the state whose transpose is at Sl, S[a][c] at Sl[c * LDS + a])
template <class E, int D, int LDS>
__device__ __forceinline__ void state_scale_add_lds_t(State<E, D>& st, float mult, const float* Sl, int wid, int l16,
                                                      int lg) {
  constexpr int NT = D / 16;
#pragma unroll
  for (int o = 0; o < State<E, D>::NOWN; ++o) {
    const int ct = wid + 4 * o;
    if (ct < NT) {
#pragma unroll
      for (int at = 0; at < NT; ++at)
        st.s[o][at] = mult * st.s[o][at] + *(const f32x4*)(Sl + (16 * ct + l16) * LDS + 16 * at + 4 * lg);
    }
  }
}

// S <- lambda^len S + sum_{c<len, e0+c>=0} lambda^(len-1-c) K[c,:]^T V[c,:] on
// an LDS copy of S (float S^T: S[a][c] at Sl[c * LDSS + a]) for a 64-row
// chunk whose K and V are row-major in LDS; NWAVES waves, wave w updating the
// column tiles w, w + NWAVES, ... (no state registers outside the update).
template <class E, int D, int LDSS, int NWAVES = 4>
__device__ __forceinline__ void lds_state_update_cols(float* Sl, const E* Ks, int ldk, const E* Vs, int ldv,
                                                      const float* pw, int len, int e0, int wid, int l16, int lg) {
  using M = Mfma<E>;
  using frag = typename M::frag;
  constexpr int NT = D / 16;
  const float decay = pw[len];
  for (int ct = wid; ct < NT; ct += NWAVES) {
    f32x4 sc[NT];
    float* col = Sl + (16 * ct + l16) * LDSS + 4 * lg;
#pragma unroll
    for (int at = 0; at < NT; ++at) sc[at] = decay * *(const f32x4*)(col + 16 * at);
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      float wv[8];
      {
        float vv[8];
        M::to_f32(ColFrag<E>::read(Vs + (kc * 32 + lg * 8) * ldv + ct * 16, ldv, l16), vv);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int c = kc * 32 + lg * 8 + j;
          // (branch-free: the LDS read is unconditional, at a clamped index)
          const float w = ((c < len && e0 + c >= 0) ? 1.0f : 0.0f) * pw[max(len - 1 - c, 0)];
          wv[j] = w * vv[j];
        }
      }
      frag bhi, blo;
      M::split(wv, bhi, blo);
#pragma unroll
      for (int at = 0; at < NT; ++at) {
        const frag af = ColFrag<E>::read(Ks + (kc * 32 + lg * 8) * ldk + at * 16, ldk, l16);
        sc[at] = M::mma(af, bhi, sc[at]);
        if (M::kSplit) sc[at] = M::mma(af, blo, sc[at]);
      }
    }
#pragma unroll
    for (int at = 0; at < NT; ++at) *(f32x4*)(col + 16 * at) = sc[at];
  }
}

// S^T into LDS: S[a][c] at Sl[c * LDS + a]
template <class E, int D, int LDS>
__device__ __forceinline__ void state_to_lds_t(const State<E, D>& st, float* Sl, int wid, int l16, int lg) {
  constexpr int NT = D / 16;
#pragma unroll
  for (int o = 0; o < State<E, D>::NOWN; ++o) {
    const int ct = wid + 4 * o;
    if (ct < NT) {
#pragma unroll
      for (int at = 0; at < NT; ++at) *(f32x4*)(Sl + (16 * ct + l16) * LDS + 16 * at + 4 * lg) = st.s[o][at];
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
// Segment states for a forward pass with BM query rows per block and G or
// G + 1 blocks per segment (segment m holds blocks b_m .. b_{m+1} - 1, b_m =
// seg_first_block, so its evictions are e in [b_m BM - W, b_{m+1} BM - W)).

// Local states L_m = S over the evictions of segment m, from zero.
// grid = BH * (nseg - 1); writes seg_state[bh][m + 1].  With final_slot the
// grid is BH * nseg and workgroup m = nseg - 1 of each head forms instead the
// local state of the last segment's evictions up to step T-1 (for the final
// state), at seg_state[BH * nseg + bh].  With nparts = P > 1 the grid is
// BH * (nseg - 1) * P: workgroup (m, p) forms the local state of tiles
// [p nt / P, (p + 1) nt / P) of the segment's nt tiles, decayed to the end
// of its own range, at parts[bh][m + 1][p] (the chain combines the parts).
//
// MEANC > 0: the chunk-mean shortcut with chunks of MEANC (64 or 128)
// evictions: L_m = sum over the segment's chunks n of lambda^(later chunks)
// kbar_n vbar_n^T, one decay per chunk; in the last segment (final_slot)
// only the chunks complete by step T-1.  Segment starts are multiples of
// MEANC evictions (the launcher requires W to be one), so chunks never
// straddle segments.
//
// RING: a continuation (row0 > 0) whose first row0 keys and values are read
// from the ring.
template <class E, int D, int BM, int MEANC = 0, int RING = 0>
__global__ void __launch_bounds__(256, 2) seg_state_kernel(FwdArgs a) {
  constexpr int LDK = D + 16 / (int)sizeof(E);
  constexpr int TILE = 64 * LDK * (int)sizeof(E);
  __shared__ __attribute__((aligned(16))) char smem[2 * TILE];
  __shared__ float pwt[64 + 72];  // pw[n] = lambda^n for 0 <= n <= 64, 0 for -64 <= n < 0
  __shared__ float cm[MEANC > 0 ? 2 * D : 1];  // means of the chunk just completed (keys, then values)
  float* const pw = pwt + 64;
  E* Ks = (E*)smem;
  E* Vs = (E*)(smem + TILE);
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int nm = a.nseg - 1 + a.final_slot;
  const int P = a.nparts > 1 ? a.nparts : 1;  // (parts: never with MEANC or a final slot)
  const int bh = blockIdx.x / (nm * P), rem = blockIdx.x - bh * nm * P;
  const int m = rem / P, part = rem - m * P;
  const bool fin = m == a.nseg - 1;  // the last segment's evictions (final_slot only)
  const int h = bh % a.H;
  const SeqRows Kg = seq_rows<E, D>(a, a.k, a.k_ring, bh);
  const SeqRows Vg = seq_rows<E, D>(a, a.v, a.v_ring, bh);
  if (tid < 64 + 65) pwt[tid] = tid >= 64 ? powi(a.lam[h], tid - 64) : 0.0f;
  State<E, D> st;
  state_zero(st);
  KVRegs<RING, E, D, 64> kl, vl;
  const int tb = seg_first_block(a, m) * BM;  // first row of segment m
  const int nts = seg_blocks(a, m) * (BM / 64);  // tiles of the segment; this part: [part nts / P, ntile)
  const int ntile = (part + 1) * nts / P;
  const int ebase = tb - a.W;
  // evictions in tile t: 64, or in the last segment those of rows up to T-1
  auto tile_len = [&](int t) { return fin ? min(64, a.T - tb - 64 * t) : 64; };
  int t0 = part * nts / P;
  while (t0 < ntile && ebase + 64 * t0 + 63 < 0) ++t0;  // tiles wholly before the first token
  load_seq<RING>(kl, Kg, ebase + 64 * t0);
  load_seq<RING>(vl, Vg, ebase + 64 * t0);
  float run = 0.0f;  // MEANC: column sum of the running chunk (thread c < D: keys, D <= c < 2D: values)
  for (int t = t0; t < ntile; ++t) {
    const int e0 = ebase + 64 * t;
    __syncthreads();
    kl.store(Ks, LDK);
    vl.store(Vs, LDK);
    __syncthreads();
    if (t + 1 < ntile) {
      load_seq<RING>(kl, Kg, e0 + 64);
      load_seq<RING>(vl, Vg, e0 + 64);
    }
    if (MEANC == 0) {
      const int len = tile_len(t);
      if (len > 0) state_update_z(st, Ks, LDK, Vs, LDK, pw, len, wid, l16, lg);
    } else {
      // (rows past the end of the sequence were loaded as zeros; an incomplete
      // chunk is never written)
      if (tid < 2 * D) run += tid < D ? tile_col_sum(Ks, LDK, tid) : tile_col_sum(Vs, LDK, tid - D);
      if ((t + 1) % (MEANC / 64 > 0 ? MEANC / 64 : 1) == 0) {
        if (tid < 2 * D) {
          cm[tid] = run * (1.0f / (MEANC > 0 ? MEANC : 1));
          run = 0.0f;
        }
        __syncthreads();
        const bool complete = !fin || tb + 64 * (t + 1) <= a.T;
        if (complete) state_rank1(st, a.lam[h], cm, cm + D, wid, l16, lg);
      }
    }
  }
  float* dst = fin ? a.seg_state + ((size_t)a.B * a.H * a.nseg + bh) * D * D
            : P > 1 ? a.parts + (((size_t)bh * a.nseg + m + 1) * P + part) * D * D
                    : a.seg_state + ((size_t)bh * a.nseg + m + 1) * D * D;
  state_store(st, dst, 1.0f, wid, l16, lg);
}

// Chain over segments, in place: seg_state[0] = S(0) (zero, or A_in / eta) and
// seg_state[m+1] = lambda^(blk_pow blocks(m)) seg_state[m] + L_m (blk_pow:
// decays per block, BM for the exact scan, BM / C for the chunk-mean shortcut).
// grid = (D*D / kChainThreads) x BH of one wave each: one thread per state
// element, so that a head's D*D chains run on D*D/64 waves spread over the
// compute units, and each thread issues the loads of 64 segments at once
// before walking its dependent chain through them (the walk is bound by how
// many loads are in flight, not by arithmetic).
constexpr int kChainThreads = 64;  // workgroup size of seg_chain_kernel (its launches use it too)
constexpr int kMaxStateParts = 4;  // most parts of one segment's state pass
template <int D, int BM>
__global__ void __launch_bounds__(kChainThreads) seg_chain_kernel(FwdArgs a) {
  const int bh = blockIdx.y;
  const int x = blockIdx.x * kChainThreads + threadIdx.x;
  if (x >= D * D) return;
  // S_m = lambda^(blk_pow blocks(m-1)) S_{m-1} + L_{m-1}
  const float decay = powi(a.lam[bh % a.H], a.blk_pow * a.G), decay1 = decay * powi(a.lam[bh % a.H], a.blk_pow);
  float* p = a.seg_state + (size_t)bh * a.nseg * D * D + x;
  const size_t stride = (size_t)D * D;
  float s = a.A_in ? a.A_in[(size_t)bh * D * D + x] / a.eta[bh % a.H] : 0.0f;  // S(0)
  p[0] = s;
  if (a.nparts > 1) {
    // L_m = sum_p lambda^(64 (nt - end_p)) L_{m,p}: part p of segment m ends
    // at tile end_p = (p + 1) nt / P of the segment's nt tiles (nt1 for the
    // first R segments, nt0 for the others)
    constexpr int MAXP = kMaxStateParts, AH = 16;
    const int P = a.nparts, nt0 = a.G * (BM / 64), nt1 = nt0 + BM / 64;
    const float lam = a.lam[bh % a.H];
    float w0[MAXP], w1[MAXP];
#pragma unroll
    for (int q = 0; q < MAXP; ++q) {
      w0[q] = q < P ? powi(lam, 64 * (nt0 - (q + 1) * nt0 / P)) : 0.0f;
      w1[q] = q < P ? powi(lam, 64 * (nt1 - (q + 1) * nt1 / P)) : 0.0f;
    }
    const float* lp = a.parts + (size_t)bh * a.nseg * P * D * D + x;
    for (int m0 = 1; m0 < a.nseg; m0 += AH) {
      float l[AH];
#pragma unroll
      for (int u = 0; u < AH; ++u) {
        l[u] = 0.0f;
        if (m0 + u < a.nseg) {
          const bool r1 = m0 + u - 1 < a.R;
#pragma unroll
          for (int q = 0; q < MAXP; ++q)
            if (q < P) l[u] += (r1 ? w1[q] : w0[q]) * lp[((size_t)(m0 + u) * P + q) * D * D];
        }
      }
#pragma unroll
      for (int u = 0; u < AH; ++u)
        if (m0 + u < a.nseg) {
          s = (m0 + u - 1 < a.R ? decay1 : decay) * s + l[u];
          p[(m0 + u) * stride] = s;
        }
    }
    return;
  }
  constexpr int AHEAD = 64;
  for (int m0 = 1; m0 < a.nseg; m0 += AHEAD) {
    float l[AHEAD];
#pragma unroll
    for (int u = 0; u < AHEAD; ++u)
      if (m0 + u < a.nseg) l[u] = p[(m0 + u) * stride];
#pragma unroll
    for (int u = 0; u < AHEAD; ++u)
      if (m0 + u < a.nseg) {
        s = (m0 + u - 1 < a.R ? decay1 : decay) * s + l[u];
        p[(m0 + u) * stride] = s;
      }
  }
}

}  // namespace tck

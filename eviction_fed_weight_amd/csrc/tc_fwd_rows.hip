// TC forward for head dimensions up to 64 on gfx950: blocks of BM = 32 NW
// query rows, NW waves of 32 rows each (NW = 4: 128-row blocks, two
// workgroups per compute unit).
//
// Method ("Tensor Cache: Eviction-conditioned Associative Memory for
// Transformers"): Section 3.1 Eq. (1) window softmax over the last W keys;
// Section 3.2 and Figure 2 write-on-evict A <- lambda A + eta k v^T, read
// m = q A, output y = y_local + sigmoid(g) m; abstract: the state is a
// weighted-sum scan of the evicted pairs.
//
// Scan.  S(e) = sum_{i<e} lambda^(e-1-i) k_i v_i^T and A_t = eta S(t-W+1).
// Block j holds rows t0 = BM j .. t0+BM-1 and evicts e0 = t0 - W .. e0+BM-1;
// for row t = t0 + r
//   A_t = eta [ lambda^(r+1) S(e0) + sum_{c<=r} lambda^(r-c) k_{e0+c} v_{e0+c}^T ]
// so the read is q S(e0) plus a lower-triangular decay-weighted BM x BM
// product with the evicted chunk (q (k outer v) = <q,k> v), and the state
// advances by BM/64 decayed rank-64 updates.
//
// Work of a workgroup: the blocks of one segment, each as a stream of 64-row
// items -- its Q block, the window's key tiles, then the tiles of the evicted
// chunk -- through a two-buffer LDS pipeline with one barrier per item.
// While an item is computed from one buffer, the next item (already in
// registers) is written to the other and the item after it is being loaded.
// Workgroups are renumbered so one head's segments run on one XCD (shared L2
// for the overlapping window rows) and a heavy segment shares its compute
// unit with a light one.  Every key/value tile fetched serves all BM rows of
// the block, so the window's overlap between neighbouring blocks is re-read
// (W + BM) / BM times per row instead of (W + 64) / 64.
//
// Per wave and item: scores for 32 rows x 64 keys (16 MFMAs; every K
// fragment read from LDS feeds both 16-row groups), softmax on the
// transposed score layout (a lane holds one query row, so row statistics need
// only a four-lane exchange), and P V (16 MFMAs, V fragments shared by both
// groups; 4 more give the row sums of P).  The running max is only moved
// when a row's maximum grows by more than 2^8 (probabilities stay below 256),
// which leaves most tiles without the rescale of the accumulators.
#include <stdlib.h>

#include <atomic>
#include <type_traits>

#include "tc_device.h"
#include "tc_fwd_common.h"
#include "tc_launch.h"

namespace tck {

template <class E, int D, int NW>
struct FRows {
  static constexpr int NTH = 64 * NW;   // threads
  static constexpr int BM = 32 * NW;    // query rows per block (32 per wave)
  static constexpr int NQ = BM / 128;   // Q items per block (128 rows each)
  static constexpr int VE = 16 / (int)sizeof(E);
  // Row strides (elements).  K, Q and S^T are read 16 rows x 16 bytes at a
  // time (odd number of 16-byte chunks per row: no bank conflicts); V is read
  // with transpose reads of 8 rows x 32 bytes (stride 10 chunks for D = 64).
  static constexpr int LDK = D + VE;
  static constexpr int LDV = D + 2 * VE;
  static constexpr int KT = 64 * LDK * (int)sizeof(E);
  static constexpr int VT = 64 * LDV * (int)sizeof(E);
  static constexpr int BUF = KT + VT;
  static constexpr int QB = BM * LDK * (int)sizeof(E);
  // L^T of the state-exchange path (float, S[a][c] at c * LDS + a, in the Q
  // area after the Q block is read).
  static constexpr int LDS = D + 4;
  // The state S(e0) that every wave reads for q S is kept in LDS as a bf16
  // hi/lo pair of S^T copies (S[a][c] at c * LDH + a; rows of an odd number
  // of 16-byte chunks), written once per block by the waves that own it; the
  // float32 state itself stays in those waves' registers (OwnS).
  static constexpr int LDH = D + 8;
  static constexpr int SB = 2 * D * LDH * 2;
  static constexpr int TOTAL = 2 * BUF + QB + SB;
  static constexpr int NT = D / 16;
  static constexpr int NKC = (D + 31) / 32;
};

// The float32 state S (D x D) of the 128-row kernel, split over the waves in
// MFMA accumulator tiles: wave w owns column tile ct = w % NT and the AT row
// tiles ar * AT .. ar * AT + AT - 1 (ar = w / NT; waves with ar >= RG own
// nothing).  s[k][i] holds S[a = 16 (ar AT + k) + 4 lg + i][c = 16 ct + l16].
template <int D, int NW>
struct OwnS {
  static constexpr int NT = D / 16;
  static constexpr int RG = (NW / NT < NT) ? NW / NT : NT;  // row-tile groups per column tile
  static constexpr int AT = NT / RG;                        // row tiles per wave
  f32x4 s[AT];
};

// Four consecutive elements S[a0 .. a0+3][c] into the bf16 hi/lo copies of
// S^T (hi = rne(x), lo = rne(x - hi): about 2^-17 relative).
__device__ __forceinline__ void put_hilo(bf16* Sh, bf16* Sm, int ldh, int c, int a0, f32x4 v) {
  bf16x4 hi, lo;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    hi[i] = (bf16)v[i];
    lo[i] = (bf16)(v[i] - (float)hi[i]);
  }
  *(bf16x4*)(Sh + c * ldh + a0) = hi;
  *(bf16x4*)(Sm + c * ldh + a0) = lo;
}

// The owner waves publish their part of S as the bf16 hi/lo copies.
template <int D, int NW>
__device__ __forceinline__ void own_publish(const OwnS<D, NW>& so, bf16* Sh, bf16* Sm, int ldh, int wid, int l16,
                                            int lg) {
  using O = OwnS<D, NW>;
  const int ct = wid % O::NT, ar = wid / O::NT;
  if (ar >= O::RG) return;
#pragma unroll
  for (int k = 0; k < O::AT; ++k) put_hilo(Sh, Sm, ldh, 16 * ct + l16, 16 * (ar * O::AT + k) + 4 * lg, so.s[k]);
}

// S <- lambda^len S + sum_{c<len} lambda^(len-1-c) K[c,:]^T V[c,:] in the
// owners' registers, for a 64-row chunk whose K and V are row-major in LDS.
// pw[n] = lambda^n for 0 <= n <= 128 and 0 for -128 <= n < 0 (so the
// columns past len get weight 0); chunk rows before token 0 were loaded as
// zeros and need no mask.
template <class E, int D, int NW>
__device__ __forceinline__ void own_state_update(OwnS<D, NW>& so, const E* Ks, int ldk, const E* Vs, int ldv,
                                                 const float* pw, int len, int wid, int l16, int lg) {
  using M = Mfma<E>;
  using frag = typename M::frag;
  constexpr int AT = OwnS<D, NW>::AT;
  const int ct = wid % OwnS<D, NW>::NT, ar = wid / OwnS<D, NW>::NT;
  if (ar >= OwnS<D, NW>::RG) return;
  f32x4 st[AT];
  const float decay = pw[len];
#pragma unroll
  for (int k = 0; k < AT; ++k) st[k] = decay * so.s[k];
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
    float wv[8];
    {
      float vv[8];
      M::to_f32(ColFrag<E>::read(Vs + (kc * 32 + lg * 8) * ldv + ct * 16, ldv, l16), vv);
      const float* wp = pw + (len - 1 - kc * 32 - lg * 8 - 7);  // weight of column c at wp[7 - (c % 8)]
#pragma unroll
      for (int j = 0; j < 8; ++j) wv[j] = wp[7 - j] * vv[j];
    }
    frag bhi, blo;
    M::split(wv, bhi, blo);
#pragma unroll
    for (int k = 0; k < AT; ++k) {
      const frag af = ColFrag<E>::read(Ks + (kc * 32 + lg * 8) * ldk + (ar * AT + k) * 16, ldk, l16);
      st[k] = M::mma(af, bhi, st[k]);
      if (M::kSplit) st[k] = M::mma(af, blo, st[k]);
    }
  }
#pragma unroll
  for (int k = 0; k < AT; ++k) so.s[k] = st[k];
}

// PUB: one block per segment, local states exchanged through flags (see
// FwdArgs::publish); otherwise the segment states come from the state pass.
//
// MEANC > 0 (64 or 128, with W a multiple of it; never with PUB): the
// chunk-mean shortcut instead of the exact scan.  The evictions form chunks
// of MEANC tokens; one write per chunk, S <- lambda S + kbar vbar^T; a row
// whose evicted token lies in chunk n reads S after chunks 0 .. n-1.  Block
// j evicts the chunks of e0 .. e0+127, so its row r reads
//   lambda^(r / MEANC) q S(e0) + [MEANC = 64, r >= 64] <q, kbar_0> vbar_0
// (kbar_0, vbar_0: the means of the block's first 64 evictions), and the
// carry is BM / MEANC such writes.  No intra-chunk triangle.
//
// RING: a continuation (row0 > 0) whose first row0 keys and values are read
// from the ring (1; 2 when row0 and W are multiples of 64, so that every tile
// lies wholly in the ring or wholly in the new tokens: one load per vector).
template <class E, int D, int NW, bool PUB, int MEANC = 0, int RING = 0>
__global__ void __launch_bounds__(64 * NW, NW == 4 ? 2 : 1) fwd_kernel_rows(FwdArgs a) {
  using M = Mfma<E>;
  using frag = typename M::frag;
  using L = FRows<E, D, NW>;
  constexpr int NT = L::NT, NKC = L::NKC, LDK = L::LDK, LDV = L::LDV;
  constexpr int NTH = L::NTH, BM = L::BM, NQ = L::NQ;
  constexpr bool MEAN = MEANC > 0;
  static_assert(D <= 64 && NW == 4, "128-row blocks: the two chunk tiles fit the two buffers");
  static_assert(!(MEAN && PUB), "the chunk-mean shortcut runs with the state pass");
  static_assert(MEANC == 0 || MEANC == 64 || MEANC == 128, "chunk-mean chunks of 64 or 128 evictions");
  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  // ptab: lambda^n at ptab[128 + n] for 0 <= n <= 128 and 0 for n < 0 (pw = ptab + 128); wtab[128 + d]
  // = sigma(g) eta lambda^d for 0 <= d < 128 and 0 for d < 0, the weights of the intra-chunk terms
  __shared__ float ptab[BM + 132];
  __shared__ float wtab[2 * BM];
  __shared__ float cm[MEAN ? 4 * D : 1];  // MEAN: chunk means kbar_0, vbar_0, kbar_1, vbar_1
  float* const pw = ptab + BM;
  E* Qs = (E*)(smem + 2 * L::BUF);
  bf16* Sh = (bf16*)(smem + 2 * L::BUF + L::QB);  // S^T hi and lo (bf16), row stride LDH
  bf16* Sm = Sh + D * L::LDH;
  constexpr int LDS = L::LDS, LDH = L::LDH;
  using O = OwnS<D, NW>;
  O so;  // (not PUB) the float32 state, in the owner waves' registers

  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  // PUB: segment-major order (workgroup b takes segment b / BH of head b % BH),
  // so a workgroup waits only for workgroups dispatched before it, and with
  // B*H a multiple of 8 all segments of a head run on one XCD (b % 8).
  // Otherwise: one head's segments on one XCD, heavy and light segments paired.
  const int BHn = a.B * a.H;
  const int wg = PUB ? (blockIdx.x % BHn) * a.nseg + blockIdx.x / BHn : xcd_remap_paired(blockIdx.x, gridDim.x);
  const int bh = wg / a.nseg, seg = wg - bh * a.nseg;
  const int h = bh % a.H;
  const int T = a.T, W = a.W;
  const auto Qg = query_rows<E, D>(a, bh);
  const SeqRows Kg = seq_rows<E, D>(a, a.k, a.k_ring, bh);
  const SeqRows Vg = seq_rows<E, D>(a, a.v, a.v_ring, bh);
  SeqRows Qr = Kg;  // the queries as a sequence whose rows below row0 read as zeros
  Qr.cur = Qg;
  Qr.ring = make_rsrc(a.q, 0);
  const int Tout = T - a.row0;  // stored rows
  E* Yg = (E*)a.y + (size_t)bh * Tout * D;
  const float seta = sigmoidf(a.gate[h]) * a.eta[h];
  const float sl2 = a.scale * kLog2e;
  const int jb = seg_first_block(a, seg);
  const int je = seg_first_block(a, seg + 1);

  // Item stream.  Block j contributes, in order: its Q block (NQ items of
  // 128 rows, each two 64-row halves written to the Q area), its window's key
  // tiles (nb items) and, when it evicts, the BM/64 tiles of its evicted chunk.
  // Key tiles of block j start at kb = t0 - W (not at multiples of 64): tile i
  // holds keys kb + 64 i .. kb + 64 i + 63, so tiles 0 and 1 are exactly the
  // block's evicted chunk.  A block that evicts visits its window tiles
  // 2 .. ihi first and tiles 0 and 1 last; after the last one (softmax done)
  // both chunk tiles are still in the two LDS buffers for the memory read and
  // the state update, so the chunk costs no items of its own.
  //
  // With PUB the evicting block visits its window tiles in order 0 .. ihi
  // instead (forming and publishing its local state while tiles 0 and 1 are
  // in the buffers, early enough for the stores to complete under the rest of
  // the window) and then loads the chunk tiles 0 and 1 once more as nlate
  // items of their own.
  struct Blk {
    int t0, kb, ilo, nfront, nlate, nwin, nb, nit;
    bool mem;
  };
  auto blk = [&](int j) {
    Blk b;
    b.t0 = j * BM;
    b.kb = b.t0 - W;
    const int ihi = (min(T - 1, b.t0 + BM - 1) - b.kb) >> 6;  // last tile with a key in range
    b.mem = !a.window_only && b.t0 + BM - 1 >= W;
    if (b.mem) {
      b.nlate = min(2, ihi + 1);
      b.ilo = PUB ? 0 : 2;
      b.nfront = PUB ? ihi + 1 : ihi + 1 - b.nlate;
      b.nwin = ihi + 1;
    } else {
      b.nlate = 0;
      b.ilo = (-b.kb - 63 > 0) ? ((-b.kb) >> 6) : 0;  // first tile with a key >= 0
      b.nfront = ihi - b.ilo + 1;
      b.nwin = b.nfront;
    }
    b.nb = b.nfront + b.nlate;  // key/value items; the first nwin are window tiles
    b.nit = NQ + b.nb;
    return b;
  };
  auto tile_of = [&](const Blk& b, int idx) { return idx < b.nfront ? b.ilo + idx : idx - b.nfront; };
  // cursor of the item held in the staging registers
  // (PUB: the Q block is loaded on its own at the start, so its loads and the
  // first key tile's are in flight together; the item stream starts at the tiles)
  int pj = jb, pidx = PUB ? NQ : 0;
  Blk pb = blk(jb);
  int kv_stored = 0;  // key/value items written to LDS so far (buffer parity)
  KVRegs<RING, E, D, 64, NTH> kr, vr;
  auto load_next = [&]() {
    const bool q = pidx < NQ;
    const int ki = pidx - NQ;
    int r0 = q ? pb.t0 + 128 * pidx : pb.kb + 64 * tile_of(pb, ki);
    if (pj >= je) r0 = T + 64;  // past the end: reads zeros
    if constexpr (RING) {  // (a select of the sources, no branch: see TileRegs)
      kr.load(q ? Qr : Kg, r0);
      vr.load(q ? Qr : Vg, q ? r0 + 64 : r0);
    } else {  // (row0 = 0)
      kr.load(q ? Qg : Kg.cur, r0);
      vr.load(q ? Qg : Vg.cur, q ? r0 + 64 : r0);
    }
  };
  auto store_next = [&]() {
    if (pidx < NQ) {
      kr.store(Qs + 128 * pidx * LDK, LDK);
      vr.store(Qs + (128 * pidx + 64) * LDK, LDK);
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

  TileRegs<E, D, BM, NTH> qr;
  if (PUB) qr.load(Qg, jb * BM - a.row0);
  load_next();

  for (int x = tid; x < 2 * BM + 1; x += NTH) {
    const float lp = x >= BM ? powi(a.lam[h], x - BM) : 0.0f;
    ptab[x] = lp;
    if (x < 2 * BM) wtab[x] = seta * lp;
  }

  // S(e0) of the segment's first block -> the owners' registers and the
  // hi/lo copies in LDS; with publish it is gathered after the window, from
  // the earlier segments' published states
  if (!PUB && !a.window_only && wid / O::NT < O::RG) {
    const int ct = wid % O::NT, ar = wid / O::NT, c = 16 * ct + l16;
#pragma unroll
    for (int k = 0; k < O::AT; ++k) so.s[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (a.prefix_direct && (seg > 0 || a.A_in)) {
      // S at the segment start from S(0) (zero, or A_in / eta) and the local
      // states L_m (stored at index m+1):
      // S_{m+1} = lambda^(blk_pow blocks(m)) S_m + L_m, in chain order
      if (a.A_in) {
        const float* g0 = a.A_in + (size_t)bh * D * D;
        const float ie = 1.0f / a.eta[h];
#pragma unroll
        for (int k = 0; k < O::AT; ++k)
#pragma unroll
          for (int i = 0; i < 4; ++i) so.s[k][i] = ie * g0[(16 * (ar * O::AT + k) + 4 * lg + i) * D + c];
      }
      const float dec = powi(a.lam[h], a.blk_pow * a.G), dec1 = dec * powi(a.lam[h], a.blk_pow);
      const float* g = a.seg_state + (size_t)bh * a.nseg * D * D;
#pragma unroll 2
      for (int m = 1; m <= seg; ++m) {
        const float dm = m - 1 < a.R ? dec1 : dec;
#pragma unroll
        for (int k = 0; k < O::AT; ++k)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            so.s[k][i] = dm * so.s[k][i] + g[(size_t)m * D * D + (16 * (ar * O::AT + k) + 4 * lg + i) * D + c];
      }
    } else if (!a.prefix_direct && (seg > 0 || a.A_in)) {  // (the chain ran: seg_state[0] = S(0))
      const float* g = a.seg_state + ((size_t)bh * a.nseg + seg) * D * D;
#pragma unroll
      for (int k = 0; k < O::AT; ++k)
#pragma unroll
        for (int i = 0; i < 4; ++i) so.s[k][i] = g[(16 * (ar * O::AT + k) + 4 * lg + i) * D + c];
    }
    own_publish(so, Sh, Sm, LDH, wid, l16, lg);
  }

  if (PUB) {
    qr.store(Qs, LDK);
    __syncthreads();
  } else {
    step();
  }

  int kv_used = 0;  // key/value items consumed (buffer parity)
  bool timed_out = false;  // a flag wait of this workgroup ran out (uniform in the workgroup)
  const int rw = 32 * wid;  // first row of this wave within the block
  // (PUB: exactly one block per segment, so no loop for the compiler to hoist out of)
  for (int j = jb; j < (PUB ? jb + 1 : je); ++j) {
    const Blk cb = blk(j);
    const int t0 = cb.t0, e0 = t0 - W;
    const int nb = cb.nb;
    const bool has_mem = cb.mem;
    const bool last = (j == a.nblk - 1);
    const bool more = j + 1 < je;
    const int R0 = t0 + rw;  // first query row of this wave

    // items 0 .. NQ-1: the Q block
    for (int qi = 1; qi < NQ; ++qi) step();  // (NQ = 1 with PUB)
    frag qf[2][NKC];
    frag ones;
    {
      float o8[8];
#pragma unroll
      for (int x = 0; x < 8; ++x) o8[x] = 1.0f;
      ones = M::pack(o8);
    }
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int dc = 0; dc < NKC; ++dc)
        qf[g][dc] = (dc * 32 + lg * 8 < D) ? M::lds8(Qs + (rw + 16 * g + l16) * LDK + dc * 32 + lg * 8) : M::zero();
    step();

    f32x4 O[2][NT];
    float mrow[2];
    f32x4 Lsum[2];  // row sums of P via the matrix core (element 0 is used)
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      mrow[g] = kNegInf;
      Lsum[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) O[g][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // scores Z[g][n][i] = <q_row, k_key>, row = R0 + 16 g + l16,
    // key = tile row 16 n + 4 lg + i of the K tile at Kt
    // (LV: bit p set when the tile's keys 32 p .. 32 p + 31 are computed; the
    // scores of a dead half are -inf without matrix-core work)
    auto scores = [&](f32x4 (&Z)[2][4], const E* Kt, auto lv_c) {
      constexpr int LV = decltype(lv_c)::value;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        if (!((LV >> (n >> 1)) & 1)) {
          Z[0][n] = f32x4{kNegInf, kNegInf, kNegInf, kNegInf};
          Z[1][n] = Z[0][n];
          continue;
        }
        Z[0][n] = f32x4{0.f, 0.f, 0.f, 0.f};
        Z[1][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dc = 0; dc < NKC; ++dc) {
          const frag ka =
              (dc * 32 + lg * 8 < D) ? M::lds8(Kt + (16 * n + l16) * LDK + dc * 32 + lg * 8) : M::zero();
          Z[0][n] = M::mma(ka, qf[0][dc], Z[0][n]);
          Z[1][n] = M::mma(ka, qf[1][dc], Z[1][n]);
        }
      }
    };
    // O[g] += P[g] V with P[g][8 p + 4 (n & 1) + i] the weight of key 16 n + 4 lg + i;
    // with SUM also Lsum[g] += (row sums of P), from the same packed P; V tile at Vt
    auto accum_pv = [&](const float (&P)[2][16], auto sum_c, const E* Vt, auto lv_c) {
      constexpr bool SUM = decltype(sum_c)::value;
      constexpr int LV = decltype(lv_c)::value;  // halves with nonzero P (as in scores)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        if (!((LV >> p) & 1)) continue;
        float x0[8], x1[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          x0[jj] = P[0][8 * p + jj];
          x1[jj] = P[1][8 * p + jj];
        }
        const frag p0 = M::pack(x0), p1 = M::pack(x1);
        if (SUM) {
          Lsum[0] = M::mma(ones, p0, Lsum[0]);
          Lsum[1] = M::mma(ones, p1, Lsum[1]);
        }
#pragma unroll
        for (int dt = 0; dt < NT; ++dt) {
          const frag vf = VFrag<E>::read(Vt, LDV, 32 * p + 4 * lg, dt * 16, l16);
          O[0][dt] = M::mma(vf, p0, O[0][dt]);
          O[1][dt] = M::mma(vf, p1, O[1][dt]);
        }
      }
    };

    // One block per segment (PUB): segments m >= m_lo (blocks j0 + m >= W / BM)
    // have evictions at or after token 0 (L_m != 0);
    // S(e0) = sum_{m_lo <= m < seg} lambda^((seg-1-m) BM) L_m.
    const int m_lo = W / BM - a.j0;
    const bool pub = PUB && seg >= m_lo && seg + 1 < a.nseg;
    const bool fin = PUB && last && a.A_final != nullptr && has_mem;
    float* const Lt = (float*)Qs;  // L^T of the last block (the Q area is free after qf is read)
    float* const slots = a.seg_state + (size_t)bh * a.nseg * D * D;

    for (int it = 0; it < nb; ++it) {
      const E* Kb = (const E*)(smem + (kv_used & 1) * L::BUF);
      const E* Vb = (const E*)(smem + (kv_used & 1) * L::BUF + L::KT);

      if (it < cb.nwin) {
        // ---- window tile: keys k0 .. k0+63 ----
        const int k0 = cb.kb + 64 * tile_of(cb, it);
        // (tiles of early blocks may start before token 0: those keys are masked)
        const bool skip = (k0 > R0 + 31) || (k0 + 63 <= R0 - W) || (k0 + 63 < 0);
        const bool full = (k0 + 63 <= R0) && (k0 >= R0 + 32 - W) && (k0 >= 0);
        auto tile = [&](auto full_c, auto lv_c) {
          constexpr bool FULL = decltype(full_c)::value;
          constexpr int LV = decltype(lv_c)::value;
          f32x4 Z[2][4];
          // (state-pass instances: the wave issues its score MFMAs, and below its P V
          // MFMAs, at raised priority, so the two waves of a SIMD interleave
          // matrix-core bursts with the other's softmax more evenly: -3 % on the long
          // prefill; the flag-exchange instance measured slower with it)
          if (!PUB) __builtin_amdgcn_s_setprio(1);
          scores(Z, Kb, lv_c);
          if (!PUB) __builtin_amdgcn_s_setprio(0);
          float P[2][16];
          float mz[2];
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const int trow = R0 + 16 * g + l16;
            const unsigned wr = (unsigned)min(W, trow + 1);  // window of trow: keys trow - wr + 1 .. trow, all >= 0
            float m = kNegInf;
#pragma unroll
            for (int n = 0; n < 4; ++n)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                float z = Z[g][n][i];
                if (!FULL) {
                  // key k0 + 16 n + 4 lg + i is in the window iff 0 <= trow - key < min(W, trow + 1)
                  if ((unsigned)(trow - k0 - 4 * lg - (16 * n + i)) >= wr) z = kNegInf;
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
              Lsum[g][0] *= alpha;
#pragma unroll
              for (int dt = 0; dt < NT; ++dt) O[g][dt] *= alpha;
              mrow[g] = mnew;
            }
          }
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const float ms = (mrow[g] == kNegInf) ? 0.0f : mrow[g];
#pragma unroll
            for (int x = 0; x < 16; ++x)
              P[g][x] = ((LV >> (x >> 3)) & 1) ? fast_exp2(__builtin_fmaf(P[g][x], sl2, -ms)) : 0.0f;
          }
          if (!PUB) __builtin_amdgcn_s_setprio(1);
          accum_pv(P, std::true_type{}, Vb, lv_c);
          if (!PUB) __builtin_amdgcn_s_setprio(0);
        };
        if (!skip) {
          if (full) {
            tile(std::true_type{}, std::integral_constant<int, 3>{});
          } else if constexpr (PUB) {
            // a band-edge tile may have a half that no row of this wave sees: its
            // keys all lie after the wave's last row, or before the first key of
            // the earliest window (max(0, R0 - W + 1)); it contributes zeros, so
            // its products and exponentials are skipped (the results do not
            // change).  Only in the state-exchange instance, whose workgroups run
            // one short chain each (-1.7 %); in the state-pass instances the
            // extra tile variants cost more than they save (+3.6 %, measured).
            const int lo_key = max(0, R0 - W + 1);
            if (k0 + 31 < lo_key)
              tile(std::false_type{}, std::integral_constant<int, 2>{});
            else if (k0 + 32 > R0 + 31)
              tile(std::false_type{}, std::integral_constant<int, 1>{});
            else
              tile(std::false_type{}, std::integral_constant<int, 3>{});
          } else {
            tile(std::false_type{}, std::integral_constant<int, 3>{});
          }
        }
      }
      if (PUB && has_mem && (pub || fin) && it == min(1, cb.nwin - 1)) {
        // chunk tiles 0 .. it are the window items 0 .. it, still in the two buffers:
        // L of this block's evictions (the last block: those of rows up to T-1)
        State<E, D> st;
        state_zero(st);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int len = pub ? 64 : min(64, T - t0 - 64 * c);
          if (c <= it && len > 0) {
            const int ub = kv_used - it + c;
            state_update_z(st, (const E*)(smem + (ub & 1) * L::BUF), LDK,
                           (const E*)(smem + (ub & 1) * L::BUF + L::KT), LDV, pw, len, wid, l16, lg);
          }
        }
        if (pub)
          state_publish(st, slots + (size_t)(seg + 1) * D * D, wid, lane);
        else
          state_to_lds_t<E, D, LDS>(st, Lt, wid, l16, lg);
        __syncthreads();  // tile 0 is read by every wave before the step below overwrites its buffer
      }
      ++kv_used;
      const bool flag_now = pub && it == cb.nwin - 1;
      if (flag_now) __builtin_amdgcn_s_waitcnt(0);  // this thread's published stores are complete
      step();
      if (flag_now && tid == 0)  // (after the barrier: every thread's stores are complete)
        __hip_atomic_store(a.flags + (size_t)bh * a.nseg + seg, a.gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // ---- after the window: normalise, the evicted chunk, read S(e0), the state ----
    // (the last step wrote only the Q area: both chunk tiles are still in the buffers)
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const float l = Lsum[g][0];
      const float inv = 1.0f / l;
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) O[g][dt] *= inv;
      const int trow = R0 + 16 * g + l16;
      if (a.lse && lg == 0 && trow >= a.row0 && trow < T)
        a.lse[(size_t)bh * Tout + trow - a.row0] = (mrow[g] + __log2f(l)) * kLn2;
    }
    auto chunk_tile = [&](int c, const E*& Kc, const E*& Vc) {
      const int ub = kv_used - cb.nlate + c;  // kv index of chunk tile c (tiles 0, 1 were the last nlate items)
      Kc = (const E*)(smem + (ub & 1) * L::BUF);
      Vc = (const E*)(smem + (ub & 1) * L::BUF + L::KT);
    };
    if constexpr (MEAN) {
      // means of the block's evicted chunks (both tiles are still in the
      // buffers; rows before token 0 were loaded as zeros)
      if (has_mem) {
        const E *K0, *V0, *K1, *V1;
        chunk_tile(0, K0, V0);
        chunk_tile(1, K1, V1);
        if (MEANC == 64 && tid < 4 * D) {
          const int which = tid / D, c = tid - which * D;
          const E* tl = which == 0 ? K0 : which == 1 ? V0 : which == 2 ? K1 : V1;
          cm[tid] = tile_col_sum(tl, (which & 1) ? LDV : LDK, c) * (1.0f / 64);
        } else if (MEANC == 128 && tid < 2 * D) {
          const bool isv = tid >= D;
          const int c = tid - (isv ? D : 0);
          cm[tid] = (tile_col_sum(isv ? V0 : K0, isv ? LDV : LDK, c) + tile_col_sum(isv ? V1 : K1, isv ? LDV : LDK, c)) *
                    (1.0f / 128);
        }
        __syncthreads();
      }
    }
    // PUB: the first read of the earlier segments' flags is issued here and
    // returns while the chunk terms below are computed
    const bool poller = PUB && seg > m_lo && tid < seg - m_lo;
    const unsigned long long* const myflag = a.flags + (size_t)bh * a.nseg + m_lo + tid;
    unsigned long long flag0 = 0;
    if (poller) flag0 = __hip_atomic_load(myflag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (MEAN && MEANC == 64 && has_mem && rw >= 64) {
      // rows 64..127 are in the block's second chunk: they also read the
      // write of the first one, sigma(g) eta <q_r, kbar_0> vbar_0
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        float x[8], dotp = 0.0f;
#pragma unroll
        for (int dc = 0; dc < NKC; ++dc) {
          if (dc * 32 + lg * 8 < D) {
            M::to_f32(qf[g][dc], x);
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) dotp += x[jj] * cm[dc * 32 + lg * 8 + jj];
          }
        }
        const float f = seta * xsum4(dotp);
#pragma unroll
        for (int dt = 0; dt < NT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) O[g][dt][i] += f * cm[D + dt * 16 + 4 * lg + i];
      }
    }
    if (!MEAN && has_mem) {
      // O += sigma(g) eta sum_{c <= r} lambda^(r-c) <q_r, k_{e0+c}> v_{e0+c}
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        if (c < cb.nlate && 64 * c <= rw + 31) {
          const E *Kc, *Vc;
          chunk_tile(c, Kc, Vc);
          f32x4 Z[2][4];
          scores(Z, Kc, std::integral_constant<int, 3>{});
          // weight of row r and chunk key ci: wtab[128 + r - ci] (0 for ci > r); keys
          // before token 0 were loaded as zeros (Z = 0).  One base per lane, the
          // 32 weights at immediate offsets 51 + 16 (g - n) - i from it.
          const float* wb = wtab + (BM + rw + l16 - 4 * lg - 64 * c - 51);
          float P[2][16];
#pragma unroll
          for (int g = 0; g < 2; ++g)
#pragma unroll
            for (int n = 0; n < 4; ++n)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                P[g][8 * (n >> 1) + 4 * (n & 1) + i] = wb[51 + 16 * (g - n) - i] * Z[g][n][i];
          accum_pv(P, std::false_type{}, Vc, std::integral_constant<int, 3>{});
        }
      }
    }
    if (PUB) {
      State<E, D> acc;  // S(e0)
      state_zero(acc);
      if (a.A_in) {
        // a continuation's carried memory: S(0) = A_in / eta (m_lo = 0 then),
        // decayed by the gather below with the earlier segments' states
        state_load(acc, a.A_in + (size_t)bh * D * D, wid, l16, lg);
        state_scale(acc, 1.0f / a.eta[h]);
      }
      if (seg > m_lo) {
        // wait for the earlier segments' flags (bounded, so that every wave
        // ends; the workgroups waited for were dispatched earlier and wait for
        // nothing later, so the bound is not reached; were it reached, the
        // read would be NaN instead of a stale state)
        bool seen = !poller || (a.max_polls > 0 && flag0 == a.gen);
        for (int n = 0; !seen && n < a.max_polls; ++n) {
          __builtin_amdgcn_s_sleep(1);
          seen = __hip_atomic_load(myflag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.gen;
        }
        const bool ran_out = __syncthreads_or(!seen);
        state_gather_all(acc, pw[BM], slots, m_lo + 1, seg + 1, wid, lane);
        if (ran_out) state_fill(acc, __uint_as_float(0x7fc00000u));  // quiet NaN (bit pattern: no NaN literal here)
        timed_out = ran_out;
      }
      if (seg > m_lo || a.A_in) {
#pragma unroll
        for (int o = 0; o < State<E, D>::NOWN; ++o)
          if (wid + 4 * o < NT)
#pragma unroll
            for (int at = 0; at < NT; ++at) put_hilo(Sh, Sm, LDH, 16 * (wid + 4 * o) + l16, 16 * at + 4 * lg, acc.s[o][at]);
      }
      if (last && a.A_final) {
        // A after step T-1 = eta (lambda^n S(e0) + L), n = T - t0 evictions in
        // this block (L^T was written to the Q area by this wave's own threads)
        float* Af = a.A_final + (size_t)bh * D * D;
        if (fin) {
          state_scale_add_lds_t<E, D, LDS>(acc, pw[T - t0], Lt, wid, l16, lg);
          state_store(acc, Af, a.eta[h], wid, l16, lg);
        } else {
          for (int x = tid; x < D * D; x += NTH) Af[x] = 0.0f;  // no evictions
        }
      }
      __syncthreads();  // S(e0) in LDS for every wave
    }
    if (has_mem && (e0 > 0 || a.A_in)) {
      // O += sigma(g) eta lambda^(r+1) q S(e0), S^T read from LDS as hi/lo bf16
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) {
        f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int dc = 0; dc < NKC; ++dc) {
          const bool in = dc * 32 + lg * 8 < D;  // D = 16: upper half of the contraction is empty
          const int off = (dt * 16 + l16) * LDH + dc * 32 + lg * 8;
          const frag shi = in ? M::lds8(Sh + off) : M::zero();
          const frag slo = in ? M::lds8(Sm + off) : M::zero();
          acc[0] = M::mma(shi, qf[0][dc], acc[0]);
          acc[1] = M::mma(shi, qf[1][dc], acc[1]);
          if (M::kSplit) {
            acc[0] = M::mma(slo, qf[0][dc], acc[0]);
            acc[1] = M::mma(slo, qf[1][dc], acc[1]);
          }
        }
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          // exact: lambda^(r+1); chunk mean: lambda^(r / MEANC) (rows 64.. of a 64-chunk block)
          const float dk = MEAN ? ((MEANC == 64 && rw >= 64) ? pw[1] : 1.0f) : pw[rw + 16 * g + l16 + 1];
          O[g][dt] += (seta * dk) * acc[g];
        }
      }
    }
    if (!PUB && has_mem && (more || (last && a.A_final && !a.final_slot))) {
      __syncthreads();  // every wave has read S(e0)
      if constexpr (MEAN) {
        // the block's chunk writes, S <- lambda S + kbar vbar^T each (in the
        // last block only the chunks complete by step T-1)
        constexpr int NCH = BM / (MEANC > 0 ? MEANC : 1);
        int nw = NCH;
        if (!more)
          for (nw = 0; nw < NCH && t0 + (MEANC > 0 ? MEANC : 1) * (nw + 1) <= T; ++nw) {
          }
        const float lam = pw[1];
        if (wid / O::NT < O::RG) {
          const int ct = wid % O::NT, arow = wid / O::NT, c = 16 * ct + l16;
          for (int m = 0; m < nw; ++m) {
            const float vc = cm[(2 * m + 1) * D + c];
#pragma unroll
            for (int k = 0; k < O::AT; ++k)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                so.s[k][i] = lam * so.s[k][i] + cm[2 * m * D + 16 * (arow * O::AT + k) + 4 * lg + i] * vc;
          }
        }
        own_publish(so, Sh, Sm, LDH, wid, l16, lg);
      } else {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const int len = more ? 64 : min(64, T - t0 - 64 * c);
          if (c < cb.nlate && len > 0) {
            const E *Kc, *Vc;
            chunk_tile(c, Kc, Vc);
            own_state_update<E, D, NW>(so, Kc, LDK, Vc, LDV, pw, len, wid, l16, lg);
          }
        }
        own_publish(so, Sh, Sm, LDH, wid, l16, lg);
      }
    }

    // ---- store y ----
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const int trow = R0 + 16 * g + l16;
      if (trow >= a.row0 && trow < T) {
        const size_t o = (size_t)(trow - a.row0) * D + lg * 4;
        if (a.yadd) {
#pragma unroll
          for (int dt = 0; dt < NT; ++dt) O[g][dt] += *(const f32x4*)(a.yadd + (size_t)bh * Tout * D + o + dt * 16);
        }
#pragma unroll
        for (int dt = 0; dt < NT; ++dt) store4(Yg + o + dt * 16, O[g][dt]);
      }
    }
    if (!PUB && last && a.A_final && !a.final_slot) {
      float* Af = a.A_final + (size_t)bh * D * D;
      // (from the owners' registers, after this block's updates)
      const float eta = a.eta[h];
      if (wid / O::NT < O::RG) {
        const int ct = wid % O::NT, ar = wid / O::NT, c = 16 * ct + l16;
#pragma unroll
        for (int k = 0; k < O::AT; ++k)
#pragma unroll
          for (int i = 0; i < 4; ++i) Af[(16 * (ar * O::AT + k) + 4 * lg + i) * D + c] = has_mem ? eta * so.s[k][i] : 0.0f;
      }
    }
  }
  if (a.status && tid == 0) a.status[wg] = timed_out ? ~a.gen : a.gen;
  if (!PUB && seg == 0 && a.final_slot && a.A_final) {
    // A after step T-1 = eta (lambda^n S_last + L_final): S_last the state at
    // the last segment's start, L_final that segment's evictions (n of them)
    constexpr int PER = (D * D + NTH - 1) / NTH;
    const int last_seg = a.nseg - 1;
    const float* g = a.seg_state + (size_t)bh * a.nseg * D * D;
    const float* Lf = a.seg_state + ((size_t)a.B * a.H * a.nseg + bh) * D * D;
    float acc[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) acc[k] = 0.0f;
    if (a.prefix_direct) {
      if (a.A_in) {  // S(0) = A_in / eta
        const float ie = 1.0f / a.eta[h];
#pragma unroll
        for (int k = 0; k < PER; ++k)
          if ((D * D) % NTH == 0 || tid + NTH * k < D * D) acc[k] = ie * a.A_in[(size_t)bh * D * D + tid + NTH * k];
      }
      const float dec = powi(a.lam[h], a.blk_pow * a.G), dec1 = dec * powi(a.lam[h], a.blk_pow);
      for (int m = 1; m <= last_seg; ++m) {
        const float dm = m - 1 < a.R ? dec1 : dec;
#pragma unroll
        for (int k = 0; k < PER; ++k)
          if ((D * D) % NTH == 0 || tid + NTH * k < D * D)
            acc[k] = dm * acc[k] + g[(size_t)m * D * D + tid + NTH * k];
      }
    } else {
#pragma unroll
      for (int k = 0; k < PER; ++k)
        if ((D * D) % NTH == 0 || tid + NTH * k < D * D) acc[k] = g[(size_t)last_seg * D * D + tid + NTH * k];
    }
    // decays since the last segment's start: one per eviction (exact), one
    // per complete chunk (chunk mean)
    const int nev = T - seg_first_block(a, last_seg) * BM;
    const float dn = powi(a.lam[h], MEAN ? nev / (MEANC > 0 ? MEANC : 1) : nev);
    const float eta = a.eta[h];
    float* Af = a.A_final + (size_t)bh * D * D;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int x = tid + NTH * k;
      if ((D * D) % NTH == 0 || x < D * D) Af[x] = eta * __builtin_fmaf(dn, acc[k], Lf[x]);
    }
  }
}

// Segments up to which the fused kernel sums the local states itself (each
// workgroup reads at most this many D x D states, L2-resident) instead of a
// separate chain kernel.
constexpr int kDirectPrefixMaxSeg = 16;
// Segments up to which the workgroups exchange their local states through
// flags (each gathers at most this many states after its window).
constexpr int kPublishMaxSeg = 32;
// Waves per workgroup of the bf16 kernel: 4 waves x 32 rows = 128-row blocks,
// two workgroups per compute unit.  (Eight waves and 256-row blocks halve the
// key/value tile traffic but run all eight waves in barrier lockstep at one
// workgroup per unit, which measured slower.)
constexpr int kRowWaves = 4;

// Workgroups of the rows kernel that the current device holds at once (0 if
// unknown), kept per device after the first query.
template <class E, int D, int NW>
static long long rows_resident_capacity() {
  static std::atomic<long long> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  long long c = cache[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fwd_kernel_rows<E, D, NW, true>, 64 * NW, 0) != hipSuccess)
      return 0;
    c = (long long)cus * per;
    cache[dev].store(c, std::memory_order_relaxed);
  }
  return c;
}

template <class E, int D, int MEANC>
static hipError_t launch_rows_impl(const FwdArgs& a0, hipStream_t s) {
  constexpr int NW = kRowWaves, BM = 32 * NW;
  FwdArgs a = a0;
  const int BH = a.B * a.H;
  a.nparts = 1;  // (the state pass of the rows kernel has one workgroup per segment)
  a.parts = nullptr;
  a.prefix_direct = a.nseg <= kDirectPrefixMaxSeg ? 1 : 0;
  a.blk_pow = MEANC > 0 ? BM / MEANC : BM;
  // One block per segment and a grid the device holds at once: the
  // workgroups exchange their local states through flags and no state pass
  // runs.  (The residency test is for speed only: a workgroup waits only for
  // workgroups dispatched before it, so the waits end in any case.)
  // Not under graph capture: a replayed launch repeats this call's flag value,
  // so flags left by the previous replay would read as current.  Not for the
  // chunk-mean shortcut, which always takes the state pass.  A scan that
  // starts from a carried memory (A_in) seeds each gather with it.
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  const bool capturing = hipStreamIsCapturing(s, &capture) != hipSuccess || capture != hipStreamCaptureStatusNone;
  a.publish = (MEANC == 0 && a.G == 1 && a.R == 0 && a.nseg > 1 && a.nseg <= kPublishMaxSeg && a.flags != nullptr &&
               !a.window_only && !capturing && (long long)BH * a.nseg <= rows_resident_capacity<E, D, NW>())
                  ? 1
                  : 0;
  // otherwise the state pass also forms the last block's local state (final
  // state without a state update at the end of the critical path)
  a.final_slot = (!a.publish && a.nseg > 1 && a.A_final && !a.window_only) ? 1 : 0;
  // (TC_FORWARD_MAX_POLLS overrides the poll bound: 0 makes every wait end at
  // once, which is how the path of a wait that runs out is tested)
  const char* polls = getenv("TC_FORWARD_MAX_POLLS");
  a.max_polls = polls ? atoi(polls) : kPublishPolls;
  const bool ring = a.row0 > 0;
  const bool aligned = a.row0 % 64 == 0 && a.W % 64 == 0;  // (tiles never straddle the ring's end)
  if (a.nseg > 1 && !a.publish && !a.window_only) {
    if (ring && aligned)
      hipLaunchKernelGGL((seg_state_kernel<E, D, BM, MEANC, 2>), dim3(BH * (a.nseg - 1 + a.final_slot)),
                         dim3(256), 0, s, a);
    else if (ring)
      hipLaunchKernelGGL((seg_state_kernel<E, D, BM, MEANC, 1>), dim3(BH * (a.nseg - 1 + a.final_slot)),
                         dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((seg_state_kernel<E, D, BM, MEANC>), dim3(BH * (a.nseg - 1 + a.final_slot)), dim3(256), 0,
                         s, a);
    if (!a.prefix_direct)
      hipLaunchKernelGGL((seg_chain_kernel<D, BM>), dim3((D * D + kChainThreads - 1) / kChainThreads, BH),
                         dim3(kChainThreads), 0, s, a);
  }
  const dim3 grid(BH * a.nseg), block(64 * NW);
  if (MEANC == 0 && ring) {  // (continuations run the exact scan)
    if (a.publish && aligned)
      hipLaunchKernelGGL((fwd_kernel_rows<E, D, NW, true, 0, 2>), grid, block, 0, s, a);
    else if (a.publish)
      hipLaunchKernelGGL((fwd_kernel_rows<E, D, NW, true, 0, 1>), grid, block, 0, s, a);
    else if (aligned)
      hipLaunchKernelGGL((fwd_kernel_rows<E, D, NW, false, 0, 2>), grid, block, 0, s, a);
    else
      hipLaunchKernelGGL((fwd_kernel_rows<E, D, NW, false, 0, 1>), grid, block, 0, s, a);
  } else if (a.publish) {
    hipLaunchKernelGGL((fwd_kernel_rows<E, D, NW, true>), grid, block, 0, s, a);
  } else {
    hipLaunchKernelGGL((fwd_kernel_rows<E, D, NW, false, MEANC>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

template <class E, int D>
static hipError_t launch_rows_mode(const FwdArgs& a, hipStream_t s) {
  switch (a.mean_c) {
    case 0: return launch_rows_impl<E, D, 0>(a, s);
    case 64: return launch_rows_impl<E, D, 64>(a, s);
    case 128: return launch_rows_impl<E, D, 128>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_forward_rows(const FwdArgs& a, int D, bool is_bf16, hipStream_t s) {
  if (!is_bf16) return hipErrorInvalidValue;
  switch (D) {
    case 16: return launch_rows_mode<bf16, 16>(a, s);
    case 32: return launch_rows_mode<bf16, 32>(a, s);
    case 64: return launch_rows_mode<bf16, 64>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tck

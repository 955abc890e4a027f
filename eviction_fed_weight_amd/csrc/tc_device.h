// Device building blocks shared by the TC kernels (gfx950 / CDNA4).
//
// Matrix-core conventions used everywhere (one 64-lane wavefront, lane l,
// l16 = l % 16, lg = l / 16):
//   16x16x32 bf16 MFMA:  out[m][n] += sum_k A[m][k] * B[k][n]
//     lane l supplies A[m = l16][k = 8*lg + j] and B[k = 8*lg + j][n = l16],
//     j = 0..7, and receives out[m = 4*lg + i][n = l16], i = 0..3.
//   float32 operands use four-wide 16x16x4 MFMAs; instruction j takes element
//   j of the same eight-element fragment, so a float32 "fragment" covers the
//   same 32 contraction indices with the same lane assignment.
#pragma once

#include <type_traits>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tck {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

template <class E>
struct Mfma;

template <>
struct Mfma<bf16> {
  typedef bf16x8 frag;
  static constexpr bool kSplit = true;  // float32 operands need a hi/lo split
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ frag pack(const float (&x)[8]) {
    frag r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (bf16)x[j];
    return r;
  }
  // hi = rne(x), lo = rne(x - hi): x is represented to ~2^-17 relative.
  static __device__ __forceinline__ void split(const float (&x)[8], frag& hi, frag& lo) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const bf16 h = (bf16)x[j];
      hi[j] = h;
      lo[j] = (bf16)(x[j] - (float)h);
    }
  }
  static __device__ __forceinline__ frag zero() {
    frag r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (bf16)0.0f;
    return r;
  }
  // 8 consecutive elements from LDS (16-byte aligned).
  static __device__ __forceinline__ frag lds8(const bf16* p) { return *(const bf16x8*)p; }
  static __device__ __forceinline__ void to_f32(const frag& f, float (&x)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = (float)f[j];
  }
};

template <>
struct Mfma<float> {
  typedef f32x8 frag;
  static constexpr bool kSplit = false;
  static __device__ __forceinline__ f32x4 mma(frag a, frag b, f32x4 c) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
    return c;
  }
  static __device__ __forceinline__ frag pack(const float (&x)[8]) {
    frag r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = x[j];
    return r;
  }
  static __device__ __forceinline__ void split(const float (&x)[8], frag& hi, frag& lo) {
    hi = pack(x);
    (void)lo;
  }
  static __device__ __forceinline__ frag zero() {
    frag r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = 0.0f;
    return r;
  }
  static __device__ __forceinline__ frag lds8(const float* p) {
    const f32x4 a = *(const f32x4*)p;
    const f32x4 b = *(const f32x4*)(p + 4);
    frag r;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      r[j] = a[j];
      r[j + 4] = b[j];
    }
    return r;
  }
  static __device__ __forceinline__ void to_f32(const frag& f, float (&x)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = f[j];
  }
};

// x^n by binary powering (0^0 = 1); about log2(n) roundings.
__device__ __forceinline__ float powi(float x, int n) {
  float r = 1.0f, b = x;
  while (n > 0) {
    if (n & 1) r *= b;
    b *= b;
    n >>= 1;
  }
  return r;
}

__device__ __forceinline__ float sigmoidf(float g) { return 1.0f / (1.0f + __expf(-g)); }

// Reductions over the four lanes that share l16 (lanes l16, +16, +32, +48).
__device__ __forceinline__ float max4(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float sum4(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}
// Same reductions with the gfx950 lane-swap instructions (VALU only, no LDS
// round trip).  Every lane of the wavefront must be active.
__device__ __forceinline__ float xmax4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float xsum4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// 2^x with the hardware instruction (results below 2^-126 flush to zero;
// -inf gives 0).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}


typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Column fragment: rows 0..7 of `blk` (row stride ld elements) at column l16,
// i.e. the 8 contraction values a matrix-core operand needs when the
// contraction runs down the rows of a row-major LDS tile.  For bf16 this is
// two gfx950 transpose reads (ds_read_b64_tr_b16): within each group of 16
// lanes, lane i addresses row i/4, columns 4*(i%4)..+3 of a 4 x 16 block and
// lane n receives column n of the four rows.
template <class E>
struct ColFrag;

// The bf16 form is a transposing LDS read that exchanges data between the
// lanes of each 16-lane group: every lane must execute it (never under a
// lane-dependent condition), and every address must hold written data.
template <>
struct ColFrag<bf16> {
  static __device__ __forceinline__ bf16x8 read(const bf16* blk, int ld, int l16) {
    const bf16* p0 = blk + (l16 >> 2) * ld + 4 * (l16 & 3);
    const bf16* p1 = p0 + 4 * ld;
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
struct ColFrag<float> {
  static __device__ __forceinline__ f32x8 read(const float* blk, int ld, int l16) {
    f32x8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = blk[j * ld + l16];
    return r;
  }
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

// Buffer resource over `bytes` bytes at p: buffer loads at byte offsets
// outside [0, bytes) return zero, so tile loads need no per-lane branches
// (rows before the sequence start or past its end read as zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t rs, int byte_off) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  const v4i x = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)byte_off, 0, 0);
  return uint4{(uint32_t)x[0], (uint32_t)x[1], (uint32_t)x[2], (uint32_t)x[3]};
}
// The same load marked non-temporal (the nt cache-policy bit): for data read
// once per launch, so that streaming it does not evict what is reused.
__device__ __forceinline__ uint4 buf_load16_nt(__amdgpu_buffer_rsrc_t rs, int byte_off) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  const v4i x = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)byte_off, 0, 2);
  return uint4{(uint32_t)x[0], (uint32_t)x[1], (uint32_t)x[2], (uint32_t)x[3]};
}

// Key or value rows of a sequence that may continue an earlier one: rows
// r >= p are rows r - p of `cur` (this call's tokens); rows 0 <= r < p are the
// ring slots (s0 + r) mod W of `ring` (the re-read window of a continuation,
// in time order); rows r < 0 and rows past the end read as zeros.  p = 0 for a
// sequence that starts at token 0.
struct SeqRows {
  __amdgpu_buffer_rsrc_t cur, ring;
  int p, s0, W;
};

// Unrolled copy of NR rows of a row-major [T][D] matrix by NTH threads: load() issues every
// global load of the tile at once (through a buffer resource covering the
// sequence, so out-of-range rows read as zero) so they can be in flight while
// the previous tile is computed; store() writes the registers to a row-major
// LDS tile with leading dimension ld.
template <class E, int D, int NR, int NTH = 256>
struct TileRegs {
  static constexpr int VE = 16 / (int)sizeof(E);
  static constexpr int VPR = D / VE;
  static constexpr int NV = NR * VPR;
  static constexpr int PER = (NV + NTH - 1) / NTH;
  uint4 v[PER];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int r0) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int x = (int)threadIdx.x + NTH * p;
      const int row = x / VPR;
      const int col = (x - row * VPR) * VE;
      int off = ((r0 + row) * D + col) * (int)sizeof(E);
      if (NV % NTH != 0 && x >= NV) off = -16;  // out of range: reads zero
      v[p] = buf_load16(rs, off);
    }
  }
  __device__ __forceinline__ void store(E* lds, int ld) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int x = (int)threadIdx.x + NTH * p;
      const int row = x / VPR;
      const int col = (x - row * VPR) * VE;
      if (NV % NTH == 0 || x < NV) *(uint4*)(lds + row * ld + col) = v[p];
    }
  }
};


// Tile load from a sequence: RING = 0 for a sequence that starts at token 0
// (no prefix: the plain single-resource load, nothing else in the kernel's
// code), RING = 1 or 2 for a continuation that re-reads the ring (2: the
// prefix length p is a multiple of the tile rows).
template <int RING, class TR>
__device__ __forceinline__ void load_seq(TR& t, const SeqRows& s, int r0) {
  if constexpr (RING != 0)
    t.load(s, r0);
  else
    t.load(s.cur, r0);
}

// TileRegs for rows of a continued sequence (SeqRows): each vector is read
// from the ring or from the current tokens with a pair of loads, of which the
// other is out of range and returns zero; the pair is combined only in
// store(), a pipeline step later, so that no wait follows the loads.
template <class E, int D, int NR, int NTH = 256>
struct SeqTileRegs {
  using Base = TileRegs<E, D, NR, NTH>;
  static constexpr int VE = Base::VE, VPR = Base::VPR, NV = Base::NV, PER = Base::PER;
  uint4 v[PER], w[PER];
  __device__ __forceinline__ void load(const SeqRows& s, int r0) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int x = (int)threadIdx.x + NTH * p;
      const int row = x / VPR;
      const int col = (x - row * VPR) * VE;
      const int rr = r0 + row;
      const bool in = NV % NTH == 0 || x < NV;
      int slot = s.s0 + rr;  // (s0 < W and rr < p <= W)
      if (slot >= s.W) slot -= s.W;
      const int oc = (in && rr >= s.p) ? ((rr - s.p) * D + col) * (int)sizeof(E) : -16;
      const int orr = (in && rr >= 0 && rr < s.p) ? (slot * D + col) * (int)sizeof(E) : -16;
      v[p] = buf_load16(s.cur, oc);
      w[p] = buf_load16(s.ring, orr);
    }
  }
  __device__ __forceinline__ void store(E* lds, int ld) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int x = (int)threadIdx.x + NTH * p;
      const int row = x / VPR;
      const int col = (x - row * VPR) * VE;
      if (NV % NTH == 0 || x < NV)
        *(uint4*)(lds + row * ld + col) = uint4{v[p].x | w[p].x, v[p].y | w[p].y, v[p].z | w[p].z, v[p].w | w[p].w};
    }
  }
};

// TileRegs for rows of a continued sequence whose prefix length p is a
// multiple of NR and tiles that start at multiples of NR: a tile then lies
// wholly in the ring or wholly in the current tokens, so one load per vector
// from a resource chosen once per tile (the same for every lane) serves it.
// Ring rows wrap at most once within a tile (slot (s0 + r) mod W).
template <class E, int D, int NR, int NTH = 256>
struct AlignedSeqTileRegs {
  using Base = TileRegs<E, D, NR, NTH>;
  static constexpr int VE = Base::VE, VPR = Base::VPR, NV = Base::NV, PER = Base::PER;
  uint4 v[PER];
  __device__ __forceinline__ void load(const SeqRows& s, int r0) {
    // (r0 is the same in every lane: the branch is uniform and each side
    // loads through a scalar resource)
    if (__builtin_amdgcn_readfirstlane(r0) >= s.p) {
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int x = (int)threadIdx.x + NTH * p;
        const int row = x / VPR;
        const int col = (x - row * VPR) * VE;
        int off = ((r0 + row - s.p) * D + col) * (int)sizeof(E);
        if (NV % NTH != 0 && x >= NV) off = -16;  // out of range: reads zero
        v[p] = buf_load16(s.cur, off);
      }
    } else {
#pragma unroll
      for (int p = 0; p < PER; ++p) {
        const int x = (int)threadIdx.x + NTH * p;
        const int row = x / VPR;
        const int col = (x - row * VPR) * VE;
        const int rr = r0 + row;
        int slot = s.s0 + rr;  // (s0 < W and rr < p <= W)
        if (slot >= s.W) slot -= s.W;
        int off = (slot * D + col) * (int)sizeof(E);
        if ((NV % NTH != 0 && x >= NV) || rr < 0) off = -16;  // out of range: reads zero
        v[p] = buf_load16(s.ring, off);
      }
    }
  }
  __device__ __forceinline__ void store(E* lds, int ld) const {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int x = (int)threadIdx.x + NTH * p;
      const int row = x / VPR;
      const int col = (x - row * VPR) * VE;
      if (NV % NTH == 0 || x < NV) *(uint4*)(lds + row * ld + col) = v[p];
    }
  }
};

// Staging registers of a key/value tile: plain for a sequence from token 0
// (RING = 0), SeqTileRegs for a continuation that re-reads the ring (1), and
// AlignedSeqTileRegs when its prefix is a multiple of the tile rows (2).
template <int RING, class E, int D, int NR, int NTH = 256>
using KVRegs = typename std::conditional<
    RING == 0, TileRegs<E, D, NR, NTH>,
    typename std::conditional<RING == 1, SeqTileRegs<E, D, NR, NTH>, AlignedSeqTileRegs<E, D, NR, NTH>>::type>::type;

// Workgroup b of a grid of n runs on XCD b % 8 (the eight chiplets take
// workgroups in turn, each with its own L2).  Renumber so that each XCD gets
// one contiguous range of logical indices: neighbouring work (segments of one
// head, which share key/value rows) then shares an L2.
__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int x = b & 7, q = n >> 3, r = n & 7;
  return x * q + (x < r ? x : r) + (b >> 3);
}

// xcd_remap with the second half of each XCD's range in reverse order.  An
// XCD fills each compute unit's first slot before its second, so the two
// workgroups that share a unit get indices u and nx - 1 - u of the range: with
// one head's segments (light ones first) contiguous, a heavy segment then
// shares its unit with a light one.
__device__ __forceinline__ int xcd_remap_paired(int b, int n) {
  const int x = b & 7, q = n >> 3, r = n & 7;
  const int nx = q + (x < r ? 1 : 0), bx = x * q + (x < r ? x : r);
  const int u = b >> 3, hh = nx >> 1;
  return bx + (u < hh ? u : hh + (nx - 1 - u));
}

// Compiler-visible s_waitcnt vmcnt(0): marks every earlier vector-memory load
// complete for the compiler's own wait analysis (used after loads that feed
// loop-carried registers, so the loop body needs no conservative full waits).
__device__ __forceinline__ void vm_fence_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

}  // namespace tck

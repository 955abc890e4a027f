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
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// 16-byte vector of elements.
template <class E>
struct Vec16 {
  static constexpr int N = 16 / sizeof(E);
  typedef uint4 raw;
};

// Copy rows [r0, r0+NR) of a row-major [T][D] matrix into LDS.  Rows outside
// [0, T) read as zero.  RM: row-major copy (leading dim ldr); TR: transposed
// copy (element (row, d) at tr[d*ldt + row]).  All 256 threads participate.
template <class E, int D, int NR, bool RM, bool TR>
__device__ __forceinline__ void stage_rows(const E* __restrict__ g, int r0, int T, E* rm, int ldr,
                                           E* tr, int ldt) {
  constexpr int VE = 16 / sizeof(E);
  constexpr int VPR = D / VE;  // vectors per row
  constexpr int NV = NR * VPR;
  for (int x = threadIdx.x; x < NV; x += 256) {
    const int row = x / VPR;
    const int col = (x - row * VPR) * VE;
    const int gr = r0 + row;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (gr >= 0 && gr < T) val = *(const uint4*)(g + (size_t)gr * D + col);
    if (RM) *(uint4*)(rm + row * ldr + col) = val;
    if (TR) {
      const E* e = (const E*)&val;
#pragma unroll
      for (int j = 0; j < VE; ++j) tr[(col + j) * ldt + row] = e[j];
    }
  }
}

}  // namespace tck

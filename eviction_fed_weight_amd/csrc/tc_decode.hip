// TC decode step on gfx950 (one streaming step of Figure 2 for many streams).
//
// "Tensor Cache: Eviction-conditioned Associative Memory for Transformers",
// Section 3.2 and Figure 2: (2) the pair in the overwritten ring slot is
// evicted, (3) written A <- lambda A + eta k_old v_old^T, (4) the new pair
// takes the slot, (5) the query reads y_local over the ring and m = q A, and
// y = y_local + sigmoid(g) m.
//
// The step is bound by HBM: per (stream, head) it streams the whole K and V
// ring once (2 W D element loads) and reads+writes the D x D float32 state.
// One workgroup of four waves per (stream, head); no matrix cores.
//   * A: float4-coalesced read-modify-write fused with the partial q A.
//   * L1: each wave walks ring rows with D/VE lanes per row, 16-byte buffer
//     loads (no per-row branches), the next stage in flight while the
//     current one is reduced (DPP butterflies inside each lane group), an
//     online softmax per lane group, and a log-sum-exp merge across lanes
//     and waves at the end.
//   * The slot being overwritten is masked out of the streamed rows: its new
//     pair, known from the inputs, seeds the softmax state of one lane group.
#include "tc_device.h"
#include "tc_launch.h"

namespace tck {

// Sum over each aligned group of N lanes (N = 1 .. 32), result in every lane
// of the group: DPP butterflies inside rows of 16 lanes (xor 1, xor 2, then
// the half-row and row mirrors), a lane swap across row pairs for N = 32.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (N >= 4) x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dpp_mov<0x141>(x);  // row_half_mirror
  if constexpr (N >= 16) x += dpp_mov<0x140>(x); // row_mirror
  if constexpr (N >= 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
  return x;
}

template <class E, int D>
__global__ void __launch_bounds__(256) decode_kernel(DecArgs a) {
  constexpr int VE = 16 / (int)sizeof(E);
  constexpr int LPR = D / VE;     // lanes per ring row
  constexpr int RPW = 64 / LPR;   // ring rows per wave per load
  constexpr int UN = 2;           // ring rows per lane per stage (two stages in flight)
  constexpr int CG = D / 4;       // float4 column groups of A
  constexpr int RG = 256 / CG;    // row groups of A
  __shared__ float qs[D], kn[D], vn[D], ke[D], ve[D];
  __shared__ float mpart[RG][D];
  __shared__ float wacc[4][D];
  __shared__ float wml[4][2];

  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int sh = blockIdx.x;
  const int s = sh / a.H, h = sh - s * a.H;
  const int W = a.W;
  const int64_t t = a.pos[s];
  const int slot = (int)(t % W);
  const bool evict = t >= W;
  const int nvalid = (t + 1 < (int64_t)W) ? (int)(t + 1) : W;

  const E* qg = (const E*)a.q + (size_t)sh * D;
  const E* kg = (const E*)a.k + (size_t)sh * D;
  const E* vg = (const E*)a.v + (size_t)sh * D;
  E* kr = (E*)a.k_ring + (size_t)sh * W * D;
  E* vr = (E*)a.v_ring + (size_t)sh * W * D;

  if (tid < D) {
    qs[tid] = (float)qg[tid];
    kn[tid] = (float)kg[tid];
    vn[tid] = (float)vg[tid];
    if (evict) {
      ke[tid] = (float)kr[(size_t)slot * D + tid];
      ve[tid] = (float)vr[(size_t)slot * D + tid];
    }
  }
  __syncthreads();
  // step 4: the new pair takes the slot (after the evicted pair was read)
  if (tid < D) {
    kr[(size_t)slot * D + tid] = kg[tid];
    vr[(size_t)slot * D + tid] = vg[tid];
  }

  // ---- steps 3 and 5 (L2): A <- lam A + eta k_e v_e^T, partial m = q A ----
  {
    float* Ag = a.A + (size_t)sh * D * D;
    const float lam = a.lam[h], eta = a.eta[h];
    const int cg = tid % CG, rg = tid / CG;
    float4 mp = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int row = rg; row < D; row += RG) {
      float4* p = (float4*)(Ag + (size_t)row * D + cg * 4);
      float4 x = *p;
      if (evict) {
        const float kk = eta * ke[row];
        x.x = lam * x.x + kk * ve[cg * 4 + 0];
        x.y = lam * x.y + kk * ve[cg * 4 + 1];
        x.z = lam * x.z + kk * ve[cg * 4 + 2];
        x.w = lam * x.w + kk * ve[cg * 4 + 3];
        *p = x;
      }
      const float qa = qs[row];
      mp.x += qa * x.x;
      mp.y += qa * x.y;
      mp.z += qa * x.z;
      mp.w += qa * x.w;
    }
    mpart[rg][cg * 4 + 0] = mp.x;
    mpart[rg][cg * 4 + 1] = mp.y;
    mpart[rg][cg * 4 + 2] = mp.z;
    mpart[rg][cg * 4 + 3] = mp.w;
  }

  // ---- step 5 (L1): softmax over the resident pairs ----
  // Rows j < nvalid of the ring, except the overwritten slot, are streamed
  // with branch-free buffer loads (rows past the resource read as zero and
  // are masked); the new pair in the slot seeds the softmax state of lane
  // group 0 of wave 0.  The next stage's rows are loaded while the current
  // stage is reduced.
  const float sl2 = a.scale * kLog2e;
  const int lr = lane / LPR, lc = lane - (lane / LPR) * LPR;
  float qv[VE];
#pragma unroll
  for (int j = 0; j < VE; ++j) qv[j] = qs[lc * VE + j];
  float mloc = kNegInf, lloc = 0.0f;
  float acc[VE];
#pragma unroll
  for (int j = 0; j < VE; ++j) acc[j] = 0.0f;
  {
    float d = 0.0f;
#pragma unroll
    for (int x = 0; x < VE; ++x) d += qv[x] * kn[lc * VE + x];
    d = group_sum<LPR>(d);  // every lane (the lane exchange needs them all)
    if (wid == 0 && lr == 0) {
      mloc = d * sl2;
      lloc = 1.0f;
#pragma unroll
      for (int x = 0; x < VE; ++x) acc[x] = vn[lc * VE + x];
    }
  }
  {
    const uint32_t rbytes = (uint32_t)((size_t)W * D * sizeof(E));
    const auto Kr = make_rsrc(kr, rbytes);
    const auto Vr = make_rsrc(vr, rbytes);
    constexpr int STEP = 4 * RPW * UN;  // rows per stage per workgroup
    uint4 kc[UN], vc[UN], kx[UN], vx[UN];
    auto row_of = [&](int j0, int u) { return j0 + u * 4 * RPW + wid * RPW + lr; };
    auto load = [&](int j0, uint4 (&kd)[UN], uint4 (&vd)[UN]) {
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const int off = (row_of(j0, u) * D + lc * VE) * (int)sizeof(E);
        // (non-temporal: the ring, 94 % of the step's bytes, is read once per
        // step; kept out of the caches it no longer evicts the memory A, which
        // the next step reads again -- 0.805 -> 0.759 ms per step, measured)
        kd[u] = buf_load16_nt(Kr, off);
        vd[u] = buf_load16_nt(Vr, off);
      }
    };
    load(0, kc, vc);
    for (int j0 = 0; j0 < nvalid; j0 += STEP) {
      load(j0 + STEP, kx, vx);  // past nvalid: masked (past W: zeros)
      float sc[UN];
      float mb = mloc;
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const E* k8 = (const E*)&kc[u];
        float d = 0.0f;
#pragma unroll
        for (int x = 0; x < VE; ++x) d += qv[x] * (float)k8[x];
        d = group_sum<LPR>(d);
        const int j = row_of(j0, u);
        sc[u] = (j < nvalid && j != slot) ? d * sl2 : kNegInf;
        mb = fmaxf(mb, sc[u]);
      }
      if (mb != kNegInf) {
        const float c = fast_exp2(mloc - mb);
        lloc *= c;
#pragma unroll
        for (int x = 0; x < VE; ++x) acc[x] *= c;
#pragma unroll
        for (int u = 0; u < UN; ++u) {
          const float p = fast_exp2(sc[u] - mb);
          const E* v8 = (const E*)&vc[u];
          lloc += p;
#pragma unroll
          for (int x = 0; x < VE; ++x) acc[x] += p * (float)v8[x];
        }
        mloc = mb;
      }
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        kc[u] = kx[u];
        vc[u] = vx[u];
      }
    }
  }
  // merge lanes of the wave: common max, then sum over lanes with equal lc
  float M = mloc;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) M = fmaxf(M, __shfl_xor(M, o));
  const float f = (mloc == kNegInf) ? 0.0f : fast_exp2(mloc - M);
  lloc *= f;
#pragma unroll
  for (int x = 0; x < VE; ++x) acc[x] *= f;
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1) {
    lloc += __shfl_xor(lloc, o);
#pragma unroll
    for (int x = 0; x < VE; ++x) acc[x] += __shfl_xor(acc[x], o);
  }
  if (lr == 0) {
#pragma unroll
    for (int x = 0; x < VE; ++x) wacc[wid][lc * VE + x] = acc[x];
    if (lc == 0) {
      wml[wid][0] = M;
      wml[wid][1] = lloc;
    }
  }
  __syncthreads();
  if (tid < D) {
    float Mb = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) Mb = fmaxf(Mb, wml[w][0]);
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float fw = (wml[w][0] == kNegInf) ? 0.0f : fast_exp2(wml[w][0] - Mb);
      num += fw * wacc[w][tid];
      den += fw * wml[w][1];
    }
    float m = 0.0f;
    for (int g = 0; g < RG; ++g) m += mpart[g][tid];
    const float yv = num / den + sigmoidf(a.gate[h]) * m;
    ((E*)a.y)[(size_t)sh * D + tid] = (E)yv;
  }
}

__global__ void pos_advance_kernel(int64_t* pos, int S) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s < S) pos[s] += 1;
}

template <class E, int D>
static hipError_t launch_dec_impl(const DecArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((decode_kernel<E, D>), dim3(a.S * a.H), dim3(256), 0, st, a);
  hipLaunchKernelGGL(pos_advance_kernel, dim3((a.S + 255) / 256), dim3(256), 0, st, a.pos, a.S);
  return hipGetLastError();
}

hipError_t launch_decode(const DecArgs& a, int D, bool is_bf16, hipStream_t s) {
  if (is_bf16) {
    switch (D) {
      case 16: return launch_dec_impl<bf16, 16>(a, s);
      case 32: return launch_dec_impl<bf16, 32>(a, s);
      case 64: return launch_dec_impl<bf16, 64>(a, s);
      case 128: return launch_dec_impl<bf16, 128>(a, s);
    }
  } else {
    switch (D) {
      case 16: return launch_dec_impl<float, 16>(a, s);
      case 32: return launch_dec_impl<float, 32>(a, s);
      case 64: return launch_dec_impl<float, 64>(a, s);
      case 128: return launch_dec_impl<float, 128>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace tck

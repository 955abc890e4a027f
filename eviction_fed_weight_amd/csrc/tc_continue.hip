// Continuation of a TC sequence on gfx950: chunked prefill after earlier
// tokens, and the handoff from prefill to decode.
//
// "Tensor Cache: Eviction-conditioned Associative Memory for Transformers",
// Figure 2: a stream's layer state is the ring of its last W keys/values
// (slot = position mod W) and the memory A; each new token evicts the pair in
// its slot into A (A <- lambda A + eta k v^T, Section 3.2), takes the slot
// and reads both levels.  T new tokens after pos0 seen ones give exactly the
// result of T such steps; here they run through the parallel forward:
//
//   * the forward kernels run over an extended sequence -- the ring's
//     p = min(pos0, W) tokens in time order, then the new tokens -- with a
//     zero start state and store only rows p .. p+T-1.  Its window rows are
//     the true windows (the ring holds every key an output row can see) and
//     its state holds exactly the pairs evicted during this call;
//   * the memory carried in, A_in, is linear in the read: after n_t of this
//     call's evictions it has decayed to lambda^n_t A_in, so each row adds
//     sigmoid(g) lambda^n_t q_t A_in (formed here in float32 and added by the
//     forward kernels before the output is rounded), and the final memory is
//     the forward's state plus lambda^N A_in;
//   * the last min(pos0 + T, W) tokens go back into their ring slots.
// Steps t < W evict nothing (the memory is left as it is), so
// n_t = max(0, t + 1 - max(pos0, W)) for the step at position t.
#include "tc_device.h"
#include "tc_launch.h"

namespace tck {

// Extended sequence rows, one 16-byte vector per thread: row r < p is ring
// slot (pos0 - p + r) mod W (its query row is zero: never stored), row
// r >= p is new token r - p.
__global__ void __launch_bounds__(256) cont_gather_kernel(ContArgs a) {
  const int nv = a.D * a.esize / 16;  // vectors per row
  const long long total = (long long)a.B * a.H * a.Tx * nv;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long long)gridDim.x * 256) {
    const long long row = i / nv;
    const int c = (int)(i - row * nv);
    const long long bh = row / a.Tx;
    const int r = (int)(row - bh * a.Tx);
    uint4 qv, kv, vv;
    if (r < a.p) {
      const long long slot = (a.pos0 - a.p + r) % a.W;
      const long long src = (bh * a.W + slot) * nv + c;
      kv = ((const uint4*)a.k_ring)[src];
      vv = ((const uint4*)a.v_ring)[src];
      qv = make_uint4(0u, 0u, 0u, 0u);
    } else {
      const long long src = (bh * a.T + (r - a.p)) * nv + c;
      qv = ((const uint4*)a.q)[src];
      kv = ((const uint4*)a.k)[src];
      vv = ((const uint4*)a.v)[src];
    }
    ((uint4*)a.qx)[i] = qv;
    ((uint4*)a.kx)[i] = kv;
    ((uint4*)a.vx)[i] = vv;
  }
}

// yinit[b,h,t,:] = sigmoid(g_h) lambda_h^n_t q_t A_in[b,h] in float32.
// One workgroup per (b,h) and 16 rows; A_in and the rows staged in LDS.
template <class E, int D>
__global__ void __launch_bounds__(256) cont_init_read_kernel(ContArgs a) {
  constexpr int ROWS = 16;
  __shared__ float As[D * D];
  __shared__ float Qs[ROWS][D];
  const int tiles = (a.T + ROWS - 1) / ROWS;
  const int bh = blockIdx.x / tiles, h = bh % a.H;
  const int t0 = (blockIdx.x - bh * tiles) * ROWS;
  const float* Ag = a.A + (size_t)bh * D * D;
  for (int x = threadIdx.x; x < D * D; x += 256) As[x] = Ag[x];
  const E* qg = (const E*)a.q + (size_t)bh * a.T * D;
  for (int x = threadIdx.x; x < ROWS * D; x += 256) {
    const int t = t0 + x / D;
    Qs[x / D][x % D] = t < a.T ? (float)qg[(size_t)t * D + x % D] : 0.0f;
  }
  __syncthreads();
  const float sg = sigmoidf(a.gate[h]), lam = a.lam[h];
  const long long first = a.pos0 > a.W ? a.pos0 : (long long)a.W;  // first step of this call that evicts
  for (int x = threadIdx.x; x < ROWS * D; x += 256) {
    const int r = x / D, c = x % D, t = t0 + r;
    if (t >= a.T) continue;
    float acc = 0.0f;
#pragma unroll 8
    for (int j = 0; j < D; ++j) acc = __builtin_fmaf(Qs[r][j], As[j * D + c], acc);
    const long long n = a.pos0 + t + 1 - first;
    a.yinit[((size_t)bh * a.T + t) * D + c] = sg * powi(lam, n > 0 ? (int)n : 0) * acc;
  }
}

// A <- A_new + lambda^N A (N = evictions in this call), elementwise.
__global__ void __launch_bounds__(256) cont_state_kernel(ContArgs a) {
  const long long DD = (long long)a.D * a.D, total = (long long)a.B * a.H * DD;
  const long long first = a.pos0 > a.W ? a.pos0 : (long long)a.W;
  const long long N = a.pos0 + a.T - first;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long long)gridDim.x * 256) {
    const int h = (int)((i / DD) % a.H);
    a.A[i] = __builtin_fmaf(powi(a.lam[h], N > 0 ? (int)N : 0), a.A[i], a.A_new[i]);
  }
}

// The last min(Tx, W) extended rows into their ring slots; pos[b] = pos0 + T.
__global__ void __launch_bounds__(256) cont_ring_kernel(ContArgs a) {
  const int nv = a.D * a.esize / 16;
  const int keep = a.Tx < a.W ? a.Tx : a.W;
  const long long total = (long long)a.B * a.H * keep * nv;
  if (a.pos && blockIdx.x == 0)
    for (int b = threadIdx.x; b < a.B; b += 256) a.pos[b] = a.pos0 + a.T;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long long)gridDim.x * 256) {
    const long long row = i / nv;
    const int c = (int)(i - row * nv);
    const long long bh = row / keep;
    const int r = a.Tx - keep + (int)(row - bh * keep);  // extended row
    const long long slot = (a.pos0 - a.p + r) % a.W;
    const long long src = (bh * a.Tx + r) * nv + c, dst = (bh * a.W + slot) * nv + c;
    ((uint4*)a.k_ring)[dst] = ((const uint4*)a.kx)[src];
    ((uint4*)a.v_ring)[dst] = ((const uint4*)a.vx)[src];
  }
}

namespace {
unsigned copy_grid(long long vectors) {
  const long long g = (vectors + 255) / 256;
  return (unsigned)(g < 1 ? 1 : (g > 8192 ? 8192 : g));
}

template <class E>
hipError_t launch_init_read(const ContArgs& a, hipStream_t s) {
  const dim3 grid(a.B * a.H * ((a.T + 15) / 16));
  switch (a.D) {
    case 16: hipLaunchKernelGGL((cont_init_read_kernel<E, 16>), grid, dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL((cont_init_read_kernel<E, 32>), grid, dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL((cont_init_read_kernel<E, 64>), grid, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL((cont_init_read_kernel<E, 128>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_continue_prep(const ContArgs& a, hipStream_t s) {
  const int nv = a.D * a.esize / 16;
  hipLaunchKernelGGL(cont_gather_kernel, dim3(copy_grid((long long)a.B * a.H * a.Tx * nv)), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return a.esize == 2 ? launch_init_read<bf16>(a, s) : launch_init_read<float>(a, s);
}

hipError_t launch_continue_finish(const ContArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(cont_state_kernel, dim3(copy_grid((long long)a.B * a.H * a.D * a.D)), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nv = a.D * a.esize / 16;
  const long long keep = a.Tx < a.W ? a.Tx : a.W;
  hipLaunchKernelGGL(cont_ring_kernel, dim3(copy_grid((long long)a.B * a.H * keep * nv)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace tck

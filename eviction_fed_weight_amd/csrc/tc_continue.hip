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
//     p = min(pos0, W) tokens in time order, then the new tokens -- and store
//     only rows p .. p+T-1.  They read it in place: keys and values of rows
//     below p from their ring slots, the others from the caller's new tokens
//     (no copy).  Its window rows are the true windows (the ring holds every
//     key an output row can see) and its scan runs over exactly the pairs
//     evicted during this call;
//   * the memory carried in, A_in, decays by lambda per eviction of this call
//     (n_t of them by step t).  Once the window is full (pos0 >= W) the
//     extended sequence's evictions start at its row W = p, and when W is a
//     multiple of the forward's block rows every processed block starts at
//     or after that eviction: then the forward simply starts its scan from
//     S(0) = A_in / eta ("fold"), and its final state is the new memory.
//     Otherwise the scan starts from zero, the read of A_in,
//     sigmoid(g) lambda^n_t q_t A_in, is formed here in float32 and added by
//     the forward kernels before the output is rounded, and the final memory
//     is the forward's state plus lambda^N A_in;
//   * the last min(T, W) new tokens go into their ring slots (after the
//     forward has read the ring).
// Steps t < W evict nothing (the memory is left as it is), so
// n_t = max(0, t + 1 - max(pos0, W)) for the step at position t.
#include "tc_device.h"
#include "tc_launch.h"

namespace tck {

// yinit[b,h,t,:] = sigmoid(g_h) lambda_h^n_t q_t A_in[b,h] in float32, on
// the matrix cores.  One workgroup (four waves) per (b,h) and 128 rows; A_in
// is staged transposed in LDS (bf16 inputs: as hi/lo bf16 pairs, keeping
// ~2^-17 of its float32 precision; float32 inputs: as float32).  Computed
// transposed, Y^T = A_in^T q^T, so a lane holds one query row: its q
// fragment is 8 consecutive elements of that row and its result 4
// consecutive outputs.
template <class E, int D>
__device__ __forceinline__ void cont_init_read(const ContArgs& a, int blk) {
  using M = Mfma<E>;
  using frag = typename M::frag;
  constexpr int ROWS = 128, NT = D / 16, NKC = (D + 31) / 32;
  constexpr int LDA = D + 16 / (int)sizeof(E);  // row stride of A_in^T in LDS (elements)
  constexpr int NA = M::kSplit ? 2 : 1;          // hi (and lo) copies
  __shared__ __attribute__((aligned(16))) E At[NA][D * LDA];
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
  const int tiles = (a.T + ROWS - 1) / ROWS;
  const int bh = blk / tiles, h = bh % a.H;
  const int t0 = (blk - bh * tiles) * ROWS;
  const float* Ag = a.A + (size_t)bh * D * D;
  for (int x = tid; x < D * D; x += 256) {  // A_in[k][m] -> At[m][k]
    const int k = x / D, m = x % D;
    const float val = Ag[x];
    const E hi = (E)val;
    At[0][m * LDA + k] = hi;
    if (M::kSplit) At[NA - 1][m * LDA + k] = (E)(val - (float)hi);
  }
  __syncthreads();
  const float sg = sigmoidf(a.gate[h]), lam = a.lam[h];
  const long long first = a.pos0 > a.W ? a.pos0 : (long long)a.W;  // first step of this call that evicts
  const E* qg = (const E*)a.q + (size_t)bh * a.T * D;
  for (int rg = wid; rg < ROWS / 16; rg += 4) {
    const int t = t0 + 16 * rg + l16;  // this lane's query row
    if (t0 + 16 * rg >= a.T) break;
    frag qf[NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const int k0 = kc * 32 + lg * 8;
      qf[kc] = (t < a.T && k0 < D) ? *(const frag*)(qg + (size_t)t * D + k0) : M::zero();
    }
    const long long n = a.pos0 + t + 1 - first;
    const float f = sg * powi(lam, n > 0 ? (int)n : 0);
#pragma unroll
    for (int ct = 0; ct < NT; ++ct) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const int k0 = kc * 32 + lg * 8;
        const E* row = &At[0][(ct * 16 + l16) * LDA + k0];
        acc = M::mma(k0 < D ? M::lds8(row) : M::zero(), qf[kc], acc);
        if (M::kSplit) acc = M::mma(k0 < D ? M::lds8(row + (NA - 1) * D * LDA) : M::zero(), qf[kc], acc);
      }
      if (t < a.T) *(f32x4*)(a.yinit + ((size_t)bh * a.T + t) * D + ct * 16 + lg * 4) = f * acc;
    }
  }
}

// The initial-state read: one workgroup per (b,h) and 128 new rows.  (Not
// launched when the forward folds A_in into its scan.  A read-ahead of the
// inputs into the last-level cache in this launch was measured: it cost more
// than the forward gained from it.)
template <class E, int D>
__global__ void __launch_bounds__(256) cont_prep_kernel(ContArgs a) {
  cont_init_read<E, D>(a, blockIdx.x);
}

// Workgroups 0 .. nA-1: A <- A_new + lambda^N A (N = evictions in this call),
// elementwise; A <- A_new when the forward started its scan from A (fold).  The others: the last min(T, W) new tokens' keys and values
// into their ring slots (position mod W; the ring's other slots keep the
// earlier tokens they hold).  Workgroup 0 also sets pos[b] = pos0 + T.
__global__ void __launch_bounds__(256) cont_finish_kernel(ContArgs a, int nA) {
  if (a.pos && blockIdx.x == 0)
    for (int b = threadIdx.x; b < a.B; b += 256) a.pos[b] = a.pos0 + a.T;
  if ((int)blockIdx.x < nA) {
    const long long DD = (long long)a.D * a.D, total = (long long)a.B * a.H * DD;
    const long long first = a.pos0 > a.W ? a.pos0 : (long long)a.W;
    const long long N = a.pos0 + a.T - first;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long long)nA * 256) {
      const int h = (int)((i / DD) % a.H);
      a.A[i] = a.fold ? a.A_new[i] : __builtin_fmaf(powi(a.lam[h], N > 0 ? (int)N : 0), a.A[i], a.A_new[i]);
    }
    return;
  }
  const int nv = a.D * a.esize / 16;
  const int keep = a.T < a.W ? a.T : a.W;
  const long long total = (long long)a.B * a.H * keep * nv;
  const long long nr = gridDim.x - nA;
  for (long long i = (long long)(blockIdx.x - nA) * 256 + threadIdx.x; i < total; i += nr * 256) {
    const long long row = i / nv;
    const int cc = (int)(i - row * nv);
    const long long bh = row / keep;
    const int t = a.T - keep + (int)(row - bh * keep);  // new token
    const long long slot = (a.pos0 + t) % a.W;
    const long long src = (bh * a.T + t) * nv + cc, dst = (bh * a.W + slot) * nv + cc;
    ((uint4*)a.k_ring)[dst] = ((const uint4*)a.k)[src];
    ((uint4*)a.v_ring)[dst] = ((const uint4*)a.v)[src];
  }
}

namespace {
unsigned copy_grid(long long vectors) {
  const long long g = (vectors + 255) / 256;
  return (unsigned)(g < 1 ? 1 : (g > 8192 ? 8192 : g));
}

template <class E>
hipError_t launch_prep(const ContArgs& a, hipStream_t s) {
  if (a.fold) return hipSuccess;
  const dim3 grid((unsigned)((long long)a.B * a.H * ((a.T + 127) / 128)));  // (bounded on the host)
  switch (a.D) {
    case 16: hipLaunchKernelGGL((cont_prep_kernel<E, 16>), grid, dim3(256), 0, s, a); break;
    case 32: hipLaunchKernelGGL((cont_prep_kernel<E, 32>), grid, dim3(256), 0, s, a); break;
    case 64: hipLaunchKernelGGL((cont_prep_kernel<E, 64>), grid, dim3(256), 0, s, a); break;
    case 128: hipLaunchKernelGGL((cont_prep_kernel<E, 128>), grid, dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_continue_prep(const ContArgs& a, hipStream_t s) {
  return a.esize == 2 ? launch_prep<bf16>(a, s) : launch_prep<float>(a, s);
}

hipError_t launch_continue_finish(const ContArgs& a, hipStream_t s) {
  const int nv = a.D * a.esize / 16;
  const long long keep = a.T < a.W ? a.T : a.W;
  const unsigned nA = copy_grid((long long)a.B * a.H * a.D * a.D);
  const unsigned nR = copy_grid((long long)a.B * a.H * keep * nv);
  hipLaunchKernelGGL(cont_finish_kernel, dim3(nA + nR), dim3(256), 0, s, a, (int)nA);
  return hipGetLastError();
}

}  // namespace tck

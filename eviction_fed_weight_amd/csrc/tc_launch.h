// Internal kernel-argument blocks and launchers (host side of the kernels).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tck {

// Forward: segment walk over 64-row query blocks.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* lam;
  const float* eta;
  const float* gate;
  void* y;
  float* A_final;  // nullable
  float* lse;      // nullable
  float* seg_state;  // [B*H][nseg][D*D] segment-start states (eta factored out)
  int B, H, T, W;
  int nblk;  // ceil(T / block rows): 128 (bf16, D <= 64) or 64
  int j0;    // first query block processed (blocks below it hold only unstored rows < row0)
  int nseg;  // segments of blocks j0 .. nblk-1: the first R hold G + 1 blocks, the others G
  int G;
  int R;
  int prefix_direct;  // fused kernel combines the local segment states itself (no chain kernel)
  float scale;
  // Set by the rows launcher: the state pass also forms the local state of the
  // last segment's evictions, at seg_state[B*H*nseg + bh], and the workgroup
  // of segment 0 (an early finisher) forms A_final from it elementwise.
  int final_slot;
  // Set by the rows launcher when there is one block per segment and the
  // whole grid is resident at once: instead of a state pass, each workgroup
  // forms the local state of its evicted chunk after its window work, stores
  // it at seg_state[bh][seg + 1] and sets flags[bh * nseg + seg] = gen; a
  // later segment of the head waits for those flags before its memory read.
  int publish;
  unsigned long long* flags;  // [B*H][nseg], in the workspace after the states
  unsigned long long gen;     // this call's flag value
  int max_polls;              // bound on the polls of one flag (0: no waiting at all)
  // Output rows: query rows t >= row0 are stored at row t - row0 of y and lse
  // ([B,H,T-row0,...]); rows below row0 (a continuation's re-read prefix) are
  // computed but not stored.  yadd (nullable, float [B,H,T-row0,D]) is added
  // to each stored row before rounding.  tc_forward: row0 = 0, yadd = null.
  int row0;
  const float* yadd;
};

// First block of forward segment s (s = nseg gives nblk).
__host__ __device__ inline int seg_first_block(const FwdArgs& a, int s) { return a.j0 + s * a.G + (s < a.R ? s : a.R); }
// Blocks of forward segment s.
__host__ __device__ inline int seg_blocks(const FwdArgs& a, int s) { return a.G + (s < a.R ? 1 : 0); }

// Decode: one step for S streams x H heads.
struct DecArgs {
  const void* q;
  const void* k;
  const void* v;
  void* k_ring;
  void* v_ring;
  float* A;
  int64_t* pos;
  const float* lam;
  const float* eta;
  const float* gate;
  void* y;
  int S, H, W;
  float scale;
};

// Backward (see tc_backward.hip for the workspace plan).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* y;
  const void* dy;
  const float* lse;
  const float* lam;
  const float* eta;
  const float* gate;
  void* dq;
  void* dk;
  void* dv;
  float* dlam;
  float* deta;
  float* dgate;
  float* fstate;   // forward segment states  [BH][nseg][D*D]  (S, eta-free)
  float* tstate;   // forward tangent states  [BH][nseg][D*D]  (dS/dlambda)
  float* rstate;   // reverse adjoint states  [BH][nseg][D*D]
  float* delta;    // [BH][T] rowwise <dy, y_local>
  float* part;     // [BH][nseg][2] per-workgroup sums of <dy, mt> and <dy, d mt/dlambda>
  int B, H, T, W;
  int nblk, G, nseg;
  float scale;
};

// Continuation of a sequence (T new tokens after pos0 seen ones) through an
// extended sequence in the workspace: the ring's p = min(pos0, W) tokens in
// time order, then the new tokens (Tx = p + T rows).
struct ContArgs {
  const void* q;  // [B,H,T,D] new tokens
  const void* k;
  const void* v;
  void* k_ring;   // [B,H,W,D] slot = position mod W
  void* v_ring;
  float* A;       // [B,H,D,D] memory after step pos0-1 (in), after pos0+T-1 (out)
  int64_t* pos;   // [B] nullable: set to pos0 + T
  const float* lam;
  const float* gate;
  void* qx;       // [B,H,Tx,D] extended sequence (workspace)
  void* kx;
  void* vx;
  float* yinit;   // [B,H,T,D] sigmoid(g) lambda^n_t q_t A_in (workspace)
  const float* A_new;  // [B,H,D,D] memory of this call's evictions alone (workspace)
  long long pos0;
  int B, H, T, W, D, p, Tx;
  int esize;      // bytes per element of q/k/v and the rings
};

hipError_t launch_continue_prep(const ContArgs& a, hipStream_t s);    // extended sequence + initial-state read
hipError_t launch_continue_finish(const ContArgs& a, hipStream_t s);  // A, ring and pos updates

hipError_t launch_forward(const FwdArgs& a, int D, bool is_bf16, hipStream_t s);     // 64-row blocks: float32, and bf16 with D = 128
hipError_t launch_forward_rows(const FwdArgs& a, int D, bool is_bf16, hipStream_t s);  // 128-row blocks: bf16 with D <= 64
hipError_t launch_decode(const DecArgs& a, int D, bool is_bf16, hipStream_t s);
hipError_t launch_backward_bf16(const BwdArgs& a, int D, hipStream_t s);
hipError_t launch_backward_f32(const BwdArgs& a, int D, hipStream_t s);
inline hipError_t launch_backward(const BwdArgs& a, int D, bool is_bf16, hipStream_t s) {
  return is_bf16 ? launch_backward_bf16(a, D, s) : launch_backward_f32(a, D, s);
}

}  // namespace tck

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
  // [B*H][nseg] (nullable), in the workspace after the flags: every
  // workgroup of the call writes gen to its word, or ~gen when one of its
  // flag waits ran out (its rows and the final state are then NaN).  The
  // host reads them with tc_forward_status.
  unsigned long long* status;
  // Rows of the sequence: q, k and v hold rows row0 .. T-1 ([B,H,T-row0,D]);
  // keys and values of rows 0 .. row0-1 (a continuation's re-read window) are
  // the ring slots (ring_s0 + r) mod W of k_ring and v_ring ([B,H,W,D]).
  // Query rows t >= row0 are stored at row t - row0 of y and lse
  // ([B,H,T-row0,...]); rows below row0 have no queries and are not stored.
  // yadd (nullable, float [B,H,T-row0,D]) is added to each stored row before
  // rounding.  tc_forward: row0 = 0, no ring, yadd = null.
  int row0;
  const void* k_ring;
  const void* v_ring;
  int ring_s0;
  const float* yadd;
  // (nullable) memory carried in by a continuation whose first processed
  // block starts at eviction 0 (row0 = W, a multiple of the block rows): the
  // scan starts from S(0) = A_in / eta instead of zero.  [B,H,D,D] float.
  const float* A_in;
  // Decays of the state per query block: BM (one per evicted token) for the
  // exact scan, BM / C for the chunk-mean shortcut (one per chunk).
  int blk_pow;
  // 0: the exact scan.  64 or 128: the chunk-mean shortcut with chunks of
  // that many evictions (tc_forward_chunk_mean; bf16 rows kernel only).
  int mean_c;
  // State pass in parts (fused kernel only, exact scan, no final slot): each
  // segment's evictions are split into nparts tile ranges, one workgroup
  // each, whose local states go to parts ([B*H][nseg][nparts][D*D], slot
  // m + 1 for segment m); the chain combines them.  nparts = 1: one
  // workgroup per segment writing L_m to seg_state[m+1].
  int nparts;
  float* parts;
  // 1: the window attention alone (no state pass, no memory read, no
  // A_final): y = y_local (+ yadd).  The delta-rule forward forms its memory
  // read separately and adds it through yadd.
  int window_only;
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

// Continuation of a sequence (T new tokens after pos0 seen ones) as an
// extended sequence: the ring's p = min(pos0, W) tokens in time order, then
// the new tokens (Tx = p + T rows), read in place by the forward kernels.
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
  float* yinit;   // [B,H,T,D] sigmoid(g) lambda^n_t q_t A_in (workspace)
  const float* A_new;  // [B,H,D,D] memory of this call's evictions alone (workspace)
  long long pos0;
  int B, H, T, W, D, p, Tx;
  int esize;      // bytes per element of q/k/v and the rings
  // 1: the forward starts its scan from A_in (pos0 >= W and W a multiple of
  // its block rows), so there is no initial-state read and A <- A_new
  int fold;
};

// Memory path of the delta-rule forward (chunks of 64 evictions).
struct DeltaArgs {
  const void* q;  // [B,H,T,D]
  const void* k;
  const void* v;
  const float* lam;
  const float* eta;
  const float* gate;
  float* UpT;      // [B*H][nch][D][64] ((I+N)^-1 V)^T per chunk
  float* WmT;      // [B*H][nch][D][64] ((I+N)^-1 diag(lambda^i) K)^T per chunk
  float* Mc;       // [B*H][nch][D][D] M_c (row-major): A_{c+1} = M_c A_c + B_c
  float* BcT;      // [B*H][nch][D][D] B_c^T
  float* Mg;       // [B*H][ng][D][D] composed map of each group of G chunks (row-major)
  float* BgT;      // [B*H][ng][D][D] its offset, transposed
  float* AgT;      // [B*H][ng+1][D][D] A^T at every group start (and after the last)
  float* AcT;      // [B*H][nch][D][D] A^T at every chunk start (D = 128 only: with D <= 64 the read is fused)
  float* Ms;       // [B*H][nsg][D][D] composed map of each supergroup of G2 groups (when nsg > 0)
  float* BsT;      // [B*H][nsg][D][D] its offset, transposed
  float* AsT;      // [B*H][nsg+1][D][D] A^T at every supergroup start (and after the last)
  float* yadd;     // [B*H][T][D] sigma(g) m_t
  float* A_final;  // [B*H][D][D] (nullable)
  int B, H, T, W;
  int E;    // evictions per sequence, max(0, T - W)
  int nch;  // chunks, ceil(E / 64)
  int G;    // chunks per group
  int ng;   // groups, ceil(nch / G)
  int G2;   // groups per supergroup
  int nsg;  // supergroups, ceil(ng / G2); 0: two levels (the walk runs over the groups)
};
hipError_t launch_delta_memory(const DeltaArgs& a, int D, bool is_bf16, hipStream_t s);

hipError_t launch_continue_prep(const ContArgs& a, hipStream_t s);    // initial-state read
hipError_t launch_continue_finish(const ContArgs& a, hipStream_t s);  // A, ring and pos updates

hipError_t launch_forward_bf16(const FwdArgs& a, int D, hipStream_t s);  // 64-row blocks: bf16 with D = 128
hipError_t launch_forward_f32(const FwdArgs& a, int D, hipStream_t s);   // 64-row blocks: float32
inline hipError_t launch_forward(const FwdArgs& a, int D, bool is_bf16, hipStream_t s) {
  return is_bf16 ? launch_forward_bf16(a, D, s) : launch_forward_f32(a, D, s);
}
hipError_t launch_forward_rows(const FwdArgs& a, int D, bool is_bf16, hipStream_t s);  // 128-row blocks: bf16 with D <= 64
hipError_t launch_decode(const DecArgs& a, int D, bool is_bf16, hipStream_t s);
hipError_t launch_backward_bf16(const BwdArgs& a, int D, hipStream_t s);
hipError_t launch_backward_f32(const BwdArgs& a, int D, hipStream_t s);
inline hipError_t launch_backward(const BwdArgs& a, int D, bool is_bf16, hipStream_t s) {
  return is_bf16 ? launch_backward_bf16(a, D, s) : launch_backward_f32(a, D, s);
}

}  // namespace tck

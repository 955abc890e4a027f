// C ABI of the TC layer: host-side validation, workspace planning and
// dispatch to the gfx950 kernels.  No device allocation and no
// synchronisation (except in the explicit status query); the only global
// state is a call counter (the forward's flag values), in the rows launcher
// a per-device count of resident workgroups, and the per-device address of
// the allocation-free forward's static scratch.
#include <math.h>

#include <atomic>
#include <mutex>
#include <random>
#include <vector>
#include <stdint.h>
#include <string.h>

#include "../../include/tc.h"
#include "tc_launch.h"

constexpr size_t kScratchBytes = (size_t)32 << 20;  // 32 MiB per device
constexpr int kMaxDevices = 64;

// The allocation-free forward's workspace (see scratch_ptr below).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kBlock = 64;  // backward: query rows per block = tokens per scan chunk

// Query rows per block of the forward kernels: 128 (four waves of 32 rows)
// for bf16 with D <= 64, else 64 (four waves of 16 rows).  float32 inputs
// run on the 64-row kernel, whose float32 build keeps every matrix-core
// result in VGPRs (see the 16x16x4 float32 note in tc_forward.hip).
// Query rows per block of the forward: 128 for bf16 (the rows kernel for
// D <= 64, eight waves of the fused kernel for D = 128), 64 for float32.
int fwd_block(int D, int32_t dtype) { return dtype == TC_BF16 ? 128 : 64; }
// bf16 with D <= 64 runs the rows kernel, everything else the fused kernel.
bool rows_kernel(int D, int32_t dtype) { return D <= 64 && dtype == TC_BF16; }

bool supported_d(int D) { return D == 16 || D == 32 || D == 64 || D == 128; }

size_t elem_size(int32_t dtype) { return dtype == TC_BF16 ? 2 : 4; }

bool valid_dtype(int32_t dtype) { return dtype == TC_F32 || dtype == TC_BF16; }

// Byte ranges [p, p + n) overlap?
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

struct Plan {
  int nblk, j0, G, R, nseg;  // segments of blocks j0..nblk-1: the first R of G + 1 blocks, the others of G
  size_t state_bytes;  // one [BH][nseg][D*D] float block
  int nparts;          // workgroups per segment of the state pass (fused kernel)
  size_t parts_bytes;  // their local states, [BH][nseg][nparts][D*D] float (nparts > 1)
};

// Workgroups of the fused forward kernel resident at once on an MI355X
// (256 compute units): two per unit for D <= 64, one for D = 128.  Only the
// speed of the schedule depends on it, never the result.
long long fwd_slots(int D, int32_t dtype) {
  (void)dtype;
  return D >= 128 ? 256 : 512;
}

// Blocks per segment.  A workgroup walks G blocks after a start-up of about
// half a block (state load, first tiles), so the fused kernel takes about
// ceil(BH * nseg / slots) * (G + 1/2) block-times; the chain over segments
// adds a little per segment.  Pick the G that minimises the sum.  Then spread
// the blocks over as many segments as one round of resident workgroups holds,
// without lengthening the longest segment: segments of G' and G' + 1 blocks
// (the first R the longer).  Two workgroups share a compute unit, whose time
// follows the blocks of both, and the renumbering of the rows kernel pairs the
// longer early segments with shorter late ones (B=1 H=12 T=32768: 42 segments
// of 6 or 7 blocks instead of 37 of 7, the busiest unit 13 blocks instead of 14).
//
// Blocks j0 .. nblk-1 are processed: with row0 > 0 (a continuation's ring
// prefix, never stored) whole blocks below row0 are skipped.
Plan plan_for(const tc_shape_t& s, int row0 = 0) {
  Plan p;
  const long long BH = (long long)s.B * s.H;
  const long long slots = fwd_slots(s.D, s.dtype);
  const int bm = fwd_block(s.D, s.dtype);
  p.nblk = (s.T + bm - 1) / bm;
  p.j0 = row0 / bm;
  const int nb = p.nblk - p.j0;  // blocks to process
  long long best = -1;
  int bestG = 1;
  for (int G = 1; G <= nb; ++G) {
    const long long nseg = (nb + G - 1) / G;
    if (G > 1 && (nb + G - 2) / (G - 1) == nseg) continue;  // same split as G - 1, more work per segment
    const long long cost = ((BH * nseg + slots - 1) / slots) * (2 * G + 1) * 100 + nseg;
    if (best < 0 || cost <= best) {
      best = cost;
      bestG = G;
    }
  }
  // The 128-row kernel carries the state from block to block with two decayed
  // rank-64 updates inside the workgroup, work that the parallel state pass
  // does off the critical path when segments are short.  When pairs of blocks
  // fill more than one round of workgroups, segments of two blocks measured
  // fastest (B=1 H=12 T=32768: 0.234 ms against 0.242 ms for the 42
  // segments of 6-7 blocks this model picks, and 0.253 ms for single blocks,
  // whose chain over 256 segments per head costs more than the updates save).
  if (rows_kernel(s.D, s.dtype) && bestG > 2 && BH * ((nb + 1) / 2) > slots) bestG = 2;
  p.nseg = (nb + bestG - 1) / bestG;
  if (BH * p.nseg <= slots) {
    const long long fill = slots / BH < nb ? slots / BH : nb;
    if (fill > p.nseg) p.nseg = (int)fill;
  }
  p.G = nb / p.nseg;
  p.R = nb - p.G * p.nseg;
  // segment states, then one last-block local state per (b,h)
  p.state_bytes = (size_t)BH * (p.nseg + 1) * s.D * s.D * sizeof(float);
  // The fused kernel's segments are long (one workgroup per unit walks many
  // blocks), so its state pass has few workgroups, each a long dependent walk
  // over the segment's tiles: split each segment into up to four parts so
  // that about three workgroups per compute unit share the walk.
  p.nparts = 1;
  p.parts_bytes = 0;
  if (!rows_kernel(s.D, s.dtype) && p.nseg > 1) {
    const long long want = (768 + BH * (p.nseg - 1) - 1) / (BH * (p.nseg - 1));
    const int tiles = p.G * (bm / 64);
    p.nparts = (int)(want < 4 ? want : 4);
    if (p.nparts > tiles) p.nparts = tiles;
    if (p.nparts < 1) p.nparts = 1;
    if (p.nparts > 1) p.parts_bytes = (size_t)BH * p.nseg * p.nparts * s.D * s.D * sizeof(float);
  }
  return p;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Forward workspace: the segment states, then one 64-bit flag per segment,
// then one 64-bit status word per workgroup (one workgroup per segment),
// then the state pass's parts (fused kernel, when split).
size_t fwd_flags_bytes(const tc_shape_t& s, const Plan& p) {
  return align256((size_t)s.B * s.H * p.nseg * sizeof(unsigned long long));
}
size_t fwd_ws_bytes(const tc_shape_t& s, const Plan& p) {
  return align256(p.state_bytes) + 2 * fwd_flags_bytes(s, p) + align256(p.parts_bytes);
}

// Flag value of one forward call: a per-process random salt combined with a
// call counter, so that flags left in a reused workspace by earlier calls,
// or arbitrary initial contents, do not match it.
unsigned long long next_generation() {
  static std::atomic<unsigned long long> counter{0};
  static const unsigned long long salt = [] {
    std::random_device rd;
    return ((unsigned long long)rd() << 32) ^ ((unsigned long long)rd() << 11) ^ 0x9E3779B97F4A7C15ull;
  }();
  return salt ^ (counter.fetch_add(1) + 1);
}

tc_status_t check_shape(const tc_shape_t* s) {
  if (!s) return TC_ERR_INVALID_ARGUMENT;
  if (s->B < 1 || s->H < 1 || s->T < 1 || s->W < 1 || s->C < 1 || s->D < 1)
    return TC_ERR_INVALID_ARGUMENT;
  if (!valid_dtype(s->dtype)) return TC_ERR_UNSUPPORTED;
  if (!supported_d(s->D)) return TC_ERR_UNSUPPORTED;
  if (!(s->scale == s->scale)) return TC_ERR_INVALID_ARGUMENT;  // NaN scale
  // index arithmetic is 32-bit inside a (b,h) sequence and 64-bit across
  if ((long long)(s->T + 128) * s->D * (long long)elem_size(s->dtype) > (1LL << 31) - 1)
    return TC_ERR_UNSUPPORTED;
  if ((long long)s->B * s->H > (1LL << 24)) return TC_ERR_UNSUPPORTED;
  return TC_OK;
}

float scale_of(float scale, int D) { return scale > 0.0f ? scale : 1.0f / sqrtf((float)D); }

// One forward launch over shape s (rows >= row0 stored, yadd added to them).
tc_status_t launch_fwd(const tc_shape_t& s, const Plan& p, const void* q, const void* k, const void* v,
                       const float* lambda, const float* eta, const float* gate, void* y, float* A_final,
                       float* lse, void* ws, bool ws_ok, int row0, const float* yadd, hipStream_t stream,
                       int mean_c = 0, const void* k_ring = nullptr, const void* v_ring = nullptr,
                       int ring_s0 = 0, const float* A_in = nullptr, int window_only = 0) {
  tck::FwdArgs a{};
  a.mean_c = mean_c;
  a.q = q;
  a.k = k;
  a.v = v;
  a.lam = lambda;
  a.eta = eta;
  a.gate = gate;
  a.y = y;
  a.A_final = A_final;
  a.lse = lse;
  a.seg_state = (float*)ws;
  a.flags = ws && ws_ok ? (unsigned long long*)((char*)ws + align256(p.state_bytes)) : nullptr;
  a.status = a.flags ? (unsigned long long*)((char*)a.flags + fwd_flags_bytes(s, p)) : nullptr;
  // (the parts follow the status words; the workspace is required whenever nseg > 1)
  a.nparts = (ws && ws_ok && p.nparts > 1) ? p.nparts : 1;
  a.parts = a.nparts > 1 ? (float*)((char*)a.status + fwd_flags_bytes(s, p)) : nullptr;
  a.gen = next_generation();
  a.B = s.B;
  a.H = s.H;
  a.T = s.T;
  a.W = s.W;
  a.nblk = p.nblk;
  a.j0 = p.j0;
  a.G = p.G;
  a.R = p.R;
  a.nseg = p.nseg;
  a.scale = scale_of(s.scale, s.D);
  a.row0 = row0;
  a.k_ring = k_ring;
  a.v_ring = v_ring;
  a.ring_s0 = ring_s0;
  a.yadd = yadd;
  a.A_in = A_in;
  a.window_only = window_only;
  const bool is_bf16 = s.dtype == TC_BF16;
  const hipError_t e = rows_kernel(s.D, s.dtype) ? tck::launch_forward_rows(a, s.D, is_bf16, stream)
                                                       : tck::launch_forward(a, s.D, is_bf16, stream);
  return e == hipSuccess ? TC_OK : TC_ERR_HIP;
}

// Byte extents of tc_forward's buffers, in the order q, k, v, lambda, eta,
// gate, y, A_final, lse (0 for a null optional output).
struct FwdExtents {
  size_t sz[9];
};
FwdExtents fwd_extents(const tc_shape_t& s, const float* A_final, const float* lse) {
  const size_t n = (size_t)s.B * s.H * s.T * s.D * elem_size(s.dtype);
  const size_t nh = (size_t)s.H * 4;
  return FwdExtents{{n, n, n, nh, nh, nh, n, A_final ? (size_t)s.B * s.H * s.D * s.D * 4 : 0,
                     lse ? (size_t)s.B * s.H * s.T * 4 : 0}};
}

// Argument checks of tc_forward and tc_forward_noalloc (everything but the
// workspace): the shape, required pointers, and no output overlapping an
// input or another output.
tc_status_t check_fwd_args(const tc_shape_t* s, const void* q, const void* k, const void* v, const float* lambda,
                           const float* eta, const float* gate, const void* y, const float* A_final,
                           const float* lse) {
  const tc_status_t st = check_shape(s);
  if (st != TC_OK) return st;
  if (!q || !k || !v || !lambda || !eta || !gate || !y) return TC_ERR_INVALID_ARGUMENT;
  const FwdExtents x = fwd_extents(*s, A_final, lse);
  const void* bufs[9] = {q, k, v, lambda, eta, gate, y, A_final, lse};
  for (int o = 6; o < 9; ++o) {
    for (int i = 0; i < 6; ++i)
      if (overlap(bufs[o], x.sz[o], bufs[i], x.sz[i])) return TC_ERR_INVALID_ARGUMENT;
    for (int p = o + 1; p < 9; ++p)
      if (overlap(bufs[o], x.sz[o], bufs[p], x.sz[p])) return TC_ERR_INVALID_ARGUMENT;
  }
  return TC_OK;
}

// Scratch of tc_forward_noalloc, for callers that cannot allocate: the
// forward workspace of any shape that needs at most kScratchBytes, in the
// device's own copy of `scratch`.  Host code never passes the array's name
// to a kernel (on the host it names a stand-in, not device memory): it takes
// the device address from hipGetSymbolAddress, once per device, with that
// device current, and keeps it per device.
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

// Continuation workspace: the forward's workspace for the extended shape,
// the initial-state read and the new evictions' state.
struct ContPlan {
  tc_shape_t x;  // extended shape (T = p + new tokens)
  Plan fp;
  int p;
  size_t off_fwd, off_yinit, off_anew, total;
};

tc_status_t cont_plan_for(const tc_shape_t* s, int64_t pos0, ContPlan& c) {
  const tc_status_t st = check_shape(s);
  if (st != TC_OK) return st;
  if (pos0 < 0) return TC_ERR_INVALID_ARGUMENT;
  c.p = pos0 < s->W ? (int)pos0 : s->W;
  c.x = *s;
  if ((long long)s->T + c.p > (1LL << 30)) return TC_ERR_UNSUPPORTED;
  c.x.T = s->T + c.p;
  const tc_status_t sx = check_shape(&c.x);
  if (sx != TC_OK) return sx;
  const long long BH = (long long)s->B * s->H;
  // grid of the preparation kernel: one workgroup per (b,h) and 128 new rows
  if (BH * ((s->T + 127) / 128) > (1LL << 31) - 1) return TC_ERR_UNSUPPORTED;
  c.fp = plan_for(c.x, c.p);
  c.off_fwd = 0;
  c.off_yinit = fwd_ws_bytes(c.x, c.fp);
  c.off_anew = c.off_yinit + align256((size_t)BH * s->T * s->D * 4);
  c.total = c.off_anew + align256((size_t)BH * s->D * s->D * 4);
  return TC_OK;
}

}  // namespace

extern "C" {

const char* tc_status_string(tc_status_t st) {
  // (read as an int: callers from other languages may pass any integer, and
  // loading an out-of-range value as the enum type is undefined in C++)
  int v = 0;
  static_assert(sizeof(st) == sizeof(v), "tc_status_t is int-sized");
  memcpy(&v, &st, sizeof(v));
  switch (v) {
    case TC_OK: return "ok";
    case TC_ERR_INVALID_ARGUMENT: return "invalid argument";
    case TC_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case TC_ERR_WORKSPACE: return "workspace missing or too small";
    case TC_ERR_HIP: return "HIP launch failed";
    case TC_ERR_STATE_EXCHANGE: return "a wait for another workgroup's state ran out (outputs hold NaN)";
  }
  return "unknown status";
}

const char* tc_version(void) { return "0.1.0"; }

size_t tc_forward_workspace_size(const tc_shape_t* s) {
  if (check_shape(s) != TC_OK) return 0;
  return fwd_ws_bytes(*s, plan_for(*s));
}

tc_status_t tc_forward(const tc_shape_t* s, const void* q, const void* k, const void* v,
                       const float* lambda, const float* eta, const float* gate, void* y,
                       float* A_final, float* lse, void* ws, size_t ws_bytes, void* stream) {
  const tc_status_t st = check_fwd_args(s, q, k, v, lambda, eta, gate, y, A_final, lse);
  if (st != TC_OK) return st;
  const Plan p = plan_for(*s);
  const size_t need = fwd_ws_bytes(*s, p);
  if (p.nseg > 1 && (!ws || ws_bytes < need)) return TC_ERR_WORKSPACE;
  if (ws && ws_bytes >= need) {
    const FwdExtents x = fwd_extents(*s, A_final, lse);
    const void* bufs[9] = {q, k, v, lambda, eta, gate, y, A_final, lse};
    for (int i = 0; i < 9; ++i)
      if (overlap(ws, need, bufs[i], x.sz[i])) return TC_ERR_INVALID_ARGUMENT;
  }
  return launch_fwd(*s, p, q, k, v, lambda, eta, gate, y, A_final, lse, ws, ws_bytes >= need, 0, nullptr,
                    (hipStream_t)stream);
}

tc_status_t tc_forward_chunk_mean(const tc_shape_t* s, const void* q, const void* k, const void* v,
                                  const float* lambda, const float* eta, const float* gate, void* y,
                                  float* A_final, float* lse, void* ws, size_t ws_bytes, void* stream) {
  const tc_status_t st = check_fwd_args(s, q, k, v, lambda, eta, gate, y, A_final, lse);
  if (st != TC_OK) return st;
  // built for the 128-row bf16 kernel, with chunks that tile its blocks
  if (s->dtype != TC_BF16 || s->D > 64 || (s->C != 64 && s->C != 128) || s->W % s->C != 0) return TC_ERR_UNSUPPORTED;
  const Plan p = plan_for(*s);
  const size_t need = fwd_ws_bytes(*s, p);
  if (p.nseg > 1 && (!ws || ws_bytes < need)) return TC_ERR_WORKSPACE;
  if (ws && ws_bytes >= need) {
    const FwdExtents x = fwd_extents(*s, A_final, lse);
    const void* bufs[9] = {q, k, v, lambda, eta, gate, y, A_final, lse};
    for (int i = 0; i < 9; ++i)
      if (overlap(ws, need, bufs[i], x.sz[i])) return TC_ERR_INVALID_ARGUMENT;
  }
  return launch_fwd(*s, p, q, k, v, lambda, eta, gate, y, A_final, lse, ws, ws_bytes >= need, 0, nullptr,
                    (hipStream_t)stream, s->C);
}

tc_status_t tc_forward_noalloc(const tc_shape_t* s, const void* q, const void* k, const void* v,
                               const float* lambda, const float* eta, const float* gate, void* y,
                               float* A_final, float* lse, void* stream) {
  const tc_status_t st = check_fwd_args(s, q, k, v, lambda, eta, gate, y, A_final, lse);
  if (st != TC_OK) return st;
  const Plan p = plan_for(*s);
  if (fwd_ws_bytes(*s, p) > kScratchBytes) return TC_ERR_WORKSPACE;
  void* w = scratch_ptr();
  if (!w) return TC_ERR_HIP;
  return launch_fwd(*s, p, q, k, v, lambda, eta, gate, y, A_final, lse, w, true, 0, nullptr, (hipStream_t)stream);
}

// Delta-rule workspace: the window-only forward's, then (float32) per chunk
// U'^T and Wm^T [D][64], M_c and B_c^T [D][D]; per group M_g and B_g^T; the
// group-start states and (D = 128) the chunk-start states; the memory read
// [BH][T][D]; with three levels also per supergroup its map, offset and start
// state.
//
// Level sizes.  A scan level of n maps in groups of g costs g steps in its
// group kernel (two products a step) and g in its expand kernel (one), each
// stretched by the share of the chip its BH ceil(n/g) workgroups overfill
// (the time of a step was measured flat up to about two 512-thread
// workgroups per compute unit, and growing in proportion beyond); the walk
// over the top level costs one product per map, and a third level two
// launches more.  The sizes minimise that cost (in product latencies).
constexpr double kDeltaSlots = 512.0;  // workgroups the chip runs at full per-step speed
struct DeltaPlan {
  Plan fp;
  int E, nch, G, ng, G2, nsg;
  size_t off_up, off_wm, off_mc, off_bc, off_mg, off_bg, off_ag, off_ac, off_ms, off_bs, off_as, off_yadd, total;
};
DeltaPlan delta_plan_for(const tc_shape_t& s) {
  DeltaPlan d;
  d.fp = plan_for(s);
  d.E = s.T > s.W ? s.T - s.W : 0;
  d.nch = (d.E + 63) / 64;
  const double heads = (double)s.B * s.H;
  auto level = [&](int n, int g) {  // group + expand steps of one level
    const int groups = (n + g - 1) / g;
    return 3.0 * g * std::max(1.0, heads * groups / kDeltaSlots);
  };
  d.G = 1;
  d.G2 = 0;
  double best = 1e30;
  for (int g = 1; g <= 64; ++g) {
    const int ng = (d.nch + g - 1) / g;
    const double two = level(d.nch, g) + ng;
    if (two < best) best = two, d.G = g, d.G2 = 0;
    for (int g2 = 2; g2 <= 32 && ng > 1; ++g2) {
      const double three = level(d.nch, g) + level(ng, g2) + (ng + g2 - 1) / g2 + 2.0;
      if (three < best) best = three, d.G = g, d.G2 = g2;
    }
  }
  d.ng = (d.nch + d.G - 1) / d.G;
  d.nsg = d.G2 > 0 ? (d.ng + d.G2 - 1) / d.G2 : 0;
  const size_t BH = (size_t)s.B * s.H, D = (size_t)s.D, DD = D * D * 4;
  d.off_up = align256(fwd_ws_bytes(s, d.fp));
  d.off_wm = d.off_up + align256(BH * d.nch * 64 * D * 4);
  d.off_mc = d.off_wm + align256(BH * d.nch * 64 * D * 4);
  d.off_bc = d.off_mc + align256(BH * d.nch * DD);
  d.off_mg = d.off_bc + align256(BH * d.nch * DD);
  d.off_bg = d.off_mg + align256(BH * d.ng * DD);
  d.off_ag = d.off_bg + align256(BH * d.ng * DD);
  d.off_ac = d.off_ag + align256(BH * (d.ng + 1) * DD);
  // (D <= 64: the last expansion and the read run fused, A_c is never stored)
  d.off_ms = d.off_ac + (s.D <= 64 ? 0 : align256(BH * d.nch * DD));
  d.off_bs = d.off_ms + align256(BH * d.nsg * DD);
  d.off_as = d.off_bs + align256(BH * d.nsg * DD);
  d.off_yadd = d.off_as + (d.nsg > 0 ? align256(BH * (d.nsg + 1) * DD) : 0);
  d.total = d.off_yadd + align256(BH * s.T * D * 4);
  return d;
}

size_t tc_forward_delta_workspace_size(const tc_shape_t* s) {
  if (check_shape(s) != TC_OK) return 0;
  return delta_plan_for(*s).total;
}

tc_status_t tc_forward_delta(const tc_shape_t* s, const void* q, const void* k, const void* v, const float* lambda,
                             const float* eta, const float* gate, void* y, float* A_final, float* lse, void* ws,
                             size_t ws_bytes, void* stream) {
  const tc_status_t st = check_fwd_args(s, q, k, v, lambda, eta, gate, y, A_final, lse);
  if (st != TC_OK) return st;
  const DeltaPlan d = delta_plan_for(*s);
  if (!ws || ws_bytes < d.total) return TC_ERR_WORKSPACE;
  const FwdExtents x = fwd_extents(*s, A_final, lse);
  const void* bufs[9] = {q, k, v, lambda, eta, gate, y, A_final, lse};
  for (int i = 0; i < 9; ++i)
    if (overlap(ws, d.total, bufs[i], x.sz[i])) return TC_ERR_INVALID_ARGUMENT;
  char* w = (char*)ws;
  tck::DeltaArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.lam = lambda;
  a.eta = eta;
  a.gate = gate;
  a.UpT = (float*)(w + d.off_up);
  a.WmT = (float*)(w + d.off_wm);
  a.Mc = (float*)(w + d.off_mc);
  a.BcT = (float*)(w + d.off_bc);
  a.Mg = (float*)(w + d.off_mg);
  a.BgT = (float*)(w + d.off_bg);
  a.AgT = (float*)(w + d.off_ag);
  a.AcT = (float*)(w + d.off_ac);
  a.Ms = (float*)(w + d.off_ms);
  a.BsT = (float*)(w + d.off_bs);
  a.AsT = (float*)(w + d.off_as);
  a.yadd = (float*)(w + d.off_yadd);
  a.A_final = A_final;
  a.B = s->B;
  a.H = s->H;
  a.T = s->T;
  a.W = s->W;
  a.E = d.E;
  a.nch = d.nch;
  a.G = d.G;
  a.ng = d.ng;
  a.G2 = d.G2;
  a.nsg = d.nsg;
  if (tck::launch_delta_memory(a, s->D, s->dtype == TC_BF16, (hipStream_t)stream) != hipSuccess) return TC_ERR_HIP;
  // y = y_local + sigma(g) m, rounded once (the window-only forward adds the read)
  return launch_fwd(*s, d.fp, q, k, v, lambda, eta, gate, y, nullptr, lse, ws, true, 0, a.yadd, (hipStream_t)stream,
                    0, nullptr, nullptr, 0, nullptr, 1);
}

size_t tc_continue_workspace_size(const tc_shape_t* s, int64_t pos0) {
  ContPlan c;
  if (cont_plan_for(s, pos0, c) != TC_OK) return 0;
  return c.total;
}

tc_status_t tc_forward_status(const tc_shape_t* s, int64_t pos0, const void* ws, size_t ws_bytes, void* stream) {
  ContPlan c;
  const tc_status_t st = cont_plan_for(s, pos0, c);
  if (st != TC_OK) return st;
  // the status words sit after the states and flags of the forward part
  // (for pos0 = 0 this is exactly tc_forward's workspace layout)
  const size_t n = (size_t)s->B * s->H * c.fp.nseg;
  const size_t off = align256(c.fp.state_bytes) + fwd_flags_bytes(c.x, c.fp);
  if (!ws) return c.fp.nseg > 1 ? TC_ERR_WORKSPACE : TC_OK;  // one segment: no waits, no workspace needed
  if (ws_bytes < off + n * sizeof(unsigned long long)) return TC_ERR_WORKSPACE;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return TC_ERR_HIP;
  std::vector<unsigned long long> w(n);
  if (hipMemcpy(w.data(), (const char*)ws + off, n * sizeof(unsigned long long), hipMemcpyDeviceToHost) != hipSuccess)
    return TC_ERR_HIP;
  for (size_t i = 1; i < n; ++i)
    if (w[i] != w[0]) return TC_ERR_STATE_EXCHANGE;
  return TC_OK;
}

tc_status_t tc_forward_continue(const tc_shape_t* s, int64_t pos0, const void* q, const void* k, const void* v,
                                const float* lambda, const float* eta, const float* gate, void* k_ring,
                                void* v_ring, float* A, int64_t* pos, void* y, float* lse, void* ws,
                                size_t ws_bytes, void* stream) {
  ContPlan c;
  const tc_status_t st = cont_plan_for(s, pos0, c);
  if (st != TC_OK) return st;
  if (!q || !k || !v || !lambda || !eta || !gate || !k_ring || !v_ring || !A || !y)
    return TC_ERR_INVALID_ARGUMENT;
  const void* al[9] = {q, k, v, k_ring, v_ring, A, y, lse, ws};
  for (int i = 0; i < 9; ++i)
    if ((uintptr_t)al[i] % 16) return TC_ERR_INVALID_ARGUMENT;  // 16-byte vector copies
  if (!ws || ws_bytes < c.total) return TC_ERR_WORKSPACE;
  const size_t es = elem_size(s->dtype);
  const size_t n = (size_t)s->B * s->H * s->T * s->D * es;
  const size_t nr = (size_t)s->B * s->H * s->W * s->D * es;
  const size_t na = (size_t)s->B * s->H * s->D * s->D * 4;
  const size_t np = pos ? (size_t)s->B * 8 : 0;
  const size_t nl = lse ? (size_t)s->B * s->H * s->T * 4 : 0;
  const size_t nh = (size_t)s->H * 4;
  const void* ins[6] = {q, k, v, lambda, eta, gate};
  const size_t insz[6] = {n, n, n, nh, nh, nh};
  void* outs[7] = {k_ring, v_ring, A, pos, y, lse, ws};
  const size_t outsz[7] = {nr, nr, na, np, n, nl, c.total};
  for (int o = 0; o < 7; ++o) {
    for (int i = 0; i < 6; ++i)
      if (overlap(outs[o], outsz[o], ins[i], insz[i])) return TC_ERR_INVALID_ARGUMENT;
    for (int p = o + 1; p < 7; ++p)
      if (overlap(outs[o], outsz[o], outs[p], outsz[p])) return TC_ERR_INVALID_ARGUMENT;
  }
  char* w = (char*)ws;
  tck::ContArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.k_ring = k_ring;
  a.v_ring = v_ring;
  a.A = A;
  a.pos = pos;
  a.lam = lambda;
  a.gate = gate;
  a.yinit = (float*)(w + c.off_yinit);
  a.A_new = (const float*)(w + c.off_anew);
  a.pos0 = pos0;
  a.B = s->B;
  a.H = s->H;
  a.T = s->T;
  a.W = s->W;
  a.D = s->D;
  a.p = c.p;
  a.Tx = c.x.T;
  a.esize = (int)es;
  // Once the window is full (pos0 >= W) and W is a multiple of the forward's
  // block rows, every processed block starts at or after eviction 0 of the
  // extended sequence and the forward starts its scan from A (S(0) = A/eta);
  // otherwise the read of A is formed here (yinit) and A is combined at the end.
  a.fold = (pos0 >= s->W && s->W % fwd_block(s->D, s->dtype) == 0) ? 1 : 0;
  hipError_t e = tck::launch_continue_prep(a, (hipStream_t)stream);
  if (e != hipSuccess) return TC_ERR_HIP;
  // rows below p: ring slots (pos0 - p + r) mod W
  const int s0 = (int)((pos0 - c.p) % s->W);
  if (launch_fwd(c.x, c.fp, q, k, v, lambda, eta, gate, y, (float*)(w + c.off_anew), lse, w + c.off_fwd, true, c.p,
                 a.fold ? nullptr : a.yinit, (hipStream_t)stream, 0, k_ring, v_ring, s0, a.fold ? A : nullptr) != TC_OK)
    return TC_ERR_HIP;
  e = tck::launch_continue_finish(a, (hipStream_t)stream);
  return e == hipSuccess ? TC_OK : TC_ERR_HIP;
}

tc_status_t tc_decode_step(const tc_decode_shape_t* s, const void* q, const void* k, const void* v,
                           void* k_ring, void* v_ring, float* A, int64_t* pos, const float* lambda,
                           const float* eta, const float* gate, void* y, void* stream) {
  if (!s) return TC_ERR_INVALID_ARGUMENT;
  if (s->S < 1 || s->H < 1 || s->W < 1 || s->D < 1) return TC_ERR_INVALID_ARGUMENT;
  if (!valid_dtype(s->dtype) || !supported_d(s->D)) return TC_ERR_UNSUPPORTED;
  if (!(s->scale == s->scale)) return TC_ERR_INVALID_ARGUMENT;
  if ((long long)s->S * s->H > (1LL << 30)) return TC_ERR_UNSUPPORTED;
  // byte offsets inside one (stream, head) ring are 32-bit
  if ((long long)(s->W + 512) * s->D * (long long)elem_size(s->dtype) > (1LL << 31) - 1) return TC_ERR_UNSUPPORTED;
  if (!q || !k || !v || !k_ring || !v_ring || !A || !pos || !lambda || !eta || !gate || !y)
    return TC_ERR_INVALID_ARGUMENT;
  const size_t es = elem_size(s->dtype);
  const size_t nt = (size_t)s->S * s->H * s->D * es;
  const size_t nr = (size_t)s->S * s->H * s->W * s->D * es;
  const size_t na = (size_t)s->S * s->H * s->D * s->D * 4;
  const size_t np = (size_t)s->S * 8;
  const size_t nh = (size_t)s->H * 4;
  const void* ins[6] = {q, k, v, lambda, eta, gate};
  const size_t insz[6] = {nt, nt, nt, nh, nh, nh};
  void* outs[5] = {k_ring, v_ring, A, pos, y};
  const size_t outsz[5] = {nr, nr, na, np, nt};
  for (int o = 0; o < 5; ++o) {
    for (int i = 0; i < 6; ++i)
      if (overlap(outs[o], outsz[o], ins[i], insz[i])) return TC_ERR_INVALID_ARGUMENT;
    for (int p = o + 1; p < 5; ++p)
      if (overlap(outs[o], outsz[o], outs[p], outsz[p])) return TC_ERR_INVALID_ARGUMENT;
  }
  tck::DecArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.k_ring = k_ring;
  a.v_ring = v_ring;
  a.A = A;
  a.pos = pos;
  a.lam = lambda;
  a.eta = eta;
  a.gate = gate;
  a.y = y;
  a.S = s->S;
  a.H = s->H;
  a.W = s->W;
  a.scale = scale_of(s->scale, s->D);
  const hipError_t e = tck::launch_decode(a, s->D, s->dtype == TC_BF16, (hipStream_t)stream);
  return e == hipSuccess ? TC_OK : TC_ERR_HIP;
}

struct BwdPlan {
  int nblk, G, nseg;
  size_t off_f, off_t, off_r, off_delta, off_part, total;
};

BwdPlan bwd_plan_for(const tc_shape_t& s) {
  BwdPlan p;
  const long long BH = (long long)s.B * s.H;
  p.nblk = (s.T + kBlock - 1) / kBlock;
  // the gradient kernels run one workgroup per compute unit (256): segments
  // long enough for one round (measured faster than two rounds of half the
  // length: fewer start-ups per unit)
  long long G = (BH * p.nblk + 255) / 256;
  if (G < 1) G = 1;
  if (G > p.nblk) G = p.nblk;
  p.G = (int)G;
  p.nseg = (p.nblk + p.G - 1) / p.G;
  const size_t st = align256((size_t)BH * p.nseg * s.D * s.D * sizeof(float));
  p.off_f = 0;
  p.off_t = p.off_f + st;
  p.off_r = p.off_t + st;
  p.off_delta = p.off_r + st;
  p.off_part = p.off_delta + align256((size_t)BH * s.T * sizeof(float));
  p.total = p.off_part + align256((size_t)BH * p.nseg * 2 * sizeof(float));
  return p;
}

size_t tc_backward_workspace_size(const tc_shape_t* s) {
  if (check_shape(s) != TC_OK) return 0;
  return bwd_plan_for(*s).total;
}

tc_status_t tc_backward(const tc_shape_t* s, const void* q, const void* k, const void* v,
                        const void* y, const void* dy, const float* lse, const float* lambda,
                        const float* eta, const float* gate, void* dq, void* dk, void* dv,
                        float* dlambda, float* deta, float* dgate, void* ws, size_t ws_bytes,
                        void* stream) {
  const tc_status_t st = check_shape(s);
  if (st != TC_OK) return st;
  if (!q || !k || !v || !y || !dy || !lse || !lambda || !eta || !gate || !dq || !dk || !dv ||
      !dlambda || !deta || !dgate)
    return TC_ERR_INVALID_ARGUMENT;
  const BwdPlan p = bwd_plan_for(*s);
  if (!ws || ws_bytes < p.total) return TC_ERR_WORKSPACE;
  const size_t n = (size_t)s->B * s->H * s->T * s->D * elem_size(s->dtype);
  const size_t nl = (size_t)s->B * s->H * s->T * 4;
  const size_t nh = (size_t)s->H * 4;
  const void* ins[9] = {q, k, v, y, dy, lse, lambda, eta, gate};
  const size_t insz[9] = {n, n, n, n, n, nl, nh, nh, nh};
  void* outs[7] = {dq, dk, dv, dlambda, deta, dgate, ws};
  const size_t outsz[7] = {n, n, n, nh, nh, nh, p.total};
  for (int o = 0; o < 7; ++o) {
    for (int i = 0; i < 9; ++i)
      if (overlap(outs[o], outsz[o], ins[i], insz[i])) return TC_ERR_INVALID_ARGUMENT;
    for (int q2 = o + 1; q2 < 7; ++q2)
      if (overlap(outs[o], outsz[o], outs[q2], outsz[q2])) return TC_ERR_INVALID_ARGUMENT;
  }
  char* w = (char*)ws;
  tck::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.y = y;
  a.dy = dy;
  a.lse = lse;
  a.lam = lambda;
  a.eta = eta;
  a.gate = gate;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dlam = dlambda;
  a.deta = deta;
  a.dgate = dgate;
  a.fstate = (float*)(w + p.off_f);
  a.tstate = (float*)(w + p.off_t);
  a.rstate = (float*)(w + p.off_r);
  a.delta = (float*)(w + p.off_delta);
  a.part = (float*)(w + p.off_part);
  a.B = s->B;
  a.H = s->H;
  a.T = s->T;
  a.W = s->W;
  a.nblk = p.nblk;
  a.G = p.G;
  a.nseg = p.nseg;
  a.scale = scale_of(s->scale, s->D);
  const hipError_t e = tck::launch_backward(a, s->D, s->dtype == TC_BF16, (hipStream_t)stream);
  return e == hipSuccess ? TC_OK : TC_ERR_HIP;
}

}  // extern "C"

// C ABI of the TC layer: host-side validation, workspace planning and
// dispatch to the gfx950 kernels.  No allocation and no synchronisation;
// the only global state is a call counter (the forward's flag values) and,
// in the rows launcher, a per-device count of resident workgroups.
#include <math.h>

#include <atomic>
#include <random>
#include <stdint.h>
#include <string.h>

#include "../../include/tc.h"
#include "tc_launch.h"

namespace {

constexpr int kBlock = 64;  // backward: query rows per block = tokens per scan chunk

// Query rows per block of the forward kernels: 128 (four waves of 32 rows)
// for bf16 with D <= 64, else 64 (four waves of 16 rows).  The float32 path keeps the 64-row kernel: it runs at two
// workgroups per compute unit with every accumulator in VGPRs (see the
// 16x16x4 float32 note in tc_forward.hip).
int fwd_block(int D, int32_t dtype) { return (D <= 64 && dtype == TC_BF16) ? 128 : 64; }

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
  p.nseg = (nb + bestG - 1) / bestG;
  if (BH * p.nseg <= slots) {
    const long long fill = slots / BH < nb ? slots / BH : nb;
    if (fill > p.nseg) p.nseg = (int)fill;
  }
  p.G = nb / p.nseg;
  p.R = nb - p.G * p.nseg;
  // segment states, then one last-block local state per (b,h)
  p.state_bytes = (size_t)BH * (p.nseg + 1) * s.D * s.D * sizeof(float);
  return p;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Forward workspace: the segment states, then one 64-bit flag per segment.
size_t fwd_flags_bytes(const tc_shape_t& s, const Plan& p) {
  return align256((size_t)s.B * s.H * p.nseg * sizeof(unsigned long long));
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
                       float* lse, void* ws, bool ws_ok, int row0, const float* yadd, hipStream_t stream) {
  tck::FwdArgs a{};
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
  a.yadd = yadd;
  const bool is_bf16 = s.dtype == TC_BF16;
  const hipError_t e = fwd_block(s.D, s.dtype) == 128 ? tck::launch_forward_rows(a, s.D, is_bf16, stream)
                                                       : tck::launch_forward(a, s.D, is_bf16, stream);
  return e == hipSuccess ? TC_OK : TC_ERR_HIP;
}

// Continuation workspace: the forward's workspace for the extended shape,
// the extended q/k/v, the initial-state read and the new evictions' state.
struct ContPlan {
  tc_shape_t x;  // extended shape (T = p + new tokens)
  Plan fp;
  int p;
  size_t off_fwd, off_q, off_k, off_v, off_yinit, off_anew, total;
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
  // grid of the preparation kernel: one workgroup per (b,h) and 128 new rows, plus up to 8192 copy workgroups
  if (BH * ((s->T + 127) / 128) > (1LL << 31) - 1 - 8192) return TC_ERR_UNSUPPORTED;
  c.fp = plan_for(c.x, c.p);
  const size_t es = elem_size(s->dtype);
  const size_t nx = align256((size_t)BH * c.x.T * s->D * es);
  c.off_fwd = 0;
  c.off_q = align256(c.fp.state_bytes) + fwd_flags_bytes(c.x, c.fp);
  c.off_k = c.off_q + nx;
  c.off_v = c.off_k + nx;
  c.off_yinit = c.off_v + nx;
  c.off_anew = c.off_yinit + align256((size_t)BH * s->T * s->D * 4);
  c.total = c.off_anew + align256((size_t)BH * s->D * s->D * 4);
  return TC_OK;
}

}  // namespace

extern "C" {

const char* tc_status_string(tc_status_t st) {
  switch (st) {
    case TC_OK: return "ok";
    case TC_ERR_INVALID_ARGUMENT: return "invalid argument";
    case TC_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case TC_ERR_WORKSPACE: return "workspace missing or too small";
    case TC_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

const char* tc_version(void) { return "0.1.0"; }

size_t tc_forward_workspace_size(const tc_shape_t* s) {
  if (check_shape(s) != TC_OK) return 0;
  const Plan p = plan_for(*s);
  return align256(p.state_bytes) + fwd_flags_bytes(*s, p);
}

tc_status_t tc_forward(const tc_shape_t* s, const void* q, const void* k, const void* v,
                       const float* lambda, const float* eta, const float* gate, void* y,
                       float* A_final, float* lse, void* ws, size_t ws_bytes, void* stream) {
  const tc_status_t st = check_shape(s);
  if (st != TC_OK) return st;
  if (!q || !k || !v || !lambda || !eta || !gate || !y) return TC_ERR_INVALID_ARGUMENT;
  const size_t n = (size_t)s->B * s->H * s->T * s->D * elem_size(s->dtype);
  const size_t na = A_final ? (size_t)s->B * s->H * s->D * s->D * 4 : 0;
  const size_t nl = lse ? (size_t)s->B * s->H * s->T * 4 : 0;
  const size_t nh = (size_t)s->H * 4;
  const void* ins[6] = {q, k, v, lambda, eta, gate};
  const size_t insz[6] = {n, n, n, nh, nh, nh};
  void* outs[3] = {y, A_final, lse};
  const size_t outsz[3] = {n, na, nl};
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 6; ++i)
      if (overlap(outs[o], outsz[o], ins[i], insz[i])) return TC_ERR_INVALID_ARGUMENT;
    for (int p = o + 1; p < 3; ++p)
      if (overlap(outs[o], outsz[o], outs[p], outsz[p])) return TC_ERR_INVALID_ARGUMENT;
  }
  const Plan p = plan_for(*s);
  const size_t need = align256(p.state_bytes) + fwd_flags_bytes(*s, p);
  if (p.nseg > 1 && (!ws || ws_bytes < need)) return TC_ERR_WORKSPACE;
  if (ws && ws_bytes >= need) {
    for (int o = 0; o < 3; ++o)
      if (overlap(ws, need, outs[o], outsz[o])) return TC_ERR_INVALID_ARGUMENT;
    for (int i = 0; i < 6; ++i)
      if (overlap(ws, need, ins[i], insz[i])) return TC_ERR_INVALID_ARGUMENT;
  }
  return launch_fwd(*s, p, q, k, v, lambda, eta, gate, y, A_final, lse, ws, ws_bytes >= need, 0, nullptr,
                    (hipStream_t)stream);
}

size_t tc_continue_workspace_size(const tc_shape_t* s, int64_t pos0) {
  ContPlan c;
  if (cont_plan_for(s, pos0, c) != TC_OK) return 0;
  return c.total;
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
  a.qx = w + c.off_q;
  a.kx = w + c.off_k;
  a.vx = w + c.off_v;
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
  hipError_t e = tck::launch_continue_prep(a, (hipStream_t)stream);
  if (e != hipSuccess) return TC_ERR_HIP;
  if (launch_fwd(c.x, c.fp, a.qx, a.kx, a.vx, lambda, eta, gate, y, (float*)(w + c.off_anew), lse,
                 w + c.off_fwd, true, c.p, a.yinit, (hipStream_t)stream) != TC_OK)
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

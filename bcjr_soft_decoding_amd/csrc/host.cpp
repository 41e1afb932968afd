// Host layer of the C ABI (include/bcjr.h): argument validation, size queries and dispatch.
// Every check runs before anything touches the HIP runtime, so the error paths need no device.
#include <hip/hip_runtime.h>

#include <math.h>

#include "bcjr.h"
#include "geom.h"
#include "internal.h"

namespace bcjr {

bool sparse_geom(int n, int k, int64_t B, int kind, SparseGeom* g) {
  if (!geom_supported(n, k) || !sparse_shape_built(n, k)) return false;
  g->n = n;
  g->k = k;
  g->K = 1 << k;
  g->S = 1 << n;
  g->M = g->S / g->K;
  g->NG = geom_ng(n, k);
  g->G = geom_g(n, k, kind);
  g->LPS = geom_lps(n, k, kind);
  g->SPB = geom_spb(n, k, kind);
  g->BLOCK = geom_block(n, k, kind);
  g->B = B;
  g->units = B > 0 ? (B + g->SPB - 1) / g->SPB : 0;
  const int64_t mx = geom_max_slots(n, k, kind);
  g->slots = g->units < mx ? g->units : mx;
  return true;
}

// Persistent grid: every block must be resident at once (each loops over its chain units),
// so the grid is the smaller of the workspace slots and the device's resident capacity for
// this kernel (occupancy x compute units).
int resident_grid(const void* kernel, int block, int64_t slots) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, block, 0) != hipSuccess) return -1;
  const int64_t cap = (int64_t)(per_cu > 0 ? per_cu : 1) * (cus > 0 ? cus : 1);
  return (int)(slots < cap ? slots : cap);
}

namespace {
size_t fwd_ws_one(const SparseGeom& g, int64_t L, bool ckpt) {
  return (size_t)g.slots * sparse_fwd_slot_bytes(g, L, ckpt);
}
size_t bwd_ws_one(const SparseGeom& g, int64_t L, bool ckpt) {
  return (size_t)g.slots * sparse_bwd_slot_bytes(g, L, ckpt) +
         round256((size_t)g.slots * g.S * sizeof(float));
}
}  // namespace

// The forward and backward workspaces hold the largest of the layouts the launch may take:
// the target geometry (or, for small batches, the spread one) and the fp64-message one.
size_t sparse_fwd_ws_bytes(const SparseGeom& g, int64_t L, bool ckpt) {
  size_t need = fwd_ws_one(g, L, ckpt);
  SparseGeom p;
  if (sparse_geom(g.n, g.k, g.B, kFwdP, &p)) {
    const size_t q = fwd_ws_one(p, L, ckpt);
    if (q > need) need = q;
  }
  if (geom_spread(g.n, g.k, g.B, kFwd) && sparse_geom(g.n, g.k, g.B, kFwdS, &p)) {
    const size_t q = fwd_ws_one(p, L, ckpt);
    if (q > need) need = q;
  }
  return need;
}
size_t sparse_bwd_ws_bytes(const SparseGeom& g, int64_t L, bool ckpt) {
  size_t need = bwd_ws_one(g, L, ckpt);
  SparseGeom p;
  if (sparse_geom(g.n, g.k, g.B, kBwdP, &p)) {
    const size_t q = bwd_ws_one(p, L, ckpt);
    if (q > need) need = q;
  }
  if (geom_spread(g.n, g.k, g.B, kBwd) && sparse_geom(g.n, g.k, g.B, kBwdS, &p)) {
    const size_t q = bwd_ws_one(p, L, ckpt);
    if (q > need) need = q;
  }
  return need;
}
size_t sparse_vit_ws_bytes(const SparseGeom& g, int64_t L) {
  return round256((size_t)g.slots * L * g.BLOCK * (g.K * g.G));
}

}  // namespace bcjr

using namespace bcjr;

namespace {

bool shape_ok(const bcjr_trellis* tr) {
  return tr->state_bits >= 1 && tr->state_bits <= 16 && tr->bits_per_step >= 1 &&
         tr->bits_per_step <= tr->state_bits;
}

// Common validation. On success fills *g (for B > 0) and returns BCJR_OK.
// B * L is bounded by 2^40 (L alone too), which keeps every element offset, workspace size and
// history size of the sparse kernels exact in 64-bit arithmetic.
bool chains_ok(int64_t B, int64_t L) {
  return B >= 0 && L >= 1 && L <= ((int64_t)1 << 40) && (B == 0 || B <= ((int64_t)1 << 40) / L);
}

bcjr_status check_common(const bcjr_trellis* tr, int64_t B, int64_t L, int kind, SparseGeom* g) {
  if (tr == nullptr) return BCJR_E_ARG;
  if (!shape_ok(tr) || !chains_ok(B, L)) return BCJR_E_SHAPE;
  if (tr->weights_per_step != 1) return BCJR_E_UNSUPPORTED;
  if (!sparse_geom(tr->state_bits, tr->bits_per_step, B, kind, g)) return BCJR_E_UNSUPPORTED;
  if (B > 0 && tr->codebook == nullptr) return BCJR_E_ARG;
  return BCJR_OK;
}

bool temp_ok(float T) { return isfinite(T) && T > 0.0f; }

// Each state size meets the tolerances down to its floor (geom_floor_t) and is refused below it.
bool temp_supported(const bcjr_trellis* tr, float T) {
  return T >= geom_floor_t(tr->state_bits, tr->bits_per_step);
}

// Workspaces are accessed with 16-byte vector loads and stores.
bool ws_ok(const void* ws, size_t have, size_t need) {
  return ws != nullptr && have >= need && ((uintptr_t)ws & 15) == 0;
}

// History layout from the workspace the caller passed: the full history when it fits, else the
// checkpointed one, else an error.
bcjr_status pick_layout(const void* ws, size_t have, size_t need_full, size_t need_ckpt, bool* ckpt) {
  if (ws_ok(ws, have, need_full)) {
    *ckpt = false;
    return BCJR_OK;
  }
  if (ws_ok(ws, have, need_ckpt)) {
    *ckpt = true;
    return BCJR_OK;
  }
  return BCJR_E_WORKSPACE;
}

bcjr_status from_hip(int e) { return e == 0 ? BCJR_OK : BCJR_E_DEVICE; }

// Dense shapes: S >= 1, B >= 0, L >= 1, and every [B, L, S] array addressable with 64-bit
// offsets (B * L * S * 16 bytes below 2^62).
bcjr_status dense_check(int32_t S, int64_t B, int64_t L) {
  if (S < 1 || S > 65536 || B < 0 || L < 1) return BCJR_E_SHAPE;
  if (B > 0 && (L > ((int64_t)1 << 40) / B || B * L > ((int64_t)1 << 58) / S)) return BCJR_E_SHAPE;
  if (!dense_shape_built(S)) return BCJR_E_UNSUPPORTED;
  return BCJR_OK;
}

// Segmented forward: validation shared by the size queries and the call (no device use).
bcjr_status scan_setup(const bcjr_trellis* tr, int64_t B, int64_t L, int64_t seg_len,
                       ScanPlan* plan) {
  if (tr == nullptr) return BCJR_E_ARG;
  if (!shape_ok(tr) || B < 0 || L < 1) return BCJR_E_SHAPE;
  if (tr->weights_per_step != 1) return BCJR_E_UNSUPPORTED;
  if (seg_len < 0) return BCJR_E_ARG;
  const int n = tr->state_bits, k = tr->bits_per_step;
  if (!scan_shape_built(n, k)) return BCJR_E_UNSUPPORTED;
  const int64_t M = ((int64_t)1 << n) >> k;
  if (B > ((int64_t)1 << 40) / L) return BCJR_E_SHAPE;
  const int64_t seg = seg_len > 0 ? seg_len : scan_default_seg(n, k, B, L);
  const int64_t s_eff = seg < L ? seg : L;
  const int64_t pmain = L / s_eff;
  const int64_t ptot = pmain + (L % s_eff ? 1 : 0);
  if (B > 0 && ptot > ((int64_t)1 << 56) / M / M / B) return BCJR_E_SHAPE;
  // the segments run with the segment geometry (fp32 messages) or the fp64 one; the plan's
  // history sizes take the larger of the two (sparse_fwd_ws_bytes)
  SparseGeom gm, gt;
  if (!sparse_geom(n, k, B * pmain, kFwdS, &gm) || !sparse_geom(n, k, B, kFwdS, &gt))
    return BCJR_E_UNSUPPORTED;
  scan_plan(gm, gt, n, k, B, L, seg, plan);
  return BCJR_OK;
}

// Backward plan; the partial slots cover both message precisions' geometries of both launches.
bcjr_status scan_setup_bwd(const bcjr_trellis* tr, int64_t B, int64_t L, int64_t seg_len,
                           ScanPlan* plan) {
  ScanPlan f;
  bcjr_status st = scan_setup(tr, B, L, seg_len, &f);
  if (st != BCJR_OK) return st;
  const int n = tr->state_bits, k = tr->bits_per_step;
  SparseGeom gm, gt, pm, pt;
  if (!sparse_geom(n, k, B * f.pmain, kBwdS, &gm) || !sparse_geom(n, k, B, kBwdS, &gt) ||
      !sparse_geom(n, k, B * f.pmain, kBwdP, &pm) || !sparse_geom(n, k, B, kBwdP, &pt))
    return BCJR_E_UNSUPPORTED;
  const int64_t slots = (gm.slots > pm.slots ? gm.slots : pm.slots) +
                        (gt.slots > pt.slots ? gt.slots : pt.slots);
  scan_plan_bwd(gm, gt, slots, n, k, B, L, f.seg, plan);
  return BCJR_OK;
}

}  // namespace

extern "C" {

size_t bcjr_scan_backward_workspace_bytes(const bcjr_trellis* tr, int64_t B, int64_t L,
                                          int64_t seg_len) {
  ScanPlan plan;
  if (scan_setup_bwd(tr, B, L, seg_len, &plan) != BCJR_OK || B == 0) return 0;
  return plan.bytes;
}

bcjr_status bcjr_backward_scan(const bcjr_trellis* tr, const float* w, int64_t B, int64_t L,
                               float T, int64_t seg_len, const float* w_hat,
                               const float* grad_w_hat, const float* grad_log_z, float* grad_w,
                               float* grad_codebook, void* ws, size_t ws_bytes,
                               bcjr_stream_t stream) {
  ScanPlan plan;
  bcjr_status st = scan_setup_bwd(tr, B, L, seg_len, &plan);
  if (st != BCJR_OK) return st;
  if (!temp_ok(T)) return BCJR_E_ARG;
  if (!temp_supported(tr, T)) return BCJR_E_UNSUPPORTED;
  if (grad_codebook == nullptr || tr->codebook == nullptr) return BCJR_E_ARG;
  if (B == 0)
    return from_hip(launch_fill_zero(grad_codebook, (int64_t)1 << tr->state_bits, stream));
  if (!w || !w_hat || !grad_w_hat || !grad_w) return BCJR_E_ARG;
  if (!ws_ok(ws, ws_bytes, plan.bytes)) return BCJR_E_WORKSPACE;
  const int n = tr->state_bits, k = tr->bits_per_step;
  const int M = (1 << n) >> k, S = 1 << n;
  char* base = static_cast<char*>(ws);
  SegLaunch sl{plan.pmain, 0, plan.seg, L, plan.ptot,
               reinterpret_cast<const double*>(base + plan.lam0),
               reinterpret_cast<const double*>(base + plan.rho1),
               reinterpret_cast<const double*>(base + plan.sc0),
               reinterpret_cast<float*>(base + plan.rows),
               reinterpret_cast<double*>(base + plan.rscale),
               reinterpret_cast<const float*>(base + plan.phi0),
               reinterpret_cast<const float*>(base + plan.psi1),
               reinterpret_cast<float*>(base + plan.frows)};
  float* partial = reinterpret_cast<float*>(base + plan.partial);
  void* slots = base + plan.slots;
  int e = 0, g1 = 0, g2 = 0;
  // phase 1: transfer and moment rows of every segment
  if (plan.ptot > 1) {
    e = launch_sparse_backward_seg(2, n, k, tr->codebook, w, B * plan.pmain * M, plan.seg, T,
                                   w_hat, grad_w_hat, grad_log_z, grad_w, partial, slots, sl, &g1,
                                   stream);
    if (e == 0 && plan.tail > 0) {
      SegLaunch st2 = sl;
      st2.nseg = 1;
      st2.jbase = plan.pmain;
      e = launch_sparse_backward_seg(2, n, k, tr->codebook, w, B * M, plan.tail, T, w_hat,
                                     grad_w_hat, grad_log_z, grad_w, partial, slots, st2, &g2,
                                     stream);
    }
  }
  // phase 2: messages and conditional expectations at every segment boundary
  if (e == 0)
    e = launch_scan_bounds(sl.rows, sl.rscale, sl.frows, B, plan.ptot, M,
                           reinterpret_cast<double*>(base + plan.lam0),
                           reinterpret_cast<double*>(base + plan.rho1),
                           reinterpret_cast<double*>(base + plan.sc0),
                           reinterpret_cast<float*>(base + plan.phi0),
                           reinterpret_cast<float*>(base + plan.psi1), slots,
                           plan.bytes - plan.slots, stream);  // (the slots are free in phase 2)
  // phase 3: every segment's gradient from its boundary values, then the codebook partials
  g1 = g2 = 0;
  if (e == 0)
    e = launch_sparse_backward_seg(1, n, k, tr->codebook, w, B * plan.pmain, plan.seg, T, w_hat,
                                   grad_w_hat, grad_log_z, grad_w, partial, slots, sl, &g1,
                                   stream);
  if (e == 0 && plan.tail > 0) {
    SegLaunch st2 = sl;
    st2.nseg = 1;
    st2.jbase = plan.pmain;
    e = launch_sparse_backward_seg(1, n, k, tr->codebook, w, B, plan.tail, T, w_hat, grad_w_hat,
                                   grad_log_z, grad_w, partial + (size_t)g1 * S, slots, st2, &g2,
                                   stream);
  }
  if (e == 0) e = launch_reduce_slots(partial, g1 + g2, S, grad_codebook, stream);
  return from_hip(e);
}

int64_t bcjr_scan_segment_length(const bcjr_trellis* tr, int64_t B, int64_t L, int64_t seg_len) {
  ScanPlan plan;
  if (scan_setup(tr, B, L, seg_len, &plan) != BCJR_OK) return 0;
  return plan.seg;
}

size_t bcjr_scan_workspace_bytes(const bcjr_trellis* tr, int64_t B, int64_t L, int64_t seg_len) {
  ScanPlan plan;
  if (scan_setup(tr, B, L, seg_len, &plan) != BCJR_OK || B == 0) return 0;
  return plan.bytes;
}

bcjr_status bcjr_forward_scan(const bcjr_trellis* tr, const float* w, int64_t B, int64_t L,
                              float T, int64_t seg_len, float* w_hat, float* log_z, void* ws,
                              size_t ws_bytes, bcjr_stream_t stream) {
  ScanPlan plan;
  bcjr_status st = scan_setup(tr, B, L, seg_len, &plan);
  if (st != BCJR_OK) return st;
  if (!temp_ok(T)) return BCJR_E_ARG;
  if (!temp_supported(tr, T)) return BCJR_E_UNSUPPORTED;
  if (B == 0) return BCJR_OK;
  if (!w || !w_hat || !log_z || tr->codebook == nullptr) return BCJR_E_ARG;
  if (!ws_ok(ws, ws_bytes, plan.bytes)) return BCJR_E_WORKSPACE;
  const int n = tr->state_bits, k = tr->bits_per_step;
  const int M = (1 << n) >> k;
  char* base = static_cast<char*>(ws);
  float* rows = reinterpret_cast<float*>(base + plan.rows);
  double* rscale = reinterpret_cast<double*>(base + plan.rscale);
  double* lam0 = reinterpret_cast<double*>(base + plan.lam0);
  double* rho1 = reinterpret_cast<double*>(base + plan.rho1);
  double* sc0 = reinterpret_cast<double*>(base + plan.sc0);
  void* slots = base + plan.slots;
  int e = 0;
  // phase 1: transfer rows of every segment (not needed for a single segment)
  if (plan.ptot > 1) {
    SegLaunch sl{plan.pmain, 0, plan.seg, L, plan.ptot, nullptr, nullptr, nullptr, rows, rscale};
    e = launch_sparse_forward_seg(2, n, k, tr->codebook, w, B * plan.pmain * M, plan.seg, T,
                                  nullptr, nullptr, slots, sl, stream);
    if (e == 0 && plan.tail > 0) {
      sl.nseg = 1;
      sl.jbase = plan.pmain;
      e = launch_sparse_forward_seg(2, n, k, tr->codebook, w, B * M, plan.tail, T, nullptr,
                                    nullptr, slots, sl, stream);
    }
  }
  // phase 2: boundary messages by a scan over the segments
  if (e == 0)
    e = launch_scan_bounds(rows, rscale, nullptr, B, plan.ptot, M, lam0, rho1, sc0, nullptr,
                           nullptr, slots, plan.bytes - plan.slots, stream);  // (slots free here)
  // phase 3: every segment's forward-backward from its boundary messages
  if (e == 0) {
    SegLaunch sl{plan.pmain, 0, plan.seg, L, plan.ptot, lam0, rho1, sc0, nullptr, nullptr};
    e = launch_sparse_forward_seg(1, n, k, tr->codebook, w, B * plan.pmain, plan.seg, T, w_hat,
                                  log_z, slots, sl, stream);
    if (e == 0 && plan.tail > 0) {
      sl.nseg = 1;
      sl.jbase = plan.pmain;
      e = launch_sparse_forward_seg(1, n, k, tr->codebook, w, B, plan.tail, T, w_hat, log_z,
                                    slots, sl, stream);
    }
  }
  return from_hip(e);
}

int bcjr_supported(const bcjr_trellis* tr) {
  if (tr == nullptr || !shape_ok(tr) || tr->weights_per_step != 1) return 0;
  SparseGeom g;
  return sparse_geom(tr->state_bits, tr->bits_per_step, 1, kFwd, &g) ? 1 : 0;
}

size_t bcjr_saved_bytes(const bcjr_trellis* tr, int64_t B, int64_t L) {
  if (tr == nullptr || !shape_ok(tr) || !chains_ok(B, L)) return 0;
  return round256(bcjr::saved_bytes(B, L));
}

size_t bcjr_workspace_bytes(const bcjr_trellis* tr, int64_t B, int64_t L, int which) {
  if (tr == nullptr || !shape_ok(tr) || !chains_ok(B, L) || tr->weights_per_step != 1) return 0;
  if (which < 0 || which > 4) return 0;
  const int kind = which == 3 ? kFwd : which == 4 ? kBwd : which;
  SparseGeom g;
  if (!sparse_geom(tr->state_bits, tr->bits_per_step, B, kind, &g)) return 0;
  if (B == 0) return 0;
  switch (which) {
    case 0: return sparse_fwd_ws_bytes(g, L, false);
    case 1: return sparse_bwd_ws_bytes(g, L, false);
    case 2: return sparse_vit_ws_bytes(g, L);
    case 3: return sparse_fwd_ws_bytes(g, L, true);
    case 4: return sparse_bwd_ws_bytes(g, L, true);
    default: return 0;
  }
}

bcjr_status bcjr_forward(const bcjr_trellis* tr, const float* w, int64_t B, int64_t L, float T,
                         float* w_hat, float* log_z, void* saved, void* ws, size_t ws_bytes,
                         bcjr_stream_t stream) {
  SparseGeom g;
  bcjr_status st = check_common(tr, B, L, kFwd, &g);
  if (st != BCJR_OK) return st;
  if (!temp_ok(T)) return BCJR_E_ARG;
  if (!temp_supported(tr, T)) return BCJR_E_UNSUPPORTED;
  if (B == 0) return BCJR_OK;
  if (!w || !w_hat || !log_z || !saved) return BCJR_E_ARG;
  if (((uintptr_t)saved & 15) != 0) return BCJR_E_ARG;
  bool ckpt = false;
  st = pick_layout(ws, ws_bytes, sparse_fwd_ws_bytes(g, L, false), sparse_fwd_ws_bytes(g, L, true),
                   &ckpt);
  if (st != BCJR_OK) return st;
  return from_hip(launch_sparse_forward(g, tr->codebook, w, B, L, T, w_hat, log_z,
                                        static_cast<float*>(saved), ws, ckpt, stream));
}

bcjr_status bcjr_backward(const bcjr_trellis* tr, const float* w, int64_t B, int64_t L, float T,
                          const void* saved, const float* grad_w_hat, const float* grad_log_z,
                          float* grad_w, float* grad_codebook, void* ws, size_t ws_bytes,
                          bcjr_stream_t stream) {
  SparseGeom g;
  bcjr_status st = check_common(tr, B, L, kBwd, &g);
  if (st != BCJR_OK) return st;
  if (!temp_ok(T)) return BCJR_E_ARG;
  if (!temp_supported(tr, T)) return BCJR_E_UNSUPPORTED;
  if (grad_codebook == nullptr) return BCJR_E_ARG;
  if (B == 0) {
    // no chain contributes: the summed codebook gradient is zero
    return from_hip(launch_fill_zero(grad_codebook, (int64_t)1 << tr->state_bits, stream));
  }
  if (!w || !saved || !grad_w_hat || !grad_w) return BCJR_E_ARG;
  if (((uintptr_t)saved & 15) != 0) return BCJR_E_ARG;
  bool ckpt = false;
  st = pick_layout(ws, ws_bytes, sparse_bwd_ws_bytes(g, L, false), sparse_bwd_ws_bytes(g, L, true),
                   &ckpt);
  if (st != BCJR_OK) return st;
  return from_hip(launch_sparse_backward(g, tr->codebook, w, B, L, T,
                                         static_cast<const float*>(saved), grad_w_hat, grad_log_z,
                                         grad_w, grad_codebook, ws, ckpt, stream));
}

bcjr_status viterbi_decode(const bcjr_trellis* tr, const float* w, int64_t B, int64_t L,
                           int32_t* states, float* w_hard, void* ws, size_t ws_bytes,
                           bcjr_stream_t stream) {
  SparseGeom g;
  bcjr_status st = check_common(tr, B, L, kVit, &g);
  if (st != BCJR_OK) return st;
  if (B == 0) return BCJR_OK;
  if (!w || !states) return BCJR_E_ARG;
  const size_t need = sparse_vit_ws_bytes(g, L);
  if (!ws_ok(ws, ws_bytes, need)) return BCJR_E_WORKSPACE;
  return from_hip(launch_viterbi(g, tr->codebook, w, B, L, states, w_hard, ws, stream));
}

int64_t bcjr_code_words(const bcjr_trellis* tr, int64_t L) {
  if (tr == nullptr || !shape_ok(tr) || tr->weights_per_step != 1 || L < 1) return 0;
  return code_words(tr->state_bits, tr->bits_per_step, L);
}

bcjr_status bcjr_pack_code(const bcjr_trellis* tr, const int32_t* states, int64_t B, int64_t L,
                           uint32_t* code, bcjr_stream_t stream) {
  if (tr == nullptr) return BCJR_E_ARG;
  if (!shape_ok(tr) || B < 0 || L < 1 || (B > 0 && L > ((int64_t)1 << 40) / B)) return BCJR_E_SHAPE;
  if (tr->weights_per_step != 1) return BCJR_E_UNSUPPORTED;
  if (B == 0) return BCJR_OK;
  if (!states || !code) return BCJR_E_ARG;
  return from_hip(launch_pack_code(tr->state_bits, tr->bits_per_step, states, B, L, code, stream));
}

bcjr_status bcjr_unpack_code(const bcjr_trellis* tr, const uint32_t* code, int64_t B, int64_t L,
                             int32_t* states, float* w_hard, bcjr_stream_t stream) {
  if (tr == nullptr) return BCJR_E_ARG;
  if (!shape_ok(tr) || B < 0 || L < 1 || (B > 0 && L > ((int64_t)1 << 40) / B)) return BCJR_E_SHAPE;
  if (tr->weights_per_step != 1) return BCJR_E_UNSUPPORTED;
  if (B == 0) return BCJR_OK;
  if (!code || !states || (w_hard && !tr->codebook)) return BCJR_E_ARG;
  return from_hip(launch_unpack_code(tr->state_bits, tr->bits_per_step, code, B, L, tr->codebook,
                                     states, w_hard, stream));
}

int bcjr_dense_supported(int32_t S) { return S >= 1 && S <= 65536 && dense_shape_built(S) ? 1 : 0; }

size_t bcjr_dense_saved_bytes(int32_t S, int64_t B, int64_t L) {
  if (dense_check(S, B, L) != BCJR_OK) return 0;
  DenseLayout d;
  dense_layout(S, B, L, &d);
  return d.saved;
}

size_t bcjr_dense_workspace_bytes(int32_t S, int64_t B, int64_t L, int which) {
  if (dense_check(S, B, L) != BCJR_OK || which < 0 || which > 1 || B == 0) return 0;
  DenseLayout d;
  dense_layout(S, B, L, &d);
  return which == 0 ? d.fwd : d.bwd;
}

bcjr_status bcjr_dense_forward(int32_t S, const float* theta, const float* codebook, const float* w,
                               int64_t B, int64_t L, float T, float* w_hat, float* log_z,
                               void* saved, void* ws, size_t ws_bytes, bcjr_stream_t stream) {
  bcjr_status st = dense_check(S, B, L);
  if (st != BCJR_OK) return st;
  if (!temp_ok(T)) return BCJR_E_ARG;
  if (T < kDenseMinT) return BCJR_E_UNSUPPORTED;
  if (B == 0) return BCJR_OK;
  if (!theta || !codebook || !w || !w_hat || !log_z || !saved) return BCJR_E_ARG;
  if (((uintptr_t)saved & 15) != 0) return BCJR_E_ARG;
  DenseLayout d;
  dense_layout(S, B, L, &d);
  if (!ws_ok(ws, ws_bytes, d.fwd)) return BCJR_E_WORKSPACE;
  return from_hip(launch_dense_forward(S, theta, codebook, w, B, L, T, w_hat, log_z, saved, ws,
                                       stream));
}

bcjr_status bcjr_dense_backward(int32_t S, const float* theta, const float* codebook,
                                const float* w, int64_t B, int64_t L, float T, const void* saved,
                                const float* grad_w_hat, const float* grad_log_z, float* grad_w,
                                float* grad_codebook, float* grad_theta, void* ws, size_t ws_bytes,
                                bcjr_stream_t stream) {
  bcjr_status st = dense_check(S, B, L);
  if (st != BCJR_OK) return st;
  if (!temp_ok(T)) return BCJR_E_ARG;
  if (T < kDenseMinT) return BCJR_E_UNSUPPORTED;
  if (!grad_codebook || !grad_theta) return BCJR_E_ARG;
  if (B == 0) {
    // no chain contributes: both summed gradients are zero
    int e = launch_fill_zero(grad_codebook, S, stream);
    if (e == 0) e = launch_fill_zero(grad_theta, (int64_t)S * S, stream);
    return from_hip(e);
  }
  if (!theta || !codebook || !w || !saved || !grad_w_hat || !grad_w) return BCJR_E_ARG;
  if (((uintptr_t)saved & 15) != 0) return BCJR_E_ARG;
  DenseLayout d;
  dense_layout(S, B, L, &d);
  if (!ws_ok(ws, ws_bytes, d.bwd)) return BCJR_E_WORKSPACE;
  return from_hip(launch_dense_backward(S, theta, codebook, w, B, L, T, saved, grad_w_hat,
                                        grad_log_z, grad_w, grad_codebook, grad_theta, ws, stream));
}

const char* bcjr_status_string(bcjr_status s) {
  switch (s) {
    case BCJR_OK: return "ok";
    case BCJR_E_ARG: return "invalid argument (null pointer, bad temperature or flag)";
    case BCJR_E_SHAPE: return "invalid shape (n, k, B or L out of range)";
    case BCJR_E_WORKSPACE: return "workspace missing or smaller than the size query";
    case BCJR_E_DEVICE: return "HIP runtime or kernel launch error";
    case BCJR_E_UNSUPPORTED: return "valid shape with no kernel built for it";
  }
  return "unknown status";
}

}  // extern "C"

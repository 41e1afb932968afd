// Internal declarations shared by the host layer (host.cpp) and the kernel files (*.hip).
// Nothing here is part of the public ABI (include/bcjr.h).
#pragma once
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "bcjr.h"
#include "geom.h"

namespace bcjr {

// Launch geometry of one bitshift configuration (n, k). Every quantity is a pure function of
// (n, k, B, L), so workspace sizes can be queried without a device.
struct SparseGeom {
  int n, k;      // state bits, bits per step
  int K;         // 1 << k branches
  int S;         // 1 << n states
  int M;         // S / K butterflies (forward messages per step)
  int NG;        // S / K^2 groups of K x K states
  int G;         // groups per lane
  int LPS;       // lanes per chain
  int SPB;       // chains per block (LPS < 64: 64 / LPS, else 1)
  int BLOCK;     // threads per block
  int64_t B;     // chains
  int64_t units; // ceil(B / SPB)
  int64_t slots; // workspace slots = the most blocks a launch may use
};

// True if kernels for (n, k) are compiled into the library (sparse_kernels.hip).
bool sparse_shape_built(int n, int k);

// Returns false if no kernel is built for (n, k).
bool sparse_geom(int n, int k, int64_t B, int kind, SparseGeom* g);

// Layout of the forward -> backward context: log2 Z of every chain as a double [B] (padded to
// a multiple of 32 doubles), then the soft codeword w_hat [B, L] in fp32.
// saved_what_offset() is in floats.
inline int64_t saved_what_offset(int64_t B) { return 2 * ((B + 31) / 32 * 32); }
inline size_t saved_bytes(int64_t B, int64_t L) {
  return (size_t)(saved_what_offset(B) + B * L) * sizeof(float);
}

inline size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace layout of the sparse kernels: one slot per persistent block. A forward slot holds
// the lam history, H entries of BLOCK * K*G values with room for 8 bytes each (each entry in
// 16-byte chunks interleaved across the block's lanes), and the shift prefix [L][SPB] (double);
// a backward slot adds the Phi history [H][BLOCK][K*G] (fp32); the backward workspace ends
// with the codebook-gradient partials [slots][S] (fp32). Sizes do not depend on T.
// Full history: H = L entries, one per step. Checkpointed history: every C-th step is kept
// (C = ceil(sqrt(L))) and the reverse sweep recomputes one segment of C steps at a time into a
// C-entry buffer, so H = ceil(L / C) + C (about 2 sqrt(L)) at the cost of one more forward
// recursion.
inline int64_t sparse_seg_len(int64_t L) {
  int64_t c = (int64_t)sqrt((double)L);
  while (c * c < L) ++c;
  while (c > 1 && (c - 1) * (c - 1) >= L) --c;
  return c < 1 ? 1 : c;
}
inline int64_t sparse_hist_entries(int64_t L, bool ckpt) {
  if (!ckpt) return L;
  const int64_t c = sparse_seg_len(L);
  return (L + c - 1) / c + c;
}
inline size_t sparse_fwd_slot_bytes(const SparseGeom& g, int64_t L, bool ckpt) {
  return round256((size_t)sparse_hist_entries(L, ckpt) * g.BLOCK * (g.K * g.G) * 8 +
                  (size_t)L * g.SPB * 8);
}
// Chains of 1024 lanes (k_sparse_bwd_wide) also record their backward rows per history entry
// ([H][BLOCK][K*G], 8-byte + fp32 entries, after the shift prefix rounded to 256 bytes) and, per
// step, the posterior normaliser (double) and the centring mean (fp32).
inline size_t sparse_bwd_slot_bytes(const SparseGeom& g, int64_t L, bool ckpt) {
  const size_t hist = (size_t)sparse_hist_entries(L, ckpt) * g.BLOCK * (g.K * g.G) * 12;
  if (g.LPS >= kMaxLanesPerChain)
    return round256(hist + round256((size_t)L * 8) + hist + (size_t)L * 12);
  return round256(hist + (size_t)L * g.SPB * 8);
}
// Forward / backward workspace for the fp32-message geometry g: enough for either message
// precision (the fp64-message kernels run with the kFwdP / kBwdP geometry of the same n, k, B).
size_t sparse_fwd_ws_bytes(const SparseGeom& g, int64_t L, bool ckpt);
size_t sparse_bwd_ws_bytes(const SparseGeom& g, int64_t L, bool ckpt);
size_t sparse_vit_ws_bytes(const SparseGeom& g, int64_t L);

// Kernel launchers (defined in sparse_kernels.hip / viterbi_kernels.hip). They assume every
// argument was validated by the host layer. Return a hipError_t as int.
// ckpt selects the checkpointed history layout (see sparse_hist_entries).
int launch_sparse_forward(const SparseGeom& g, const float* codebook, const float* w, int64_t B,
                          int64_t L, float T, float* w_hat, float* log_z, float* saved_logz2,
                          void* ws, bool ckpt, void* stream);
int launch_sparse_backward(const SparseGeom& g, const float* codebook, const float* w, int64_t B,
                           int64_t L, float T, const float* saved_logz2, const float* grad_w_hat,
                           const float* grad_log_z, float* grad_w, float* grad_codebook, void* ws,
                           bool ckpt, void* stream);
// The fp32-message forward / backward of the shapes built in sparse_kernels.hip's second
// translation unit (max-ILP scheduling); called by the launchers above for those shapes.
int run_fwd_fast_ilp(int n, const SparseGeom& g, const float* cb, const float* w, long long B,
                     long long L, float T, float* w_hat, float* log_z, float* saved, void* ws,
                     bool ckpt, void* stream);
int run_bwd_fast_ilp(int n, const SparseGeom& g, const float* cb, const float* w, long long B,
                     long long L, float T, const float* saved, const float* gup, const float* hup,
                     float* grad_w, float* grad_c, void* ws, bool ckpt, void* stream);
// The same in the spread geometry of small batches (k = 2, n <= 12; see geom_spread).
int run_fwd_spread_ilp(int n, const SparseGeom& g, const float* cb, const float* w, long long B,
                       long long L, float T, float* w_hat, float* log_z, float* saved, void* ws,
                       bool ckpt, void* stream);
int run_bwd_spread_ilp(int n, const SparseGeom& g, const float* cb, const float* w, long long B,
                       long long L, float T, const float* saved, const float* gup,
                       const float* hup, float* grad_w, float* grad_c, void* ws, bool ckpt,
                       void* stream);
int launch_fill_zero(float* dst, int64_t count, void* stream);
// Grid of a persistent kernel: min(slots, resident blocks on the current device), or -1.
int resident_grid(const void* kernel, int block, int64_t slots);
int launch_viterbi(const SparseGeom& g, const float* codebook, const float* w, int64_t B,
                   int64_t L, int32_t* states, float* w_hard, void* ws, void* stream);

// ---- segmented forward of long chains (parallel in L) ---------------------------------------
// A chain of L steps is cut into pmain segments of seg steps plus, if L is not a multiple, one
// tail segment (ptot segments in all). Phase 1 computes every segment's M x M transfer matrix
// (M = S/K) from M one-hot starts, phase 2 scans the boundary messages over the segments,
// phase 3 runs the forward-backward of all segments at once from their boundary messages.
struct SegLaunch {
  int64_t nseg, jbase, seglen, lfull, ptot;
  const double* lam0;
  const double* rho1;
  const double* sc0;
  float* rows;
  double* rscale;
  const float* phi0 = nullptr;  // backward only
  const float* psi1 = nullptr;
  float* frows = nullptr;
};
// mode 2: transfer rows (Bv = chains * segments * M virtual chains); mode 1: segments with
// boundary messages (Bv = chains * segments).
int launch_sparse_forward_seg(int mode, int n, int k, const float* codebook, const float* w,
                              int64_t Bv, int64_t L, float T, float* w_hat, float* log_z, void* ws,
                              const SegLaunch& sl, void* stream);
// Backward counterparts: mode 2 writes transfer rows and moment rows, mode 1 runs the segments
// and writes the codebook-gradient partials of *grid_used slots at `partial` (not reduced).
int launch_sparse_backward_seg(int mode, int n, int k, const float* codebook, const float* w,
                               int64_t Bv, int64_t L, float T, const float* w_hat,
                               const float* grad_w_hat, const float* grad_log_z, float* grad_w,
                               float* partial, void* ws, const SegLaunch& sl, int* grid_used,
                               void* stream);
// The fp32 launches of launch_sparse_backward_seg for the shapes built in sparse_kernels.hip's
// max-ILP translation unit.
int launch_sparse_backward_seg_ilp(int mode, int n, int k, const float* codebook, const float* w,
                                   int64_t Bv, int64_t L, float T, const float* w_hat,
                                   const float* grad_w_hat, const float* grad_log_z, float* grad_w,
                                   float* partial, void* ws, const SegLaunch& sl, int* grid_used,
                                   void* stream);
// out[s] = sum over slots of partial[slot][s] in a fixed order (partial is scratch: overwritten).
int launch_reduce_slots(float* partial, int64_t slots, int S, float* out, void* stream);
bool scan_shape_built(int n, int k);
// Boundary scan; with frows (moment rows) also the conditional expectations phi0 / psi1. With
// enough segments and M <= 64 it runs as a tree over the segments in tree_ws (scratch of
// tree_ws_bytes bytes, free during the call; null: the sequential scan).
int launch_scan_bounds(const float* rows, const double* rscale, const float* frows, int64_t chains,
                       int64_t ptot, int M, double* lam0, double* rho1, double* sc0, float* phi0,
                       float* psi1, void* tree_ws, size_t tree_ws_bytes, void* stream);

// The boundary scan runs as a tree over the segments (scan_kernels.hip) for M <= 64 from this
// many segments on; below it the sequential scan's few steps cost less than the tree's launches.
constexpr int64_t kTreeMinSegments = 64;
// Bytes of the tree's scratch for `chains` chains of `ptot` segments: per level above the
// segments, the composed matrices (and moment matrices), row scales and both boundary vectors
// (and expectations) of every node; 0 where the sequential scan runs.
inline size_t scan_tree_bytes(int64_t chains, int64_t ptot, int64_t M, bool mom) {
  if (M > 64 || ptot < kTreeMinSegments) return 0;
  size_t b = 0;
  for (int64_t n = (ptot + 1) / 2;; n = (n + 1) / 2) {
    const size_t nodes = (size_t)chains * (size_t)n;
    b += round256(nodes * (size_t)M * (size_t)M * sizeof(float)) * (mom ? 2 : 1);
    b += round256(nodes * (size_t)M * sizeof(double)) * 3;
    if (mom) b += round256(nodes * (size_t)M * sizeof(float)) * 2;
    if (n == 1) break;
  }
  return b;
}

constexpr int64_t kScanMinSeg = 16;

// Default segment length. A chain's time is about P * t2 (the boundary scan over its
// P = L / seg segments) + seg * t3 (each segment's own sweeps, sequential in its steps),
// smallest at seg = sqrt(L * t2 / t3). Measured on MI355X: t3 = 1.5 us per step (forward and
// backward sweep of one chain, with the segment geometry kFwdS / kBwdS). The sequential scan
// costs t2 = 1.0 us + 0.03 us * M per segment for M = S/K <= 64 (one wave per chain and
// direction) and 2.5 us + 3.7e-4 us * M^2 above (one block). The tree over the segments
// (M <= 64, from kTreeMinSegments segments) costs about t2 = 0.0015 us * M * B per segment
// (fitted to segment-length sweeps at S = 16, 64, 256 with B = 1, 2, 16 chains of 2^16..2^20
// steps, whose optima it places within 1.3x), so where it applies its optimum is used.
// A segment shorter than the others (when seg does not divide L) runs in launches of its own
// after the others, so the default prefers a divisor of L within 1.5x of that optimum, else
// seg = floor(L / P) for P = ceil(L / optimum), which keeps the short segment under P steps.
inline int64_t scan_default_seg(int n, int k, int64_t B, int64_t L) {
  const double M = (double)(((int64_t)1 << n) >> k);
  const double t3 = 1.5;
  double opt = sqrt((double)L * (M <= 64 ? 1.0 + 0.03 * M : 2.5 + 3.7e-4 * M * M) / t3);
  if (M <= 64) {
    const double tree = sqrt((double)L * 0.0015 * M * (double)(B > 1 ? B : 1) / t3);
    if ((double)L / tree >= (double)kTreeMinSegments) opt = tree;
  }
  if (opt <= (double)kScanMinSeg) return kScanMinSeg;
  if (opt >= (double)L) return L;
  const int64_t lo = (int64_t)ceil(opt / 1.5), hi = (int64_t)floor(opt * 1.5);
  int64_t best = 0;
  double best_r = 0.0;
  for (int64_t d = lo < kScanMinSeg ? kScanMinSeg : lo; d <= hi && d <= L; ++d) {
    if (L % d) continue;
    const double r = d > opt ? d / opt : opt / d;
    if (best == 0 || r < best_r) { best = d; best_r = r; }
  }
  if (best) return best;
  const int64_t P = (int64_t)ceil((double)L / opt);
  const int64_t seg = L / P;
  return seg < kScanMinSeg ? kScanMinSeg : seg;
}

struct ScanPlan {
  int64_t seg, pmain, tail, ptot;
  size_t rows, rscale, lam0, rho1, sc0, slots, bytes;  // workspace offsets and total
  // backward only: moment rows, Phi / Psi boundaries, codebook-gradient partials
  size_t frows = 0, phi0 = 0, psi1 = 0, partial = 0;
};

inline void scan_plan(const SparseGeom& gmain, const SparseGeom& gtail, int n, int k, int64_t B,
                      int64_t L, int64_t seg, ScanPlan* p) {
  const int64_t M = ((int64_t)1 << n) >> k;
  p->seg = seg < L ? seg : L;
  p->pmain = L / p->seg;
  p->tail = L - p->pmain * p->seg;
  p->ptot = p->pmain + (p->tail > 0 ? 1 : 0);
  const size_t cp = (size_t)B * (size_t)p->ptot;
  p->rows = 0;
  p->rscale = p->ptot > 1 ? round256(cp * (size_t)M * (size_t)M * sizeof(float)) : 0;
  p->lam0 = p->rscale + (p->ptot > 1 ? round256(cp * (size_t)M * sizeof(double)) : 0);
  p->rho1 = p->lam0 + round256(cp * (size_t)M * sizeof(double));
  p->sc0 = p->rho1 + round256(cp * (size_t)M * sizeof(double));
  p->slots = p->sc0 + round256(cp * 2 * sizeof(double));
  size_t a = sparse_fwd_ws_bytes(gmain, p->seg, false);
  if (p->tail > 0) {
    const size_t b = sparse_fwd_ws_bytes(gtail, p->tail, false);
    if (b > a) a = b;
  }
  // the boundary scan's tree uses the same region (free between the segment launches)
  const size_t tb = scan_tree_bytes(B, p->ptot, M, false);
  if (tb > a) a = tb;
  p->bytes = p->slots + round256(a);
}

// Backward plan: transfer and moment rows, the four boundary vectors and their scales, the
// codebook-gradient partials of both segment launches (up to `partial_slots` slots), then the
// segment kernels' per-slot histories. gmain / gtail are fp32-message backward geometries.
inline void scan_plan_bwd(const SparseGeom& gmain, const SparseGeom& gtail, int64_t partial_slots,
                          int n, int k, int64_t B, int64_t L, int64_t seg, ScanPlan* p) {
  const int64_t M = ((int64_t)1 << n) >> k;
  const int64_t S = (int64_t)1 << n;
  p->seg = seg < L ? seg : L;
  p->pmain = L / p->seg;
  p->tail = L - p->pmain * p->seg;
  p->ptot = p->pmain + (p->tail > 0 ? 1 : 0);
  const size_t cp = (size_t)B * (size_t)p->ptot;
  const size_t mm = p->ptot > 1 ? round256(cp * (size_t)M * (size_t)M * sizeof(float)) : 0;
  p->rows = 0;
  p->frows = mm;
  p->rscale = 2 * mm;
  p->lam0 = p->rscale + (p->ptot > 1 ? round256(cp * (size_t)M * sizeof(double)) : 0);
  p->rho1 = p->lam0 + round256(cp * (size_t)M * sizeof(double));
  p->sc0 = p->rho1 + round256(cp * (size_t)M * sizeof(double));
  p->phi0 = p->sc0 + round256(cp * 2 * sizeof(double));
  p->psi1 = p->phi0 + round256(cp * (size_t)M * sizeof(float));
  p->partial = p->psi1 + round256(cp * (size_t)M * sizeof(float));
  p->slots = p->partial + round256((size_t)partial_slots * (size_t)S * sizeof(float));
  size_t a = sparse_bwd_ws_bytes(gmain, p->seg, false);
  if (p->tail > 0) {
    const size_t b = sparse_bwd_ws_bytes(gtail, p->tail, false);
    if (b > a) a = b;
  }
  const size_t tb = scan_tree_bytes(B, p->ptot, M, true);  // (as in scan_plan)
  if (tb > a) a = tb;
  p->bytes = p->slots + round256(a);
}

// ---- hard-code export (bitshift trellis) -----------------------------------------------------
// 32-bit words of one chain's code: n bits of the initial state + k bits per later step.
inline int64_t code_words(int n, int k, int64_t L) { return ((int64_t)n + (int64_t)k * (L - 1) + 31) / 32; }
int launch_pack_code(int n, int k, const int32_t* states, int64_t B, int64_t L, uint32_t* code,
                     void* stream);
int launch_unpack_code(int n, int k, const uint32_t* code, int64_t B, int64_t L,
                       const float* codebook, int32_t* states, float* w_hard, void* stream);

// ---- dense (fully connected) trellis -------------------------------------------------------
// Sweep kernels use one persistent block per 4 chains, at most kDenseSweepMaxGrid blocks; the
// theta-gradient product at most kDenseGemmMaxGrid blocks. Both bounds size workspace partials.
constexpr int64_t kDenseSweepMaxGrid = 1024;
constexpr int64_t kDenseGemmMaxGrid = 512;
inline int64_t dense_sweep_slots(int64_t units) {
  return units < kDenseSweepMaxGrid ? units : kDenseSweepMaxGrid;
}

// Byte offsets of the dense context (`saved`) and workspace. saved: log2 Z [B] (double), the
// per-step scalars [B, L, 4] (w_hat_t, 1/zz_t, ref_t, 1/n_{t-1}), the forward messages a and the
// backward messages u, each [B, L, S]. Workspace: the transition matrix M [S, S] and kappa * cm
// [S] (forward and backward); the backward adds L1, R1, R2 [B, L, S], the codebook-gradient
// partials of its two sweeps [2, kDenseSweepMaxGrid, S] and the theta-gradient partials
// [kDenseGemmMaxGrid, S, S].
struct DenseLayout {
  size_t lz2, pack, ha, hb, saved;
  size_t mat, cmk, fwd, l1, r1, r2, gcp, gp, bwd;
};
inline void dense_layout(int S, int64_t B, int64_t L, DenseLayout* d) {
  const size_t bl = (size_t)B * (size_t)L;
  const size_t bls = bl * (size_t)S * sizeof(float);
  d->lz2 = 0;
  d->pack = round256((size_t)B * sizeof(double));
  d->ha = d->pack + round256(bl * 4 * sizeof(float));
  d->hb = d->ha + round256(bls);
  d->saved = d->hb + round256(bls);
  d->mat = 0;
  d->cmk = round256((size_t)S * S * sizeof(float));
  d->fwd = d->cmk + round256((size_t)S * sizeof(float));
  d->l1 = d->fwd;
  d->r1 = d->l1 + round256(bls);
  d->r2 = d->r1 + round256(bls);
  d->gcp = d->r2 + round256(bls);
  d->gp = d->gcp + round256((size_t)2 * kDenseSweepMaxGrid * S * sizeof(float));
  d->bwd = d->gp + round256((size_t)kDenseGemmMaxGrid * S * S * sizeof(float));
}

// The dense path works in the linear domain: with every step rescaled to its maximum, a state
// whose relative weight falls below 2^-126 is dropped. At unit-scale theta, c and w this keeps
// ŵ and the gradients within tolerance down to T = 0.1 (measured on MI355X for S = 32 ... 256:
// at T = 0.05 ŵ errs by 4e-3 at S = 256, and below 0.03 whole steps underflow to NaN), so the
// entry points refuse lower temperatures.
constexpr float kDenseMinT = 0.1f;

// True if dense kernels for S states are compiled in (dense_kernels.hip).
bool dense_shape_built(int S);
int launch_dense_forward(int S, const float* theta, const float* codebook, const float* w, int64_t B,
                         int64_t L, float T, float* w_hat, float* log_z, void* saved, void* ws,
                         void* stream);
int launch_dense_backward(int S, const float* theta, const float* codebook, const float* w,
                          int64_t B, int64_t L, float T, const void* saved, const float* grad_w_hat,
                          const float* grad_log_z, float* grad_w, float* grad_codebook,
                          float* grad_theta, void* ws, void* stream);

}  // namespace bcjr

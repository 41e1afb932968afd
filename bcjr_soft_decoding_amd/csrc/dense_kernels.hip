// Fully connected (dense) trellis on gfx950: every state may follow every state, with transition
// log-potentials theta(s, s'). Same method as the bitshift kernels (BCJR-QAT abstract: the
// forward-backward recursion at temperature T, Boltzmann posteriors over paths, the soft
// codeword and its exact gradient), written in the transfer-matrix form the abstract names (a
// 1D Ising-like chain): every step is a dense S x S product, done on the matrix cores.
//
// Linear domain, log2 units, kappa = log2(e)/T. Per call:
//   cm(s')   = max_s theta(s, s')                 (column maximum)
//   M(s, s') = 2^(kappa (theta(s, s') - cm(s')))  (every column has maximum 1)
// The column shift is folded into the emission of every step after the first:
//   ell_0(s) = -kappa (w_0 - c(s))^2,  ell_t(s) = -kappa (w_t - c(s))^2 + kappa cm(s)  (t >= 1)
//   ref_t = max_s ell_t(s),  e_t(s) = 2^(ell_t(s) - ref_t)
// Forward (alpha) sweep, normalised by the previous step's sum:
//   a_0 = e_0,  a_t = ((a_{t-1} M) / n_{t-1}) o e_t,  n_t = sum_s a_t(s)
//   log2 Z = sum_t (ref_t + log2 n_t)
// Backward (beta) sweep, normalised by the posterior mass zz_t:
//   u_{L-1} = 1,  zz_t = sum_s a_t u_t,  u_{t-1} = (M (e_t o u_t)) / zz_t
//   gamma_t = a_t o u_t / zz_t,  w_hat_t = sum_s c(s) gamma_t(s)
// Gradient of F = sum_t g_t w_hat_t + h log Z, with the centred conditional expectations of the
// bitshift kernels carried as message-weighted vectors (v = u o Psi, at = a o Phi):
//   v_{L-1} = 0,  z_{t-1} = e_t o (v_t + u_t g_t (c - w_hat_t)),  v_{t-1} = (M z_{t-1}) / zz_t
//   at_0 = 0,  x_t = at_t + a_t g_t (c - w_hat_t),  at_t = ((x_{t-1} M) / n_{t-1}) o e_t
//   D_t = (a_t o (u_t g_t (c - w_hat_t) + v_t) + at_t o u_t) / zz_t
//   dF/dw_t = (2/T)(sum_s c D_t + h (w_hat_t - w_t))
//   dF/dc   = sum_t [g_t gamma_t + (2/T)(w_t - c)(D_t + h gamma_t)]
//   dF/dtheta = (M / T) o sum_{chains} sum_{t >= 1} [L1_{t-1} (x) R1_t + a_{t-1} (x) R2_t]
//     L1_t = x_t + h a_t,  R1_t = e_t o u_t / (n_{t-1} zz_t),  R2_t = z_{t-1} / (n_{t-1} zz_t)
// The edge posterior of (s, s') between steps t-1 and t is a_{t-1}(s) M(s,s') e_t(s') u_t(s') /
// (n_{t-1} zz_t), which is where the two rank-one terms come from.
//
// Messages are fp32. Every state can reach every state, so a weight that underflows is below
// 2^-126 of the step's best state and its posterior is negligible at the tolerances used here.
//
// Kernels: k_dense_prep (M, kappa cm), four sweeps (alpha and beta in the forward call; Psi then
// Phi in the backward call), k_dense_theta_gemm (the theta gradient as one split-K product over
// all chains and steps) and k_dense_sum_parts (fixed-order sums of the block partials).
//
// Sweep tiling: one block per 4 chains, S/32 waves; wave wv owns output states 32wv..32wv+31.
// The step product runs on v_mfma_f32_4x4x1f32 (16 independent 4x4 outer products): block b of
// an instruction takes chain i = lane & 3, input state k = 4 kc + (lane >> 4) and output state
// 32 wv + 16 set + (lane & 15), so lane l keeps M[4kc + l/16][32wv + 16set + l%16] (the
// transposed entry for the backward sweeps) in registers for the whole launch: the matrix lives
// in the register files of one block. The four partial sums over k (lane bits 4 and 5) of each
// 16-state set are folded with v_permlane32_swap / v_permlane16_swap as a reduce-scatter, which
// leaves lane l with chain l >> 4 at two states, so per-chain sums over states are 16-lane row
// reductions. Messages are staged in LDS as [k % 4][chain][k / 4] so that a lane reads four
// consecutive MFMA operands with one 16-byte load.
#include <hip/hip_runtime.h>

#include <math.h>

#include "internal.h"

namespace bcjr {
namespace {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));

constexpr double kLn2D = 0.69314718055994530942;
constexpr float kLog2eF = 1.44269504088896340736f;
constexpr int kChunk = 32;  // steps per LDS chunk of per-step scalars

enum Mode { kAlpha = 0, kBeta = 1, kPsi = 2, kPhi = 3 };

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <bool MX>
__device__ __forceinline__ float comb(float a, float b) {
  return MX ? fmaxf(a, b) : a + b;
}
// Sum (or max) over the 16 lanes of a row; every lane of the row gets the result.
template <bool MX>
__device__ __forceinline__ float row_red(float v) {
  v = comb<MX>(v, dpp<0x128>(v));  // row_ror:8
  v = comb<MX>(v, dpp<0x124>(v));  // row_ror:4
  v = comb<MX>(v, dpp<0x122>(v));  // row_ror:2
  v = comb<MX>(v, dpp<0x121>(v));  // row_ror:1
  return v;
}
// Sum (or max) over aligned groups of N consecutive lanes (N in 1, 2, 4, 8).
template <int N, bool MX>
__device__ __forceinline__ float group_red(float v) {
  if (N >= 2) v = comb<MX>(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]
  if (N >= 4) v = comb<MX>(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]
  if (N >= 8) v = comb<MX>(v, dpp<0x141>(v));  // row_half_mirror
  return v;
}

struct P2 {
  float lo, hi;
};
// v_permlane32_swap: lo = [x lanes 0-31 | y lanes 0-31], hi = [x lanes 32-63 | y lanes 32-63].
__device__ __forceinline__ P2 swap32(float x, float y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
// v_permlane16_swap: lo = [x row0, y row0, x row2, y row2], hi = [x row1, y row1, x row3, y row3].
__device__ __forceinline__ P2 swap16(float x, float y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}

template <int S_>
struct DGeo {
  static constexpr int S = S_;
  static constexpr int NW = S / 32;        // waves per block
  static constexpr int BLOCK = 64 * NW;
  static constexpr int KC = S / 4;         // MFMA k-steps per product
  static constexpr int MR = S / 2;         // transition-matrix registers per lane
  static constexpr int XSTR = KC + 4;      // LDS row stride of a staged message (floats)
  static constexpr int XBUF = 16 * XSTR;   // one staged message (16 rows of [k%4][chain])
  static_assert(S >= 32 && S <= 256 && (S & (S - 1)) == 0, "S must be 32, 64, 128 or 256");
};

// Reduce the four k-partials of one 16-state set (lane bits 4 and 5) and scatter the chains:
// returns out[chain lane >> 4][state (lane & 15) of the set].
__device__ __forceinline__ float scatter_set(const f4 s) {
  const P2 a = swap32(s[0], s[2]);  // lanes 0-31 keep chain 0, lanes 32-63 chain 2
  const P2 b = swap32(s[1], s[3]);  // chain 1, chain 3
  const P2 q = swap16(a.lo + a.hi, b.lo + b.hi);
  return q.lo + q.hi;
}

// Product of the staged message (4 chains) with the register-resident matrix. Lane l gets chain
// l >> 4 at states 32wv + (l & 15) (o[0]) and 32wv + 16 + (l & 15) (o[1]).
template <class C>
__device__ __forceinline__ void product(const float* __restrict__ xs, const float (&m)[C::MR], int l,
                                        float (&o)[2]) {
  const float* xr = xs + ((l >> 4) * 4 + (l & 3)) * C::XSTR;
  f4 acc[2][2];
#pragma unroll
  for (int s = 0; s < 2; ++s) acc[s][0] = acc[s][1] = f4{0.f, 0.f, 0.f, 0.f};
  // The message operands are read from LDS PD chunks (8 MFMAs each) ahead of their matrix
  // instructions; the scheduling barrier keeps each read in its chunk (left to itself the
  // scheduler sinks every read to one chunk ahead, and each chunk then waits for its read).
  constexpr int PD = 3, NCH = C::KC / 4;
  f4 pre[NCH];
#pragma unroll
  for (int i = 0; i < PD && i < NCH; ++i) pre[i] = *reinterpret_cast<const f4*>(xr + 4 * i);
#pragma unroll
  for (int kc = 0; kc < C::KC; kc += 4) {
    if (kc / 4 + PD < NCH) pre[kc / 4 + PD] = *reinterpret_cast<const f4*>(xr + kc + 4 * PD);
    __builtin_amdgcn_sched_barrier(0);
    const f4 a = pre[kc / 4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[0][e & 1] = __builtin_amdgcn_mfma_f32_4x4x1f32(a[e], m[2 * (kc + e)], acc[0][e & 1], 0, 0, 0);
      acc[1][e & 1] = __builtin_amdgcn_mfma_f32_4x4x1f32(a[e], m[2 * (kc + e) + 1], acc[1][e & 1], 0, 0, 0);
    }
  }
  o[0] = scatter_set(acc[0][0] + acc[0][1]);
  o[1] = scatter_set(acc[1][0] + acc[1][1]);
}

// Block-wide reduction of per-chain quantities over the S states, in two halves around the
// step's barrier. publish(): v[q] is this lane's value of quantity q for its chain (lane >> 4,
// already combined over the lane's two states); bit q of MAXQ selects a max instead of a sum;
// the wave totals go to red[(q * 4 + chain) * NW + wave]. collect(), after the barrier: the
// block total for the lane's chain in out[q].
template <int NQR, int MAXQ, int NW>
__device__ __forceinline__ void publish(const float (&v)[NQR], float* __restrict__ red, int l, int wv) {
#pragma unroll
  for (int q = 0; q < NQR; ++q) {
    const float tot = ((MAXQ >> q) & 1) ? row_red<true>(v[q]) : row_red<false>(v[q]);
    if ((l & 15) == 0) red[(q * 4 + (l >> 4)) * NW + wv] = tot;
  }
}
template <int NQR, int MAXQ, int NW>
__device__ __forceinline__ void collect(const float* __restrict__ red, int l, float (&out)[NQR]) {
  const float x = l < NQR * 4 * NW ? red[l] : 0.f;
  const float sx = group_red<NW, false>(x);
  const float mx = group_red<NW, true>(x);
  const int ql = l / (4 * NW);
  const float tot = ((MAXQ >> ql) & 1) ? mx : sx;
#pragma unroll
  for (int q = 0; q < NQR; ++q) out[q] = __shfl(tot, (q * 4 + (l >> 4)) * NW, 64);
}

struct SweepArgs {
  const float* mat;   // M [S][S]
  const float* cmk;   // kappa * cm [S]
  const float* cb;    // codebook [S]
  const float* w;     // [B, L]
  const float* g;     // [B, L] upstream gradient of w_hat (Psi, Phi)
  const float* h;     // [B] upstream gradient of log Z, or null
  long long B, L, units;
  float kap;          // log2(e) / T
  float two_t;        // 2 / T
  float* pack;        // [B, L, 4]: w_hat_t, 1/zz_t, ref_t, 1/n_{t-1}
  double* lz2;        // [B] log2 Z
  float* log_z;       // [B]
  float* w_hat;       // [B, L]
  float* ha;          // [B, L, S] a_t
  float* hb;          // [B, L, S] u_t
  float* l1;          // [B, L, S] L1_t
  float* r1;          // [B, L, S] R1_t
  float* r2;          // [B, L, S] R2_t
  float* grad_w;      // [B, L]
  float* gc_part;     // [gridDim.x, S] codebook-gradient partials of this sweep
};

template <int MODE>
struct ModeTraits {
  static constexpr bool FWD = MODE == kAlpha || MODE == kPhi;  // t ascending, product x M
  static constexpr int NQ = MODE == kAlpha ? 1 : MODE == kBeta ? 2 : 6;  // staged scalars
};

// Per-step scalar q of chain b at step t (staged through LDS in chunks).
template <int MODE>
__device__ __forceinline__ float fetch_scalar(const SweepArgs& A, int q, long long b, long long t) {
  const long long i = b * A.L + t;
  if (MODE == kAlpha) return t + 1 < A.L ? A.w[i + 1] : 0.f;  // w_{t+1}
  if (MODE == kBeta) return q == 0 ? A.w[i] : A.pack[i * 4 + 2];  // w_t, ref_t
  if (q == 0) return A.w[i];
  if (q == 1) return A.g[i];
  return A.pack[i * 4 + (q - 2)];  // w_hat_t, 1/zz_t, ref_t, 1/n_{t-1}
}

template <int S, int MODE>
__global__ void __launch_bounds__(DGeo<S>::BLOCK)
k_dense_sweep(SweepArgs A) {
  using C = DGeo<S>;
  using TR = ModeTraits<MODE>;
  constexpr bool FWD = TR::FWD;
  constexpr int NQ = TR::NQ;
  constexpr int NSC = kChunk * NQ * 4;
  constexpr int NPT = (NSC + C::BLOCK - 1) / C::BLOCK;
  __shared__ __attribute__((aligned(16))) float xs[2][C::XBUF];
  __shared__ float red[2][64];
  __shared__ __attribute__((aligned(16))) float sc[2][NSC];

  const int tid = threadIdx.x, l = tid & 63, wv = tid >> 6;
  const int ch = l >> 4;                  // chain of this lane within a unit of 4
  const int col0 = 32 * wv + (l & 15);    // this lane's states: col0 and col0 + 16
  float cc[2], ck[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    cc[e] = A.cb[col0 + 16 * e];
    ck[e] = A.cmk[col0 + 16 * e];
  }
  const float kap = A.kap;
  const long long L = A.L, B = A.B;
  const long long nch = (L + kChunk - 1) / kChunk;

  float m[C::MR];
#pragma unroll
  for (int kc = 0; kc < C::KC; ++kc)
#pragma unroll
    for (int set = 0; set < 2; ++set) {
      const int k = 4 * kc + (l >> 4);
      const int o = 32 * wv + 16 * set + (l & 15);
      m[2 * kc + set] = FWD ? A.mat[k * S + o] : A.mat[o * S + k];
    }
  // where this lane stages its values: X[ch][k] at ((k % 4) * 4 + ch) * XSTR + k / 4
  const int xo = ((col0 & 3) * 4 + ch) * C::XSTR + (col0 >> 2);  // state col0 + 16: xo + 4
  float gc[2] = {0.f, 0.f};

  for (long long unit = blockIdx.x; unit < A.units; unit += gridDim.x) {
    const long long b0 = unit * 4;
    const bool valid = b0 + ch < B;
    const long long b = valid ? b0 + ch : B - 1;
    const float fv = valid ? 1.f : 0.f;
    const float hh = ((MODE == kPsi || MODE == kPhi) && A.h != nullptr) ? A.h[b] : 0.f;

    float sr[NPT];
    auto stage_load = [&](long long c) {
#pragma unroll
      for (int p = 0; p < NPT; ++p) {
        const int idx = tid + p * C::BLOCK;
        sr[p] = 0.f;
        if (idx < NSC) {
          const int tt = idx / (NQ * 4), q = (idx >> 2) % NQ, cq = idx & 3;
          const long long j = c * kChunk + tt;
          const long long bq = b0 + cq < B ? b0 + cq : B - 1;
          if (j < L) sr[p] = fetch_scalar<MODE>(A, q, bq, FWD ? j : L - 1 - j);
        }
      }
    };
    auto stage_store = [&](int buf) {
#pragma unroll
      for (int p = 0; p < NPT; ++p) {
        const int idx = tid + p * C::BLOCK;
        if (idx < NSC) sc[buf][idx] = sr[p];
      }
    };
    auto hist_load = [&](long long j, float (&ra)[2], float (&rb)[2]) {
      if (MODE == kAlpha || j >= L) return;
      const long long t = FWD ? j : L - 1 - j;
      const long long i0 = (b * L + t) * S + col0;
      ra[0] = A.ha[i0];
      ra[1] = A.ha[i0 + 16];
      if (MODE == kPsi || MODE == kPhi) {
        rb[0] = A.hb[i0];
        rb[1] = A.hb[i0 + 16];
      }
    };

    __syncthreads();  // the previous unit is done with every LDS buffer
    stage_load(0);
    stage_store(0);
    __syncthreads();

    // per-chain state carried between steps
    float ell[2] = {0.f, 0.f}, ref = 0.f;  // alpha: emission and shift of step t
    float nl[2] = {0.f, 0.f};              // alpha: emission of the step after
    float sc_prev = 1.f;                   // scale of the next product output
    float p_wh = 0.f, p_wt = 0.f;          // Psi: w_hat_t and w_t of the step awaiting its sum
    double lz = 0.0;                       // alpha: log2 Z
    if (MODE == kAlpha) {
      const float w0 = A.w[b * L];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float d = w0 - cc[e];
        ell[e] = -kap * d * d;
      }
      const float v[1] = {fmaxf(ell[0], ell[1])};
      float out[1];
      publish<1, 1, C::NW>(v, red[1], l, wv);
      __syncthreads();
      collect<1, 1, C::NW>(red[1], l, out);
      ref = out[0];
    }

    // Per-chain sums of step jp, published before the barrier that ended it, are collected in
    // the next step after its product has been issued, so that they overlap the matrix work.
    auto finish = [&](long long jp) {
      const long long tp = FWD ? jp : L - 1 - jp;
      const long long itp = b * L + tp;
      const bool writer = wv == 0 && (l & 15) == 0 && valid;  // one lane per chain
      if constexpr (MODE == kAlpha) {
        float out[2];
        collect<2, 2, C::NW>(red[jp & 1], l, out);
        sc_prev = 1.f / out[0];
        lz += (double)ref + (double)lg2(out[0]);
        if (writer) {
          A.pack[itp * 4 + 2] = ref;
          if (tp == 0) A.pack[itp * 4 + 3] = 1.f;
          if (tp + 1 < L) A.pack[(itp + 1) * 4 + 3] = sc_prev;
        }
        ref = out[1];
        ell[0] = nl[0];
        ell[1] = nl[1];
      } else if constexpr (MODE == kBeta) {
        float out[2];
        collect<2, 0, C::NW>(red[jp & 1], l, out);
        sc_prev = 1.f / out[0];
        if (writer) {
          const float wh = out[1] / out[0];
          A.pack[itp * 4 + 0] = wh;
          A.pack[itp * 4 + 1] = sc_prev;
          A.w_hat[itp] = wh;
        }
      } else if constexpr (MODE == kPsi) {
        float out[1];
        collect<1, 0, C::NW>(red[jp & 1], l, out);
        if (writer) A.grad_w[itp] = A.two_t * (out[0] + hh * (p_wh - p_wt));
      } else {
        float out[1];
        collect<1, 0, C::NW>(red[jp & 1], l, out);
        if (writer) A.grad_w[itp] += A.two_t * out[0];
      }
    };

    auto step = [&](long long j, float (&rn)[2], float (&rbn)[2]) {
      const long long t = FWD ? j : L - 1 - j;
      const int buf = (int)(j & 1);
      const long long cidx = j / kChunk;
      const int tt = (int)(j - cidx * kChunk);
      const float* scb = sc[cidx & 1] + tt * NQ * 4 + ch;
      // this step's history values, then the loads of step j + 2 into the same registers:
      // issued before this step's stores, since loads and stores share one in-order
      // completion counter and a later wait for the loads would also wait for those stores
      const float ra[2] = {rn[0], rn[1]}, rb[2] = {rbn[0], rbn[1]};
      hist_load(j + 2, rn, rbn);
      float o[2] = {0.f, 0.f};
      if (j > 0) {
        product<C>(xs[buf ^ 1], m, l, o);
        finish(j - 1);
      }
      float* xw = xs[buf] + xo;
      const long long i0 = (b * L + t) * S + col0;

      if constexpr (MODE == kAlpha) {
        const float wn = scb[0];  // w_{t+1}
        float a[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          a[e] = (j > 0 ? o[e] * sc_prev : 1.f) * ex2(ell[e] - ref);
          xw[4 * e] = a[e];
          if (valid) A.ha[i0 + 16 * e] = a[e];
          const float d = wn - cc[e];
          nl[e] = ck[e] - kap * d * d;
        }
        const float v[2] = {a[0] + a[1], fmaxf(nl[0], nl[1])};
        publish<2, 2, C::NW>(v, red[buf], l, wv);
      } else if constexpr (MODE == kBeta) {
        const float wt = scb[0], rf = scb[4];
        float p[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float u = j > 0 ? o[e] * sc_prev : 1.f;
          if (valid) A.hb[i0 + 16 * e] = u;
          if (t > 0) {
            const float d = wt - cc[e];
            xw[4 * e] = ex2(ck[e] - kap * d * d - rf) * u;
          }
          p[e] = ra[e] * u;
        }
        const float v[2] = {p[0] + p[1], cc[0] * p[0] + cc[1] * p[1]};
        publish<2, 0, C::NW>(v, red[buf], l, wv);
      } else if constexpr (MODE == kPsi) {
        const float wt = scb[0], gt = scb[4], wh = scb[8], rz = scb[12], rf = scb[16], inv = scb[20];
        float D[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float a = ra[e], u = rb[e];
          const float bu = u * (gt * (cc[e] - wh)) + (j > 0 ? o[e] * sc_prev : 0.f);
          D[e] = a * bu * rz;
          const float gm = a * u * rz;
          gc[e] += fv * (gt * gm + A.two_t * (wt - cc[e]) * (D[e] + hh * gm));
          if (t > 0) {
            const float d = wt - cc[e];
            const float ee = ex2(ck[e] - kap * d * d - rf);
            const float z = ee * bu;
            xw[4 * e] = z;
            const float q = inv * rz;
            if (valid) {
              A.r1[i0 + 16 * e] = ee * u * q;
              A.r2[i0 + 16 * e] = z * q;
            }
          }
        }
        const float v[1] = {cc[0] * D[0] + cc[1] * D[1]};
        publish<1, 0, C::NW>(v, red[buf], l, wv);
        sc_prev = rz;
        p_wh = wh;
        p_wt = wt;
      } else {  // kPhi
        const float wt = scb[0], gt = scb[4], wh = scb[8], rz = scb[12], rf = scb[16], inv = scb[20];
        float D[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          float at = 0.f;
          if (j > 0) {
            const float d = wt - cc[e];
            at = o[e] * inv * ex2(ck[e] - kap * d * d - rf);
          }
          const float a = ra[e], u = rb[e];
          D[e] = at * u * rz;
          gc[e] += fv * (A.two_t * (wt - cc[e]) * D[e]);
          if (t + 1 < L) {
            const float x = at + a * (gt * (cc[e] - wh));
            xw[4 * e] = x;
            if (valid) A.l1[i0 + 16 * e] = x + hh * a;
          }
        }
        const float v[1] = {cc[0] * D[0] + cc[1] * D[1]};
        publish<1, 0, C::NW>(v, red[buf], l, wv);
      }
      if (tt == kChunk - 1 && cidx + 1 < nch) stage_store((int)((cidx + 1) & 1));
      __syncthreads();
      if (tt == 0 && cidx + 1 < nch) stage_load(cidx + 1);
    };

    float ra0[2] = {0.f, 0.f}, rb0[2] = {0.f, 0.f}, ra1[2] = {0.f, 0.f}, rb1[2] = {0.f, 0.f};
    hist_load(0, ra0, rb0);
    hist_load(1, ra1, rb1);
    for (long long j = 0; j < L; j += 2) {
      step(j, ra0, rb0);
      if (j + 1 < L) step(j + 1, ra1, rb1);
    }
    finish(L - 1);
    if (MODE == kAlpha && wv == 0 && (l & 15) == 0 && valid) {
      A.lz2[b] = lz;
      A.log_z[b] = (float)(lz * kLn2D);
    }
  }
  if (MODE == kPsi || MODE == kPhi) {
    // sum the four chains (rows) of every state
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const P2 r = swap32(gc[e], gc[e]);
      const float x = r.lo + r.hi;
      const P2 q = swap16(x, x);
      if (l < 16) A.gc_part[(long long)blockIdx.x * S + col0 + 16 * e] = q.lo + q.hi;
    }
  }
}

// Column maxima cm(s') of theta, M = 2^(kappa (theta - cm)) and kappa cm. One block per column.
__global__ void __launch_bounds__(256)
k_dense_prep(const float* __restrict__ theta, int S, float kap, float* __restrict__ mat,
             float* __restrict__ cmk) {
  __shared__ float red[4];
  const int sp = blockIdx.x, s = threadIdx.x;
  const float th = s < S ? theta[s * S + sp] : -INFINITY;
  float m = th;
  m = fmaxf(m, __shfl_xor(m, 32, 64));
  m = fmaxf(m, __shfl_xor(m, 16, 64));
  m = fmaxf(m, __shfl_xor(m, 8, 64));
  m = fmaxf(m, __shfl_xor(m, 4, 64));
  m = fmaxf(m, __shfl_xor(m, 2, 64));
  m = fmaxf(m, __shfl_xor(m, 1, 64));
  if ((s & 63) == 0) red[s >> 6] = m;
  __syncthreads();
  const float cm = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  if (s < S) mat[s * S + sp] = ex2(kap * (th - cm));
  if (s == 0) cmk[sp] = kap * cm;
}

// ---- theta gradient: G = sum over (chain, t >= 1) of L1_{t-1} (x) R1_t + a_{t-1} (x) R2_t ----
// Split-K over all (chain, step) pairs: block j sums a contiguous range of 8-pair chunks into a
// full S x S partial. A chunk is 16 rows (pair p, term) of left and right vectors, staged in LDS
// as [state][row % 4][row / 4] (row stride 20 floats) so that one 16-byte read gives the four
// k-steps of an MFMA 16x16x4 operand. Loader lanes take the 16 rows of one group of 4 states in
// turn, so that their transposing LDS stores fall into distinct banks.
template <int S_>
struct GGeo {
  static constexpr int S = S_;
  static constexpr int WT = S >= 64 ? 64 : S;  // wave tile edge
  static constexpr int WD = S / WT;            // wave tiles per dimension
  static constexpr int NWG = WD * WD;
  static constexpr int BLOCK = 64 * NWG;
  static constexpr int TPW = WT / 16;          // 16x16 tiles per wave per dimension
  static constexpr int PC = 8;                 // pairs per chunk (16 rows)
  static constexpr int LSTR = 20;
  static constexpr int NI = (16 * S / 4 + BLOCK - 1) / BLOCK;  // float4 loads per thread per operand
};

struct GemmArgs {
  const float* l1;
  const float* ha;
  const float* r1;
  const float* r2;
  long long L, pairs, chunks;
  float* part;  // [gridDim.x, S, S]
};

template <int S>
__global__ void __launch_bounds__(GGeo<S>::BLOCK)
k_dense_theta_gemm(GemmArgs A) {
  using G = GGeo<S>;
  __shared__ __attribute__((aligned(16))) float ls[2][S * G::LSTR];
  __shared__ __attribute__((aligned(16))) float rs[2][S * G::LSTR];
  const int tid = threadIdx.x, l = tid & 63, wv = tid >> 6;
  const int sb = (wv / G::WD) * G::WT, sbp = (wv % G::WD) * G::WT;
  const long long c0 = A.chunks * blockIdx.x / gridDim.x;
  const long long c1 = A.chunks * (blockIdx.x + 1) / gridDim.x;
  const long long Lm1 = A.L - 1;

  f4 vl[G::NI], vr[G::NI];
  auto load = [&](long long c) {
#pragma unroll
    for (int p = 0; p < G::NI; ++p) {
      const int idx = tid + p * G::BLOCK;
      vl[p] = vr[p] = f4{0.f, 0.f, 0.f, 0.f};
      if (idx < 16 * S / 4) {
        const int kr = idx & 15, s = 4 * (idx >> 4);
        const long long pr = c * G::PC + (kr >> 1);
        if (pr < A.pairs) {
          const long long b = pr / Lm1, t = 1 + pr % Lm1;
          const long long li = (b * A.L + t - 1) * S + s, ri = (b * A.L + t) * S + s;
          const float* lp = (kr & 1) ? A.ha : A.l1;
          const float* rp = (kr & 1) ? A.r2 : A.r1;
          vl[p] = *reinterpret_cast<const f4*>(lp + li);
          vr[p] = *reinterpret_cast<const f4*>(rp + ri);
        }
      }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int p = 0; p < G::NI; ++p) {
      const int idx = tid + p * G::BLOCK;
      if (idx < 16 * S / 4) {
        const int kr = idx & 15, s = 4 * (idx >> 4);
        const int off = (kr & 3) * 4 + (kr >> 2);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ls[buf][(s + e) * G::LSTR + off] = vl[p][e];
          rs[buf][(s + e) * G::LSTR + off] = vr[p][e];
        }
      }
    }
  };

  f4 acc[G::TPW][G::TPW];
#pragma unroll
  for (int i = 0; i < G::TPW; ++i)
#pragma unroll
    for (int k = 0; k < G::TPW; ++k) acc[i][k] = f4{0.f, 0.f, 0.f, 0.f};

  if (c0 < c1) {
    load(c0);
    store(0);
  }
  __syncthreads();
  for (long long c = c0; c < c1; ++c) {
    const int buf = (int)((c - c0) & 1);
    if (c + 1 < c1) load(c + 1);
    f4 af[G::TPW], bf[G::TPW];
#pragma unroll
    for (int i = 0; i < G::TPW; ++i) {
      af[i] = *reinterpret_cast<const f4*>(&ls[buf][(sb + 16 * i + (l & 15)) * G::LSTR + (l >> 4) * 4]);
      bf[i] = *reinterpret_cast<const f4*>(&rs[buf][(sbp + 16 * i + (l & 15)) * G::LSTR + (l >> 4) * 4]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < G::TPW; ++i)
#pragma unroll
        for (int k = 0; k < G::TPW; ++k)
          acc[i][k] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i][q], bf[k][q], acc[i][k], 0, 0, 0);
    if (c + 1 < c1) store(buf ^ 1);
    __syncthreads();
  }
  float* out = A.part + (long long)blockIdx.x * S * S;
#pragma unroll
  for (int i = 0; i < G::TPW; ++i)
#pragma unroll
    for (int k = 0; k < G::TPW; ++k)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        out[(sb + 16 * i + 4 * (l >> 4) + r) * S + sbp + 16 * k + (l & 15)] = acc[i][k][r];
}

// out[e] = scale * mul[e] * sum_j part[j * n + e] (mul may be null), summed over j in a fixed
// order: four contiguous quarters of j, each in order, then the quarters in order. A block
// covers 64 consecutive e.
__global__ void __launch_bounds__(256)
k_dense_sum_parts(const float* __restrict__ part, int np, long long n, const float* __restrict__ mul,
                  float scale, float* __restrict__ out) {
  __shared__ float red[4][64];
  const int el = threadIdx.x & 63, q = threadIdx.x >> 6;
  const long long e = (long long)blockIdx.x * 64 + el;
  float acc = 0.f;
  if (e < n) {
    const int j0 = np * q / 4, j1 = np * (q + 1) / 4;
    int j = j0;
    for (; j + 8 <= j1; j += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[(long long)(j + u) * n + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += v[u];
    }
    for (; j < j1; ++j) acc += part[(long long)j * n + e];
  }
  red[q][el] = acc;
  __syncthreads();
  if (q == 0 && e < n) {
    const float tot = ((red[0][el] + red[1][el]) + red[2][el]) + red[3][el];
    out[e] = mul != nullptr ? scale * mul[e] * tot : tot;
  }
}

template <int S, int MODE>
int sweep_grid(long long units) {
  const void* kern = reinterpret_cast<const void*>(&k_dense_sweep<S, MODE>);
  return resident_grid(kern, DGeo<S>::BLOCK, dense_sweep_slots(units));
}

template <int S, int MODE>
int run_sweep(const SweepArgs& a, int grid, hipStream_t st) {
  hipLaunchKernelGGL((k_dense_sweep<S, MODE>), dim3(grid), dim3(DGeo<S>::BLOCK), 0, st, a);
  return (int)hipGetLastError();
}

template <int S>
int run_forward(const float* theta, const float* cb, const float* w, int64_t B, int64_t L, float T,
                float* w_hat, float* log_z, void* saved, void* ws, hipStream_t st) {
  DenseLayout d;
  dense_layout(S, B, L, &d);
  char* sv = static_cast<char*>(saved);
  char* wk = static_cast<char*>(ws);
  const float kap = kLog2eF / T;
  float* mat = reinterpret_cast<float*>(wk + d.mat);
  float* cmk = reinterpret_cast<float*>(wk + d.cmk);
  SweepArgs a = {};
  a.mat = mat;
  a.cmk = cmk;
  a.cb = cb;
  a.w = w;
  a.B = B;
  a.L = L;
  a.units = (B + 3) / 4;
  a.kap = kap;
  a.two_t = 2.f / T;
  a.pack = reinterpret_cast<float*>(sv + d.pack);
  a.lz2 = reinterpret_cast<double*>(sv + d.lz2);
  a.log_z = log_z;
  a.w_hat = w_hat;
  a.ha = reinterpret_cast<float*>(sv + d.ha);
  a.hb = reinterpret_cast<float*>(sv + d.hb);
  const int ga = sweep_grid<S, kAlpha>(a.units), gb = sweep_grid<S, kBeta>(a.units);
  if (ga <= 0 || gb <= 0) return (int)hipErrorInvalidDevice;
  hipLaunchKernelGGL(k_dense_prep, dim3(S), dim3(256), 0, st, theta, S, kap, mat, cmk);
  int e = (int)hipGetLastError();
  if (e) return e;
  if ((e = run_sweep<S, kAlpha>(a, ga, st))) return e;
  return run_sweep<S, kBeta>(a, gb, st);
}

template <int S>
int run_backward(const float* theta, const float* cb, const float* w, int64_t B, int64_t L, float T,
                 const void* saved, const float* g, const float* h, float* grad_w, float* grad_c,
                 float* grad_theta, void* ws, hipStream_t st) {
  using G = GGeo<S>;
  DenseLayout d;
  dense_layout(S, B, L, &d);
  char* sv = const_cast<char*>(static_cast<const char*>(saved));
  char* wk = static_cast<char*>(ws);
  const float kap = kLog2eF / T;
  float* mat = reinterpret_cast<float*>(wk + d.mat);
  float* cmk = reinterpret_cast<float*>(wk + d.cmk);
  float* gcp = reinterpret_cast<float*>(wk + d.gcp);
  SweepArgs a = {};
  a.mat = mat;
  a.cmk = cmk;
  a.cb = cb;
  a.w = w;
  a.g = g;
  a.h = h;
  a.B = B;
  a.L = L;
  a.units = (B + 3) / 4;
  a.kap = kap;
  a.two_t = 2.f / T;
  a.pack = reinterpret_cast<float*>(sv + d.pack);
  a.ha = reinterpret_cast<float*>(sv + d.ha);
  a.hb = reinterpret_cast<float*>(sv + d.hb);
  a.l1 = reinterpret_cast<float*>(wk + d.l1);
  a.r1 = reinterpret_cast<float*>(wk + d.r1);
  a.r2 = reinterpret_cast<float*>(wk + d.r2);
  a.grad_w = grad_w;

  GemmArgs ga;
  ga.l1 = a.l1;
  ga.ha = a.ha;
  ga.r1 = a.r1;
  ga.r2 = a.r2;
  ga.L = L;
  ga.pairs = B * (L - 1);
  ga.chunks = (ga.pairs + G::PC - 1) / G::PC;
  ga.part = reinterpret_cast<float*>(wk + d.gp);

  const int gpsi = sweep_grid<S, kPsi>(a.units), gphi = sweep_grid<S, kPhi>(a.units);
  int gg = resident_grid(reinterpret_cast<const void*>(&k_dense_theta_gemm<S>), G::BLOCK,
                         kDenseGemmMaxGrid);
  if (gpsi <= 0 || gphi <= 0 || gg <= 0) return (int)hipErrorInvalidDevice;
  if (ga.chunks > 0 && gg > ga.chunks) gg = (int)ga.chunks;

  hipLaunchKernelGGL(k_dense_prep, dim3(S), dim3(256), 0, st, theta, S, kap, mat, cmk);
  int e = (int)hipGetLastError();
  if (e) return e;
  a.gc_part = gcp;
  if ((e = run_sweep<S, kPsi>(a, gpsi, st))) return e;
  a.gc_part = gcp + (size_t)gpsi * S;
  if ((e = run_sweep<S, kPhi>(a, gphi, st))) return e;
  hipLaunchKernelGGL(k_dense_theta_gemm<S>, dim3(gg), dim3(G::BLOCK), 0, st, ga);
  if ((e = (int)hipGetLastError())) return e;
  const long long nt = (long long)S * S;
  hipLaunchKernelGGL(k_dense_sum_parts, dim3((unsigned)((nt + 63) / 64)), dim3(256), 0, st, ga.part,
                     gg, nt, mat, 1.f / T, grad_theta);
  if ((e = (int)hipGetLastError())) return e;
  hipLaunchKernelGGL(k_dense_sum_parts, dim3((unsigned)((S + 63) / 64)), dim3(256), 0, st, gcp,
                     gpsi + gphi, (long long)S, nullptr, 1.f, grad_c);
  return (int)hipGetLastError();
}

}  // namespace

bool dense_shape_built(int S) { return S == 32 || S == 64 || S == 128 || S == 256; }

int launch_dense_forward(int S, const float* theta, const float* codebook, const float* w, int64_t B,
                         int64_t L, float T, float* w_hat, float* log_z, void* saved, void* ws,
                         void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (S) {
    case 32: return run_forward<32>(theta, codebook, w, B, L, T, w_hat, log_z, saved, ws, st);
    case 64: return run_forward<64>(theta, codebook, w, B, L, T, w_hat, log_z, saved, ws, st);
    case 128: return run_forward<128>(theta, codebook, w, B, L, T, w_hat, log_z, saved, ws, st);
    case 256: return run_forward<256>(theta, codebook, w, B, L, T, w_hat, log_z, saved, ws, st);
  }
  return (int)hipErrorInvalidValue;
}

int launch_dense_backward(int S, const float* theta, const float* codebook, const float* w,
                          int64_t B, int64_t L, float T, const void* saved, const float* grad_w_hat,
                          const float* grad_log_z, float* grad_w, float* grad_codebook,
                          float* grad_theta, void* ws, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  switch (S) {
    case 32:
      return run_backward<32>(theta, codebook, w, B, L, T, saved, grad_w_hat, grad_log_z, grad_w,
                              grad_codebook, grad_theta, ws, st);
    case 64:
      return run_backward<64>(theta, codebook, w, B, L, T, saved, grad_w_hat, grad_log_z, grad_w,
                              grad_codebook, grad_theta, ws, st);
    case 128:
      return run_backward<128>(theta, codebook, w, B, L, T, saved, grad_w_hat, grad_log_z, grad_w,
                               grad_codebook, grad_theta, ws, st);
    case 256:
      return run_backward<256>(theta, codebook, w, B, L, T, saved, grad_w_hat, grad_log_z, grad_w,
                               grad_codebook, grad_theta, ws, st);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace bcjr

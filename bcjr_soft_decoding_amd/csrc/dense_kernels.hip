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
// all chains and steps) and k_dense_finalize (fixed-order sums of the block partials).
//
// Sweep tiling: one block per 4 chains, S/32 waves; wave wv owns output states 32wv..32wv+31.
// The step product runs on v_mfma_f32_4x4x1f32 (16 independent 4x4 outer products): block b of
// an instruction takes chain i = lane & 3, input state k = 4 kc + (lane >> 4) and output state
// 32 wv + 16 set + (lane & 15), so lane l keeps M[4kc + l/16][32wv + 16set + l%16] (the
// transposed entry for the backward sweeps) in registers for the whole launch: the matrix lives
// in the register files of one block. The four partial sums over k (lane bits 4 and 5) are
// folded with v_permlane32_swap / v_permlane16_swap as a reduce-scatter, which leaves each lane
// with two (chain, state) results. Messages are staged in LDS as [k % 4][chain][k / 4] so that a
// lane reads four consecutive MFMA operands with one 16-byte load.
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

// out[chain 2*bit4 + r][state 32wv + 16*bit5 + (lane & 15)] of the product of the staged message
// (4 chains) with the register-resident matrix.
template <class C>
__device__ __forceinline__ void product(const float* __restrict__ xs, const float (&m)[C::MR], int l,
                                        float& o0, float& o1) {
  const float* xr = xs + ((l >> 4) * 4 + (l & 3)) * C::XSTR;
  f4 acc[2][2];
#pragma unroll
  for (int s = 0; s < 2; ++s) acc[s][0] = acc[s][1] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kc = 0; kc < C::KC; kc += 4) {
    const f4 a = *reinterpret_cast<const f4*>(xr + kc);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[0][e & 1] = __builtin_amdgcn_mfma_f32_4x4x1f32(a[e], m[2 * (kc + e)], acc[0][e & 1], 0, 0, 0);
      acc[1][e & 1] = __builtin_amdgcn_mfma_f32_4x4x1f32(a[e], m[2 * (kc + e) + 1], acc[1][e & 1], 0, 0, 0);
    }
  }
  const f4 s0 = acc[0][0] + acc[0][1];
  const f4 s1 = acc[1][0] + acc[1][1];
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const P2 r = swap32(s0[i], s1[i]);  // lanes 0-31 keep set 0, lanes 32-63 set 1
    v[i] = r.lo + r.hi;
  }
  const P2 r0 = swap16(v[0], v[2]);  // rows 0, 2 keep chain 0; rows 1, 3 chain 2
  const P2 r1 = swap16(v[1], v[3]);
  o0 = r0.lo + r0.hi;
  o1 = r1.lo + r1.hi;
}

// Block-wide reduction of per-chain quantities over the S states. v[q][r] is this lane's value
// of quantity q for chain ch0 + r; bit q of MAXQ selects a max instead of a sum. Returns the
// block totals for the lane's two chains in out[q][r]. Contains the step's barrier.
template <int NQR, int MAXQ, int NW>
__device__ __forceinline__ void chain_reduce(const float (&v)[NQR][2], float* __restrict__ red, int l,
                                             int wv, float (&out)[NQR][2]) {
#pragma unroll
  for (int q = 0; q < NQR; ++q) {
    float tot;
    if ((MAXQ >> q) & 1) {
      const P2 r = swap32(row_red<true>(v[q][0]), row_red<true>(v[q][1]));
      tot = fmaxf(r.lo, r.hi);
    } else {
      const P2 r = swap32(row_red<false>(v[q][0]), row_red<false>(v[q][1]));
      tot = r.lo + r.hi;
    }
    // lanes 0, 16, 32, 48 hold chains 0, 2, 1, 3
    if ((l & 15) == 0) red[(q * 4 + 2 * ((l >> 4) & 1) + (l >> 5)) * NW + wv] = tot;
  }
  __syncthreads();
  const float x = l < NQR * 4 * NW ? red[l] : 0.f;
  const float sx = group_red<NW, false>(x);
  const float mx = group_red<NW, true>(x);
  const int ql = l / (4 * NW);
  const float tot = ((MAXQ >> ql) & 1) ? mx : sx;
  const int ch0 = 2 * ((l >> 4) & 1);
#pragma unroll
  for (int q = 0; q < NQR; ++q) {
    out[q][0] = __shfl(tot, (q * 4 + ch0) * NW, 64);
    out[q][1] = __shfl(tot, (q * 4 + ch0 + 1) * NW, 64);
  }
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
  const int col = 32 * wv + (l & 15) + 16 * (l >> 5);
  const int ch0 = 2 * ((l >> 4) & 1);
  const float cc = A.cb[col];
  const float cmk = A.cmk[col];
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
  // where this lane stages its two values (state col, chains ch0 and ch0 + 1)
  const int xo = ((col & 3) * 4 + ch0) * C::XSTR + (col >> 2);
  float gc = 0.f;

  for (long long unit = blockIdx.x; unit < A.units; unit += gridDim.x) {
    const long long b0 = unit * 4;
    const long long bA = b0 + ch0 < B ? b0 + ch0 : B - 1;
    const long long bB = b0 + ch0 + 1 < B ? b0 + ch0 + 1 : B - 1;
    const bool vA = b0 + ch0 < B, vB = b0 + ch0 + 1 < B;
    const float fA = vA ? 1.f : 0.f, fB = vB ? 1.f : 0.f;
    float hA = 0.f, hB = 0.f;
    if ((MODE == kPsi || MODE == kPhi) && A.h != nullptr) {
      hA = A.h[bA];
      hB = A.h[bB];
    }

    float sr[NPT];
    auto stage_load = [&](long long c) {
#pragma unroll
      for (int p = 0; p < NPT; ++p) {
        const int idx = tid + p * C::BLOCK;
        sr[p] = 0.f;
        if (idx < NSC) {
          const int tt = idx / (NQ * 4), q = (idx >> 2) % NQ, ch = idx & 3;
          const long long j = c * kChunk + tt;
          const long long b = b0 + ch < B ? b0 + ch : B - 1;
          if (j < L) sr[p] = fetch_scalar<MODE>(A, q, b, FWD ? j : L - 1 - j);
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
      const long long iA = (bA * L + t) * S + col, iB = (bB * L + t) * S + col;
      ra[0] = A.ha[iA];
      ra[1] = A.ha[iB];
      if (MODE == kPsi || MODE == kPhi) {
        rb[0] = A.hb[iA];
        rb[1] = A.hb[iB];
      }
    };

    __syncthreads();  // the previous unit is done with every LDS buffer
    stage_load(0);
    stage_store(0);
    __syncthreads();

    // per-chain state carried between steps
    float ellA = 0.f, ellB = 0.f, refA = 0.f, refB = 0.f;  // alpha: emission and shift of step t
    float sA = 1.f, sB = 1.f;                              // scale of the next product output
    double lzA = 0.0, lzB = 0.0;                           // alpha: log2 Z
    if (MODE == kAlpha) {
      const float d0 = A.w[bA * L] - cc, d1 = A.w[bB * L] - cc;
      ellA = -kap * d0 * d0;
      ellB = -kap * d1 * d1;
      const float v[1][2] = {{ellA, ellB}};
      float out[1][2];
      chain_reduce<1, 1, C::NW>(v, red[1], l, wv, out);
      refA = out[0][0];
      refB = out[0][1];
    }

    auto step = [&](long long j, float (&ra)[2], float (&rb)[2]) {
      const long long t = FWD ? j : L - 1 - j;
      const int buf = (int)(j & 1);
      const long long cidx = j / kChunk;
      const int tt = (int)(j - cidx * kChunk);
      const float* scb = sc[cidx & 1] + tt * NQ * 4 + ch0;
      float o0 = 0.f, o1 = 0.f;
      if (j > 0) product<C>(xs[buf ^ 1], m, l, o0, o1);
      float* xw = xs[buf] + xo;
      const long long iA = bA * L + t, iB = bB * L + t;
      const bool last = tt == kChunk - 1 && cidx + 1 < nch;

      if constexpr (MODE == kAlpha) {
        const float aA = (j > 0 ? o0 * sA : 1.f) * ex2(ellA - refA);
        const float aB = (j > 0 ? o1 * sB : 1.f) * ex2(ellB - refB);
        xw[0] = aA;
        xw[C::XSTR] = aB;
        if (vA) A.ha[iA * S + col] = aA;
        if (vB) A.ha[iB * S + col] = aB;
        const f2 wn = *reinterpret_cast<const f2*>(scb);  // w_{t+1}
        const float dA = wn[0] - cc, dB = wn[1] - cc;
        const float nA = cmk - kap * dA * dA, nB = cmk - kap * dB * dB;
        const float v[2][2] = {{aA, aB}, {nA, nB}};
        float out[2][2];
        if (last) stage_store((int)((cidx + 1) & 1));
        chain_reduce<2, 2, C::NW>(v, red[buf], l, wv, out);
        if (tt == 0 && cidx + 1 < nch) stage_load(cidx + 1);
        sA = 1.f / out[0][0];
        sB = 1.f / out[0][1];
        lzA += (double)refA + (double)lg2(out[0][0]);
        lzB += (double)refB + (double)lg2(out[0][1]);
        if (wv == 0 && (l & 47) == 0) {  // lanes 0 and 16: chains (0, 1) and (2, 3)
          if (vA) {
            A.pack[iA * 4 + 2] = refA;
            if (t == 0) A.pack[iA * 4 + 3] = 1.f;
            if (t + 1 < L) A.pack[(iA + 1) * 4 + 3] = sA;
          }
          if (vB) {
            A.pack[iB * 4 + 2] = refB;
            if (t == 0) A.pack[iB * 4 + 3] = 1.f;
            if (t + 1 < L) A.pack[(iB + 1) * 4 + 3] = sB;
          }
        }
        ellA = nA;
        ellB = nB;
        refA = out[1][0];
        refB = out[1][1];
      } else if constexpr (MODE == kBeta) {
        const float uA = j > 0 ? o0 * sA : 1.f;
        const float uB = j > 0 ? o1 * sB : 1.f;
        const float aA = ra[0], aB = ra[1];
        if (vA) A.hb[iA * S + col] = uA;
        if (vB) A.hb[iB * S + col] = uB;
        if (t > 0) {
          const f2 wt = *reinterpret_cast<const f2*>(scb);
          const f2 rf = *reinterpret_cast<const f2*>(scb + 4);
          const float dA = wt[0] - cc, dB = wt[1] - cc;
          xw[0] = ex2(cmk - kap * dA * dA - rf[0]) * uA;
          xw[C::XSTR] = ex2(cmk - kap * dB * dB - rf[1]) * uB;
        }
        const float pA = aA * uA, pB = aB * uB;
        const float v[2][2] = {{pA, pB}, {cc * pA, cc * pB}};
        float out[2][2];
        if (last) stage_store((int)((cidx + 1) & 1));
        chain_reduce<2, 0, C::NW>(v, red[buf], l, wv, out);
        if (tt == 0 && cidx + 1 < nch) stage_load(cidx + 1);
        sA = 1.f / out[0][0];
        sB = 1.f / out[0][1];
        if (wv == 0 && (l & 47) == 0) {
          if (vA) {
            const float wh = out[1][0] / out[0][0];
            A.pack[iA * 4 + 0] = wh;
            A.pack[iA * 4 + 1] = sA;
            A.w_hat[iA] = wh;
          }
          if (vB) {
            const float wh = out[1][1] / out[0][1];
            A.pack[iB * 4 + 0] = wh;
            A.pack[iB * 4 + 1] = sB;
            A.w_hat[iB] = wh;
          }
        }
      } else if constexpr (MODE == kPsi) {
        const f2 wt = *reinterpret_cast<const f2*>(scb);
        const f2 gt = *reinterpret_cast<const f2*>(scb + 4);
        const f2 wh = *reinterpret_cast<const f2*>(scb + 8);
        const f2 rz = *reinterpret_cast<const f2*>(scb + 12);
        const f2 rf = *reinterpret_cast<const f2*>(scb + 16);
        const f2 inv = *reinterpret_cast<const f2*>(scb + 20);
        const float vvA = j > 0 ? o0 * sA : 0.f, vvB = j > 0 ? o1 * sB : 0.f;
        const float aA = ra[0], aB = ra[1], uA = rb[0], uB = rb[1];
        const float buA = uA * (gt[0] * (cc - wh[0])) + vvA;
        const float buB = uB * (gt[1] * (cc - wh[1])) + vvB;
        const float DA = aA * buA * rz[0], DB = aB * buB * rz[1];
        const float gmA = aA * uA * rz[0], gmB = aB * uB * rz[1];
        gc += fA * (gt[0] * gmA + A.two_t * (wt[0] - cc) * (DA + hA * gmA));
        gc += fB * (gt[1] * gmB + A.two_t * (wt[1] - cc) * (DB + hB * gmB));
        if (t > 0) {
          const float dA = wt[0] - cc, dB = wt[1] - cc;
          const float eA = ex2(cmk - kap * dA * dA - rf[0]);
          const float eB = ex2(cmk - kap * dB * dB - rf[1]);
          const float zA = eA * buA, zB = eB * buB;
          xw[0] = zA;
          xw[C::XSTR] = zB;
          const float qA = inv[0] * rz[0], qB = inv[1] * rz[1];
          if (vA) {
            A.r1[iA * S + col] = eA * uA * qA;
            A.r2[iA * S + col] = zA * qA;
          }
          if (vB) {
            A.r1[iB * S + col] = eB * uB * qB;
            A.r2[iB * S + col] = zB * qB;
          }
        }
        const float v[1][2] = {{cc * DA, cc * DB}};
        float out[1][2];
        if (last) stage_store((int)((cidx + 1) & 1));
        chain_reduce<1, 0, C::NW>(v, red[buf], l, wv, out);
        if (tt == 0 && cidx + 1 < nch) stage_load(cidx + 1);
        sA = rz[0];
        sB = rz[1];
        if (wv == 0 && (l & 47) == 0) {
          if (vA) A.grad_w[iA] = A.two_t * (out[0][0] + hA * (wh[0] - wt[0]));
          if (vB) A.grad_w[iB] = A.two_t * (out[0][1] + hB * (wh[1] - wt[1]));
        }
      } else {  // kPhi
        const f2 wt = *reinterpret_cast<const f2*>(scb);
        const f2 gt = *reinterpret_cast<const f2*>(scb + 4);
        const f2 wh = *reinterpret_cast<const f2*>(scb + 8);
        const f2 rz = *reinterpret_cast<const f2*>(scb + 12);
        const f2 rf = *reinterpret_cast<const f2*>(scb + 16);
        const f2 inv = *reinterpret_cast<const f2*>(scb + 20);
        float atA = 0.f, atB = 0.f;
        if (j > 0) {
          const float dA = wt[0] - cc, dB = wt[1] - cc;
          atA = o0 * inv[0] * ex2(cmk - kap * dA * dA - rf[0]);
          atB = o1 * inv[1] * ex2(cmk - kap * dB * dB - rf[1]);
        }
        const float aA = ra[0], aB = ra[1], uA = rb[0], uB = rb[1];
        const float DA = atA * uA * rz[0], DB = atB * uB * rz[1];
        gc += fA * (A.two_t * (wt[0] - cc) * DA);
        gc += fB * (A.two_t * (wt[1] - cc) * DB);
        if (t + 1 < L) {
          const float xA = atA + aA * (gt[0] * (cc - wh[0]));
          const float xB = atB + aB * (gt[1] * (cc - wh[1]));
          xw[0] = xA;
          xw[C::XSTR] = xB;
          if (vA) A.l1[iA * S + col] = xA + hA * aA;
          if (vB) A.l1[iB * S + col] = xB + hB * aB;
        }
        const float v[1][2] = {{cc * DA, cc * DB}};
        float out[1][2];
        if (last) stage_store((int)((cidx + 1) & 1));
        chain_reduce<1, 0, C::NW>(v, red[buf], l, wv, out);
        if (tt == 0 && cidx + 1 < nch) stage_load(cidx + 1);
        if (wv == 0 && (l & 47) == 0) {
          if (vA) A.grad_w[iA] += A.two_t * out[0][0];
          if (vB) A.grad_w[iB] += A.two_t * out[0][1];
        }
      }
      hist_load(j + 2, ra, rb);
    };

    float ra0[2] = {0.f, 0.f}, rb0[2] = {0.f, 0.f}, ra1[2] = {0.f, 0.f}, rb1[2] = {0.f, 0.f};
    hist_load(0, ra0, rb0);
    hist_load(1, ra1, rb1);
    for (long long j = 0; j < L; j += 2) {
      step(j, ra0, rb0);
      if (j + 1 < L) step(j + 1, ra1, rb1);
    }
    if (MODE == kAlpha && wv == 0 && (l & 47) == 0) {
      if (vA) {
        A.lz2[bA] = lzA;
        A.log_z[bA] = (float)(lzA * kLn2D);
      }
      if (vB) {
        A.lz2[bB] = lzB;
        A.log_z[bB] = (float)(lzB * kLn2D);
      }
    }
  }
  if (MODE == kPsi || MODE == kPhi) {
    // lanes l and l ^ 16 hold the same state (chains 0, 1 and 2, 3)
    const P2 r = swap16(gc, gc);
    if (((l >> 4) & 1) == 0) A.gc_part[(long long)blockIdx.x * S + col] = r.lo + r.hi;
  }
}

// M = 2^(kappa (theta - cm)), kappa cm; one thread per column s'.
__global__ void __launch_bounds__(256)
k_dense_prep(const float* __restrict__ theta, int S, float kap, float* __restrict__ mat,
             float* __restrict__ cmk) {
  const int sp = threadIdx.x;
  if (sp >= S) return;
  float cm = theta[sp];
  for (int s = 1; s < S; ++s) cm = fmaxf(cm, theta[s * S + sp]);
  for (int s = 0; s < S; ++s) mat[s * S + sp] = ex2(kap * (theta[s * S + sp] - cm));
  cmk[sp] = kap * cm;
}

// ---- theta gradient: G = sum over (chain, t >= 1) of L1_{t-1} (x) R1_t + a_{t-1} (x) R2_t ----
// Split-K over all (chain, step) pairs: block j sums a contiguous range of 8-pair chunks into a
// full S x S partial. A chunk is 16 rows (pair p, term) of left and right vectors, staged in LDS
// as [state][row % 4][row / 4] (row stride 20 floats) so that one 16-byte read gives the four
// k-steps of an MFMA 16x16x4 operand.
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
        const int kr = idx / (S / 4), s = 4 * (idx % (S / 4));
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
        const int kr = idx / (S / 4), s = 4 * (idx % (S / 4));
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

// grad_theta = (M / T) o sum_j part_j; grad_c = sum of the two sweeps' partials (fixed order).
__global__ void __launch_bounds__(256)
k_dense_finalize(const float* __restrict__ gpart, int ngrid, const float* __restrict__ mat,
                 float inv_t, float* __restrict__ grad_theta, const float* __restrict__ gcpart,
                 int ngc, float* __restrict__ grad_c, int S) {
  const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long SS = (long long)S * S;
  if (e < SS) {
    float acc = 0.f;
    for (int j = 0; j < ngrid; ++j) acc += gpart[j * SS + e];
    grad_theta[e] = inv_t * mat[e] * acc;
  } else if (e < SS + S) {
    const long long s = e - SS;
    float acc = 0.f;
    for (int j = 0; j < ngc; ++j) acc += gcpart[j * (long long)S + s];
    grad_c[s] = acc;
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
  hipLaunchKernelGGL(k_dense_prep, dim3(1), dim3(256), 0, st, theta, S, kap, mat, cmk);
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

  hipLaunchKernelGGL(k_dense_prep, dim3(1), dim3(256), 0, st, theta, S, kap, mat, cmk);
  int e = (int)hipGetLastError();
  if (e) return e;
  a.gc_part = gcp;
  if ((e = run_sweep<S, kPsi>(a, gpsi, st))) return e;
  a.gc_part = gcp + (size_t)gpsi * S;
  if ((e = run_sweep<S, kPhi>(a, gphi, st))) return e;
  hipLaunchKernelGGL(k_dense_theta_gemm<S>, dim3(gg), dim3(G::BLOCK), 0, st, ga);
  if ((e = (int)hipGetLastError())) return e;
  const long long n = (long long)S * S + S;
  hipLaunchKernelGGL(k_dense_finalize, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, ga.part,
                     gg, mat, 1.f / T, grad_theta, gcp, gpsi + gphi, grad_c, S);
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

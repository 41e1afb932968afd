// Forward-backward kernels for the bitshift trellis on gfx950.
//
// Method: the BCJR forward-backward sum-product recursion at temperature T of "BCJR-QAT: A
// Differentiable Relaxation of Trellis-Coded Weight Quantization" (abstract; gist.science
// technical summary, "Core mechanism" and "Key technical innovations"): Boltzmann posteriors
// over trellis paths, the soft codeword w_hat_t = sum_s c(s) p_T(s_t = s | w), log Z, and the
// exact gradient of sum_t g_t w_hat_t + h log Z with respect to w and the codebook.
//
// Arithmetic is in base-2 log units: the emission log2-potential is
// ell_t(s) = -(log2(e)/T) (w_t - c(s))^2.
//
// Factorisation used here (exact, a property of the bitshift trellis): the K successors
// s' = K*j + b of butterfly j share the predecessors j + a*M, so the forward message is one
// number per butterfly,
//     alpha_t(s) = ell_t(s) + lam_t(s >> k),   lam_{t+1}(j) = LSE_a alpha_t(j + a*M),
// and likewise beta_t(s) = rho_t(s mod M), rho_{t-1}(j) = LSE_b [ell_t(K*j+b) + rho_t((K*j+b) mod M)].
// Each LSE is evaluated once per butterfly instead of once per state: one exp2 per
// state-step and one log2 per butterfly-step per direction. See geom.h for the K x K block
// layout that makes both recursions lane-local.
//
// Normalisation: after every step the messages are shifted by the integer floor of their
// chain-wide maximum. The integer shifts are summed exactly, and log2 Z is kept next to them
// in double precision, so the per-step posterior normaliser
// log2 Z - (forward shifts up to t) - (backward shifts down to t) carries no rounding drift.
//
// Precision policies. The messages lam and rho are sums along the trellis of emission terms
// whose size grows like 1/T. In fp32 their accumulated rounding (about an ulp of a value of
// size log2(e)/T per step) limits the gradient, whose sensitivity to posterior errors is
// large when T is small, so below T = 0.05 (kPreciseBelowT) the messages are carried in fp64 and the emission
// is formed from the unscaled difference w - c; exponentials, the posterior weights and the
// conditional expectations stay fp32 in both policies. The 2^16-state trellis keeps fp32
// messages at every T (its fp64 backward messages would not fit in LDS) and below T = 0.05 forms
// only the emission in fp64 (the Mixed policy).
//
// One persistent block per workspace slot loops over chain units. Phase A runs the forward
// recursion and stores each lane's column offsets lam_t(x + a*NG) (the alpha-side inputs of
// its K x K blocks) in the slot's history; phase B runs the backward recursion, reads the
// history back in reverse and forms posteriors, the soft codeword and the gradients.
#include <hip/hip_runtime.h>

#include <math.h>

#include "geom.h"
#include "internal.h"
#include "sparse_device.h"

// Multiply-adds are fused only within one expression (or explicitly with __builtin_fmaf), never
// across statements: the forward step is inlined twice (the sweep and, with checkpoints, the
// segment replay), and both copies must round identically.
#pragma clang fp contract(on)

namespace bcjr {
namespace {

// ---------------------------------------------------------------------------------------------
// Forward: soft codeword and log Z.
//
// Boundary modes (BM) for the segmented forward of long chains (parallel in L). The forward
// and backward butterfly messages obey lam_{t+1} = lam_t (x) A_t and rho_t = A_{t+1} (x) rho_{t+1}
// in the (log-sum-exp, +) semiring with ONE M x M matrix per step, A_t(i, j) = emission of the
// state s with s >> k = i and s mod M = j. A segment [t0, t1) therefore has one transfer matrix
// Q = A_{t0} ... A_{t1-1} serving both directions: lam_{t1} = lam_{t0} (x) Q and
// rho_{t0-1} = Q (x) rho_{t1-1}.
//   BM = 0: a whole chain, free start and end (the ordinary forward).
//   BM = 2: transfer rows. Virtual chain v*M + i runs segment v from lam_{t0} = one-hot(i)
//           (-kFar elsewhere) and writes its final LSE lam_{t1}(j) for all j as row i of the
//           segment's Q: fp32 offsets from the row's integer-floor maximum, plus that row
//           scale (N + the floor, log2, double). Phase A only; no history.
//   BM = 1: a segment with boundary messages: lam_{t0} = lam0 + N0, rho_{t1-1} = rho1 + Np0
//           (normalised vectors and their scales from the scan over segments), so that
//           log2 Z = N + Np0 + LSE_j (lam_{t1}(j) - N + rho1(j)) and the posteriors are the
//           whole chain's. Writes w_hat for the segment's steps and log Z from segment 0.
// Virtual chain v (BM 1) or v = chain / M (BM 2) is segment jbase + v % nseg of original chain
// v / nseg; its weights start at (v / nseg) * lfull + (jbase + v % nseg) * seglen.
// ---------------------------------------------------------------------------------------------
struct SegArgs {
  long long nseg, jbase, seglen, lfull, ptot;
  const double* lam0;  // [chains][ptot][M] normalised forward boundary messages
  const double* rho1;  // [chains][ptot][M] normalised backward boundary messages
  const double* sc0;   // [chains][ptot][2] their scales N0, Np0
  float* rows;         // BM 2 output: [chains][ptot][M][M] offsets from each row's scale
  double* rscale;      // BM 2 output: [chains][ptot][M] row scales
  // backward only: the conditional expectations Phi at segment starts and Psi at segment ends
  // ([chains][ptot][M], fp32), and (BM 2) the segment moment rows F [chains][ptot][M][M]
  const float* phi0;
  const float* psi1;
  float* frows;
};
constexpr float kFar = 1e30f;  // stands in for -infinity without producing inf - inf

template <class C, bool CK, int BM = 0>
__global__ void __launch_bounds__(C::BLOCK)
k_sparse_fwd(const float* __restrict__ cb, const float* __restrict__ w, long long B, long long L,
             Consts k, float* __restrict__ w_hat, float* __restrict__ log_z,
             double* __restrict__ saved_lz, float* __restrict__ saved_what, void* __restrict__ ws,
             size_t slot_bytes, long long units, long long seg_arg, SegArgs sa) {
  static_assert(BM == 0 || !CK, "segmented modes use the full history");
  using P = typename C::P;
  using MT = typename C::MT;
  constexpr int K = C::K, G = C::G, LPS = C::LPS, NG = C::NG, M = C::M, KG = C::KG;
  constexpr int SPB = C::SPB, BLOCK = C::BLOCK;
  __shared__ __attribute__((aligned(16))) MT msg[C::NBUF][SPB * M];
  __shared__ double red[2 * C::NWAVES * 4];

  const int tid = threadIdx.x;
  const int q = LPS < 64 ? tid / LPS : 0;    // chain within the block
  const int p = LPS < 64 ? tid % LPS : tid;  // lane within the chain

  CodebookLane<C> vsrc;
  vsrc.init(cb, k.sc, p);

  // slot layout: lam history [H] entries of BLOCK * KG values (room for 8 bytes each; 16-byte
  // chunks interleaved across the lanes, store_hist), shift prefix N [L][SPB] (double).
  // Full history (CK false): H = L, entry t is step t. Checkpointed (CK, seg = C): entries
  // 0 .. ncp-1 are the checkpoints of steps 0, C, 2C, ..., entries ncp .. ncp+C-1 the segment
  // being replayed.
  const long long seg = CK ? seg_arg : 0;
  const long long ncp = seg ? (L + seg - 1) / seg : L;
  const long long nh = seg ? ncp + seg : L;
  char* sb = static_cast<char*>(ws) + (size_t)blockIdx.x * slot_bytes;
  MT* __restrict__ hs = reinterpret_cast<MT*>(sb);
  double* __restrict__ ns = reinterpret_cast<double*>(sb + (size_t)nh * BLOCK * KG * 8);
  auto hist = [&](long long e) { return hs + (size_t)e * BLOCK * KG + (size_t)tid * (16 / sizeof(MT)); };
  int mb = 0, rp = 0;

  for (long long unit = blockIdx.x; unit < units; unit += gridDim.x) {
    const long long b = unit * SPB + q;
    const bool valid = b < B;
    const long long bb = valid ? b : B - 1;
    // segment of an original chain (BM 1, 2): its weights, and its boundary-vector index
    const long long vch = BM == 2 ? bb / M : bb;
    const long long sg = BM ? vch / sa.nseg * sa.ptot + sa.jbase + vch % sa.nseg : 0;
    const long long wofs = BM ? vch / sa.nseg * sa.lfull + (sa.jbase + vch % sa.nseg) * sa.seglen
                              : bb * L;
    const float* __restrict__ wb = w + wofs;

    MT lc[G][K];
    double N = 0.0, lz2 = 0.0;
    if constexpr (BM == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int a = 0; a < K; ++a) lc[g][a] = (MT)0;
    } else if constexpr (BM == 1) {
      const double* l0 = sa.lam0 + sg * M;
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int a = 0; a < K; ++a) lc[g][a] = (MT)l0[p + g * LPS + a * NG];
      N = sa.sc0[sg * 2];
    } else {
      const long long i0 = bb % M;
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int a = 0; a < K; ++a) lc[g][a] = (p + g * LPS + a * NG == i0) ? (MT)0 : (MT)-kFar;
    }

    // The step's weight is loaded a step ahead, before the previous step's history stores:
    // loads and stores share one in-order completion counter, so a load issued after them
    // would also wait for the stores. wnx holds w_t when advance(t) starts.
    float wnx = wb[0];
    // One forward step: the column offsets lc of step t -> those of step t + 1 (t < L - 1).
    auto advance = [&](long long t) {
      const float u = k.sc * wnx;
      wnx = wb[t != L - 1 ? t + 1 : t];  // (t < L: a scalar 64-bit compare)
      MT out[G][K];
      MT mx = (MT)-INFINITY;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float Vg[K][K];
        vsrc.get(g, Vg);
#pragma unroll
        for (int r = 0; r < K; ++r) {
          MT x[K];
          MT m = (MT)-INFINITY;
#pragma unroll
          for (int a = 0; a < K; ++a) {
            x[a] = emit<P>(u, Vg[r][a], lc[g][a], k.kap);
            m = tmax(m, x[a]);
          }
          float s = ex2((float)(x[0] - m));
#pragma unroll
          for (int a = 1; a < K; ++a) s += ex2((float)(x[a] - m));
          out[g][r] = m + (MT)lg2(s);
          mx = tmax(mx, out[g][r]);
        }
      }
      MT* mw = msg[mb] + q * M;
#pragma unroll
      for (int g = 0; g < G; ++g) store_vec<K>(mw + K * (p + g * LPS), out[g]);
      MT v1[1] = {mx};
      chain_reduce<C, 1, 1u>(v1, red, rp);
      const MT sh = floor(v1[0]);
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int a = 0; a < K; ++a) lc[g][a] = mw[p + g * LPS + a * NG] - sh;
      N += (double)sh;
      if constexpr (C::DB) mb ^= 1; else __syncthreads();
    };

    // ---- phase A: forward messages lam, t = 0 .. L-1 -------------------------------------
    for (long long t = 0; t < L; ++t) {
      if constexpr (BM != 2) {
        if (seg == 0 || t % seg == 0) store_hist<KG, BLOCK>(hist(seg ? t / seg : t), &lc[0][0]);
        if (p == 0) ns[t * SPB + q] = N;
      }
      if (t == L - 1) {
        const float u = k.sc * wnx;
        MT out[G][K];
        MT mx = (MT)-INFINITY;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float Vg[K][K];
          vsrc.get(g, Vg);
#pragma unroll
          for (int r = 0; r < K; ++r) {
            MT x[K];
            MT m = (MT)-INFINITY;
#pragma unroll
            for (int a = 0; a < K; ++a) {
              x[a] = emit<P>(u, Vg[r][a], lc[g][a], k.kap);
              m = tmax(m, x[a]);
            }
            float s = ex2((float)(x[0] - m));
#pragma unroll
            for (int a = 1; a < K; ++a) s += ex2((float)(x[a] - m));
            out[g][r] = m + (MT)lg2(s);
            mx = tmax(mx, out[g][r]);
          }
        }
        if constexpr (BM == 2) {  // row i0 of the segment's transfer matrix
          MT v1[1] = {mx};
          chain_reduce<C, 1, 1u>(v1, red, rp);
          const MT sh = floor(v1[0]);
          if (valid) {
            const long long ri = sg * M + bb % M;
            float* row = sa.rows + ri * M;
#pragma unroll
            for (int g = 0; g < G; ++g) {
              float o4[K];
#pragma unroll
              for (int r = 0; r < K; ++r) o4[r] = (float)(out[g][r] - sh);
              store_vec<K>(row + K * (p + g * LPS), o4);
            }
            if (p == 0) sa.rscale[ri] = N + (double)sh;
          }
          break;
        }
        if constexpr (BM == 1) {  // the end boundary: weight by rho_{t1-1}
          const double* r1 = sa.rho1 + sg * M;
          mx = (MT)-INFINITY;
#pragma unroll
          for (int g = 0; g < G; ++g)
#pragma unroll
            for (int r = 0; r < K; ++r) {
              out[g][r] += (MT)r1[K * (p + g * LPS) + r];
              mx = tmax(mx, out[g][r]);
            }
        }
        MT v1[1] = {mx};
        chain_reduce<C, 1, 1u>(v1, red, rp);
        float s2 = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int r = 0; r < K; ++r) s2 += ex2((float)(out[g][r] - v1[0]));  // once per chain
        float v2[1] = {s2};
        chain_reduce<C, 1, 0u>(v2, red, rp);
        lz2 = N + ((double)v1[0] + (double)lg2(v2[0]));
        if constexpr (BM == 1) lz2 += sa.sc0[sg * 2 + 1];
        break;
      }
      advance(t);
    }
    if constexpr (BM == 2) {
      continue;  // transfer rows need no backward sweep
    }
    __syncthreads();  // phase-A history writes (incl. other lanes' N) visible to phase B

    // ---- phase B: backward messages rho, posterior and soft codeword, t = L-1 .. 0 -------
    // Segment by segment (the whole chain is one segment with the full history); with
    // checkpoints, each segment's forward offsets are replayed from its checkpoint first.
    MT rr[G][K];
    double Np = 0.0;
    if constexpr (BM == 1) {
      const double* r1 = sa.rho1 + sg * M;
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int r = 0; r < K; ++r) rr[g][r] = (MT)r1[K * (p + g * LPS) + r];
      Np = sa.sc0[sg * 2 + 1];
    } else {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int r = 0; r < K; ++r) rr[g][r] = (MT)0;
    }
    // Per-step outputs of a chain are kept by lane t mod LPS and written together when that
    // lane's value for step t is in (t mod LPS == 0): the phase-B loop then issues no vector
    // store on most steps, so its waits for each block's history loads count only those loads
    // (a store in every step, issued by one lane under a branch, made the compiler's wait counts
    // cover the next blocks' loads too).
    float whs = 0.f;
    const long long nseg = seg ? ncp : 1;
    for (long long sgi = nseg - 1; sgi >= 0; --sgi) {
      const long long t0 = seg ? sgi * seg : 0;
      const long long t1 = seg ? (t0 + seg < L ? t0 + seg : L) : L;
      if (CK) {
        load_hist<KG, BLOCK>(hist(sgi), &lc[0][0]);
        wnx = wb[t0];
        for (long long t = t0; t < t1; ++t) {
          store_hist<KG, BLOCK>(hist(ncp + (t - t0)), &lc[0][0]);
          if (t + 1 < t1) advance(t);
        }
      }
      auto entry = [&](long long t) { return seg ? ncp + (t - t0) : t; };
      // lam offsets of the step being processed: each block's are replaced by the previous
      // step's right after their last use, so the loads have a step to land and need no
      // registers of their own (loaded a step ahead, they would be copied every step)
      MT lcur[G][K];
      load_hist<KG, BLOCK>(hist(entry(t1 - 1)), &lcur[0][0]);
      double Nn = ns[(t1 - 1) * SPB + q];
      wait_vm0();
      for (long long t = t1 - 1; t >= t0; --t) {
        // unconditional (at the segment's first step the loads re-read step t): a conditional
        // load makes the compiler copy the carried rows out and back every step
        const long long tp = t > t0 ? t - 1 : t;
        const float u = k.sc * wb[t];
        const MT LZ = (MT)((lz2 - Nn) - Np);
        Nn = ns[tp * SPB + q];
        // (issued before the step's history loads, so that the next step's wait for it does not
        // also wait for them)
        __builtin_amdgcn_sched_barrier(0);
        gptr<MT> hn = global(hist(entry(tp)));
        float num = 0.f, den = 0.f;
        MT mx = (MT)-INFINITY;
        MT rout[G][K];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float Vg[K][K];
          vsrc.get(g, Vg);
          float fa[K];
#pragma unroll
          for (int a = 0; a < K; ++a) {
            MT y[K];
            MT m = (MT)-INFINITY;
#pragma unroll
            for (int r = 0; r < K; ++r) {
              y[r] = emit<P>(u, Vg[r][a], rr[g][r], k.kap);
              m = tmax(m, y[r]);
            }
            float e0 = ex2((float)(y[0] - m));
            float cs = e0, cw = Vg[0][a] * e0;
#pragma unroll
            for (int r = 1; r < K; ++r) {
              const float e = ex2((float)(y[r] - m));
              cs += e;
              cw = __builtin_fmaf(Vg[r][a], e, cw);
            }
            rout[g][a] = m + (MT)lg2(cs);
            mx = tmax(mx, rout[g][a]);
            const float f = ex2((float)((m + lcur[g][a]) - LZ));
            fa[a] = f;
            num = __builtin_fmaf(f, cw, num);
            den = __builtin_fmaf(f, cs, den);
          }
          hn = after(hn, fa);
          load_hist_part<K, BLOCK>(hn, g * K, lcur[g]);
        }
        MT* mw = msg[mb] + q * M;
        if (t > 0) {
#pragma unroll
          for (int g = 0; g < G; ++g)
#pragma unroll
            for (int a = 0; a < K; ++a) mw[p + g * LPS + a * NG] = rout[g][a];
        }
        MT v3[3] = {(MT)num, (MT)den, mx};
        chain_reduce<C, 3, 4u>(v3, red, rp);
        {  // kept by lane t mod LPS, written once per LPS steps (step_out)
          const float wh = ((float)v3[0] / (float)v3[1]) * k.csc;
          if (p == (int)(t % LPS)) whs = wh;
          if (t % LPS == 0) {
            // (the lane offset is formed here: folded into the addresses by the loop's strength
            // reduction, it would keep two 64-bit address registers per lane live all along)
            const unsigned lane = opaque((unsigned)p);
            if (valid && t + lane < L) {
              w_hat[wofs + t + lane] = whs;
              if constexpr (BM == 0) saved_what[b * L + t + lane] = whs;
            }
          }
        }
        if (t == 0) break;
        const MT sh = floor(v3[2]);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          MT tmp[K];
          load_vec<K>(mw + K * (p + g * LPS), tmp);
#pragma unroll
          for (int r = 0; r < K; ++r) rr[g][r] = tmp[r] - sh;
        }
        Np += (double)sh;
        if constexpr (C::DB) mb ^= 1; else __syncthreads();
      }
    }
    if constexpr (BM == 0) {
      if (valid && p == 0) {
        log_z[b] = (float)(lz2 * (double)kLn2);
        saved_lz[b] = lz2;
      }
    } else {
      if (valid && p == 0 && sa.jbase + vch % sa.nseg == 0)
        log_z[vch / sa.nseg] = (float)(lz2 * (double)kLn2);
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Forward for chains of 1024 lanes (one 16-wave block per chain, so at most 128 registers per
// lane). There the lane's blocks do not fit in registers together with their messages, codebook
// values and intermediates, so the G blocks are visited in a rolled loop: a block's column
// offsets are read from LDS when it is processed, its outputs go straight to the other message
// buffer (one buffer per step parity), and the codebook values and history entries of the next
// block are loaded while the current one is computed, into the other of two register sets
// (over_blocks). The per-block arithmetic and the history layout are those of k_sparse_fwd
// (mode 0).
// ---------------------------------------------------------------------------------------------
template <class C, bool CK>
__global__ void __launch_bounds__(C::BLOCK)
k_sparse_fwd_wide(const float* __restrict__ cb, const float* __restrict__ w, long long B,
                  long long L, Consts k, float* __restrict__ w_hat, float* __restrict__ log_z,
                  double* __restrict__ saved_lz, float* __restrict__ saved_what,
                  void* __restrict__ ws, size_t slot_bytes, long long units, long long seg_arg) {
  using P = typename C::P;
  using MT = typename C::MT;
  constexpr int K = C::K, G = C::G, LPS = C::LPS, NG = C::NG, M = C::M, KG = C::KG;
  static_assert(C::SPB == 1 && C::BLOCK == LPS && C::DB, "one chain per block, two buffers");
  __shared__ __attribute__((aligned(16))) MT msg[2][M];
  __shared__ double red[2 * C::NWAVES * 4];
  const int p = threadIdx.x;
  // codebook value of state K*(p + g*LPS) + r + a*M: block-uniform base + 32-bit lane offset
  const unsigned lo4 = K * p;
  // Raw codebook values c[a][r] of block g, loaded a block ahead (over_blocks): loads and
  // stores share one in-order completion counter, so a load must be issued before the stores
  // it should not wait for, and not be consumed right after it is issued.
  auto cblock = [&](int g, float (&c)[K][K]) {
#pragma unroll
    for (int a = 0; a < K; ++a) {
      const float* __restrict__ ub = cb + (g * K * LPS + a * M);
      load_vec<K>(at_lane(ub, lo4), c[a]);
    }
  };
  struct FIn {  // inputs of a forward block loaded ahead
    float c[K][K];
  };
  struct BIn {  // inputs of a backward block loaded ahead: codebook values and history entry
    float c[K][K];
    MT l[K];
  };

  const long long seg = CK ? seg_arg : 0;
  const long long ncp = seg ? (L + seg - 1) / seg : L;
  const long long nh = seg ? ncp + seg : L;
  char* sb = static_cast<char*>(ws) + (size_t)blockIdx.x * slot_bytes;
  MT* __restrict__ hs = reinterpret_cast<MT*>(sb);
  double* __restrict__ ns = reinterpret_cast<double*>(sb + (size_t)nh * LPS * KG * 8);
  // history entries are block-major, [H][G][LPS][K]: hist(e, g) is block g of this lane in
  // entry e
  auto hist = [&](long long e, int g) {
    return at_lane(hs + (size_t)e * LPS * KG + (size_t)g * (LPS * K), lo4);
  };
  int rp = 0;

  // units == B (one chain per unit), so every unit is a chain
  for (long long b = blockIdx.x; b < units; b += gridDim.x) {
    const float* __restrict__ wb = w + b * L;
    __syncthreads();  // the previous chain is done with both buffers
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int a = 0; a < K; ++a) msg[0][p + g * LPS + a * NG] = (MT)0;
    __syncthreads();

    int cur = 0;    // buffer holding the current step's column values
    MT sh = (MT)0;  // shift still to be subtracted from them
    // the column offsets of step t (msg[cur] - sh) as history entry e
    auto record = [&](long long e) {
#pragma unroll 1
      for (int g = 0; g < G; ++g) {
        MT lc[K];
#pragma unroll
        for (int a = 0; a < K; ++a) lc[a] = msg[cur][p + g * LPS + a * NG] - sh;
        store_vec<K>(hist(e, g), lc);
      }
    };
    // Loaded ahead of their use: the next block's raw codebook values (block 0 when a run of
    // steps starts, and after a step's last block; fa, with fb the second register set) and
    // the next step's weight (wn = w_t when fstep(t) starts).
    FIn fa, fb;
    float wn = 0.f;
    // One forward step: offsets of step t -> raw outputs of step t + 1 in msg[cur ^ 1]; records
    // the offsets as history entry e (e >= 0) and returns the outputs' chain-wide maximum.
    auto fstep = [&](long long t, long long e) -> MT {
      const float u = k.sc * wn;
      wn = vload(wb, t != L - 1 ? t + 1 : t);
      const MT* __restrict__ src = msg[cur];
      MT* __restrict__ dst = msg[cur ^ 1];
      MT mx = (MT)-INFINITY;
      over_blocks<G>(
          fa, fb, [&](int gn, FIn& in) { cblock(gn < G ? gn : 0, in.c); },
          [&](int g, const FIn& in) {
            MT lc[K];
#pragma unroll
            for (int a = 0; a < K; ++a) lc[a] = src[p + g * LPS + a * NG] - sh;
            if (e >= 0) store_vec<K>(hist(e, g), lc);
            MT out[K];
#pragma unroll
            for (int r = 0; r < K; ++r) {
              MT x[K];
              MT m = (MT)-INFINITY;
#pragma unroll
              for (int a = 0; a < K; ++a) {
                x[a] = emit_c<P>(u, k.sc, in.c[a][r], lc[a], k.kap);
                m = tmax(m, x[a]);
              }
              float s = ex2((float)(x[0] - m));
#pragma unroll
              for (int a = 1; a < K; ++a) s += ex2((float)(x[a] - m));
              out[r] = m + (MT)lg2(s);
              mx = tmax(mx, out[r]);
            }
            store_vec<K>(dst + K * (p + g * LPS), out);
          });
      MT v1[1] = {mx};
      chain_reduce<C, 1, 1u>(v1, red, rp);
      return v1[0];
    };

    // ---- phase A: forward messages, t = 0 .. L-1 ---------------------------------------------
    double N = 0.0, lz2 = 0.0;
    cblock(0, fa.c);
    wn = vload(wb, 0);
    for (long long t = 0;; ++t) {
      if (p == 0) ns[t] = N;
      const long long e = seg == 0 ? t : (t % seg == 0 ? t / seg : -1);
      const MT mx = fstep(t, e);
      if (t == L - 1) {  // log2 Z = N + LSE of the last outputs (this lane's own rows)
        float s2 = 0.f;
#pragma unroll 1
        for (int g = 0; g < G; ++g) {
          MT o[K];
          load_vec<K>(msg[cur ^ 1] + K * (p + g * LPS), o);
#pragma unroll
          for (int r = 0; r < K; ++r) s2 += ex2((float)(o[r] - mx));
        }
        float v2[1] = {s2};
        chain_reduce<C, 1, 0u>(v2, red, rp);
        lz2 = N + ((double)mx + (double)lg2(v2[0]));
        break;
      }
      sh = floor(mx);
      N += (double)sh;
      cur ^= 1;
    }

    // ---- phase B: backward messages, posterior and soft codeword, t = L-1 .. 0 ---------------
    // A lane reads only its own rows K*(p + g*LPS) + r of the current buffer (rho at step t,
    // raw, minus shp) and writes its columns of the other.
    __syncthreads();  // phase-A history (incl. lane 0's N) visible; buffers free
    int rb = 0;
    MT shp = (MT)0;
    double Np = 0.0;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      MT z[K];
#pragma unroll
      for (int r = 0; r < K; ++r) z[r] = (MT)0;
      store_vec<K>(msg[0] + K * (p + g * LPS), z);
    }
    const long long nseg = seg ? ncp : 1;
    for (long long sgi = nseg - 1; sgi >= 0; --sgi) {
      const long long t0 = seg ? sgi * seg : 0;
      const long long t1 = seg ? (t0 + seg < L ? t0 + seg : L) : L;
      if (CK) {
        // replay the segment's forward offsets from its checkpoint through both buffers,
        // keeping this lane's rows of the backward buffer in registers meanwhile
        MT keep[G][K];
#pragma unroll
        for (int g = 0; g < G; ++g) load_vec<K>(msg[rb] + K * (p + g * LPS), keep[g]);
        __syncthreads();
        MT c0[KG];
#pragma unroll
        for (int g = 0; g < G; ++g) load_vec<K>(hist(sgi, g), c0 + g * K);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int a = 0; a < K; ++a) msg[0][p + g * LPS + a * NG] = c0[g * K + a];
        __syncthreads();
        cur = 0;
        sh = (MT)0;
        cblock(0, fa.c);
        wn = vload(wb, t0);
        for (long long t = t0; t + 1 < t1; ++t) {
          const MT mx = fstep(t, ncp + (t - t0));
          sh = floor(mx);
          cur ^= 1;
        }
        record(ncp + (t1 - 1 - t0));
        __syncthreads();
#pragma unroll
        for (int g = 0; g < G; ++g) store_vec<K>(msg[rb] + K * (p + g * LPS), keep[g]);
      }
      auto entry = [&](long long t) { return seg ? ncp + (t - t0) : t; };
      BIn ba, bb;  // block-ahead loads, two register sets in turn
      cblock(0, ba.c);
      load_vec<K>(hist(entry(t1 - 1), 0), ba.l);
      // the step's scalars, loaded a step ahead (a load consumed at once would also wait for
      // the stores issued before it)
      double nsn = ns[t1 - 1];
      float wn = vload(wb, t1 - 1);
      for (long long t = t1 - 1; t >= t0; --t) {
        const double Nt = nsn;
        const float u = k.sc * wn;
        {
          const long long tp = t > t0 ? t - 1 : t;
          nsn = ns[tp];
          wn = vload(wb, tp);
        }
        const MT LZ = (MT)((lz2 - Nt) - Np);
        const MT* __restrict__ src = msg[rb];
        MT* __restrict__ dst = msg[rb ^ 1];
        float num = 0.f, den = 0.f;
        MT mx = (MT)-INFINITY;
        over_blocks<G>(
            ba, bb,
            [&](int gn, BIn& in) {
              // block 0 of step t - 1 after the last block (after the segment's last step this
              // re-reads an entry of the segment)
              cblock(gn < G ? gn : 0, in.c);
              const long long en = gn < G ? entry(t) : entry(t > t0 ? t - 1 : t);
              load_vec<K>(hist(en, gn < G ? gn : 0), in.l);
            },
            [&](int g, const BIn& in) {
              MT rr[K];
              load_vec<K>(src + K * (p + g * LPS), rr);
#pragma unroll
              for (int r = 0; r < K; ++r) rr[r] -= shp;
#pragma unroll
              for (int a = 0; a < K; ++a) {
                MT y[K];
                MT m = (MT)-INFINITY;
#pragma unroll
                for (int r = 0; r < K; ++r) {
                  y[r] = emit_c<P>(u, k.sc, in.c[a][r], rr[r], k.kap);
                  m = tmax(m, y[r]);
                }
                // cw: the column's weighted sum of raw codebook values
                float e0 = ex2((float)(y[0] - m));
                float cs = e0, cw = in.c[a][0] * e0;
#pragma unroll
                for (int r = 1; r < K; ++r) {
                  const float e = ex2((float)(y[r] - m));
                  cs += e;
                  cw = __builtin_fmaf(in.c[a][r], e, cw);
                }
                const MT ro = m + (MT)lg2(cs);
                mx = tmax(mx, ro);
                const float f = ex2((float)((m + in.l[a]) - LZ));
                num = __builtin_fmaf(f, cw, num);
                den = __builtin_fmaf(f, cs, den);
                // (at t = 0 the write is dead: the next chain starts behind a barrier)
                dst[p + g * LPS + a * NG] = ro;
              }
            });
        MT v3[3] = {(MT)num, (MT)den, mx};
        chain_reduce<C, 3, 4u>(v3, red, rp);
        if (p == 0) {
          const float wh = (float)v3[0] / (float)v3[1];
          w_hat[b * L + t] = wh;
          saved_what[b * L + t] = wh;
        }
        if (t == 0) break;
        shp = floor(v3[2]);
        Np += (double)shp;
        rb ^= 1;
      }
    }
    if (p == 0) {
      log_z[b] = (float)(lz2 * (double)kLn2);
      saved_lz[b] = lz2;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Backward: gradient of F = sum_t g_t w_hat_t + h log Z w.r.t. w and the codebook.
// With the posterior written as a Markov chain, E[F | s_t = s] = Fwd_t(s) + g_t c(s) + Bwd_t(s)
// where the conditional expectations obey the same butterfly factorisation as the messages:
//   Fwd_t(s) = Phi_t(s >> k),  Phi_{t+1}(j)  = sum_a q(a|j) (Phi_t((j+aM)>>k) + g_t c(j+aM)),
//   Bwd_t(s) = Psi_t(s mod M), Psi_{t-1}(j') = sum_b r(b|j') (Psi_t((Kj'+b) mod M) + g_t c(Kj'+b)),
// q and r being the softmax weights of the forward / backward LSEs (no extra exponentials).
// D_t(s) = gamma_t(s) (E[F | s_t = s] - E[F]). The recursions carry the centred codeword
// c(s) - w_hat_t (w_hat from the forward): Phi and Psi then hold conditional expectations of
// sum_u g_u (c(s_u) - w_hat_u), which are small wherever the posterior is sharp, E[F] drops
// out (its centred value is 0), and D_t(s) = gamma_t(s) (Phi + g_t (c(s) - w_hat_t) + Psi).
// With E_t = D_t + h gamma_t:
//   dF/dw_t  = (2/T) (sum_s c(s) E_t(s) - h w_t)
//   dF/dc(s) = sum_t [ g_t gamma_t(s) + (2/T)(w_t - c(s)) E_t(s) ].
// ---------------------------------------------------------------------------------------------
//
// Boundary modes as in k_sparse_fwd. The conditional expectations compose over a segment
// [t0, t1) through its moment matrix F(i, j) = E[sum_{t0 <= u < t1} g_u (c(s_u) - w_hat_u) |
// butterfly i at t0, butterfly j at t1]: the forward one at t1 is a softmax-weighted average
// over i of Phi_{t0}(i) + F(i, j), the backward one at t0 - 1 one over j of F(i, j) + Psi(j).
//   BM = 2: virtual chain v*M + i runs segment v's lam and Phi recursions from lam = one-hot(i),
//           Phi = 0, and writes row i of Q (as k_sparse_fwd) and of F. Phase A only.
//   BM = 1: a segment from its boundary values lam0 + N0, Phi0 at t0 and rho1 + Np0, Psi1 at
//           t1 - 1; log2 Z is the segment's own (as in k_sparse_fwd's mode 1), grad_w is written
//           at the segment's steps and the codebook-gradient partials cover all its segments.
template <class C, bool CK, int BM = 0>
__global__ void __launch_bounds__(C::BLOCK)
k_sparse_bwd(const float* __restrict__ cb, const float* __restrict__ w, long long B, long long L,
             Consts k, const double* __restrict__ saved_lz, const float* __restrict__ saved_what,
             const float* __restrict__ gup, const float* __restrict__ hup,
             float* __restrict__ grad_w, float* __restrict__ partial, void* __restrict__ ws,
             size_t slot_bytes, long long units, long long seg_arg, SegArgs sa) {
  static_assert(BM == 0 || !CK, "segmented modes use the full history");
  using P = typename C::P;
  using MT = typename C::MT;
  constexpr int K = C::K, G = C::G, LPS = C::LPS, NG = C::NG, M = C::M, KG = C::KG;
  constexpr int SPB = C::SPB, BLOCK = C::BLOCK;
  const long long seg = CK ? seg_arg : 0;
  __shared__ __attribute__((aligned(16))) MT msgl[C::NBUF][SPB * M];
  __shared__ __attribute__((aligned(16))) float msgp[C::NBUF][SPB * M];
  __shared__ double red[2 * C::NWAVES * 4];

  const int tid = threadIdx.x;
  const int q = LPS < 64 ? tid / LPS : 0;
  const int p = LPS < 64 ? tid % LPS : tid;
  const float k2 = 2.0f * k.inv_t * k.csc;  // (2/T)(w - c) = k2 * (u - v)
  // The codebook-gradient sums are carried divided by k2 (one multiply fewer per state and
  // step): acc = sum_t [(g_t / k2) gamma + (u - v) E], times k2 when the partials are written.
  const float ik2 = 1.0f / k2;

  CodebookLane<C> vsrc;
  vsrc.init(cb, k.sc, p);
  float acc[G][K][K];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int r = 0; r < K; ++r)
#pragma unroll
      for (int a = 0; a < K; ++a) acc[g][r][a] = 0.f;

  // slot layout: lam history [H] entries of BLOCK * KG values (room for 8 bytes each), Phi
  // history [H] entries of BLOCK * KG (fp32), both in lane-interleaved 16-byte chunks
  // (store_hist), shift prefix N [L][SPB] (double); H and the entry order as in k_sparse_fwd.
  const long long ncp = seg ? (L + seg - 1) / seg : L;
  const long long nh = seg ? ncp + seg : L;
  char* sb = static_cast<char*>(ws) + (size_t)blockIdx.x * slot_bytes;
  MT* __restrict__ hl = reinterpret_cast<MT*>(sb);
  float* __restrict__ hp = reinterpret_cast<float*>(sb + (size_t)nh * BLOCK * KG * 8);
  double* __restrict__ ns = reinterpret_cast<double*>(sb + (size_t)nh * BLOCK * KG * 12);
  auto histl = [&](long long e) { return hl + (size_t)e * BLOCK * KG + (size_t)tid * (16 / sizeof(MT)); };
  auto histp = [&](long long e) { return hp + (size_t)e * BLOCK * KG + (size_t)tid * 4; };
  int mb = 0, rp = 0;

  for (long long unit = blockIdx.x; unit < units; unit += gridDim.x) {
    const long long b = unit * SPB + q;
    const bool valid = b < B;
    const long long bb = valid ? b : B - 1;
    // segment of an original chain (BM 1, 2), as in k_sparse_fwd
    const long long vch = BM == 2 ? bb / M : bb;
    const long long chain = BM ? vch / sa.nseg : bb;
    const long long sg = BM ? chain * sa.ptot + sa.jbase + vch % sa.nseg : 0;
    const long long wofs = BM ? chain * sa.lfull + (sa.jbase + vch % sa.nseg) * sa.seglen : bb * L;
    const float* __restrict__ wb = w + wofs;
    const float* __restrict__ gb = gup + wofs;
    const float* __restrict__ whb = saved_what + wofs;
    const float h = (BM != 2 && hup != nullptr && valid) ? hup[chain] : 0.f;
    double lz2 = BM ? 0.0 : saved_lz[bb];

    MT lc[G][K];
    float pc[G][K];
    double N = 0.0;
    if constexpr (BM == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int a = 0; a < K; ++a) { lc[g][a] = (MT)0; pc[g][a] = 0.f; }
    } else if constexpr (BM == 1) {
      const double* l0 = sa.lam0 + sg * M;
      const float* f0 = sa.phi0 + sg * M;
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int a = 0; a < K; ++a) {
          lc[g][a] = (MT)l0[p + g * LPS + a * NG];
          pc[g][a] = f0[p + g * LPS + a * NG];
        }
      N = sa.sc0[sg * 2];
    } else {
      const long long i0 = bb % M;
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int a = 0; a < K; ++a) {
          lc[g][a] = (p + g * LPS + a * NG == i0) ? (MT)0 : (MT)-kFar;
          pc[g][a] = 0.f;
        }
    }

    // The step's inputs are loaded a step ahead, before the previous step's history stores
    // (loads and stores share one in-order completion counter): wn, gn, hn hold w_t, g_t and
    // w_hat_t when advance(t) starts.
    float wn = wb[0], gn = gb[0], hn = whb[0];
    auto inputs_at = [&](long long t) {
      wn = wb[t];
      gn = gb[t];
      hn = whb[t];
    };
    // One forward step: (lam, Phi) column offsets of step t -> those of step t + 1 (t < L - 1).
    auto advance = [&](long long t) {
      const float u = k.sc * wn;
      const float gtp = gn * k.csc;     // g_t c(s) = gtp * v(s)
      const float gwh = gn * hn;        // g_t w_hat_t
      inputs_at(t != L - 1 ? t + 1 : t);  // (as in k_sparse_fwd)
      MT out[G][K];
      float pout[G][K];
      float pcc[G][K];  // Phi_t - g_t w_hat_t at the column offsets
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int a = 0; a < K; ++a) pcc[g][a] = pc[g][a] - gwh;
      MT mx = (MT)-INFINITY;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float Vg[K][K];
        vsrc.get(g, Vg);
#pragma unroll
        for (int r = 0; r < K; ++r) {
          // wave priority up a level at each quarter of the step (lowered after the reduction)
          if (g * K + r == G * K / 4) exchange_prio<C, 1>();
          if (g * K + r == G * K / 2) exchange_prio<C, 2>();
          if (g * K + r == 3 * G * K / 4) exchange_prio<C, 3>();
          MT x[K];
          MT m = (MT)-INFINITY;
#pragma unroll
          for (int a = 0; a < K; ++a) {
            x[a] = emit<P>(u, Vg[r][a], lc[g][a], k.kap);
            m = tmax(m, x[a]);
          }
          float e0 = ex2((float)(x[0] - m));
          float s = e0, ph = e0 * __builtin_fmaf(gtp, Vg[r][0], pcc[g][0]);
#pragma unroll
          for (int a = 1; a < K; ++a) {
            const float e = ex2((float)(x[a] - m));
            s += e;
            ph = __builtin_fmaf(e, __builtin_fmaf(gtp, Vg[r][a], pcc[g][a]), ph);
          }
          out[g][r] = m + (MT)lg2(s);
          pout[g][r] = ph * rcp_w<P>(s);
          mx = tmax(mx, out[g][r]);
        }
      }
      MT* mw = msgl[mb] + q * M;
      float* pw = msgp[mb] + q * M;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        store_vec<K>(mw + K * (p + g * LPS), out[g]);
        store_vec<K>(pw + K * (p + g * LPS), pout[g]);
      }
      MT v1[1] = {mx};
      chain_reduce<C, 1, 1u>(v1, red, rp);
      exchange_prio<C, 0>();
      const MT sh = floor(v1[0]);
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int a = 0; a < K; ++a) {
          lc[g][a] = mw[p + g * LPS + a * NG] - sh;
          pc[g][a] = pw[p + g * LPS + a * NG];
        }
      N += (double)sh;
      if constexpr (C::DB) mb ^= 1; else __syncthreads();
    };

    // ---- phase A: lam and Phi, t = 0 .. L-1 ----------------------------------------------
    for (long long t = 0; t < L; ++t) {
      if constexpr (BM != 2) {
        if (seg == 0 || t % seg == 0) {
          const long long e = seg ? t / seg : t;
          store_hist<KG, BLOCK>(histl(e), &lc[0][0]);
          store_hist<KG, BLOCK>(histp(e), &pc[0][0]);
        }
        if (p == 0) ns[t * SPB + q] = N;
      }
      if (t == L - 1) break;
      advance(t);
    }
    // One more step: lam and Phi at t1 = L, in butterfly order in the message buffer just
    // written. They give the transfer and moment rows (BM 2), the segment's log2 Z (BM 1) and
    // the posterior mean of the centred expectation at the last step (xbar, below).
    float xbar = 0.f;
    {
      const double n_before = N;
      advance(L - 1);
      const double sh = N - n_before;
      const MT* lm = msgl[C::DB ? mb ^ 1 : mb] + q * M;
      const float* pm = msgp[C::DB ? mb ^ 1 : mb] + q * M;
      if constexpr (BM == 2) {
        if (valid) {
          const long long ri = sg * M + bb % M;
#pragma unroll
          for (int g = 0; g < G; ++g)
#pragma unroll
            for (int r = 0; r < K; ++r) {
              const int j = K * (p + g * LPS) + r;
              sa.rows[ri * M + j] = (float)(lm[j] - (MT)sh);
              sa.frows[ri * M + j] = pm[j];
            }
          if (p == 0) sa.rscale[ri] = N;
        }
        continue;  // transfer and moment rows need no backward sweep
      } else {
        // posterior weights of butterfly j at the last step, 2^(lam_L(j) + rho(j)), rho = 0 at a
        // free end: their LSE is log2 Z (BM 1: N + Np0 + the LSE of the relative values), and
        // the weighted mean of Phi_L(j) + Psi(j) is the mean xbar of the centred expectation
        const double* r1 = BM == 1 ? sa.rho1 + sg * M : nullptr;
        const float* s1 = BM == 1 ? sa.psi1 + sg * M : nullptr;
        MT y[G][K];
        MT mx = (MT)-INFINITY;
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int r = 0; r < K; ++r) {
            const int j = K * (p + g * LPS) + r;
            y[g][r] = lm[j] - (MT)sh;
            if constexpr (BM == 1) y[g][r] += (MT)r1[j];
            mx = tmax(mx, y[g][r]);
          }
        MT v1[1] = {mx};
        chain_reduce<C, 1, 1u>(v1, red, rp);
        float s2 = 0.f, s3 = 0.f;
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int r = 0; r < K; ++r) {
            const int j = K * (p + g * LPS) + r;
            const float e = ex2((float)(y[g][r] - v1[0]));
            s2 += e;
            s3 = __builtin_fmaf(e, BM == 1 ? pm[j] + s1[j] : pm[j], s3);
          }
        float v2[2] = {s2, s3};
        chain_reduce<C, 2, 0u>(v2, red, rp);
        if constexpr (BM == 1)
          lz2 = N + ((double)v1[0] + (double)lg2(v2[0])) + sa.sc0[sg * 2 + 1];
        xbar = v2[1] / v2[0];
      }
    }
    __syncthreads();

    // ---- phase B: rho and Psi, posterior, D, gradients, t = L-1 .. 0 ---------------------
    // Segment by segment, replaying each segment's forward offsets from its checkpoint first
    // when the history is checkpointed (one segment of length L otherwise).
    MT rr[G][K];
    float qr[G][K];
    double Np = 0.0;
    if constexpr (BM == 1) {
      const double* r1 = sa.rho1 + sg * M;
      const float* s1 = sa.psi1 + sg * M;
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int r = 0; r < K; ++r) {
          rr[g][r] = (MT)r1[K * (p + g * LPS) + r];
          qr[g][r] = s1[K * (p + g * LPS) + r];
        }
      Np = sa.sc0[sg * 2 + 1];
    } else {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int r = 0; r < K; ++r) { rr[g][r] = (MT)0; qr[g][r] = 0.f; }
    }
    float gws = 0.f;  // grad_w of step t, kept by lane t mod LPS (as w_hat in k_sparse_fwd)
    const long long nseg = seg ? ncp : 1;
    for (long long sgi = nseg - 1; sgi >= 0; --sgi) {
      const long long t0 = seg ? sgi * seg : 0;
      const long long t1 = seg ? (t0 + seg < L ? t0 + seg : L) : L;
      if (CK) {
        load_hist<KG, BLOCK>(histl(sgi), &lc[0][0]);
        load_hist<KG, BLOCK>(histp(sgi), &pc[0][0]);
        inputs_at(t0);
        for (long long t = t0; t < t1; ++t) {
          store_hist<KG, BLOCK>(histl(ncp + (t - t0)), &lc[0][0]);
          store_hist<KG, BLOCK>(histp(ncp + (t - t0)), &pc[0][0]);
          if (t + 1 < t1) advance(t);
        }
      }
      auto entry = [&](long long t) { return seg ? ncp + (t - t0) : t; };
      // lam and Phi offsets of the step being processed, each block's replaced by the previous
      // step's right after their last use (as in k_sparse_fwd)
      MT lcur[G][K];
      float pcur[G][K];
      load_hist<KG, BLOCK>(histl(entry(t1 - 1)), &lcur[0][0]);
      load_hist<KG, BLOCK>(histp(entry(t1 - 1)), &pcur[0][0]);
      double Nn = ns[(t1 - 1) * SPB + q];
      wait_vm0();
      for (long long t = t1 - 1; t >= t0; --t) {
        // unconditional (at the segment's first step the loads re-read step t), as in k_sparse_fwd
        const long long tp = t > t0 ? t - 1 : t;
        const float u = k.sc * wb[t];
        const float gt = gb[t];
        const float gtp = gt * k.csc;
        const float gtk = gt * ik2;
        const float gwh = gt * whb[t];
        const MT LZ = (MT)((lz2 - Nn) - Np);
        Nn = ns[tp * SPB + q];
        __builtin_amdgcn_sched_barrier(0);  // (as in k_sparse_fwd)
        gptr<MT> hln = global(histl(entry(tp)));
        gptr<float> hpn = global(histp(entry(tp)));
        float qrc[G][K];  // Psi_t - g_t w_hat_t at the row offsets
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int r = 0; r < K; ++r) qrc[g][r] = qr[g][r] - gwh;
        // E_t(s) = gamma (X - xbar + h) with X = Phi + g (c - w_hat) + Psi; xs sums it over the
        // states, so xs - h is the part of the mean of X that xbar did not remove
        const float hx = h - xbar;
        float gw = 0.f, xs = 0.f;
        MT mx = (MT)-INFINITY;
        MT rout[G][K];
        float qout[G][K];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float Vg[K][K];
          vsrc.get(g, Vg);
          float fa[K], pv[K];
#pragma unroll
          for (int a = 0; a < K; ++a) {
            // wave priority up a level at each quarter of the step (as in advance)
            if (g * K + a == G * K / 4) exchange_prio<C, 1>();
            if (g * K + a == G * K / 2) exchange_prio<C, 2>();
            if (g * K + a == 3 * G * K / 4) exchange_prio<C, 3>();
            MT y[K];
            float dd[K];
            MT m = (MT)-INFINITY;
#pragma unroll
            for (int r = 0; r < K; ++r) {
              dd[r] = u - Vg[r][a];
              y[r] = emit<P>(u, Vg[r][a], rr[g][r], k.kap);
              m = tmax(m, y[r]);
            }
            float e[K], t2[K];
#pragma unroll
            for (int r = 0; r < K; ++r) {
              e[r] = ex2((float)(y[r] - m));
              t2[r] = __builtin_fmaf(gtp, Vg[r][a], qrc[g][r]);
            }
            float cs = e[0], ps = e[0] * t2[0];
#pragma unroll
            for (int r = 1; r < K; ++r) {
              cs += e[r];
              ps = __builtin_fmaf(e[r], t2[r], ps);
            }
            rout[g][a] = m + (MT)lg2(cs);
            qout[g][a] = ps * rcp_w<P>(cs);
            mx = tmax(mx, rout[g][a]);
            const float f = ex2((float)((m + lcur[g][a]) - LZ));
            const float pa = pcur[g][a] + hx;
            fa[a] = f;
            pv[a] = pa;
            xs = __builtin_fmaf(f, __builtin_fmaf(pa, cs, ps), xs);
            // (a uniform branch per 4x4 block: it also bounds the live ranges the scheduler
            // builds across blocks, which keeps this kernel at two waves per SIMD)
            if (valid) {
#pragma unroll
              for (int r = 0; r < K; ++r) {
                const float gm = e[r] * f;
                const float eh = gm * (t2[r] + pa);
                gw = __builtin_fmaf(Vg[r][a], eh, gw);
                acc[g][r][a] = __builtin_fmaf(gtk, gm, __builtin_fmaf(dd[r], eh, acc[g][r][a]));
              }
            }
          }
          hln = after(hln, fa);
          hpn = after(hpn, pv);
          load_hist_part<K, BLOCK>(hln, g * K, lcur[g]);
          load_hist_part<K, BLOCK>(hpn, g * K, pcur[g]);
        }
        MT* mw = msgl[mb] + q * M;
        float* pw = msgp[mb] + q * M;
        if (t > 0) {
#pragma unroll
          for (int g = 0; g < G; ++g)
#pragma unroll
            for (int a = 0; a < K; ++a) {
              mw[p + g * LPS + a * NG] = rout[g][a];
              pw[p + g * LPS + a * NG] = qout[g][a];
            }
        }
        MT v2[3] = {(MT)gw, mx, (MT)xs};
        chain_reduce<C, 3, 2u>(v2, red, rp);
        exchange_prio<C, 0>();
        xbar += (float)v2[2] - h;
        {  // kept by lane t mod LPS and written once per LPS steps, as w_hat in k_sparse_fwd
          const float gwt = 2.0f * k.inv_t * ((float)v2[0] * k.csc - h * wb[t]);
          if (p == (int)(t % LPS)) gws = gwt;
          if (t % LPS == 0) {
            const unsigned lane = opaque((unsigned)p);  // (as in k_sparse_fwd)
            if (valid && t + lane < L) grad_w[wofs + t + lane] = gws;
          }
        }
        if (t == 0) break;
        const MT sh = floor(v2[1]);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          MT tm[K];
          float tp[K];
          load_vec<K>(mw + K * (p + g * LPS), tm);
          load_vec<K>(pw + K * (p + g * LPS), tp);
#pragma unroll
          for (int r = 0; r < K; ++r) { rr[g][r] = tm[r] - sh; qr[g][r] = tp[r]; }
        }
        Np += (double)sh;
        if constexpr (C::DB) mb ^= 1; else __syncthreads();
      }
    }
  }

  // Codebook-gradient partial of this slot: combine the chains of the block (fixed xor order),
  // then one copy writes its states.
  if constexpr (BM == 2) return;  // transfer and moment rows have no gradient part
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int r = 0; r < K; ++r)
#pragma unroll
      for (int a = 0; a < K; ++a) {
        float v = acc[g][r][a];
        if constexpr (SPB > 1) {
#pragma unroll
          for (int o = LPS; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
        }
        if (q == 0) partial[(size_t)blockIdx.x * C::S + K * (p + g * LPS) + r + a * M] = k2 * v;
      }
}

// ---------------------------------------------------------------------------------------------
// ---------------------------------------------------------------------------------------------
// Backward for chains of 1024 lanes. Each message array of a chain (lam / rho and Phi / Psi)
// fills LDS with a single buffer, so a recursion step reads its inputs from LDS while it
// computes, keeps its outputs in registers until every lane has read (the chain reduction's
// barrier), then writes them. The per-state codebook-gradient sums (64 per lane) do not fit in
// registers next to that, so they get a phase of their own:
//   phase A: lam and Phi forward, recording the lane's column offsets per step (as k_sparse_bwd);
//   phase B: rho and Psi backward with the posterior-weighted sums that give grad_w and the
//            centring mean, recording the lane's row offsets and the per-step normaliser;
//   phase C: block by block, the lane's 16 codebook-gradient sums over the steps, from the two
//            recorded histories; the block's codebook values stay in registers for the pass and
//            the sums are added into the slot's partial row once per pass.
// With checkpoints, phases B and C run segment by segment after each segment's replay; the
// lane's backward rows are parked meanwhile in the history entry of the checkpoint after the
// segment's, which the backward sweep no longer needs.
// ---------------------------------------------------------------------------------------------
template <class C, bool CK>
__global__ void __launch_bounds__(C::BLOCK)
k_sparse_bwd_wide(const float* __restrict__ cb, const float* __restrict__ w, long long B,
                  long long L, Consts k, const double* __restrict__ saved_lz,
                  const float* __restrict__ saved_what, const float* __restrict__ gup,
                  const float* __restrict__ hup, float* __restrict__ grad_w,
                  float* __restrict__ partial, void* __restrict__ ws, size_t slot_bytes,
                  long long units, long long seg_arg) {
  using P = typename C::P;
  using MT = typename C::MT;
  constexpr int K = C::K, G = C::G, LPS = C::LPS, NG = C::NG, M = C::M, KG = C::KG;
  static_assert(C::SPB == 1 && C::BLOCK == LPS, "one chain per block");
  __shared__ __attribute__((aligned(16))) MT msgl[M];
  __shared__ __attribute__((aligned(16))) float msgp[M];
  __shared__ double red[2 * C::NWAVES * 4];
  const int p = threadIdx.x;
  const float k2 = 2.0f * k.inv_t * k.csc;  // (2/T)(w - c) = k2 * (u - v)
  // State K*(p + g*LPS) + r + a*M (block g, row r, column a) of the codebook and of the slot's
  // accumulators: a block-uniform base plus the 32-bit lane offset lo4 = K*p, so that the
  // per-column addresses stay in scalar registers.
  const unsigned lo4 = K * p;
  float* __restrict__ accs = partial + (size_t)blockIdx.x * C::S;
  auto col = [](int g, int a) { return g * K * LPS + a * M; };
  // the block's raw codebook values c[a][r]; the scaled differences u - sc * c are formed
  // from them where used (sdiff), so a load issued a block ahead is not waited for at once
  auto cblock = [&](int g, float (&c)[K][K]) {
#pragma unroll
    for (int a = 0; a < K; ++a) {
      const float* __restrict__ ub = cb + col(g, a);
      load_vec<K>(ub + opaque(lo4), c[a]);
    }
  };
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int a = 0; a < K; ++a) {
      float z[K];
#pragma unroll
      for (int r = 0; r < K; ++r) z[r] = 0.f;
      float* __restrict__ ub = accs + col(g, a);
      store_vec<K>(ub + opaque(lo4), z);
    }

  const long long seg = CK ? seg_arg : 0;
  const long long ncp = seg ? (L + seg - 1) / seg : L;
  const long long nh = seg ? ncp + seg : L;
  char* sb = static_cast<char*>(ws) + (size_t)blockIdx.x * slot_bytes;
  MT* __restrict__ hl = reinterpret_cast<MT*>(sb);
  float* __restrict__ hp = reinterpret_cast<float*>(sb + (size_t)nh * LPS * KG * 8);
  double* __restrict__ ns = reinterpret_cast<double*>(sb + (size_t)nh * LPS * KG * 12);
  // backward rows: rho (8-byte entries) and Psi [H][LPS][KG], then per step the posterior
  // normaliser LZ (double) and the centring mean xbar used at that step (fp32)
  char* sr = sb + (size_t)nh * LPS * KG * 12 + (((size_t)L * 8 + 255) & ~(size_t)255);
  MT* __restrict__ hr = reinterpret_cast<MT*>(sr);
  float* __restrict__ hq = reinterpret_cast<float*>(sr + (size_t)nh * LPS * KG * 8);
  double* __restrict__ lzt = reinterpret_cast<double*>(sr + (size_t)nh * LPS * KG * 12);
  float* __restrict__ xbt = reinterpret_cast<float*>(lzt + L);
  // History entries are block-major, [H][G][LPS][K]: block g of this lane in entry e is at
  // the block-uniform base histX(e) + g*LPS*K plus the 32-bit lane offset lh = K*p.
  const unsigned lh = K * p;
  auto histl = [&](long long e) { return hl + (size_t)e * LPS * KG; };
  auto histp = [&](long long e) { return hp + (size_t)e * LPS * KG; };
  auto histr = [&](long long e) { return hr + (size_t)e * LPS * KG; };
  auto histq = [&](long long e) { return hq + (size_t)e * LPS * KG; };
  int rp = 0;

  for (long long b = blockIdx.x; b < units; b += gridDim.x) {
    const float* __restrict__ wb = w + b * L;
    const float* __restrict__ gb = gup + b * L;
    const float* __restrict__ whb = saved_what + b * L;
    const float h = hup != nullptr ? hup[b] : 0.f;
    const double lz2 = saved_lz[b];

    __syncthreads();  // the previous chain is done with the buffers
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int a = 0; a < K; ++a) {
        msgl[p + g * LPS + a * NG] = (MT)0;
        msgp[p + g * LPS + a * NG] = 0.f;
      }
    __syncthreads();

    MT sh = (MT)0;  // shift still to be subtracted from the column values in msgl
    // the column offsets (lam - sh, Phi) of the current step as history entry e
    auto record = [&](long long e) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        MT lc[K];
        float pc[K];
#pragma unroll
        for (int a = 0; a < K; ++a) {
          lc[a] = msgl[p + g * LPS + a * NG] - sh;
          pc[a] = msgp[p + g * LPS + a * NG];
        }
        store_vec_nt<K>(histl(e) + g * (LPS * K) + opaque(lh), lc);
        store_vec_nt<K>(histp(e) + g * (LPS * K) + opaque(lh), pc);
      }
    };
    // Loads and stores share one in-order completion counter (vmcnt), so waiting for a load
    // also waits for every store issued before it. The steps below therefore issue each block's
    // loads one block ahead, before the stores of the block being computed. Vn holds the next
    // block's raw codebook values (block 0 when a run of steps starts: the codebook is fixed, so
    // the last block of a step loads block 0 for the next). The block loops of advance and of
    // phase B are unrolled (their outputs stay in registers across the chain reduction), so
    // the values loaded ahead are renamed, not copied.
    float Vn[K][K];  // raw, [a][r]
    // The step's scalars w_t, g_t, w_hat_t, likewise loaded a step ahead (steps_from(t) when
    // a run of steps starts at t).
    float wn = 0.f, gn = 0.f, whn = 0.f;
    auto steps_from = [&](long long t) {
      wn = vload(wb, t);
      gn = vload(gb, t);
      whn = vload(whb, t);
    };
    // One forward step (lam, Phi) of step t -> raw rows of step t + 1, written over the buffer
    // once every lane has read; records the inputs as entry e (e >= 0); returns the outputs'
    // chain-wide maximum.
    auto advance = [&](long long t, long long e) -> MT {
      const float u = k.sc * wn;
      const float gt = gn;           // g_t c(s) from the raw codebook value
      const float gwh = gn * whn;    // g_t w_hat_t
      steps_from(t != L - 1 ? t + 1 : t);
      MT lo[G][K];
      float po[G][K];
      MT mx = (MT)-INFINITY;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float Vg[K][K];
#pragma unroll
        for (int a = 0; a < K; ++a)
#pragma unroll
          for (int r = 0; r < K; ++r) Vg[a][r] = Vn[a][r];
        cblock((g + 1) % G, Vn);
        MT lc[K];
        float pc[K], pcc[K];
#pragma unroll
        for (int a = 0; a < K; ++a) {
          lc[a] = msgl[p + g * LPS + a * NG] - sh;
          pc[a] = msgp[p + g * LPS + a * NG];
          pcc[a] = pc[a] - gwh;
        }
        if (e >= 0) {
          store_vec_nt<K>(histl(e) + g * (LPS * K) + opaque(lh), lc);
          store_vec_nt<K>(histp(e) + g * (LPS * K) + opaque(lh), pc);
        }
#pragma unroll
        for (int r = 0; r < K; ++r) {
          MT x[K];
          MT m = (MT)-INFINITY;
#pragma unroll
          for (int a = 0; a < K; ++a) {
            x[a] = emit_c<P>(u, k.sc, Vg[a][r], lc[a], k.kap);
            m = tmax(m, x[a]);
          }
          float e0 = ex2((float)(x[0] - m));
          float s = e0, ph = e0 * __builtin_fmaf(gt, Vg[0][r], pcc[0]);
#pragma unroll
          for (int a = 1; a < K; ++a) {
            const float ea = ex2((float)(x[a] - m));
            s += ea;
            ph = __builtin_fmaf(ea, __builtin_fmaf(gt, Vg[a][r], pcc[a]), ph);
          }
          lo[g][r] = m + (MT)lg2(s);
          po[g][r] = ph * rcp_w<P>(s);
          pin(lo[g][r]);
          pin(po[g][r]);
          mx = tmax(mx, lo[g][r]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      MT v1[1] = {mx};
      chain_reduce<C, 1, 1u>(v1, red, rp);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        store_vec<K>(msgl + K * (p + g * LPS), lo[g]);
        store_vec<K>(msgp + K * (p + g * LPS), po[g]);
      }
      __syncthreads();
      return v1[0];
    };

    // ---- phase A: lam and Phi, t = 0 .. L-1, plus one step to t = L -------------------------
    double N = 0.0;
    MT shL = (MT)0;
    cblock(0, Vn);
    steps_from(0);
    for (long long t = 0; t < L; ++t) {
      if (p == 0) ns[t] = N;
      const long long e = seg == 0 ? t : (t % seg == 0 ? t / seg : -1);
      const MT s = floor(advance(t, e));
      if (t == L - 1) {
        shL = s;
        break;
      }
      sh = s;
      N += (double)s;
    }
    // posterior weights of butterfly j at t = L (rho = 0 at the free end): the weighted mean of
    // Phi_L(j) is the mean xbar of the centred expectation at the last step
    float xbar;
    {
      MT ymx = (MT)-INFINITY;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        MT y[K];
        load_vec<K>(msgl + K * (p + g * LPS), y);
#pragma unroll
        for (int r = 0; r < K; ++r) ymx = tmax(ymx, y[r] - shL);
      }
      MT v1[1] = {ymx};
      chain_reduce<C, 1, 1u>(v1, red, rp);
      float s2 = 0.f, s3 = 0.f;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        MT y[K];
        float pm[K];
        load_vec<K>(msgl + K * (p + g * LPS), y);
        load_vec<K>(msgp + K * (p + g * LPS), pm);
#pragma unroll
        for (int r = 0; r < K; ++r) {
          const float e = ex2((float)((y[r] - shL) - v1[0]));
          s2 += e;
          s3 = __builtin_fmaf(e, pm[r], s3);
        }
      }
      float v2[2] = {s2, s3};
      chain_reduce<C, 2, 0u>(v2, red, rp);
      xbar = v2[1] / v2[0];
    }

    // ---- phase B: rho and Psi, posterior, D, gradients, t = L-1 .. 0 ------------------------
    // A lane reads its own rows K*(p + g*LPS) + r (rho raw minus shp, Psi) and writes columns.
    MT shp = (MT)0;
    double Np = 0.0;
    auto set_rows = [&](const MT* lsrc, const float* psrc) {  // own rows from history-shaped data
#pragma unroll
      for (int g = 0; g < G; ++g) {
        MT l4[K];
        float p4[K];
#pragma unroll
        for (int r = 0; r < K; ++r) {
          l4[r] = lsrc ? lsrc[g * K + r] : (MT)0;
          p4[r] = psrc ? psrc[g * K + r] : 0.f;
        }
        store_vec<K>(msgl + K * (p + g * LPS), l4);
        store_vec<K>(msgp + K * (p + g * LPS), p4);
      }
    };
    set_rows(nullptr, nullptr);
    const long long nseg = seg ? ncp : 1;
    for (long long sgi = nseg - 1; sgi >= 0; --sgi) {
      const long long t0 = seg ? sgi * seg : 0;
      const long long t1 = seg ? (t0 + seg < L ? t0 + seg : L) : L;
      if (CK) {
        const bool park = sgi + 1 < nseg;
        if (park) {
#pragma unroll
          for (int g = 0; g < G; ++g) {
            MT l4[K];
            float p4[K];
            load_vec<K>(msgl + K * (p + g * LPS), l4);
            load_vec<K>(msgp + K * (p + g * LPS), p4);
            store_vec_nt<K>(histl(sgi + 1) + g * (LPS * K) + opaque(lh), l4);
            store_vec_nt<K>(histp(sgi + 1) + g * (LPS * K) + opaque(lh), p4);
          }
        }
        __syncthreads();
        {
          MT c0[KG];
          float q0[KG];
#pragma unroll
          for (int g = 0; g < G; ++g) {
            load_vec_nt<K>(histl(sgi) + g * (LPS * K) + opaque(lh), c0 + g * K);
            load_vec_nt<K>(histp(sgi) + g * (LPS * K) + opaque(lh), q0 + g * K);
          }
#pragma unroll
          for (int g = 0; g < G; ++g)
#pragma unroll
            for (int a = 0; a < K; ++a) {
              msgl[p + g * LPS + a * NG] = c0[g * K + a];
              msgp[p + g * LPS + a * NG] = q0[g * K + a];
            }
        }
        __syncthreads();
        sh = (MT)0;
        cblock(0, Vn);
        steps_from(t0);
        for (long long t = t0; t + 1 < t1; ++t) sh = floor(advance(t, ncp + (t - t0)));
        record(ncp + (t1 - 1 - t0));
        __syncthreads();
        if (park) {
          MT c1[KG];
          float q1[KG];
#pragma unroll
          for (int g = 0; g < G; ++g) {
            load_vec_nt<K>(histl(sgi + 1) + g * (LPS * K) + opaque(lh), c1 + g * K);
            load_vec_nt<K>(histp(sgi + 1) + g * (LPS * K) + opaque(lh), q1 + g * K);
          }
          set_rows(c1, q1);
        } else {
          set_rows(nullptr, nullptr);
        }
      }
      auto entry = [&](long long t) { return seg ? ncp + (t - t0) : t; };
      // block-ahead loads (see advance): the next block's codebook values and history entry
      float Vb[K][K];  // raw, [a][r]
      MT hln[K];
      float hpn[K];
      cblock(0, Vb);
      load_vec_nt<K>(histl(entry(t1 - 1)) + opaque(lh), hln);
      load_vec_nt<K>(histp(entry(t1 - 1)) + opaque(lh), hpn);
      double nsn = ns[t1 - 1];  // with steps_from: the step's scalars, a step ahead
      steps_from(t1 - 1);
      for (long long t = t1 - 1; t >= t0; --t) {
        const double Nt = nsn;
        const float wt = wn;
        const float u = k.sc * wn;
        const float gt = gn;
        const float gwh = gn * whn;
        {
          const long long tp = t > t0 ? t - 1 : t;
          nsn = ns[tp];
          steps_from(tp);
        }
        const MT LZ = (MT)((lz2 - Nt) - Np);
        // E_t(s) = gamma (X - xbar + h) with X = Phi + g (c - w_hat) + Psi; xs sums it over the
        // states, so xs - h is the part of the mean of X that xbar did not remove
        const float hx = h - xbar;
        if (p == 0) {
          lzt[t] = (double)LZ;
          xbt[t] = xbar;
        }
        const long long e = entry(t);
        float gw = 0.f, xs = 0.f;
        MT mx = (MT)-INFINITY;
        MT ro[G][K];
        float qo[G][K];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          MT lcur[K], rr[K];
          float pcur[K], qr[K], qrc[K], Vg[K][K];  // Vg raw, [a][r]
#pragma unroll
          for (int i = 0; i < K; ++i) {
            lcur[i] = hln[i];
            pcur[i] = hpn[i];
#pragma unroll
            for (int a = 0; a < K; ++a) Vg[a][i] = Vb[a][i];
          }
          {  // the next block's loads, before this block's stores (the block after the
             // segment's last one re-reads an entry of this segment, which is harmless)
            const long long en = g + 1 < G ? e : entry(t > t0 ? t - 1 : t);
            const int gn = (g + 1) % G;
            cblock(gn, Vb);
            load_vec_nt<K>(histl(en) + gn * (LPS * K) + opaque(lh), hln);
            load_vec_nt<K>(histp(en) + gn * (LPS * K) + opaque(lh), hpn);
          }
          load_vec<K>(msgl + K * (p + g * LPS), rr);
          load_vec<K>(msgp + K * (p + g * LPS), qr);
#pragma unroll
          for (int r = 0; r < K; ++r) {
            rr[r] -= shp;
            qrc[r] = qr[r] - gwh;  // Psi_t - g_t w_hat_t at the row offsets
          }
          store_vec_nt<K>(histr(e) + g * (LPS * K) + opaque(lh), rr);
          store_vec_nt<K>(histq(e) + g * (LPS * K) + opaque(lh), qr);
#pragma unroll
          for (int a = 0; a < K; ++a) {
            const float (&V)[K] = Vg[a];
            MT y[K];
            MT m = (MT)-INFINITY;
#pragma unroll
            for (int r = 0; r < K; ++r) {
              y[r] = emit_c<P>(u, k.sc, V[r], rr[r], k.kap);
              m = tmax(m, y[r]);
            }
            float e4[K], t2[K];
#pragma unroll
            for (int r = 0; r < K; ++r) {
              e4[r] = ex2((float)(y[r] - m));
              t2[r] = __builtin_fmaf(gt, V[r], qrc[r]);
            }
            float cs = e4[0], ps = e4[0] * t2[0];
#pragma unroll
            for (int r = 1; r < K; ++r) {
              cs += e4[r];
              ps = __builtin_fmaf(e4[r], t2[r], ps);
            }
            ro[g][a] = m + (MT)lg2(cs);
            qo[g][a] = ps * rcp_w<P>(cs);
            pin(ro[g][a]);
            pin(qo[g][a]);
            mx = tmax(mx, ro[g][a]);
            const float f = ex2((float)((m + lcur[a]) - LZ));
            const float pa = pcur[a] + hx;
            xs = __builtin_fmaf(f, __builtin_fmaf(pa, cs, ps), xs);
            // sum_r c(s) E_t(s) over the column: f * sum_r c e (t2 + pa)
            float cv = 0.f;
#pragma unroll
            for (int r = 0; r < K; ++r) cv = __builtin_fmaf(V[r] * e4[r], t2[r] + pa, cv);
            gw = __builtin_fmaf(f, cv, gw);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        MT v2[3] = {(MT)gw, mx, (MT)xs};
        chain_reduce<C, 3, 2u>(v2, red, rp);
        xbar += (float)v2[2] - h;
        if (p == 0) grad_w[b * L + t] = 2.0f * k.inv_t * ((float)v2[0] - h * wt);
        if (t == 0) break;
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int a = 0; a < K; ++a) {
            msgl[p + g * LPS + a * NG] = ro[g][a];
            msgp[p + g * LPS + a * NG] = qo[g][a];
          }
        __syncthreads();
        shp = floor(v2[1]);
        Np += (double)shp;
      }

      // ---- phase C: codebook-gradient sums over the segment, block by block ------------------
      // dF/dc(s) = sum_t [ g_t gamma_t(s) + (2/T)(w_t - c(s)) E_t(s) ], gamma_t(s) =
      // 2^(emission + lam column + rho row - LZ_t), E_t(s) = gamma (X - xbar_t + h).
      __syncthreads();  // lane 0's per-step LZ and xbar visible to every lane
#pragma unroll 1
      for (int g = 0; g < G; ++g) {
        float Vg[K][K], ac[K][K];  // raw codebook values and sums, both [a][r]
        cblock(g, Vg);
#pragma unroll
        for (int a = 0; a < K; ++a) {
          const float* __restrict__ ub = accs + col(g, a);
          load_vec<K>(ub + opaque(lo4), ac[a]);
        }
        // A step's inputs: the block's four recorded rows and the step's scalars, loaded one
        // step ahead of the arithmetic into two register sets used in turn (as over_blocks).
        struct CIn {
          MT l[K], r[K];
          float p[K], q[K];
          float w, g, wh, xb;
          double lz;
        };
        auto cload = [&](long long t, CIn& in) {
          const long long e = entry(t);
          load_vec_nt<K>(histl(e) + g * (LPS * K) + opaque(lh), in.l);
          load_vec_nt<K>(histp(e) + g * (LPS * K) + opaque(lh), in.p);
          load_vec_nt<K>(histr(e) + g * (LPS * K) + opaque(lh), in.r);
          load_vec_nt<K>(histq(e) + g * (LPS * K) + opaque(lh), in.q);
          in.w = wb[t];
          in.g = gb[t];
          in.wh = whb[t];
          in.xb = xbt[t];
          in.lz = lzt[t];
        };
        auto cstep = [&](const CIn& in) {
          const float u = k.sc * in.w;
          const float gt = in.g;
          const float gwh = gt * in.wh;
          const MT LZ = (MT)in.lz;
          const float hx = h - in.xb;
#pragma unroll
          for (int a = 0; a < K; ++a) {
            const MT lz = in.l[a] - LZ;
            const float pa = in.p[a] + hx;
#pragma unroll
            for (int r = 0; r < K; ++r) {
              const float c = Vg[a][r];
              const float dd = sdiff<P>(u, k.sc, c);
              const float gm = ex2((float)(emit_c<P>(u, k.sc, c, in.r[r], k.kap) + lz));
              const float eh = gm * (__builtin_fmaf(gt, c, in.q[r] - gwh) + pa);
              ac[a][r] = __builtin_fmaf(gt, gm, __builtin_fmaf(k2 * dd, eh, ac[a][r]));
            }
          }
        };
        CIn ca, cc;
        cload(t1 - 1, ca);
        for (long long t = t1 - 1;; t -= 2) {  // steps t and t - 1 (when t > t0)
          cload(t > t0 ? t - 1 : t, cc);
          cstep(ca);
          if (t == t0) break;
          cload(t - 1 > t0 ? t - 2 : t - 1, ca);
          cstep(cc);
          if (t - 1 == t0) break;
        }
#pragma unroll
        for (int a = 0; a < K; ++a) {
          float* __restrict__ ub = accs + col(g, a);
          store_vec<K>(ub + opaque(lo4), ac[a]);
        }
      }
    }
  }
}

// out[s] = sum over slots i = 0, stride, 2 stride, ... of partial[i][s], in that order
// (deterministic); with no slots, 0.
__global__ void __launch_bounds__(256)
k_reduce_slots(const float* __restrict__ partial, long long slots, long long count,
               long long stride, float* __restrict__ out) {
  const long long s = (long long)blockIdx.x * 256 + threadIdx.x;
  if (s >= count) return;
  float acc = 0.f;
  for (long long i = 0; i < slots; i += stride) acc += partial[(size_t)i * count + s];
  out[s] = acc;
}

// Many slots are summed in two fixed-order passes instead of one chain of dependent loads per
// state: block (x, c) adds the slots of chunk c in order and writes the sum over the chunk's
// first row (which only that block reads), then k_reduce_slots adds the chunk sums in order.
constexpr long long kReduceChunk = 32;
__global__ void __launch_bounds__(256)
k_reduce_chunks(float* __restrict__ partial, long long slots, long long count) {
  const long long s = (long long)blockIdx.x * 256 + threadIdx.x;
  if (s >= count) return;
  const long long i0 = (long long)blockIdx.y * kReduceChunk;
  const long long i1 = i0 + kReduceChunk < slots ? i0 + kReduceChunk : slots;
  float acc = 0.f;
  for (long long i = i0; i < i1; ++i) acc += partial[(size_t)i * count + s];
  partial[(size_t)i0 * count + s] = acc;
}

// out[s] = sum over the slots of partial[slot][s] (partial is scratch and may be overwritten)
int reduce_slots(float* partial, long long slots, long long count, float* out, hipStream_t st) {
  const unsigned gx = (unsigned)((count + 255) / 256);
  long long stride = 1;
  if (slots > 2 * kReduceChunk) {
    hipLaunchKernelGGL(k_reduce_chunks, dim3(gx, (unsigned)((slots + kReduceChunk - 1) / kReduceChunk)),
                       dim3(256), 0, st, partial, slots, count);
    stride = kReduceChunk;
  }
  hipLaunchKernelGGL(k_reduce_slots, dim3(gx), dim3(256), 0, st, partial, slots, count, stride, out);
  return (int)hipGetLastError();
}

template <int n, int k, class P, int KIND = fwd_kind<P>()>
int run_fwd_p(const SparseGeom& g, const float* cb, const float* w, long long B, long long L,
              float T, float* w_hat, float* log_z, float* saved, void* ws, bool ckpt,
              hipStream_t st) {
  using C = Cfg<(1 << k), geom_g(n, k, KIND), geom_lps(n, k, KIND), P, false>;
  static_assert(C::S == (1 << n), "geometry mismatch");
  if (g.G != C::G || g.LPS != C::LPS) return (int)hipErrorInvalidValue;
  const Consts kc = make_consts(T, P::kExactEmit);
  const size_t slot = sparse_fwd_slot_bytes(g, L, ckpt);
  const long long seg = ckpt ? (long long)sparse_seg_len(L) : 0;
  double* slz = reinterpret_cast<double*>(saved);
  float* swh = saved + saved_what_offset(B);
  if constexpr (C::WIDE) {
    const void* kern = ckpt ? reinterpret_cast<const void*>(&k_sparse_fwd_wide<C, true>)
                            : reinterpret_cast<const void*>(&k_sparse_fwd_wide<C, false>);
    const int grid = resident_grid(kern, C::BLOCK, g.slots);
    if (grid <= 0) return (int)hipErrorInvalidConfiguration;
    if (ckpt)
      hipLaunchKernelGGL((k_sparse_fwd_wide<C, true>), dim3((unsigned)grid), dim3(C::BLOCK), 0, st,
                         cb, w, B, L, kc, w_hat, log_z, slz, swh, ws, slot, (long long)g.units,
                         seg);
    else
      hipLaunchKernelGGL((k_sparse_fwd_wide<C, false>), dim3((unsigned)grid), dim3(C::BLOCK), 0,
                         st, cb, w, B, L, kc, w_hat, log_z, slz, swh, ws, slot,
                         (long long)g.units, seg);
    return (int)hipGetLastError();
  } else {
    const void* kern = ckpt ? reinterpret_cast<const void*>(&k_sparse_fwd<C, true>)
                            : reinterpret_cast<const void*>(&k_sparse_fwd<C, false>);
    const int grid = resident_grid(kern, C::BLOCK, g.slots);
    if (grid <= 0) return (int)hipErrorInvalidConfiguration;
    if (ckpt)
      hipLaunchKernelGGL((k_sparse_fwd<C, true>), dim3((unsigned)grid), dim3(C::BLOCK), 0, st, cb,
                         w, B, L, kc, w_hat, log_z, slz, swh, ws, slot, (long long)g.units, seg,
                         SegArgs{});
    else
      hipLaunchKernelGGL((k_sparse_fwd<C, false>), dim3((unsigned)grid), dim3(C::BLOCK), 0, st, cb,
                         w, B, L, kc, w_hat, log_z, slz, swh, ws, slot, (long long)g.units, seg,
                         SegArgs{});
    return (int)hipGetLastError();
  }
}

template <int n, int k, class P, int KIND = bwd_kind<P>()>
int run_bwd_p(const SparseGeom& g, const float* cb, const float* w, long long B, long long L,
              float T, const float* saved, const float* gup, const float* hup, float* grad_w,
              float* grad_c, void* ws, bool ckpt, hipStream_t st) {
  using C = Cfg<(1 << k), geom_g(n, k, KIND), geom_lps(n, k, KIND), P, true>;
  static_assert(C::S == (1 << n), "geometry mismatch");
  if (g.G != C::G || g.LPS != C::LPS) return (int)hipErrorInvalidValue;
  const Consts kc = make_consts(T, P::kExactEmit);
  const size_t slot = sparse_bwd_slot_bytes(g, L, ckpt);
  const long long seg = ckpt ? (long long)sparse_seg_len(L) : 0;
  float* partial = reinterpret_cast<float*>(static_cast<char*>(ws) + slot * (size_t)g.slots);
  const double* slz = reinterpret_cast<const double*>(saved);
  const float* swh = saved + saved_what_offset(B);
  int grid;
  if constexpr (C::WIDE) {
    const void* kern = ckpt ? reinterpret_cast<const void*>(&k_sparse_bwd_wide<C, true>)
                            : reinterpret_cast<const void*>(&k_sparse_bwd_wide<C, false>);
    grid = resident_grid(kern, C::BLOCK, g.slots);
    if (grid <= 0) return (int)hipErrorInvalidConfiguration;
    if (ckpt)
      hipLaunchKernelGGL((k_sparse_bwd_wide<C, true>), dim3((unsigned)grid), dim3(C::BLOCK), 0, st,
                         cb, w, B, L, kc, slz, swh, gup, hup, grad_w, partial, ws, slot,
                         (long long)g.units, seg);
    else
      hipLaunchKernelGGL((k_sparse_bwd_wide<C, false>), dim3((unsigned)grid), dim3(C::BLOCK), 0,
                         st, cb, w, B, L, kc, slz, swh, gup, hup, grad_w, partial, ws, slot,
                         (long long)g.units, seg);
  } else {
    const void* kern = ckpt ? reinterpret_cast<const void*>(&k_sparse_bwd<C, true>)
                            : reinterpret_cast<const void*>(&k_sparse_bwd<C, false>);
    grid = resident_grid(kern, C::BLOCK, g.slots);
    if (grid <= 0) return (int)hipErrorInvalidConfiguration;
    if (ckpt)
      hipLaunchKernelGGL((k_sparse_bwd<C, true>), dim3((unsigned)grid), dim3(C::BLOCK), 0, st, cb,
                         w, B, L, kc, slz, swh, gup, hup, grad_w, partial, ws, slot,
                         (long long)g.units, seg, SegArgs{});
    else
      hipLaunchKernelGGL((k_sparse_bwd<C, false>), dim3((unsigned)grid), dim3(C::BLOCK), 0, st, cb,
                         w, B, L, kc, slz, swh, gup, hup, grad_w, partial, ws, slot,
                         (long long)g.units, seg, SegArgs{});
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  return reduce_slots(partial, (long long)grid, (long long)C::S, grad_c, st);
}

// Shapes whose fp32-message kernels are built in a second translation unit of this file
// (BCJR_ILP_TU) with the machine scheduler that maximises instruction-level parallelism: on
// MI355X (T = 0.1, L = 256, every CU busy) it took the forward at n = 12, 13, 15, 16 and the
// backward at n = 9..14 down by 1.5-4% with bitwise the same results, and made the forward at
// n <= 11 8-15% slower (where the default schedule keeps a higher occupancy).
constexpr bool ilp_fwd_shape(int n, int k) {
  return k == 2 && (n == 12 || n == 13 || n == 15 || n == 16);
}
constexpr bool ilp_bwd_shape(int n, int k) { return k == 2 && n >= 9 && n <= 14; }
// The spread-geometry kernels of small batches (one wave or less per SIMD, so bound by each
// step's latency) are built there too: forward 2-5% faster at n = 8, 10, 12, backward within 1%.
// The segmented backward's transfer and moment rows (BM 2): 4.5-8.4% faster at n = 8, 10, 12
// with that schedule (neutral at n = 4; its segment launches, BM 1, are neutral too).
constexpr bool ilp_bwd_seg_shape(int n, int k, int BM) { return k == 2 && n <= 12 && BM == 2; }

template <int n, int k>
int run_fwd(const SparseGeom& g, const float* cb, const float* w, long long B, long long L,
            float T, float* w_hat, float* log_z, float* saved, void* ws, bool ckpt,
            hipStream_t st) {
  if constexpr (precise_fits<n, k>()) {
    if (use_precise<n, k>(T)) {
      SparseGeom gp;
      if (!sparse_geom(n, k, B, kFwdP, &gp)) return (int)hipErrorInvalidValue;
      return run_fwd_p<n, k, Precise>(gp, cb, w, B, L, T, w_hat, log_z, saved, ws, ckpt, st);
    }
  } else {
    if (T < kPreciseBelowT)
      return run_fwd_p<n, k, Mixed>(g, cb, w, B, L, T, w_hat, log_z, saved, ws, ckpt, st);
  }
  if constexpr (k == 2 && n <= 12) {
    if (geom_spread(n, k, B, kFwd)) {  // a batch too small for the target geometry
      SparseGeom gs;
      if (!sparse_geom(n, k, B, kFwdS, &gs)) return (int)hipErrorInvalidValue;
      return run_fwd_spread_ilp(n, gs, cb, w, B, L, T, w_hat, log_z, saved, ws, ckpt, st);
    }
  }
  if constexpr (ilp_fwd_shape(n, k))
    return run_fwd_fast_ilp(n, g, cb, w, B, L, T, w_hat, log_z, saved, ws, ckpt, st);
  else
    return run_fwd_p<n, k, Fast>(g, cb, w, B, L, T, w_hat, log_z, saved, ws, ckpt, st);
}

template <int n, int k>
int run_bwd(const SparseGeom& g, const float* cb, const float* w, long long B, long long L,
            float T, const float* saved, const float* gup, const float* hup, float* grad_w,
            float* grad_c, void* ws, bool ckpt, hipStream_t st) {
  if constexpr (precise_fits<n, k>()) {
    if (use_precise<n, k>(T)) {
      SparseGeom gp;
      if (!sparse_geom(n, k, B, kBwdP, &gp)) return (int)hipErrorInvalidValue;
      return run_bwd_p<n, k, Precise>(gp, cb, w, B, L, T, saved, gup, hup, grad_w, grad_c, ws,
                                      ckpt, st);
    }
  } else {
    if (T < kPreciseBelowT)
      return run_bwd_p<n, k, Mixed>(g, cb, w, B, L, T, saved, gup, hup, grad_w, grad_c, ws, ckpt,
                                    st);
  }
  if constexpr (k == 2 && n <= 12) {
    if (geom_spread(n, k, B, kBwd)) {  // a batch too small for the target geometry
      SparseGeom gs;
      if (!sparse_geom(n, k, B, kBwdS, &gs)) return (int)hipErrorInvalidValue;
      return run_bwd_spread_ilp(n, gs, cb, w, B, L, T, saved, gup, hup, grad_w, grad_c, ws, ckpt,
                                st);
    }
  }
  if constexpr (ilp_bwd_shape(n, k))
    return run_bwd_fast_ilp(n, g, cb, w, B, L, T, saved, gup, hup, grad_w, grad_c, ws, ckpt, st);
  else
    return run_bwd_p<n, k, Fast>(g, cb, w, B, L, T, saved, gup, hup, grad_w, grad_c, ws, ckpt,
                                 st);
}

// Segmented forward launches (BM 1: segments with boundary messages, BM 2: transfer rows).
template <int n, int k, class P, int BM>
int run_fwd_seg_p(const float* cb, const float* w, long long Bv, long long L, float T,
                  float* w_hat, float* log_z, void* ws, const SegArgs& sa, hipStream_t st) {
  SparseGeom g;
  constexpr int kind = fwd_seg_kind<P, BM>();
  if (!sparse_geom(n, k, Bv, kind, &g)) return (int)hipErrorInvalidValue;
  using C = Cfg<(1 << k), geom_g(n, k, kind), geom_lps(n, k, kind), P, false>;
  if (g.G != C::G || g.LPS != C::LPS) return (int)hipErrorInvalidValue;
  const Consts kc = make_consts(T, P::kExactEmit);
  const size_t slot = BM == 2 ? 0 : sparse_fwd_slot_bytes(g, L, false);
  const int grid = resident_grid(reinterpret_cast<const void*>(&k_sparse_fwd<C, false, BM>),
                                 C::BLOCK, g.slots);
  if (grid <= 0) return (int)hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((k_sparse_fwd<C, false, BM>), dim3((unsigned)grid), dim3(C::BLOCK), 0, st, cb,
                     w, Bv, L, kc, w_hat, log_z, (double*)nullptr, (float*)nullptr, ws, slot,
                     (long long)g.units, 0LL, sa);
  return (int)hipGetLastError();
}

template <int n, int k, int BM>
int run_fwd_seg(const float* cb, const float* w, long long Bv, long long L, float T,
                float* w_hat, float* log_z, void* ws, const SegArgs& sa, hipStream_t st) {
  if constexpr (precise_fits<n, k>())
    if (use_precise<n, k>(T))
      return run_fwd_seg_p<n, k, Precise, BM>(cb, w, Bv, L, T, w_hat, log_z, ws, sa, st);
  return run_fwd_seg_p<n, k, Fast, BM>(cb, w, Bv, L, T, w_hat, log_z, ws, sa, st);
}

// Segmented backward launches (BM 1: segments, writing codebook-gradient partials of `grid`
// slots at `partial`; BM 2: transfer and moment rows). No slot reduction here: the caller sums
// the partials of every launch once.
template <int n, int k, class P, int BM>
int run_bwd_seg_p(const float* cb, const float* w, long long Bv, long long L, float T,
                  const float* w_hat, const float* gup, const float* hup, float* grad_w,
                  float* partial, void* ws, const SegArgs& sa, int* grid_used, hipStream_t st) {
  SparseGeom g;
  constexpr int kind = bwd_seg_kind<P, BM>();
  if (!sparse_geom(n, k, Bv, kind, &g)) return (int)hipErrorInvalidValue;
  using C = Cfg<(1 << k), geom_g(n, k, kind), geom_lps(n, k, kind), P, true>;
  if (g.G != C::G || g.LPS != C::LPS) return (int)hipErrorInvalidValue;
  const Consts kc = make_consts(T, P::kExactEmit);
  const size_t slot = BM == 2 ? 0 : sparse_bwd_slot_bytes(g, L, false);
  const int grid = resident_grid(reinterpret_cast<const void*>(&k_sparse_bwd<C, false, BM>),
                                 C::BLOCK, g.slots);
  if (grid <= 0) return (int)hipErrorInvalidConfiguration;
  *grid_used = grid;
  hipLaunchKernelGGL((k_sparse_bwd<C, false, BM>), dim3((unsigned)grid), dim3(C::BLOCK), 0, st, cb,
                     w, Bv, L, kc, (const double*)nullptr, w_hat, gup, hup, grad_w, partial, ws,
                     slot, (long long)g.units, 0LL, sa);
  return (int)hipGetLastError();
}

template <int n, int k, int BM>
int run_bwd_seg(const float* cb, const float* w, long long Bv, long long L, float T,
                const float* w_hat, const float* gup, const float* hup, float* grad_w,
                float* partial, void* ws, const SegArgs& sa, int* grid_used, hipStream_t st) {
  if constexpr (precise_fits<n, k>())
    if (use_precise<n, k>(T))
      return run_bwd_seg_p<n, k, Precise, BM>(cb, w, Bv, L, T, w_hat, gup, hup, grad_w, partial,
                                              ws, sa, grid_used, st);
  if constexpr (ilp_bwd_seg_shape(n, k, BM)) {
    const SegLaunch sl{sa.nseg, sa.jbase, sa.seglen, sa.lfull, sa.ptot, sa.lam0, sa.rho1, sa.sc0,
                       sa.rows, sa.rscale, sa.phi0, sa.psi1, sa.frows};
    return launch_sparse_backward_seg_ilp(BM, n, k, cb, w, Bv, L, T, w_hat, gup, hup, grad_w,
                                          partial, ws, sl, grid_used, st);
  } else {
    return run_bwd_seg_p<n, k, Fast, BM>(cb, w, Bv, L, T, w_hat, gup, hup, grad_w, partial, ws,
                                         sa, grid_used, st);
  }
}

}  // namespace

#ifdef BCJR_ILP_TU
int run_fwd_fast_ilp(int n, const SparseGeom& g, const float* cb, const float* w, long long B,
                     long long L, float T, float* w_hat, float* log_z, float* saved, void* ws,
                     bool ckpt, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
#define X(N_)                    \
  if constexpr (ilp_fwd_shape(N_, 2)) \
    if (n == N_) return run_fwd_p<N_, 2, Fast>(g, cb, w, B, L, T, w_hat, log_z, saved, ws, ckpt, st);
  X(9) X(10) X(11) X(12) X(13) X(14) X(15) X(16)
#undef X
  return (int)hipErrorInvalidValue;
}

int run_bwd_fast_ilp(int n, const SparseGeom& g, const float* cb, const float* w, long long B,
                     long long L, float T, const float* saved, const float* gup, const float* hup,
                     float* grad_w, float* grad_c, void* ws, bool ckpt, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
#define X(N_)                    \
  if constexpr (ilp_bwd_shape(N_, 2)) \
    if (n == N_)                 \
      return run_bwd_p<N_, 2, Fast>(g, cb, w, B, L, T, saved, gup, hup, grad_w, grad_c, ws, ckpt, st);
  X(9) X(10) X(11) X(12) X(13) X(14) X(15) X(16)
#undef X
  return (int)hipErrorInvalidValue;
}

int run_fwd_spread_ilp(int n, const SparseGeom& g, const float* cb, const float* w, long long B,
                       long long L, float T, float* w_hat, float* log_z, float* saved, void* ws,
                       bool ckpt, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
#define X(N_) \
  if (n == N_) return run_fwd_p<N_, 2, Fast, kFwdS>(g, cb, w, B, L, T, w_hat, log_z, saved, ws, ckpt, st);
  X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12)
#undef X
  return (int)hipErrorInvalidValue;
}

int run_bwd_spread_ilp(int n, const SparseGeom& g, const float* cb, const float* w, long long B,
                       long long L, float T, const float* saved, const float* gup,
                       const float* hup, float* grad_w, float* grad_c, void* ws, bool ckpt,
                       void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
#define X(N_)                                                                                 \
  if (n == N_)                                                                                \
    return run_bwd_p<N_, 2, Fast, kBwdS>(g, cb, w, B, L, T, saved, gup, hup, grad_w, grad_c, ws, \
                                         ckpt, st);
  X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12)
#undef X
  return (int)hipErrorInvalidValue;
}

int launch_sparse_backward_seg_ilp(int mode, int n, int k, const float* codebook, const float* w,
                                   int64_t Bv, int64_t L, float T, const float* w_hat,
                                   const float* grad_w_hat, const float* grad_log_z, float* grad_w,
                                   float* partial, void* ws, const SegLaunch& sl, int* grid_used,
                                   void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const SegArgs sa{sl.nseg, sl.jbase, sl.seglen, sl.lfull, sl.ptot, sl.lam0, sl.rho1, sl.sc0,
                   sl.rows, sl.rscale, sl.phi0, sl.psi1, sl.frows};
  if (k != 2) return (int)hipErrorInvalidValue;
#define X(N_)                                                                               \
  if (n == N_) {                                                                            \
    if constexpr (ilp_bwd_seg_shape(N_, 2, 1))                                              \
      if (mode == 1)                                                                        \
        return run_bwd_seg_p<N_, 2, Fast, 1>(codebook, w, Bv, L, T, w_hat, grad_w_hat,      \
                                             grad_log_z, grad_w, partial, ws, sa, grid_used, st); \
    if constexpr (ilp_bwd_seg_shape(N_, 2, 2))                                              \
      if (mode == 2)                                                                        \
        return run_bwd_seg_p<N_, 2, Fast, 2>(codebook, w, Bv, L, T, w_hat, grad_w_hat,      \
                                             grad_log_z, grad_w, partial, ws, sa, grid_used, st); \
  }
  X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12)
#undef X
  return (int)hipErrorInvalidValue;
}
#else
// Instantiated shapes: see geom_supported().
#define BCJR_SPARSE_SHAPES(X) \
  X(4, 2) X(5, 2) X(6, 2) X(7, 2) X(8, 2) X(9, 2) X(10, 2) X(11, 2) X(12, 2) X(13, 2) X(14, 2) \
  X(15, 2) X(16, 2)
// Shapes with the segmented forward for long chains (its transfer matrices grow as (S/K)^2).
#define BCJR_SCAN_SHAPES(X) \
  X(4, 2) X(5, 2) X(6, 2) X(7, 2) X(8, 2) X(9, 2) X(10, 2) X(11, 2) X(12, 2)

int launch_sparse_forward(const SparseGeom& g, const float* codebook, const float* w, int64_t B,
                          int64_t L, float T, float* w_hat, float* log_z, float* saved, void* ws,
                          bool ckpt, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
#define X(N_, K_)                                                                              \
  if (g.n == N_ && g.k == K_)                                                                  \
    return run_fwd<N_, K_>(g, codebook, w, B, L, T, w_hat, log_z, saved, ws, ckpt, st);
  BCJR_SPARSE_SHAPES(X)
#undef X
  return (int)hipErrorInvalidValue;
}

int launch_sparse_backward(const SparseGeom& g, const float* codebook, const float* w, int64_t B,
                           int64_t L, float T, const float* saved, const float* grad_w_hat,
                           const float* grad_log_z, float* grad_w, float* grad_codebook, void* ws,
                           bool ckpt, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
#define X(N_, K_)                                                                          \
  if (g.n == N_ && g.k == K_)                                                              \
    return run_bwd<N_, K_>(g, codebook, w, B, L, T, saved, grad_w_hat, grad_log_z, grad_w, \
                           grad_codebook, ws, ckpt, st);
  BCJR_SPARSE_SHAPES(X)
#undef X
  return (int)hipErrorInvalidValue;
}

int launch_fill_zero(float* dst, int64_t count, void* stream) {
  if (count <= 0) return 0;
  hipLaunchKernelGGL(k_reduce_slots, dim3((unsigned)((count + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), nullptr, 0LL, (long long)count, 1LL, dst);
  return (int)hipGetLastError();
}

bool sparse_shape_built(int n, int k) {
#define X(N_, K_) if (n == N_ && k == K_) return true;
  BCJR_SPARSE_SHAPES(X)
#undef X
  return false;
}

int launch_sparse_forward_seg(int mode, int n, int k, const float* codebook, const float* w,
                              int64_t Bv, int64_t L, float T, float* w_hat, float* log_z, void* ws,
                              const SegLaunch& sl, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const SegArgs sa{sl.nseg, sl.jbase, sl.seglen, sl.lfull, sl.ptot, sl.lam0, sl.rho1, sl.sc0,
                   sl.rows, sl.rscale, nullptr, nullptr, nullptr};
#define X(N_, K_)                                                                            \
  if (n == N_ && k == K_)                                                                    \
    return mode == 2 ? run_fwd_seg<N_, K_, 2>(codebook, w, Bv, L, T, w_hat, log_z, ws, sa, st) \
                     : run_fwd_seg<N_, K_, 1>(codebook, w, Bv, L, T, w_hat, log_z, ws, sa, st);
  BCJR_SCAN_SHAPES(X)
#undef X
  return (int)hipErrorInvalidValue;
}

int launch_sparse_backward_seg(int mode, int n, int k, const float* codebook, const float* w,
                               int64_t Bv, int64_t L, float T, const float* w_hat,
                               const float* grad_w_hat, const float* grad_log_z, float* grad_w,
                               float* partial, void* ws, const SegLaunch& sl, int* grid_used,
                               void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const SegArgs sa{sl.nseg, sl.jbase, sl.seglen, sl.lfull, sl.ptot, sl.lam0, sl.rho1, sl.sc0,
                   sl.rows, sl.rscale, sl.phi0, sl.psi1, sl.frows};
#define X(N_, K_)                                                                          \
  if (n == N_ && k == K_)                                                                  \
    return mode == 2 ? run_bwd_seg<N_, K_, 2>(codebook, w, Bv, L, T, w_hat, grad_w_hat,    \
                                              grad_log_z, grad_w, partial, ws, sa,         \
                                              grid_used, st)                               \
                     : run_bwd_seg<N_, K_, 1>(codebook, w, Bv, L, T, w_hat, grad_w_hat,    \
                                              grad_log_z, grad_w, partial, ws, sa,         \
                                              grid_used, st);
  BCJR_SCAN_SHAPES(X)
#undef X
  return (int)hipErrorInvalidValue;
}

int launch_reduce_slots(float* partial, int64_t slots, int S, float* out, void* stream) {
  return reduce_slots(partial, (long long)slots, (long long)S, out, static_cast<hipStream_t>(stream));
}

bool scan_shape_built(int n, int k) {
#define X(N_, K_) \
  if (n == N_ && k == K_) return true;
  BCJR_SCAN_SHAPES(X)
#undef X
  return false;
}

#endif  // BCJR_ILP_TU
}  // namespace bcjr

// Boundary messages of the segmented forward for long chains (parallel in L).
//
// The bitshift trellis's butterfly messages obey lam_{t+1} = lam_t (x) A_t and
// rho_t = A_{t+1} (x) rho_{t+1} in the (log-sum-exp, +) semiring, one M x M matrix A_t per step
// (the transfer-matrix view of the BCJR-QAT abstract). A chain cut into segments j = 0..P-1
// with transfer matrices Q_j (rows from k_sparse_fwd's transfer-row mode) has
//   lam at the start of segment j+1  = lam at the start of segment j (x) Q_j,   lam_0 = 0,
//   rho at the end of segment j-1    = Q_j (x) rho at the end of segment j,    rho_{P-1} = 0
// (free start and free end). k_scan_bounds runs these two scans, one block per chain and
// direction, sequentially over the segments, and stores every boundary vector normalised by
// the integer floor of its maximum together with that scale, the form the segment kernels take.
//
// With moments (the backward's scan), the conditional expectations travel with the messages:
//   Phi at the start of segment j+1 (j') = sum_i w(i, j') (Phi at the start of j (i) + F_j(i, j')),
//   Psi at the end of segment j-1 (i)    = sum_j' v(i, j') (F_j(i, j') + Psi at the end of j (j')),
// w and v being the softmax weights of the corresponding log-sum-exp, F_j the segment's moment
// rows (k_sparse_bwd's transfer-row mode), Phi = 0 at the start and Psi = 0 at the end.
//
// Q_j arrives as fp32 row offsets Qn(i, .) <= 0 plus a double row scale rs(i):
// Q(i, j) = rs(i) + Qn(i, j) (log2). Vectors and scales are double; each log-sum-exp is formed
// against its own maximum with fp32 exponentials, so only offsets below the maximum are
// rounded to fp32. Row tiles of Q_j are staged through LDS (padded stride), the next tile
// being loaded into registers while the current one is reduced; every output's reduction is
// split over 256/M threads (adjacent lanes, combined with shuffles).
#include <hip/hip_runtime.h>

#include <math.h>

#include "internal.h"

namespace bcjr {
namespace {

constexpr int kScanBlock = 256;
constexpr int kTileFloats = 8192;                           // one staged tile of Q rows
constexpr int kTileVec = kTileFloats / 4 / kScanBlock;      // float4 loads per thread

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }

__device__ double block_max(double v, double* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) red[wv] = v;
  __syncthreads();
  double r = red[0];
  for (int i = 1; i < kScanBlock / 64; ++i) r = fmax(r, red[i]);
  return r;
}

// Running log-sum-exp (max m, sum s relative to m, and the weighted moment sum t) merged with
// another.
__device__ __forceinline__ void lse_merge(float& m, float& s, float& t, float m2, float s2,
                                          float t2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  const float a = ex2(m - mn), b = ex2(m2 - mn);
  s = s * a + s2 * b;
  t = t * a + t2 * b;
  m = mn;
}

// Combine the partial (m, s, t) of the `width` adjacent lanes that share an output.
__device__ __forceinline__ void group_lse(float& m, float& s, float& t, int width) {
  for (int o = 1; o < width; o <<= 1) {
    const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(s, o), t2 = __shfl_xor(t, o);
    lse_merge(m, s, t, m2, s2, t2);
  }
}

// rows: [chains][ptot][M][M] fp32 offsets; rscale: [chains][ptot][M];
// lam0, rho1: [chains][ptot][M]; sc0: [chains][ptot][2]. R rows per tile, R * M <= kTileFloats.
// MOM: also frows [chains][ptot][M][M] (moment rows) -> phi0, psi1 [chains][ptot][M].
template <bool MOM>
__global__ void __launch_bounds__(kScanBlock)
k_scan_bounds(const float* __restrict__ rows, const double* __restrict__ rscale,
              const float* __restrict__ frows, long long ptot, int M, int R,
              double* __restrict__ lam0, double* __restrict__ rho1, double* __restrict__ sc0,
              float* __restrict__ phi0, float* __restrict__ psi1) {
  extern __shared__ __attribute__((aligned(16))) double smd[];
  const int RS = M + 4;  // padded tile row stride (keeps 16-byte alignment)
  double* va = smd;                                  // current boundary vector [M]
  double* vb = va + M;                               // next one [M]; first the row scales
  double* red = vb + M;                              // reduction scratch [4]
  float* vf = reinterpret_cast<float*>(red + 4);     // fp32 relative vector [M]
  float* ma = vf + M;                                // current moment vector [M] (MOM)
  float* mbv = ma + M;                               // next one [M] (MOM)
  float* tile = mbv + M;                             // [R][RS]
  float* ftile = tile + R * RS;                      // [R][RS] (MOM)
  const long long c = blockIdx.x;
  const bool fwd = blockIdx.y == 0;
  const int tid = threadIdx.x;
  const int ntile = M / R;
  const long long nstep = ptot - 1;  // matrix-vector steps of the scan
  for (int i = tid; i < M; i += kScanBlock) {
    va[i] = 0.0;
    if (MOM) ma[i] = 0.f;
  }

  // segment of scan step q: forward Q_q, backward Q_{ptot-1-q}
  auto seg_of = [&](long long q) { return c * ptot + (fwd ? q : ptot - 1 - q); };
  const int nv = R * M / 4;  // float4 vectors per tile
  // Prefetch registers: tile u of scan step q (lanes past the tile reload its first vector) and,
  // with tile 0, the thread's share of the segment's row scales (rows tid + 256 x).
  float4 rv[kTileVec], fv[MOM ? kTileVec : 1];
  double rr[4];
#define BCJR_LOAD_TILE(Q_, U_)                                                              \
  do {                                                                                      \
    const long long sg_ = seg_of(Q_);                                                       \
    const long long o_ = (sg_ * M + (long long)(U_) * R) * M;                               \
    const float4* src_ = reinterpret_cast<const float4*>(rows + o_);                        \
    _Pragma("unroll") for (int v_ = 0; v_ < kTileVec; ++v_) {                               \
      const int f_ = tid + v_ * kScanBlock;                                                 \
      rv[v_] = src_[f_ < nv ? f_ : 0];                                                      \
    }                                                                                       \
    if constexpr (MOM) {                                                                    \
      const float4* fs_ = reinterpret_cast<const float4*>(frows + o_);                      \
      _Pragma("unroll") for (int v_ = 0; v_ < kTileVec; ++v_) {                             \
        const int f_ = tid + v_ * kScanBlock;                                               \
        fv[v_] = fs_[f_ < nv ? f_ : 0];                                                     \
      }                                                                                     \
    }                                                                                       \
    if ((U_) == 0) {                                                                        \
      _Pragma("unroll") for (int x_ = 0; x_ < 4; ++x_) {                                    \
        const int i_ = tid + x_ * kScanBlock;                                               \
        rr[x_] = rscale[sg_ * M + (i_ < M ? i_ : 0)];                                       \
      }                                                                                     \
    }                                                                                       \
  } while (0)
  auto store_normalised = [&](const double* v, long long sg, double* out, double* scale) {
    double m = -INFINITY;
    for (int i = tid; i < M; i += kScanBlock) m = fmax(m, v[i]);
    const double sh = floor(block_max(m, red));
    for (int i = tid; i < M; i += kScanBlock) out[sg * M + i] = v[i] - sh;
    if (tid == 0) *scale = sh;
  };

  // thread roles: forward output o = tid / tpo with rows ch, ch + tpo, ...; M > 256 loops outputs
  const int tpo = M >= kScanBlock ? 1 : kScanBlock / M;
  const int tpr = kScanBlock / R;  // backward: threads per row of a tile (R <= 256)
#pragma unroll
  for (int v = 0; v < kTileVec; ++v) rv[v] = float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int v = 0; v < (MOM ? kTileVec : 1); ++v) fv[v] = float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int x = 0; x < 4; ++x) rr[x] = 0.0;
  if (nstep > 0) BCJR_LOAD_TILE(0, 0);
  for (long long q = 0;; ++q) {
    const long long sgb = c * ptot + (fwd ? q : ptot - 1 - q);  // boundary this vector belongs to
    __syncthreads();
    store_normalised(va, sgb, fwd ? lam0 : rho1, sc0 + sgb * 2 + (fwd ? 0 : 1));
    if constexpr (MOM) {
      float* mo = (fwd ? phi0 : psi1) + sgb * M;
      for (int i = tid; i < M; i += kScanBlock) mo[i] = ma[i];
    }
    if (q == nstep) break;

    // row scales of this step's segment (in the output buffer: the forward consumes them
    // before any output is written, the backward reads row i's just before writing row i),
    // and the fp32 relative input vector
    double* rsd = vb;
#pragma unroll
    for (int x = 0; x < 4; ++x)
      if (tid + x * kScanBlock < M) rsd[tid + x * kScanBlock] = rr[x];
    __syncthreads();
    double m_in = -INFINITY;
    for (int i = tid; i < M; i += kScanBlock) m_in = fmax(m_in, fwd ? va[i] + rsd[i] : va[i]);
    m_in = block_max(m_in, red);
    for (int i = tid; i < M; i += kScanBlock)
      vf[i] = (float)((fwd ? va[i] + rsd[i] : va[i]) - m_in);

    float pm[4], ps[4], pt[4];  // forward partials for up to 4 outputs (M <= 1024)
#pragma unroll
    for (int x = 0; x < 4; ++x) { pm[x] = -INFINITY; ps[x] = 0.f; pt[x] = 0.f; }
    for (int u = 0; u < ntile; ++u) {
      __syncthreads();
#pragma unroll
      for (int v = 0; v < kTileVec; ++v) {
        const int f = tid + v * kScanBlock;
        if (f < nv) {
          const int e = (4 * f / M) * RS + (4 * f % M);
          *reinterpret_cast<float4*>(tile + e) = rv[v];
          if constexpr (MOM) *reinterpret_cast<float4*>(ftile + e) = fv[v];
        }
      }
      __syncthreads();
      if (u + 1 < ntile) BCJR_LOAD_TILE(q, u + 1);
      else if (q + 1 < nstep) BCJR_LOAD_TILE(q + 1, 0);
      const int i0 = u * R;
      if (fwd) {
        // out(o) += over tile rows i: vf(i) + Qn(i, o)
        const int nout = M > kScanBlock ? M / kScanBlock : 1;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          if (x >= nout) break;
          const int o = M > kScanBlock ? tid + x * kScanBlock : tid / tpo;
          const int ch = M > kScanBlock ? 0 : tid % tpo;
          float tm = -INFINITY;
          for (int r = ch; r < R; r += tpo) tm = fmaxf(tm, vf[i0 + r] + tile[r * RS + o]);
          if (tm == -INFINITY) continue;
          float ts = 0.f, tt = 0.f;
          for (int r = ch; r < R; r += tpo) {
            const float e = ex2(vf[i0 + r] + tile[r * RS + o] - tm);
            ts += e;
            if constexpr (MOM) tt = __builtin_fmaf(e, ma[i0 + r] + ftile[r * RS + o], tt);
          }
          lse_merge(pm[x], ps[x], pt[x], tm, ts, tt);
        }
      } else {
        // out(i0 + row) = rs + m_in + LSE_j' (Qn(i, j') + vf(j')), complete within the tile
        const int row = tid / tpr, ch = tid % tpr;
        float tm = -INFINITY;
        for (int j = ch; j < M; j += tpr) tm = fmaxf(tm, tile[row * RS + j] + vf[j]);
        float ts = 0.f, tt = 0.f;
        if (tm != -INFINITY)
          for (int j = ch; j < M; j += tpr) {
            const float e = ex2(tile[row * RS + j] + vf[j] - tm);
            ts += e;
            if constexpr (MOM) tt = __builtin_fmaf(e, ftile[row * RS + j] + ma[j], tt);
          }
        group_lse(tm, ts, tt, tpr);
        if (ch == 0) {
          vb[i0 + row] = rsd[i0 + row] + m_in + (double)tm + (double)lg2(ts);
          if constexpr (MOM) mbv[i0 + row] = tt / ts;
        }
      }
    }
    if (fwd) {
      const int nout = M > kScanBlock ? M / kScanBlock : 1;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        if (x >= nout) break;
        group_lse(pm[x], ps[x], pt[x], M > kScanBlock ? 1 : tpo);
        const int o = M > kScanBlock ? tid + x * kScanBlock : tid / tpo;
        if (M > kScanBlock || tid % tpo == 0) {
          vb[o] = m_in + (double)pm[x] + (double)lg2(ps[x]);
          if constexpr (MOM) mbv[o] = pt[x] / ps[x];
        }
      }
    }
    __syncthreads();
    double* t = va; va = vb; vb = t;
    if constexpr (MOM) {
      float* tf = ma; ma = mbv; mbv = tf;
    }
  }
#undef BCJR_LOAD_TILE
}

// ---------------------------------------------------------------------------------------------
// The same scans for M <= 64 with one wave per chain and direction: lane l owns element l of the
// boundary vectors and output l of each step, reductions are wave shuffles, and each segment's
// rows (and moment rows) are staged in LDS with a padded stride (M + 1: the backward reads a row
// per lane without bank conflicts) while the next segment's are loaded into registers.
// ---------------------------------------------------------------------------------------------
constexpr int kWaveTile = 64 * 64 / 4 / 64;  // float4 per lane for a 64 x 64 tile

__device__ __forceinline__ double wave_max(double v) {
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  return v;
}

template <int M, bool MOM>
__global__ void __launch_bounds__(64)
k_scan_wave(const float* __restrict__ rows, const double* __restrict__ rscale,
            const float* __restrict__ frows, long long ptot, double* __restrict__ lam0,
            double* __restrict__ rho1, double* __restrict__ sc0, float* __restrict__ phi0,
            float* __restrict__ psi1) {
  static_assert(M >= 4 && M <= 64, "one wave per chain and direction");
  constexpr int RS = M + 1;
  constexpr int nv = M * M / 4;  // float4 per tile
  __shared__ float tq[M * RS];
  __shared__ float tf[MOM ? M * RS : 1];
  __shared__ float vin[M];
  __shared__ float min_[M];
  const long long c = blockIdx.x;
  const bool fwd = blockIdx.y == 0;
  const int l = threadIdx.x;
  const bool own = l < M;
  const long long nstep = ptot - 1;
  auto seg_of = [&](long long q) { return c * ptot + (fwd ? q : ptot - 1 - q); };

  double v = 0.0;   // boundary vector element l (log2, absolute)
  float mom = 0.f;  // conditional expectation element l (MOM)
  float4 rq[kWaveTile], rf[MOM ? kWaveTile : 1];
  double rs = 0.0;
#define BCJR_WAVE_LOAD(Q_)                                                                  \
  do {                                                                                      \
    const long long sg_ = seg_of(Q_);                                                       \
    const float4* sq_ = reinterpret_cast<const float4*>(rows + sg_ * M * M);                \
    _Pragma("unroll") for (int u_ = 0; u_ < kWaveTile; ++u_) {                              \
      const int f_ = l + 64 * u_;                                                           \
      rq[u_] = sq_[f_ < nv ? f_ : 0];                                                       \
    }                                                                                       \
    if constexpr (MOM) {                                                                    \
      const float4* sf_ = reinterpret_cast<const float4*>(frows + sg_ * M * M);             \
      _Pragma("unroll") for (int u_ = 0; u_ < kWaveTile; ++u_) {                            \
        const int f_ = l + 64 * u_;                                                         \
        rf[u_] = sf_[f_ < nv ? f_ : 0];                                                     \
      }                                                                                     \
    }                                                                                       \
    rs = rscale[sg_ * M + (own ? l : 0)];                                                   \
  } while (0)
  if (nstep > 0) BCJR_WAVE_LOAD(0);
  for (long long q = 0;; ++q) {
    // store the boundary vector (normalised) and expectations of this segment
    const long long sgb = seg_of(q);
    const double sh = floor(wave_max(own ? v : -INFINITY));
    if (own) {
      (fwd ? lam0 : rho1)[sgb * M + l] = v - sh;
      if constexpr (MOM) (fwd ? phi0 : psi1)[sgb * M + l] = mom;
    }
    if (l == 0) sc0[sgb * 2 + (fwd ? 0 : 1)] = sh;
    if (q == nstep) break;
    // stage this step's rows; start loading the next step's
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kWaveTile; ++u) {
      const int f = l + 64 * u;
      if (f < nv) {
        const int e = 4 * f, i = e / M, j = e % M;
        float* d = tq + i * RS + j;
        d[0] = rq[u].x; d[1] = rq[u].y; d[2] = rq[u].z; d[3] = rq[u].w;
        if constexpr (MOM) {
          float* g = tf + i * RS + j;
          g[0] = rf[u].x; g[1] = rf[u].y; g[2] = rf[u].z; g[3] = rf[u].w;
        }
      }
    }
    const double rsq = rs;
    // fwd input a(i) = v(i) + rs(i); bwd input rho(j) = v(j)
    const double a = own ? (fwd ? v + rsq : v) : -INFINITY;
    const double m_in = wave_max(a);
    if (own) {
      vin[l] = (float)(a - m_in);
      if constexpr (MOM) min_[l] = mom;
    }
    __syncthreads();
    if (q + 1 < nstep) BCJR_WAVE_LOAD(q + 1);
    if (own) {
      // forward: column l of the rows (over i); backward: row l (over j)
      const int base = fwd ? l : l * RS;
      const int stride = fwd ? RS : 1;
      // (the moment variant re-reads the LDS in the second pass, unrolled by 8 only: it
      // already holds two prefetched tiles in registers)
      float mx = -INFINITY, sm = 0.f, tm = 0.f;
      if constexpr (!MOM) {
        float x[M];
#pragma unroll
        for (int i = 0; i < M; ++i) {
          x[i] = vin[i] + tq[base + i * stride];
          mx = fmaxf(mx, x[i]);
        }
#pragma unroll
        for (int i = 0; i < M; ++i) sm += ex2(x[i] - mx);
      } else {
#pragma unroll 8
        for (int i = 0; i < M; ++i) mx = fmaxf(mx, vin[i] + tq[base + i * stride]);
#pragma unroll 8
        for (int i = 0; i < M; ++i) {
          const float e = ex2(vin[i] + tq[base + i * stride] - mx);
          sm += e;
          tm = __builtin_fmaf(e, min_[i] + tf[base + i * stride], tm);
        }
      }
      v = (fwd ? m_in : rsq + m_in) + (double)mx + (double)lg2(sm);
      if constexpr (MOM) mom = tm / sm;
    }
  }
#undef BCJR_WAVE_LOAD
}

// ---------------------------------------------------------------------------------------------
// The same boundary vectors (and expectations) by a binary tree over a chain's segments, for
// M <= 64 and chains of many segments. The scan's steps are associative: node i of level l
// covers segments [i 2^l, (i + 1) 2^l) (clipped to the chain) and holds their composed transfer
// matrix, C = C_left (x) C_right in the (log-sum-exp, +) semiring, with, for the moments, the
// composed moment matrix F_C(a, b) = sum_k w(a, k, b) (F_left(a, k) + F_right(k, b)), w the
// softmax weights of C(a, b)'s log-sum-exp. The vectors then come down the tree from the root
// (free start and free end: 0): the forward vector at the start of a node's right child is the
// one at the node's start times the left child's product, the backward vector at the end of its
// left child the right child's product times the one at the node's end. Depth log2 P instead of P
// sequential steps, for M times the arithmetic of the scan (a product costs M^3 terms where a
// step costs M^2). Composed matrices keep the rows' form: fp32 offsets <= 0 and double row
// scales. A node without a right child is its left child.
// ---------------------------------------------------------------------------------------------
template <int M>
struct TreeGeo {
  static constexpr int TPB = M * M < 1024 ? M * M : 1024;  // threads per product
  static constexpr int TPR = TPB / M;                       // threads per output row
  static constexpr int CPT = M / TPR;                       // columns per thread (consecutive)
  static constexpr int RS = M + 4;                          // LDS row stride (16-byte aligned)
  static_assert(TPR <= 64 && (64 % TPR) == 0 && CPT * TPR == M, "tree product geometry");
};

template <int W, class T>
__device__ __forceinline__ T group_max(T v) {
  for (int o = 1; o < W; o <<= 1) v = fmax(v, __shfl_xor(v, o));
  return v;
}

// One product per block: parent node `node` of level (np nodes per chain) from children 2i and
// 2i + 1 of the level below (nc nodes per chain).
template <int M, bool MOM>
__global__ void __launch_bounds__(TreeGeo<M>::TPB)
k_tree_compose(const float* __restrict__ cq, const double* __restrict__ crs,
               const float* __restrict__ cf, long long nc, float* __restrict__ pq,
               double* __restrict__ prs, float* __restrict__ pf, long long np) {
  using G = TreeGeo<M>;
  constexpr int RS = G::RS, TPR = G::TPR, CPT = G::CPT;
  __shared__ __attribute__((aligned(16))) float qb[M * RS];
  __shared__ __attribute__((aligned(16))) float fb[MOM ? M * RS : 4];
  __shared__ float br[M * RS];
  __shared__ float fa[MOM ? M * RS : 1];
  __shared__ double rsb[M];
  const long long node = blockIdx.x;
  const long long ch = node / np, i = node % np;
  const long long left = ch * nc + 2 * i;
  const int t = threadIdx.x;
  const float* __restrict__ aq = cq + left * (M * M);
  const double* __restrict__ ars = crs + left * M;
  float* __restrict__ oq = pq + node * (M * M);
  if (2 * i + 1 >= nc) {  // no right child: the node is its left child
    for (int e = t; e < M * M; e += G::TPB) {
      oq[e] = aq[e];
      if constexpr (MOM) pf[node * (M * M) + e] = cf[left * (M * M) + e];
    }
    for (int e = t; e < M; e += G::TPB) prs[node * M + e] = ars[e];
    return;
  }
  const float* __restrict__ bq = cq + (left + 1) * (M * M);
  for (int e = t; e < M * M; e += G::TPB) {
    qb[(e / M) * RS + e % M] = bq[e];
    if constexpr (MOM) fb[(e / M) * RS + e % M] = cf[(left + 1) * (M * M) + e];
  }
  for (int e = t; e < M; e += G::TPB) rsb[e] = crs[(left + 1) * M + e];
  __syncthreads();
  // row a of A against B's row scales: br(a, k) = QnA(a, k) + rsB(k) - ma, ma the row's maximum
  const int a = t / TPR, c0 = t % TPR;
  double ma = -INFINITY;
  for (int k = c0; k < M; k += TPR) ma = fmax(ma, (double)aq[a * M + k] + rsb[k]);
  ma = group_max<TPR>(ma);
  for (int k = c0; k < M; k += TPR) {
    br[a * RS + k] = (float)(((double)aq[a * M + k] + rsb[k]) - ma);
    if constexpr (MOM) fa[a * RS + k] = cf[left * (M * M) + a * M + k];
  }
  __syncthreads();
  // columns b0 .. b0 + CPT - 1 of row a: C(a, b) = rsA(a) + ma + LSE_k (br(a, k) + QnB(k, b))
  const int b0 = c0 * CPT;
  float mx[CPT], sm[CPT], tm[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) { mx[u] = -INFINITY; sm[u] = 0.f; tm[u] = 0.f; }
  for (int k = 0; k < M; ++k) {
    const float x0 = br[a * RS + k];
#pragma unroll
    for (int u = 0; u < CPT; ++u) mx[u] = fmaxf(mx[u], x0 + qb[k * RS + b0 + u]);
  }
  for (int k = 0; k < M; ++k) {
    const float x0 = br[a * RS + k];
    const float f0 = MOM ? fa[a * RS + k] : 0.f;
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const float e = ex2(x0 + qb[k * RS + b0 + u] - mx[u]);
      sm[u] += e;
      if constexpr (MOM) tm[u] = __builtin_fmaf(e, f0 + fb[k * RS + b0 + u], tm[u]);
    }
  }
  float out[CPT];
  float rmax = -INFINITY;
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    out[u] = mx[u] + lg2(sm[u]);
    rmax = fmaxf(rmax, out[u]);
  }
  rmax = group_max<TPR>(rmax);
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    oq[a * M + b0 + u] = out[u] - rmax;
    if constexpr (MOM) pf[node * (M * M) + a * M + b0 + u] = tm[u] / sm[u];
  }
  if (c0 == 0) prs[node * M + a] = ars[a] + ma + (double)rmax;
}

// One wave per parent node and direction (blockIdx.y: 0 forward, 1 backward): the children's
// boundary vectors from the parent's (zeros at the root, pv == null). Children of level 0 are
// the segments, whose vectors are written normalised (as k_scan_wave stores them).
struct TreeVec {
  double* vf;  // forward vector at each node's start [chains][n][M]
  double* vb;  // backward vector at each node's end
  float* mf;   // Phi at the start (moments)
  float* mb;   // Psi at the end (moments)
};
template <int M, bool MOM>
__global__ void __launch_bounds__(64)
k_tree_down(const float* __restrict__ cq, const double* __restrict__ crs,
            const float* __restrict__ cf, long long nc, TreeVec pv, long long np, TreeVec cv,
            double* __restrict__ lam0, double* __restrict__ rho1, double* __restrict__ sc0,
            float* __restrict__ phi0, float* __restrict__ psi1) {
  __shared__ float vin[M];
  __shared__ float min_[M];
  const long long node = blockIdx.x;
  const long long ch = node / np, i = node % np;
  const bool fwd = blockIdx.y == 0;
  const int l = threadIdx.x;
  const bool own = l < M;
  const long long left = ch * nc + 2 * i;
  const bool has_right = 2 * i + 1 < nc;
  // the parent's vector
  double v = 0.0;
  float mom = 0.f;
  if (pv.vf != nullptr && own) {
    v = (fwd ? pv.vf : pv.vb)[node * M + l];
    if constexpr (MOM) mom = (fwd ? pv.mf : pv.mb)[node * M + l];
  }
  auto put = [&](long long child, double x, float mo) {  // child: global index at level below
    if (cv.vf != nullptr) {
      if (own) {
        (fwd ? cv.vf : cv.vb)[child * M + l] = x;
        if constexpr (MOM) (fwd ? cv.mf : cv.mb)[child * M + l] = mo;
      }
    } else {
      const double sh = floor(wave_max(own ? x : -INFINITY));
      if (own) {
        (fwd ? lam0 : rho1)[child * M + l] = x - sh;
        if constexpr (MOM) (fwd ? phi0 : psi1)[child * M + l] = mo;
      }
      if (l == 0) sc0[child * 2 + (fwd ? 0 : 1)] = sh;
    }
  };
  // the child that inherits the parent's vector: the left one going forward, the right one (or
  // the left one without a right sibling) going backward
  put(fwd || !has_right ? left : left + 1, v, mom);
  if (!has_right) return;
  // the other child: forward, start of the right child = v (x) C_left; backward, end of the left
  // child = C_right (x) v
  const long long m = fwd ? left : left + 1;
  const float* __restrict__ q = cq + m * (M * M);
  const double* __restrict__ rs = crs + m * M;
  const float* __restrict__ f = MOM ? cf + m * (M * M) : nullptr;
  const double rsl = own ? rs[l] : 0.0;
  const double a_in = own ? (fwd ? v + rsl : v) : -INFINITY;
  const double m_in = wave_max(a_in);
  if (own) {
    vin[l] = (float)(a_in - m_in);
    if constexpr (MOM) min_[l] = mom;
  }
  __syncthreads();
  double x = 0.0;
  float mo = 0.f;
  if (own) {
    float mx = -INFINITY, sm = 0.f, tm = 0.f;
    for (int j = 0; j < M; ++j)
      mx = fmaxf(mx, vin[j] + (fwd ? q[j * M + l] : q[l * M + j]));
    for (int j = 0; j < M; ++j) {
      const int e = fwd ? j * M + l : l * M + j;
      const float w = ex2(vin[j] + q[e] - mx);
      sm += w;
      if constexpr (MOM) tm = __builtin_fmaf(w, min_[j] + f[e], tm);
    }
    x = (fwd ? m_in : rsl + m_in) + (double)mx + (double)lg2(sm);
    mo = MOM ? tm / sm : 0.f;
  }
  put(fwd ? left + 1 : left, x, mo);
}

template <int M, bool MOM>
int run_tree(const float* rows, const double* rscale, const float* frows, int64_t chains,
             int64_t ptot, double* lam0, double* rho1, double* sc0, float* phi0, float* psi1,
             void* tree_ws, hipStream_t st) {
  struct Level {
    long long n;
    const float* q;
    const double* rs;
    const float* f;
    TreeVec v;
  };
  Level lv[64];
  int top = 0;
  lv[0] = Level{(long long)ptot, rows, rscale, frows, TreeVec{nullptr, nullptr, nullptr, nullptr}};
  char* p = static_cast<char*>(tree_ws);
  auto take = [&](size_t bytes) { char* r = p; p += round256(bytes); return r; };
  for (long long n = (ptot + 1) / 2;; n = (n + 1) / 2) {
    const size_t nodes = (size_t)chains * (size_t)n;
    Level& L = lv[++top];
    L.n = n;
    float* q = reinterpret_cast<float*>(take(nodes * M * M * sizeof(float)));
    float* f = MOM ? reinterpret_cast<float*>(take(nodes * M * M * sizeof(float))) : nullptr;
    double* rs = reinterpret_cast<double*>(take(nodes * M * sizeof(double)));
    L.v.vf = reinterpret_cast<double*>(take(nodes * M * sizeof(double)));
    L.v.vb = reinterpret_cast<double*>(take(nodes * M * sizeof(double)));
    L.v.mf = MOM ? reinterpret_cast<float*>(take(nodes * M * sizeof(float))) : nullptr;
    L.v.mb = MOM ? reinterpret_cast<float*>(take(nodes * M * sizeof(float))) : nullptr;
    L.q = q;
    L.rs = rs;
    L.f = f;
    hipLaunchKernelGGL((k_tree_compose<M, MOM>), dim3((unsigned)nodes), dim3(TreeGeo<M>::TPB), 0,
                       st, lv[top - 1].q, lv[top - 1].rs, lv[top - 1].f, lv[top - 1].n, q, rs, f,
                       (long long)n);
    if (hipGetLastError() != hipSuccess) return (int)hipErrorLaunchFailure;
    if (n == 1) break;
  }
  for (int l = top; l >= 1; --l) {
    const TreeVec pv = l == top ? TreeVec{nullptr, nullptr, nullptr, nullptr} : lv[l].v;
    const TreeVec cv = l == 1 ? TreeVec{nullptr, nullptr, nullptr, nullptr} : lv[l - 1].v;
    hipLaunchKernelGGL((k_tree_down<M, MOM>), dim3((unsigned)(chains * lv[l].n), 2), dim3(64), 0,
                       st, lv[l - 1].q, lv[l - 1].rs, lv[l - 1].f, lv[l - 1].n, pv, lv[l].n, cv,
                       lam0, rho1, sc0, phi0, psi1);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  return 0;
}

}  // namespace

int launch_scan_bounds(const float* rows, const double* rscale, const float* frows, int64_t chains,
                       int64_t ptot, int M, double* lam0, double* rho1, double* sc0, float* phi0,
                       float* psi1, void* tree_ws, size_t tree_ws_bytes, void* stream) {
  if (chains <= 0) return 0;
  if (M < 4 || M > 1024 || (M & (M - 1))) return (int)hipErrorInvalidValue;
  const bool mom = frows != nullptr;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the tree where it applies (scan_tree_bytes > 0) and its workspace is given
  const size_t need = scan_tree_bytes(chains, ptot, M, mom);
  if (need > 0 && tree_ws != nullptr && need <= tree_ws_bytes) {
#define BCJR_TREE(M_)                                                                           \
  if (M == M_)                                                                                  \
    return mom ? run_tree<M_, true>(rows, rscale, frows, chains, ptot, lam0, rho1, sc0, phi0,    \
                                    psi1, tree_ws, st)                                          \
               : run_tree<M_, false>(rows, rscale, frows, chains, ptot, lam0, rho1, sc0, phi0,   \
                                     psi1, tree_ws, st);
    BCJR_TREE(4) BCJR_TREE(8) BCJR_TREE(16) BCJR_TREE(32) BCJR_TREE(64)
#undef BCJR_TREE
  }
  if (M <= 64) {
#define BCJR_WAVE(M_)                                                                           \
  if (M == M_) {                                                                                \
    if (mom)                                                                                    \
      hipLaunchKernelGGL((k_scan_wave<M_, true>), dim3((unsigned)chains, 2), dim3(64), 0, st,    \
                         rows, rscale, frows, (long long)ptot, lam0, rho1, sc0, phi0, psi1);    \
    else                                                                                        \
      hipLaunchKernelGGL((k_scan_wave<M_, false>), dim3((unsigned)chains, 2), dim3(64), 0, st,   \
                         rows, rscale, frows, (long long)ptot, lam0, rho1, sc0, phi0, psi1);    \
    return (int)hipGetLastError();                                                              \
  }
    BCJR_WAVE(4) BCJR_WAVE(8) BCJR_WAVE(16) BCJR_WAVE(32) BCJR_WAVE(64)
#undef BCJR_WAVE
  }
  // rows per staged tile: R * M <= 8192 floats (4096 with the moment tile beside it), so the
  // LDS stays under 64 KiB up to M = 1024; R >= 4 keeps a backward row within one wave
  const int tf = mom ? kTileFloats / 2 : kTileFloats;
  const int R = M * M <= tf ? M : tf / M;
  const size_t lds = (size_t)(2 * M + 4) * sizeof(double) + (size_t)3 * M * sizeof(float) +
                     (size_t)(mom ? 2 : 1) * R * (M + 4) * sizeof(float);
  if (mom)
    hipLaunchKernelGGL(k_scan_bounds<true>, dim3((unsigned)chains, 2), dim3(kScanBlock), lds, st,
                       rows, rscale, frows, (long long)ptot, M, R, lam0, rho1, sc0, phi0, psi1);
  else
    hipLaunchKernelGGL(k_scan_bounds<false>, dim3((unsigned)chains, 2), dim3(kScanBlock), lds, st,
                       rows, rscale, frows, (long long)ptot, M, R, lam0, rho1, sc0, phi0, psi1);
  return (int)hipGetLastError();
}

}  // namespace bcjr

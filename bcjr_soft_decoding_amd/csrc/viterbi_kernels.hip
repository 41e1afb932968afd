// Viterbi decoding of the bitshift trellis on gfx950: the T -> 0 limit of the BCJR soft
// codeword ("recovering the hard QTIP code as T -> 0", BCJR-QAT abstract).
//
// fp32 min-sum with a fixed op order so that the decoded path is reproducible bit for bit:
//   e_t(s)  = fl(d*d), d = fl(w_t - c(s))            (no contraction in this file)
//   m_0(s)  = e_0(s);  m_t(s') = fl(best + e_t(s')), best = first strict minimum of
//             m_{t-1}(p_a(s')) over a = 0 .. K-1 with p_a(s') = (s' >> k) + a*(S/K)
//   end     = lowest state index attaining min_s m_{L-1}(s); traceback by backpointers.
// The minimum over predecessors depends on s' only through s' >> k, so it is taken once per
// butterfly j: mu_t(j) = min_a m_{t-1}(j + a*M), m_t(s') = fl(mu_t(s' >> k) + e_t(s')), with
// the same K x K block layout as the soft decoder (geom.h). mu_0 = 0 makes m_0 = e_0 exact.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "geom.h"
#include "internal.h"

#pragma clang fp contract(off)

namespace bcjr {
namespace {

template <int K_, int G_, int LPS_>
struct VCfg {
  static constexpr int K = K_, G = G_, LPS = LPS_;
  static constexpr int NG = G * LPS, M = K * NG, S = K * M, KG = K * G;
  static constexpr int SPB = LPS < 64 ? 64 / LPS : 1;
  static constexpr int BLOCK = LPS < 64 ? 64 : LPS;
  static constexpr int NWAVES = BLOCK / 64;
  static constexpr bool DB = (long long)2 * SPB * M * 4 <= 128 * 1024;
  static constexpr int NBUF = DB ? 2 : 1;
};

// (value, state) argmin with the lowest state index on an exact tie.
__device__ __forceinline__ void amin_merge(float& v, int& s, float v2, int s2) {
  if (v2 < v || (v2 == v && s2 < s)) { v = v2; s = s2; }
}

template <class C>
__global__ void __launch_bounds__(C::BLOCK)
k_viterbi(const float* __restrict__ cb, const float* __restrict__ w, long long B, long long L,
          int32_t* __restrict__ states, float* __restrict__ w_hard, uint8_t* __restrict__ bp,
          long long units) {
  constexpr int K = C::K, G = C::G, LPS = C::LPS, NG = C::NG, M = C::M, KG = C::KG;
  constexpr int SPB = C::SPB, BLOCK = C::BLOCK;
  __shared__ float msg[C::NBUF][SPB * M];
  __shared__ float redv[C::NWAVES];
  __shared__ int reds[C::NWAVES];

  const int tid = threadIdx.x;
  const int q = LPS < 64 ? tid / LPS : 0;
  const int p = LPS < 64 ? tid % LPS : tid;

  float c[G][K][K];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int r = 0; r < K; ++r)
#pragma unroll
      for (int a = 0; a < K; ++a) c[g][r][a] = cb[K * (p + g * LPS) + r + a * M];

  uint8_t* __restrict__ bps = bp + (size_t)blockIdx.x * (size_t)L * BLOCK * KG;
  int mb = 0;

  for (long long unit = blockIdx.x; unit < units; unit += gridDim.x) {
    const long long b = unit * SPB + q;
    const bool valid = b < B;
    const float* __restrict__ wb = w + (valid ? b : B - 1) * L;

    float mc[G][K];  // mu_t at this lane's column offsets x + a*NG
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int a = 0; a < K; ++a) mc[g][a] = 0.f;

    for (long long t = 0; t + 1 < L; ++t) {
      const float wt = wb[t];
      float best[G][K];
      uint8_t arg[G][K];
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int r = 0; r < K; ++r) {
          float bv = 0.f;
          int ba = 0;
#pragma unroll
          for (int a = 0; a < K; ++a) {
            const float d = wt - c[g][r][a];
            const float e = d * d;
            const float mval = mc[g][a] + e;
            if (a == 0 || mval < bv) { bv = mval; ba = a; }
          }
          best[g][r] = bv;
          arg[g][r] = (uint8_t)ba;
        }
      // backpointers of step t+1 for this lane's butterflies K*x + r
      uint8_t* bq = bps + ((size_t)(t + 1) * BLOCK + tid) * KG;
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int r = 0; r < K; ++r) bq[g * K + r] = arg[g][r];
      float* mw = msg[mb] + q * M;
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int r = 0; r < K; ++r) mw[K * (p + g * LPS) + r] = best[g][r];
      __syncthreads();
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int a = 0; a < K; ++a) mc[g][a] = mw[p + g * LPS + a * NG];
      if constexpr (C::DB) mb ^= 1; else __syncthreads();
    }

    // final metrics m_{L-1}(s) and the chain-wide argmin (lowest state on a tie)
    float vbest = INFINITY;
    int sbest = K * p;  // a valid state even if every metric is NaN
    {
      const float wt = wb[L - 1];
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int r = 0; r < K; ++r)
#pragma unroll
          for (int a = 0; a < K; ++a) {
            const float d = wt - c[g][r][a];
            const float e = d * d;
            const float mval = mc[g][a] + e;
            amin_merge(vbest, sbest, mval, K * (p + g * LPS) + r + a * M);
          }
    }
    constexpr int W = LPS < 64 ? LPS : 64;
#pragma unroll
    for (int o = W / 2; o >= 1; o >>= 1) {
      const float v2 = __shfl_xor(vbest, o, 64);
      const int s2 = __shfl_xor(sbest, o, 64);
      amin_merge(vbest, sbest, v2, s2);
    }
    if constexpr (LPS > 64) {
      if ((tid & 63) == 0) { redv[tid >> 6] = vbest; reds[tid >> 6] = sbest; }
      __syncthreads();
      vbest = redv[0];
      sbest = reds[0];
      for (int i = 1; i < C::NWAVES; ++i) amin_merge(vbest, sbest, redv[i], reds[i]);
    }
    __syncthreads();  // backpointer writes of every lane visible to the traceback lane

    // traceback by one lane per chain
    if (valid && p == 0) {
      int s = sbest;
      int32_t* st = states + b * L;
      float* wh = w_hard ? w_hard + b * L : nullptr;
      for (long long t = L - 1; t >= 0; --t) {
        st[t] = s;
        if (wh) wh[t] = cb[s];
        if (t == 0) break;
        const int j = s / K;                          // butterfly of s
        const int x = j / K, r = j - K * x;           // j = K*x + r
        const int pl = x % LPS, g = x / LPS;          // owner lane and its block index
        const uint8_t a = bps[((size_t)t * BLOCK + q * LPS + pl) * KG + g * K + r];
        s = j + (int)a * M;
      }
    }
    __syncthreads();  // traceback reads done before the next unit rewrites the backpointers
  }
}

template <int n, int k>
int run_vit(const SparseGeom& g, const float* cb, const float* w, long long B, long long L,
            int32_t* states, float* w_hard, void* ws, hipStream_t st) {
  using C = VCfg<(1 << k), geom_g(n, k, kVit), geom_lps(n, k, kVit)>;
  static_assert(C::S == (1 << n), "geometry mismatch");
  const int grid = resident_grid(reinterpret_cast<const void*>(&k_viterbi<C>), C::BLOCK, g.slots);
  if (grid <= 0) return (int)hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((k_viterbi<C>), dim3((unsigned)grid), dim3(C::BLOCK), 0, st, cb, w, B, L,
                     states, w_hard, static_cast<uint8_t*>(ws), (long long)g.units);
  return (int)hipGetLastError();
}

}  // namespace

#define BCJR_VIT_SHAPES(X) \
  X(4, 2) X(5, 2) X(6, 2) X(7, 2) X(8, 2) X(9, 2) X(10, 2) X(11, 2) X(12, 2) X(13, 2) X(14, 2) \
  X(15, 2) X(16, 2)

int launch_viterbi(const SparseGeom& g, const float* codebook, const float* w, int64_t B,
                   int64_t L, int32_t* states, float* w_hard, void* ws, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
#define X(N_, K_) \
  if (g.n == N_ && g.k == K_) return run_vit<N_, K_>(g, codebook, w, B, L, states, w_hard, ws, st);
  BCJR_VIT_SHAPES(X)
#undef X
  return (int)hipErrorInvalidValue;
}

}  // namespace bcjr

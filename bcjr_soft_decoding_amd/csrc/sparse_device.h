// Device helpers shared by the bitshift-trellis kernel files (sparse_kernels.hip,
// sparse_keep.hip): message precision policies, the emission, cross-lane reductions, vector and
// history copies, the register-resident codebook, and the per-call constants.
#pragma once
#include <hip/hip_runtime.h>

#include <math.h>

#include <type_traits>

#include "geom.h"
#include "internal.h"

// Multiply-adds are fused only within one expression (or explicitly with __builtin_fmaf), never
// across statements, so that every copy of a recursion step rounds identically.
#pragma clang fp contract(on)

namespace bcjr {
namespace {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr double kLog2e = 1.4426950408889634074;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }

// fp32 messages; emission -(u - v)^2 with u = q w, v = q c, q = sqrt(log2(e)/T).
struct Fast {
  using MT = float;
  static constexpr bool kPrecise = false;    // fp64 messages (and their lane geometry)
  static constexpr bool kExactEmit = false;  // emission formed in fp64 from unscaled w and c
};
// fp64 messages; emission -kappa (w - c)^2 with kappa = log2(e)/T applied in fp64.
struct Precise {
  using MT = double;
  static constexpr bool kPrecise = true;
  static constexpr bool kExactEmit = true;
};
// fp32 messages with the emission formed as in Precise: w - c exactly, kappa (w - c)^2 and its
// sum with the message offset in fp64, rounded to fp32 once. For shapes whose fp64 message
// buffers do not fit LDS (the 2^16-state kernels) below kPreciseBelowT.
struct Mixed {
  using MT = float;
  static constexpr bool kPrecise = false;
  static constexpr bool kExactEmit = true;
};

// 1/x for the sums of a softmax (x in [1, K]) that normalise the conditional expectations'
// weights. v_rcp_f32 is within 0.88 ulp of 1/x over [1, 4) (all 2^24 inputs, measured on
// MI355X; mean -0.07 ulp); with fp32 messages and emission, whose rounding at the message
// magnitudes is far larger, it is used as is. The policies with the fp64 emission (the lowest
// temperatures) refine it by one Newton step, to the correctly rounded quotient.
template <class P>
__device__ __forceinline__ float rcp_w(float x) {
  const float r = __builtin_amdgcn_rcpf(x);
  if constexpr (P::kExactEmit) return __builtin_fmaf(__builtin_fmaf(-x, r, 1.0f), r, r);
  return r;
}

// Per-call constants: per-state values v = sc * c, per-step u = sc * w, c = csc * v.
struct Consts {
  float sc, csc;
  double kap;   // log2(e)/T (used by the precise emission)
  float inv_t;  // 1/T
};

// With fp64 messages the difference w - c is itself formed in fp64 (exactly: both are fp32);
// rounded to fp32 it would move the emission by ~kappa (w - c)^2 * 2^-23, which at small T is
// enough to shift near-tied posteriors.
template <class P>
__device__ __forceinline__ typename P::MT emit(float u, float v, typename P::MT off, double kap) {
  if constexpr (P::kExactEmit) {
    // (converted at each use: hoisted out of the step loop, the fp64 codebook values would
    // take twice the registers of the fp32 ones)
    float vv = v;
    asm volatile("" : "+v"(vv));
    const double dd = (double)u - (double)vv;
    return (typename P::MT)__builtin_fma(-(kap * dd), dd, (double)off);
  } else {
    (void)kap;
    const float d = u - v;
    return __builtin_fmaf(-d, d, off);
  }
}
// The scaled difference u - v = u - sc * c from a raw codebook value c, as one fma (with the
// fp64 emission sc = 1, and this is u - c), and the emission from it.
template <class P>
__device__ __forceinline__ float sdiff(float u, float sc, float c) {
  if constexpr (P::kExactEmit) {
    (void)sc;
    return u - c;
  } else {
    return __builtin_fmaf(-sc, c, u);
  }
}
// The emission from a raw codebook value: emit(u, sc * c) with the fp32 difference as one fma
// (with the fp64 emission sc = 1 and the difference is formed in fp64, as in emit).
template <class P>
__device__ __forceinline__ typename P::MT emit_c(float u, float sc, float c, typename P::MT off,
                                                 double kap) {
  if constexpr (P::kExactEmit) {
    (void)sc;
    return emit<P>(u, c, off, kap);
  } else {
    (void)kap;
    const float d = __builtin_fmaf(-sc, c, u);
    return __builtin_fmaf(-d, d, off);
  }
}
// Runs body(g, in) over a lane's G blocks while the inputs of the block after g are loaded by
// load(g + 1, in') into the other of two register sets, used in turn, so that inputs loaded
// ahead are never copied between registers; load(G, .) fetches block 0 of the next step.
template <int G, class In, class Load, class Body>
__device__ __forceinline__ void over_blocks(In& a, In& b, Load&& load, Body&& body) {
  if constexpr (G == 1) {
    b = a;
    load(1, a);
    body(0, b);
  } else {
    static_assert(G % 2 == 0, "blocks are visited in pairs");
#pragma unroll 1
    for (int g = 0; g < G; g += 2) {
      // the barriers keep the scheduler from interleaving the two blocks (which would hold
      // both blocks' intermediates at once)
      load(g + 1, b);
      body(g, a);
      __builtin_amdgcn_sched_barrier(0);
      load(g + 2, a);
      body(g + 1, b);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}
// max through the hardware max instructions (v_max3_f32 / v_max_f64)
__device__ __forceinline__ float tmax(float a, float b) { return fmaxf(a, b); }
__device__ __forceinline__ double tmax(double a, double b) { return fmax(a, b); }

template <int K_, int G_, int LPS_, class P_, bool BWD_>
struct Cfg {
  using P = P_;
  using MT = typename P_::MT;
  static constexpr int K = K_, G = G_, LPS = LPS_;
  static constexpr bool BWD = BWD_;
  static constexpr int NG = G * LPS;  // K x K blocks per chain
  static constexpr int M = K * NG;    // butterflies per chain
  static constexpr int S = K * M;     // states
  static constexpr int KG = K * G;    // message values a lane reads per step
  static constexpr int SPB = LPS < 64 ? 64 / LPS : 1;
  static constexpr int BLOCK = LPS < 64 ? 64 : LPS;
  static constexpr int NWAVES = BLOCK / 64;
  // LDS per buffer: the MT message (+ the fp32 expectation message in the backward).
  static constexpr long long BUF_BYTES = (long long)SPB * M * ((long long)sizeof(MT) + (BWD ? 4 : 0));
  // Double-buffer the message arrays when both buffers fit in 128 KiB, else one buffer and a
  // second barrier per step.
  static constexpr bool DB = 2 * BUF_BYTES <= 128 * 1024;
  static constexpr int NBUF = DB ? 2 : 1;
  // chains of 1024 lanes run the rolled-loop kernels (k_sparse_fwd_wide)
  static constexpr bool WIDE = LPS >= 1024;
};

// Cross-lane moves through DPP (no LDS round trip). CTRL: 0xB1 / 0x4E = quad_perm xor 1 / 2,
// 0x141 = row_half_mirror (lane i <-> 7-i in each 8), 0x140 = row_mirror (i <-> 15-i).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ double dpp(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(b & 0xffffffffLL), CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, 0xF, 0xF, false);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}
template <class T>
__device__ __forceinline__ T comb(T a, T b, bool is_max) { return is_max ? tmax(a, b) : a + b; }

// comb of v with the value of lane l ^ 16 (X32 false) or l ^ 32 (X32 true): a register swapped
// with itself by v_permlane16_swap / v_permlane32_swap holds {own, partner} in its two results
// (in either order), and comb is commutative, so every lane of a pair gets the same bits.
// A VALU move, no LDS round trip.
template <bool X32>
__device__ __forceinline__ void swap_self(unsigned u, unsigned& r0, unsigned& r1) {
  const auto r = X32 ? __builtin_amdgcn_permlane32_swap(u, u, false, false)
                     : __builtin_amdgcn_permlane16_swap(u, u, false, false);
  r0 = r[0];
  r1 = r[1];
}
template <bool X32>
__device__ __forceinline__ float xor_comb(float v, bool is_max) {
  unsigned r0, r1;
  swap_self<X32>(__float_as_uint(v), r0, r1);
  return comb(__uint_as_float(r0), __uint_as_float(r1), is_max);
}
template <bool X32>
__device__ __forceinline__ double xor_comb(double v, bool is_max) {
  const long long b = __double_as_longlong(v);
  unsigned l0, l1, h0, h1;
  swap_self<X32>((unsigned)(b & 0xffffffffLL), l0, l1);
  swap_self<X32>((unsigned)(b >> 32), h0, h1);
  const double d0 = __longlong_as_double(((long long)h0 << 32) | l0);
  const double d1 = __longlong_as_double(((long long)h1 << 32) | l1);
  return comb(d0, d1, is_max);
}

// Reduction over aligned groups of W lanes inside a wave. Every step combines two disjoint
// halves symmetrically (a op b in one half, b op a in the other), so every lane of the group
// ends with the bitwise-identical result.
template <int W, class T>
__device__ __forceinline__ T lanes_reduce(T v, bool is_max) {
  if constexpr (W >= 2) v = comb(v, dpp<0xB1>(v), is_max);
  if constexpr (W >= 4) v = comb(v, dpp<0x4E>(v), is_max);
  if constexpr (W >= 8) v = comb(v, dpp<0x141>(v), is_max);
  if constexpr (W >= 16) v = comb(v, dpp<0x140>(v), is_max);
  if constexpr (W >= 32) v = xor_comb<false>(v, is_max);
  if constexpr (W >= 64) v = xor_comb<true>(v, is_max);
  return v;
}

// Chain-wide reduction of NV values (MASK bit i set = max, clear = sum). Includes one
// workgroup barrier, which also publishes any LDS message writes made before the call.
// For chains wider than a wave the per-wave partials go through `red` (double-buffered by
// `rp`) and are combined in wave order, so every lane gets the same bits.
template <class C, int NV, unsigned MASK, class T>
__device__ __forceinline__ void chain_reduce(T (&v)[NV], double* red, int& rp) {
  if constexpr (C::LPS <= 64) {
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = lanes_reduce<C::LPS>(v[i], (MASK >> i) & 1u);
    __syncthreads();
  } else {
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = lanes_reduce<64>(v[i], (MASK >> i) & 1u);
    // per-wave partials in their own type; the two halves of the double buffer are counted in
    // doubles, so that a float reduction never lands in the half a double reduction just used
    T* r = reinterpret_cast<T*>(red + rp * (C::NWAVES * 4));
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
#pragma unroll
      for (int i = 0; i < NV; ++i) r[wave * 4 + i] = v[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      T acc = r[i];
      for (int wv = 1; wv < C::NWAVES; ++wv)
        acc = ((MASK >> i) & 1u) ? tmax(acc, r[wv * 4 + i]) : acc + r[wv * 4 + i];
      v[i] = acc;
    }
    rp ^= 1;
  }
}

// Wave priority by progress through a step, for chains that span several waves: the chain's
// waves meet at the step's barrier, so a wave that is late holds its partners. Two waves of
// different chains share a SIMD; the step's butterfly rows raise the priority a level at each
// quarter (0 to 3), and the chain reduction lowers it to 0 once its partial sums are read, so the
// wave nearer its barrier issues first. Used in the backward: measured 6-10% faster at 4096 and
// 8192 states (one raised level from the last butterfly block on: 5-7%; from the message stores
// on: 1.7-2.4%), within 1% at 16384; in the forward at 8192 states a raised window cost two
// registers and the second wave per SIMD (+13%), and in the 1024-lane kernels, whose waves are all
// of one chain, 1-2%.
template <class C, int LEVEL>
__device__ __forceinline__ void exchange_prio() {
  if constexpr (C::LPS > 64) __builtin_amdgcn_s_setprio(LEVEL);
}

// Vector copies between registers and memory (LDS or global), 16 bytes at a time.
template <int N, class T>
__device__ __forceinline__ void store_vec(T* __restrict__ dst, const T* src) {
  constexpr int V = 16 / (int)sizeof(T);
  if constexpr (N % V == 0) {
    using Vec = __attribute__((ext_vector_type(V))) T;
#pragma unroll
    for (int i = 0; i < N; i += V) {
      Vec x;
#pragma unroll
      for (int j = 0; j < V; ++j) x[j] = src[i + j];
      *reinterpret_cast<Vec*>(dst + i) = x;
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) dst[i] = src[i];
  }
}
template <int N, class T>
__device__ __forceinline__ void load_vec(const T* __restrict__ src, T* dst) {
  constexpr int V = 16 / (int)sizeof(T);
  if constexpr (N % V == 0) {
    using Vec = __attribute__((ext_vector_type(V))) T;
#pragma unroll
    for (int i = 0; i < N; i += V) {
      const Vec x = *reinterpret_cast<const Vec*>(src + i);
#pragma unroll
      for (int j = 0; j < V; ++j) dst[i + j] = x[j];
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) dst[i] = src[i];
  }
}

// History rows in 16-byte chunks interleaved across the block's lanes: chunk c of lane l of an
// entry sits at entry + (c * BLK + l) * V (V values of 16 bytes), so each vector store or load
// of one chunk moves BLK * 16 contiguous bytes (whole cache lines), not 16 bytes per lane at the
// row's stride. `dst` / `src` point at the lane's first chunk of the entry. The non-temporal
// hint keeps the streams (each entry is written once and read once, a chain later) from
// displacing cached inputs; both changes measured 2-4% faster at S = 4096 (the sweeps are
// power-limited, and fewer partial-line and cached writes cost less energy).
template <int N, int BLK, class T>
__device__ __forceinline__ void store_hist(T* __restrict__ dst, const T* src) {
  constexpr int V = 16 / (int)sizeof(T);
  static_assert(N % V == 0, "whole 16-byte chunks");
  using Vec = __attribute__((ext_vector_type(V))) T;
#pragma unroll
  for (int i = 0; i < N; i += V) {
    Vec x;
#pragma unroll
    for (int j = 0; j < V; ++j) x[j] = src[i + j];
    __builtin_nontemporal_store(x, reinterpret_cast<Vec*>(dst + (size_t)(i / V) * BLK * V));
  }
}
template <int N, int BLK, class T>
__device__ __forceinline__ void load_hist(const T* __restrict__ src, T* dst) {
  constexpr int V = 16 / (int)sizeof(T);
  static_assert(N % V == 0, "whole 16-byte chunks");
  using Vec = __attribute__((ext_vector_type(V))) T;
#pragma unroll
  for (int i = 0; i < N; i += V) {
    const Vec x = __builtin_nontemporal_load(reinterpret_cast<const Vec*>(src + (size_t)(i / V) * BLK * V));
#pragma unroll
    for (int j = 0; j < V; ++j) dst[i + j] = x[j];
  }
}

// A history row pointer in the global address space, made to depend on the values v (no
// instruction): a load through it cannot be issued before v is computed. The phase-B history
// loads replace registers whose last use is in v; hoisted above it they would need registers of
// their own and a copy every step. (Kept global: a generic pointer would turn the loads into
// flat loads, which LDS waits would then also wait for.)
template <class T>
using gptr = const __attribute__((address_space(1))) T*;
template <int N, class T, class V>
__device__ __forceinline__ gptr<T> after(gptr<T> p, const V (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) asm("" : "+v"(p) : "v"(v[i]));
  return p;
}
template <class T>
__device__ __forceinline__ gptr<T> global(const T* p) {
  return (gptr<T>)p;
}

// Waits for every outstanding vector memory access (s_waitcnt vmcnt(0); the expcnt and lgkmcnt
// fields at their maxima). Before a loop whose history loads are waited for by count, so that
// loads issued ahead of it in another order do not make those counts cover the younger loads.
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Values [off, off + N) of a lane's history row (whole 16-byte chunks), as load_hist.
template <int N, int BLK, class T>
__device__ __forceinline__ void load_hist_part(gptr<T> src, int off, T* dst) {
  constexpr int V = 16 / (int)sizeof(T);
  static_assert(N % V == 0, "whole 16-byte chunks");
  using Vec = __attribute__((ext_vector_type(V))) T;
#pragma unroll
  for (int i = 0; i < N; i += V) {
    const Vec x = __builtin_nontemporal_load((gptr<Vec>)(src + (size_t)((off + i) / V) * BLK * V));
#pragma unroll
    for (int j = 0; j < V; ++j) dst[i + j] = x[j];
  }
}

// The same copies with the non-temporal hint, for the 1024-lane backward's history streams
// (written once, read once or twice a whole chain later): they then do not push the codebook,
// which every block rereads each step, out of L2 (measured 4% faster at S = 65536).
template <int N, class T>
__device__ __forceinline__ void store_vec_nt(T* __restrict__ dst, const T* src) {
  constexpr int V = 16 / (int)sizeof(T);
  static_assert(N % V == 0, "whole 16-byte vectors");
  using Vec = __attribute__((ext_vector_type(V))) T;
#pragma unroll
  for (int i = 0; i < N; i += V) {
    Vec x;
#pragma unroll
    for (int j = 0; j < V; ++j) x[j] = src[i + j];
    __builtin_nontemporal_store(x, reinterpret_cast<Vec*>(dst + i));
  }
}
template <int N, class T>
__device__ __forceinline__ void load_vec_nt(const T* __restrict__ src, T* dst) {
  constexpr int V = 16 / (int)sizeof(T);
  static_assert(N % V == 0, "whole 16-byte vectors");
  using Vec = __attribute__((ext_vector_type(V))) T;
#pragma unroll
  for (int i = 0; i < N; i += V) {
    const Vec x = __builtin_nontemporal_load(reinterpret_cast<const Vec*>(src + i));
#pragma unroll
    for (int j = 0; j < V; ++j) dst[i + j] = x[j];
  }
}

// Per-lane codebook values v(s) = sc * c(s) of the lane's K x K blocks, register-resident (the
// 1024-lane kernels, which have no room for them, read them block by block instead).
template <class C>
struct CodebookLane {
  float v[C::G][C::K][C::K];
  __device__ __forceinline__ void init(const float* __restrict__ cb, float sc, int p) {
#pragma unroll
    for (int g = 0; g < C::G; ++g)
#pragma unroll
      for (int r = 0; r < C::K; ++r)
#pragma unroll
        for (int a = 0; a < C::K; ++a) v[g][r][a] = sc * cb[C::K * (p + g * C::LPS) + r + a * C::M];
  }
  __device__ __forceinline__ void get(int g, float (&out)[C::K][C::K]) const {
#pragma unroll
    for (int r = 0; r < C::K; ++r)
#pragma unroll
      for (int a = 0; a < C::K; ++a) out[r][a] = v[g][r][a];
  }
};

// A lane offset made opaque to the optimiser at each use, so that addresses built from it are
// formed where they are used instead of being hoisted out of the step loops as 64-bit address
// registers (one pair per block column, which would not fit next to the messages).
__device__ __forceinline__ unsigned opaque(unsigned x) {
  asm volatile("" : "+v"(x));
  return x;
}
// base + a lane's element offset, formed as a block-uniform base plus an opaque 32-bit byte
// offset: the form the scalar-base global addressing takes (SGPR pair + 32-bit VGPR offset), so
// no 64-bit address is added per use. (With the element index itself opaque, its scaling to bytes
// is a 64-bit offset that addressing cannot take, and every use costs a 64-bit add.)
// The base (the same in every lane) is read into scalar registers first, so that the compiler
// does not fold part of it into a per-lane 64-bit sum.
template <class T>
__device__ __forceinline__ T* at_lane(T* base, unsigned elem) {
  using GB = typename std::conditional<std::is_const<T>::value,
                                       const __attribute__((address_space(1))) char,
                                       __attribute__((address_space(1))) char>::type;
  const unsigned long long a = (unsigned long long)base;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)a);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
  GB* b = (GB*)(((unsigned long long)hi << 32) | lo);
  return (T*)(b + opaque(elem * (unsigned)sizeof(T)));
}

// A per-step scalar read through the vector memory path, behind a zero offset the compiler
// cannot see through. A scalar load shares its completion counter with LDS accesses, and scalar
// loads complete out of order, so the first LDS wait after a scalar load issued a step ahead
// also waits for that load; a vector load is counted in order with the other vector memory
// accesses and is waited for only where it is used.
template <class T>
__device__ __forceinline__ T vload(const T* __restrict__ base, long long i) {
  return base[i + opaque(0u)];
}
// Pins a value's computation at this point. The step outputs are stored only after the chain
// reduction's barrier; without the pin the compiler sinks their arithmetic past it and keeps
// every intermediate of the step alive across the reduction.
template <class T>
__device__ __forceinline__ void pin(T& x) {
  asm volatile("" : "+v"(x));
}

// Messages are carried in fp64 below kPreciseBelowT (geom.h), for every shape whose backward
// message buffers (fp64 + fp32 per butterfly, single-buffered) fit in LDS; the other shapes keep
// fp32 messages there with the fp64 emission (Mixed), and the host layer refuses temperatures
// below their floor (geom_floor_t) for them. The fp64-message kernels use their own lane geometry
// (kFwdP / kBwdP): fewer states per lane, since every message takes two registers.
template <int n, int k>
constexpr bool precise_fits() {
  return geom_precise_fits(n, k);
}
template <class P>
constexpr int fwd_kind() { return P::kPrecise ? kFwdP : kFwd; }
template <class P>
constexpr int bwd_kind() { return P::kPrecise ? kBwdP : kBwd; }
// the segments of the segmented path (boundary mode 1): few chains, more lanes each
template <class P, int BM>
constexpr int fwd_seg_kind() { return BM == 1 && !P::kPrecise ? kFwdS : fwd_kind<P>(); }
template <class P, int BM>
constexpr int bwd_seg_kind() { return BM == 1 && !P::kPrecise ? kBwdS : bwd_kind<P>(); }
template <int n, int k>
bool use_precise(float T) {
  return precise_fits<n, k>() && T < kPreciseBelowT;
}

Consts make_consts(float T, bool precise) {
  Consts c;
  const double kap = kLog2e / (double)T;
  c.kap = kap;
  c.inv_t = 1.0f / T;
  if (precise) {
    c.sc = 1.0f;
    c.csc = 1.0f;
  } else {
    c.sc = (float)sqrt(kap);
    c.csc = 1.0f / c.sc;
  }
  return c;
}

}  // namespace
}  // namespace bcjr

// Hard-code export for the bitshift trellis: the zero-temperature end of the method (BCJR-QAT
// abstract: the hard QTIP code is recovered as T -> 0). A state path is fixed by its first state
// and the k bits each step shifts in, s_t = ((s_{t-1} << k) | b_t) & (S - 1), b_t = s_t mod K.
// The code of a chain is the bit string s_0 (n bits, most significant first) followed by
// b_1 .. b_{L-1} (k bits each, most significant first) in 32-bit words, the first bit in the most
// significant position of word 0 and the unused tail of the last word zero.
//
// Because every state is the last n bits of the stream written so far, s_t is simply the n-bit
// window of the code starting at bit k t: unpacking is one independent window read per state.
// Packing assembles one 32-bit word per thread from the (at most 32/k + 2) fields it covers.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace bcjr {
namespace {

__global__ void __launch_bounds__(256)
k_pack_code(const int* __restrict__ states, long long B, long long L, int n, int k, long long W,
            unsigned* __restrict__ code) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= B * W) return;
  const long long q = idx / W, wi = idx - q * W;
  const long long nbits = (long long)n + (long long)k * (L - 1);
  const long long i0 = wi * 32;
  const long long i1 = i0 + 32 < nbits ? i0 + 32 : nbits;
  const int* __restrict__ st = states + q * L;
  const unsigned S1 = (1u << n) - 1u, K1 = (1u << k) - 1u;
  unsigned word = 0;
  long long i = i0;
  while (i < i1) {
    unsigned v;
    int len, off;
    if (i < n) {  // a bit of the initial state
      v = (unsigned)st[0] & S1;
      len = n;
      off = (int)i;
    } else {      // a bit of the field of step t
      const long long j = i - n;
      const long long t = 1 + j / k;
      v = (unsigned)st[t] & K1;
      len = k;
      off = (int)(j - (t - 1) * k);
    }
    const int room = (int)(i1 - i);
    const int take = len - off < room ? len - off : room;
    const unsigned bits = (v >> (len - off - take)) & ((1u << take) - 1u);
    word |= bits << (32 - (int)(i - i0) - take);
    i += take;
  }
  code[idx] = word;
}

__global__ void __launch_bounds__(256)
k_unpack_code(const unsigned* __restrict__ code, long long B, long long L, int n, int k,
              long long W, const float* __restrict__ cb, int* __restrict__ states,
              float* __restrict__ w_hard) {
  const long long idx = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= B * L) return;
  const long long q = idx / L, t = idx - q * L;
  const unsigned* __restrict__ cw = code + q * W;
  const long long p = (long long)k * t;  // first bit of the window
  const long long w0 = p >> 5;
  const int off = (int)(p & 31);
  const unsigned long long hi = cw[w0];
  const unsigned long long lo = off + n > 32 ? cw[w0 + 1] : 0ull;
  const unsigned long long x = (hi << 32) | lo;
  const int s = (int)((x >> (64 - off - n)) & ((1ull << n) - 1ull));
  states[idx] = s;
  if (w_hard != nullptr) w_hard[idx] = cb[s];
}

}  // namespace

int launch_pack_code(int n, int k, const int32_t* states, int64_t B, int64_t L, uint32_t* code,
                     void* stream) {
  const long long W = code_words(n, k, L);
  const long long total = B * W;
  if (total <= 0) return 0;
  hipLaunchKernelGGL(k_pack_code, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), reinterpret_cast<const int*>(states),
                     (long long)B, (long long)L, n, k, W, reinterpret_cast<unsigned*>(code));
  return (int)hipGetLastError();
}

int launch_unpack_code(int n, int k, const uint32_t* code, int64_t B, int64_t L,
                       const float* codebook, int32_t* states, float* w_hard, void* stream) {
  const long long W = code_words(n, k, L);
  const long long total = B * L;
  if (total <= 0) return 0;
  hipLaunchKernelGGL(k_unpack_code, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), reinterpret_cast<const unsigned*>(code),
                     (long long)B, (long long)L, n, k, W, codebook, reinterpret_cast<int*>(states),
                     w_hard);
  return (int)hipGetLastError();
}

}  // namespace bcjr

// Compile-time geometry of the bitshift-trellis kernels, shared by the host layer and the
// kernels so that both agree on every size.
//
// Bitshift trellis with S = 2^n states and K = 2^k branches: s' = ((s << k) | b) & (S - 1).
// The predecessors of s' are (s' >> k) + a*M (a < K, M = S/K), so the K states s' = K*j + b
// (one "butterfly" j) share the same K predecessors j + a*M. Grouping K butterflies whose
// predecessor sets share their own predecessor messages gives K x K blocks of states,
//     s(x, r, a) = K*x + r + a*M,   x < NG = S/K^2,  r, a < K,
// for which the forward message of butterfly K*x + r is an LSE over a (a row of the block)
// and the backward message of butterfly x + a*NG is an LSE over r (a column of the block).
// One lane owns G such blocks; LPS lanes cover one chain.
#pragma once

namespace bcjr {

constexpr int kMaxLanesPerChain = 1024;

// Kernels are built for k in {1, 2, 3} and 2k <= n <= 16, except where the two backward
// messages of one chain (2 * S/K floats, single-buffered) would not fit the 160 KiB of LDS.
constexpr bool geom_supported(int n, int k) {
  return k >= 1 && k <= 3 && n >= 2 * k && n <= 16 && 2LL * ((1LL << n) >> k) * 4 <= 160 * 1024;
}
constexpr int geom_ng(int n, int k) { return 1 << (n - 2 * k); }
constexpr int geom_lps(int n, int k) {
  return geom_ng(n, k) < kMaxLanesPerChain ? geom_ng(n, k) : kMaxLanesPerChain;
}
constexpr int geom_g(int n, int k) { return geom_ng(n, k) / geom_lps(n, k); }
constexpr int geom_spb(int n, int k) { return geom_lps(n, k) < 64 ? 64 / geom_lps(n, k) : 1; }
constexpr int geom_block(int n, int k) { return geom_lps(n, k) < 64 ? 64 : geom_lps(n, k); }
// Blocks are persistent: each loops over chain units; about 16 waves per CU on 256 CUs.
constexpr long long geom_max_slots(int n, int k) {
  return (256LL * 16 * 64) / geom_block(n, k);
}

}  // namespace bcjr

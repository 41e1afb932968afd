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

// kFwd / kBwd: forward and backward with fp32 messages; kFwdP / kBwdP: the same kernels with
// fp64 messages (twice the message registers, so fewer states per lane); kVit: Viterbi;
// kFwdS / kBwdS: the fp32 kernels over the segments of the segmented (parallel-in-L) path, which
// has few chains in flight, so it spreads each over more lanes.
enum Kind { kFwd = 0, kBwd = 1, kVit = 2, kFwdP = 3, kBwdP = 4, kFwdS = 5, kBwdS = 6 };

constexpr int kMaxLanesPerChain = 1024;

// States per lane each kernel aims for (more states per lane: fewer lanes per chain, cheaper
// per-step exchanges and reductions, more registers). Measured on MI355X at S = 4096.
constexpr int geom_target_states(int kind) {
  return kind == kFwd ? 64 : kind == kBwd ? 32 : kind == kFwdP ? 32 : 16;  // kBwdP, kVit, kFwdS, kBwdS: 16
}

// Kernels are built for k in {1, 2, 3} and 2k <= n <= 16, except where the two backward
// messages of one chain (2 * S/K floats, single-buffered) would not fit the 160 KiB of LDS.
constexpr bool geom_supported(int n, int k) {
  return k >= 1 && k <= 3 && n >= 2 * k && n <= 16 && 2LL * ((1LL << n) >> k) * 4 <= 160 * 1024;
}
constexpr int geom_ng(int n, int k) { return 1 << (n - 2 * k); }
constexpr int geom_cmin(int a, int b) { return a < b ? a : b; }
constexpr int geom_cmax(int a, int b) { return a > b ? a : b; }
// blocks per lane: the target (at least 1, at most NG), raised if needed to keep LPS <= 1024
constexpr int geom_g(int n, int k, int kind) {
  return geom_cmax(geom_cmin(geom_cmax(geom_target_states(kind) >> (2 * k), 1), geom_ng(n, k)),
                   geom_ng(n, k) / kMaxLanesPerChain);
}
constexpr int geom_lps(int n, int k, int kind) { return geom_ng(n, k) / geom_g(n, k, kind); }
constexpr int geom_spb(int n, int k, int kind) {
  return geom_lps(n, k, kind) < 64 ? 64 / geom_lps(n, k, kind) : 1;
}
constexpr int geom_block(int n, int k, int kind) {
  return geom_lps(n, k, kind) < 64 ? 64 : geom_lps(n, k, kind);
}
// Batches too small to fill the device in the target geometry: the fp32-message forward and
// backward of whole chains then take the segment kinds' geometry (16 states per lane: 4x the
// forward's lanes per chain, 2x the backward's), which spreads each step's work over more
// waves. Chosen from (n, k, B) alone, so that the workspace query and the launch agree; built
// where the segment kernels are (k = 2, n <= 12) and only where it adds lanes. Thresholds, in
// waves of the target geometry on the 1024 SIMDs, measured on MI355X (L = 256, n = 6..12):
// below them the spread geometry was up to 2.5x faster, above them up to 19% slower.
constexpr long long kSpreadFwdBelowWaves = 2048, kSpreadBwdBelowWaves = 1024;
constexpr bool geom_spread(int n, int k, long long B, int kind) {
  return (kind == kFwd || kind == kBwd) && k == 2 && n <= 12 &&
         geom_g(n, k, kind == kFwd ? kFwdS : kBwdS) < geom_g(n, k, kind) &&
         (B + geom_spb(n, k, kind) - 1) / geom_spb(n, k, kind) * (geom_block(n, k, kind) / 64) <
             (kind == kFwd ? kSpreadFwdBelowWaves : kSpreadBwdBelowWaves);
}

// Below this temperature the forward-backward carries its messages in fp64 (their fp32
// rounding, which grows like 1/T, puts rare chains' gradients outside 1e-3 or close to it:
// randomized sweeps at unit-scale inputs, n = 5..12, L up to 256, found with fp32 messages
// 1.2e-3 at T = 0.012, 9.1e-4 at 0.025 and 8.4e-4 at 0.03 (near-ties between paths), and at most
// 3.1e-4 over 454 cases at 0.04, 2.8e-4 over 321 at 0.05, 1.4e-4 over 322 at 0.06; with fp64
// messages at most 6.4e-5 below the threshold). The fp64-message
// backward needs both of a chain's message buffers (fp64 + fp32 per butterfly, single-buffered)
// in LDS; shapes where they do not fit (S = 2^16 at k = 2) keep fp32 messages and form only the
// emission in fp64 below the threshold.
constexpr float kPreciseBelowT = 0.05f;
// Lowest temperature each state size meets the tolerances at; the soft entry points refuse lower
// ones (the Viterbi decoder is the T -> 0 limit). Exponentials, posteriors and expectations are
// fp32 on every path, and near-ties between paths amplify their rounding in the gradient like 1/T,
// more often the more states there are. Randomized sweeps at unit-scale inputs (L up to 256),
// worst grad_w: n <= 12 (fp64 messages) 1.7e-4 at T = 0.002..0.003, 2.1e-3 at 0.0005;
// n = 13..15 (fp64 messages) 1.0e-3 at 0.01, 7.2e-3 and 0.24 at 0.002, within 9.6e-5 over 76
// cases at 0.012; n = 16 (fp32 messages, fp64 emission) 5.5e-3 at 0.01, 4.0e-3 at 0.02, within
// 9.5e-5 over 71 cases at 0.025-0.03.
constexpr float geom_floor_t(int n, int k) {
  return (k == 2 && n <= 12) ? 0.002f : n <= 15 ? 0.015f : 0.03f;
}
constexpr bool geom_precise_fits(int n, int k) {
  return (long long)geom_spb(n, k, kBwdP) * ((1LL << n) >> k) * 12 <= 150 * 1024;
}
// Blocks are persistent: each loops over chain units. Workspace slots cover the largest
// resident grid on a 256-CU device at 8 waves per SIMD (32 per CU); a launch uses
// min(slots, resident blocks) of them.
constexpr long long geom_max_slots(int n, int k, int kind) {
  return (256LL * 32 * 64) / geom_block(n, k, kind);
}

static_assert(geom_g(12, 2, kFwd) == 4 && geom_lps(12, 2, kFwd) == 64, "S=4096 forward geometry");
static_assert(geom_g(12, 2, kBwd) == 2 && geom_lps(12, 2, kBwd) == 128, "S=4096 backward geometry");
static_assert(geom_g(16, 2, kBwd) == 4 && geom_lps(16, 2, kBwd) == 1024, "S=65536 geometry");
static_assert(geom_g(4, 2, kFwd) == 1 && geom_lps(4, 2, kFwd) == 1, "S=16 geometry");
static_assert(geom_g(8, 2, kBwd) == 2 && geom_lps(8, 2, kBwd) == 8, "S=256 geometry");
static_assert(geom_g(8, 2, kFwdS) == 1 && geom_lps(8, 2, kBwdS) == 16, "S=256 segment geometry");
static_assert(geom_precise_fits(15, 2) && !geom_precise_fits(16, 2), "fp64 messages up to S=2^15");
static_assert(geom_spread(8, 2, 4096, kFwd) && geom_spread(8, 2, 4096, kBwd) &&
              !geom_spread(12, 2, 65536, kFwd) && !geom_spread(12, 2, 65536, kBwd) &&
              !geom_spread(4, 2, 16, kFwd) && !geom_spread(16, 2, 1, kBwd), "spread geometry rule");

}  // namespace bcjr

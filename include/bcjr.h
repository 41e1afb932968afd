/*
 * bcjr.h -- C ABI of the MI355X (gfx950) BCJR soft trellis decoder.
 *
 * Method: "BCJR-QAT: A Differentiable Relaxation of Trellis-Coded Weight Quantization"
 * (V. Iyengar, arXiv 2605.10655). The paper's abstract (gptget.net/papers/2605.10655,
 * "Abstract") replaces the non-differentiable Viterbi argmax of trellis-coded weight
 * quantisation by the BCJR forward-backward sum-product recursion at temperature T; the soft
 * codeword is the Boltzmann expectation over trellis paths, exactly differentiable, equal to
 * the hard code as T -> 0, and computed like the transfer matrix of a 1D Ising-like chain.
 * The gist.science technical summary ("Core mechanism") writes the soft codeword as
 *   w_hat_t(T) = <c(s_t)>_{p_T} = sum_s c(s) p_T(s_t = s | w),
 * and ("Key technical innovations") states that the O(L*S^2) forward-backward gives exact
 * gradients through the trellis, fused into one launch at fp32 parity.
 *
 * Readings used where the pages are silent (the pages give neither the energy nor the
 * trellis shape):
 *   - path energy E = sum_t (w_t - c(s_t))^2, path weight exp(-E/T), natural-log log Z;
 *   - bitshift trellis: S = 2^n states, K = 2^k branches, s' = ((s << k) | b) & (S - 1),
 *     free start and free end state, one weight per step;
 *   - dense trellis: every state may follow every state; theta(s, s') is a transition
 *     log-potential that enters the energy as -theta, so the edge weight is exp(theta/T).
 *
 * Conventions shared by every entry point
 *   - Pointers marked DEVICE are device (HBM) pointers; arrays are row-major, contiguous,
 *     fp32 unless stated. "B, L" are the number of chains and the weights per chain.
 *   - The caller owns every buffer. The library allocates no device memory and keeps no
 *     mutable global state, except the fixed scratch array of bcjr_forward_noalloc (below). Workspaces (ws) must be 16-byte aligned (BCJR_E_WORKSPACE
 *     otherwise); their contents on entry are irrelevant and on return unspecified.
 *   - All arguments are validated on the host before anything is enqueued. On any error
 *     nothing is enqueued and no output buffer is touched.
 *   - Calls are asynchronous on the given stream (NULL = the default stream) and never
 *     synchronise. A launch failure is reported as BCJR_E_DEVICE by the call that sees it.
 *   - Inputs are not checked for NaN or Inf; non-finite values propagate. A NaN or +-Inf in
 *     one chain's weights makes that chain's w_hat, log_z and grad_w NaN, and the gradients
 *     that sum over chains (the codebook's and theta's) NaN; every other chain's w_hat, log_z,
 *     grad_w and decoded path are bitwise unchanged (chains are independent). A NaN or Inf in
 *     the codebook or theta makes every output of the call NaN. The Viterbi decoder is
 *     IEEE-exact.
 *   - Results are bitwise deterministic for a given device, input and argument set.
 *   - The library is thread safe (no shared mutable state); use one stream per thread.
 */
#ifndef BCJR_H_
#define BCJR_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* bcjr_stream_t; /* a hipStream_t */

typedef enum {
  BCJR_OK = 0,
  BCJR_E_ARG = 1,         /* null required pointer, T <= 0 or not finite, bad flag        */
  BCJR_E_SHAPE = 2,       /* n outside [1,16], k outside [1,n], B < 0, L < 1, S mismatch   */
  BCJR_E_WORKSPACE = 3,   /* ws_bytes smaller than the matching *_workspace_bytes query    */
  BCJR_E_DEVICE = 4,      /* a HIP call or kernel launch failed                            */
  BCJR_E_UNSUPPORTED = 5  /* valid shape with no kernel built for it (see bcjr_supported)  */
} bcjr_status;

/* Bitshift trellis (the pages do not give the trellis shape; this is the reading above). */
typedef struct {
  int32_t state_bits;       /* n in [1,16]; S = 1 << n states                              */
  int32_t bits_per_step;    /* k in [1,n];  K = 1 << k; successor s' = ((s<<k)|b) & (S-1)  */
  int32_t weights_per_step; /* V; must be 1 (else BCJR_E_UNSUPPORTED)                      */
  const float* codebook;    /* DEVICE [S]: codeword c(s) emitted in state s                 */
} bcjr_trellis;

/* Query: 1 if a kernel exists for this (n, k, V), else 0. Host only. */
int bcjr_supported(const bcjr_trellis* tr);

/* Bytes of the forward -> backward context: the forward's per-chain log2 Z (double [B], padded
 * to a multiple of 32), which the backward uses to normalise the posteriors, and its soft
 * codeword (fp32 [B,L]), on which the backward centres its conditional expectations. Returns 0
 * for an invalid shape. Host only, needs no device. */
size_t bcjr_saved_bytes(const bcjr_trellis* tr, int64_t B, int64_t L);

/* Bytes of device workspace for a call: which = 0 forward, 1 backward, 2 viterbi, 3 forward
 * with checkpointed history, 4 backward with checkpointed history.
 * Returns 0 for an invalid shape or flag. Host only, needs no device. The workspace holds
 * per-slot message histories (the alpha-side messages of one sweep, read back by the
 * sweep in the other direction; a slot is one chain, or a few narrow chains, in flight) and,
 * for the backward, per-slot codebook-gradient partials. The full history keeps every step (L
 * entries per slot); the checkpointed one keeps every C-th step, C = ceil(sqrt(L)), and the
 * reverse sweep recomputes one segment of C steps at a time (about 2 sqrt(L) entries per slot,
 * for one more forward recursion of work; results are bitwise identical). bcjr_forward and
 * bcjr_backward use the full history when ws_bytes covers it, else the checkpointed one. */
size_t bcjr_workspace_bytes(const bcjr_trellis* tr, int64_t B, int64_t L, int which);

/*
 * Forward: soft codeword and log partition function of every chain.
 *   w_hat[b,t] = sum_s c(s) p_T(s_t = s | w_b)      (technical summary, "Core mechanism")
 *   log_z[b]   = log sum_paths exp(-E(path)/T)      (abstract: Boltzmann distribution over
 *                                                     trellis paths, transfer-matrix form)
 * w      DEVICE [B,L]  weight preimage, read only
 * T      temperature, finite and > 0
 * w_hat  DEVICE [B,L]  written
 * log_z  DEVICE [B]    written
 * saved  DEVICE, bcjr_saved_bytes() bytes, written; pass it unchanged to bcjr_backward
 * saved  DEVICE, 16-byte aligned (BCJR_E_ARG otherwise)
 * ws     DEVICE, ws_bytes >= bcjr_workspace_bytes(tr, B, L, 3) (checkpointed history) or
 *        >= bcjr_workspace_bytes(tr, B, L, 0) (full history); contents are scratch
 * B = 0 is valid and enqueues nothing. B * L may not exceed 2^40 (BCJR_E_SHAPE).
 * Temperature and precision: below T = 0.05 the messages are carried in fp64 (their fp32
 * rounding grows like 1/T; at unit-scale inputs it put rare chains' gradients at 0.8-1.2e-3 for
 * T in [0.012, 0.03] and within 3.1e-4 from T = 0.04 on), from T = 0.05 on in fp32. The fp64
 * kernels exist for every state size whose backward message buffers fit the 160 KiB of LDS,
 * i.e. n <= 15 at k = 2. For n = 16 (S = 2^16) the messages stay fp32 and below T = 0.05 only
 * the emission -(w - c)^2 / T and its sum with the message are formed in fp64 (w - c exactly),
 * Every state size meets the tolerances down to a floor (exponentials, posteriors and
 * expectations are fp32 on every path, and near-tied paths amplify their rounding like 1/T,
 * more often the more states there are): T = 0.002 for n <= 12, 0.015 for n = 13..15 and 0.03
 * for n = 16, measured at w and c of unit scale (inputs of scale lam behave like unit-scale ones
 * at T / lam^2). Below its floor the soft entry points (bcjr_forward, bcjr_backward,
 * bcjr_forward_scan, bcjr_backward_scan) return BCJR_E_UNSUPPORTED before enqueueing anything;
 * viterbi_decode is the T -> 0 limit.
 */
bcjr_status bcjr_forward(const bcjr_trellis* tr, const float* w, int64_t B, int64_t L, float T,
                         float* w_hat, float* log_z, void* saved, void* ws, size_t ws_bytes,
                         bcjr_stream_t stream);

/* ---- Forward that allocates nothing -------------------------------------------------------------
 * For callers that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. bcjr_forward (same kernels, same validation, bitwise
 * the same outputs) with its workspace taken from a fixed device array of the library,
 * BCJR_NOALLOC_SCRATCH_BYTES long, which the runtime places on every device the library runs on
 * when it loads the library's code and keeps until the process ends. The call makes no
 * allocation, free or allocating library call.
 *   - Shapes whose checkpointed history, bcjr_workspace_bytes(tr, B, L, 3), exceeds
 *     BCJR_NOALLOC_SCRATCH_BYTES are refused with BCJR_E_WORKSPACE before any device call (at
 *     S = 4096, L = 256 that admits up to about 1000 chains; the full history is used where it
 *     fits, else the checkpointed one).
 *   - The first call on a device (any arguments, B = 0 included) looks up the array's device
 *     address with that device current (BCJR_E_DEVICE if that fails); make it before any graph
 *     capture. The stream must belong to the current device, as for every call.
 *   - Every call on a device shares that device's array, and the array keeps the last call's
 *     contents (nothing in it needs to start at zero). Calls whose execution overlaps on one
 *     device (other streams, other threads) race on it: serialise them.
 * Other arguments and errors as bcjr_forward.
 */
#define BCJR_NOALLOC_SCRATCH_BYTES ((size_t)256 << 20)
bcjr_status bcjr_forward_noalloc(const bcjr_trellis* tr, const float* w, int64_t B, int64_t L,
                                 float T, float* w_hat, float* log_z, void* saved,
                                 bcjr_stream_t stream);

/*
 * Backward: exact reverse-mode gradient of  F = sum_{b,t} g[b,t] w_hat[b,t] + sum_b h[b] log_z[b]
 * ("exactly differentiable", abstract; "exact gradients", technical summary, "Key technical
 * innovations") with respect to the weights and the codebook. T is not differentiated.
 * w, T, tr   exactly as given to the forward that wrote `saved`
 * saved      DEVICE, read only
 * grad_w_hat DEVICE [B,L] upstream gradient g
 * grad_log_z DEVICE [B] upstream gradient h, or NULL for h = 0
 * grad_w     DEVICE [B,L] written
 * grad_codebook DEVICE [S] written (overwritten, summed over all B chains, fixed-order sum)
 * ws         DEVICE, ws_bytes >= bcjr_workspace_bytes(tr, B, L, 4) (checkpointed history) or
 *            >= bcjr_workspace_bytes(tr, B, L, 1) (full history)
 * Errors as bcjr_forward, including BCJR_E_UNSUPPORTED for S = 2^16 below T = 0.004 (with the
 * fp32 emission the gradient erred by up to 0.51 at T = 0.002 on an input with nearly tied
 * paths; with the fp64 emission by 2.6e-4 there, and by 1.3e-3 on another input).
 */
bcjr_status bcjr_backward(const bcjr_trellis* tr, const float* w, int64_t B, int64_t L, float T,
                          const void* saved, const float* grad_w_hat, const float* grad_log_z,
                          float* grad_w, float* grad_codebook, void* ws, size_t ws_bytes,
                          bcjr_stream_t stream);

/*
 * Viterbi decode, the T -> 0 limit ("recovering the hard QTIP code as T -> 0", abstract).
 * fp32 min-sum with a fixed op order: e = fl(d*d), d = fl(w_t - c(s)); m_1 = e_1;
 * m_t(s') = fl(min_a m_{t-1}(p_a(s')) + e_t(s')) where p_a(s') = (s' >> k) | (a << (n-k)) and
 * the lowest a wins an exact tie; the final state is the lowest index attaining min m_L.
 * states DEVICE int32 [B,L] written: the decoded state path
 * w_hard DEVICE [B,L] written with c(states), or NULL
 * ws     DEVICE, ws_bytes >= bcjr_workspace_bytes(tr, B, L, 2) (backpointers)
 */
bcjr_status viterbi_decode(const bcjr_trellis* tr, const float* w, int64_t B, int64_t L,
                           int32_t* states, float* w_hard, void* ws, size_t ws_bytes,
                           bcjr_stream_t stream);

/* ---- Segmented forward for few, long chains (parallel in L) -----------------------------------
 * The same w_hat and log_z as bcjr_forward (up to rounding), computed with parallelism along
 * the chain. The abstract identifies the forward-backward with the transfer-matrix computation
 * of a 1D Ising-like chain; transfer matrices compose associatively, so a chain can be cut
 * into segments whose transfer matrices are formed independently and then combined. Here a
 * chain is cut into segments of seg_len steps (the last one shorter if seg_len does not divide
 * L); each segment's (S/K) x (S/K) log-semiring transfer matrix between butterfly messages is
 * computed from S/K one-hot starts, the boundary messages are scanned over the segments in
 * double precision, and every segment runs its forward-backward from its boundary messages.
 * Phase 1 costs S/K times the forward recursion's work, so this pays where chains are too few
 * to fill the device and L is long (e.g. one chain of 2^20 steps at S = 256: ~300x faster
 * than bcjr_forward; at S = 4096 it is not faster). Its backward is bcjr_backward_scan below.
 *
 * seg_len  segment length in steps, > 0, or 0 for the default, about sqrt(L) steps scaled by
 *          the boundary scan's cost per segment (which grows with (S/K)^2), at least 16;
 *          a value >= L runs the chain as one segment
 * Built for k = 2, n = 4..12 (BCJR_E_UNSUPPORTED otherwise). Errors as bcjr_forward, plus
 * BCJR_E_ARG for seg_len < 0.
 */
/* The segment length a call with these arguments uses (0 if the arguments are invalid). */
int64_t bcjr_scan_segment_length(const bcjr_trellis* tr, int64_t B, int64_t L, int64_t seg_len);
/* Workspace bytes for bcjr_forward_scan; no device needed; 0 if invalid or B == 0. Holds the
 * transfer matrices (B x segments x (S/K)^2 doubles), the boundary messages and the segment
 * kernels' per-slot histories. */
size_t bcjr_scan_workspace_bytes(const bcjr_trellis* tr, int64_t B, int64_t L, int64_t seg_len);
/*
 * w      DEVICE [B,L]  read only
 * w_hat  DEVICE [B,L]  written
 * log_z  DEVICE [B]    written
 * ws     DEVICE, ws_bytes >= bcjr_scan_workspace_bytes(tr, B, L, seg_len), 16-byte aligned
 */
bcjr_status bcjr_forward_scan(const bcjr_trellis* tr, const float* w, int64_t B, int64_t L,
                              float T, int64_t seg_len, float* w_hat, float* log_z, void* ws,
                              size_t ws_bytes, bcjr_stream_t stream);

/*
 * Segmented backward: the gradient of F = sum g * w_hat + sum h * log_z (as bcjr_backward,
 * "exactly differentiable", abstract) with parallelism along the chain. The centred conditional
 * expectations the gradient is built from (Phi forward, Psi backward) compose over a segment
 * through its moment matrix F(i, j) = E[sum over the segment of g_u (c(s_u) - w_hat_u) |
 * butterfly i at its start, j at its end]: phase 1 forms the transfer and moment rows from
 * S/K one-hot starts per segment, phase 2 scans messages and expectations over the segments,
 * phase 3 runs every segment's backward from its boundary values. Same shapes, defaults and
 * cost profile as bcjr_forward_scan.
 * w_hat      DEVICE [B,L] the soft codeword from bcjr_forward_scan (or bcjr_forward) with the
 *            same w, T and codebook, read only (it centres the expectations)
 * grad_w_hat DEVICE [B,L] upstream gradient g
 * grad_log_z DEVICE [B] upstream gradient h, or NULL for h = 0
 * grad_w     DEVICE [B,L] written
 * grad_codebook DEVICE [S] written (overwritten, summed over all chains; zero for B = 0)
 * ws         DEVICE, ws_bytes >= bcjr_scan_backward_workspace_bytes(tr, B, L, seg_len)
 * Any seg_len may be used (it need not equal the forward's).
 */
size_t bcjr_scan_backward_workspace_bytes(const bcjr_trellis* tr, int64_t B, int64_t L,
                                          int64_t seg_len);
bcjr_status bcjr_backward_scan(const bcjr_trellis* tr, const float* w, int64_t B, int64_t L,
                               float T, int64_t seg_len, const float* w_hat,
                               const float* grad_w_hat, const float* grad_log_z, float* grad_w,
                               float* grad_codebook, void* ws, size_t ws_bytes,
                               bcjr_stream_t stream);

/* ---- Hard-code export (bitshift trellis) ------------------------------------------------------
 * The zero-temperature end of the method: the hard code that the abstract says is recovered as
 * T -> 0. A state path of the bitshift trellis is fixed by its first state and the k bits each
 * step shifts in, s_t = ((s_{t-1} << k) | b_t) & (S-1), b_t = s_t mod K, so a chain's code is
 * the bit string s_0 (n bits, most significant first) followed by b_1 .. b_{L-1} (k bits each,
 * most significant first): n + k (L-1) bits in 32-bit words, the first bit in the most
 * significant position of word 0, the tail of the last word zero (the pages give no packing;
 * this is the reading). Every s_t is the n-bit window of the code starting at bit k t.
 */

/* 32-bit words per chain, ceil((n + k (L-1)) / 32); 0 for an invalid shape. Host only. */
int64_t bcjr_code_words(const bcjr_trellis* tr, int64_t L);

/*
 * Pack state paths into codes.
 * states DEVICE int32 [B,L], a path of the trellis (e.g. from viterbi_decode; a step whose state
 *        is not a successor of the previous one keeps only its low k bits)
 * code   DEVICE uint32 [B, bcjr_code_words(tr, L)] written
 * The codebook pointer of tr is not used. Errors: BCJR_E_SHAPE, BCJR_E_ARG (null pointer with
 * B > 0), BCJR_E_UNSUPPORTED (weights_per_step != 1). B = 0 enqueues nothing.
 */
bcjr_status bcjr_pack_code(const bcjr_trellis* tr, const int32_t* states, int64_t B, int64_t L,
                           uint32_t* code, bcjr_stream_t stream);

/*
 * Unpack codes into state paths and, optionally, the hard codeword c(s_t).
 * code   DEVICE uint32 [B, bcjr_code_words(tr, L)]
 * states DEVICE int32 [B,L] written
 * w_hard DEVICE [B,L] written with c(states), or NULL (then tr->codebook may be NULL)
 */
bcjr_status bcjr_unpack_code(const bcjr_trellis* tr, const uint32_t* code, int64_t B, int64_t L,
                             int32_t* states, float* w_hard, bcjr_stream_t stream);

/* ---- Dense (fully connected) trellis --------------------------------------------------------
 * Every state may follow every state; theta [S,S] (DEVICE, row-major, theta[s*S + s'] for the
 * transition s -> s') holds transition log-potentials. A path's weight is
 *   exp( ( sum_{t>=1} theta(s_{t-1}, s_t) - sum_t (w_t - c(s_t))^2 ) / T ),
 * free start and free end state. This is the transfer-matrix form of the method (abstract: the
 * computation is identical to the transfer matrix of a 1D Ising-like chain; technical summary,
 * "Key technical innovations": O(L*S^2) forward-backward with exact gradients through the
 * trellis parameters), run as rescaled linear-domain matrix products on the matrix cores.
 * Messages are fp32 in the linear domain, rescaled every step; a state whose relative weight
 * falls below the fp32 range (2^-126 of the step's best) is dropped. That limits the path to
 * moderate T: at theta, c and w of unit scale it meets the tolerances from T = 0.1 up (tested
 * to T = 5), while at T = 0.05 w_hat errs by 4e-3 and below T = 0.03 whole steps underflow.
 * Both dense entry points therefore return BCJR_E_UNSUPPORTED for T < 0.1. Inputs of scale
 * lam behave like unit-scale ones at T / lam^2 ((w, c, theta, T) -> (lam w, lam c, lam^2 theta,
 * lam^2 T) leaves the posteriors unchanged), so T >= 0.1 lam^2 is the range to use. The
 * bitshift entry points cover the near-hard regime.
 * Supported S: 32, 64, 128, 256 (bcjr_dense_supported). B >= 0, L >= 1.
 */

/* 1 if dense kernels exist for S states, else 0. Host only. */
int bcjr_dense_supported(int32_t S);

/* Bytes of the dense forward -> backward context: log2 Z per chain (double [B]), per-step
 * scalars (fp32 [B,L,4]) and the forward and backward message histories (fp32 [B,L,S] each).
 * 0 for an invalid or unsupported shape. Host only. The context must be 16-byte aligned. */
size_t bcjr_dense_saved_bytes(int32_t S, int64_t B, int64_t L);

/* Bytes of dense workspace: which = 0 forward (the transition matrix), 1 backward (adds three
 * [B,L,S] fp32 operand arrays of the theta gradient and fixed-size partial sums). 0 for an
 * invalid shape, an unsupported S, a bad flag or B = 0. Host only. */
size_t bcjr_dense_workspace_bytes(int32_t S, int64_t B, int64_t L, int which);

/*
 * Dense forward: soft codeword and log partition function, as bcjr_forward.
 * theta    DEVICE [S,S] read only;  codebook DEVICE [S];  w DEVICE [B,L]
 * w_hat    DEVICE [B,L] written;    log_z DEVICE [B] written
 * saved    DEVICE, bcjr_dense_saved_bytes() bytes, 16-byte aligned, written
 * ws       DEVICE, ws_bytes >= bcjr_dense_workspace_bytes(S, B, L, 0)
 * Errors: BCJR_E_SHAPE (S < 1, B < 0, L < 1, sizes beyond 64-bit offsets), BCJR_E_UNSUPPORTED
 * (no kernel for S), BCJR_E_ARG (null pointer with B > 0, misaligned saved, bad T),
 * BCJR_E_WORKSPACE. B = 0 enqueues nothing.
 */
bcjr_status bcjr_dense_forward(int32_t S, const float* theta, const float* codebook, const float* w,
                               int64_t B, int64_t L, float T, float* w_hat, float* log_z,
                               void* saved, void* ws, size_t ws_bytes, bcjr_stream_t stream);

/*
 * Dense backward: gradient of F = sum g w_hat + sum h log_z (as bcjr_backward) with respect to
 * w, the codebook and theta.
 * saved       DEVICE, written by bcjr_dense_forward with the same S, theta, codebook, w, B, L, T
 * grad_w_hat  DEVICE [B,L];  grad_log_z DEVICE [B] or NULL (h = 0)
 * grad_w      DEVICE [B,L] written
 * grad_codebook DEVICE [S] written, grad_theta DEVICE [S,S] written (both overwritten and summed
 *             over all B chains in a fixed order)
 * ws          DEVICE, ws_bytes >= bcjr_dense_workspace_bytes(S, B, L, 1)
 * B = 0 writes zeros to grad_codebook and grad_theta.
 */
bcjr_status bcjr_dense_backward(int32_t S, const float* theta, const float* codebook,
                                const float* w, int64_t B, int64_t L, float T, const void* saved,
                                const float* grad_w_hat, const float* grad_log_z, float* grad_w,
                                float* grad_codebook, float* grad_theta, void* ws, size_t ws_bytes,
                                bcjr_stream_t stream);

/* Text of a status code (static storage). */
const char* bcjr_status_string(bcjr_status s);

#ifdef __cplusplus
}
#endif
#endif /* BCJR_H_ */

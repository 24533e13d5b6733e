/*
 * nystrom.h -- C ABI of the MI355X (gfx950) Nyström self-attention forward.
 *
 * What is computed (per batch b and head h, all indices 0-based):
 *   Qt, Kt  segment means of Q and K over m contiguous blocks of l = n/m rows
 *           ("Nyströmformer: A Nyström-Based Algorithm for Approximating
 *           Self-Attention", sec. 3.4 "Landmark Selection: Segment-Means",
 *           Eq. 16, divisor read as l).  That section assumes m divides n
 *           and says padding provides it: otherwise the sequence counts as
 *           padded at its end with zero rows up to m * ceil(n/m), l is
 *           ceil(n/m), and the pad rows, which are not tokens, are masked
 *           out of B's keys and produce no output rows;
 *   F = softmax(Q Kt^T / sqrt(d)), A = softmax(Qt Kt^T / sqrt(d)),
 *   B = softmax(Qt K^T / sqrt(d)), all row-wise (same page, Eq. 13);
 *   Z = `iters` steps of Z <- Z (13I - AZ(15I - AZ(7I - AZ))) / 4 from
 *       Z0 = A^T / (||A||_1 ||A||_inf) (same page, "Moore-Penrose
 *       Pseudoinverse Computation", Lemma 1 and the initialisation);
 *   out = F (Z (B V)) + DConv(V) (same page, "Putting It Together", Eq. 17
 *       and the depthwise-convolution skip of Figure 4), where
 *       DConv(V)[i, c] = sum_t w[h, c, t] V[i + t - (k-1)/2, c], zero outside.
 * The n x n score matrix is never formed.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     never frees caller memory and keeps no tensor data between calls.  The
 *     forward entry points create no streams or events: every kernel runs on
 *     `stream`, in order.  Three per-device objects are created on first use
 *     and kept for the life of the process: by nystrom_attn_bwd (bf16,
 *     d = 32 or 64) a second stream and four events, which it forks from and
 *     joins back to `stream`; by nystrom_layer_fwd a rocBLAS handle; and,
 *     while nystrom_timing_enable is on, timing events.
 *   - Q, K, V, out: [batch][heads][n][d], contiguous, element type `dtype`
 *     (NYS_F32 = IEEE fp32, NYS_BF16 = bfloat16).  conv_w: fp32
 *     [heads][d][conv_k], contiguous, or NULL for no skip.
 *   - All arithmetic accumulates in fp32; the output is rounded to `dtype`
 *     (round-to-nearest-even for bf16).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream).  Arguments are validated on the host before anything is
 *     enqueued; an invalid call returns a negative code and launches nothing.
 *   - No exception crosses the ABI.  NaN/Inf inputs are not checked and
 *     propagate.
 */
#ifndef NYSTROM_H
#define NYSTROM_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of Q, K, V and out. */
typedef enum { NYS_F32 = 0, NYS_BF16 = 1 } nys_dtype;

/* Return codes. */
enum {
  NYS_OK = 0,
  NYS_EINVAL = -1,       /* bad argument: NULL tensor, size < 1, m > n,
                            iters < 0, even or non-positive conv_k with a filter,
                            unknown dtype */
  NYS_EUNSUPPORTED = -2, /* valid but outside what the kernels handle:
                            d not in {16, 32, 64, 128}, m > 256, n > 2^24,
                            n * d >= 2^29 (one head's rows as fp32 reach
                            2 GiB: the kernels use 32-bit byte offsets
                            within a head), batch * heads > 65535 */
  NYS_EWORKSPACE = -3,   /* caller workspace smaller than nystrom_attn_workspace_bytes() */
  NYS_EHIP = -4,         /* a HIP runtime call or launch failed */
  NYS_ENOTIMPL = -5
};

/* Which intermediate to locate in the workspace (see nystrom_attn_workspace_offset). */
enum {
  NYS_WS_QT = 0, /* fp32 [batch*heads][m][d]   segment means of Q            */
  NYS_WS_KT = 1, /* fp32 [batch*heads][m][d]   segment means of K            */
  NYS_WS_A = 2,  /* fp32 [batch*heads][m][m]   softmax(Qt Kt^T / sqrt d)     */
  NYS_WS_Z = 3,  /* fp32 [batch*heads][m][m]   pseudoinverse after `iters`   */
  NYS_WS_BV = 4, /* fp32 [batch*heads][m][d]   softmax(Qt K^T / sqrt d) V    */
  NYS_WS_W = 5,  /* fp32 [batch*heads][m][d]   Z (B V)                       */
  NYS_WS_COUNT = 6
};

/* Bytes of device workspace nystrom_attn_fwd needs for this shape (the same
 * for both dtypes), or 0 if the shape is invalid or unsupported. */
size_t nystrom_attn_workspace_bytes(int batch, int heads, int n, int d, int m);

/* Byte offset of intermediate `which` (NYS_WS_*) inside the workspace, or -1
 * for an invalid shape or `which`.  After a completed nystrom_attn_fwd call
 * the region holds that call's values, laid out as documented above. */
long long nystrom_attn_workspace_offset(int which, int batch, int heads, int n, int d, int m);

/* Nyström self-attention forward (the computation described at the top).
 *   Q, K, V     inputs, [batch][heads][n][d] of `dtype`
 *   conv_w      fp32 [heads][d][conv_k] depthwise filters, or NULL (no skip;
 *               conv_k is then ignored)
 *   n           sequence length, n >= m (padded as described at the top
 *               when m does not divide it)
 *   d           head dimension, one of 16, 32, 64, 128
 *   m           number of landmarks, 1 <= m <= min(n, 256)
 *   heads       heads per batch entry
 *   iters       pseudoinverse iterations (>= 0; 0 returns the start Z0)
 *   out         output, [batch][heads][n][d] of `dtype`; must not alias inputs
 *   batch       batch size
 *   conv_k      odd filter length when conv_w != NULL
 *   dtype       NYS_F32 or NYS_BF16 (Q, K, V and out share it)
 *   workspace   device buffer of at least nystrom_attn_workspace_bytes(), or
 *               NULL: the call then allocates and frees one in stream order
 *               (hipMallocAsync / hipFreeAsync on `stream`)
 *   workspace_bytes  size of `workspace` (ignored when it is NULL)
 *   stream      hipStream_t the work is ordered on; NULL = default stream
 * Returns NYS_OK, or a negative code (nothing was launched when validation
 * fails). */
int nystrom_attn_fwd(const void* Q, const void* K, const void* V, const float* conv_w,
                     int n, int d, int m, int heads, int iters, void* out,
                     int batch, int conv_k, int dtype,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the built-in scratch of nystrom_attn_fwd_noalloc (per GPU). */
#define NYS_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/* nystrom_attn_fwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, kernels and results, bit for bit, with
 * the workspace taken from a scratch array of NYS_NOALLOC_SCRATCH_BYTES that
 * the library holds on every GPU it runs on until the process ends.  The call
 * never allocates or frees device memory.
 *   Arguments as for nystrom_attn_fwd, without the workspace.
 * Returns NYS_EWORKSPACE when the shape's workspace
 * (nystrom_attn_workspace_bytes) exceeds NYS_NOALLOC_SCRATCH_BYTES (every
 * workload up to batch 1 x 16 heads, n = 32768, d = 128, m = 256 fits);
 * NYS_EHIP if the scratch's device address cannot be looked up; otherwise as
 * nystrom_attn_fwd.  All calls on one GPU share that GPU's scratch: calls
 * that overlap on one GPU (other streams, other host threads) race and must
 * be serialised by the caller.  The scratch keeps the last call's
 * intermediates (laid out as nystrom_attn_workspace_offset describes) until
 * the next call overwrites them. */
int nystrom_attn_fwd_noalloc(const void* Q, const void* K, const void* V, const float* conv_w,
                             int n, int d, int m, int heads, int iters, void* out,
                             int batch, int conv_k, int dtype, void* stream);

/* Nyström self-attention forward over a batch of right-padded sequences, the
 * key-padding mask given as one length per batch entry.  The pages leave
 * masking out ("Approximating self-attention in linear time and memory via
 * the Nyström method", "How is Nyströmformer implemented?"); the reading
 * taken is that padding tokens are not part of a sequence: batch entry b is
 * what nystrom_attn_fwd computes for its first L_b rows alone, padded with
 * zero rows to a multiple of m as described at the top when m does not
 * divide L_b.  A sequence shorter than m is padded to m rows the same way
 * (l = 1): its landmarks are its L_b rows followed by zero vectors, and B
 * spans its L_b keys.
 *   lengths     DEVICE pointer to int32 [batch], L_b = tokens of entry b;
 *               read on the device only, each clamped to [0, n] there (the
 *               host cannot check them without a synchronisation).  NULL =
 *               every entry has n tokens, the same as nystrom_attn_fwd.
 * Rows L_b .. n-1 of Q, K and V are never read (they may hold anything,
 * NaN included); rows L_b .. n-1 of out are written as zero; the workspace
 * intermediates of entry b are those of its own sequence.  An entry with
 * L_b = 0 has an all-zero output; its B V and W are zero and its other
 * intermediates are those of zero landmarks.  All other arguments, the
 * workspace size, the return codes and the stream behaviour are those of
 * nystrom_attn_fwd. */
int nystrom_attn_fwd_masked(const void* Q, const void* K, const void* V, const float* conv_w,
                            int n, int d, int m, int heads, int iters, void* out,
                            int batch, int conv_k, int dtype, const int* lengths,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Backward pass: gradients of nystrom_attn_fwd's output with respect to Q,
 * K, V and the skip filters, given dO = dL/d(out).  The pages train through
 * the fixed number of pseudoinverse steps ("Nyströmformer: ...", sec. 3.4,
 * "Moore-Penrose Pseudoinverse Computation"); this is the exact derivative of
 * the forward computation described at the top, taken through every step
 * (segment means with their padding, the three softmaxes, the `iters`
 * Lemma-1 steps and the Pan-Schreiber start, W = Z (B V), the skip).  The
 * derivative of each maximum in the start is taken at its first maximiser.
 * The landmark side of the forward pass is recomputed inside the call.
 *   Q, K, V, conv_w, n, d, m, heads, iters, batch, conv_k, dtype: as for
 *               nystrom_attn_fwd (the same values as the forward call)
 *   dO          [batch][heads][n][d] of `dtype`, the upstream gradient
 *   dQ, dK, dV  outputs, [batch][heads][n][d] of `dtype`, written (not
 *               accumulated); must not alias any input
 *   dconv_w     fp32 [heads][d][conv_k], written with the filter gradient
 *               summed over the batch, or NULL to skip it; ignored when
 *               conv_w is NULL
 *   workspace   device buffer of at least nystrom_attn_bwd_workspace_bytes(),
 *               or NULL (allocated and freed in stream order)
 * Supported: m <= 64 and conv_k <= 33 (NYS_EUNSUPPORTED otherwise), every d
 * and n of the forward.  Return codes and stream behaviour as for
 * nystrom_attn_fwd.  For bf16 with d = 32 or 64 part of the work runs on a
 * second stream that the library keeps per device, forked from and joined
 * back to `stream` by events: the call stays ordered with the caller's other
 * work on `stream`, and can be captured into a graph with it. */
size_t nystrom_attn_bwd_workspace_bytes(int batch, int heads, int n, int d, int m, int iters, int conv_k);
int nystrom_attn_bwd(const void* Q, const void* K, const void* V, const float* conv_w, const void* dO,
                     int n, int d, int m, int heads, int iters,
                     void* dQ, void* dK, void* dV, float* dconv_w,
                     int batch, int conv_k, int dtype,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Backward pass under a key-padding mask: the gradients of
 * nystrom_attn_fwd_masked's output (the method on the first L_b rows of
 * each batch entry, the pages leaving masking to the implementation), so
 * that entry b's gradients are those of its own sequence.
 *   lengths     DEVICE pointer to int32 [batch], as for
 *               nystrom_attn_fwd_masked (each L_b clamped to [0, n] on the
 *               device); NULL = the same as nystrom_attn_bwd.
 * Rows L_b .. n-1 of Q, K, V and dO are never read (they may hold anything,
 * NaN included); rows L_b .. n-1 of dQ, dK and dV are written as zero; the
 * filter gradient sums over the real rows of every entry (an empty entry
 * adds nothing).  All other arguments, the workspace size
 * (nystrom_attn_bwd_workspace_bytes), the supported shapes, the return
 * codes and the stream behaviour are those of nystrom_attn_bwd. */
int nystrom_attn_bwd_masked(const void* Q, const void* K, const void* V, const float* conv_w, const void* dO,
                            int n, int d, int m, int heads, int iters,
                            void* dQ, void* dK, void* dV, float* dconv_w,
                            int batch, int conv_k, int dtype, const int* lengths,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Training pair: the forward pass that keeps its landmark-side state, and
 * the backward pass that starts from it instead of recomputing it (the same
 * method and results as nystrom_attn_fwd and nystrom_attn_bwd, bit for bit).
 *   nystrom_attn_fwd_save  arguments as for nystrom_attn_fwd; O is written to
 *                          `out`, and Q~, K~, A, Z, BV, W, the row statistics
 *                          of B~ and each Lemma-1 step (Z_k, X_k, T1_k, T2_k)
 *                          to `saved`
 *   nystrom_attn_bwd_saved arguments as for nystrom_attn_bwd, with `saved`
 *                          in place of the workspace
 *   saved        DEVICE buffer owned by the caller, not NULL (NYS_EINVAL):
 *                for nystrom_attn_bwd_saved at least
 *                nystrom_attn_bwd_workspace_bytes() (the state, then the
 *                backward's scratch); nystrom_attn_fwd_save writes only its
 *                first nystrom_attn_bwd_state_bytes() and needs no more
 *                (NYS_EWORKSPACE below that).  Between the two calls it must
 *                stay untouched, and the two calls must get the same Q, K, V,
 *                conv_w, shape, iters, conv_k and dtype; the backward may be
 *                called more than once on one saved forward.  The buffer's
 *                contents are the library's; its layout is not part of this
 *                interface.
 *   nystrom_attn_bwd_from_state  the same backward with the saved state and
 *                the scratch in separate buffers, so that a caller keeps only
 *                the state between the two calls: `state` as
 *                nystrom_attn_fwd_save left it (state_bytes >=
 *                nystrom_attn_bwd_state_bytes(), else NYS_EWORKSPACE; read
 *                only, not written), `scratch` a DEVICE buffer of at least
 *                nystrom_attn_bwd_workspace_bytes() - nystrom_attn_bwd_state_bytes()
 *                bytes (NYS_EWORKSPACE below that), or NULL for the library to
 *                allocate it on `stream`.  Results are bitwise those of
 *                nystrom_attn_bwd_saved.
 *   nystrom_attn_bwd_state_bytes  the state's size for the shape (either
 *                dtype); 0 for shapes the backward does not handle.
 * Supported shapes, return codes and stream behaviour as for
 * nystrom_attn_bwd. */
size_t nystrom_attn_bwd_state_bytes(int batch, int heads, int n, int d, int m, int iters, int conv_k);
int nystrom_attn_fwd_save(const void* Q, const void* K, const void* V, const float* conv_w,
                          int n, int d, int m, int heads, int iters, void* out,
                          int batch, int conv_k, int dtype,
                          void* saved, size_t saved_bytes, void* stream);
int nystrom_attn_bwd_saved(const void* Q, const void* K, const void* V, const float* conv_w, const void* dO,
                           int n, int d, int m, int heads, int iters,
                           void* dQ, void* dK, void* dV, float* dconv_w,
                           int batch, int conv_k, int dtype,
                           void* saved, size_t saved_bytes, void* stream);
int nystrom_attn_bwd_from_state(const void* Q, const void* K, const void* V, const float* conv_w, const void* dO,
                                int n, int d, int m, int heads, int iters,
                                void* dQ, void* dK, void* dV, float* dconv_w,
                                int batch, int conv_k, int dtype,
                                const void* state, size_t state_bytes,
                                void* scratch, size_t scratch_bytes, void* stream);

/* Full self-attention layer: the learned projections around the attention
 * ("Nyströmformer: ...", "Standard Self-Attention": Q = X W_Q, K = X W_K,
 * V = X W_V, with no bias; the attention-output projection the page mentions
 * with the skip connection).  With E = heads * d:
 *   QKV = X [W_Q | W_K | W_V], split into heads (head h owns columns
 *   h*d .. h*d+d-1 of each block), Nyström attention with the DConv skip per
 *   head as in nystrom_attn_fwd, heads concatenated, Y = O W_O.
 *   X           [batch][n][E] of `dtype`
 *   Wqkv        [E][3E] of `dtype`, row-major, column blocks W_Q | W_K | W_V
 *   Wo          [E][E] of `dtype`, row-major
 *   Y           [batch][n][E] of `dtype`, written; must not alias the inputs
 *   conv_w, n, d, m, heads, iters, batch, conv_k, dtype: as for nystrom_attn_fwd
 *   workspace   device buffer of at least nystrom_layer_workspace_bytes(), or
 *               NULL (allocated and freed in stream order)
 * The two projections run on rocBLAS (bf16 operands with fp32 accumulation
 * for NYS_BF16, fp32 otherwise); the library keeps one rocBLAS handle per
 * device for the life of the process, and calls on one device from several
 * host threads at once are not supported.  Return codes as for
 * nystrom_attn_fwd (a rocBLAS failure is NYS_EHIP); NYS_EUNSUPPORTED also for
 * 3 * batch * n * E >= 2^31. */
size_t nystrom_layer_workspace_bytes(int batch, int heads, int n, int d, int m, int dtype);
int nystrom_layer_fwd(const void* X, const void* Wqkv, const void* Wo, const float* conv_w,
                      int n, int d, int m, int heads, int iters, void* Y,
                      int batch, int conv_k, int dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Approximation-error diagnostic: for every (batch, head), the relative
 * Frobenius distance between the attention output of nystrom_attn_fwd (skip
 * excluded: it is exact) and exact softmax attention softmax(Q K^T / sqrt d) V
 * ("Nyströmformer: ...", Eq. 2; the page's closing discussion proposes
 * measuring the approximation error per example):
 *   err[b * heads + h] = ||O_nys - O_exact||_F / ||O_exact||_F
 *   Q, K, V, n, d, m, heads, iters, batch, dtype: as for nystrom_attn_fwd
 *   err         DEVICE pointer, fp32 [batch][heads], written
 *   workspace   at least nystrom_attn_error_workspace_bytes(), or NULL
 * The exact attention costs O(n^2 d) per head (matrix cores, online softmax,
 * no n x n matrix is stored).  O_nys is rounded to `dtype` as the forward's
 * output is; for NYS_BF16 the exact side uses bf16 operands with fp32
 * accumulation, so err carries an absolute uncertainty of about 2e-3.
 * Return codes and stream behaviour as for nystrom_attn_fwd. */
size_t nystrom_attn_error_workspace_bytes(int batch, int heads, int n, int d, int m, int dtype);
int nystrom_attn_error(const void* Q, const void* K, const void* V, int n, int d, int m, int heads,
                       int iters, float* err, int batch, int dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

/* Depthwise-convolution skip alone: out = DConv(V) with the filters and
 * padding described at the top ("Putting It Together", Figure 4's DConv path).
 *   V, out      [batch][heads][n][d] of `dtype` (out must not alias V)
 *   conv_w      fp32 [heads][d][conv_k], non-NULL; conv_k odd, >= 1
 *   d           one of 16, 32, 64, 128
 * Returns NYS_OK or a negative code. */
int nystrom_dconv_fwd(const void* V, const float* conv_w, int n, int d, int heads, int batch,
                      int conv_k, int dtype, void* out, void* stream);

/* Diagnostics: per-kernel timing.  While enabled, every kernel the library
 * launches is bracketed by two HIP events recorded on the launch's stream
 * (the library then holds those events between calls).  Returns the previous
 * setting.  Intended for profiling runs, not production calls. */
int nystrom_timing_enable(int on);

/* Waits for the recorded events and reports, per kernel name, the summed
 * milliseconds and the number of launches since the previous read; the
 * accumulators are cleared.  Fills at most `max_entries` entries; the name
 * pointers stay valid until the next read.  Returns the number of distinct
 * kernels (which may exceed max_entries). */
int nystrom_timing_read(int max_entries, const char** names, double* total_ms, long long* launches);

/* Static, human-readable text for a return code. */
const char* nystrom_strerror(int code);

/* ABI version of this header (major * 100 + minor). */
int nystrom_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NYSTROM_H */

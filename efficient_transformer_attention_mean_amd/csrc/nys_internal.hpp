// Host-side view of the workspace and the launch stages (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nys {

// Byte offsets of every region in the caller's workspace (256-byte aligned).
struct WsLayout {
  size_t qt, kt, a, z, bv, w;      // documented fp32 intermediates (NYS_WS_*)
  size_t z2, x, t, u, v;           // fp32 pseudoinverse scratch for m > 64 (X, T, U; Z ping-pong in v)
  size_t colp, rsum;               // fp32 m > 64: A's column sums per 16-row block, row sums
  size_t pacc, pmax, psum;         // fp32 split-n partials of softmax(Qt K^T) V
  size_t kt_hi, kt_lo;             // bf16 planes of Kt * log2(e)/sqrt(d), [bh][mpa][d]
  size_t qt_hi, qt_lo;             // bf16 planes of Qt, [bh][mpa][d] (rows m..mpa-1 zero)
  size_t wt_hi, wt_lo;             // bf16 planes of W^T, [bh][d][mpa], landmark order permuted
  size_t cwop;                     // matrix-core operands of the skip filters, [heads][d][4][9] x 16 B
  size_t sync;                     // uint32 [2][bh]: per-head arrival counters of the landmark pass
  size_t total;
  int nchunks, chunk;              // split-n: blocks per head, keys per block
  int mpa;                         // landmarks padded for the output stage: 32, 64, 128 or 256
};

// Returns false for shapes the kernels do not handle.
bool make_layout(int batch, int heads, int n, int d, int m, WsLayout* L);

// The same regions as device pointers.
struct Ws {
  float *Qt, *Kt, *A, *Z, *BV, *W;
  float *Z2, *X, *T, *U, *V;
  float *colp, *rsum;
  float *pacc, *pmax, *psum;
  uint16_t *kt_hi, *kt_lo, *qt_hi, *qt_lo, *wt_hi, *wt_lo;
  uint4* cwop;
  unsigned* sync;
  int nchunks, chunk, mpa;
};

Ws resolve(const WsLayout& L, char* base);

// Where an input tensor's rows are: head bh = b * heads + h starts
// b * bs + h * hs elements in, its rows ld elements apart.
struct InLayout {
  int ld;
  long long hs, bs;
};

struct Problem {
  const void* Q;
  const void* K;
  const void* V;
  const float* conv_w;
  void* out;
  int batch, heads, n, d, m, iters, conv_k;
  bool bf16;
  const int* lens = nullptr;  // device int32 [batch]: tokens per sequence (right padding), or none
  // Backward pass only: where the pseudoinverse kernels save each step
  // (Z_k, X_k, T1_k, T2_k as fp32 [zmp][zmp], per head and step), or none.
  float* zsave = nullptr;
  int zmp = 0;
  // out as [batch][n][heads][d] (the heads merged per token) instead of
  // [batch][heads][n][d].
  bool out_merged = false;
  // Q, K, V in a layout of their own (in_ld > 0: rows in_ld elements apart,
  // heads in_hs and batch entries in_bs apart), or [batch][heads][n][d].
  int in_ld = 0;
  long long in_hs = 0, in_bs = 0;
};

inline InLayout in_layout(const Problem& p) {
  if (p.in_ld > 0) return InLayout{p.in_ld, p.in_hs, p.in_bs};
  return InLayout{p.d, (long long)p.n * p.d, (long long)p.heads * p.n * p.d};
}

// Brackets the kernel launched inside its scope with events when per-kernel
// timing is on (nystrom_timing_enable); otherwise does nothing.
class KernelTimer {
 public:
  KernelTimer(const char* name, hipStream_t s);
  ~KernelTimer();
  KernelTimer(const KernelTimer&) = delete;
  KernelTimer& operator=(const KernelTimer&) = delete;

 private:
  const char* name_;
  hipStream_t s_;
  hipEvent_t start_ = nullptr;
};

// hipFuncSetAttribute(fn, MaxDynamicSharedMemorySize, bytes) once per
// (kernel, device); later calls return the first call's result.  Safe to call
// from several host threads.
hipError_t ensure_dynamic_smem(const void* fn, int bytes);

// Stages of the forward pass, in stream order.
hipError_t stage_segment_means(const Problem& p, const Ws& w, hipStream_t s);  // Qt, Kt, Kt planes
// Split-n partials of B V; with bf16 I/O and m <= 64 also A and Z (the
// pseudoinverse blocks run beside the key pass) and the skip-filter operands.
hipError_t stage_landmark_pass(const Problem& p, const Ws& w, hipStream_t s);
hipError_t stage_pinv(const Problem& p, const Ws& w, hipStream_t s);           // A, Z when not in the pass above
hipError_t stage_bv_finish(const Problem& p, const Ws& w, hipStream_t s);      // B V, W, W^T planes (needs Z)
// Split-n partial entries (pmax, psum, pacc) per head that the forward leaves:
// one per key chunk, or one per pair of chunks when the landmark pass merges them.
int forward_partials(const Problem& p, const Ws& w);
hipError_t stage_apply(const Problem& p, const Ws& w, hipStream_t s);          // out

hipError_t launch_forward(const Problem& p, const WsLayout& L, char* ws, hipStream_t s);
// Whether the forward reads Q, K, V in place from a layout of their own
// (Problem::in_ld) for this shape: d = 32 or 64, m <= 64, no skip or 3..33 taps.
bool apply_in_place(const Problem& p);

// Backward pass: the forward's workspace regions (recomputed landmark side)
// followed by its own (byte offsets, 256-byte aligned).
struct BwdLayout {
  WsLayout fwd;
  size_t pdw, pdkt;    // fp32 [bh][nq][m][d] query-side partials of dW and dKt
  size_t dw, dbv;      // fp32 [bh][m][d] dW, dBV
  size_t dkt, dqta;    // fp32 [bh][m][d] dKt (total), the landmark-side part of dQt
  size_t pdqt, dqt;    // fp32 [bh][nk][m][d] key-side partials of dQt; dQt (total)
  size_t pdwc;         // fp32 [bh][nk][d][conv_k] partials of the filter gradient
  size_t zs;           // fp32 [bh][iters][4][mp][mp] forward steps: Z_k, X_k, T1_k, T2_k
  size_t wflip;        // fp32 [heads][d][conv_k] skip filters with their taps reversed
  size_t state;        // bytes of the saved state: the forward's regions and zs come first
  size_t total;
  int qchunk, nq;      // query rows per block of the reduction pass, blocks per head
  int kchunk, nk;      // keys per block of the key pass, blocks per head
  int mp;              // landmarks padded to 32 or 64
};

// Returns false for shapes the backward kernels do not handle (m > 64,
// conv_k > 33, or anything the forward rejects).
bool make_bwd_layout(int batch, int heads, int n, int d, int m, int iters, int conv_k, bool bf16,
                     BwdLayout* L);

struct BwdProblem {
  Problem fwd;
  const void* dO;
  void *dQ, *dK, *dV;
  float* dconv_w;  // fp32 [heads][d][conv_k] or nullptr
};

// Where the regions of a backward workspace live: the saved state (offsets
// below L.state) from st, the scratch (offsets from L.state on) from scr,
// which may be a buffer of its own.  One buffer: st = ws, scr = ws + L.state.
struct BwdBuf {
  char* st;
  char* scr;
  size_t scr_off;
  char* state(size_t o) const { return st + o; }
  char* scratch(size_t o) const { return scr + (o - scr_off); }
};

// recompute = false: the forward's landmark-side state (and its saved
// pseudoinverse steps) is already in the state part, written by
// launch_forward_save.
hipError_t launch_backward(const BwdProblem& p, const BwdLayout& L, const BwdBuf& b, hipStream_t s,
                           bool recompute = true);
// The forward pass on the forward regions of a backward workspace, saving the
// pseudoinverse steps there too, so that launch_backward can skip its recompute.
hipError_t launch_forward_save(const Problem& p, const BwdLayout& L, char* ws, hipStream_t s);

// Full layer (projections around the attention): the forward's regions, then
// the fused QKV projection, read in place by the attention, and the attention
// output with the heads merged.
struct LayerLayout {
  WsLayout fwd;
  size_t qkv, o;  // the QKV product [batch*n][3E]; the attention output, heads merged
  size_t q, k, v;  // head-major copies of Q, K, V (shapes not read in place)
  size_t total;
};

bool make_layer_layout(int batch, int heads, int n, int d, int m, bool bf16, LayerLayout* L);

struct LayerProblem {
  Problem attn;      // shape, iters, filters, dtype (its Q, K, V, out are set inside)
  const void* X;     // [batch][n][heads*d]
  const void* Wqkv;  // [heads*d][3*heads*d], column blocks W_Q | W_K | W_V
  const void* Wo;    // [heads*d][heads*d]
  void* Y;           // [batch][n][heads*d]
};

hipError_t launch_layer(const LayerProblem& p, const LayerLayout& L, char* ws, hipStream_t s);

// Approximation-error diagnostic: the forward's regions, the attention
// output without the skip ([bh][n][d], I/O type) and per-block partial sums.
struct ErrLayout {
  WsLayout fwd;
  size_t onys, part;
  size_t total;
  int ntile;  // 64-query blocks per head
};

bool make_error_layout(int batch, int heads, int n, int d, int m, bool bf16, ErrLayout* L);
hipError_t launch_error(const Problem& p, const ErrLayout& L, char* ws, float* err, hipStream_t s);
// lens (device int32 [batch], or none): rows past each sequence's end read
// as zero and are written as zero.
hipError_t launch_dconv(const void* V, const float* conv_w, void* out, int batch, int heads, int n,
                        int d, int conv_k, bool bf16, hipStream_t s, const int* lens = nullptr);

}  // namespace nys

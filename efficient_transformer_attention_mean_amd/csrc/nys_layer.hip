// Nyström self-attention layer: the learned projections around the
// attention ("Nyströmformer: A Nyström-Based Algorithm for Approximating
// Self-Attention", paper deep-dive page, "Standard Self-Attention":
// Q = X W_Q, K = X W_K, V = X W_V; the attention-output projection the page
// mentions in its discussion of the skip connection).
//
// For a batch of sequences X [batch][n][E], E = heads * d:
//   QKV = X [W_Q | W_K | W_V]            one library GEMM, [batch*n][3E]
//   O = Nyström attention + DConv skip    the forward kernels, reading each
//                                         head's Q, K, V in place in QKV (rows
//                                         3E apart; d = 32 or 64, m <= 64, no
//                                         skip or 3..33 taps, else after a
//                                         head-major copy, k_split_heads) and
//                                         writing O with the heads
//                                         concatenated per token, [batch*n][E]
//   Y = concat_heads(O) W_O               one library GEMM
// The two projections are plain GEMMs and run on rocBLAS (bf16 operands with
// fp32 accumulation for bf16 I/O, fp32 otherwise).
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <mutex>

#include "nys_common.hpp"
#include "nys_internal.hpp"

namespace nys {

namespace {

// One rocBLAS handle per device, created on first use and kept for the life
// of the process (creating one per call costs milliseconds).
rocblas_handle handle_for_current_device(hipStream_t s) {
  static std::mutex mu;
  static rocblas_handle handles[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!handles[dev]) {
    rocblas_handle h = nullptr;
    if (rocblas_create_handle(&h) != rocblas_status_success) return nullptr;
    // No atomics: a GEMM gives the same bits on every call.
    if (rocblas_set_atomics_mode(h, rocblas_atomics_not_allowed) != rocblas_status_success) {
      rocblas_destroy_handle(h);
      return nullptr;
    }
    handles[dev] = h;
  }
  if (handles[dev] && rocblas_set_stream(handles[dev], s) != rocblas_status_success) return nullptr;
  return handles[dev];
}

// Row-major C[rows][cols] = A[rows][k] B[k][cols], as the column-major
// product C^T = B^T A^T.
bool gemm_rm(rocblas_handle h, bool bf16, int rows, int cols, int k, const void* A, const void* B, void* C) {
  const float one = 1.f, zero = 0.f;
  const rocblas_datatype t = bf16 ? rocblas_datatype_bf16_r : rocblas_datatype_f32_r;
  return rocblas_gemm_ex(h, rocblas_operation_none, rocblas_operation_none, cols, rows, k, &one, B, t, cols, A, t, k,
                         &zero, C, t, cols, C, t, cols, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0,
                         0) == rocblas_status_success;
}


// QKV [batch*n][3][heads][d] -> Q, K, V [batch][heads][n][d]; one 16-byte
// vector per thread, read in source order (coalesced), written per head row.
__global__ __launch_bounds__(256) void k_split_heads(const uint4* __restrict__ qkv, uint4* __restrict__ q,
                                                     uint4* __restrict__ k, uint4* __restrict__ v, int n, int heads,
                                                     int dv, long long total) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= total) return;
  const int jv = (int)(e % dv);
  long long r = e / dv;
  const int h = (int)(r % heads);
  r /= heads;
  const int which = (int)(r % 3);
  const long long tok = r / 3;  // b * n + i
  const long long b = tok / n, i = tok % n;
  uint4* dst = which == 0 ? q : (which == 1 ? k : v);
  dst[((b * heads + h) * n + i) * dv + jv] = qkv[e];
}

}  // namespace

bool make_layer_layout(int batch, int heads, int n, int d, int m, bool bf16, LayerLayout* L) {
  if (!make_layout(batch, heads, n, d, m, &L->fwd)) return false;
  const size_t elems = (size_t)batch * n * heads * d, es = bf16 ? 2 : 4;
  size_t off = L->fwd.total;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  L->qkv = take(3 * elems * es);
  L->o = take(elems * es);
  L->q = take(elems * es);  // Q, K, V head-major, for shapes the attention cannot read in place
  L->k = take(elems * es);
  L->v = take(elems * es);
  L->total = off;
  return true;
}

hipError_t launch_layer(const LayerProblem& lp, const LayerLayout& L, char* ws, hipStream_t s) {
  const Problem& p = lp.attn;
  const int E = p.heads * p.d, rows = p.batch * p.n;
  const size_t es = p.bf16 ? 2 : 4;
  rocblas_handle h = handle_for_current_device(s);
  if (!h) return hipErrorUnknown;
  char* qkv = ws + L.qkv;
  {
    KernelTimer kt_("qkv_gemm", s);
    if (!gemm_rm(h, p.bf16, rows, 3 * E, E, lp.X, lp.Wqkv, qkv)) return hipErrorUnknown;
  }
  // The attention reads each head's Q, K and V where the product left them:
  // token rows 3E elements apart, head h at column h*d of its block.  The
  // output stage writes the heads merged per token ([batch*n][E]), the output
  // projection's input.
  Problem a = p;
  if (apply_in_place(p)) {
    a.Q = qkv;
    a.K = qkv + (size_t)E * es;
    a.V = qkv + (size_t)2 * E * es;
    a.in_ld = 3 * E;
    a.in_hs = p.d;
    a.in_bs = (long long)p.n * 3 * E;
  } else {
    // Other shapes: Q, K, V copied out head-major first.
    const long long total = 3LL * rows * E * (long long)es / 16;
    KernelTimer kt_("split_heads", s);
    k_split_heads<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(
        reinterpret_cast<const uint4*>(qkv), reinterpret_cast<uint4*>(ws + L.q), reinterpret_cast<uint4*>(ws + L.k),
        reinterpret_cast<uint4*>(ws + L.v), p.n, p.heads, (int)(p.d * es / 16), total);
    a.Q = ws + L.q;
    a.K = ws + L.k;
    a.V = ws + L.v;
  }
  char* oc = ws + L.o;
  a.out = oc;
  a.out_merged = true;
  hipError_t e = launch_forward(a, L.fwd, ws, s);
  if (e != hipSuccess) return e;
  {
    KernelTimer kt_("out_gemm", s);
    if (!gemm_rm(h, p.bf16, rows, E, E, oc, lp.Wo, lp.Y)) return hipErrorUnknown;
  }
  return hipGetLastError();
}

}  // namespace nys

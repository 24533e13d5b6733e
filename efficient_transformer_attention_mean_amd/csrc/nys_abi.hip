// C ABI of the Nyström attention library: argument validation, workspace
// contract and the stream-ordered launch of the kernels (nys_landmarks.hip,
// nys_apply.hip, nys_backward.hip, nys_layer.hip, nys_error.hip).
#include <hip/hip_runtime.h>

#include <mutex>
#include <new>

#include "../../include/nystrom.h"
#include "nys_internal.hpp"

namespace {

bool supported_d(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

// Shared validation; returns NYS_OK or the code to report.
int check_shape(int batch, int heads, int n, int d, int m, int iters) {
  if (batch < 1 || heads < 1 || n < 1 || d < 1 || m < 1 || iters < 0) return NYS_EINVAL;
  if (m > n) return NYS_EINVAL;
  if (!supported_d(d) || m > 256 || n > (1 << 24)) return NYS_EUNSUPPORTED;
  if ((long long)n * d >= (1LL << 29)) return NYS_EUNSUPPORTED;  // one head's rows as fp32 stay under 2 GiB
  if ((long long)batch * heads > 65535) return NYS_EUNSUPPORTED;  // batch*heads is a grid dimension
  if ((long long)batch * heads * (long long)n * d > (1LL << 40)) return NYS_EUNSUPPORTED;
  return NYS_OK;
}

}  // namespace

extern "C" {

int nystrom_abi_version(void) { return 100; }

const char* nystrom_strerror(int code) {
  switch (code) {
    case NYS_OK: return "success";
    case NYS_EINVAL: return "invalid argument";
    case NYS_EUNSUPPORTED: return "unsupported shape (d must be 16/32/64/128, m <= 256)";
    case NYS_EWORKSPACE: return "workspace too small";
    case NYS_EHIP: return "HIP runtime error";
    case NYS_ENOTIMPL: return "not implemented";
    default: return "unknown error code";
  }
}

size_t nystrom_attn_workspace_bytes(int batch, int heads, int n, int d, int m) {
  if (check_shape(batch, heads, n, d, m, 0) != NYS_OK) return 0;
  nys::WsLayout L;
  if (!nys::make_layout(batch, heads, n, d, m, &L)) return 0;
  return L.total;
}

long long nystrom_attn_workspace_offset(int which, int batch, int heads, int n, int d, int m) {
  if (check_shape(batch, heads, n, d, m, 0) != NYS_OK) return -1;
  nys::WsLayout L;
  if (!nys::make_layout(batch, heads, n, d, m, &L)) return -1;
  switch (which) {
    case NYS_WS_QT: return (long long)L.qt;
    case NYS_WS_KT: return (long long)L.kt;
    case NYS_WS_A: return (long long)L.a;
    case NYS_WS_Z: return (long long)L.z;
    case NYS_WS_BV: return (long long)L.bv;
    case NYS_WS_W: return (long long)L.w;
    default: return -1;
  }
}

}  // extern "C"

namespace {

int forward(const void* Q, const void* K, const void* V, const float* conv_w, int n, int d, int m, int heads,
            int iters, void* out, int batch, int conv_k, int dtype, const int* lengths, void* workspace,
            size_t workspace_bytes, void* stream) {
  try {
    if (!Q || !K || !V || !out) return NYS_EINVAL;
    if (dtype != NYS_F32 && dtype != NYS_BF16) return NYS_EINVAL;
    if (conv_w && (conv_k < 1 || conv_k % 2 == 0)) return NYS_EINVAL;
    const int rc = check_shape(batch, heads, n, d, m, iters);
    if (rc != NYS_OK) return rc;
    nys::WsLayout L;
    if (!nys::make_layout(batch, heads, n, d, m, &L)) return NYS_EUNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    bool owned = false;
    if (!ws) {
      if (hipMallocAsync(reinterpret_cast<void**>(&ws), L.total, s) != hipSuccess) return NYS_EHIP;
      owned = true;
    } else if (workspace_bytes < L.total) {
      return NYS_EWORKSPACE;
    }
    nys::Problem p{Q, K, V, conv_w, out, batch, heads, n, d, m, iters, conv_w ? conv_k : 0, dtype == NYS_BF16,
                   lengths};
    hipError_t e = nys::launch_forward(p, L, ws, s);
    if (owned) {
      hipError_t f = hipFreeAsync(ws, s);
      if (e == hipSuccess) e = f;
    }
    return e == hipSuccess ? NYS_OK : NYS_EHIP;
  } catch (...) {
    return NYS_EHIP;
  }
}

}  // namespace

namespace {

// Scratch of nystrom_attn_fwd_noalloc: the forward's workspace regions, one
// copy per GPU the library runs on, held until the process ends.  In host
// code `scratch` names a host-side stand-in, never the device memory: every
// host use goes through the per-device address from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[NYS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;

// Device address of this device's `scratch`, looked up once per device (with
// that device current), or nullptr if the lookup failed.
void* scratch_address() {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  static hipError_t status[kMaxDevices] = {};
  static bool looked[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!looked[dev]) {
    void* p = nullptr;
    status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    addr[dev] = status[dev] == hipSuccess ? p : nullptr;
    looked[dev] = true;
  }
  return addr[dev];
}

}  // namespace

extern "C" {

int nystrom_attn_fwd_noalloc(const void* Q, const void* K, const void* V, const float* conv_w, int n, int d, int m,
                             int heads, int iters, void* out, int batch, int conv_k, int dtype, void* stream) {
  try {
    // Validation first: an invalid call returns its code before any HIP call.
    if (!Q || !K || !V || !out) return NYS_EINVAL;
    if (dtype != NYS_F32 && dtype != NYS_BF16) return NYS_EINVAL;
    if (conv_w && (conv_k < 1 || conv_k % 2 == 0)) return NYS_EINVAL;
    const int rc = check_shape(batch, heads, n, d, m, iters);
    if (rc != NYS_OK) return rc;
    nys::WsLayout L;
    if (!nys::make_layout(batch, heads, n, d, m, &L)) return NYS_EUNSUPPORTED;
    if (L.total > NYS_NOALLOC_SCRATCH_BYTES) return NYS_EWORKSPACE;
    void* ws = scratch_address();
    if (!ws) return NYS_EHIP;
    return forward(Q, K, V, conv_w, n, d, m, heads, iters, out, batch, conv_k, dtype, nullptr, ws,
                   NYS_NOALLOC_SCRATCH_BYTES, stream);
  } catch (...) {
    return NYS_EHIP;
  }
}

int nystrom_attn_fwd(const void* Q, const void* K, const void* V, const float* conv_w, int n, int d, int m,
                     int heads, int iters, void* out, int batch, int conv_k, int dtype, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return forward(Q, K, V, conv_w, n, d, m, heads, iters, out, batch, conv_k, dtype, nullptr, workspace,
                 workspace_bytes, stream);
}

int nystrom_attn_fwd_masked(const void* Q, const void* K, const void* V, const float* conv_w, int n, int d, int m,
                            int heads, int iters, void* out, int batch, int conv_k, int dtype, const int* lengths,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return forward(Q, K, V, conv_w, n, d, m, heads, iters, out, batch, conv_k, dtype, lengths, workspace,
                 workspace_bytes, stream);
}

size_t nystrom_attn_bwd_workspace_bytes(int batch, int heads, int n, int d, int m, int iters, int conv_k) {
  if (check_shape(batch, heads, n, d, m, iters) != NYS_OK) return 0;
  // Enough for either dtype (their chunkings differ).
  nys::BwdLayout L, Lb;
  const int ck = conv_k < 0 ? 0 : conv_k;
  if (!nys::make_bwd_layout(batch, heads, n, d, m, iters, ck, false, &L)) return 0;
  if (!nys::make_bwd_layout(batch, heads, n, d, m, iters, ck, true, &Lb)) return 0;
  return L.total > Lb.total ? L.total : Lb.total;
}

size_t nystrom_attn_bwd_state_bytes(int batch, int heads, int n, int d, int m, int iters, int conv_k) {
  if (check_shape(batch, heads, n, d, m, iters) != NYS_OK) return 0;
  nys::BwdLayout L, Lb;
  const int ck = conv_k < 0 ? 0 : conv_k;
  if (!nys::make_bwd_layout(batch, heads, n, d, m, iters, ck, false, &L)) return 0;
  if (!nys::make_bwd_layout(batch, heads, n, d, m, iters, ck, true, &Lb)) return 0;
  return L.state > Lb.state ? L.state : Lb.state;
}

}  // extern "C"

namespace {

// The backward entry points: saved = false recomputes the forward's landmark
// side in `workspace` (allocated when NULL); saved = true takes it from
// `workspace` as nystrom_attn_fwd_save left it (which must then be given).
// With `state` given, the saved state is there instead (state_bytes long) and
// `workspace` is only the scratch (allocated when NULL).
// lengths: device int32 [batch] of sequence lengths, or NULL.
int backward(const void* Q, const void* K, const void* V, const float* conv_w, const void* dO, int n, int d, int m,
             int heads, int iters, void* dQ, void* dK, void* dV, float* dconv_w, int batch, int conv_k, int dtype,
             void* workspace, size_t workspace_bytes, void* stream, bool saved, const int* lengths = nullptr,
             const void* state = nullptr, size_t state_bytes = 0) {
  try {
    if (!Q || !K || !V || !dO || !dQ || !dK || !dV) return NYS_EINVAL;
    if (saved && !workspace && !state) return NYS_EINVAL;
    if (dtype != NYS_F32 && dtype != NYS_BF16) return NYS_EINVAL;
    if (conv_w && (conv_k < 1 || conv_k % 2 == 0)) return NYS_EINVAL;
    const int rc = check_shape(batch, heads, n, d, m, iters);
    if (rc != NYS_OK) return rc;
    const int ck = conv_w ? conv_k : 0;
    nys::BwdLayout L;
    if (!nys::make_bwd_layout(batch, heads, n, d, m, iters, ck, dtype == NYS_BF16, &L)) return NYS_EUNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // Bytes the caller's `workspace` must hold: everything, or the scratch alone.
    const size_t need = state ? L.total - L.state : L.total;
    if (state && state_bytes < L.state) return NYS_EWORKSPACE;
    char* ws = static_cast<char*>(workspace);
    bool owned = false;
    if (!ws) {
      if (hipMallocAsync(reinterpret_cast<void**>(&ws), need, s) != hipSuccess) return NYS_EHIP;
      owned = true;
    } else if (workspace_bytes < need) {
      return NYS_EWORKSPACE;
    }
    nys::BwdProblem p{{Q, K, V, conv_w, nullptr, batch, heads, n, d, m, iters, ck, dtype == NYS_BF16}, dO, dQ, dK,
                      dV, conv_w ? dconv_w : nullptr};
    p.fwd.lens = lengths;
    // The backward reads the saved state and writes only the scratch.
    const nys::BwdBuf buf = state ? nys::BwdBuf{static_cast<char*>(const_cast<void*>(state)), ws, L.state}
                                  : nys::BwdBuf{ws, ws + L.state, L.state};
    hipError_t e = nys::launch_backward(p, L, buf, s, !saved);
    if (owned) {
      hipError_t f = hipFreeAsync(ws, s);
      if (e == hipSuccess) e = f;
    }
    return e == hipSuccess ? NYS_OK : NYS_EHIP;
  } catch (...) {
    return NYS_EHIP;
  }
}

}  // namespace

extern "C" {

int nystrom_attn_bwd(const void* Q, const void* K, const void* V, const float* conv_w, const void* dO, int n, int d,
                     int m, int heads, int iters, void* dQ, void* dK, void* dV, float* dconv_w, int batch, int conv_k,
                     int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return backward(Q, K, V, conv_w, dO, n, d, m, heads, iters, dQ, dK, dV, dconv_w, batch, conv_k, dtype, workspace,
                  workspace_bytes, stream, false);
}

int nystrom_attn_bwd_masked(const void* Q, const void* K, const void* V, const float* conv_w, const void* dO, int n,
                            int d, int m, int heads, int iters, void* dQ, void* dK, void* dV, float* dconv_w,
                            int batch, int conv_k, int dtype, const int* lengths, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return backward(Q, K, V, conv_w, dO, n, d, m, heads, iters, dQ, dK, dV, dconv_w, batch, conv_k, dtype, workspace,
                  workspace_bytes, stream, false, lengths);
}

int nystrom_attn_fwd_save(const void* Q, const void* K, const void* V, const float* conv_w, int n, int d, int m,
                          int heads, int iters, void* out, int batch, int conv_k, int dtype, void* saved,
                          size_t saved_bytes, void* stream) {
  try {
    if (!Q || !K || !V || !out || !saved) return NYS_EINVAL;
    if (dtype != NYS_F32 && dtype != NYS_BF16) return NYS_EINVAL;
    if (conv_w && (conv_k < 1 || conv_k % 2 == 0)) return NYS_EINVAL;
    const int rc = check_shape(batch, heads, n, d, m, iters);
    if (rc != NYS_OK) return rc;
    const int ck = conv_w ? conv_k : 0;
    nys::BwdLayout L;
    if (!nys::make_bwd_layout(batch, heads, n, d, m, iters, ck, dtype == NYS_BF16, &L)) return NYS_EUNSUPPORTED;
    if (saved_bytes < L.state) return NYS_EWORKSPACE;
    nys::Problem p{Q, K, V, conv_w, out, batch, heads, n, d, m, iters, ck, dtype == NYS_BF16};
    const hipError_t e = nys::launch_forward_save(p, L, static_cast<char*>(saved), static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NYS_OK : NYS_EHIP;
  } catch (...) {
    return NYS_EHIP;
  }
}

int nystrom_attn_bwd_saved(const void* Q, const void* K, const void* V, const float* conv_w, const void* dO, int n,
                           int d, int m, int heads, int iters, void* dQ, void* dK, void* dV, float* dconv_w, int batch,
                           int conv_k, int dtype, void* saved, size_t saved_bytes, void* stream) {
  return backward(Q, K, V, conv_w, dO, n, d, m, heads, iters, dQ, dK, dV, dconv_w, batch, conv_k, dtype, saved,
                  saved_bytes, stream, true);
}

int nystrom_attn_bwd_from_state(const void* Q, const void* K, const void* V, const float* conv_w, const void* dO,
                                int n, int d, int m, int heads, int iters, void* dQ, void* dK, void* dV,
                                float* dconv_w, int batch, int conv_k, int dtype, const void* state,
                                size_t state_bytes, void* scratch, size_t scratch_bytes, void* stream) {
  if (!state) return NYS_EINVAL;
  return backward(Q, K, V, conv_w, dO, n, d, m, heads, iters, dQ, dK, dV, dconv_w, batch, conv_k, dtype, scratch,
                  scratch_bytes, stream, true, nullptr, state, state_bytes);
}

size_t nystrom_layer_workspace_bytes(int batch, int heads, int n, int d, int m, int dtype) {
  if (check_shape(batch, heads, n, d, m, 0) != NYS_OK) return 0;
  if (dtype != NYS_F32 && dtype != NYS_BF16) return 0;
  nys::LayerLayout L;
  if (!nys::make_layer_layout(batch, heads, n, d, m, dtype == NYS_BF16, &L)) return 0;
  return L.total;
}

int nystrom_layer_fwd(const void* X, const void* Wqkv, const void* Wo, const float* conv_w, int n, int d, int m,
                      int heads, int iters, void* Y, int batch, int conv_k, int dtype, void* workspace,
                      size_t workspace_bytes, void* stream) {
  try {
    if (!X || !Wqkv || !Wo || !Y) return NYS_EINVAL;
    if (dtype != NYS_F32 && dtype != NYS_BF16) return NYS_EINVAL;
    if (conv_w && (conv_k < 1 || conv_k % 2 == 0)) return NYS_EINVAL;
    const int rc = check_shape(batch, heads, n, d, m, iters);
    if (rc != NYS_OK) return rc;
    if ((long long)batch * n * heads * d * 3 >= (1LL << 31)) return NYS_EUNSUPPORTED;  // GEMM sizes are 32-bit
    nys::LayerLayout L;
    if (!nys::make_layer_layout(batch, heads, n, d, m, dtype == NYS_BF16, &L)) return NYS_EUNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    bool owned = false;
    if (!ws) {
      if (hipMallocAsync(reinterpret_cast<void**>(&ws), L.total, s) != hipSuccess) return NYS_EHIP;
      owned = true;
    } else if (workspace_bytes < L.total) {
      return NYS_EWORKSPACE;
    }
    nys::LayerProblem p{{nullptr, nullptr, nullptr, conv_w, nullptr, batch, heads, n, d, m, iters, conv_w ? conv_k : 0,
                         dtype == NYS_BF16},
                        X, Wqkv, Wo, Y};
    hipError_t e = nys::launch_layer(p, L, ws, s);
    if (owned) {
      hipError_t f = hipFreeAsync(ws, s);
      if (e == hipSuccess) e = f;
    }
    return e == hipSuccess ? NYS_OK : NYS_EHIP;
  } catch (...) {
    return NYS_EHIP;
  }
}

size_t nystrom_attn_error_workspace_bytes(int batch, int heads, int n, int d, int m, int dtype) {
  if (check_shape(batch, heads, n, d, m, 0) != NYS_OK) return 0;
  if (dtype != NYS_F32 && dtype != NYS_BF16) return 0;
  nys::ErrLayout L;
  if (!nys::make_error_layout(batch, heads, n, d, m, dtype == NYS_BF16, &L)) return 0;
  return L.total;
}

int nystrom_attn_error(const void* Q, const void* K, const void* V, int n, int d, int m, int heads, int iters,
                       float* err, int batch, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    if (!Q || !K || !V || !err) return NYS_EINVAL;
    if (dtype != NYS_F32 && dtype != NYS_BF16) return NYS_EINVAL;
    const int rc = check_shape(batch, heads, n, d, m, iters);
    if (rc != NYS_OK) return rc;
    nys::ErrLayout L;
    if (!nys::make_error_layout(batch, heads, n, d, m, dtype == NYS_BF16, &L)) return NYS_EUNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    bool owned = false;
    if (!ws) {
      if (hipMallocAsync(reinterpret_cast<void**>(&ws), L.total, s) != hipSuccess) return NYS_EHIP;
      owned = true;
    } else if (workspace_bytes < L.total) {
      return NYS_EWORKSPACE;
    }
    nys::Problem p{Q, K, V, nullptr, nullptr, batch, heads, n, d, m, iters, 0, dtype == NYS_BF16};
    hipError_t e = nys::launch_error(p, L, ws, err, s);
    if (owned) {
      hipError_t f = hipFreeAsync(ws, s);
      if (e == hipSuccess) e = f;
    }
    return e == hipSuccess ? NYS_OK : NYS_EHIP;
  } catch (...) {
    return NYS_EHIP;
  }
}

int nystrom_dconv_fwd(const void* V, const float* conv_w, int n, int d, int heads, int batch, int conv_k, int dtype,
                      void* out, void* stream) {
  try {
    if (!V || !conv_w || !out) return NYS_EINVAL;
    if (dtype != NYS_F32 && dtype != NYS_BF16) return NYS_EINVAL;
    if (conv_k < 1 || conv_k % 2 == 0) return NYS_EINVAL;
    if (batch < 1 || heads < 1 || n < 1 || d < 1) return NYS_EINVAL;
    if (!supported_d(d) || n > (1 << 24) || (long long)batch * heads > 65535) return NYS_EUNSUPPORTED;
    if ((long long)n * d >= (1LL << 29)) return NYS_EUNSUPPORTED;
    hipError_t e = nys::launch_dconv(V, conv_w, out, batch, heads, n, d, conv_k, dtype == NYS_BF16,
                                     static_cast<hipStream_t>(stream));
    return e == hipSuccess ? NYS_OK : NYS_EHIP;
  } catch (...) {
    return NYS_EHIP;
  }
}

}  // extern "C"

// Host-side view of the workspace and the launch sequence (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace nys {

// Byte offsets of every region in the caller's workspace.  All regions are
// fp32 (counters are u32) and 256-byte aligned.
struct WsLayout {
  size_t qt, kt, a, z, bv, w;      // documented intermediates (NYS_WS_*)
  size_t z2, x, t, u;              // pseudoinverse scratch for m > 64
  size_t pacc, pmax, psum;         // split-n partials of softmax(Qt K^T) V
  size_t total;
  int nchunks, chunk;              // keys per landmark_bv block, blocks per head
};

// Returns false for shapes the kernels do not handle.
bool make_layout(int batch, int heads, int n, int d, int m, WsLayout* L);

struct Problem {
  const void* Q;
  const void* K;
  const void* V;
  const float* conv_w;
  void* out;
  int batch, heads, n, d, m, iters, conv_k;
  bool bf16;
};

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

hipError_t launch_forward(const Problem& p, const WsLayout& L, char* ws, hipStream_t s);
hipError_t launch_dconv(const void* V, const float* conv_w, void* out, int batch, int heads, int n,
                        int d, int conv_k, bool bf16, hipStream_t s);

}  // namespace nys

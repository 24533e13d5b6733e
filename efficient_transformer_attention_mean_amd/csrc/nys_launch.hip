// Workspace layout and the stream-ordered sequence of forward stages.
#include <mutex>
#include <vector>

#include "nys_internal.hpp"

namespace nys {

static long long cdiv(long long a, long long b) { return (a + b - 1) / b; }

bool make_layout(int batch, int heads, int n, int d, int m, WsLayout* L) {
  if (batch < 1 || heads < 1 || n < 1 || m < 1 || m > n || n % m != 0) return false;
  if (!(d == 16 || d == 32 || d == 64 || d == 128) || m > 256 || n > (1 << 24)) return false;
  const long long BH = (long long)batch * heads;
  // Key chunking for the split-n pass: aim for about 2 blocks per CU over 256
  // CUs; chunks are a multiple of the 64-key tile.
  long long want = cdiv(512, BH);
  long long maxch = cdiv(n, 64);
  long long nch = want < 1 ? 1 : (want > maxch ? maxch : want);
  long long chunk = cdiv(cdiv(n, nch), 64) * 64;
  nch = cdiv(n, chunk);
  L->nchunks = (int)nch;
  L->chunk = (int)chunk;
  L->mpa = m <= 32 ? 32 : m <= 64 ? 64 : m <= 128 ? 128 : 256;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  const size_t md = (size_t)BH * m * d * 4, mm = (size_t)BH * m * m * 4;
  L->qt = take(md);
  L->kt = take(md);
  L->a = take(mm);
  L->z = take(mm);
  L->bv = take(md);
  L->w = take(md);
  const bool big = m > 64;
  L->z2 = take(big ? mm : 0);
  L->x = take(big ? mm : 0);
  L->t = take(big ? mm : 0);
  L->u = take(big ? mm : 0);
  L->pacc = take((size_t)BH * nch * m * d * 4);
  L->pmax = take((size_t)BH * nch * m * 4);
  L->psum = take((size_t)BH * nch * m * 4);
  L->kt_hi = take((size_t)BH * L->mpa * d * 2);
  L->kt_lo = take((size_t)BH * L->mpa * d * 2);
  L->wt_hi = take((size_t)BH * d * L->mpa * 2);
  L->wt_lo = take((size_t)BH * d * L->mpa * 2);
  L->cwop = take((size_t)heads * d * 4 * 9 * 16);
  L->total = off;
  return true;
}

Ws resolve(const WsLayout& L, char* b) {
  Ws w;
  w.Qt = reinterpret_cast<float*>(b + L.qt);
  w.Kt = reinterpret_cast<float*>(b + L.kt);
  w.A = reinterpret_cast<float*>(b + L.a);
  w.Z = reinterpret_cast<float*>(b + L.z);
  w.BV = reinterpret_cast<float*>(b + L.bv);
  w.W = reinterpret_cast<float*>(b + L.w);
  w.Z2 = reinterpret_cast<float*>(b + L.z2);
  w.X = reinterpret_cast<float*>(b + L.x);
  w.T = reinterpret_cast<float*>(b + L.t);
  w.U = reinterpret_cast<float*>(b + L.u);
  w.pacc = reinterpret_cast<float*>(b + L.pacc);
  w.pmax = reinterpret_cast<float*>(b + L.pmax);
  w.psum = reinterpret_cast<float*>(b + L.psum);
  w.kt_hi = reinterpret_cast<uint16_t*>(b + L.kt_hi);
  w.kt_lo = reinterpret_cast<uint16_t*>(b + L.kt_lo);
  w.wt_hi = reinterpret_cast<uint16_t*>(b + L.wt_hi);
  w.wt_lo = reinterpret_cast<uint16_t*>(b + L.wt_lo);
  w.cwop = reinterpret_cast<uint4*>(b + L.cwop);
  w.nchunks = L.nchunks;
  w.chunk = L.chunk;
  w.mpa = L.mpa;
  return w;
}

namespace {

// A side stream (default priority, non-blocking) and two events, reused
// across calls on one device.  Enqueued waits capture an event's state when
// they are enqueued, so an entry can be handed to the next call as soon as
// the join has been enqueued.
struct Side {
  int device;
  hipStream_t stream;
  hipEvent_t fork, join;
};
std::mutex g_side_mu;
std::vector<Side*> g_side_free;

hipError_t acquire_side(Side** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  {
    std::lock_guard<std::mutex> lk(g_side_mu);
    for (size_t i = 0; i < g_side_free.size(); ++i) {
      if (g_side_free[i]->device == dev) {
        *out = g_side_free[i];
        g_side_free.erase(g_side_free.begin() + i);
        return hipSuccess;
      }
    }
  }
  Side* sd = new Side{dev, nullptr, nullptr, nullptr};
  if ((e = hipStreamCreateWithFlags(&sd->stream, hipStreamNonBlocking)) != hipSuccess ||
      (e = hipEventCreateWithFlags(&sd->fork, hipEventDisableTiming)) != hipSuccess ||
      (e = hipEventCreateWithFlags(&sd->join, hipEventDisableTiming)) != hipSuccess) {
    delete sd;  // handles created so far are kept alive by the runtime until exit
    return e;
  }
  *out = sd;
  return hipSuccess;
}

void release_side(Side* sd) {
  std::lock_guard<std::mutex> lk(g_side_mu);
  g_side_free.push_back(sd);
}

}  // namespace

hipError_t launch_forward(const Problem& p, const WsLayout& L, char* ws, hipStream_t s) {
  const Ws w = resolve(L, ws);
  hipError_t e;
  if ((e = stage_segment_means(p, w, s)) != hipSuccess) return e;
  Side* sd = nullptr;
  if ((e = acquire_side(&sd)) != hipSuccess) return e;
  // Fork: the pseudoinverse (landmarks only) and the skip-filter operands
  // beside the split-n pass over K, V.
  if ((e = hipEventRecord(sd->fork, s)) == hipSuccess && (e = hipStreamWaitEvent(sd->stream, sd->fork, 0)) == hipSuccess &&
      (e = stage_conv_ops(p, w, sd->stream)) == hipSuccess && (e = stage_pinv(p, w, sd->stream)) == hipSuccess &&
      (e = hipEventRecord(sd->join, sd->stream)) == hipSuccess &&
      (e = stage_bv(p, w, s)) == hipSuccess) {
    e = hipStreamWaitEvent(s, sd->join, 0);
  }
  release_side(sd);
  if (e != hipSuccess) return e;
  if ((e = stage_bv_finish(p, w, s)) != hipSuccess) return e;
  return stage_apply(p, w, s);
}

}  // namespace nys

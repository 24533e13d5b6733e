// Workspace layout and the stream-ordered sequence of forward stages.
#include <map>
#include <mutex>
#include <utility>

#include "nys_internal.hpp"

namespace nys {

hipError_t ensure_dynamic_smem(const void* fn, int bytes) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, hipError_t> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(fn, dev);
  auto it = done.find(key);
  if (it != done.end()) return it->second;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  done.emplace(key, e);
  return e;
}

static long long cdiv(long long a, long long b) { return (a + b - 1) / b; }

bool make_layout(int batch, int heads, int n, int d, int m, WsLayout* L) {
  if (batch < 1 || heads < 1 || n < 1 || m < 1 || m > n) return false;
  if (!(d == 16 || d == 32 || d == 64 || d == 128) || m > 256 || n > (1 << 24)) return false;
  const long long BH = (long long)batch * heads;
  // Key chunking for the split-n pass: 512-thread blocks of two chunks each,
  // one block per CU over 256 CUs together with the one pseudoinverse block
  // per head that shares the launch; chunks are a multiple of the 64-key
  // tile, and their count is even (a trailing chunk may be empty).
  // For m > 128 a chunk takes a whole block (8 waves) and no pseudoinverse
  // blocks share the launch.
  const bool one = m > 128;
  long long want = one ? 256 / BH : 2 * ((256 - (BH < 256 ? BH : 256)) / BH);
  long long maxch = cdiv(n, 64);
  long long nch = want < 1 ? 1 : (want > maxch ? maxch : want);
  if (nch > 32) nch = 32;  // bounds the partials one block combines per head
  long long chunk = cdiv(cdiv(n, nch), 64) * 64;
  nch = cdiv(n, chunk);
  L->nchunks = (int)(one ? nch : nch + (nch & 1));
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
  L->v = take(big ? mm : 0);
  L->colp = take(big ? (size_t)BH * cdiv(m, 16) * m * 4 : 0);
  L->rsum = take(big ? (size_t)BH * m * 4 : 0);
  L->pacc = take((size_t)BH * L->nchunks * m * d * 4);
  L->pmax = take((size_t)BH * L->nchunks * m * 4);
  L->psum = take((size_t)BH * L->nchunks * m * 4);
  L->kt_hi = take((size_t)BH * L->mpa * d * 2);
  L->kt_lo = take((size_t)BH * L->mpa * d * 2);
  L->qt_hi = take((size_t)BH * L->mpa * d * 2);
  L->qt_lo = take((size_t)BH * L->mpa * d * 2);
  L->wt_hi = take((size_t)BH * d * L->mpa * 2);
  L->wt_lo = take((size_t)BH * d * L->mpa * 2);
  L->cwop = take((size_t)heads * d * 4 * 9 * 16);
  L->sync = take((size_t)BH * 2 * 4);
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
  w.V = reinterpret_cast<float*>(b + L.v);
  w.colp = reinterpret_cast<float*>(b + L.colp);
  w.rsum = reinterpret_cast<float*>(b + L.rsum);
  w.pacc = reinterpret_cast<float*>(b + L.pacc);
  w.pmax = reinterpret_cast<float*>(b + L.pmax);
  w.psum = reinterpret_cast<float*>(b + L.psum);
  w.kt_hi = reinterpret_cast<uint16_t*>(b + L.kt_hi);
  w.kt_lo = reinterpret_cast<uint16_t*>(b + L.kt_lo);
  w.qt_hi = reinterpret_cast<uint16_t*>(b + L.qt_hi);
  w.qt_lo = reinterpret_cast<uint16_t*>(b + L.qt_lo);
  w.wt_hi = reinterpret_cast<uint16_t*>(b + L.wt_hi);
  w.wt_lo = reinterpret_cast<uint16_t*>(b + L.wt_lo);
  w.cwop = reinterpret_cast<uint4*>(b + L.cwop);
  w.sync = reinterpret_cast<unsigned*>(b + L.sync);
  w.nchunks = L.nchunks;
  w.chunk = L.chunk;
  w.mpa = L.mpa;
  return w;
}

hipError_t launch_forward(const Problem& p, const WsLayout& L, char* ws, hipStream_t s) {
  // strided inputs: kernels compiled for these shapes only, forward-only (no saved steps)
  if (p.in_ld > 0 && (!apply_in_place(p) || p.zsave)) return hipErrorInvalidValue;
  const Ws w = resolve(L, ws);
  hipError_t e;
  if ((e = stage_segment_means(p, w, s)) != hipSuccess) return e;
  if ((e = stage_landmark_pass(p, w, s)) != hipSuccess) return e;
  if ((e = stage_pinv(p, w, s)) != hipSuccess) return e;
  if ((e = stage_bv_finish(p, w, s)) != hipSuccess) return e;
  return stage_apply(p, w, s);
}

}  // namespace nys

// Approximation-error diagnostic: per (batch, head), the relative Frobenius
// distance between the method's attention output and exact softmax attention
// ("Nyströmformer: A Nyström-Based Algorithm for Approximating
// Self-Attention", paper deep-dive page: Eq. 2 for exact attention; the
// page's closing discussion proposes measuring the approximation error per
// example).
//
//   O_nys = the forward's attention output without the skip (the skip is
//           exact), written to the workspace in the I/O type;
//   O_ex  = softmax(Q K^T / sqrt d) V by k_exact_error: one block per 64
//           queries of a head, online softmax over 64-key tiles on the matrix
//           cores (scores computed transposed, keys x queries, so a lane holds
//           16 keys of one query and its C tile is the B operand of O^T +=
//           V^T P^T with V^T stored in the permuted chunk order);
//   err   = sqrt(sum (O_nys - O_ex)^2 / sum O_ex^2), partial sums per block
//           folded in block order by k_error_finish.
// Products: single bf16 operands for bf16 I/O, bf16x3 splits for fp32 I/O;
// the operands sit in LDS as ready bf16 planes (one 16-byte read per fragment).
#include <math.h>

#include "nys_common.hpp"
#include "nys_internal.hpp"

namespace nys {

namespace {

constexpr int kQT = 64;  // queries per block (16 per wave)
constexpr int kKT = 64;  // keys per tile

// Position of key j of a 64-key tile in the order {4g..4g+3, 16+4g..16+4g+3}
// of its chunk of 32: the order in which a lane holds its probabilities.
__device__ __forceinline__ int err_slot(int j) {
  const int jj = j & 31;
  return (j & ~31) + 8 * ((jj & 15) >> 2) + (jj & 3) + ((jj & 16) ? 4 : 0);
}

// Operand planes in LDS: bf16 rows (hi, and lo for fp32 I/O where every
// product is the bf16x3 sum hi*hi + hi*lo + lo*hi), written once per tile so
// that each fragment is one 16-byte read.
template <int NPL, int ROWS, int COLS>
struct Planes {
  static constexpr int P = COLS + 8;
  uint16_t v[NPL][ROWS][P];
};

template <int NPL, int ROWS, int COLS>
__device__ __forceinline__ void put(Planes<NPL, ROWS, COLS>& pl, int r, int c, float x) {
  const uint16_t h = f32_to_bf16(x);
  pl.v[0][r][c] = h;
  if constexpr (NPL == 2) pl.v[1][r][c] = f32_to_bf16(x - bf16_to_f32(h));
}

template <int NPL, int ROWS, int COLS>
__device__ __forceinline__ void frag(const Planes<NPL, ROWS, COLS>& pl, int r, int c0, B8& h, B8& l) {
  h.q = *reinterpret_cast<const uint4*>(&pl.v[0][r][c0]);
  if constexpr (NPL == 2) l.q = *reinterpret_cast<const uint4*>(&pl.v[1][r][c0]);
}

template <typename IO, int D>
struct ErrSmem {
  static constexpr int NPL = IO::kBf16 ? 1 : 2;
  static constexpr int DP = D < 32 ? 32 : D;  // feature axis padded to a whole 32-wide chunk
  Planes<NPL, kQT, DP> q;   // Q * log2(e)/sqrt(d), query rows
  Planes<NPL, kKT, DP> k;   // key rows of the tile
  Planes<NPL, D, kKT> vT;   // V^T of the tile, keys in err_slot order
  float red[8];
};

template <typename IO, int D>
__global__ __launch_bounds__(256) void k_exact_error(const typename IO::T* __restrict__ Q,
                                                     const typename IO::T* __restrict__ K,
                                                     const typename IO::T* __restrict__ V,
                                                     const typename IO::T* __restrict__ Onys,
                                                     float* __restrict__ part, int n, int ntile, float sl2e) {
  using SM = ErrSmem<IO, D>;
  constexpr int NPL = SM::NPL, DP = SM::DP, KC = DP / 32, ND = D / 16;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  SM& sm = *reinterpret_cast<SM*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c = lane & 15, g = lane >> 4;
  const int qt = blockIdx.x, bh = blockIdx.y, q0 = qt * kQT;
  const size_t hoff = (size_t)bh * n * D;

  for (int e = tid; e < kQT * DP; e += 256) {
    const int r = e / DP, f = e % DP, row = q0 + r;
    put(sm.q, r, f, (row < n && f < D) ? load_elem<IO>(Q + hoff + (size_t)row * D + f) * sl2e : 0.f);
    if (DP > D && f >= D) put(sm.k, r, f, 0.f);  // padding columns of the key planes stay zero
  }
  const int ql = 16 * wave + c;  // this lane's query within the block
  float mrun = -INFINITY, lrun = 0.f;
  f32x4_t acc[ND];
#pragma unroll
  for (int nd = 0; nd < ND; ++nd) acc[nd] = zero4();

  // Key and value rows travel as 16-byte vectors; the next tile's vectors
  // are fetched into registers while the current tile is computed.
  using T = typename IO::T;
  constexpr int VEC = 16 / (int)sizeof(T), RV = D / VEC, NV = kKT * RV, VPT = (NV + 255) / 256;
  uint4 kv[VPT], vv[VPT];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int e = tid + 256 * u, key = k0 + e / RV, c0 = (e % RV) * VEC;
      const bool in = e < NV && key < n;
      kv[u] = in ? *reinterpret_cast<const uint4*>(K + hoff + (size_t)key * D + c0) : make_uint4(0, 0, 0, 0);
      vv[u] = in ? *reinterpret_cast<const uint4*>(V + hoff + (size_t)key * D + c0) : make_uint4(0, 0, 0, 0);
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int e = tid + 256 * u;
      if (e >= NV) continue;
      const int r = e / RV, c0 = (e % RV) * VEC, slot = err_slot(r);
      float xk[VEC], xv[VEC];
      if constexpr (IO::kBf16) {
        B8 a, b;
        a.q = kv[u];
        b.q = vv[u];
        *reinterpret_cast<uint4*>(&sm.k.v[0][r][c0]) = kv[u];  // one plane: the bits themselves
#pragma unroll
        for (int q = 0; q < VEC; ++q) sm.vT.v[0][c0 + q][slot] = b.h[q];
        (void)xk;
        (void)xv;
        (void)a;
      } else {
        const float4 a = __builtin_bit_cast(float4, kv[u]), b = __builtin_bit_cast(float4, vv[u]);
        xk[0] = a.x; xk[1] = a.y; xk[2] = a.z; xk[3] = a.w;
        xv[0] = b.x; xv[1] = b.y; xv[2] = b.z; xv[3] = b.w;
#pragma unroll
        for (int q = 0; q < VEC; ++q) {
          put(sm.k, r, c0 + q, xk[q]);
          put(sm.vT, c0 + q, slot, xv[q]);
        }
      }
    }
  };
  fetch(0);

  for (int k0 = 0; k0 < n; k0 += kKT) {
    __syncthreads();
    stage();
    __syncthreads();
    if (k0 + kKT < n) fetch(k0 + kKT);

    // S^T (keys x queries) for 4 tiles of 16 keys.
    B8 bq[KC], bql[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) frag(sm.q, ql, kc * 32 + 8 * g, bq[kc], bql[kc]);
    f32x4_t s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      s[kt] = zero4();
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        B8 ah, al;
        frag(sm.k, kt * 16 + c, kc * 32 + 8 * g, ah, al);
        if constexpr (NPL == 2) s[kt] = mfma3(ah, al, bq[kc], bql[kc], s[kt]);
        else s[kt] = mfma(ah, bq[kc], s[kt]);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (k0 + kt * 16 + 4 * g + i >= n) s[kt][i] = -INFINITY;
        mx = fmaxf(mx, s[kt][i]);
      }
    mx = max_over_groups(mx);
    const float mnew = fmaxf(mrun, mx);
    const float corr = exp2f(mrun - mnew);  // 0 on the first tile (mrun = -inf)
    float ps = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s[kt][i] = exp2f(s[kt][i] - mnew);
        ps += s[kt][i];
      }
    lrun = lrun * corr + sum_over_groups(ps);
    mrun = mnew;
    // O^T += V^T P^T over the tile's keys.
    B8 ph[2], pl[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      float b[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        b[i] = s[2 * kk][i];
        b[4 + i] = s[2 * kk + 1][i];
      }
      if constexpr (NPL == 2) split8(b, ph[kk], pl[kk]); else round8(b, ph[kk]);
    }
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) {
      acc[nd] *= corr;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        B8 ah, al;
        frag(sm.vT, nd * 16 + c, kk * 32 + 8 * g, ah, al);
        if constexpr (NPL == 2) acc[nd] = mfma3(ah, al, ph[kk], pl[kk], acc[nd]);
        else acc[nd] = mfma(ah, ph[kk], acc[nd]);
      }
    }
  }

  // Lane: query q0 + ql, features nd*16 + 4g + i.
  const int row = q0 + ql;
  float dsum = 0.f, esum = 0.f;
  if (row < n) {
    const float inv = 1.f / lrun;
#pragma unroll
    for (int nd = 0; nd < ND; ++nd)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ex = acc[nd][i] * inv;
        const float dv = load_elem<IO>(Onys + hoff + (size_t)row * D + nd * 16 + 4 * g + i) - ex;
        dsum = fmaf(dv, dv, dsum);
        esum = fmaf(ex, ex, esum);
      }
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    dsum += shfl_xor(dsum, o);
    esum += shfl_xor(esum, o);
  }
  if (lane == 0) {
    sm.red[wave] = dsum;
    sm.red[4 + wave] = esum;
  }
  __syncthreads();
  if (tid == 0) {
    part[((size_t)bh * ntile + qt) * 2] = (sm.red[0] + sm.red[1]) + (sm.red[2] + sm.red[3]);
    part[((size_t)bh * ntile + qt) * 2 + 1] = (sm.red[4] + sm.red[5]) + (sm.red[6] + sm.red[7]);
  }
}

__global__ __launch_bounds__(256) void k_error_finish(const float* __restrict__ part, float* __restrict__ err,
                                                      int bhs, int ntile) {
  const int bh = blockIdx.x * 256 + threadIdx.x;
  if (bh >= bhs) return;
  float a = 0.f, b = 0.f;
  for (int t = 0; t < ntile; ++t) {
    a += part[((size_t)bh * ntile + t) * 2];
    b += part[((size_t)bh * ntile + t) * 2 + 1];
  }
  err[bh] = b > 0.f ? sqrtf(a / b) : 0.f;
}

int ceil_div_i(long long a, long long b) { return (int)((a + b - 1) / b); }

}  // namespace

bool make_error_layout(int batch, int heads, int n, int d, int m, bool bf16, ErrLayout* L) {
  if (!make_layout(batch, heads, n, d, m, &L->fwd)) return false;
  size_t off = L->fwd.total;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  L->ntile = ceil_div_i(n, kQT);
  L->onys = take((size_t)batch * heads * n * d * (bf16 ? 2 : 4));
  L->part = take((size_t)batch * heads * L->ntile * 2 * 4);
  L->total = off;
  return true;
}

template <typename IO, int D>
static hipError_t error_t(const Problem& p, const ErrLayout& L, char* ws, float* err, hipStream_t s) {
  using T = typename IO::T;
  const int bytes = (int)sizeof(ErrSmem<IO, D>);
  auto kern = &k_exact_error<IO, D>;
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (attr != hipSuccess) return attr;
  const int BH = p.batch * p.heads;
  float* part = reinterpret_cast<float*>(ws + L.part);
  {
    KernelTimer kt_("exact_error", s);
    kern<<<dim3(L.ntile, BH), 256, bytes, s>>>(static_cast<const T*>(p.Q), static_cast<const T*>(p.K),
                                               static_cast<const T*>(p.V), reinterpret_cast<const T*>(ws + L.onys),
                                               part, p.n, L.ntile, kLog2e / sqrtf((float)D));
  }
  {
    KernelTimer kt_("error_finish", s);
    k_error_finish<<<ceil_div_i(BH, 256), 256, 0, s>>>(part, err, BH, L.ntile);
  }
  return hipGetLastError();
}

hipError_t launch_error(const Problem& p, const ErrLayout& L, char* ws, float* err, hipStream_t s) {
  Problem a = p;
  a.conv_w = nullptr;  // attention output only
  a.conv_k = 0;
  a.out = ws + L.onys;
  hipError_t e = launch_forward(a, L.fwd, ws, s);
  if (e != hipSuccess) return e;
  switch (p.d) {
    case 16: return p.bf16 ? error_t<BF16, 16>(p, L, ws, err, s) : error_t<F32, 16>(p, L, ws, err, s);
    case 32: return p.bf16 ? error_t<BF16, 32>(p, L, ws, err, s) : error_t<F32, 32>(p, L, ws, err, s);
    case 64: return p.bf16 ? error_t<BF16, 64>(p, L, ws, err, s) : error_t<F32, 64>(p, L, ws, err, s);
    case 128: return p.bf16 ? error_t<BF16, 128>(p, L, ws, err, s) : error_t<F32, 128>(p, L, ws, err, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nys

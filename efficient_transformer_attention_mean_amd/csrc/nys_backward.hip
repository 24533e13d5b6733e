// Nyström self-attention backward: HIP kernels for gfx950 (CDNA4).
//
// Gradients of the forward pass ("Nyströmformer: A Nyström-Based Algorithm
// for Approximating Self-Attention", paper deep-dive page, sec. 3.4: Eq. 13,
// Eq. 16, Lemma 1 and its initialisation, Eq. 17 and the DConv skip of
// Figure 4) with respect to Q, K, V and the skip filters.  The pages train
// through the fixed number of pseudoinverse steps; the derivative here is
// that of the forward computation as written, step by step in reverse.
//
// Per (batch, head), with s = 1/sqrt(d), P' = softmax backward
// (dS = P * (dP - rowsum(dP * P))):
//   dW = F^T dO,  dF = dO W^T,  dS_F = F'(dF)               -> k_bwd_rows (partials)
//   dW, dKt_F = s dS_F^T Q summed, dBV = Z^T dW              -> k_bwd_land_prep
//   dZ = dW BV^T, dA = Lemma-1 backward, dS_A = A'(dA),
//   dKt = dKt_F + s dS_A^T Qt, dQt_A = s dS_A Kt             -> k_bwd_land
//   B = softmax(s Qt K^T) from the forward's row statistics, dB = dBV V^T,
//   dS_B = B'(dB), dK = s dS_B^T Qt + seg^T dKt, dV = B^T dBV + DConv^T(dO),
//   dQt_B = s dS_B K, dw = sum dO (x) V                      -> k_bwd_key (+ partials)
//   dQt = dQt_A + dQt_B, dw summed over batch and chunks     -> k_bwd_finish
//   dQ = s dS_F Kt + seg^T dQt                               -> k_bwd_rows
// where seg^T spreads landmark j's gradient over the real rows of segment j,
// divided by the (padded) segment length.  The landmark-side forward values
// (Qt, Kt, A, Z, BV, W and the split-n softmax statistics of B) are
// recomputed by the forward's own kernels at the start of the call.
//
// On the matrix-core path (bf16 I/O, d = 32 or 64) the key side needs only
// dBV, so it runs on a second stream beside k_bwd_land (one block per head),
// after the skip's share, which reads only inputs: the filter gradient
// (k_bwd_skip_grad, forked at the start of the call, beside the forward's
// stages) and dV = DConv^T(dO) by the forward's convolution with the taps
// reversed (forked after them, beside the query-side reduction).  The query-side pass
// k_bwd_rows_mm also writes dQ's first term s dS_F Kt, and k_bwd_key_mm
// leaves out the seg^T dKt term of dK; once the landmark side is done,
// k_bwd_spread adds seg^T dQt to dQ and seg^T dKt to dK.
//
// The n-sized passes run in fp32 on the vector units with their operands in
// LDS; the m x m products of the pseudoinverse backward use the matrix cores
// with split-bf16 operands (bf16x3 for bf16 I/O, three-way for fp32 I/O).
#include <math.h>

#include <mutex>

#include "nys_common.hpp"
#include "nys_internal.hpp"

namespace nys {

namespace {

constexpr int kRowTile = 32;  // query rows per tile of k_bwd_rows
constexpr int kKeyTile = 16;  // key rows per tile of k_bwd_key

template <typename IO>
__device__ __forceinline__ float ld(const typename IO::T* p) {
  return load_elem<IO>(p);
}

// ---------------------------------------------------------------------------
// Query side.  Grid (chunks, batch*heads); each block walks tiles of 32 rows
// of its chunk.  Per row i (thread group of 8 lanes, landmarks jl + 8u):
//   F_i = softmax(s Q_i Kt^T), dF_i = dO_i W^T, dS_i = F_i * (dF_i - F_i . dF_i).
// DQ = false: accumulates dW = sum_i F_i^T dO_i and dKt_F = s sum_i dS_i^T Q_i
//             per chunk (fixed order) and writes the chunk's partials.
// DQ = true:  writes dQ_i = s dS_i Kt + dQt[seg(i)] / l.
template <typename IO, int D, bool DQ>
__global__ __launch_bounds__(256) void k_bwd_rows(const typename IO::T* __restrict__ Q,
                                                  const typename IO::T* __restrict__ dO,
                                                  const float* __restrict__ Kt, const float* __restrict__ W,
                                                  const float* __restrict__ dqt, typename IO::T* __restrict__ dQ,
                                                  float* __restrict__ pdw, float* __restrict__ pdkt,
                                                  const int* __restrict__ lens, int heads, int n, int m,
                                                  int chunk, int nchunks, float sl2e, float scale) {
  constexpr int P = D + 1;  // LDS pitch of d-wide rows
  constexpr int NE = 64 * D / 256;
  extern __shared__ __align__(16) float lds[];
  float* kt = lds;                  // [64][P]
  float* ws = kt + 64 * P;          // [64][P]
  float* qs = ws + 64 * P;          // [kRowTile][P]
  float* gs = qs + kRowTile * P;    // [kRowTile][P]
  float* fs = gs + kRowTile * P;    // [kRowTile][65]
  float* ds = fs + kRowTile * 65;   // [kRowTile][65]
  const int tid = threadIdx.x, ch = blockIdx.x, bh = blockIdx.y;
  const int r = tid >> 3, jl = tid & 7;
  const size_t hoff = (size_t)bh * n * D;

  for (int e = tid; e < 64 * D; e += 256) {
    const int j = e / D, c = e % D;
    kt[j * P + c] = j < m ? Kt[((size_t)bh * m + j) * D + c] : 0.f;
    ws[j * P + c] = j < m ? W[((size_t)bh * m + j) * D + c] : 0.f;
  }
  float aw[NE], ak[NE];
#pragma unroll
  for (int v = 0; v < NE; ++v) aw[v] = ak[v] = 0.f;
  // Rows of the sequence (all n without a mask); the segment length is
  // that of the sequence's own padding to m rows.
  const int nb = seq_rows(lens, bh / heads, n);
  const int seg = max(1, (nb + m - 1) / m);
  const float inv_seg = 1.f / (float)seg;

  const int rbeg = ch * chunk, rend = min(nb, rbeg + chunk);
  for (int t0 = rbeg; t0 < rend; t0 += kRowTile) {
    __syncthreads();  // previous tile's readers done (and the landmark rows visible)
    for (int e = tid; e < kRowTile * D; e += 256) {
      const int rr = e / D, c = e % D, row = t0 + rr;
      const bool in = row < rend;
      qs[rr * P + c] = in ? ld<IO>(Q + hoff + (size_t)row * D + c) : 0.f;
      gs[rr * P + c] = in ? ld<IO>(dO + hoff + (size_t)row * D + c) : 0.f;
    }
    __syncthreads();

    float sc[8], df[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) sc[u] = df[u] = 0.f;
    for (int k = 0; k < D; ++k) {
      const float q = qs[r * P + k], gv = gs[r * P + k];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        sc[u] = fmaf(q, kt[(jl + 8 * u) * P + k], sc[u]);
        df[u] = fmaf(gv, ws[(jl + 8 * u) * P + k], df[u]);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      sc[u] = (jl + 8 * u < m) ? sc[u] * sl2e : -INFINITY;
      mx = fmaxf(mx, sc[u]);
    }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) mx = fmaxf(mx, shfl_xor(mx, o));
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      sc[u] = exp2f(sc[u] - mx);  // 0 for the padding landmarks
      sum += sc[u];
    }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) sum += shfl_xor(sum, o);
    const float inv = 1.f / sum;
    float delta = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      sc[u] *= inv;  // F
      delta = fmaf(sc[u], df[u], delta);
    }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) delta += shfl_xor(delta, o);
    const bool live = t0 + r < rend;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = jl + 8 * u;
      if (j < 64) {
        fs[r * 65 + j] = live ? sc[u] : 0.f;
        ds[r * 65 + j] = live ? sc[u] * (df[u] - delta) : 0.f;
      }
    }
    __syncthreads();

    if constexpr (DQ) {
      // dQ row r, features c = jl + 8w.
      const int row = t0 + r;
      if (row < rend) {
        const float* qtr = dqt + ((size_t)bh * m + row / seg) * D;
        for (int c = jl; c < D; c += 8) {
          float acc = 0.f;
          for (int j = 0; j < m; ++j) acc = fmaf(ds[r * 65 + j], kt[j * P + c], acc);
          store_elem<IO>(dQ + hoff + (size_t)row * D + c, fmaf(scale, acc, qtr[c] * inv_seg));
        }
      }
    } else {
#pragma unroll
      for (int v = 0; v < NE; ++v) {
        const int e = tid + 256 * v, j = e / D, c = e % D;
        float a0 = aw[v], a1 = ak[v];
#pragma unroll 4
        for (int rr = 0; rr < kRowTile; ++rr) {
          a0 = fmaf(fs[rr * 65 + j], gs[rr * P + c], a0);
          a1 = fmaf(ds[rr * 65 + j], qs[rr * P + c], a1);
        }
        aw[v] = a0;
        ak[v] = a1;
      }
    }
  }
  if constexpr (!DQ) {
    const size_t base = ((size_t)bh * nchunks + ch) * m * D;
#pragma unroll
    for (int v = 0; v < NE; ++v) {
      const int e = tid + 256 * v, j = e / D;
      if (j < m) {
        pdw[base + e] = aw[v];
        pdkt[base + e] = scale * ak[v];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Landmark side, one block per head (512 threads for MP = 64, 256 for
// MP = 32; m <= MP, MP x MP matrices in LDS with pitch MP + 4).

template <int MP>
struct LandSmem {
  static constexpr int LP = MP + 4;
  float A[MP][LP], dA[MP][LP], dZ[MP][LP], T2[MP][LP], Zk[MP][LP], X[MP][LP], T1[MP][LP], dT2[MP][LP],
      dX[MP][LP];
  float col[MP], row[MP], red[16];
};

// C = op(P) op(Q) on MP x MP LDS matrices (pitch MP + 4), where op(P) =
// pa * P' + pb * I on the first m diagonal entries (P' = P or P^T) and the
// same for Q.  Computed by the NQ = (MP/32)^2 waves [w0, w0 + NQ) of the
// block, each one 32 x 32 quadrant as 2 x 2 tiles of 16 x 16, so that each
// operand row or column is read from LDS by NQ1 = MP/32 waves rather than
// by every tile; the other waves return at once (the test is wave-uniform,
// so every matrix-core instruction runs on whole waves).  Lane (c, g) of a
// tile gets rows row0 + 4g + i, column col + c, and epi(t, row0, col, v)
// receives them, t = 2 * (tile row) + (tile column) within the quadrant.
template <int MP>
struct LandTiles {
  static constexpr int NQ1 = MP / 32, NQ = NQ1 * NQ1;     // quadrant waves per product
  static constexpr int NTH = MP == 64 ? 512 : 256, NW = NTH / 64;  // two products at once
};

template <int MP, int PR, bool TPa, bool TQa, typename Epi>
__device__ __forceinline__ void land_mm(int w0, const float (*Pm)[MP + 4], float pa, float pb,
                                        const float (*Qm)[MP + 4], float qa, float qb, int m, Epi epi) {
  constexpr int NQ1 = LandTiles<MP>::NQ1, NQ = LandTiles<MP>::NQ;
  const int lane = threadIdx.x & 63, qw = (int)(threadIdx.x >> 6) - w0;
  if (qw < 0 || qw >= NQ) return;
  const int c = lane & 15, g = lane >> 4;
  const int bi = (qw / NQ1) * 32, bj = (qw % NQ1) * 32;
  f32x4_t acc[2][2];
#pragma unroll
  for (int si = 0; si < 2; ++si)
#pragma unroll
    for (int sj = 0; sj < 2; ++sj) acc[si][sj] = zero4();
#pragma unroll 1
  for (int kc = 0; kc < MP; kc += 32) {
    float a[2][8], b[2][8];
#pragma unroll
    for (int sx = 0; sx < 2; ++sx) {
      const int i = bi + 16 * sx + c, j = bj + 16 * sx + c;
      // Row-contiguous operands (P untransposed, Q transposed) are read as
      // two 16-byte vectors; the others one element per k.
      float pv[8], qv[8];
      if constexpr (!TPa) {
        const float4 u0 = *reinterpret_cast<const float4*>(&Pm[i][kc + 8 * g]);
        const float4 u1 = *reinterpret_cast<const float4*>(&Pm[i][kc + 8 * g + 4]);
        pv[0] = u0.x; pv[1] = u0.y; pv[2] = u0.z; pv[3] = u0.w;
        pv[4] = u1.x; pv[5] = u1.y; pv[6] = u1.z; pv[7] = u1.w;
      } else {
#pragma unroll
        for (int u = 0; u < 8; ++u) pv[u] = Pm[kc + 8 * g + u][i];
      }
      if constexpr (TQa) {
        const float4 u0 = *reinterpret_cast<const float4*>(&Qm[j][kc + 8 * g]);
        const float4 u1 = *reinterpret_cast<const float4*>(&Qm[j][kc + 8 * g + 4]);
        qv[0] = u0.x; qv[1] = u0.y; qv[2] = u0.z; qv[3] = u0.w;
        qv[4] = u1.x; qv[5] = u1.y; qv[6] = u1.z; qv[7] = u1.w;
      } else {
#pragma unroll
        for (int u = 0; u < 8; ++u) qv[u] = Qm[kc + 8 * g + u][j];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = kc + 8 * g + u;
        a[sx][u] = pa * pv[u] + ((i == k && k < m) ? pb : 0.f);
        b[sx][u] = qa * qv[u] + ((k == j && k < m) ? qb : 0.f);
      }
    }
#pragma unroll
    for (int si = 0; si < 2; ++si)
#pragma unroll
      for (int sj = 0; sj < 2; ++sj) acc[si][sj] = mma_f32<PR>(a[si], b[sj], acc[si][sj]);
  }
#pragma unroll
  for (int si = 0; si < 2; ++si)
#pragma unroll
    for (int sj = 0; sj < 2; ++sj) epi(2 * si + sj, bi + 16 * si + 4 * g, bj + 16 * sj + c, acc[si][sj]);
}

template <int MP, int PR>
__device__ __forceinline__ void land_body(const float* __restrict__ Qt, const float* __restrict__ Kt,
                                          const float* __restrict__ Aw, const float* __restrict__ BV,
                                          const float* __restrict__ dWg, float* __restrict__ dKt,
                                          float* __restrict__ dQtA, const float* __restrict__ zs, int m, int D,
                                          int iters, float scale, int bh, unsigned char* smem_raw) {
  LandSmem<MP>& sm = *reinterpret_cast<LandSmem<MP>*>(smem_raw);
  using Mat = float (*)[MP + 4];
  constexpr int NTH = LandTiles<MP>::NTH, NQ = LandTiles<MP>::NQ;
  const int tid = threadIdx.x;
  const size_t md = (size_t)bh * m * D, mm = (size_t)bh * m * m;

  constexpr int ZPT = MP * MP / NTH;  // entries e = tid + NTH * q of an MP x MP matrix
  // A (zero padded), and dZ = dW BV^T (dW is the sum of the query-side
  // partials) on the matrix cores over MP-feature slices staged in LDS (the
  // T1 and dT2 slots are free until the iterates): T1[i][cc] = dW[i][c0 +
  // cc], dT2[j][cc] = BV[j][c0 + cc], zero padded.  A and the first slice
  // are loaded together.
  {
    float ar[ZPT], wr[ZPT], br[ZPT];
    auto slice = [&](int c0) {
#pragma unroll
      for (int q = 0; q < ZPT; ++q) {
        const int e = tid + NTH * q, i = e / MP, cc = e % MP;
        const bool in = i < m && c0 + cc < D;
        wr[q] = in ? dWg[md + (size_t)i * D + c0 + cc] : 0.f;
        br[q] = in ? BV[md + (size_t)i * D + c0 + cc] : 0.f;
      }
    };
#pragma unroll
    for (int q = 0; q < ZPT; ++q) {
      const int e = tid + NTH * q, i = e / MP, j = e % MP;
      ar[q] = (i < m && j < m) ? Aw[mm + i * m + j] : 0.f;
    }
    slice(0);
#pragma unroll
    for (int q = 0; q < ZPT; ++q) {
      const int e = tid + NTH * q;
      sm.A[e / MP][e % MP] = ar[q];
    }
    for (int c0 = 0; c0 < D; c0 += MP) {
      if (c0 > 0) {
        __syncthreads();
        slice(c0);
      }
#pragma unroll
      for (int q = 0; q < ZPT; ++q) {
        const int e = tid + NTH * q;
        sm.T1[e / MP][e % MP] = wr[q];
        sm.dT2[e / MP][e % MP] = br[q];
      }
      __syncthreads();
      land_mm<MP, PR, false, true>(0, sm.T1, 1.f, 0.f, sm.dT2, 1.f, 0.f, m, [&](int, int r0, int cc, const f32x4_t& v) {
        for (int i = 0; i < 4; ++i) sm.dZ[r0 + i][cc] = (c0 == 0 ? 0.f : sm.dZ[r0 + i][cc]) + v[i];
      });
    }
  }
  __syncthreads();

  // Start Z0 = c A^T; column and row sums of A (entries are positive), one
  // wave per row and column, lane = the summed index.
  const int lane = tid & 63, wave = tid >> 6;
  for (int r = wave; r < MP; r += NTH / 64) {
    float rs = lane < MP ? sm.A[r][lane] : 0.f, cs = lane < MP ? sm.A[lane][r] : 0.f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      rs += shfl_xor(rs, o);
      cs += shfl_xor(cs, o);
    }
    if (lane == 0) {
      sm.row[r] = rs;
      sm.col[r] = cs;
    }
  }
  __syncthreads();
  // n1 = the largest column sum (first maximiser jstar), ninf = the largest row sum.
  if (wave == 0) {
    float cv = lane < m ? sm.col[lane] : -1.f, rv = lane < m ? sm.row[lane] : 0.f;
    int ci = lane;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float ov = shfl_xor(cv, o);
      const int oi = __shfl_xor(ci, o, 64);
      if (ov > cv || (ov == cv && oi < ci)) {
        cv = ov;
        ci = oi;
      }
      rv = fmaxf(rv, shfl_xor(rv, o));
    }
    if (lane == 0) {
      sm.red[0] = cv;
      sm.red[1] = rv;
      sm.red[2] = __int_as_float(ci);
    }
  }
  __syncthreads();
  const float n1 = sm.red[0], ninf = sm.red[1];
  const int jstar = __float_as_int(sm.red[2]);
  const float cz = 1.f / (n1 * ninf);
  const float* zsh = zs + (size_t)bh * iters * 4 * MP * MP;

  // The forward steps Z_k, X_k, T1_k = X_k (7I - X_k), T2_k = X_k (15I -
  // T1_k) for k < iters were saved to zs by the forward's pseudoinverse
  // kernel (recomputed at the start of the call); the reverse pass reads them.
  const size_t MM2 = (size_t)MP * MP;
  for (int e = tid; e < MP * MP; e += NTH) sm.dA[e / MP][e % MP] = 0.f;
  __syncthreads();

  // Reverse through the steps, four dependency levels of two independent
  // products each, one barrier per level.  dZ and three free slots rotate
  // among the dZ, T2, dT2 and dX slots (fa receives T2_k, fb and fc the
  // level-1 results, the old dZ slot dX).
  Mat dZ = sm.dZ, fa = sm.T2, fb = sm.dT2, fc = sm.dX;
  // Z_k, X_k, T1_k, T2_k of step k, read one step ahead into registers.
  float zr[4][ZPT];

  auto zfetch = [&](int k) {
#pragma unroll
    for (int q = 0; q < ZPT; ++q)
#pragma unroll
      for (int t = 0; t < 4; ++t) zr[t][q] = zsh[((size_t)k * 4 + t) * MM2 + tid + NTH * q];
  };
  if (iters > 0) zfetch(iters - 1);
  for (int k = iters - 1; k >= 0; --k) {
#pragma unroll
    for (int q = 0; q < ZPT; ++q) {
      const int e = tid + NTH * q, i = e / MP, j = e % MP;
      sm.Zk[i][j] = zr[0][q];
      sm.X[i][j] = zr[1][q];
      sm.T1[i][j] = zr[2][q];
      fa[i][j] = zr[3][q];
    }
    __syncthreads();
    if (k > 0) zfetch(k - 1);
    // Level 1: dT2 = -Z_k^T dZ / 4 -> fb;  dZ_k = dZ (13I - T2)^T / 4 -> fc.
    land_mm<MP, PR, true, false>(0, sm.Zk, -0.25f, 0.f, dZ, 1.f, 0.f, m, [&](int, int r0, int cc, const f32x4_t& v) {
      for (int i = 0; i < 4; ++i) fb[r0 + i][cc] = v[i];
    });
    land_mm<MP, PR, false, true>(NQ, dZ, 0.25f, 0.f, fa, -1.f, 13.f, m, [&](int, int r0, int cc, const f32x4_t& v) {
      for (int i = 0; i < 4; ++i) fc[r0 + i][cc] = v[i];
    });
    __syncthreads();
    // Level 2: dX = dT2 (15I - T1)^T -> the old dZ slot;  dT1 = -X^T dT2 -> fa.
    Mat dX = dZ;
    land_mm<MP, PR, false, true>(0, fb, 1.f, 0.f, sm.T1, -1.f, 15.f, m, [&](int, int r0, int cc, const f32x4_t& v) {
      for (int i = 0; i < 4; ++i) dX[r0 + i][cc] = v[i];
    });
    land_mm<MP, PR, true, false>(NQ, sm.X, -1.f, 0.f, fb, 1.f, 0.f, m, [&](int, int r0, int cc, const f32x4_t& v) {
      for (int i = 0; i < 4; ++i) fa[r0 + i][cc] = v[i];
    });
    __syncthreads();
    // Level 3: dX += dT1 (7I - X)^T - X^T dT1 (both products by the same
    // waves, the first kept in registers).
    {
      f32x4_t keep[4];
      land_mm<MP, PR, false, true>(0, fa, 1.f, 0.f, sm.X, -1.f, 7.f, m,
                                   [&](int q, int, int, const f32x4_t& v) { keep[q] = v; });
      land_mm<MP, PR, true, false>(0, sm.X, -1.f, 0.f, fa, 1.f, 0.f, m, [&](int q, int r0, int cc, const f32x4_t& v) {
        for (int i = 0; i < 4; ++i) dX[r0 + i][cc] += keep[q][i] + v[i];
      });
    }
    __syncthreads();
    // Level 4: dA += dX Z_k^T;  dZ_k += A^T dX.
    land_mm<MP, PR, false, true>(0, dX, 1.f, 0.f, sm.Zk, 1.f, 0.f, m, [&](int, int r0, int cc, const f32x4_t& v) {
      for (int i = 0; i < 4; ++i) sm.dA[r0 + i][cc] += v[i];
    });
    land_mm<MP, PR, true, false>(NQ, sm.A, 1.f, 0.f, dX, 1.f, 0.f, m, [&](int, int r0, int cc, const f32x4_t& v) {
      for (int i = 0; i < 4; ++i) fc[r0 + i][cc] += v[i];
    });
    __syncthreads();
    // dZ_k becomes the incoming gradient of the next (earlier) step.
    Mat old_dz = dZ;
    dZ = fc;
    fc = old_dz;
  }

  // The first feature slice of Kt, Qt and dKt for the end, in flight while
  // the start's gradient and the softmax backward run.
  float er[3][ZPT];
  auto efetch = [&]() {
#pragma unroll
    for (int q = 0; q < ZPT; ++q) {
      const int e = tid + NTH * q, k = e / MP, cc = e % MP;
      const bool in = k < m && cc < D;
      er[0][q] = in ? Kt[md + (size_t)k * D + cc] : 0.f;
      er[1][q] = in ? Qt[md + (size_t)k * D + cc] : 0.f;
      er[2][q] = in ? dKt[md + (size_t)k * D + cc] : 0.f;
    }
  };
  efetch();

  // The start Z0 = cz A^T: dA += cz dZ^T, and through cz = 1/(n1 ninf):
  // dcz = sum dZ * A^T; n1 = column sum jstar adds -dcz cz / n1 to column
  // jstar.  The ninf term is constant along a row and cancels in the softmax
  // backward below, so it is left out.
  float part = 0.f;
  for (int e = tid; e < MP * MP; e += NTH) {
    const int i = e / MP, j = e % MP;
    part = fmaf(dZ[i][j], sm.A[j][i], part);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) part += shfl_xor(part, o);
  if ((tid & 63) == 0) sm.red[tid >> 6] = part;
  __syncthreads();
  float dcz = 0.f;
  for (int w = 0; w < LandTiles<MP>::NW; ++w) dcz += sm.red[w];
  for (int e = tid; e < MP * MP; e += NTH) {
    const int i = e / MP, j = e % MP;
    if (i < m && j < m) sm.dA[i][j] += cz * dZ[j][i] + (j == jstar ? -dcz * cz / n1 : 0.f);
  }
  __syncthreads();
  // dS_A = A * (dA - rowsum(dA * A)), in place of dA; one wave per row.
  for (int r = wave; r < MP; r += NTH / 64) {
    float v = lane < MP ? sm.dA[r][lane] * sm.A[r][lane] : 0.f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v += shfl_xor(v, o);
    if (lane == 0) sm.row[r] = v;
  }
  __syncthreads();
  for (int e = tid; e < MP * MP; e += NTH) {
    const int i = e / MP, j = e % MP;
    sm.dA[i][j] = sm.A[i][j] * (sm.dA[i][j] - sm.row[i]);
  }
  // dQt_A = s dS_A Kt;  dKt += s dS_A^T Qt, on the matrix cores over
  // MP-feature slices of Kt and Qt staged in the T1 and dT2 slots, dKt's
  // values so far in the Zk slot (the first slice was read during the last
  // step).
  for (int c0 = 0; c0 < D; c0 += MP) {
    if (c0 > 0) {
#pragma unroll
      for (int q = 0; q < ZPT; ++q) {
        const int e = tid + NTH * q, k = e / MP, cc = e % MP;
        const bool in = k < m && c0 + cc < D;
        er[0][q] = in ? Kt[md + (size_t)k * D + c0 + cc] : 0.f;
        er[1][q] = in ? Qt[md + (size_t)k * D + c0 + cc] : 0.f;
        er[2][q] = in ? dKt[md + (size_t)k * D + c0 + cc] : 0.f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < ZPT; ++q) {
      const int e = tid + NTH * q, k = e / MP, cc = e % MP;
      sm.T1[k][cc] = er[0][q];
      sm.dT2[k][cc] = er[1][q];
      sm.Zk[k][cc] = er[2][q];
    }
    __syncthreads();
    land_mm<MP, PR, false, false>(0, sm.dA, 1.f, 0.f, sm.T1, 1.f, 0.f, m, [&](int, int r0, int cc, const f32x4_t& v) {
      if (c0 + cc < D)
        for (int i = 0; i < 4; ++i)
          if (r0 + i < m) dQtA[md + (size_t)(r0 + i) * D + c0 + cc] = scale * v[i];
    });
    land_mm<MP, PR, true, false>(NQ, sm.dA, 1.f, 0.f, sm.dT2, 1.f, 0.f, m, [&](int, int r0, int cc, const f32x4_t& v) {
      if (c0 + cc < D)
        for (int i = 0; i < 4; ++i)
          if (r0 + i < m) dKt[md + (size_t)(r0 + i) * D + c0 + cc] = sm.Zk[r0 + i][cc] + scale * v[i];
    });
  }
}

// ---------------------------------------------------------------------------
// Key side.  Grid (chunks, batch*heads); tiles of 16 keys with a halo of R =
// (conv_k - 1)/2 rows of V and dO for the skip.  Per key i (16 lanes,
// landmarks jl + 16u):
//   B_:i = 2^(s' Qt K_i - M) / L (the forward's row statistics of B),
//   dB_:i = dBV V_i, dS_:i = B_:i * (dB_:i - delta), delta_j = dBV_j . BV_j.
// Writes dK_i = s dS_:i^T Qt + dKt[seg(i)] / l and dV_i = B_:i^T dBV +
// DConv^T(dO)_i; partials of dQt_B = s sum_i dS_:i K_i and of the filter
// gradient dw[c][t] = sum_i dO[i][c] V[i + t - R][c].
template <typename IO, int D>
__global__ __launch_bounds__(256) void k_bwd_key(const typename IO::T* __restrict__ K,
                                                 const typename IO::T* __restrict__ V,
                                                 const typename IO::T* __restrict__ dO,
                                                 const float* __restrict__ conv_w, const float* __restrict__ Qt,
                                                 const float* __restrict__ BV, const float* __restrict__ dBVg,
                                                 const float* __restrict__ dKt, const float* __restrict__ pmax,
                                                 const float* __restrict__ psum, typename IO::T* __restrict__ dK,
                                                 typename IO::T* __restrict__ dV, float* __restrict__ pdqt,
                                                 float* __restrict__ pdwc, const int* __restrict__ lens, int n,
                                                 int m, int heads, int conv_k, int chunk, int nchunks, int fchunks,
                                                 float sl2e, float scale) {
  constexpr int P = D + 1;
  constexpr int NE = 64 * D / 256;
  const int R = conv_k > 0 ? (conv_k - 1) / 2 : 0;
  const int HR = kKeyTile + 2 * R;  // rows of the V / dO tiles
  extern __shared__ __align__(16) float lds[];
  float* qt = lds;                     // [64][P]  Qt (unscaled)
  float* db = qt + 64 * P;             // [64][P]  dBV
  float* kk = db + 64 * P;             // [kKeyTile][P]
  float* vv = kk + kKeyTile * P;       // [HR][P]
  float* gg = vv + 48 * P;             // [HR][P]
  float* bs = gg + 48 * P;             // [kKeyTile][65]
  float* dss = bs + kKeyTile * 65;     // [kKeyTile][65]
  float* stm = dss + kKeyTile * 65;    // [64] M
  float* stl = stm + 64;               // [64] 1/L
  float* dlt = stl + 64;               // [64] delta
  float* wsh = dlt + 64;               // [D][conv_k]
  const int tid = threadIdx.x, ch = blockIdx.x, bh = blockIdx.y, h = bh % heads;
  const size_t hoff = (size_t)bh * n * D, md = (size_t)bh * m * D;

  for (int e = tid; e < 64 * D; e += 256) {
    const int j = e / D, c = e % D;
    qt[j * P + c] = j < m ? Qt[md + e] : 0.f;
    db[j * P + c] = j < m ? dBVg[md + e] : 0.f;
  }
  for (int e = tid; e < D * conv_k; e += 256) wsh[e] = conv_w[(size_t)h * D * conv_k + e];
  if (tid < 64) {
    // Row statistics of B from the forward's split-n partials (same fixed
    // order as its finish) and delta_j = dBV_j . BV_j.
    const int j = tid;
    float M = -INFINITY, L = 0.f, dl = 0.f;
    if (j < m) {
      for (int c = 0; c < fchunks; ++c) M = fmaxf(M, pmax[((size_t)bh * fchunks + c) * m + j]);
      for (int c = 0; c < fchunks; ++c) {
        const float pm = pmax[((size_t)bh * fchunks + c) * m + j];
        if (pm != -INFINITY) L += psum[((size_t)bh * fchunks + c) * m + j] * exp2f(pm - M);
      }
      for (int c = 0; c < D; ++c) dl = fmaf(dBVg[md + (size_t)j * D + c], BV[md + (size_t)j * D + c], dl);
    }
    stm[j] = M;
    stl[j] = j < m ? 1.f / L : 0.f;
    dlt[j] = dl;
  }
  float aq[NE];
#pragma unroll
  for (int v = 0; v < NE; ++v) aq[v] = 0.f;
  float awc[17];  // filter-gradient entries tid + 256 v (d * conv_k <= 128 * 33)
#pragma unroll
  for (int v = 0; v < 17; ++v) awc[v] = 0.f;
  // Keys of the sequence; V and dO rows past them read as zero in the skip.
  const int nb = seq_rows(lens, bh / heads, n);
  const int seg = max(1, (nb + m - 1) / m);
  const float inv_seg = 1.f / (float)seg;
  const int r = tid >> 4, jl = tid & 15;

  const int kbeg = ch * chunk, kend = min(nb, kbeg + chunk);
  for (int i0 = kbeg; i0 < kend; i0 += kKeyTile) {
    __syncthreads();
    for (int e = tid; e < kKeyTile * D; e += 256) {
      const int rr = e / D, c = e % D, row = i0 + rr;
      kk[rr * P + c] = row < kend ? ld<IO>(K + hoff + (size_t)row * D + c) : 0.f;
    }
    for (int e = tid; e < HR * D; e += 256) {
      const int rr = e / D, c = e % D, row = i0 - R + rr;
      const bool in = row >= 0 && row < nb;
      vv[rr * P + c] = in ? ld<IO>(V + hoff + (size_t)row * D + c) : 0.f;
      gg[rr * P + c] = in ? ld<IO>(dO + hoff + (size_t)row * D + c) : 0.f;
    }
    __syncthreads();

    float sc[4], dbv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) sc[u] = dbv[u] = 0.f;
    for (int k = 0; k < D; ++k) {
      const float kv = kk[r * P + k], vk = vv[(R + r) * P + k];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        sc[u] = fmaf(kv, qt[(jl + 16 * u) * P + k], sc[u]);
        dbv[u] = fmaf(vk, db[(jl + 16 * u) * P + k], dbv[u]);
      }
    }
    const bool live = i0 + r < kend;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = jl + 16 * u;
      const float b = (live && j < m) ? exp2f(sc[u] * sl2e - stm[j]) * stl[j] : 0.f;
      bs[r * 65 + j] = b;
      dss[r * 65 + j] = b * (dbv[u] - dlt[j]);
    }
    __syncthreads();

    {
      const int row = i0 + r;
      if (row < kend) {
        const float* ktr = dKt + md + (size_t)(row / seg) * D;
        for (int c = jl; c < D; c += 16) {
          float a = 0.f, b = 0.f;
          for (int j = 0; j < m; ++j) {
            a = fmaf(dss[r * 65 + j], qt[j * P + c], a);
            b = fmaf(bs[r * 65 + j], db[j * P + c], b);
          }
          // Skip transpose: dV[i][c] += sum_t w[c][t] dO[i - t + R][c].
          for (int t = 0; t < conv_k; ++t) b = fmaf(wsh[c * conv_k + t], gg[(r - t + 2 * R) * P + c], b);
          store_elem<IO>(dK + hoff + (size_t)row * D + c, fmaf(scale, a, ktr[c] * inv_seg));
          store_elem<IO>(dV + hoff + (size_t)row * D + c, b);
        }
      }
    }
#pragma unroll
    for (int v = 0; v < NE; ++v) {
      const int e = tid + 256 * v, j = e / D, c = e % D;
      float a = aq[v];
#pragma unroll 4
      for (int rr = 0; rr < kKeyTile; ++rr) a = fmaf(dss[rr * 65 + j], kk[rr * P + c], a);
      aq[v] = a;
    }
#pragma unroll
    for (int v = 0; v < 17; ++v) {
      const int e = tid + 256 * v;
      if (e < D * conv_k) {
        const int c = e / conv_k, t = e % conv_k;
        float a = awc[v];
#pragma unroll 4
        for (int rr = 0; rr < kKeyTile; ++rr)
          if (i0 + rr < kend) a = fmaf(gg[(R + rr) * P + c], vv[(rr + t) * P + c], a);
        awc[v] = a;
      }
    }
  }
  {
    const size_t base = ((size_t)bh * nchunks + ch) * m * D;
#pragma unroll
    for (int v = 0; v < NE; ++v) {
      const int e = tid + 256 * v, j = e / D;
      if (j < m) pdqt[base + e] = scale * aq[v];
    }
    const size_t wb = ((size_t)bh * nchunks + ch) * D * conv_k;
#pragma unroll
    for (int v = 0; v < 17; ++v) {
      const int e = tid + 256 * v;
      if (e < D * conv_k) pdwc[wb + e] = awc[v];
    }
  }
}

// ---------------------------------------------------------------------------
// Matrix-core versions of the n-sized passes for bf16 I/O at d = 32 or 64
// (single bf16 products with fp32 accumulation, as in the forward's output
// stage).  Matrix-core convention of nys_common.hpp: lane (c, g) holds
// A[c][8g..8g+7], B[8g..8g+7][c] and C[4g..4g+3][c].  Score-type products
// are computed transposed (landmarks x rows) so that a lane holds 16
// landmarks of one row; such a C tile is the B operand of the next product
// when the landmark axis is taken, within each chunk of 32, in the order
// {4g..4g+3, 16+4g..16+4g+3}; the A operands of those products are stored
// in LDS in that order (mm_slot).

constexpr int kMmTile = 64;  // rows (keys or queries) per tile, 16 per wave

// Position of landmark j in the permuted order of its chunk of 32.
__device__ __forceinline__ int mm_slot(int j) {
  const int jj = j & 31;
  return (j & ~31) + 8 * ((jj & 15) >> 2) + (jj & 3) + ((jj & 16) ? 4 : 0);
}

__device__ __forceinline__ uint16_t bf(float x) { return f32_to_bf16(x); }

__device__ __forceinline__ B8 lds8(const uint16_t* p) {
  B8 b;
  b.q = *reinterpret_cast<const uint4*>(p);
  return b;
}

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

// B operand of a 16x16x32 product, M[kb + 8g + u][nb + c] for lane (c, g),
// read from a row-major bf16 tile in LDS (pitch PD) with two transpose reads:
// in each group of 16 lanes, lane j gives the address of 4 consecutive
// elements of row kb + 8g + j/4 (+ 4 for the second read), columns
// nb + 4(j % 4) .. +3, and lane i of the group receives column nb + i of
// the four rows the group read.
template <int PD>
__device__ __forceinline__ B8 tr_b(const uint16_t (*M)[PD], int kb, int nb) {
  const int lane = threadIdx.x & 63, g = lane >> 4, j = lane & 15;
  const uint16_t* p0 = &M[kb + 8 * g + (j >> 2)][nb + 4 * (j & 3)];
  const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(p0));
  const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(p0 + 4 * PD));
  const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
  B8 b;
  b.u[0] = l2.x;
  b.u[1] = l2.y;
  b.u[2] = h2.x;
  b.u[3] = h2.y;
  return b;
}

// C-layout values of landmark tiles 2kk and 2kk+1 as a B operand.
__device__ __forceinline__ B8 pack_b(const f32x4_t& lo, const f32x4_t& hi) {
  B8 b;
  b.u[0] = pack_bf16x2(lo[0], lo[1]);
  b.u[1] = pack_bf16x2(lo[2], lo[3]);
  b.u[2] = pack_bf16x2(hi[0], hi[1]);
  b.u[3] = pack_bf16x2(hi[2], hi[3]);
  return b;
}

// The skip's filter gradient on the matrix-core path: partials over a chunk
// of rows of dw[f][t] = sum_i dO[i][f] V[i + t - 16][f], a filter of
// conv_k <= 33 taps centred in 33 (offset off).  Tiles of 64 rows with a
// 16-row halo of V; thread (f, rg) owns feature f and rows rg*16 ..
// rg*16 + 15 of each tile, holds those 16 dO values and the 48 V values they
// pair with in registers and accumulates all 33 taps there; the four row
// groups are summed in LDS (fixed-order tree) after the last tile.  Grid
// (chunks, batch*heads), 4*D threads.
template <int D>
struct SkipSmem {
  static constexpr int PD = D + 8, HR = kMmTile + 32;
  uint16_t vh[HR][PD];       // V rows with the halo
  uint16_t gh[kMmTile][PD];  // dO rows of the tile
};

template <int D>
__global__ __launch_bounds__(4 * D) void k_bwd_skip_grad(const uint16_t* __restrict__ V,
                                                         const uint16_t* __restrict__ dO, float* __restrict__ pdwc,
                                                         const int* __restrict__ lens, int heads, int n, int conv_k,
                                                         int chunk, int nchunks) {
  using SM = SkipSmem<D>;
  constexpr int NTH = 4 * D, KPT = 16, RG = 4, WN = KPT + 32;
  constexpr int NV = SM::HR * (D / 8) / NTH, NG = kMmTile * (D / 8) / NTH;
  static_assert(KPT * RG == kMmTile && NV * NTH == SM::HR * (D / 8) && NG * NTH == kMmTile * (D / 8), "tiling");
  static_assert((RG / 2) * D * 33 * 4 <= (int)sizeof(SM), "tap-sum scratch");
  extern __shared__ __align__(16) unsigned char smem_raw[];
  SM& sm = *reinterpret_cast<SM*>(smem_raw);
  const int tid = threadIdx.x, f = tid % D, rg = tid / D, r0 = rg * KPT;
  const int ch = blockIdx.x, bh = blockIdx.y;
  const size_t hoff = (size_t)bh * n * D;
  float acc[33];
#pragma unroll
  for (int t = 0; t < 33; ++t) acc[t] = 0.f;

  // Rows of the sequence: V rows past them read as zero, dO rows past them
  // are not output rows.
  const int nb = seq_rows(lens, bh / heads, n);
  const int kbeg = ch * chunk, kend = min(nb, kbeg + chunk);
  // V rows (with the halo) and dO rows of a tile, 16 bytes per load; dO rows
  // past the chunk's end belong to the next chunk and read as zero.  The
  // next tile's are in flight while the current one is computed.
  uint4 vn[NV], gn[NG];
  auto fetch = [&](int t0) {
#pragma unroll
    for (int l = 0; l < NV; ++l) {
      const int e = tid + NTH * l, rr = e / (D / 8), c8 = (e % (D / 8)) * 8, row = t0 - 16 + rr;
      vn[l] = (row >= 0 && row < nb) ? *reinterpret_cast<const uint4*>(V + hoff + (size_t)row * D + c8)
                                    : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int l = 0; l < NG; ++l) {
      const int e = tid + NTH * l, rr = e / (D / 8), c8 = (e % (D / 8)) * 8, row = t0 + rr;
      gn[l] = row < kend ? *reinterpret_cast<const uint4*>(dO + hoff + (size_t)row * D + c8) : make_uint4(0, 0, 0, 0);
    }
  };
  fetch(kbeg);
  for (int i0 = kbeg; i0 < kend; i0 += kMmTile) {
    __syncthreads();
#pragma unroll
    for (int l = 0; l < NV; ++l) {
      const int e = tid + NTH * l;
      *reinterpret_cast<uint4*>(&sm.vh[e / (D / 8)][(e % (D / 8)) * 8]) = vn[l];
    }
#pragma unroll
    for (int l = 0; l < NG; ++l) {
      const int e = tid + NTH * l;
      *reinterpret_cast<uint4*>(&sm.gh[e / (D / 8)][(e % (D / 8)) * 8]) = gn[l];
    }
    __syncthreads();
    if (i0 + kMmTile < kend) fetch(i0 + kMmTile);
    // dO row r0 + u pairs with V row r0 + u + t - 16 (halo row r0 + u + t).
    float gw[KPT], vw[WN];
#pragma unroll
    for (int u = 0; u < KPT; ++u) gw[u] = bf16_to_f32(sm.gh[r0 + u][f]);
#pragma unroll
    for (int p = 0; p < WN; ++p) vw[p] = bf16_to_f32(sm.vh[r0 + p][f]);
#pragma unroll
    for (int u = 0; u < KPT; ++u)
#pragma unroll
      for (int t = 0; t < 33; ++t) acc[t] = fmaf(gw[u], vw[u + t], acc[t]);
  }
  // Sum the row groups' taps: group rg + half hands its sums to group rg.
  float* red = reinterpret_cast<float*>(smem_raw);  // [RG / 2][D][33]
#pragma unroll
  for (int half = RG / 2; half >= 1; half /= 2) {
    __syncthreads();
    if (rg >= half && rg < 2 * half) {
#pragma unroll
      for (int t = 0; t < 33; ++t) red[((rg - half) * D + f) * 33 + t] = acc[t];
    }
    __syncthreads();
    if (rg < half) {
#pragma unroll
      for (int t = 0; t < 33; ++t) acc[t] += red[(rg * D + f) * 33 + t];
    }
  }
  if (rg == 0) {
    const int off = (33 - conv_k) / 2;
    const size_t wb = ((size_t)bh * nchunks + ch) * D * conv_k;
#pragma unroll
    for (int t = 0; t < 33; ++t) {
      const int tt = t - off;  // tap of the conv_k-tap filter
      if (tt >= 0 && tt < conv_k) pdwc[wb + (size_t)f * conv_k + tt] = acc[t];
    }
  }
}

// Filters with their taps reversed: the transposed depthwise convolution
// DConv^T(dO)[i] = sum_t w[t] dO[i - t + R] is the convolution of dO with
// the reversed filter.  One thread per tap.
__global__ __launch_bounds__(256) void k_flip_taps(const float* __restrict__ w, float* __restrict__ wf, int k,
                                                   int total) {
  const int e = blockIdx.x * 256 + (int)threadIdx.x;
  if (e >= total) return;
  const int t = e % k;
  wf[e] = w[e - t + (k - 1 - t)];
}

// Fixed-order sums over chunks of p[ch * stride] and p2[ch * stride] (p2
// may be null), 24 chunks' loads of both in flight at a time (the loads past
// the last chunk read nothing and add zero, which leaves the sums' bits
// unchanged).
__device__ __forceinline__ void chunk_sum2(const float* __restrict__ p, const float* __restrict__ p2, size_t stride,
                                           int nchunks, float& a, float& a2) {
  constexpr int NB = 24;
  for (int ch = 0; ch < nchunks; ch += NB) {
    float x[NB], y[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const bool in = ch + u < nchunks;
      x[u] = in ? p[(size_t)(ch + u) * stride] : 0.f;
      y[u] = (in && p2) ? p2[(size_t)(ch + u) * stride] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      a += x[u];
      a2 += y[u];
    }
  }
}

__device__ __forceinline__ float chunk_sum(const float* __restrict__ p, size_t stride, int nchunks, float a) {
  float unused = 0.f;
  chunk_sum2(p, nullptr, stride, nchunks, a, unused);
  return a;
}

// dW = sum of the query-side partials of F^T dO, dKt_F likewise (fixed chunk
// order), and dBV = Z^T dW.  Grid (D / 16, batch*heads), 1024 threads;
// thread (j, cl) owns landmark j and feature 16 * blockIdx.x + cl.  The key
// side needs only dBV, so it can start before the pseudoinverse backward.
__global__ __launch_bounds__(1024) void k_bwd_land_prep(const float* __restrict__ Zw, const float* __restrict__ pdw,
                                                        const float* __restrict__ pdkt, float* __restrict__ dWg,
                                                        float* __restrict__ dKt, float* __restrict__ dBV, int m, int D,
                                                        int nchunks) {
  __shared__ float zl[64][65];
  __shared__ float wl[64][17];
  const int tid = threadIdx.x, bh = blockIdx.y, c0 = blockIdx.x * 16;
  const int j = tid >> 4, cl = tid & 15;
  const size_t md = (size_t)bh * m * D, mm = (size_t)bh * m * m, stride = (size_t)m * D;
  // Z's loads and the partials' are in flight together.
  float zr[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid + 1024 * q, r = e / 64, cc = e % 64;
    zr[q] = (r < m && cc < m) ? Zw[mm + (size_t)r * m + cc] : 0.f;
  }
  float a = 0.f, k = 0.f;
  if (j < m) {
    const size_t o = (size_t)bh * nchunks * stride + (size_t)j * D + c0 + cl;
    chunk_sum2(pdw + o, pdkt + o, stride, nchunks, a, k);
    dWg[md + (size_t)j * D + c0 + cl] = a;
    dKt[md + (size_t)j * D + c0 + cl] = k;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int e = tid + 1024 * q;
    zl[e / 64][e % 64] = zr[q];
  }
  wl[j][cl] = a;
  __syncthreads();
  if (j < m) {
    float b = 0.f;
#pragma unroll 8
    for (int i = 0; i < 64; ++i) b = fmaf(zl[i][j], wl[i][cl], b);  // rows past m are zero
    dBV[md + (size_t)j * D + c0 + cl] = b;
  }
}

// Landmark side: one block per (batch, head).
struct LandArgs {
  const float *Qt, *Kt, *Aw, *BV, *dWg;
  float *dKt, *dQtA;
  const float* zs;
  int m, D, iters;
  float scale;
};

template <int MP, int PR>
__global__ __launch_bounds__(LandTiles<MP>::NTH) void k_bwd_land(LandArgs a) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  land_body<MP, PR>(a.Qt, a.Kt, a.Aw, a.BV, a.dWg, a.dKt, a.dQtA, a.zs, a.m, a.D, a.iters, a.scale,
                    (int)blockIdx.x, smem_raw);
}

template <int D>
struct KeyMmSmem {
  static constexpr int PD = D + 8, PK = 64 + 8;
  uint16_t qa[64][PD];       // Qt * log2(e)/sqrt(d), landmark rows (A of the scores)
  uint16_t da[64][PD];       // dBV rows (A of dB)
  uint16_t qT[D][PK];        // Qt^T, landmarks in mm_slot order (A of dK^T)
  uint16_t dT[D][PK];        // dBV^T, mm_slot order (A of dV^T)
  uint16_t kr[kMmTile][PD];  // key rows of the tile (also B of dQt, read transposed)
  uint16_t vr[kMmTile][PD];  // V rows of the tile
  uint16_t sT[64][PK];       // dS^T of the tile (A of dQt)
  float stm[64], stl[64], dlt[64];
};

// Writes dK without the landmark term seg^T dKt (the dQ pass adds it once the
// pseudoinverse backward, which runs beside this kernel, has produced dKt).
// skip_in_dv: dV already holds the skip's part (the transposed convolution,
// written earlier on the same stream) and the attention part is added to it.
template <int D>
__global__ __launch_bounds__(256) void k_bwd_key_mm(const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
                                                    const float* __restrict__ Qt, const float* __restrict__ BV,
                                                    const float* __restrict__ dBVg, const float* __restrict__ pmax, const float* __restrict__ psum,
                                                    uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
                                                    float* __restrict__ pdqt, const int* __restrict__ lens, int heads,
                                                    int n, int m, int skip_in_dv, int chunk, int nchunks, int fchunks,
                                                    float sl2e, float scale) {
  using SM = KeyMmSmem<D>;
  constexpr int KC = D / 32, ND = D / 16, PER = ND;  // dQt tiles per wave: 4 * ND / 4
  extern __shared__ __align__(16) unsigned char smem_raw[];
  SM& sm = *reinterpret_cast<SM*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c = lane & 15, g = lane >> 4;
  const int ch = blockIdx.x, bh = blockIdx.y;
  const size_t hoff = (size_t)bh * n * D, md = (size_t)bh * m * D;

  for (int e = tid; e < 64 * D; e += 256) {
    const int j = e / D, f = e % D;
    const float q = j < m ? Qt[md + e] : 0.f, db = j < m ? dBVg[md + e] : 0.f;
    sm.qa[j][f] = bf(q * sl2e);
    sm.da[j][f] = bf(db);
    sm.qT[f][mm_slot(j)] = bf(q);
    sm.dT[f][mm_slot(j)] = bf(db);
  }
  if (tid < 64) {
    const int j = tid;
    float M = -INFINITY, L = 0.f, dl = 0.f;
    if (j < m) {
      for (int q = 0; q < fchunks; ++q) M = fmaxf(M, pmax[((size_t)bh * fchunks + q) * m + j]);
      for (int q = 0; q < fchunks; ++q) {
        const float pm = pmax[((size_t)bh * fchunks + q) * m + j];
        if (pm != -INFINITY) L += psum[((size_t)bh * fchunks + q) * m + j] * exp2f(pm - M);
      }
      for (int f = 0; f < D; ++f) dl = fmaf(dBVg[md + (size_t)j * D + f], BV[md + (size_t)j * D + f], dl);
    }
    sm.stm[j] = j < m ? M : 0.f;
    sm.stl[j] = j < m ? 1.f / L : 0.f;
    sm.dlt[j] = dl;
  }
  f32x4_t aq[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) aq[u] = zero4();

  const int kbeg = ch * chunk, kend = min(seq_rows(lens, bh / heads, n), kbeg + chunk);  // keys of the sequence
  // K and V rows of a tile, 16 bytes per load; the next tile's are in flight
  // while the current one is computed.
  constexpr int NL = kMmTile * (D / 8) / 256;
  uint4 kn[NL], vn[NL];
  auto fetch = [&](int t0) {
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      const int e = tid + 256 * l, rr = e / (D / 8), c8 = (e % (D / 8)) * 8, key = t0 + rr;
      const bool in = key < kend;
      kn[l] = in ? *reinterpret_cast<const uint4*>(K + hoff + (size_t)key * D + c8) : make_uint4(0, 0, 0, 0);
      vn[l] = in ? *reinterpret_cast<const uint4*>(V + hoff + (size_t)key * D + c8) : make_uint4(0, 0, 0, 0);
    }
  };
  fetch(kbeg);
  for (int i0 = kbeg; i0 < kend; i0 += kMmTile) {
    __syncthreads();
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      const int e = tid + 256 * l, rr = e / (D / 8), c8 = (e % (D / 8)) * 8;
      *reinterpret_cast<uint4*>(&sm.kr[rr][c8]) = kn[l];
      *reinterpret_cast<uint4*>(&sm.vr[rr][c8]) = vn[l];
    }
    __syncthreads();
    if (i0 + kMmTile < kend) fetch(i0 + kMmTile);

    // Scores S'^T and dB^T for this wave's 16 keys (key = i0 + 16 wave + c).
    const int kl = 16 * wave + c, key = i0 + kl;
    const bool live = key < kend;
    // The skip's part of dV for these keys, read now and added at the end.
    uint2 skp[ND];
#pragma unroll
    for (int nd = 0; nd < ND; ++nd)
      skp[nd] = (skip_in_dv && live) ? *reinterpret_cast<const uint2*>(dV + hoff + (size_t)key * D + nd * 16 + 4 * g)
                                     : make_uint2(0, 0);
    f32x4_t pb[4], ds[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4_t s = zero4(), db = zero4();
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const B8 kb = lds8(&sm.kr[kl][kc * 32 + 8 * g]);
        const B8 vb = lds8(&sm.vr[kl][kc * 32 + 8 * g]);
        s = mfma(lds8(&sm.qa[mt * 16 + c][kc * 32 + 8 * g]), kb, s);
        db = mfma(lds8(&sm.da[mt * 16 + c][kc * 32 + 8 * g]), vb, db);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = mt * 16 + 4 * g + i;
        const float b = (live && j < m) ? exp2f(s[i] - sm.stm[j]) * sm.stl[j] : 0.f;
        pb[mt][i] = b;
        ds[mt][i] = b * (db[i] - sm.dlt[j]);
      }
    }
    // dK^T = Qt^T dS^T and dV^T = dBV^T B^T (added to the skip's part).
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) {
      f32x4_t ak = zero4(), av = zero4();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        ak = mfma(lds8(&sm.qT[nd * 16 + c][kk * 32 + 8 * g]), pack_b(ds[2 * kk], ds[2 * kk + 1]), ak);
        av = mfma(lds8(&sm.dT[nd * 16 + c][kk * 32 + 8 * g]), pack_b(pb[2 * kk], pb[2 * kk + 1]), av);
      }
      if (live) {
        const int f0 = nd * 16 + 4 * g;
        uint2* vdst = reinterpret_cast<uint2*>(dV + hoff + (size_t)key * D + f0);
        const uint2 prev = skp[nd];  // zero without a skip
        const float sk[4] = {__uint_as_float(prev.x << 16), __uint_as_float(prev.x & 0xffff0000u),
                             __uint_as_float(prev.y << 16), __uint_as_float(prev.y & 0xffff0000u)};
        float vk[4], vv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          vk[i] = scale * ak[i];
          vv[i] = av[i] + sk[i];
        }
        *reinterpret_cast<uint2*>(dK + hoff + (size_t)key * D + f0) =
            make_uint2(pack_bf16x2(vk[0], vk[1]), pack_bf16x2(vk[2], vk[3]));
        *vdst = make_uint2(pack_bf16x2(vv[0], vv[1]), pack_bf16x2(vv[2], vv[3]));
      }
    }
    // dS^T of the tile -> LDS, then dQt_B += dS^T K over the tile's keys.
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.sT[mt * 16 + 4 * g + i][kl] = bf(ds[mt][i]);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int t = wave + 4 * u, mt = t & 3, nd = t >> 2;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc)
        aq[u] = mfma(lds8(&sm.sT[mt * 16 + c][kc * 32 + 8 * g]), tr_b<SM::PD>(sm.kr, kc * 32, nd * 16), aq[u]);
    }
  }
  const size_t base = ((size_t)bh * nchunks + ch) * m * D;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int t = wave + 4 * u, mt = t & 3, nd = t >> 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = mt * 16 + 4 * g + i;
      if (j < m) pdqt[base + (size_t)j * D + nd * 16 + c] = scale * aq[u][i];
    }
  }
}

// Query side on the matrix cores; grid (chunks, batch*heads), tiles of 64
// rows: partials of dW = F^T dO and dKt_F = s dS_F^T Q per chunk, and
// dQ_i = s dS_i Kt, written as the first dQ (the landmark term seg^T dQt
// needs the pseudoinverse backward; k_bwd_spread adds it).
template <int D>
struct RowMmSmem {
  static constexpr int PD = D + 8, PK = 64 + 8;
  uint16_t ka[64][PD];   // Kt * log2(e)/sqrt(d) rows (A of the scores)
  uint16_t wa[64][PD];   // W rows (A of dF)
  uint16_t qr[kMmTile][PD], gr[kMmTile][PD];  // Q and dO rows of the tile (also B of dKt, dW, read transposed)
  uint16_t fT[64][PK], sT[64][PK];            // F^T, dS^T of the tile (A of dW, dKt); Kt^T before the first tile
};

template <int D>
__global__ __launch_bounds__(256) void k_bwd_rows_mm(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ dO,
                                                     const float* __restrict__ Kt, const float* __restrict__ W,
                                                     uint16_t* __restrict__ dQ, float* __restrict__ pdw,
                                                     float* __restrict__ pdkt, const int* __restrict__ lens, int heads,
                                                     int n, int m, int chunk, int nchunks, float sl2e, float scale) {
  using SM = RowMmSmem<D>;
  constexpr int KC = D / 32, ND = D / 16, PER = ND;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  SM& sm = *reinterpret_cast<SM*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c = lane & 15, g = lane >> 4;
  const int ch = blockIdx.x, bh = blockIdx.y;
  const size_t hoff = (size_t)bh * n * D, md = (size_t)bh * m * D;

  for (int e = tid; e < 64 * D; e += 256) {
    const int j = e / D, f = e % D;
    const float k = j < m ? Kt[md + e] : 0.f;
    sm.ka[j][f] = bf(k * sl2e);
    sm.wa[j][f] = bf(j < m ? W[md + e] : 0.f);
    sm.fT[f][mm_slot(j)] = bf(k);  // Kt^T, landmarks in mm_slot order (f < D <= 64)
  }
  __syncthreads();
  // Kt^T fragments (A of dQ^T = Kt^T dS^T) to registers; the tile loop's
  // first barrier comes before fT is written again.
  B8 kfr[ND][2];
#pragma unroll
  for (int nd = 0; nd < ND; ++nd)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) kfr[nd][kk] = lds8(&sm.fT[nd * 16 + c][kk * 32 + 8 * g]);
  f32x4_t aw[PER], ak[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) aw[u] = ak[u] = zero4();

  const int rbeg = ch * chunk, rend = min(seq_rows(lens, bh / heads, n), rbeg + chunk);  // rows of the sequence
  // Q and dO rows of a tile, 16 bytes per load; the next tile's are in
  // flight while the current one is computed.
  constexpr int NL = kMmTile * (D / 8) / 256;
  uint4 qn[NL], gn[NL];
  auto fetch = [&](int r0) {
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      const int e = tid + 256 * l, rr = e / (D / 8), c8 = (e % (D / 8)) * 8, row = r0 + rr;
      const bool in = row < rend;
      qn[l] = in ? *reinterpret_cast<const uint4*>(Q + hoff + (size_t)row * D + c8) : make_uint4(0, 0, 0, 0);
      gn[l] = in ? *reinterpret_cast<const uint4*>(dO + hoff + (size_t)row * D + c8) : make_uint4(0, 0, 0, 0);
    }
  };
  fetch(rbeg);
  for (int t0 = rbeg; t0 < rend; t0 += kMmTile) {
    __syncthreads();
#pragma unroll
    for (int l = 0; l < NL; ++l) {
      const int e = tid + 256 * l, rr = e / (D / 8), c8 = (e % (D / 8)) * 8;
      B8 q, gv;
      q.q = qn[l];
      gv.q = gn[l];
      *reinterpret_cast<uint4*>(&sm.qr[rr][c8]) = q.q;
      *reinterpret_cast<uint4*>(&sm.gr[rr][c8]) = gv.q;
    }
    __syncthreads();
    if (t0 + kMmTile < rend) fetch(t0 + kMmTile);

    const int rl = 16 * wave + c, row = t0 + rl;
    const bool live = row < rend;
    f32x4_t sc[4], df[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      sc[mt] = zero4();
      df[mt] = zero4();
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        sc[mt] = mfma(lds8(&sm.ka[mt * 16 + c][kc * 32 + 8 * g]), lds8(&sm.qr[rl][kc * 32 + 8 * g]), sc[mt]);
        df[mt] = mfma(lds8(&sm.wa[mt * 16 + c][kc * 32 + 8 * g]), lds8(&sm.gr[rl][kc * 32 + 8 * g]), df[mt]);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (mt * 16 + 4 * g + i >= m) sc[mt][i] = -INFINITY;
        mx = fmaxf(mx, sc[mt][i]);
      }
    mx = max_over_groups(mx);
    float sum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sc[mt][i] = exp2f(sc[mt][i] - mx);
        sum += sc[mt][i];
      }
    const float inv = 1.f / sum_over_groups(sum);
    float delta = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sc[mt][i] *= inv;  // F
        delta = fmaf(sc[mt][i], df[mt][i], delta);
      }
    delta = sum_over_groups(delta);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        df[mt][i] = live ? sc[mt][i] * (df[mt][i] - delta) : 0.f;  // dS
        if (!live) sc[mt][i] = 0.f;
      }

    // dQ^T of the tile = Kt^T dS^T.  The products run on every lane (a
    // matrix-core instruction reads the operands of the whole wave); only
    // the stores are per row.
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) {
      f32x4_t a = zero4();
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) a = mfma(kfr[nd][kk], pack_b(df[2 * kk], df[2 * kk + 1]), a);
      if (live)
        *reinterpret_cast<uint2*>(dQ + hoff + (size_t)row * D + nd * 16 + 4 * g) =
            make_uint2(pack_bf16x2(scale * a[0], scale * a[1]), pack_bf16x2(scale * a[2], scale * a[3]));
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sm.fT[mt * 16 + 4 * g + i][rl] = bf(sc[mt][i]);
        sm.sT[mt * 16 + 4 * g + i][rl] = bf(df[mt][i]);
      }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int t = wave + 4 * u, mt = t & 3, nd = t >> 2;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        aw[u] = mfma(lds8(&sm.fT[mt * 16 + c][kc * 32 + 8 * g]), tr_b<SM::PD>(sm.gr, kc * 32, nd * 16), aw[u]);
        ak[u] = mfma(lds8(&sm.sT[mt * 16 + c][kc * 32 + 8 * g]), tr_b<SM::PD>(sm.qr, kc * 32, nd * 16), ak[u]);
      }
    }
  }
  const size_t base = ((size_t)bh * nchunks + ch) * m * D;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int t = wave + 4 * u, mt = t & 3, nd = t >> 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = mt * 16 + 4 * g + i;
      if (j < m) {
        pdw[base + (size_t)j * D + nd * 16 + c] = aw[u][i];
        pdkt[base + (size_t)j * D + nd * 16 + c] = scale * ak[u][i];
      }
    }
  }
}

// The landmark terms of the matrix-core path, once dQt and dKt are complete:
// dQ_i += dQt[seg(i)] / l and dK_i += dKt[seg(i)] / l, rows i of the
// segment of landmark min(i / l, m - 1).  One thread per 16-byte vector of 8
// bf16 features of dQ and of dK; grid over batch*heads*n*D/8.  Rows past a
// sequence's end are left as they are.
template <int D>
__global__ __launch_bounds__(256) void k_bwd_spread(const float* __restrict__ dqt, const float* __restrict__ dkt,
                                                    uint16_t* __restrict__ dQ, uint16_t* __restrict__ dK,
                                                    const int* __restrict__ lens, int heads, int n, int m,
                                                    long long total) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= total) return;
  constexpr int V = D / 8;
  const int c8 = (int)(e % V) * 8;
  const long long r = e / V;  // bh * n + row
  const int row = (int)(r % n);
  const long long bh = r / n;
  const int nb = seq_rows(lens, (int)(bh / heads), n);
  if (row >= nb) return;
  const int seg = max(1, (nb + m - 1) / m);
  const float inv_seg = 1.f / (float)seg;
  const size_t so = ((size_t)bh * m + min(row / seg, m - 1)) * D + c8;
  const float4 qa = *reinterpret_cast<const float4*>(dqt + so), qb = *reinterpret_cast<const float4*>(dqt + so + 4);
  const float4 ka = *reinterpret_cast<const float4*>(dkt + so), kb = *reinterpret_cast<const float4*>(dkt + so + 4);
  uint4* qp = reinterpret_cast<uint4*>(dQ) + e;
  uint4* kp = reinterpret_cast<uint4*>(dK) + e;
  B8 qv, kv, qo, ko;
  qv.q = *qp;
  kv.q = *kp;
  const float qf[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
  const float kf[8] = {ka.x, ka.y, ka.z, ka.w, kb.x, kb.y, kb.z, kb.w};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    qo.u[u] = pack_bf16x2(bf16_to_f32(qv.h[2 * u]) + qf[2 * u] * inv_seg,
                          bf16_to_f32(qv.h[2 * u + 1]) + qf[2 * u + 1] * inv_seg);
    ko.u[u] = pack_bf16x2(bf16_to_f32(kv.h[2 * u]) + kf[2 * u] * inv_seg,
                          bf16_to_f32(kv.h[2 * u + 1]) + kf[2 * u + 1] * inv_seg);
  }
  *qp = qo.q;
  *kp = ko.q;
}

// dQt = dQt_A + sum of the key-side partials (chunk order); grid
// (entries / 256, batch*heads), one entry per thread.
__global__ __launch_bounds__(256) void k_bwd_qt_finish(const float* __restrict__ dQtA, const float* __restrict__ pdqt,
                                                       float* __restrict__ dQt, int md, int nchunks) {
  const int bh = blockIdx.y, e = blockIdx.x * 256 + (int)threadIdx.x;
  if (e >= md) return;
  dQt[(size_t)bh * md + e] = chunk_sum(pdqt + (size_t)bh * nchunks * md + e, md, nchunks, dQtA[(size_t)bh * md + e]);
}

// dconv_w[h] = sum over batch entries and key chunks (fixed order); grid
// (entries / 256, heads).
__global__ __launch_bounds__(256) void k_bwd_dw_finish(const float* __restrict__ pdwc, float* __restrict__ dw,
                                                       int batch, int heads, int nchunks, int dk) {
  const int h = blockIdx.y, e = blockIdx.x * 256 + (int)threadIdx.x;
  if (e >= dk) return;
  float a = 0.f;
  for (int b = 0; b < batch; ++b) a = chunk_sum(pdwc + ((size_t)(b * heads + h)) * nchunks * dk + e, dk, nchunks, a);
  dw[(size_t)h * dk + e] = a;
}

// Masked calls: rows past each sequence's end of dQ, dK and dV are zero.
// One thread per 16-byte vector of a row; grid over batch*heads*n*VPR.
__global__ __launch_bounds__(256) void k_bwd_zero_pad(uint4* __restrict__ dQ, uint4* __restrict__ dK,
                                                      uint4* __restrict__ dV, const int* __restrict__ lens, int heads,
                                                      int n, int vpr, long long total) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  if (e >= total) return;
  const long long r = e / vpr;  // bh * n + row
  const int row = (int)(r % n), b = (int)(r / n / heads);
  if (row < seq_rows(lens, b, n)) return;
  const uint4 z = make_uint4(0, 0, 0, 0);
  dQ[e] = z;
  dK[e] = z;
  dV[e] = z;
}

static int cdivi(long long a, long long b) { return (int)((a + b - 1) / b); }

// A second stream per device, on which the matrix-core path's key side runs
// beside the landmark-side kernel (fork and join by events on the caller's
// stream); created on first use and kept for the life of the process.  One
// call's fork and join are enqueued under the lock, so that calls from
// several host threads cannot take each other's event records.
struct SideStream {
  hipStream_t st = nullptr;
  hipEvent_t start = nullptr, mid = nullptr, fork = nullptr, join = nullptr;
};
// One call's use of the side stream: `pending` while work forked onto it has
// not been joined back to the caller's stream.
struct SideCall {
  SideStream* ss = nullptr;
  bool pending = false;
};
std::mutex g_side_mu;
SideStream g_side[64];

hipError_t side_stream_locked(SideStream** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  SideStream& ss = g_side[dev];
  if (!ss.st) {
    hipStream_t st = nullptr;
    hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
    if ((e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking)) != hipSuccess) return e;
    for (int i = 0; i < 4; ++i) {
      if ((e = hipEventCreateWithFlags(&ev[i], hipEventDisableTiming)) != hipSuccess) {
        for (int k = 0; k < i; ++k) (void)hipEventDestroy(ev[k]);
        (void)hipStreamDestroy(st);
        return e;
      }
    }
    ss.start = ev[0];
    ss.mid = ev[1];
    ss.fork = ev[2];
    ss.join = ev[3];
    ss.st = st;
  }
  *out = &ss;
  return hipSuccess;
}

// Chunks per head for the split passes: at most `slots` blocks in all, so
// that every block starts in the first round (a second round of a few
// full-length blocks would double the pass's time).  The passes hold two
// blocks per CU (their LDS); the key side shares the chip with the
// landmark-side blocks, one per head, whose LDS fills their CUs.
static int split_chunks(long long rows, long long bh, int tile, long long slots) {
  long long want = slots / bh;
  long long maxc = (rows + tile - 1) / tile;
  if (want < 1) want = 1;
  if (want > maxc) want = maxc;
  return (int)want;
}

}  // namespace

// ---------------------------------------------------------------------------
// Workspace of the backward pass: the forward's regions, then its own.

bool make_bwd_layout(int batch, int heads, int n, int d, int m, int iters, int conv_k, bool bf16, BwdLayout* L) {
  if (!make_layout(batch, heads, n, d, m, &L->fwd)) return false;
  if (m > 64 || conv_k > 33) return false;
  const long long BH = (long long)batch * heads;
  // Chunks are multiples of 64 rows, a whole number of tiles for every pass.
  const int tq = split_chunks(n, BH, kMmTile, 2 * 256);
  L->qchunk = cdivi(cdivi(n, tq), kMmTile) * kMmTile;
  L->nq = cdivi(n, L->qchunk);
  // On the matrix-core path the key side runs beside the landmark-side blocks.
  const bool side = bf16 && (d == 32 || d == 64);
  const int tk = split_chunks(n, BH, kMmTile, side ? 2 * (256 - (BH < 128 ? BH : 128)) : 2 * 256);
  L->kchunk = cdivi(cdivi(n, tk), kMmTile) * kMmTile;
  L->nk = cdivi(n, L->kchunk);
  L->mp = m <= 32 ? 32 : 64;
  size_t off = L->fwd.total;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  const size_t md = (size_t)BH * m * d * 4;
  // The saved state first (the forward's regions, then its steps), so that
  // the training pair can keep it apart from the backward's scratch.
  L->zs = take((size_t)BH * (iters > 0 ? iters : 1) * 4 * L->mp * L->mp * 4);
  L->state = off;
  L->pdw = take(md * L->nq);
  L->pdkt = take(md * L->nq);
  L->dw = take(md);
  L->dbv = take(md);
  L->dkt = take(md);
  L->dqta = take(md);
  L->pdqt = take(md * L->nk);
  L->dqt = take(md);
  L->pdwc = take((size_t)BH * L->nk * d * (conv_k > 0 ? conv_k : 1) * 4);
  L->wflip = take((size_t)heads * d * (conv_k > 0 ? conv_k : 1) * 4);
  L->total = off;
  return true;
}

template <typename IO, int D>
static hipError_t bwd_t(const BwdProblem& bp, const BwdLayout& L, const BwdBuf& ws, hipStream_t s, SideCall& sc) {
  using T = typename IO::T;
  const Problem& p = bp.fwd;
  const Ws w = resolve(L.fwd, ws.st);
  auto F = [&](size_t o) { return reinterpret_cast<float*>(ws.scratch(o)); };  // scratch regions
  const int BH = p.batch * p.heads;
  const float sl2e = kLog2e / sqrtf((float)D), scale = 1.f / sqrtf((float)D);
  constexpr int P = D + 1;

  constexpr bool MM = IO::kBf16 && (D == 32 || D == 64);  // matrix-core n-sized passes
  // Query side, partials of dW and dKt_F (on the matrix-core path also the
  // first dQ, s dS_F Kt).
  if constexpr (MM) {
    const int bytes = (int)sizeof(RowMmSmem<D>);
    auto kern = &k_bwd_rows_mm<D>;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (attr != hipSuccess) return attr;
    KernelTimer kt_("bwd_rows_reduce", s);
    kern<<<dim3(L.nq, BH), 256, bytes, s>>>(static_cast<const uint16_t*>(p.Q), static_cast<const uint16_t*>(bp.dO),
                                            w.Kt, w.W, static_cast<uint16_t*>(bp.dQ), F(L.pdw), F(L.pdkt), p.lens,
                                            p.heads, p.n, p.m, L.qchunk, L.nq, sl2e, scale);
  } else {
    const int bytes = (2 * 64 * P + 2 * kRowTile * P + 2 * kRowTile * 65) * 4;
    auto kern = &k_bwd_rows<IO, D, false>;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (attr != hipSuccess) return attr;
    KernelTimer kt_("bwd_rows_reduce", s);
    kern<<<dim3(L.nq, BH), 256, bytes, s>>>(static_cast<const T*>(p.Q), static_cast<const T*>(bp.dO), w.Kt, w.W,
                                            nullptr, nullptr, F(L.pdw), F(L.pdkt), p.lens, p.heads, p.n, p.m,
                                            L.qchunk, L.nq, sl2e, scale);
  }
  // dW, dKt_F and dBV from the partials.
  {
    KernelTimer kt_("bwd_land_prep", s);
    k_bwd_land_prep<<<dim3(D / 16, BH), 1024, 0, s>>>(w.Z, F(L.pdw), F(L.pdkt), F(L.dw), F(L.dkt), F(L.dbv), p.m, D,
                                                     L.nq);
  }
  // Landmark side: the pseudoinverse backward, dKt and dQt_A.
  const LandArgs la{w.Qt,      w.Kt,     w.A,     w.BV, F(L.dw), F(L.dkt), F(L.dqta),
                    reinterpret_cast<const float*>(ws.state(L.zs)), p.m, D,  p.iters, scale};
  auto land = [&]() -> hipError_t {
    auto go = [&](auto kern, int nth, int bytes) -> hipError_t {
      // One attribute per kernel variant: the four variants share go's type.
      const hipError_t e = ensure_dynamic_smem(reinterpret_cast<const void*>(kern), bytes);
      if (e != hipSuccess) return e;
      KernelTimer kt_("bwd_landmarks", s);
      kern<<<BH, nth, bytes, s>>>(la);
      return hipSuccess;
    };
    if (L.mp == 32)
      return IO::kBf16 ? go(&k_bwd_land<32, 3>, LandTiles<32>::NTH, (int)sizeof(LandSmem<32>))
                       : go(&k_bwd_land<32, 6>, LandTiles<32>::NTH, (int)sizeof(LandSmem<32>));
    return IO::kBf16 ? go(&k_bwd_land<64, 3>, LandTiles<64>::NTH, (int)sizeof(LandSmem<64>))
                     : go(&k_bwd_land<64, 6>, LandTiles<64>::NTH, (int)sizeof(LandSmem<64>));
  };
  const int ck = p.conv_w ? p.conv_k : 0;
  auto dw_finish = [&](hipStream_t st) {
    if (ck > 0 && bp.dconv_w) {
      KernelTimer kt_("bwd_dw_finish", st);
      k_bwd_dw_finish<<<dim3(cdivi(D * p.conv_k, 256), p.heads), 256, 0, st>>>(F(L.pdwc), bp.dconv_w, p.batch,
                                                                                p.heads, L.nk, D * p.conv_k);
    }
  };
  if constexpr (MM) {
    // The key side (dK, dV and the dQt_B partials) needs only dBV: it runs
    // on the side stream, after the skip's share forked there at the start
    // of the call, while the landmark-side blocks, one per head, run on this
    // one.
    SideStream* ss = sc.ss;
    hipError_t e;
    if ((e = hipEventRecord(ss->fork, s)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(ss->st, ss->fork, 0)) != hipSuccess) return e;
    const hipStream_t ks = ss->st;
    {
      const int bytes = (int)sizeof(KeyMmSmem<D>);
      auto kern = &k_bwd_key_mm<D>;
      static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                         hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
      if (attr != hipSuccess) return attr;
      KernelTimer kt_("bwd_keys", ks);
      kern<<<dim3(L.nk, BH), 256, bytes, ks>>>(static_cast<const uint16_t*>(p.K), static_cast<const uint16_t*>(p.V),
                                               w.Qt, w.BV, F(L.dbv), w.pmax, w.psum, static_cast<uint16_t*>(bp.dK),
                                               static_cast<uint16_t*>(bp.dV), F(L.pdqt), p.lens, p.heads, p.n, p.m,
                                               ck > 0 ? 1 : 0, L.kchunk, L.nk, forward_partials(p, w), sl2e, scale);
    }
    dw_finish(ks);
    if ((e = hipEventRecord(ss->join, ks)) != hipSuccess) return e;
    const hipError_t el = land();
    // Join even when the launch above failed: the caller's stream must not
    // run ahead of the side stream's work.
    if ((e = hipStreamWaitEvent(s, ss->join, 0)) != hipSuccess) return e;
    sc.pending = false;
    if (el != hipSuccess) return el;
  } else {
    hipError_t e = land();
    if (e != hipSuccess) return e;
    // Key side: dK, dV and the partials of dQt_B and the filter gradient.
    const int bytes = (2 * 64 * P + kKeyTile * P + 2 * 48 * P + 2 * kKeyTile * 65 + 3 * 64 + D * (ck > 0 ? ck : 1)) * 4;
    auto kern = &k_bwd_key<IO, D>;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       (2 * 64 * P + kKeyTile * P + 2 * 48 * P + 2 * kKeyTile * 65 +
                                                        3 * 64 + D * 33) * 4);
    if (attr != hipSuccess) return attr;
    {
      KernelTimer kt_("bwd_keys", s);
      kern<<<dim3(L.nk, BH), 256, bytes, s>>>(static_cast<const T*>(p.K), static_cast<const T*>(p.V),
                                              static_cast<const T*>(bp.dO), p.conv_w, w.Qt, w.BV, F(L.dbv), F(L.dkt),
                                              w.pmax, w.psum, static_cast<T*>(bp.dK), static_cast<T*>(bp.dV),
                                              F(L.pdqt), F(L.pdwc), p.lens, p.n, p.m, p.heads, ck, L.kchunk, L.nk,
                                              forward_partials(p, w), sl2e, scale);
    }
    dw_finish(s);
  }
  {
    KernelTimer kt_("bwd_finish", s);
    k_bwd_qt_finish<<<dim3(cdivi(p.m * D, 256), BH), 256, 0, s>>>(F(L.dqta), F(L.pdqt), F(L.dqt), p.m * D, L.nk);
  }
  // The landmark terms of dQ and dK (matrix-core path), or the query side
  // again for dQ (vector path).
  if constexpr (MM) {
    const long long total = (long long)BH * p.n * (D / 8);
    KernelTimer kt_("bwd_spread", s);
    k_bwd_spread<D><<<(unsigned)((total + 255) / 256), 256, 0, s>>>(F(L.dqt), F(L.dkt), static_cast<uint16_t*>(bp.dQ),
                                                                     static_cast<uint16_t*>(bp.dK), p.lens, p.heads,
                                                                     p.n, p.m, total);
  } else {
    const int bytes = (2 * 64 * P + 2 * kRowTile * P + 2 * kRowTile * 65) * 4;
    auto kern = &k_bwd_rows<IO, D, true>;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (attr != hipSuccess) return attr;
    const int nt = cdivi(p.n, kRowTile);
    KernelTimer kt_("bwd_rows_dq", s);
    kern<<<dim3(nt, BH), 256, bytes, s>>>(static_cast<const T*>(p.Q), static_cast<const T*>(bp.dO), w.Kt, w.W,
                                          F(L.dqt), static_cast<T*>(bp.dQ), nullptr, nullptr, p.lens, p.heads, p.n,
                                          p.m, kRowTile, nt, sl2e, scale);
  }
  if (p.lens) {
    // The passes above leave the rows past each sequence's end alone.
    const int vpr = D * (int)sizeof(T) / 16;
    const long long total = (long long)BH * p.n * vpr;
    KernelTimer kt_("bwd_zero_pad", s);
    k_bwd_zero_pad<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(
        static_cast<uint4*>(bp.dQ), static_cast<uint4*>(bp.dK), static_cast<uint4*>(bp.dV), p.lens, p.heads, p.n,
        vpr, total);
  }
  return hipGetLastError();
}

// The skip's share of the matrix-core path, on the side stream; it reads
// only inputs.  dV = DConv^T(dO): the forward's convolution with the taps
// reversed, written as the initial dV.
template <int D>
static hipError_t skip_transpose(const BwdProblem& bp, const BwdLayout& L, const BwdBuf& ws, hipStream_t ks) {
  const Problem& p = bp.fwd;
  float* wf = reinterpret_cast<float*>(ws.scratch(L.wflip));
  const int total = p.heads * D * p.conv_k;
  k_flip_taps<<<cdivi(total, 256), 256, 0, ks>>>(p.conv_w, wf, p.conv_k, total);
  return launch_dconv(bp.dO, wf, bp.dV, p.batch, p.heads, p.n, D, p.conv_k, true, ks, p.lens);
}

// The filter-gradient partials.
template <int D>
static hipError_t skip_grad(const BwdProblem& bp, const BwdLayout& L, const BwdBuf& ws, hipStream_t ks) {
  const Problem& p = bp.fwd;
  KernelTimer kt_("bwd_skip_grad", ks);
  k_bwd_skip_grad<D><<<dim3(L.nk, p.batch * p.heads), 4 * D, (int)sizeof(SkipSmem<D>), ks>>>(
      static_cast<const uint16_t*>(p.V), static_cast<const uint16_t*>(bp.dO), reinterpret_cast<float*>(ws.scratch(L.pdwc)),
      p.lens, p.heads, p.n, p.conv_k, L.kchunk, L.nk);
  return hipSuccess;
}

static hipError_t backward_body(const BwdProblem& bp, const BwdLayout& L, const BwdBuf& ws, hipStream_t s, SideCall& sc,
                                bool recompute) {
  const Problem& p = bp.fwd;
  const Ws w = resolve(L.fwd, ws.st);
  hipError_t e;
  const bool skip = sc.ss && p.conv_w && p.conv_k > 0;
  if (sc.ss) {
    // Fork: the skip's filter gradient needs only the inputs; it runs
    // beside the forward's stages.
    if ((e = hipEventRecord(sc.ss->start, s)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(sc.ss->st, sc.ss->start, 0)) != hipSuccess) return e;
    sc.pending = true;
    if (skip) {
      e = p.d == 32 ? skip_grad<32>(bp, L, ws, sc.ss->st) : skip_grad<64>(bp, L, ws, sc.ss->st);
      if (e != hipSuccess) return e;
    }
  }
  // The forward's landmark side: Qt, Kt, A, Z, BV, W and B's statistics
  // (already in the state part when the forward saved them).
  if (recompute) {
    if ((e = stage_segment_means(p, w, s)) != hipSuccess) return e;
    if ((e = stage_landmark_pass(p, w, s)) != hipSuccess) return e;
    if ((e = stage_pinv(p, w, s)) != hipSuccess) return e;
    if ((e = stage_bv_finish(p, w, s)) != hipSuccess) return e;
  }
  if (skip) {
    // The skip's transpose (a streaming convolution that would slow the
    // landmark pass) runs beside the query-side reduction.
    if ((e = hipEventRecord(sc.ss->mid, s)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(sc.ss->st, sc.ss->mid, 0)) != hipSuccess) return e;
    e = p.d == 32 ? skip_transpose<32>(bp, L, ws, sc.ss->st) : skip_transpose<64>(bp, L, ws, sc.ss->st);
    if (e != hipSuccess) return e;
  }
  switch (p.d) {
    case 16: return p.bf16 ? bwd_t<BF16, 16>(bp, L, ws, s, sc) : bwd_t<F32, 16>(bp, L, ws, s, sc);
    case 32: return p.bf16 ? bwd_t<BF16, 32>(bp, L, ws, s, sc) : bwd_t<F32, 32>(bp, L, ws, s, sc);
    case 64: return p.bf16 ? bwd_t<BF16, 64>(bp, L, ws, s, sc) : bwd_t<F32, 64>(bp, L, ws, s, sc);
    case 128: return p.bf16 ? bwd_t<BF16, 128>(bp, L, ws, s, sc) : bwd_t<F32, 128>(bp, L, ws, s, sc);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_forward_save(const Problem& p0, const BwdLayout& L, char* ws, hipStream_t s) {
  Problem p = p0;
  p.zsave = reinterpret_cast<float*>(ws + L.zs);
  p.zmp = L.mp;
  return launch_forward(p, L.fwd, ws, s);
}

hipError_t launch_backward(const BwdProblem& bp0, const BwdLayout& L, const BwdBuf& ws, hipStream_t s,
                           bool recompute) {
  // The forward's pseudoinverse kernel also saves its steps for the reverse pass.
  BwdProblem bp = bp0;
  bp.fwd.zsave = reinterpret_cast<float*>(ws.state(L.zs));
  bp.fwd.zmp = L.mp;
  const Problem& p = bp.fwd;
  if (!(p.bf16 && (p.d == 32 || p.d == 64))) {
    SideCall none;
    return backward_body(bp, L, ws, s, none, recompute);
  }
  // Matrix-core path: this call's forks and joins are enqueued under the lock.
  std::lock_guard<std::mutex> lock(g_side_mu);
  SideCall sc;
  hipError_t e = side_stream_locked(&sc.ss);
  if (e != hipSuccess) return e;
  e = backward_body(bp, L, ws, s, sc, recompute);
  if (sc.pending) {
    // An error left work on the side stream: join it all the same.
    if (hipEventRecord(sc.ss->join, sc.ss->st) == hipSuccess) (void)hipStreamWaitEvent(s, sc.ss->join, 0);
  }
  return e;
}

}  // namespace nys

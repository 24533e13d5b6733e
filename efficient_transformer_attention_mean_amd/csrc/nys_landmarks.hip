// Nyström self-attention forward, landmark side: HIP kernels for gfx950 (CDNA4).
//
// Method: "Nyströmformer: A Nyström-Based Algorithm for Approximating
// Self-Attention" (paper deep-dive page, sec. 3.2 and 3.4).  Per (batch, head):
//   segment means Qt, Kt (Eq. 16)         -> k_segment_mean
//   A = softmax(Qt Kt^T / sqrt d), Z = Lemma-1 iterations from the
//   Pan-Schreiber start                    -> k_pinv_lds (m <= 64) or
//                                             k_landmark_softmax + k_pinv_start + k_mm chain
//   B V = softmax(Qt K^T / sqrt d) V       -> k_landmark_bv (split over keys,
//                                             online softmax) + k_bv_combine
//   W = Z (B V)                            -> k_mm, then k_prep_w (bf16 planes)
// The output stage (softmax(Q Kt^T / sqrt d) W + DConv(V)) is in nys_apply.hip.
// Softmaxes run in base 2: scores are pre-multiplied by log2(e)/sqrt(d), which
// leaves every softmax unchanged.
#include <math.h>

#include "nys_common.hpp"
#include "nys_internal.hpp"

namespace nys {

// ---------------------------------------------------------------------------
// Segment means: grid (m, batch*heads, 2); z = 0 -> Q, z = 1 -> K.
// One block per segment of l = n/m contiguous rows; 16-byte coalesced loads,
// fp32 partial sums per thread, fixed-order reduction through LDS.
// Key landmarks are also written as bf16 hi/lo planes [bh][mpa][D] (rows
// m..mpa-1 zero), the operand layout of the output stage.
template <typename IO, int D>
__global__ __launch_bounds__(256) void k_segment_mean(const typename IO::T* __restrict__ Q,
                                                      const typename IO::T* __restrict__ K,
                                                      float* __restrict__ Qt, float* __restrict__ Kt,
                                                      uint16_t* __restrict__ kt_hi, uint16_t* __restrict__ kt_lo,
                                                      int n, int m, int mpa) {
  using T = typename IO::T;
  constexpr int VEC = 16 / sizeof(T);
  constexpr int SLOTS = D / VEC;
  constexpr int RS = 256 / SLOTS;
  __shared__ float part[RS * D];
  const int j = blockIdx.x, bh = blockIdx.y;
  const int seg = n / m;
  const T* X = (blockIdx.z == 0 ? Q : K) + ((size_t)bh * n + (size_t)j * seg) * D;
  float* out = (blockIdx.z == 0 ? Qt : Kt) + ((size_t)bh * m + j) * D;
  const int slot = threadIdx.x % SLOTS, r0 = threadIdx.x / SLOTS;
  float acc[VEC];
#pragma unroll
  for (int q = 0; q < VEC; ++q) acc[q] = 0.f;
  for (int r = r0; r < seg; r += RS) {
    const T* p = X + (size_t)r * D + slot * VEC;
    if constexpr (IO::kBf16) {
      B8 b;
      b.q = *reinterpret_cast<const uint4*>(p);
#pragma unroll
      for (int q = 0; q < VEC; ++q) acc[q] += bf16_to_f32(b.h[q]);
    } else {
      const float4 a = *reinterpret_cast<const float4*>(p);
      acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
    }
  }
#pragma unroll
  for (int q = 0; q < VEC; ++q) part[r0 * D + slot * VEC + q] = acc[q];
  __syncthreads();
  if (threadIdx.x < D) {
    float s = 0.f;
    for (int p = 0; p < RS; ++p) s += part[p * D + threadIdx.x];
    const float mean = s / (float)seg;
    out[threadIdx.x] = mean;
    if (blockIdx.z == 1) {
      uint16_t hi, lo;
      split_hi_lo(mean, hi, lo);
      const size_t o = ((size_t)bh * mpa + j) * D + threadIdx.x;
      kt_hi[o] = hi;
      kt_lo[o] = lo;
      if (j == m - 1) {
        for (int r = m; r < mpa; ++r) {
          kt_hi[((size_t)bh * mpa + r) * D + threadIdx.x] = 0;
          kt_lo[((size_t)bh * mpa + r) * D + threadIdx.x] = 0;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Pseudoinverse for m <= 64: one block (4 waves) per head, every iterate in LDS.
// Products are bf16x3 on the matrix cores with fp32 accumulation.
template <int MP>
struct PinvSmem {
  __align__(16) float A[MP][MP + 4];
  float Z[MP][MP + 4];
  float X[MP][MP + 4];
  float T[MP][MP + 4];
  float U[MP][MP + 4];
  float red[2][MP];
};

// C = P * Qm over MP x MP LDS matrices, computed as C^T = Qm^T P^T so that a
// lane ends with 4 consecutive columns of one row of C: epi(row, col0, v)
// stores v[i] at (row, col0 + i) with one 16-byte LDS write per matrix.
template <int MP, int PR, typename Epi>
__device__ __forceinline__ void lds_mm(const float (*P)[MP + 4], const float (*Qm)[MP + 4], Epi epi) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  constexpr int NT = MP / 16;
  for (int t = wave; t < NT * NT; t += 4) {
    const int ti = t / NT, tj = t % NT;  // C rows ti*16.., columns tj*16..
    f32x4_t acc = zero4();
#pragma unroll
    for (int kc = 0; kc < MP; kc += 32) {
      float a[8], b[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        a[q] = Qm[kc + 8 * g + q][tj * 16 + c];  // A = Qm^T: row = column of C
        b[q] = P[ti * 16 + c][kc + 8 * g + q];   // B = P^T: column = row of C
      }
      acc = mma_f32<PR>(a, b, acc);
    }
    epi(ti * 16 + c, tj * 16 + 4 * g, acc);
  }
}

// v + alpha * I restricted to the 4 entries (row, col0 .. col0+3).
__device__ __forceinline__ float4 plus_diag(int row, int col0, const f32x4_t& v, float scale, float alpha) {
  float r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = scale * v[i] + (row == col0 + i ? alpha : 0.f);
  return make_float4(r[0], r[1], r[2], r[3]);
}

template <int MP, int PR>
__global__ __launch_bounds__(256) void k_pinv_lds(const float* __restrict__ Qt, const float* __restrict__ Kt,
                                                  float* __restrict__ Aout, float* __restrict__ Zout, int m,
                                                  int d, float sl2e, int iters) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  PinvSmem<MP>& sm = *reinterpret_cast<PinvSmem<MP>*>(smem_raw);
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, c = lane & 15, g = lane >> 4;
  const float* qt = Qt + (size_t)bh * m * d;
  const float* kt = Kt + (size_t)bh * m * d;
  constexpr int NT = MP / 16;

  // Scaled scores Qt Kt^T * log2(e)/sqrt(d); rows/cols >= m are zero padding.
  // Computed as (Kt Qt^T)^T: a lane ends with row ti*16+c, columns tj*16+4g..+3.
  for (int t = wave; t < NT * NT; t += 4) {
    const int ti = t / NT, tj = t % NT;
    const int rq = ti * 16 + c, rk = tj * 16 + c;
    f32x4_t acc = zero4();
    for (int kc = 0; kc < d; kc += 32) {
      float a[8], b[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int kk = kc + 8 * g + q;
        a[q] = (rk < m && kk < d) ? kt[rk * d + kk] : 0.f;
        b[q] = (rq < m && kk < d) ? qt[rq * d + kk] : 0.f;
      }
      acc = mma_f32<PR>(a, b, acc);
    }
    *reinterpret_cast<float4*>(&sm.A[rq][tj * 16 + 4 * g]) =
        make_float4(acc[0] * sl2e, acc[1] * sl2e, acc[2] * sl2e, acc[3] * sl2e);
  }
  __syncthreads();

  // Row softmax over the m real columns; padded rows and columns become 0.
  {
    constexpr int TPR = 256 / MP;
    const int r = tid / TPR, sub = tid % TPR;
    float mx = -INFINITY;
    for (int j = sub; j < m; j += TPR) mx = fmaxf(mx, sm.A[r][j]);
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) mx = fmaxf(mx, shfl_xor(mx, o));
    float s = 0.f;
    for (int j = sub; j < MP; j += TPR) {
      const float e = (r < m && j < m) ? exp2f(sm.A[r][j] - mx) : 0.f;
      sm.A[r][j] = e;
      s += e;
    }
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) s += shfl_xor(s, o);
    if (r < m) {
      const float inv = 1.f / s;
      for (int j = sub; j < m; j += TPR) sm.A[r][j] *= inv;
    }
  }
  __syncthreads();

  // Z0 = A^T / (max column abs sum * max row abs sum).
  if (tid < MP) {
    float cs = 0.f, rs = 0.f;
    for (int i = 0; i < MP; ++i) {
      cs += fabsf(sm.A[i][tid]);
      rs += fabsf(sm.A[tid][i]);
    }
    sm.red[0][tid] = cs;
    sm.red[1][tid] = rs;
  }
  __syncthreads();
  float n1 = 0.f, ninf = 0.f;
  for (int i = 0; i < MP; ++i) {
    n1 = fmaxf(n1, sm.red[0][i]);
    ninf = fmaxf(ninf, sm.red[1][i]);
  }
  const float cz = 1.f / (n1 * ninf);
  for (int e = tid; e < MP * MP; e += 256) {
    const int i = e / MP, j = e % MP;
    sm.Z[i][j] = cz * sm.A[j][i];
  }
  __syncthreads();

  // Z <- Z (13I - X(15I - X(7I - X))) / 4,  X = A Z.
  float(*Z)[MP + 4] = sm.Z;
  float(*Xb)[MP + 4] = sm.X;
  for (int it = 0; it < iters; ++it) {
    lds_mm<MP, PR>(sm.A, Z, [&](int r, int c0, const f32x4_t& v) {
      *reinterpret_cast<float4*>(&Xb[r][c0]) = plus_diag(r, c0, v, 1.f, 0.f);
      *reinterpret_cast<float4*>(&sm.T[r][c0]) = plus_diag(r, c0, v, -1.f, 7.f);
    });
    __syncthreads();
    lds_mm<MP, PR>(Xb, sm.T, [&](int r, int c0, const f32x4_t& v) {
      *reinterpret_cast<float4*>(&sm.U[r][c0]) = plus_diag(r, c0, v, -1.f, 15.f);
    });
    __syncthreads();
    lds_mm<MP, PR>(Xb, sm.U, [&](int r, int c0, const f32x4_t& v) {
      *reinterpret_cast<float4*>(&sm.T[r][c0]) = plus_diag(r, c0, v, -1.f, 13.f);
    });
    __syncthreads();
    lds_mm<MP, PR>(Z, sm.T, [&](int r, int c0, const f32x4_t& v) {
      *reinterpret_cast<float4*>(&Xb[r][c0]) = plus_diag(r, c0, v, 0.25f, 0.f);
    });
    __syncthreads();
    float(*tmp)[MP + 4] = Z;
    Z = Xb;
    Xb = tmp;
  }

  float* ao = Aout + (size_t)bh * m * m;
  float* zo = Zout + (size_t)bh * m * m;
  for (int e = tid; e < m * m; e += 256) {
    const int i = e / m, j = e % m;
    ao[e] = sm.A[i][j];
    zo[e] = Z[i][j];
  }
}

// ---------------------------------------------------------------------------
// Pseudoinverse for 64 < m <= 256, step 1: A rows.  grid (ceil(m/16), batch*heads).
// Each block computes 16 rows of the scaled scores with the matrix cores,
// then row softmax in LDS.
template <int PR>
__global__ __launch_bounds__(256) void k_landmark_softmax(const float* __restrict__ Qt,
                                                          const float* __restrict__ Kt,
                                                          float* __restrict__ Aout, int m, int d,
                                                          float sl2e) {
  __shared__ __align__(16) float S[16][256 + 4];
  const int bh = blockIdx.y, r0 = blockIdx.x * 16, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, c = lane & 15, g = lane >> 4;
  const float* qt = Qt + (size_t)bh * m * d;
  const float* kt = Kt + (size_t)bh * m * d;
  const int ntile = (m + 15) / 16;
  // (Kt Qt^T)^T tiles: a lane ends with score row r0+c, columns tj*16+4g..+3.
  for (int tj = wave; tj < ntile; tj += 4) {
    const int rq = r0 + c, rk = tj * 16 + c;
    f32x4_t acc = zero4();
    for (int kc = 0; kc < d; kc += 32) {
      float a[8], b[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int kk = kc + 8 * g + q;
        a[q] = (rk < m && kk < d) ? kt[rk * d + kk] : 0.f;
        b[q] = (rq < m && kk < d) ? qt[rq * d + kk] : 0.f;
      }
      acc = mma_f32<PR>(a, b, acc);
    }
    *reinterpret_cast<float4*>(&S[c][tj * 16 + 4 * g]) =
        make_float4(acc[0] * sl2e, acc[1] * sl2e, acc[2] * sl2e, acc[3] * sl2e);
  }
  __syncthreads();
  // 16 rows x 16 threads per row.
  const int r = tid >> 4, sub = tid & 15;
  float mx = -INFINITY;
  for (int j = sub; j < m; j += 16) mx = fmaxf(mx, S[r][j]);
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) mx = fmaxf(mx, shfl_xor(mx, o));
  float s = 0.f;
  for (int j = sub; j < m; j += 16) {
    const float e = exp2f(S[r][j] - mx);
    S[r][j] = e;
    s += e;
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) s += shfl_xor(s, o);
  const float inv = 1.f / s;
  if (r0 + r < m) {
    float* ao = Aout + ((size_t)bh * m + r0 + r) * m;
    for (int j = sub; j < m; j += 16) ao[j] = S[r][j] * inv;
  }
}

// Step 2: Z0 = A^T / (||A||_1 ||A||_inf).  grid (batch*heads).
__global__ __launch_bounds__(256) void k_pinv_start(const float* __restrict__ A, float* __restrict__ Z0, int m) {
  __shared__ float red[2][256];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const float* a = A + (size_t)bh * m * m;
  float cs = 0.f, rs = 0.f;
  if (tid < m) {
    for (int i = 0; i < m; ++i) {
      cs += fabsf(a[(size_t)i * m + tid]);
      rs += fabsf(a[(size_t)tid * m + i]);
    }
  }
  red[0][tid] = cs;
  red[1][tid] = rs;
  __syncthreads();
  float n1 = 0.f, ninf = 0.f;
  for (int i = 0; i < m; ++i) {
    n1 = fmaxf(n1, red[0][i]);
    ninf = fmaxf(ninf, red[1][i]);
  }
  const float cz = 1.f / (n1 * ninf);
  float* z = Z0 + (size_t)bh * m * m;
  for (int e = tid; e < m * m; e += 256) {
    const int i = e / m, j = e % m;
    z[e] = cz * a[(size_t)j * m + i];
  }
}

// Batched fp32 product with an affine epilogue:
//   C1 = a1 * (P Q) + d1 * I,  and if C2 != null also C2 = a2 * (P Q) + d2 * I.
// P: M x K, Q: K x N, row-major, per batch entry strides sP, sQ, sC (elements).
// grid (ceil(N/64), ceil(M/64), batch); 4 waves, each 16 rows x 64 columns.
struct MMArgs {
  const float* P;
  const float* Q;
  float* C1;
  float* C2;
  int M, N, K;
  long long sP, sQ, sC;
  float a1, d1, a2, d2;
};

template <int PR>
__global__ __launch_bounds__(256) void k_mm(MMArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, c = lane & 15, g = lane >> 4;
  const int bz = blockIdx.z;
  const float* P = a.P + bz * a.sP;
  const float* Qm = a.Q + bz * a.sQ;
  const int row0 = blockIdx.y * 64 + wave * 16, col0 = blockIdx.x * 64;
  if (row0 >= a.M) return;
  f32x4_t acc[4] = {zero4(), zero4(), zero4(), zero4()};
  for (int kc = 0; kc < a.K; kc += 32) {
    float x[8];
    const int r = row0 + c;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int kk = kc + 8 * g + q;
      x[q] = (r < a.M && kk < a.K) ? P[(size_t)r * a.K + kk] : 0.f;
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int col = col0 + nt * 16 + c;
      float y[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int kk = kc + 8 * g + q;
        y[q] = (col < a.N && kk < a.K) ? Qm[(size_t)kk * a.N + col] : 0.f;
      }
      acc[nt] = mma_f32<PR>(x, y, acc[nt]);
    }
  }
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int col = col0 + nt * 16 + c;
    if (col >= a.N) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = row0 + 4 * g + i;
      if (r >= a.M) continue;
      const float v = acc[nt][i];
      const float diag = (r == col) ? 1.f : 0.f;
      a.C1[bz * a.sC + (size_t)r * a.N + col] = a.a1 * v + a.d1 * diag;
      if (a.C2) a.C2[bz * a.sC + (size_t)r * a.N + col] = a.a2 * v + a.d2 * diag;
    }
  }
}

// ---------------------------------------------------------------------------
// softmax(Qt K^T / sqrt d) V, split over keys.  grid (nchunks, batch*heads).
// Each block streams its chunk of keys in tiles of 64 through LDS (K row-major,
// V transposed) and keeps, per landmark, a running max, a running sum and the
// unnormalised accumulator (online softmax); it writes those three partials.
// Scores are computed transposed (keys x landmarks) so a landmark's statistics
// and its accumulator column live in the same lanes.
// Wave w owns landmark tiles w*NTW .. w*NTW+NTW-1 (16 landmarks each).
template <typename IO, int D>
struct BvSmem {
  static constexpr int KP = D + 8;   // K row pitch (bf16 elements)
  static constexpr int VP = 64 + 8;  // V^T row pitch
  static constexpr int PL = IO::kBf16 ? 1 : 2;  // planes: bf16 input is exact, fp32 is split hi/lo
  uint16_t k[PL][64 * KP];
  uint16_t vt[PL][D * VP];
};

template <typename IO, int D, int NTW>
__global__ __launch_bounds__(256) void k_landmark_bv(const typename IO::T* __restrict__ Kin,
                                                     const typename IO::T* __restrict__ Vin,
                                                     const float* __restrict__ Qt, float* __restrict__ pacc,
                                                     float* __restrict__ pmax, float* __restrict__ psum,
                                                     int n, int m, int chunk, int nchunks, float sl2e) {
  using T = typename IO::T;
  using SM = BvSmem<IO, D>;
  constexpr int KC = (D + 31) / 32;  // 32-wide k chunks over the head dimension
  constexpr int MD = D / 16;         // 16-row tiles of V^T
  __shared__ SM sm;
  const int ch = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, c = lane & 15, g = lane >> 4;
  const int kbeg = ch * chunk, kend = min(n, kbeg + chunk);
  const T* Kh = Kin + (size_t)bh * n * D;
  const T* Vh = Vin + (size_t)bh * n * D;
  const float* qt = Qt + (size_t)bh * m * D;

  // Landmark-query operands (B of S^T = K Qt^T), split hi/lo, in registers.
  B8 qh[NTW][KC], ql[NTW][KC];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int lm = (wave * NTW + t) * 16 + c;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      float x[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int dd = kc * 32 + 8 * g + q;
        x[q] = (lm < m && dd < D) ? qt[lm * D + dd] : 0.f;
      }
      split8(x, qh[t][kc], ql[t][kc]);
    }
  }

  float run_max[NTW], run_sum[NTW];
  f32x4_t acc[NTW][MD];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    run_max[t] = -INFINITY;
    run_sum[t] = 0.f;
#pragma unroll
    for (int md = 0; md < MD; ++md) acc[t][md] = zero4();
  }

  for (int k0 = kbeg; k0 < kend; k0 += 64) {
    // Stage 64 keys of K (row-major) and V (transposed) in LDS, zero past kend.
    constexpr int SLOTS = D / 8;
    for (int e = tid; e < 64 * SLOTS; e += 256) {
      const int r = e / SLOTS, s8 = (e % SLOTS) * 8;
      float kx[8], vx[8];
      if (k0 + r < kend) {
        load8f<IO>(Kh + (size_t)(k0 + r) * D + s8, kx);
        load8f<IO>(Vh + (size_t)(k0 + r) * D + s8, vx);
      } else {
#pragma unroll
        for (int q = 0; q < 8; ++q) kx[q] = vx[q] = 0.f;
      }
      B8 kh, kl, vh, vl;
      split8(kx, kh, kl);
      split8(vx, vh, vl);
      *reinterpret_cast<uint4*>(&sm.k[0][r * SM::KP + s8]) = kh.q;
      if constexpr (SM::PL == 2) *reinterpret_cast<uint4*>(&sm.k[1][r * SM::KP + s8]) = kl.q;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        sm.vt[0][(s8 + q) * SM::VP + r] = vh.h[q];
        if constexpr (SM::PL == 2) sm.vt[1][(s8 + q) * SM::VP + r] = vl.h[q];
      }
    }
    __syncthreads();

    // K operand fragments for the 4 key tiles of 16 (shared by all landmark tiles).
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      if ((wave * NTW + t) * 16 >= m) continue;
      f32x4_t s[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        s[mt] = zero4();
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          B8 kh, kl;
          const int dd = kc * 32 + 8 * g;
          if (dd < D) {
            kh.q = *reinterpret_cast<const uint4*>(&sm.k[0][(mt * 16 + c) * SM::KP + dd]);
            if constexpr (SM::PL == 2) kl.q = *reinterpret_cast<const uint4*>(&sm.k[1][(mt * 16 + c) * SM::KP + dd]);
          } else {
            kh.q = make_uint4(0, 0, 0, 0);
            kl.q = make_uint4(0, 0, 0, 0);
          }
          if constexpr (SM::PL == 2) {
            s[mt] = mfma3(kh, kl, qh[t][kc], ql[t][kc], s[mt]);
          } else {
            s[mt] = mfma(kh, ql[t][kc], s[mt]);
            s[mt] = mfma(kh, qh[t][kc], s[mt]);
          }
        }
      }
      // Online softmax over this tile's keys for landmark (wave*NTW+t)*16 + c.
      float tmax = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = k0 + mt * 16 + 4 * g + i;
          s[mt][i] = (key < kend) ? s[mt][i] * sl2e : -INFINITY;
          tmax = fmaxf(tmax, s[mt][i]);
        }
      tmax = max_over_groups(tmax);
      const float nmax = fmaxf(run_max[t], tmax);
      const float corr = exp2f(run_max[t] - nmax);
      float psum_l = 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s[mt][i] = exp2f(s[mt][i] - nmax);
          psum_l += s[mt][i];
        }
      run_sum[t] = run_sum[t] * corr + sum_over_groups(psum_l);
      run_max[t] = nmax;
#pragma unroll
      for (int md = 0; md < MD; ++md) acc[t][md] *= corr;
      // acc^T (d x landmarks) += V^T (d x keys) P^T (keys x landmarks), keys in
      // chunks of 32 ordered {4g..4g+3, 16+4g..16+4g+3} within each chunk.
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        float p[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = s[2 * kk][i];
          p[4 + i] = s[2 * kk + 1][i];
        }
        B8 ph, pl;
        split8(p, ph, pl);
#pragma unroll
        for (int md = 0; md < MD; ++md) {
          const int dd = md * 16 + c;
          B8 vh, vl;
          const uint16_t* r0 = &sm.vt[0][dd * SM::VP + kk * 32 + 4 * g];
          vh.u[0] = *reinterpret_cast<const uint32_t*>(r0);
          vh.u[1] = *reinterpret_cast<const uint32_t*>(r0 + 2);
          vh.u[2] = *reinterpret_cast<const uint32_t*>(r0 + 16);
          vh.u[3] = *reinterpret_cast<const uint32_t*>(r0 + 18);
          if constexpr (SM::PL == 2) {
            const uint16_t* r1 = &sm.vt[1][dd * SM::VP + kk * 32 + 4 * g];
            vl.u[0] = *reinterpret_cast<const uint32_t*>(r1);
            vl.u[1] = *reinterpret_cast<const uint32_t*>(r1 + 2);
            vl.u[2] = *reinterpret_cast<const uint32_t*>(r1 + 16);
            vl.u[3] = *reinterpret_cast<const uint32_t*>(r1 + 18);
            acc[t][md] = mfma3(vh, vl, ph, pl, acc[t][md]);
          } else {
            acc[t][md] = mfma(vh, pl, acc[t][md]);
            acc[t][md] = mfma(vh, ph, acc[t][md]);
          }
        }
      }
    }
    __syncthreads();
  }

  // Partials for landmarks < m.
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int lm = (wave * NTW + t) * 16 + c;
    if (lm >= m) continue;
    const size_t base = ((size_t)bh * nchunks + ch) * m + lm;
    if (g == 0) {
      pmax[base] = run_max[t];
      psum[base] = run_sum[t];
    }
#pragma unroll
    for (int md = 0; md < MD; ++md) {
      float4 v = make_float4(acc[t][md][0], acc[t][md][1], acc[t][md][2], acc[t][md][3]);
      *reinterpret_cast<float4*>(&pacc[base * D + md * 16 + 4 * g]) = v;
    }
  }
}

// Fixed-order combine of the split-n partials.  grid (ceil(m*D/256), batch*heads).
__global__ __launch_bounds__(256) void k_bv_combine(const float* __restrict__ pacc, const float* __restrict__ pmax,
                                                    const float* __restrict__ psum, float* __restrict__ BV, int m,
                                                    int D, int nchunks) {
  const int bh = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= m * D) return;
  const int j = e / D, cc = e % D;
  const size_t b0 = (size_t)bh * nchunks * m + j;
  float M = -INFINITY;
  for (int ch = 0; ch < nchunks; ++ch) M = fmaxf(M, pmax[b0 + (size_t)ch * m]);
  float L = 0.f, S = 0.f;
  for (int ch = 0; ch < nchunks; ++ch) {
    const float w = exp2f(pmax[b0 + (size_t)ch * m] - M);
    L += psum[b0 + (size_t)ch * m] * w;
    S += pacc[(b0 + (size_t)ch * m) * D + cc] * w;
  }
  BV[((size_t)bh * m + j) * D + cc] = S / L;
}


// W (fp32 [bh][m][D]) -> bf16 hi/lo planes of W^T [bh][D][mpa], the A operand
// of the output stage: within each chunk of 32 landmarks, position 8g + q
// holds landmark 4g + q (q < 4) or 16 + 4g + q - 4 (q >= 4), the order in
// which that stage's softmax lanes hold their landmarks.  Padding is zero.
// grid (ceil(D*mpa/256), batch*heads).
__global__ __launch_bounds__(256) void k_prep_w(const float* __restrict__ W, uint16_t* __restrict__ wt_hi,
                                                uint16_t* __restrict__ wt_lo, int m, int D, int mpa) {
  const int bh = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= D * mpa) return;
  const int dd = e / mpa, pos = e % mpa;
  const int kk = pos >> 5, r = pos & 31, g = r >> 3, q = r & 7;
  const int lm = kk * 32 + (q < 4 ? 4 * g + q : 16 + 4 * g + q - 4);
  const float v = lm < m ? W[((size_t)bh * m + lm) * D + dd] : 0.f;
  uint16_t hi, lo;
  split_hi_lo(v, hi, lo);
  wt_hi[(size_t)bh * D * mpa + e] = hi;
  wt_lo[(size_t)bh * D * mpa + e] = lo;
}

// ---------------------------------------------------------------------------
// Stage launchers.

static int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

template <typename IO, int D>
static void seg_means_t(const Problem& p, const Ws& w, hipStream_t s) {
  using T = typename IO::T;
  const int BH = p.batch * p.heads;
  KernelTimer kt_("segment_mean", s);
  k_segment_mean<IO, D><<<dim3(p.m, BH, 2), 256, 0, s>>>(static_cast<const T*>(p.Q), static_cast<const T*>(p.K),
                                                         w.Qt, w.Kt, w.kt_hi, w.kt_lo, p.n, p.m, w.mpa);
}

hipError_t stage_segment_means(const Problem& p, const Ws& w, hipStream_t s) {
  switch (p.d) {
    case 16: p.bf16 ? seg_means_t<BF16, 16>(p, w, s) : seg_means_t<F32, 16>(p, w, s); break;
    case 32: p.bf16 ? seg_means_t<BF16, 32>(p, w, s) : seg_means_t<F32, 32>(p, w, s); break;
    case 64: p.bf16 ? seg_means_t<BF16, 64>(p, w, s) : seg_means_t<F32, 64>(p, w, s); break;
    case 128: p.bf16 ? seg_means_t<BF16, 128>(p, w, s) : seg_means_t<F32, 128>(p, w, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Landmark-side m x m products: fp32-grade for fp32 I/O, bf16x3 for bf16 I/O
// (where the output rounding dominates the error).
template <int PR>
static hipError_t pinv_t(const Problem& p, const Ws& w, hipStream_t s) {
  const int BH = p.batch * p.heads, m = p.m, D = p.d;
  const float sl2e = kLog2e / sqrtf((float)D);
  if (m <= 32) {
    KernelTimer kt_("pinv", s);
    k_pinv_lds<32, PR><<<BH, 256, sizeof(PinvSmem<32>), s>>>(w.Qt, w.Kt, w.A, w.Z, m, D, sl2e, p.iters);
  } else if (m <= 64) {
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_pinv_lds<64, PR>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       (int)sizeof(PinvSmem<64>));
    if (attr != hipSuccess) return attr;
    KernelTimer kt_("pinv", s);
    k_pinv_lds<64, PR><<<BH, 256, sizeof(PinvSmem<64>), s>>>(w.Qt, w.Kt, w.A, w.Z, m, D, sl2e, p.iters);
  } else {
    {
      KernelTimer kt_("landmark_softmax", s);
      k_landmark_softmax<PR><<<dim3(ceil_div(m, 16), BH), 256, 0, s>>>(w.Qt, w.Kt, w.A, m, D, sl2e);
    }
    // Ping-pong so that the last iterate lands in Z.
    float* zc = (p.iters % 2 == 0) ? w.Z : w.Z2;
    float* zn = (p.iters % 2 == 0) ? w.Z2 : w.Z;
    {
      KernelTimer kt_("pinv_start", s);
      k_pinv_start<<<BH, 256, 0, s>>>(w.A, zc, m);
    }
    const long long st = (long long)m * m;
    const dim3 grid(ceil_div(m, 64), ceil_div(m, 64), BH);
    for (int it = 0; it < p.iters; ++it) {
      KernelTimer kt_("pinv_mm", s);
      k_mm<PR><<<grid, 256, 0, s>>>(MMArgs{w.A, zc, w.X, w.T, m, m, m, st, st, st, 1.f, 0.f, -1.f, 7.f});
      k_mm<PR><<<grid, 256, 0, s>>>(MMArgs{w.X, w.T, w.U, nullptr, m, m, m, st, st, st, -1.f, 15.f, 0.f, 0.f});
      k_mm<PR><<<grid, 256, 0, s>>>(MMArgs{w.X, w.U, w.T, nullptr, m, m, m, st, st, st, -1.f, 13.f, 0.f, 0.f});
      k_mm<PR><<<grid, 256, 0, s>>>(MMArgs{zc, w.T, zn, nullptr, m, m, m, st, st, st, 0.25f, 0.f, 0.f, 0.f});
      float* tmp = zc;
      zc = zn;
      zn = tmp;
    }
  }
  return hipGetLastError();
}

hipError_t stage_pinv(const Problem& p, const Ws& w, hipStream_t s) {
  return p.bf16 ? pinv_t<3>(p, w, s) : pinv_t<6>(p, w, s);
}

template <typename IO, int D>
static void bv_t(const Problem& p, const Ws& w, hipStream_t s) {
  using T = typename IO::T;
  const int BH = p.batch * p.heads, m = p.m;
  const float sl2e = kLog2e / sqrtf((float)D);
  const T* K = static_cast<const T*>(p.K);
  const T* V = static_cast<const T*>(p.V);
  const dim3 g(w.nchunks, BH);
  {
    KernelTimer kt_("landmark_bv", s);
    if (m <= 64)
      k_landmark_bv<IO, D, 1><<<g, 256, 0, s>>>(K, V, w.Qt, w.pacc, w.pmax, w.psum, p.n, m, w.chunk, w.nchunks, sl2e);
    else if (m <= 128)
      k_landmark_bv<IO, D, 2><<<g, 256, 0, s>>>(K, V, w.Qt, w.pacc, w.pmax, w.psum, p.n, m, w.chunk, w.nchunks, sl2e);
    else
      k_landmark_bv<IO, D, 4><<<g, 256, 0, s>>>(K, V, w.Qt, w.pacc, w.pmax, w.psum, p.n, m, w.chunk, w.nchunks, sl2e);
  }
  KernelTimer kt_("bv_combine", s);
  k_bv_combine<<<dim3(ceil_div((long long)m * D, 256), BH), 256, 0, s>>>(w.pacc, w.pmax, w.psum, w.BV, m, D,
                                                                        w.nchunks);
}

hipError_t stage_bv(const Problem& p, const Ws& w, hipStream_t s) {
  switch (p.d) {
    case 16: p.bf16 ? bv_t<BF16, 16>(p, w, s) : bv_t<F32, 16>(p, w, s); break;
    case 32: p.bf16 ? bv_t<BF16, 32>(p, w, s) : bv_t<F32, 32>(p, w, s); break;
    case 64: p.bf16 ? bv_t<BF16, 64>(p, w, s) : bv_t<F32, 64>(p, w, s); break;
    case 128: p.bf16 ? bv_t<BF16, 128>(p, w, s) : bv_t<F32, 128>(p, w, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int PR>
static void w_t(const Problem& p, const Ws& w, hipStream_t s) {
  const int BH = p.batch * p.heads, m = p.m, D = p.d;
  {
    KernelTimer kt_("w_mm", s);
    k_mm<PR><<<dim3(ceil_div(D, 64), ceil_div(m, 64), BH), 256, 0, s>>>(
        MMArgs{w.Z, w.BV, w.W, nullptr, m, D, m, (long long)m * m, (long long)m * D, (long long)m * D, 1.f, 0.f,
               0.f, 0.f});
  }
  KernelTimer kt_("prep_w", s);
  k_prep_w<<<dim3(ceil_div((long long)D * w.mpa, 256), BH), 256, 0, s>>>(w.W, w.wt_hi, w.wt_lo, m, D, w.mpa);
}

hipError_t stage_w(const Problem& p, const Ws& w, hipStream_t s) {
  p.bf16 ? w_t<3>(p, w, s) : w_t<6>(p, w, s);
  return hipGetLastError();
}

}  // namespace nys

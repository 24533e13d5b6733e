// Nyström self-attention forward, landmark side: HIP kernels for gfx950 (CDNA4).
//
// Method: "Nyströmformer: A Nyström-Based Algorithm for Approximating
// Self-Attention" (paper deep-dive page, sec. 3.2 and 3.4).  Per (batch, head):
//   segment means Qt, Kt (Eq. 16)         -> k_segment_mean
//   A = softmax(Qt Kt^T / sqrt d), Z = Lemma-1 iterations from the
//   Pan-Schreiber start                    -> k_pinv_planes (m <= 64, bf16 I/O),
//                                             k_pinv_lds (m <= 64, fp32 I/O) or
//                                             k_landmark_softmax + k_pinv_start + k_mm chain
//   B V = softmax(Qt K^T / sqrt d) V       -> k_landmark_bv (split over keys,
//                                             online softmax), then k_bv_finish
//   W = Z (B V), W^T bf16 planes           -> k_bv_finish
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
  constexpr int SLOTS = D / VEC;   // 16-byte vectors per row
  constexpr int RS = 256 / SLOTS;  // rows covered per pass
  __shared__ float part[4][D];
  const int j = blockIdx.x, bh = blockIdx.y;
  const int seg = n / m;
  const T* X = (blockIdx.z == 0 ? Q : K) + ((size_t)bh * n + (size_t)j * seg) * D;
  float* out = (blockIdx.z == 0 ? Qt : Kt) + ((size_t)bh * m + j) * D;
  const int slot = threadIdx.x % SLOTS, r0 = threadIdx.x / SLOTS;
  float acc[VEC];
#pragma unroll
  for (int q = 0; q < VEC; ++q) acc[q] = 0.f;
  // 8 independent 16-byte loads in flight per thread, accumulated in row order.
  for (int r = r0; r < seg; r += 8 * RS) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int rr = r + u * RS;
      v[u] = rr < seg ? *reinterpret_cast<const uint4*>(X + (size_t)rr * D + slot * VEC) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if constexpr (IO::kBf16) {
        B8 b;
        b.q = v[u];
#pragma unroll
        for (int q = 0; q < VEC; ++q) acc[q] += bf16_to_f32(b.h[q]);
      } else {
        acc[0] += __uint_as_float(v[u].x);
        acc[1] += __uint_as_float(v[u].y);
        acc[2] += __uint_as_float(v[u].z);
        acc[3] += __uint_as_float(v[u].w);
      }
    }
  }
  // Butterfly over the lanes of a wave that share a slot (lane = r*SLOTS + slot),
  // then a fixed-order sum over the 4 waves.
#pragma unroll
  for (int o = SLOTS; o < 64; o <<= 1)
#pragma unroll
    for (int q = 0; q < VEC; ++q) acc[q] += shfl_xor(acc[q], o);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane < SLOTS) {
#pragma unroll
    for (int q = 0; q < VEC; ++q) part[wave][slot * VEC + q] = acc[q];
  }
  __syncthreads();
  if (threadIdx.x < D) {
    const float s = ((part[0][threadIdx.x] + part[1][threadIdx.x]) + part[2][threadIdx.x]) + part[3][threadIdx.x];
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
// Pseudoinverse for m <= 64 with bf16x3 products (bf16 I/O): every iterate is
// kept in LDS only as bf16 hi/lo planes, written once by the wave that
// produces it in the layout its consumers read, so a matrix-core fragment is
// one 16-byte LDS read per plane.  In C = P Q, P is read row-major ([row][k])
// and Q column-major ([col][k]).  A wave's result tile holds 4 consecutive
// rows of one column: column-major outputs are 8-byte writes, row-major ones
// 2-byte writes.
//   1. X  = A Z      -> X row-major, T1 = 7I - X column-major
//   2. U  = X T1     -> T3 = 15I - U column-major
//   3. V  = X T3     -> T5 = 13I - V column-major
//   4. Z' = Z T5 / 4 -> Z' row-major and column-major
// Row buffers: A, R0, R1 (X and Z alternate); column buffers K0, K1, K2
// (Z^T and the two T's rotate).
template <int MP>
struct PinvPlanes {
  static constexpr int LD = MP + 8;  // plane row pitch (bf16): rows stay 16-byte aligned
  static constexpr int PL = MP * LD;
  __align__(16) uint16_t rowb[3][2][PL];
  __align__(16) uint16_t colb[3][2][PL];
  float red[2][MP];
};

template <int MP>
__device__ __forceinline__ void put_split(uint16_t* hi, uint16_t* lo, int idx, float v) {
  uint16_t h, l;
  split_hi_lo(v, h, l);
  hi[idx] = h;
  lo[idx] = l;
}

// C = P Q (MP x MP) from planes; epi(ti, tj, acc) gets the tile whose lane
// (c, g) holds C[ti*16 + 4g + i][tj*16 + c], i = 0..3.
template <int MP, typename Epi>
__device__ __forceinline__ void planes_mm(const uint16_t* Ph, const uint16_t* Pl, const uint16_t* Qh,
                                          const uint16_t* Ql, Epi epi) {
  constexpr int LD = PinvPlanes<MP>::LD, NT = MP / 16, TPW = NT * NT / 4, KC = MP / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, c = lane & 15, g = lane >> 4;
  const int ti = (wave * TPW) / NT;  // every tile of a wave shares its row block
  B8 ah[KC], al[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    const int o = (ti * 16 + c) * LD + kc * 32 + 8 * g;
    ah[kc].q = *reinterpret_cast<const uint4*>(Ph + o);
    al[kc].q = *reinterpret_cast<const uint4*>(Pl + o);
  }
#pragma unroll
  for (int tt = 0; tt < TPW; ++tt) {
    const int tj = (wave * TPW + tt) % NT;
    f32x4_t acc = zero4();
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int o = (tj * 16 + c) * LD + kc * 32 + 8 * g;
      B8 bh, bl;
      bh.q = *reinterpret_cast<const uint4*>(Qh + o);
      bl.q = *reinterpret_cast<const uint4*>(Ql + o);
      acc = mfma3(ah[kc], al[kc], bh, bl, acc);
    }
    epi(ti, tj, acc);
  }
}

// Writers for a result tile (lane (c, g): rows ti*16+4g+i, column tj*16+c)
// of alpha*I + scale*acc.
template <int MP>
__device__ __forceinline__ void put_col(uint16_t* h, uint16_t* l, int ti, int tj, const f32x4_t& acc, float scale,
                                        float alpha) {
  constexpr int LD = PinvPlanes<MP>::LD;
  const int lane = threadIdx.x & 63, c = lane & 15, g = lane >> 4;
  const int col = tj * 16 + c, row0 = ti * 16 + 4 * g;
  B8 hv, lv;
#pragma unroll
  for (int i = 0; i < 4; ++i) split_hi_lo(scale * acc[i] + (row0 + i == col ? alpha : 0.f), hv.h[i], lv.h[i]);
  *reinterpret_cast<uint2*>(h + col * LD + row0) = make_uint2(hv.u[0], hv.u[1]);
  *reinterpret_cast<uint2*>(l + col * LD + row0) = make_uint2(lv.u[0], lv.u[1]);
}

template <int MP>
__device__ __forceinline__ void put_row(uint16_t* h, uint16_t* l, int ti, int tj, const f32x4_t& acc, float scale,
                                        float alpha) {
  constexpr int LD = PinvPlanes<MP>::LD;
  const int lane = threadIdx.x & 63, c = lane & 15, g = lane >> 4;
  const int col = tj * 16 + c, row0 = ti * 16 + 4 * g;
#pragma unroll
  for (int i = 0; i < 4; ++i) put_split<MP>(h, l, (row0 + i) * LD + col, scale * acc[i] + (row0 + i == col ? alpha : 0.f));
}

template <int MP>
__global__ __launch_bounds__(256) void k_pinv_planes(const float* __restrict__ Qt, const float* __restrict__ Kt,
                                                     float* __restrict__ Aout, float* __restrict__ Zout, int m,
                                                     int d, float sl2e, int iters) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  using SM = PinvPlanes<MP>;
  constexpr int LD = SM::LD, NT = MP / 16, SP = MP + 4;
  SM& sm = *reinterpret_cast<SM*>(smem_raw);
  // fp32 scratch for the scores / A, aliased on column buffers K1, K2.
  float* S = reinterpret_cast<float*>(&sm.colb[1][0][0]);
  static_assert(sizeof(float) * MP * SP <= sizeof(uint16_t) * 4 * SM::PL, "scratch does not fit");
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, c = lane & 15, g = lane >> 4;
  const float* qt = Qt + (size_t)bh * m * d;
  const float* kt = Kt + (size_t)bh * m * d;

  // Scaled scores (Kt Qt^T)^T: lane ends with row ti*16+c, columns tj*16+4g..+3.
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
      acc = mma_f32<3>(a, b, acc);
    }
    *reinterpret_cast<float4*>(&S[rq * SP + tj * 16 + 4 * g]) =
        make_float4(acc[0] * sl2e, acc[1] * sl2e, acc[2] * sl2e, acc[3] * sl2e);
  }
  __syncthreads();
  // Row softmax over the m real columns; padded rows/columns are 0.
  {
    constexpr int TPR = 256 / MP;
    const int r = tid / TPR, sub = tid % TPR;
    float mx = -INFINITY;
    for (int j = sub; j < m; j += TPR) mx = fmaxf(mx, S[r * SP + j]);
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) mx = fmaxf(mx, shfl_xor(mx, o));
    float s = 0.f;
    for (int j = sub; j < MP; j += TPR) {
      const float e = (r < m && j < m) ? exp2f(S[r * SP + j] - mx) : 0.f;
      S[r * SP + j] = e;
      s += e;
    }
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) s += shfl_xor(s, o);
    if (r < m) {
      const float inv = 1.f / s;
      for (int j = sub; j < m; j += TPR) S[r * SP + j] *= inv;
    }
  }
  __syncthreads();
  if (tid < MP) {
    float cs = 0.f, rs = 0.f;
    for (int i = 0; i < MP; ++i) {
      cs += fabsf(S[i * SP + tid]);
      rs += fabsf(S[tid * SP + i]);
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
  // A -> row planes (buffer 0) and the output; Z0 = cz A^T -> row planes R0 and
  // column planes K0 (Z0^T = cz A, i.e. K0[j][i] = cz A[j][i]).
  float* ao = Aout + (size_t)bh * m * m;
  for (int e = tid; e < MP * MP; e += 256) {
    const int i = e / MP, j = e % MP;
    const float a = S[i * SP + j];
    put_split<MP>(sm.rowb[0][0], sm.rowb[0][1], i * LD + j, a);
    put_split<MP>(sm.colb[0][0], sm.colb[0][1], i * LD + j, cz * a);
    put_split<MP>(sm.rowb[1][0], sm.rowb[1][1], j * LD + i, cz * a);
    if (i < m && j < m) ao[i * m + j] = a;
  }
  __syncthreads();

  int zr = 1, xr = 2;          // row buffers holding Z and X
  int zc = 0, ta = 1, tb = 2;  // column buffers holding Z^T and the two T's
  for (int it = 0; it < iters; ++it) {
    planes_mm<MP>(sm.rowb[0][0], sm.rowb[0][1], sm.colb[zc][0], sm.colb[zc][1],
                  [&](int ti, int tj, const f32x4_t& v) {
                    put_row<MP>(sm.rowb[xr][0], sm.rowb[xr][1], ti, tj, v, 1.f, 0.f);
                    put_col<MP>(sm.colb[ta][0], sm.colb[ta][1], ti, tj, v, -1.f, 7.f);
                  });
    __syncthreads();
    planes_mm<MP>(sm.rowb[xr][0], sm.rowb[xr][1], sm.colb[ta][0], sm.colb[ta][1],
                  [&](int ti, int tj, const f32x4_t& v) {
                    put_col<MP>(sm.colb[tb][0], sm.colb[tb][1], ti, tj, v, -1.f, 15.f);
                  });
    __syncthreads();
    planes_mm<MP>(sm.rowb[xr][0], sm.rowb[xr][1], sm.colb[tb][0], sm.colb[tb][1],
                  [&](int ti, int tj, const f32x4_t& v) {
                    put_col<MP>(sm.colb[ta][0], sm.colb[ta][1], ti, tj, v, -1.f, 13.f);
                  });
    __syncthreads();
    // Z' = Z T5 / 4 into the dead X row buffer and the dead T3 column buffer.
    planes_mm<MP>(sm.rowb[zr][0], sm.rowb[zr][1], sm.colb[ta][0], sm.colb[ta][1],
                  [&](int ti, int tj, const f32x4_t& v) {
                    put_row<MP>(sm.rowb[xr][0], sm.rowb[xr][1], ti, tj, v, 0.25f, 0.f);
                    put_col<MP>(sm.colb[tb][0], sm.colb[tb][1], ti, tj, v, 0.25f, 0.f);
                  });
    __syncthreads();
    const int t0 = zr;
    zr = xr;
    xr = t0;
    const int t1 = zc;
    zc = tb;
    tb = t1;
  }
  float* zo = Zout + (size_t)bh * m * m;
  for (int e = tid; e < m * m; e += 256) {
    const int i = e / m, j = e % m;
    zo[e] = bf16_to_f32(sm.rowb[zr][0][i * LD + j]) + bf16_to_f32(sm.rowb[zr][1][i * LD + j]);
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
  static constexpr int KP = D + 8;   // K row pitch (bf16 elements; rows 16-byte aligned)
  static constexpr int VP = 64 + 2;  // V^T row pitch: 33 dwords spreads the 2-row writes over all banks
  static constexpr int PL = IO::kBf16 ? 1 : 2;  // planes: bf16 input is exact, fp32 is split hi/lo
  __align__(16) uint16_t k[PL][64 * KP];
  __align__(16) uint16_t vt[PL][D * VP];
};

// One staging task = 2 consecutive keys x 8 features of K and of V.
template <typename IO>
struct BvStage {
  using T = typename IO::T;
  static constexpr int W = IO::kBf16 ? 1 : 2;  // uint4 per 8 elements
  uint4 k[2][W], v[2][W];
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

  // Staging is software-pipelined: the next tile's K and V rows are loaded
  // into registers while the current tile is computed from LDS.
  constexpr int SLOTS = D / 8;
  constexpr int TASKS = 32 * SLOTS;               // (key pair, 8-feature slot)
  constexpr int TPT = (TASKS + 255) / 256;         // tasks per thread
  BvStage<IO> st[TPT];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int e = tid + 256 * u;
      const int rp = e / SLOTS, s8 = (e % SLOTS) * 8;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int key = k0 + 2 * rp + h;
        const bool in = e < TASKS && key < kend;
#pragma unroll
        for (int w = 0; w < BvStage<IO>::W; ++w) {
          st[u].k[h][w] = in ? reinterpret_cast<const uint4*>(Kh + (size_t)key * D + s8)[w] : make_uint4(0, 0, 0, 0);
          st[u].v[h][w] = in ? reinterpret_cast<const uint4*>(Vh + (size_t)key * D + s8)[w] : make_uint4(0, 0, 0, 0);
        }
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int e = tid + 256 * u;
      if (e >= TASKS) continue;
      const int rp = e / SLOTS, s8 = (e % SLOTS) * 8;
      B8 kh[2], kl[2], vh[2], vl[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        if constexpr (IO::kBf16) {
          kh[h].q = st[u].k[h][0];
          vh[h].q = st[u].v[h][0];
        } else {
          float kx[8], vx[8];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            kx[q] = __uint_as_float((&st[u].k[h][0].x)[q]);
            kx[4 + q] = __uint_as_float((&st[u].k[h][1].x)[q]);
            vx[q] = __uint_as_float((&st[u].v[h][0].x)[q]);
            vx[4 + q] = __uint_as_float((&st[u].v[h][1].x)[q]);
          }
          split8(kx, kh[h], kl[h]);
          split8(vx, vh[h], vl[h]);
        }
        *reinterpret_cast<uint4*>(&sm.k[0][(2 * rp + h) * SM::KP + s8]) = kh[h].q;
        if constexpr (SM::PL == 2) *reinterpret_cast<uint4*>(&sm.k[1][(2 * rp + h) * SM::KP + s8]) = kl[h].q;
      }
      // V^T: feature s8+q, keys 2rp and 2rp+1 packed in one dword.
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        *reinterpret_cast<uint32_t*>(&sm.vt[0][(s8 + q) * SM::VP + 2 * rp]) =
            (uint32_t)vh[0].h[q] | ((uint32_t)vh[1].h[q] << 16);
        if constexpr (SM::PL == 2)
          *reinterpret_cast<uint32_t*>(&sm.vt[1][(s8 + q) * SM::VP + 2 * rp]) =
              (uint32_t)vl[0].h[q] | ((uint32_t)vl[1].h[q] << 16);
      }
    }
  };

  load_tile(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += 64) {
    store_tile();
    __syncthreads();
    if (k0 + 64 < kend) load_tile(k0 + 64);

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

// Finish of the split-n pass, one block per (16-feature slice, head):
//   BV[j][f] = sum_c pacc_c[j][f] 2^(pmax_c[j] - M_j) / sum_c psum_c[j] 2^(pmax_c[j] - M_j)
//   (M_j = max_c pmax_c[j]; chunks in fixed order), then W = Z BV for the
//   slice in fp32, then the slice's rows of the W^T bf16 planes [bh][D][mpa],
//   the A operand of the output stage: within each chunk of 32 landmarks,
//   position 8g + q holds landmark 4g + q (q < 4) or 16 + 4g + q - 4 (q >= 4),
//   the order in which that stage's softmax lanes hold their landmarks;
//   padding is zero.  grid (D/16, batch*heads).
template <bool ZLDS>
__global__ __launch_bounds__(1024) void k_bv_finish(const float* __restrict__ pacc, const float* __restrict__ pmax,
                                                    const float* __restrict__ psum, const float* __restrict__ Z,
                                                    float* __restrict__ BV, float* __restrict__ W,
                                                    uint16_t* __restrict__ wt_hi, uint16_t* __restrict__ wt_lo, int m,
                                                    int D, int nchunks, int mpa) {
  __shared__ float sbv[256][17];
  __shared__ float sw[256][17];
  __shared__ __align__(16) float sz[ZLDS ? 64 * 68 : 4];
  const int bh = blockIdx.y, f0 = blockIdx.x * 16, tid = threadIdx.x;
  const int f = tid & 15;
  const float* z = Z + (size_t)bh * m * m;
  if constexpr (ZLDS) {
    for (int e = tid; e < m * m; e += 1024) sz[(e / m) * 68 + e % m] = z[e];
  }
  const size_t pb = (size_t)bh * nchunks * m;
  for (int j = tid >> 4; j < m; j += 64) {
    // Online combine over the chunks in fixed order, 8 chunks' loads in flight.
    float M = -INFINITY, L = 0.f, S = 0.f;
    for (int c0 = 0; c0 < nchunks; c0 += 8) {
      float pm[8], ps[8], pa[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool in = c0 + u < nchunks;
        const size_t o = pb + (size_t)(in ? c0 + u : 0) * m + j;
        pm[u] = in ? pmax[o] : -INFINITY;
        ps[u] = in ? psum[o] : 0.f;
        pa[u] = in ? pacc[o * D + f0 + f] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (c0 + u < nchunks) {
          const float Mn = fmaxf(M, pm[u]);
          const float a = exp2f(M - Mn), b = exp2f(pm[u] - Mn);
          L = L * a + ps[u] * b;
          S = S * a + pa[u] * b;
          M = Mn;
        }
      }
    }
    const float v = S / L;
    sbv[j][f] = v;
    BV[((size_t)bh * m + j) * D + f0 + f] = v;
  }
  __syncthreads();
  for (int i = tid >> 4; i < m; i += 64) {
    float acc = 0.f;
    if constexpr (ZLDS) {
      for (int k = 0; k < m; ++k) acc = fmaf(sz[i * 68 + k], sbv[k][f], acc);
    } else {
      for (int k = 0; k < m; ++k) acc = fmaf(z[(size_t)i * m + k], sbv[k][f], acc);
    }
    sw[i][f] = acc;
    W[((size_t)bh * m + i) * D + f0 + f] = acc;
  }
  __syncthreads();
  for (int e = tid; e < 16 * mpa; e += 1024) {
    const int ff = e / mpa, pos = e % mpa;
    const int kk = pos >> 5, r = pos & 31, g = r >> 3, q = r & 7;
    const int lm = kk * 32 + (q < 4 ? 4 * g + q : 16 + 4 * g + q - 4);
    const float v = lm < m ? sw[lm][ff] : 0.f;
    uint16_t hi, lo;
    split_hi_lo(v, hi, lo);
    const size_t o = ((size_t)bh * D + f0 + ff) * mpa + pos;
    wt_hi[o] = hi;
    wt_lo[o] = lo;
  }
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
template <int MP>
static hipError_t pinv_planes_t(const Problem& p, const Ws& w, hipStream_t s) {
  const int BH = p.batch * p.heads;
  const float sl2e = kLog2e / sqrtf((float)p.d);
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_pinv_planes<MP>),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     (int)sizeof(PinvPlanes<MP>));
  if (attr != hipSuccess) return attr;
  KernelTimer kt_("pinv", s);
  k_pinv_planes<MP><<<BH, 256, sizeof(PinvPlanes<MP>), s>>>(w.Qt, w.Kt, w.A, w.Z, p.m, p.d, sl2e, p.iters);
  return hipSuccess;
}

template <int PR>
static hipError_t pinv_t(const Problem& p, const Ws& w, hipStream_t s) {
  const int BH = p.batch * p.heads, m = p.m, D = p.d;
  const float sl2e = kLog2e / sqrtf((float)D);
  if (PR == 3 && m <= 32) {
    hipError_t e = pinv_planes_t<32>(p, w, s);
    return e != hipSuccess ? e : hipGetLastError();
  } else if (PR == 3 && m <= 64) {
    hipError_t e = pinv_planes_t<64>(p, w, s);
    return e != hipSuccess ? e : hipGetLastError();
  } else if (m <= 32) {
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
  KernelTimer kt_("landmark_bv", s);
  if (m <= 64)
    k_landmark_bv<IO, D, 1><<<g, 256, 0, s>>>(K, V, w.Qt, w.pacc, w.pmax, w.psum, p.n, m, w.chunk, w.nchunks, sl2e);
  else if (m <= 128)
    k_landmark_bv<IO, D, 2><<<g, 256, 0, s>>>(K, V, w.Qt, w.pacc, w.pmax, w.psum, p.n, m, w.chunk, w.nchunks, sl2e);
  else
    k_landmark_bv<IO, D, 4><<<g, 256, 0, s>>>(K, V, w.Qt, w.pacc, w.pmax, w.psum, p.n, m, w.chunk, w.nchunks, sl2e);
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

hipError_t stage_bv_finish(const Problem& p, const Ws& w, hipStream_t s) {
  const int BH = p.batch * p.heads;
  KernelTimer kt_("bv_finish", s);
  if (p.m <= 64)
    k_bv_finish<true><<<dim3(p.d / 16, BH), 1024, 0, s>>>(w.pacc, w.pmax, w.psum, w.Z, w.BV, w.W, w.wt_hi, w.wt_lo,
                                                         p.m, p.d, w.nchunks, w.mpa);
  else
    k_bv_finish<false><<<dim3(p.d / 16, BH), 1024, 0, s>>>(w.pacc, w.pmax, w.psum, w.Z, w.BV, w.W, w.wt_hi, w.wt_lo,
                                                          p.m, p.d, w.nchunks, w.mpa);
  return hipGetLastError();
}

}  // namespace nys

// Nyström self-attention forward, landmark side: HIP kernels for gfx950 (CDNA4).
//
// Method: "Nyströmformer: A Nyström-Based Algorithm for Approximating
// Self-Attention" (paper deep-dive page, sec. 3.2 and 3.4).  Per (batch, head):
//   segment means Qt, Kt (Eq. 16)         -> k_segment_mean
//   A = softmax(Qt Kt^T / sqrt d), Z = Lemma-1 iterations from the
//   Pan-Schreiber start                    -> pinv_head inside k_landmark_pass (m <= 64,
//                                             bf16 I/O), k_pinv_lds (m <= 64, fp32 I/O) or
//                                             k_landmark_softmax + a k_mmr chain (m > 64)
//   B V = softmax(Qt K^T / sqrt d) V       -> bv_chunk inside k_landmark_pass (split over
//                                             keys, online softmax), then k_bv_finish
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
// One block per segment of l = ceil(n/m) contiguous rows; 16-byte coalesced
// loads, fp32 partial sums per thread, fixed-order reduction through LDS.
// When m does not divide n the sequence counts as padded with zero rows to
// m*l: a segment reads only its rows below n and still divides by l.  With
// per-sequence lengths, n is that batch entry's length (the row pitch of a
// head stays the buffer's n).
// Both landmark sets are also written as bf16 hi/lo planes [bh][mpa][D] (rows
// m..mpa-1 zero), the operand layout of the pseudoinverse's scores and of the
// output stage: Qt as it is, Kt pre-multiplied by log2(e)/sqrt(d), so that
// scores come out in base-2 units.
// WS (short segments): one wave per segment, four segments per
// block, grid (ceil(m/4), batch*heads, 2); the lanes of a wave cover whole
// rows, so a short segment is one round of loads and the sum needs only lane
// shuffles (no LDS, no barrier).
// SIN: Q and K rows where il says; otherwise the [batch][heads][n][d] layout.
template <typename IO, int D, bool WS = false, bool SIN = false>
__global__ __launch_bounds__(256) void k_segment_mean(const typename IO::T* __restrict__ Q,
                                                      const typename IO::T* __restrict__ K,
                                                      float* __restrict__ Qt, float* __restrict__ Kt,
                                                      uint16_t* __restrict__ kt_hi, uint16_t* __restrict__ kt_lo,
                                                      uint16_t* __restrict__ qt_hi, uint16_t* __restrict__ qt_lo,
                                                      const int* __restrict__ lens, int heads, int n, int m,
                                                      int mpa, float sl2e, unsigned* __restrict__ sync,
                                                      int nsync, InLayout il) {
  using T = typename IO::T;
  // The landmark pass's per-head counters start at zero (it runs after this
  // launch on the same stream).
  if ((blockIdx.x | blockIdx.y | blockIdx.z) == 0)
    for (int i = threadIdx.x; i < nsync; i += 256) sync[i] = 0u;
  constexpr int VEC = 16 / sizeof(T);
  constexpr int SLOTS = D / VEC;   // 16-byte vectors per row
  constexpr int RS = (WS ? 64 : 256) / SLOTS;  // rows covered per pass (by a wave with WS)
  __shared__ float part[4][D];
  const int j = WS ? 4 * blockIdx.x + (threadIdx.x >> 6) : blockIdx.x, bh = blockIdx.y;
  if (WS && j >= m) return;  // wave-uniform; no barrier follows with WS
  const int nb = seq_rows(lens, bh / heads, n);
  const int seg = max(1, (nb + m - 1) / m);  // l = 1 for a sequence shorter than m (empty included)
  const int rows = max(0, min(seg, nb - j * seg));  // real rows of this segment
  const int ild = SIN ? il.ld : D;
  const T* X = (blockIdx.z == 0 ? Q : K) +
               (SIN ? (bh / heads) * il.bs + (bh % heads) * il.hs + (size_t)j * seg * il.ld
                    : ((size_t)bh * n + (size_t)j * seg) * D);
  float* out = (blockIdx.z == 0 ? Qt : Kt) + ((size_t)bh * m + j) * D;
  const int slot = threadIdx.x % SLOTS, r0 = (WS ? threadIdx.x & 63 : threadIdx.x) / SLOTS;
  float acc[VEC];
#pragma unroll
  for (int q = 0; q < VEC; ++q) acc[q] = 0.f;
  // 8 independent 16-byte loads in flight per thread, accumulated in row order.
  for (int r = r0; r < rows; r += 8 * RS) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int rr = r + u * RS;
      v[u] = rr < rows ? *reinterpret_cast<const uint4*>(X + (size_t)rr * ild + slot * VEC) : make_uint4(0, 0, 0, 0);
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
  auto emit = [&](int f, float s) {  // feature f of this segment's mean, sum s
    const float mean = s / (float)seg;
    out[f] = mean;
    uint16_t* ph = blockIdx.z == 1 ? kt_hi : qt_hi;
    uint16_t* pl = blockIdx.z == 1 ? kt_lo : qt_lo;
    uint16_t hi, lo;
    split_hi_lo(blockIdx.z == 1 ? mean * sl2e : mean, hi, lo);
    const size_t o = ((size_t)bh * mpa + j) * D + f;
    ph[o] = hi;
    pl[o] = lo;
    if (j == m - 1) {
      for (int r = m; r < mpa; ++r) {
        ph[((size_t)bh * mpa + r) * D + f] = 0;
        pl[((size_t)bh * mpa + r) * D + f] = 0;
      }
    }
  };
  if constexpr (WS) {
    if (lane < SLOTS) {
#pragma unroll
      for (int q = 0; q < VEC; ++q) emit(slot * VEC + q, acc[q]);
    }
    return;
  }
  if (lane < SLOTS) {
#pragma unroll
    for (int q = 0; q < VEC; ++q) part[wave][slot * VEC + q] = acc[q];
  }
  __syncthreads();
  if (threadIdx.x < D) {
    const float s = ((part[0][threadIdx.x] + part[1][threadIdx.x]) + part[2][threadIdx.x]) + part[3][threadIdx.x];
    emit(threadIdx.x, s);
  }
}

// ---------------------------------------------------------------------------
// Pseudoinverse for m <= 64: one block (16 waves) per head, every iterate in LDS.
// Products are split-bf16 on the matrix cores with fp32 accumulation (PR = 6,
// the three-way split, for fp32 I/O).
constexpr int kPinvWaves = 16;  // one 16 x 16 output tile per wave and product at m = 64

template <int MP>
struct PinvSmem {
  __align__(16) float A[MP][MP + 4];
  float Z[MP][MP + 4];
  float X[MP][MP + 4];
  float T[MP][MP + 4];
  float U[MP][MP + 4];
  float red[2][MP];
  float colp[64 * kPinvWaves / MP][MP];  // column sums of A over parts of its rows
};

// C = P * Qm over MP x MP LDS matrices, computed as C^T = Qm^T P^T so that a
// lane ends with 4 consecutive columns of one row of C: epi(row, col0, v)
// stores v[i] at (row, col0 + i) with one 16-byte LDS write per matrix.
template <int MP, int PR, typename Epi>
__device__ __forceinline__ void lds_mm(const float (*P)[MP + 4], const float (*Qm)[MP + 4], Epi epi) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  constexpr int NT = MP / 16;
  for (int t = wave; t < NT * NT; t += kPinvWaves) {
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

// The pseudoinverse of head bh by a block of 64 * kPinvWaves threads.
template <int MP, int PR>
__device__ __forceinline__ void pinv_lds_head(unsigned char* smem_raw, int bh, const float* __restrict__ Qt,
                                              const float* __restrict__ Kt, float* __restrict__ Aout,
                                              float* __restrict__ Zout, int m, int d, float sl2e, int iters,
                                              float* __restrict__ zsave, int zmp) {
  PinvSmem<MP>& sm = *reinterpret_cast<PinvSmem<MP>*>(smem_raw);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, c = lane & 15, g = lane >> 4;
  const float* qt = Qt + (size_t)bh * m * d;
  const float* kt = Kt + (size_t)bh * m * d;
  constexpr int NT = MP / 16;

  // Scaled scores Qt Kt^T * log2(e)/sqrt(d); rows/cols >= m are zero padding.
  // Computed as (Kt Qt^T)^T: a lane ends with row ti*16+c, columns tj*16+4g..+3.
  // Every fragment load (clamped in bounds, masked) is issued before the
  // first product.
  for (int t = wave; t < NT * NT; t += kPinvWaves) {
    const int ti = t / NT, tj = t % NT;
    const int rq = ti * 16 + c, rk = tj * 16 + c;
    float a[4][8], b[4][8];
#pragma unroll
    for (int kq = 0; kq < 4; ++kq)
      if (32 * kq < d) {
        load8_masked(kt, rk, m, 32 * kq + 8 * g, d, d, a[kq]);
        load8_masked(qt, rq, m, 32 * kq + 8 * g, d, d, b[kq]);
      }
    f32x4_t acc = zero4();
#pragma unroll
    for (int kq = 0; kq < 4; ++kq)
      if (32 * kq < d) acc = mma_f32<PR>(a[kq], b[kq], acc);
    *reinterpret_cast<float4*>(&sm.A[rq][tj * 16 + 4 * g]) =
        make_float4(acc[0] * sl2e, acc[1] * sl2e, acc[2] * sl2e, acc[3] * sl2e);
  }
  __syncthreads();

  // Row softmax over the m real columns (padded rows and columns become 0),
  // in registers: TPR threads per row, CPT consecutive columns each; the
  // row sums of A go to red[1].
  if (tid < 256) {
    constexpr int TPR = 256 / MP, CPT = MP / TPR;
    const int r = tid / TPR, j0 = (tid % TPR) * CPT;
    float v[CPT];
#pragma unroll
    for (int u = 0; u < CPT / 4; ++u) {
      const float4 x = *reinterpret_cast<const float4*>(&sm.A[r][j0 + 4 * u]);
      v[4 * u] = x.x;
      v[4 * u + 1] = x.y;
      v[4 * u + 2] = x.z;
      v[4 * u + 3] = x.w;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int q = 0; q < CPT; ++q)
      if (j0 + q < m) mx = fmaxf(mx, v[q]);
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) mx = fmaxf(mx, shfl_xor(mx, o));
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      v[q] = (r < m && j0 + q < m) ? exp2f(v[q] - mx) : 0.f;
      s += v[q];
    }
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) s += shfl_xor(s, o);
    const float inv = r < m ? 1.f / s : 0.f;
    float rs = 0.f;
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      v[q] *= inv;
      rs += v[q];
    }
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) rs += shfl_xor(rs, o);
#pragma unroll
    for (int u = 0; u < CPT / 4; ++u)
      *reinterpret_cast<float4*>(&sm.A[r][j0 + 4 * u]) = make_float4(v[4 * u], v[4 * u + 1], v[4 * u + 2], v[4 * u + 3]);
    if (tid % TPR == 0) sm.red[1][r] = rs;
  }
  __syncthreads();

  // Z0 = A^T / (max column abs sum * max row abs sum) (entries are >= 0).
  // Column sums in parts of RPP rows (fixed order), then over the parts.
  {
    constexpr int NPART = 64 * kPinvWaves / MP, RPP = MP / NPART > 0 ? MP / NPART : 1;
    const int col = tid % MP, part = tid / MP;
    if (part < NPART && part * RPP < MP) {
      float cs = 0.f;
#pragma unroll
      for (int rr = 0; rr < RPP; ++rr) cs += sm.A[part * RPP + rr][col];
      sm.colp[part][col] = cs;
    }
  }
  __syncthreads();
  if (wave == 0) {
    constexpr int NPART = 64 * kPinvWaves / MP;
    float cs = 0.f, rs = 0.f;
    if (lane < MP) {
#pragma unroll
      for (int pp = 0; pp < NPART; ++pp) cs += sm.colp[pp][lane];
      rs = sm.red[1][lane];
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      cs = fmaxf(cs, shfl_xor(cs, o));
      rs = fmaxf(rs, shfl_xor(rs, o));
    }
    if (lane == 0) sm.red[0][0] = 1.f / (cs * rs);
  }
  __syncthreads();
  const float cz = sm.red[0][0];
  for (int e = tid; e < MP * MP; e += 64 * kPinvWaves) {
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
    if (zsave) {
      // For the backward pass: Z_k, X_k, T1_k = 15I - U, T2_k = 13I - T
      // ([zmp][zmp] fp32 each, zero beyond m).
      float* zs = zsave + ((size_t)bh * iters + it) * 4 * zmp * zmp;
      for (int e = tid; e < zmp * zmp; e += 64 * kPinvWaves) {
        const int i = e / zmp, j = e % zmp;
        const bool in = i < MP && j < MP;
        const float dg = i == j ? 1.f : 0.f;
        zs[e] = in ? Z[i][j] : 0.f;
        zs[zmp * zmp + e] = in ? Xb[i][j] : 0.f;
        zs[2 * zmp * zmp + e] = in ? 15.f * dg - sm.U[i][j] : 0.f;
        zs[3 * zmp * zmp + e] = in ? 13.f * dg - sm.T[i][j] : 0.f;
      }
    }
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
  for (int e = tid; e < m * m; e += 64 * kPinvWaves) {
    const int i = e / m, j = e % m;
    ao[e] = sm.A[i][j];
    zo[e] = Z[i][j];
  }
}

template <int MP, int PR>
__global__ __launch_bounds__(64 * kPinvWaves) void k_pinv_lds(const float* __restrict__ Qt, const float* __restrict__ Kt,
                                                  float* __restrict__ Aout, float* __restrict__ Zout, int m,
                                                  int d, float sl2e, int iters, float* __restrict__ zsave,
                                                  int zmp) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  pinv_lds_head<MP, PR>(smem_raw, (int)blockIdx.x, Qt, Kt, Aout, Zout, m, d, sl2e, iters, zsave, zmp);
}

// ---------------------------------------------------------------------------
// Pseudoinverse for m <= MP (MP = 32 or 64) with bf16x3 products (bf16 I/O),
// one block of 8 waves per head.
//
// Lemma 1's step Z <- Z (13I - X(15I - X(7I - X))) / 4 with X = A Z is run
// through the residual E = I - A Z.  Since 13 - 15x + 7x^2 - x^3 = 4 (1 + e +
// e^2 + e^3/4) and 1 - x (13 - 15x + 7x^2 - x^3)/4 = (3e^3 + e^4)/4 for
// x = 1 - e, the same iterates follow from
//   E_0 = I - A Z_0,  Z_0 = A^T / (||A||_1 ||A||_inf),
//   Z_{t+1} = Z_t P_t,  P_t = I + E_t + E_t^2 + E_t^3 / 4,
//   E_{t+1} = (3 E_t^3 + E_t^4) / 4 = E_t^2 N_t,  N_t = (3 E_t + E_t^2) / 4,
// an identity of the printed iteration, not an approximation.  (I is the
// identity on the m real landmarks: the zero padding up to MP stays zero.)
//
// E_t and every polynomial in it are symmetric, so the right operand of a
// product reads its columns as rows, and Z_{t+1}^T = P_t Z_t^T reads Z by
// rows too: every matrix sits in LDS as row-major bf16 hi/lo planes and every
// operand fragment is one 16-byte read per plane.  A result tile (lane (c, g)
// holds rows 4g..4g+3 of column c) is stored as the rows of the transposed
// tile (8-byte writes), which for a symmetric result is the result itself and
// for Z^T is Z.
//
// Two groups of 4 waves, each wave owning one quadrant of tiles (rows of
// tiles TA.., columns TB..) of the products its group forms, so that two
// waves share each SIMD and one's conversions and LDS traffic overlap the
// other's matrix-core work.  Per step, two product levels and two barriers:
//   level 1: E group: E^2 = E E, N = (3E + E^2)/4      Z group: Z_t^T = P_{t-1} Z_{t-1}^T
//   level 2: E group: E^3 = E E^2, P_t = I + E + E^2 + E^3/4
//            Z group: E_{t+1} = E^2 N (also handed to the E group in fp32)
template <int MP>
struct PinvSmemE {
  static constexpr int LD = MP + 8;  // plane row pitch (bf16): 16-byte aligned rows, rows spread over banks
  static constexpr int PL = MP * LD;
  static constexpr int SP = MP + 4;  // fp32 score row pitch
  static constexpr int NW = MP / 32; // tiles per dimension of a quadrant
  __align__(16) uint16_t e[2][PL];   // E_t planes [hi, lo]
  __align__(16) uint16_t e2[2][PL];  // E_t^2; the fp32 scores and A alias it before the iterations
  __align__(16) uint16_t nn[2][PL];  // N_t
  __align__(16) uint16_t p[2][PL];   // P_t; A's planes before the iterations
  __align__(16) uint16_t z[2][PL];   // Z_t
  float ex[4][NW * NW * 4][64];      // E_{t+1} in fp32, quadrant by quadrant, handed from the Z group to the E group
  float colp[256 / MP][MP];          // partial column sums of A
  float rows[MP];                    // row sums of A
  __device__ float* S() { return reinterpret_cast<float*>(&e2[0][0]); }
  static_assert(sizeof(float) * MP * SP <= sizeof(uint16_t) * 2 * PL, "scores do not fit the E^2 planes");
};

template <int MP>
struct PinvQuad {
  static constexpr int NT = MP / 16;  // 16-row tiles per dimension
  static constexpr int NW = NT / 2;   // tiles per dimension of a wave's quadrant
  static constexpr int KC = MP / 32;  // 32-wide contraction chunks
};

// Row fragments of rows 16 t0 + 16 u + c (u < NW), every contraction chunk,
// from a plane pair.
template <int MP>
__device__ __forceinline__ void rows_frag(const uint16_t (&pl)[2][PinvSmemE<MP>::PL], int t0,
                                          B8 (&h)[PinvQuad<MP>::NW][PinvQuad<MP>::KC],
                                          B8 (&l)[PinvQuad<MP>::NW][PinvQuad<MP>::KC]) {
  constexpr int LD = PinvSmemE<MP>::LD, NW = PinvQuad<MP>::NW, KC = PinvQuad<MP>::KC;
  const int lane = threadIdx.x & 63, c = lane & 15, g = lane >> 4;
#pragma unroll
  for (int u = 0; u < NW; ++u)
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const int o = (16 * (t0 + u) + c) * LD + 32 * kc + 8 * g;
      h[u][kc].q = *reinterpret_cast<const uint4*>(&pl[0][o]);
      l[u][kc].q = *reinterpret_cast<const uint4*>(&pl[1][o]);
    }
}

// acc[u][v] = (left rows) (right rows)^T for the wave's quadrant (bf16x3).
template <int MP>
__device__ __forceinline__ void quad_mm(const B8 (&ah)[PinvQuad<MP>::NW][PinvQuad<MP>::KC],
                                        const B8 (&al)[PinvQuad<MP>::NW][PinvQuad<MP>::KC],
                                        const B8 (&bh)[PinvQuad<MP>::NW][PinvQuad<MP>::KC],
                                        const B8 (&bl)[PinvQuad<MP>::NW][PinvQuad<MP>::KC],
                                        f32x4_t (&acc)[PinvQuad<MP>::NW][PinvQuad<MP>::NW]) {
  constexpr int NW = PinvQuad<MP>::NW, KC = PinvQuad<MP>::KC;
#pragma unroll
  for (int u = 0; u < NW; ++u)
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      acc[u][v] = zero4();
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) acc[u][v] = mfma3(ah[u][kc], al[u][kc], bh[v][kc], bl[v][kc], acc[u][v]);
    }
}

// Stores the quadrant's tiles transposed (rows of tile (TB + v, TA + u)) into
// a plane pair, split into bf16 hi/lo.
template <int MP>
__device__ __forceinline__ void quad_store_t(uint16_t (&pl)[2][PinvSmemE<MP>::PL], int TA, int TB,
                                             const f32x4_t (&v)[PinvQuad<MP>::NW][PinvQuad<MP>::NW]) {
  constexpr int LD = PinvSmemE<MP>::LD, NW = PinvQuad<MP>::NW;
  const int lane = threadIdx.x & 63, c = lane & 15, g = lane >> 4;
#pragma unroll
  for (int u = 0; u < NW; ++u)
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      uint2 hv, lv;
      split_pair(v[u][w][0], v[u][w][1], hv.x, lv.x);
      split_pair(v[u][w][2], v[u][w][3], hv.y, lv.y);
      const int o = (16 * (TB + w) + c) * LD + 16 * (TA + u) + 4 * g;
      *reinterpret_cast<uint2*>(&pl[0][o]) = hv;
      *reinterpret_cast<uint2*>(&pl[1][o]) = lv;
    }
}

// Pseudoinverse of one head, run by a block of 512 threads.  The landmarks
// come as the bf16 hi/lo planes the segment means wrote ([bh][MP][D], Kt
// pre-scaled by log2(e)/sqrt(d)).  SAVE: also write each step's Z_k,
// X_k = A Z_k, T1_k = X_k (7I - X_k) and T2_k = X_k (15I - T1_k) to zsave
// ([zmp][zmp] fp32 each, zero beyond m) for the backward pass; in the residual
// form X = I - E, T1 = 6I - 5E - E^2 and T2 = 9I - 4E - 4E^2 - E^3.  The plain
// forward's kernel has none of it.
//
// The final Z goes to Zout with device-coherent stores and, as bf16 hi/lo
// row planes (pitch MP + 8), to zdst: LDS that aliases only the E planes,
// which no wave reads after the last step.
template <int MP, int D, bool SAVE>
__device__ __forceinline__ void pinv_head(PinvSmemE<MP>& sm, int bh, const uint16_t* __restrict__ qt_hi,
                                          const uint16_t* __restrict__ qt_lo, const uint16_t* __restrict__ kt_hi,
                                          const uint16_t* __restrict__ kt_lo, float* __restrict__ Aout,
                                          float* __restrict__ Zout, int m, int iters, float* __restrict__ zsave,
                                          int zmp, uint16_t (*zdst)[PinvSmemE<MP>::PL]) {
  using SM = PinvSmemE<MP>;
  using QD = PinvQuad<MP>;
  constexpr int SP = SM::SP, NW = QD::NW, KC = QD::KC;
  constexpr int TPR = 256 / MP, CPT = MP / TPR;  // softmax (threads 0..255): threads per row, columns per thread
  constexpr int KCD = (D + 31) / 32;             // 32-wide chunks of the head dimension
  float* const S = sm.S();
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, c = lane & 15, g = lane >> 4;
  const bool egrp = wave < 4;  // E group (waves 0..3) or Z group (waves 4..7); wave-uniform
  const int qd = wave & 3;
  const int TA = NW * (qd >> 1), TB = NW * (qd & 1);  // the wave's quadrant: row tiles TA.., column tiles TB..

  // Diagonal of the m real landmarks within the quadrant: element i of tile
  // (u, v) is on it iff the quadrant is diagonal, u == v, 4g + i == c, and the
  // row is below m.
  float dgv[NW][4];
#pragma unroll
  for (int u = 0; u < NW; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) dgv[u][i] = (TA == TB && 4 * g + i == c && 16 * (TA + u) + c < m) ? 1.f : 0.f;
  auto dg = [&](int u, int v, int i) { return u == v ? dgv[u][i] : 0.f; };

  // Scores in base-2 units (E group), computed transposed (S^T = Kt' Qt^T) so
  // that a lane ends with row 16 (TB + v) + c, columns 16 (TA + u) + 4g .. +3:
  // one 16-byte store per tile.  Fragments are 16-byte loads of the planes
  // (rows past m are zero there), all issued before the first product.
  if (egrp) {
    B8 kh[NW][KCD], kl[NW][KCD], qh[NW][KCD], ql[NW][KCD];
#pragma unroll
    for (int u = 0; u < NW; ++u)
#pragma unroll
      for (int kc = 0; kc < KCD; ++kc) {
        const int col = min(32 * kc + 8 * g, D - 8);
        const size_t ok_ = ((size_t)bh * MP + 16 * (TA + u) + c) * D + col;
        const size_t oq_ = ((size_t)bh * MP + 16 * (TB + u) + c) * D + col;
        kh[u][kc].q = *reinterpret_cast<const uint4*>(kt_hi + ok_);
        kl[u][kc].q = *reinterpret_cast<const uint4*>(kt_lo + ok_);
        qh[u][kc].q = *reinterpret_cast<const uint4*>(qt_hi + oq_);
        ql[u][kc].q = *reinterpret_cast<const uint4*>(qt_lo + oq_);
        if (32 * kc + 8 * g >= D) {  // d = 16: lanes past the head dimension contribute zero
          kh[u][kc].q = kl[u][kc].q = make_uint4(0, 0, 0, 0);
        }
      }
#pragma unroll
    for (int u = 0; u < NW; ++u)
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        f32x4_t acc = zero4();
#pragma unroll
        for (int kc = 0; kc < KCD; ++kc) acc = mfma3(kh[u][kc], kl[u][kc], qh[v][kc], ql[v][kc], acc);
        *reinterpret_cast<float4*>(&S[(16 * (TB + v) + c) * SP + 16 * (TA + u) + 4 * g]) =
            make_float4(acc[0], acc[1], acc[2], acc[3]);
      }
  }
  __syncthreads();

  // Row softmax (threads 0..255): TPR adjacent lanes per row, CPT columns
  // each; padded rows and columns become 0.  A goes to global memory, to S
  // (fp32, in place, for the column sums) and to the P planes (bf16 hi/lo,
  // row-major); row sums to sm.rows.
  if (tid < 256) {
    const int r = tid / TPR, sub = tid % TPR, j0 = sub * CPT;
    float a[CPT];
#pragma unroll
    for (int u = 0; u < CPT / 4; ++u) {
      const float4 v = *reinterpret_cast<const float4*>(&S[r * SP + j0 + 4 * u]);
      a[4 * u] = v.x; a[4 * u + 1] = v.y; a[4 * u + 2] = v.z; a[4 * u + 3] = v.w;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int q = 0; q < CPT; ++q)
      if (j0 + q < m) mx = fmaxf(mx, a[q]);
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) mx = fmaxf(mx, shfl_xor(mx, o));
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      a[q] = (r < m && j0 + q < m) ? __builtin_amdgcn_exp2f(a[q] - mx) : 0.f;  // arguments <= 0
      sum += a[q];
    }
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) sum += shfl_xor(sum, o);
    const float inv = r < m ? 1.f / sum : 0.f;
    float rs = 0.f;
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      a[q] *= inv;
      rs += a[q];
    }
#pragma unroll
    for (int o = 1; o < TPR; o <<= 1) rs += shfl_xor(rs, o);
#pragma unroll
    for (int u = 0; u < CPT / 4; ++u) {
      *reinterpret_cast<float4*>(&S[r * SP + j0 + 4 * u]) = make_float4(a[4 * u], a[4 * u + 1], a[4 * u + 2], a[4 * u + 3]);
      uint2 hv, lv;
      split_pair(a[4 * u], a[4 * u + 1], hv.x, lv.x);
      split_pair(a[4 * u + 2], a[4 * u + 3], hv.y, lv.y);
      *reinterpret_cast<uint2*>(&sm.p[0][r * SM::LD + j0 + 4 * u]) = hv;
      *reinterpret_cast<uint2*>(&sm.p[1][r * SM::LD + j0 + 4 * u]) = lv;
    }
    if (sub == 0) sm.rows[r] = rs;
    if (r < m) {
      float* ao = Aout + (size_t)bh * m * m + (size_t)r * m;
      if (m == MP) {
#pragma unroll
        for (int u = 0; u < CPT / 4; ++u)
          *reinterpret_cast<float4*>(ao + j0 + 4 * u) = make_float4(a[4 * u], a[4 * u + 1], a[4 * u + 2], a[4 * u + 3]);
      } else {
#pragma unroll
        for (int q = 0; q < CPT; ++q)
          if (j0 + q < m) ao[j0 + q] = a[q];
      }
    }
  }
  __syncthreads();
  if (tid < 256) {  // partial column sums over parts of the rows
    const int col = tid % MP, part = tid / MP;
    constexpr int RPP = MP * MP / 256;  // rows per part
    float s = 0.f;
#pragma unroll 4
    for (int rr = 0; rr < RPP; ++rr) s += S[(part * RPP + rr) * SP + col];
    sm.colp[part][col] = s;
  }
  // A's row fragments (the A planes are complete since the last barrier).
  B8 aah[NW][KC], aal[NW][KC];
  rows_frag<MP>(sm.p, TA, aah, aal);
  __syncthreads();
  // ||A||_1 (max column sum) and ||A||_inf (max row sum; entries are >= 0).
  float cz;
  {
    constexpr int NP = 256 / MP;  // parts of the column sums
    const int k = lane % MP;
    float cs = 0.f;
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) cs += sm.colp[pp][k];
    float rm = sm.rows[k];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      cs = fmaxf(cs, shfl_xor(cs, o));
      rm = fmaxf(rm, shfl_xor(rm, o));
    }
    cz = 1.f / (cs * rm);
  }

  // E group: E_0 = I - cz A A^T.  Z group: Z_0^T = cz A, in the layout of
  // every later Z^T product, as A times the identity on the matrix cores (hi
  // and lo planes of A; the identity is exact in bf16), so that its tiles are
  // stored transposed as Z_0's rows like any other product.  Neither buffer
  // is read before the next barrier.
  f32x4_t ef[NW][NW], zt[NW][NW];
  if (egrp) {
    B8 abh[NW][KC], abl[NW][KC];
    rows_frag<MP>(sm.p, TB, abh, abl);
    quad_mm<MP>(aah, aal, abh, abl, ef);
#pragma unroll
    for (int u = 0; u < NW; ++u)
#pragma unroll
      for (int v = 0; v < NW; ++v)
#pragma unroll
        for (int i = 0; i < 4; ++i) ef[u][v][i] = dg(u, v, i) - cz * ef[u][v][i];
    quad_store_t<MP>(sm.e, TA, TB, ef);
  } else {
    B8 id[NW][KC];
#pragma unroll
    for (int v = 0; v < NW; ++v)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
#pragma unroll
        for (int q = 0; q < 8; ++q) id[v][kc].h[q] = 32 * kc + 8 * g + q == 16 * (TB + v) + c ? 0x3F80 : 0;
#pragma unroll
    for (int u = 0; u < NW; ++u)
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        f32x4_t acc = zero4();
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          acc = mfma(aal[u][kc], id[v][kc], acc);
          acc = mfma(aah[u][kc], id[v][kc], acc);
        }
        zt[u][v] = cz * acc;
      }
    quad_store_t<MP>(sm.z, TA, TB, zt);
  }

  // For the backward pass: the quadrant of a step's matrix ([zmp][zmp] fp32);
  // trans: v holds tiles of the transpose (Z^T).
  auto save = [&](const f32x4_t (&v)[NW][NW], int it, int which, bool trans) {
    float* zs = zsave + (((size_t)bh * iters + it) * 4 + which) * zmp * zmp;
#pragma unroll
    for (int u = 0; u < NW; ++u)
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int a = 16 * (TA + u) + 4 * g + i, b = 16 * (TB + w) + c;
          const int row = trans ? b : a, col = trans ? a : b;
          if (row < zmp && col < zmp) zs[(size_t)row * zmp + col] = v[u][w][i];
        }
  };

  __syncthreads();  // E_0 and Z_0 planes visible
  for (int it = 0; it < iters; ++it) {
    // Level 1.
    B8 eah[NW][KC], eal[NW][KC];  // E rows TA (E group), kept for level 2
    f32x4_t e2[NW][NW];
    if (egrp) {
      B8 ebh[NW][KC], ebl[NW][KC];
      rows_frag<MP>(sm.e, TA, eah, eal);
      rows_frag<MP>(sm.e, TB, ebh, ebl);
      quad_mm<MP>(eah, eal, ebh, ebl, e2);
      f32x4_t nt[NW][NW];
#pragma unroll
      for (int u = 0; u < NW; ++u)
#pragma unroll
        for (int v = 0; v < NW; ++v) nt[u][v] = 0.75f * ef[u][v] + 0.25f * e2[u][v];
      // Neither E^2 nor N is read again before the next barrier (their
      // readers of the last step finished before its closing barrier).
      quad_store_t<MP>(sm.e2, TA, TB, e2);
      quad_store_t<MP>(sm.nn, TA, TB, nt);
    } else if (it > 0) {  // Z_t^T = P_{t-1} Z_{t-1}^T (Z_0 is given)
      B8 pah[NW][KC], pal[NW][KC], zbh[NW][KC], zbl[NW][KC];
      rows_frag<MP>(sm.p, TA, pah, pal);
      rows_frag<MP>(sm.z, TB, zbh, zbl);
      quad_mm<MP>(pah, pal, zbh, zbl, zt);
    }
    if constexpr (SAVE) {
      if (!egrp) save(zt, it, 0, true);
    }
    __syncthreads();  // E^2 and N visible; every read of Z_{t-1} and P_{t-1} done
    // Level 2.
    if (egrp) {
      B8 fbh[NW][KC], fbl[NW][KC];
      rows_frag<MP>(sm.e2, TB, fbh, fbl);
      f32x4_t e3[NW][NW];
      quad_mm<MP>(eah, eal, fbh, fbl, e3);
      f32x4_t pt[NW][NW];
#pragma unroll
      for (int u = 0; u < NW; ++u)
#pragma unroll
        for (int v = 0; v < NW; ++v)
#pragma unroll
          for (int i = 0; i < 4; ++i) pt[u][v][i] = dg(u, v, i) + ef[u][v][i] + e2[u][v][i] + 0.25f * e3[u][v][i];
      if constexpr (SAVE) {
        f32x4_t x[NW][NW], t1[NW][NW], t2[NW][NW];
#pragma unroll
        for (int u = 0; u < NW; ++u)
#pragma unroll
          for (int v = 0; v < NW; ++v)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float d1 = dg(u, v, i);
              x[u][v][i] = d1 - ef[u][v][i];
              t1[u][v][i] = 6.f * d1 - 5.f * ef[u][v][i] - e2[u][v][i];
              t2[u][v][i] = 9.f * d1 - 4.f * ef[u][v][i] - 4.f * e2[u][v][i] - e3[u][v][i];
            }
        save(x, it, 1, false);
        save(t1, it, 2, false);
        save(t2, it, 3, false);
      }
      quad_store_t<MP>(sm.p, TA, TB, pt);  // P_{t-1}'s readers finished before the last barrier
    } else {
      if (it > 0) quad_store_t<MP>(sm.z, TA, TB, zt);  // Z_{t-1}'s readers finished before the last barrier
      B8 fah[NW][KC], fal[NW][KC], nbh[NW][KC], nbl[NW][KC];
      rows_frag<MP>(sm.e2, TA, fah, fal);
      rows_frag<MP>(sm.nn, TB, nbh, nbl);
      f32x4_t en[NW][NW];
      quad_mm<MP>(fah, fal, nbh, nbl, en);
      // E's planes are not read in this level (the E group keeps its row
      // fragments from level 1).
      quad_store_t<MP>(sm.e, TA, TB, en);
#pragma unroll
      for (int u = 0; u < NW; ++u)
#pragma unroll
        for (int v = 0; v < NW; ++v)
#pragma unroll
          for (int i = 0; i < 4; ++i) sm.ex[qd][(u * NW + v) * 4 + i][lane] = en[u][v][i];
    }
    __syncthreads();  // E_{t+1}, P_t (and Z_t) visible
    if (egrp) {
#pragma unroll
      for (int u = 0; u < NW; ++u)
#pragma unroll
        for (int v = 0; v < NW; ++v)
#pragma unroll
          for (int i = 0; i < 4; ++i) ef[u][v][i] = sm.ex[qd][(u * NW + v) * 4 + i][lane];
    }
  }
  if (!egrp) {
    if (iters > 0) {  // Z = Z_iters, Z_iters^T = P_{iters-1} Z_{iters-1}^T
      B8 pah[NW][KC], pal[NW][KC], zbh[NW][KC], zbl[NW][KC];
      rows_frag<MP>(sm.p, TA, pah, pal);
      rows_frag<MP>(sm.z, TB, zbh, zbl);
      quad_mm<MP>(pah, pal, zbh, zbl, zt);
    }
    // Z in fp32: tile element i of (u, v) is Z[16 (TB + v) + c][16 (TA + u) + 4g + i].
    // Device-coherent stores: a key block of the same launch reads Z.
    const __amdgpu_buffer_rsrc_t rz = head_rsrc(Zout + (size_t)bh * m * m, m * m * 4);
#pragma unroll
    for (int u = 0; u < NW; ++u)
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        const int row = 16 * (TB + v) + c, col = 16 * (TA + u) + 4 * g;
        if (row >= m) continue;
        if (m == MP) {
          st_coh4(rz, 4 * (row * m + col), make_float4(zt[u][v][0], zt[u][v][1], zt[u][v][2], zt[u][v][3]));
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (col + i < m) st_coh(rz, 4 * (row * m + col + i), zt[u][v][i]);
        }
      }
    quad_store_t<MP>(*reinterpret_cast<uint16_t(*)[2][SM::PL]>(zdst), TA, TB, zt);
  }
}

// ---------------------------------------------------------------------------
// Pseudoinverse for 64 < m <= 256, step 1: A rows.  grid (ceil(m/16), batch*heads).
// Each block computes 16 rows of the scaled scores with the matrix cores,
// then row softmax in LDS.  For the starting scale it also writes its rows'
// sums (rsum[bh][row]) and the column sums over its 16 rows
// (colp[bh][block][col]); summed in block order they give ||A||_inf and
// ||A||_1 without atomics.
template <int PR>
__global__ __launch_bounds__(256) void k_landmark_softmax(const float* __restrict__ Qt,
                                                          const float* __restrict__ Kt,
                                                          float* __restrict__ Aout, float* __restrict__ colp,
                                                          float* __restrict__ rsum, int m, int d,
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
      load8_masked(kt, rk, m, kc + 8 * g, d, d, a);
      load8_masked(qt, rq, m, kc + 8 * g, d, d, b);
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
  const bool live = r0 + r < m;
  float rs = 0.f;
  for (int j = sub; j < m; j += 16) {
    const float a = live ? S[r][j] * inv : 0.f;
    S[r][j] = a;
    rs += a;
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) rs += shfl_xor(rs, o);
  if (live) {
    float* ao = Aout + ((size_t)bh * m + r0 + r) * m;
    for (int j = sub; j < m; j += 16) ao[j] = S[r][j];
    if (sub == 0) rsum[(size_t)bh * m + r0 + r] = rs;
  }
  __syncthreads();
  for (int j = tid; j < m; j += 256) {
    float cs = 0.f;
#pragma unroll 4
    for (int rr = 0; rr < 16; ++rr) cs += S[rr][j];
    colp[((size_t)bh * gridDim.x + blockIdx.x) * m + j] = cs;
  }
}

// Step 2 onwards: Z_0 = cz A^T, cz = 1 / (||A||_1 ||A||_inf) (the
// Pan-Schreiber start), then the Lemma-1 iteration as the pages write it,
// four dependent products per step:
//   X = A Z, T = 7X - X X, U = 15X - X T, Z' = (13Z - Z U) / 4,
// each one launch of batched m x m products on the matrix cores.  (The
// residual form the m <= 64 blocks use, E = I - A Z carried from step to
// step, holds I - A Z only to the absolute precision of E; at m = 256 that
// loses the small singular directions of A Z, so this path recomputes X.)
// One block = one 64 x 64 output tile of one head (8 waves, each 16 rows x
// 32 columns).  The contraction runs in chunks of 128 whose operand panels are
// staged in LDS in fp32 (left rows; right operand by columns), and the
// fragments are split into bf16 parts as they are read (PR = 3: bf16x3;
// PR = 6: three-way split, fp32-grade).
enum MmrMode { kMmProduct = 0, kMmZ0 = 1 };

struct MmrJob {
  int mode;
  const float *X, *Y;  // left and right operands, [bh][m][m] row-major
  float* C;            // output
  const float* F;      // C = alpha (X Y) + beta F (F unused when beta = 0)
  float alpha, beta;
};

struct MmrArgs {
  MmrJob job;
  const float *colp, *rsum;  // kMmZ0: A's column sums per 16-row block and row sums
  int m, nb;
};

constexpr int kMmrK = 128;           // contraction chunk
constexpr int kMmrP = kMmrK + 4;     // LDS panel row pitch (floats)

constexpr int kMmrSmem = 2 * 64 * kMmrP * 4;  // the two operand panels

// One chunk of the operand panels in registers: X rows [i0, i0 + 64) x
// columns [k0, k0 + kMmrK), Y rows [k0, k0 + kMmrK) x columns [j0, j0 + 64),
// 16-byte loads (m a multiple of 4), zero outside the matrices.  All loads of
// a chunk are issued before any is used.
struct MmrChunk {
  float4 x[4], y[4];
};

// Byte offset the buffer range check drops (stores) or reads as zero (loads):
// masked elements use it instead of a branch per access.
constexpr int kMmrOut = 0x7ffffff0;

__device__ __forceinline__ void mmr_load(MmrChunk& r, __amdgpu_buffer_rsrc_t rx, __amdgpu_buffer_rsrc_t ry, int m,
                                         int i0, int j0, int k0) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = tid + 512 * u;
    const int xr = e / (kMmrK / 4), xq = 4 * (e % (kMmrK / 4));  // 64 rows x 32 quads
    const int yk = e / 16, yq = 4 * (e % 16);                     // 128 rows x 16 quads
    const bool xin = i0 + xr < m && k0 + xq < m, yin = k0 + yk < m && j0 + yq < m;
    r.x[u] = __builtin_bit_cast(float4, buf_load16(rx, xin ? 4 * ((i0 + xr) * m + k0 + xq) : kMmrOut));
    r.y[u] = __builtin_bit_cast(float4, buf_load16(ry, yin ? 4 * ((k0 + yk) * m + j0 + yq) : kMmrOut));
  }
}

// The chunk into LDS: X rows [64][kMmrP], Y by columns [64][kMmrP].
__device__ __forceinline__ void mmr_store(const MmrChunk& r, float* __restrict__ sx, float* __restrict__ sy) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int e = tid + 512 * u;
    const int xr = e / (kMmrK / 4), xq = 4 * (e % (kMmrK / 4));
    const int yk = e / 16, yq = 4 * (e % 16);
    *reinterpret_cast<float4*>(&sx[xr * kMmrP + xq]) = r.x[u];
    sy[(yq + 0) * kMmrP + yk] = r.y[u].x;
    sy[(yq + 1) * kMmrP + yk] = r.y[u].y;
    sy[(yq + 2) * kMmrP + yk] = r.y[u].z;
    sy[(yq + 3) * kMmrP + yk] = r.y[u].w;
  }
}

// The same for any m (element loads), used when m is not a multiple of 4.
__device__ __forceinline__ void mmr_stage_scalar(float* __restrict__ sx, float* __restrict__ sy,
                                                 const float* __restrict__ X, const float* __restrict__ Y, int m,
                                                 int i0, int j0, int k0) {
  const int tid = threadIdx.x;
  for (int e = tid; e < 64 * kMmrK; e += 512) {
    const int r = e / kMmrK, q = e % kMmrK;
    sx[r * kMmrP + q] = (i0 + r < m && k0 + q < m) ? X[(size_t)(i0 + r) * m + k0 + q] : 0.f;
    const int k = e / 64, cc = e % 64;
    sy[cc * kMmrP + k] = (k0 + k < m && j0 + cc < m) ? Y[(size_t)(k0 + k) * m + j0 + cc] : 0.f;
  }
}

// Grid: one block per (head, output tile), numbered so that each XCD (block
// L runs on XCD L mod 8) takes a contiguous run of them: a head's tiles share
// their operand panels through that XCD's L2.
template <int PR>
__global__ __launch_bounds__(512) void k_mmr(MmrArgs a) {
  extern __shared__ __align__(16) float smr[];
  const int tiles = (a.m + 63) / 64;
  const int G = gridDim.x, L = blockIdx.x, xcd = L & 7, per = G >> 3, rem = G & 7;
  const int rank = xcd * per + (xcd < rem ? xcd : rem) + (L >> 3);
  const int bh = rank / (tiles * tiles), tt = rank % (tiles * tiles);
  const MmrJob& J = a.job;
  const int m = a.m, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, c = lane & 15, g = lane >> 4;
  const int i0 = (tt / tiles) * 64, j0 = (tt % tiles) * 64;
  const size_t hb = (size_t)bh * m * m;
  if (J.mode == kMmZ0) {
    // cz = 1 / (max column sum x max row sum); column sums in block order.
    __shared__ float red[2][8];
    float cs = 0.f, rs = 0.f;
    if (tid < m) {
      for (int b = 0; b < a.nb; ++b) cs += a.colp[((size_t)bh * a.nb + b) * m + tid];
      rs = a.rsum[(size_t)bh * m + tid];
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      cs = fmaxf(cs, shfl_xor(cs, o));
      rs = fmaxf(rs, shfl_xor(rs, o));
    }
    if (lane == 0) {
      red[0][wave] = cs;
      red[1][wave] = rs;
    }
    __syncthreads();
    cs = red[0][0];
    rs = red[1][0];
#pragma unroll
    for (int w2 = 1; w2 < 8; ++w2) {
      cs = fmaxf(cs, red[0][w2]);
      rs = fmaxf(rs, red[1][w2]);
    }
    const float cz = 1.f / (cs * rs);
    // Z_0 tile (i0.., j0..) = cz A^T: rows j0.. of A through LDS.
    float* tr = smr;  // [64][65]
    for (int e = tid; e < 64 * 64; e += 512) {
      const int r = e / 64, cc = e % 64;
      tr[r * 65 + cc] = (j0 + r < m && i0 + cc < m) ? J.X[hb + (size_t)(j0 + r) * m + i0 + cc] : 0.f;
    }
    __syncthreads();
    for (int e = tid; e < 64 * 64; e += 512) {
      const int r = e / 64, cc = e % 64;
      if (i0 + r < m && j0 + cc < m) J.C[hb + (size_t)(i0 + r) * m + j0 + cc] = cz * tr[cc * 65 + r];
    }
    return;
  }
  float* sx = smr;
  float* sy = smr + 64 * kMmrP;
  const int rw = 16 * (wave & 3), ct0 = 2 * (wave >> 2);  // the wave's rows and first column tile
  f32x4_t acc[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) acc[nt] = zero4();
  auto compute = [&](int kn) {
#pragma unroll
    for (int kc = 0; kc < kMmrK; kc += 32) {
      if (kc >= kn) break;
      float x[8];
      const float* px = &sx[(rw + c) * kMmrP + kc + 8 * g];
#pragma unroll
      for (int q = 0; q < 8; ++q) x[q] = px[q];
      if constexpr (PR == 3) {
        B8 xh, xl;
        split8(x, xh, xl);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          float y[8];
          const float* py = &sy[(16 * (ct0 + nt) + c) * kMmrP + kc + 8 * g];
#pragma unroll
          for (int q = 0; q < 8; ++q) y[q] = py[q];
          B8 yh, yl;
          split8(y, yh, yl);
          acc[nt] = mfma3(xh, xl, yh, yl, acc[nt]);
        }
      } else {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          float y[8];
          const float* py = &sy[(16 * (ct0 + nt) + c) * kMmrP + kc + 8 * g];
#pragma unroll
          for (int q = 0; q < 8; ++q) y[q] = py[q];
          acc[nt] = mma_f32<PR>(x, y, acc[nt]);
        }
      }
    }
  };
  const float* X = J.X + hb;
  const float* Y = J.Y + hb;
  const int mb = m * m * 4;  // bytes of one head's matrix
  // The epilogue's F values of this lane's outputs, loaded up front (F is
  // C's own input only through other launches).
  float fv[2][4];
  const __amdgpu_buffer_rsrc_t rf = head_rsrc(J.F ? J.F + hb : J.C + hb, J.F ? mb : 0);
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = i0 + 16 * (wave & 3) + 4 * g + i, col = j0 + 16 * (2 * (wave >> 2) + nt) + c;
      fv[nt][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rf, (unsigned)(r < m && col < m ? 4 * (r * m + col) : kMmrOut), 0, 0));
    }
  if ((m & 3) == 0) {
    // m <= 256: at most two chunks, both loaded before the first is used.
    MmrChunk ra, rb;
    const bool two = m > kMmrK;
    const __amdgpu_buffer_rsrc_t rx = head_rsrc(X, mb), ry = head_rsrc(Y, mb);
    mmr_load(ra, rx, ry, m, i0, j0, 0);
    if (two) mmr_load(rb, rx, ry, m, i0, j0, kMmrK);
    mmr_store(ra, sx, sy);
    __syncthreads();
    compute(min(kMmrK, m));
    if (two) {
      __syncthreads();  // the first chunk's readers are done
      mmr_store(rb, sx, sy);
      __syncthreads();
      compute(m - kMmrK);
    }
  } else {
    for (int k0 = 0; k0 < m; k0 += kMmrK) {
      if (k0 > 0) __syncthreads();
      mmr_stage_scalar(sx, sy, X, Y, m, i0, j0, k0);
      __syncthreads();
      compute(min(kMmrK, m - k0));
    }
  }
  // Lane (c, g) of wave w holds rows i0 + 16 (w % 4) + 4g + i, columns
  // j0 + 16 (2 (w / 4) + nt) + c.  Unconditional stores: elements outside the
  // matrix go to the dropped offset.
  const __amdgpu_buffer_rsrc_t rc = head_rsrc(J.C + hb, mb);
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = i0 + rw + 4 * g + i, col = j0 + 16 * (ct0 + nt) + c;
      const float v = J.alpha * acc[nt][i] + J.beta * fv[nt][i];
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rc, (unsigned)(r < m && col < m ? 4 * (r * m + col)
                                                                                              : kMmrOut), 0, 0);
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
  // V^T row pitch: 70 elements (35 dwords) keeps both the packed 2-key
  // staging writes and the P V operand reads (lanes c, g at column 4g of row
  // c) at most 3 deep in any bank.
  static constexpr int VP = 64 + 6;
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

// One (key chunk, head) of the split-n pass, run by a block of 256 threads.
// PAIR: the block's two groups run chunks 2j and 2j + 1 of one head; group 1
// hands its partial to group 0 through `xch` (the block's LDS, free once both
// groups are past their last tile), which merges the two and writes one partial, entry
// j of nchunks / 2 per head, with device-coherent stores (the head's last key
// block of the same launch reads them).  Otherwise each group writes its own
// chunk's partial, entry ch of nchunks, with plain stores.
// NWC: waves per chunk (4: two chunks per 512-thread block; 8: one).
// SIN: K and V rows where il says; otherwise the [batch][heads][n][d] layout.
template <typename IO, int D, int NTW, bool PAIR, int NWC = 4, bool SIN = false>
__device__ __forceinline__ void bv_chunk(BvSmem<IO, D>& sm, float* xch, int ch, int bh,
                                         const typename IO::T* __restrict__ Kin,
                                         const typename IO::T* __restrict__ Vin, const float* __restrict__ Qt,
                                         float* __restrict__ pacc, float* __restrict__ pmax,
                                         float* __restrict__ psum, int n, int nb, int m, int chunk, int nchunks,
                                         float sl2e, const InLayout& il, int heads) {
  using T = typename IO::T;
  using SM = BvSmem<IO, D>;
  constexpr int KC = (D + 31) / 32;  // 32-wide k chunks over the head dimension
  constexpr int MD = D / 16;         // 16-row tiles of V^T
  static_assert(!PAIR || NWC == 4, "pairs are the two 4-wave groups of a block");
  constexpr int NTH = 64 * NWC;           // threads per chunk
  const int tid = threadIdx.x & (NTH - 1);  // the chunk's group of waves
  const int lane = tid & 63, wave = tid >> 6, c = lane & 15, g = lane >> 4;
  // Keys [kbeg, kend) of this chunk; nb <= n is the head's number of real
  // keys (chunks past it are empty and leave max -inf, sum 0).
  const int kbeg = ch * chunk, kend = min(nb, kbeg + chunk);
  const long long hoff = SIN ? (bh / heads) * il.bs + (bh % heads) * il.hs : (long long)bh * n * D;
  const int ild = SIN ? il.ld : D;
  const T* Kh = Kin + hoff;
  const T* Vh = Vin + hoff;
  const float* qt = Qt + (size_t)bh * m * D;

  // Landmark-query operands (B of S^T = K Qt^T), pre-multiplied by
  // log2(e)/sqrt(d) so that scores come out in base-2 units, in registers:
  // rounded to bf16 for bf16 I/O (single bf16 products, fp32 accumulation),
  // split hi/lo for fp32 I/O.
  B8 qh[NTW][KC], ql[NTW][KC];
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int lm = (wave * NTW + t) * 16 + c;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      float x[8];
      load8_masked(qt, lm, m, kc * 32 + 8 * g, D, D, x);  // branch-free: all loads in flight together
#pragma unroll
      for (int q = 0; q < 8; ++q) x[q] *= sl2e;
      if constexpr (IO::kBf16) round8(x, qh[t][kc]); else split8(x, qh[t][kc], ql[t][kc]);
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

  // Staging is software-pipelined: the K and V rows of the next tile are
  // loaded into registers while the current tile is computed from LDS.  (Two
  // or three tiles in flight per 4-wave group measured slower: 25.0 and 25.8
  // against 24.5 us for the pass at 2 x 12 heads, n = 8192, d = 64, m = 64.)
  constexpr int SLOTS = D / 8;
  constexpr int TASKS = 32 * SLOTS;               // (key pair, 8-feature slot)
  constexpr int TPT = (TASKS + NTH - 1) / NTH;     // tasks per thread
  BvStage<IO> stage[TPT];
  auto load_tile = [&](BvStage<IO> (&st)[TPT], int k0) {
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int e = tid + NTH * u;
      const int rp = e / SLOTS, s8 = (e % SLOTS) * 8;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int key = k0 + 2 * rp + h;
        const bool in = e < TASKS && key < kend;
#pragma unroll
        for (int w = 0; w < BvStage<IO>::W; ++w) {
          st[u].k[h][w] = in ? reinterpret_cast<const uint4*>(Kh + (size_t)key * ild + s8)[w] : make_uint4(0, 0, 0, 0);
          st[u].v[h][w] = in ? reinterpret_cast<const uint4*>(Vh + (size_t)key * ild + s8)[w] : make_uint4(0, 0, 0, 0);
        }
      }
    }
  };
  auto store_tile = [&](const BvStage<IO> (&st)[TPT]) {
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int e = tid + NTH * u;
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
      // V^T: feature s8+q, keys 2rp and 2rp+1 packed in one dword (byte
      // selects 0x05040100 = low halves, 0x07060302 = high halves).
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        *reinterpret_cast<uint32_t*>(&sm.vt[0][(s8 + 2 * j) * SM::VP + 2 * rp]) =
            __builtin_amdgcn_perm(vh[1].u[j], vh[0].u[j], 0x05040100u);
        *reinterpret_cast<uint32_t*>(&sm.vt[0][(s8 + 2 * j + 1) * SM::VP + 2 * rp]) =
            __builtin_amdgcn_perm(vh[1].u[j], vh[0].u[j], 0x07060302u);
        if constexpr (SM::PL == 2) {
          *reinterpret_cast<uint32_t*>(&sm.vt[1][(s8 + 2 * j) * SM::VP + 2 * rp]) =
              __builtin_amdgcn_perm(vl[1].u[j], vl[0].u[j], 0x05040100u);
          *reinterpret_cast<uint32_t*>(&sm.vt[1][(s8 + 2 * j + 1) * SM::VP + 2 * rp]) =
              __builtin_amdgcn_perm(vl[1].u[j], vl[0].u[j], 0x07060302u);
        }
      }
    }
  };

  auto compute_tile = [&](int k0) {
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
            s[mt] = mfma(kh, qh[t][kc], s[mt]);
          }
        }
      }
      // Online softmax over this tile's keys for landmark (wave*NTW+t)*16 + c;
      // scores are in base-2 units; keys past the chunk end only in its
      // last tile.
      if (k0 + 64 > kend) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (k0 + mt * 16 + 4 * g + i >= kend) s[mt][i] = -INFINITY;
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, s[mt][i]);
      tmax = max_over_groups(tmax);
      const float nmax = fmaxf(run_max[t], tmax);
      const float corr = __builtin_amdgcn_exp2f(run_max[t] - nmax);  // arguments <= 0; exp2(-inf) = 0
      float psum_l = 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s[mt][i] = __builtin_amdgcn_exp2f(s[mt][i] - nmax);
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
        if constexpr (SM::PL == 2) split8(p, ph, pl); else round8(p, ph);
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
            acc[t][md] = mfma(vh, ph, acc[t][md]);
          }
        }
      }
    }
  };

  // Both groups of the block run the same number of steps (their barriers
  // are the block's); a group past its chunk's end only waits.
  const int ntile = (chunk + 63) / 64;
  if (kbeg < kend) load_tile(stage, kbeg);
  for (int t = 0; t < ntile; ++t) {
    const int kt = kbeg + 64 * t;
    const bool live = kt < kend;  // uniform over the group
    if (live) store_tile(stage);
    __syncthreads();
    if (kt + 64 < kend) load_tile(stage, kt + 64);
    if (live) compute_tile(kt);
    __syncthreads();
  }

  if constexpr (PAIR) {
    // Group 1's partial -> group 0, which merges it into its own:
    // M = max(M0, M1), sum = sum0 2^(M0 - M) + sum1 2^(M1 - M), likewise the
    // accumulators (an empty chunk has M = -inf and contributes nothing).
    constexpr int NV = NTW * (MD * 4 + 2);  // floats per lane
    const int grp = threadIdx.x >> 8;
    float* xw = xch + wave * NV * 64 + lane;
    if (grp == 1) {
#pragma unroll
      for (int t = 0; t < NTW; ++t) {
        float* x = xw + t * (MD * 4 + 2) * 64;
        x[0] = run_max[t];
        x[64] = run_sum[t];
#pragma unroll
        for (int md = 0; md < MD; ++md)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[(2 + 4 * md + i) * 64] = acc[t][md][i];
      }
    }
    __syncthreads();
    if (grp == 1) return;  // no barrier follows in this function
#pragma unroll
    for (int t = 0; t < NTW; ++t) {
      const float* x = xw + t * (MD * 4 + 2) * 64;
      const float m1 = x[0], s1 = x[64];
      const float M = fmaxf(run_max[t], m1);
      const float e0 = run_max[t] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(run_max[t] - M);
      const float e1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
      run_sum[t] = run_sum[t] * e0 + s1 * e1;
      run_max[t] = M;
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t][md][i] = acc[t][md][i] * e0 + x[(2 + 4 * md + i) * 64] * e1;
    }
  }

  // Partials for landmarks < m.
  constexpr bool COH = PAIR;
  const int np = PAIR ? nchunks / 2 : nchunks;  // partial entries per head
  const size_t hb = (size_t)bh * np * m;        // the head's first (entry, landmark)
  const __amdgpu_buffer_rsrc_t ra = head_rsrc(pacc + hb * D, np * m * D * 4);
  const __amdgpu_buffer_rsrc_t rm = head_rsrc(pmax + hb, np * m * 4);
  const __amdgpu_buffer_rsrc_t rs = head_rsrc(psum + hb, np * m * 4);
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const int lm = (wave * NTW + t) * 16 + c;
    if (lm >= m) continue;
    const int e = (PAIR ? ch >> 1 : ch) * m + lm;
    if (g == 0) {
      if constexpr (COH) {
        st_coh(rm, 4 * e, run_max[t]);
        st_coh(rs, 4 * e, run_sum[t]);
      } else {
        pmax[hb + e] = run_max[t];
        psum[hb + e] = run_sum[t];
      }
    }
#pragma unroll
    for (int md = 0; md < MD; ++md) {
      float4 v = make_float4(acc[t][md][0], acc[t][md][1], acc[t][md][2], acc[t][md][3]);
      if constexpr (COH)
        st_coh4(ra, 4 * (e * D + md * 16 + 4 * g), v);
      else
        *reinterpret_cast<float4*>(&pacc[(hb + e) * D + md * 16 + 4 * g]) = v;
    }
  }
}

// Finish of the split-n pass for one head, inside the landmark pass (blocks
// of 512 threads):
//   BV[j][f] = sum_c pacc_c[j][f] 2^(pmax_c[j] - M_j) / sum_c psum_c[j] 2^(pmax_c[j] - M_j)
//   (M_j = max_c pmax_c[j]; entries folded in order, in batches with a running
//   maximum), computed by the head's last key block to arrive; and
//   W = Z BV on the matrix cores (bf16x3) with the W^T bf16 plane [bh][D][MP]
//   the output stage reads (within each chunk of 32 landmarks, position
//   8g + q holds landmark 4g + q (q < 4) or 16 + 4g + q - 4 (q >= 4), the
//   order in which that stage's softmax lanes hold their landmarks; padding
//   is zero), computed by whichever of that block and the head's
//   pseudoinverse block arrives second: it holds one operand in LDS and reads
//   the other, which the first left in global memory with device-coherent
//   stores.  No block waits for another.
template <int MP, int D>
struct FinishSmem {
  static constexpr int LD = MP + 8;      // plane row pitch (bf16): 16-byte aligned rows
  __align__(16) uint16_t z[2][MP * LD];  // Z rows, hi / lo (zero past m)
  __align__(16) uint16_t bt[2][D * LD];  // BV^T rows (feature-major), hi / lo (zero past m)
};

// BV of head bh from np partial entries -> BV (device-coherent stores) and
// the BV^T planes.
template <int MP, int D>
__device__ __forceinline__ void combine_bv(FinishSmem<MP, D>& sm, int bh, const float* __restrict__ pacc,
                                           const float* __restrict__ pmax, const float* __restrict__ psum,
                                           float* __restrict__ BV, int m, int np) {
  constexpr int LD = FinishSmem<MP, D>::LD, NQ = D / 4, ITEMS = MP * NQ;
  constexpr int IPT = (ITEMS + 511) / 512;                    // (landmark, feature quad) items per thread
  constexpr int NB = IPT >= 4 ? 4 : (IPT == 2 ? 10 : 16);     // entries per batch of loads
  const int tid = threadIdx.x;
  const size_t hb = (size_t)bh * np * m;
  const __amdgpu_buffer_rsrc_t ra = head_rsrc(pacc + hb * D, np * m * D * 4);
  const __amdgpu_buffer_rsrc_t rm = head_rsrc(pmax + hb, np * m * 4);
  const __amdgpu_buffer_rsrc_t rs = head_rsrc(psum + hb, np * m * 4);
  float M[IPT], L[IPT];
  float4 S[IPT];
  int jj[IPT], qq[IPT];
#pragma unroll
  for (int r = 0; r < IPT; ++r) {
    const int it = min(tid + 512 * r, ITEMS - 1);
    jj[r] = it / NQ;
    qq[r] = it % NQ;
    M[r] = -INFINITY;
    L[r] = 0.f;
    S[r] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int c0 = 0; c0 < np; c0 += NB) {
    float pm[IPT][NB], ps[IPT][NB];
    float4 pa[IPT][NB];
#pragma unroll
    for (int r = 0; r < IPT; ++r)
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int e = min(c0 + u, np - 1) * m + min(jj[r], m - 1);
        pm[r][u] = ld_coh(rm, 4 * e);
        ps[r][u] = ld_coh(rs, 4 * e);
        pa[r][u] = ld_coh4(ra, 4 * (e * D + 4 * qq[r]));
      }
#pragma unroll
    for (int r = 0; r < IPT; ++r) {
      float Mb = M[r];
#pragma unroll
      for (int u = 0; u < NB; ++u)
        if (c0 + u < np) Mb = fmaxf(Mb, pm[r][u]);
      // Arguments <= 0.  Entries past a sequence's end are empty (max -inf):
      // a batch of only those keeps M = Mb = -inf and must not form -inf - -inf.
      const float sc = M[r] == Mb ? 1.f : __builtin_amdgcn_exp2f(M[r] - Mb);
      L[r] *= sc;
      S[r].x *= sc;
      S[r].y *= sc;
      S[r].z *= sc;
      S[r].w *= sc;
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        if (c0 + u < np) {
          const float e = pm[r][u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(pm[r][u] - Mb);
          L[r] += ps[r][u] * e;
          S[r].x += pa[r][u].x * e;
          S[r].y += pa[r][u].y * e;
          S[r].z += pa[r][u].z * e;
          S[r].w += pa[r][u].w * e;
        }
      }
      M[r] = Mb;
    }
  }
  const __amdgpu_buffer_rsrc_t rb = head_rsrc(BV + (size_t)bh * m * D, m * D * 4);
#pragma unroll
  for (int r = 0; r < IPT; ++r) {
    if (tid + 512 * r >= ITEMS) continue;
    const int j = jj[r], q = qq[r];
    // A sequence with no keys (length 0) has every entry empty: BV = 0.
    const bool ok = j < m && M[r] != -INFINITY;
    const float inv = ok ? 1.f / L[r] : 0.f;
    const float v[4] = {ok ? S[r].x * inv : 0.f, ok ? S[r].y * inv : 0.f, ok ? S[r].z * inv : 0.f,
                        ok ? S[r].w * inv : 0.f};
    if (j < m) st_coh4(rb, 4 * (j * D + 4 * q), make_float4(v[0], v[1], v[2], v[3]));
#pragma unroll
    for (int i = 0; i < 4; ++i) split_hi_lo(v[i], sm.bt[0][(4 * q + i) * LD + j], sm.bt[1][(4 * q + i) * LD + j]);
  }
}

// Z of head bh (device-coherent loads) -> the Z planes.
template <int MP, int D>
__device__ __forceinline__ void load_z_planes(FinishSmem<MP, D>& sm, int bh, const float* __restrict__ Z, int m) {
  constexpr int LD = FinishSmem<MP, D>::LD;
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t rz = head_rsrc(Z + (size_t)bh * m * m, m * m * 4);
#pragma unroll
  for (int k = 0; k < (MP * MP / 4 + 511) / 512; ++k) {
    const int e4 = tid + 512 * k;
    if (e4 >= MP * MP / 4) break;
    const int r = e4 / (MP / 4), c4 = 4 * (e4 % (MP / 4));
    float v[4];
    if (m == MP) {
      const float4 x = ld_coh4(rz, 4 * (r * m + c4));
      v[0] = x.x;
      v[1] = x.y;
      v[2] = x.z;
      v[3] = x.w;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = ld_coh(rz, 4 * (min(r, m - 1) * m + min(c4 + i, m - 1)));
        v[i] = (r < m && c4 + i < m) ? x : 0.f;
      }
    }
    uint2 hv, lv;
    split_pair(v[0], v[1], hv.x, lv.x);
    split_pair(v[2], v[3], hv.y, lv.y);
    *reinterpret_cast<uint2*>(&sm.z[0][r * LD + c4]) = hv;
    *reinterpret_cast<uint2*>(&sm.z[1][r * LD + c4]) = lv;
  }
}

// BV of head bh (device-coherent loads) -> the BV^T planes.
template <int MP, int D>
__device__ __forceinline__ void load_bv_planes(FinishSmem<MP, D>& sm, int bh, const float* __restrict__ BV, int m) {
  constexpr int LD = FinishSmem<MP, D>::LD, NQ = D / 4;
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t rb = head_rsrc(BV + (size_t)bh * m * D, m * D * 4);
#pragma unroll
  for (int k = 0; k < (MP * NQ + 511) / 512; ++k) {
    const int it = tid + 512 * k;
    if (it >= MP * NQ) break;
    const int j = it / NQ, q = it % NQ;
    const float4 x = ld_coh4(rb, 4 * (min(j, m - 1) * D + 4 * q));
    const float v[4] = {j < m ? x.x : 0.f, j < m ? x.y : 0.f, j < m ? x.z : 0.f, j < m ? x.w : 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) split_hi_lo(v[i], sm.bt[0][(4 * q + i) * LD + j], sm.bt[1][(4 * q + i) * LD + j]);
  }
}

// W = Z BV from the planes -> W (fp32) and the W^T bf16 plane.  8 waves; tile
// (row tile ti of landmarks, feature tile nd): lane (c, g) ends with
// W[16 ti + 4g + i][16 nd + c].
template <int MP, int D>
__device__ __forceinline__ void form_w(const FinishSmem<MP, D>& sm, int bh, float* __restrict__ W,
                                       uint16_t* __restrict__ wt_hi, int m) {
  constexpr int LD = FinishSmem<MP, D>::LD, NTR = MP / 16, NTF = D / 16, KC = MP / 32;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, c = lane & 15, g = lane >> 4;
#pragma unroll
  for (int t = wave; t < NTR * NTF; t += 8) {
    const int ti = t % NTR, nd = t / NTR;
    f32x4_t acc = zero4();
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      B8 ah, al, bh8, bl8;
      const int oa = (16 * ti + c) * LD + 32 * kc + 8 * g, ob = (16 * nd + c) * LD + 32 * kc + 8 * g;
      ah.q = *reinterpret_cast<const uint4*>(&sm.z[0][oa]);
      al.q = *reinterpret_cast<const uint4*>(&sm.z[1][oa]);
      bh8.q = *reinterpret_cast<const uint4*>(&sm.bt[0][ob]);
      bl8.q = *reinterpret_cast<const uint4*>(&sm.bt[1][ob]);
      acc = mfma3(ah, al, bh8, bl8, acc);
    }
    const int f = 16 * nd + c;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * ti + 4 * g + i;
      if (r < m) W[((size_t)bh * m + r) * D + f] = acc[i];
    }
    // Landmarks 16 ti + 4g .. +3 sit at positions 32 (ti / 2) + 8g + 4 (ti % 2) .. +3.
    const size_t o = ((size_t)bh * D + f) * MP + 32 * (ti >> 1) + 8 * g + 4 * (ti & 1);
    *reinterpret_cast<uint2*>(&wt_hi[o]) = make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
  }
}

// Skip-filter operands for the matrix-core conv of the output stage.
// Entry ((h * d + f) * 4 + i) * 9 + s holds taps 4s + k - i - off (k = 0..3)
// of filter (h, f) as bf16 hi (k = 0..3) then bf16 lo, where off =
// (33 - conv_k) / 2 centres a filter of conv_k <= 33 taps in 33 slots.
__device__ __forceinline__ void conv_operand(const float* __restrict__ conv_w, uint4* __restrict__ ops, int idx,
                                             int conv_k) {
  constexpr int NS = 9;
  const int st = idx % NS, i = (idx / NS) % 4, hf = idx / (4 * NS);
  const int off = (33 - conv_k) / 2;
  B8 hl;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int tt = 4 * st + k - i - off;
    const float wl = conv_w[(size_t)hf * conv_k + min(max(tt, 0), conv_k - 1)];  // clamped: no branch per load
    const float w = (tt >= 0 && tt < conv_k) ? wl : 0.f;
    split_hi_lo(w, hl.h[k], hl.h[4 + k]);
  }
  ops[idx] = hl.q;
}

// The landmark-side pass in one launch.  Blocks [0, npinv): the
// pseudoinverse of head blockIdx.x (it depends only on the landmarks);
// then nconv blocks of skip-filter operands; then the split-n pass, block
// (bh * nchunks + chunk).  The pseudoinverse blocks come first so that they
// are placed while the key-pass blocks fill the rest of the machine.
struct LandmarkPassArgs {
  const void* K;
  const void* V;
  float* zsave;  // the pseudoinverse steps for the backward pass, or nullptr
  int zmp;
  const float *Qt, *Kt;
  const uint16_t *qt_hi, *qt_lo, *kt_hi, *kt_lo;  // landmark planes (pseudoinverse blocks)
  float *A, *Z, *pacc, *pmax, *psum;
  const float* conv_w;
  uint4* cwop;
  const int* lens;  // tokens per sequence, or nullptr
  // With the pseudoinverse in the launch: per-head arrival counters ([0, bhn):
  // key blocks; [bhn, 2 bhn): Z and BV complete), zero at the start, and the
  // finish's outputs.
  unsigned* sync;
  float *BV, *W;
  uint16_t* wt_hi;
  int bhn;
  int n, heads, m, chunk, nchunks, iters, npinv, nconv, conv_total, conv_k;
  float sl2e;
  InLayout il;  // where K's and V's rows are
};

template <int PMP, int D, typename B>
union LandmarkPassSmem {
  PinvSmemE<PMP> p;
  FinishSmem<PMP, D> f;
  B b[2];
};
template <int D, typename B>
union LandmarkPassSmem<0, D, B> {
  B b[2];
};

// PMP: landmarks padded to 32 or 64 for the pseudoinverse blocks, 0 for none.
// CPB: key chunks per block (2: one per group of 4 waves; 1: one chunk on all
// 8 waves, for m > 128, where 4 waves would hold too many accumulators).
template <typename IO, int D, int NTW, int PMP, bool SAVE, int CPB = 2, bool SIN = false>
__global__ __launch_bounds__(512) void k_landmark_pass(LandmarkPassArgs a) {
  using T = typename IO::T;
  constexpr bool FOLD = PMP > 0;  // the split-n finish runs in this launch
  __shared__ LandmarkPassSmem<PMP, D, BvSmem<IO, D>> sm;
  __shared__ unsigned last;
  int blk = blockIdx.x;
  if constexpr (FOLD) {
    if (blk < a.npinv) {
      static_assert(sizeof(sm.f.z) == sizeof(sm.p.e), "the Z planes of the finish alias the E planes");
      pinv_head<PMP, D, SAVE>(sm.p, blk, a.qt_hi, a.qt_lo, a.kt_hi, a.kt_lo, a.A, a.Z, a.m, a.iters, a.zsave,
                              a.zmp, sm.f.z);
      // Z complete (every lane's stores done): arrive; the second to arrive
      // (this block or the head's last key block, with BV) forms W.
      wait_stores();
      __syncthreads();
      if (threadIdx.x == 0)
        last = __hip_atomic_fetch_add(&a.sync[a.bhn + blk], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 1u;
      __syncthreads();
      if (last) {
        load_bv_planes<PMP, D>(sm.f, blk, a.BV, a.m);
        __syncthreads();
        form_w<PMP, D>(sm.f, blk, a.W, a.wt_hi, a.m);
      }
      return;
    }
    blk -= a.npinv;
  }
  if (blk < a.nconv) {
    const int idx = blk * 512 + (int)threadIdx.x;
    if (idx < a.conv_total) conv_operand(a.conv_w, a.cwop, idx, a.conv_k);
    return;
  }
  blk -= a.nconv;
  if constexpr (CPB == 1) {
    const int bh = blk / a.nchunks;
    bv_chunk<IO, D, NTW, false, 8, SIN>(sm.b[0], nullptr, blk % a.nchunks, bh, static_cast<const T*>(a.K),
                                   static_cast<const T*>(a.V), a.Qt, a.pacc, a.pmax, a.psum, a.n,
                                   seq_rows(a.lens, bh / a.heads, a.n), a.m, a.chunk, a.nchunks, a.sl2e, a.il, a.heads);
    return;
  }
  // Key blocks: chunks 2 j and 2 j + 1 of a head, one per group of 4 waves.
  const int half = a.nchunks / 2, bh = blk / half, grp = threadIdx.x >> 8;
  bv_chunk<IO, D, NTW, FOLD, 4, SIN>(sm.b[grp], reinterpret_cast<float*>(&sm), 2 * (blk % half) + grp, bh,
                             static_cast<const T*>(a.K), static_cast<const T*>(a.V), a.Qt, a.pacc, a.pmax,
                             a.psum, a.n, seq_rows(a.lens, bh / a.heads, a.n), a.m, a.chunk, a.nchunks, a.sl2e, a.il, a.heads);
  if constexpr (FOLD) {
    static_assert(sizeof(float) * 4 * (D / 16 * 4 + 2) * 64 <= sizeof(sm), "the pair exchange fits the LDS");
    // The head's last key block to arrive combines its partials into BV,
    // then arrives at the head's second counter; the second to arrive (this
    // block or the pseudoinverse block, with Z) forms W.
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0)
      last = __hip_atomic_fetch_add(&a.sync[bh], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             (unsigned)(half - 1);
    __syncthreads();
    if (!last) return;
    combine_bv<PMP, D>(sm.f, bh, a.pacc, a.pmax, a.psum, a.BV, a.m, half);
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0)
      last = __hip_atomic_fetch_add(&a.sync[a.bhn + bh], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 1u;
    __syncthreads();
    if (!last) return;
    load_z_planes<PMP, D>(sm.f, bh, a.Z, a.m);
    __syncthreads();
    form_w<PMP, D>(sm.f, bh, a.W, a.wt_hi, a.m);
  }
}

// The split-n pass for 128 < m <= 256 in blocks of 16 waves, one key chunk
// each, one 16-landmark tile per wave (the 8-wave form holds two tiles per
// wave, whose accumulators leave room for two waves per SIMD; here four fit).
// Blocks [0, nconv) write the skip-filter operands (1024 entries each).
template <typename IO, int D>
__global__ __launch_bounds__(1024) void k_key_pass16(LandmarkPassArgs a) {
  using T = typename IO::T;
  __shared__ BvSmem<IO, D> sm;
  int blk = blockIdx.x;
  if (blk < a.nconv) {
    const int idx = blk * 1024 + (int)threadIdx.x;
    if (idx < a.conv_total) conv_operand(a.conv_w, a.cwop, idx, a.conv_k);
    return;
  }
  blk -= a.nconv;
  const int bh = blk / a.nchunks;
  bv_chunk<IO, D, 1, false, 16>(sm, nullptr, blk % a.nchunks, bh, static_cast<const T*>(a.K),
                                static_cast<const T*>(a.V), a.Qt, a.pacc, a.pmax, a.psum, a.n,
                                seq_rows(a.lens, bh / a.heads, a.n), a.m, a.chunk, a.nchunks, a.sl2e, a.il, a.heads);
}

// fp32 I/O, m <= 64, d <= 64: the pseudoinverse (blocks [0, npinv), one
// head each, as k_pinv_lds) and the split-n key pass (two chunks per block,
// 8 waves each; partial entry per chunk, combined by k_bv_finish) in one
// launch, since the pseudoinverse needs only the landmarks.
template <int PMP, int D, bool SIN = false>
__global__ __launch_bounds__(64 * kPinvWaves) void k_landmark_pass_f32(LandmarkPassArgs a, float sl2e_d) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  static_assert(64 * kPinvWaves == 1024, "two 8-wave chunk groups per block");
  int blk = blockIdx.x;
  if (blk < a.npinv) {
    pinv_lds_head<PMP, 6>(smem_raw, blk, a.Qt, a.Kt, a.A, a.Z, a.m, D, sl2e_d, a.iters, a.zsave, a.zmp);
    return;
  }
  blk -= a.npinv;
  const int half = a.nchunks / 2, bh = blk / half, grp = threadIdx.x >> 9;
  BvSmem<F32, D>& sm = reinterpret_cast<BvSmem<F32, D>*>(smem_raw)[grp];
  bv_chunk<F32, D, 1, false, 8, SIN>(sm, nullptr, 2 * (blk % half) + grp, bh, static_cast<const float*>(a.K),
                                static_cast<const float*>(a.V), a.Qt, a.pacc, a.pmax, a.psum, a.n,
                                seq_rows(a.lens, bh / a.heads, a.n), a.m, a.chunk, a.nchunks, a.sl2e, a.il, a.heads);
}

// Finish of the split-n pass, one block per (16-feature slice, head):
//   BV[j][f] = sum_c pacc_c[j][f] 2^(pmax_c[j] - M_j) / sum_c psum_c[j] 2^(pmax_c[j] - M_j)
//   (M_j = max_c pmax_c[j]; chunks in fixed order), then W = Z BV for the
//   slice, then the slice's rows of the W^T bf16 planes [bh][D][mpa], the A
//   operand of the output stage: within each chunk of 32 landmarks, position
//   8g + q holds landmark 4g + q (q < 4) or 16 + 4g + q - 4 (q >= 4), the
//   order in which that stage's softmax lanes hold their landmarks; padding
//   is zero.  grid (D/16, batch*heads).
// ZLDS (m <= 64): Z staged in LDS and W on the matrix cores, PR = 3 (bf16x3,
// bf16 I/O: hi plane only) or 6 (three-way split, fp32 I/O: hi and lo
// planes); otherwise fp32 FMAs from global Z.
template <bool ZLDS, int PR>
__global__ __launch_bounds__(1024) void k_bv_finish(const float* __restrict__ pacc, const float* __restrict__ pmax,
                                                    const float* __restrict__ psum, const float* __restrict__ Z,
                                                    float* __restrict__ BV, float* __restrict__ W,
                                                    uint16_t* __restrict__ wt_hi, uint16_t* __restrict__ wt_lo, int m,
                                                    int D, int nchunks, int mpa) {
  __shared__ float sbv[256][17];
  __shared__ float sw[256][17];
  __shared__ __align__(16) float sz[ZLDS ? 64 * 68 : 4];
  const int bh = blockIdx.y, f0 = blockIdx.x * 16, tid = threadIdx.x;
  const float* z = Z + (size_t)bh * m * m;
  // Z (m <= 64: at most 4 values per thread) is loaded first, beside the
  // partials, and stored to LDS after the combine.
  float zv[4];
  if constexpr (ZLDS) {
#pragma unroll
    for (int u = 0; u < 4; ++u) zv[u] = z[min(tid + 1024 * u, m * m - 1)];
  }
  const size_t pb = (size_t)bh * nchunks * m;
  // Combine over the chunks.  Thread (part, j, q): chunk subset `part` (of 4,
  // interleaved), landmark j, features f0 + 4q .. +3 (16-byte loads); each
  // part folds its chunks in order (running max per batch of NB), then part
  // 0 folds the 4 parts in order, so the result does not depend on timing.
  __shared__ float red[4][64][2];        // per part and landmark: max, sum
  __shared__ float reds[4][64][4][4];    // per part, landmark, feature quad: accumulator
  {
    const int part = tid >> 8, r = tid & 255, jl = r >> 2, q = r & 3;
    for (int j0 = 0; j0 < m; j0 += 64) {
      const int j = j0 + jl;
      const int jc = min(j, m - 1);
      constexpr int NB = 8;
      float M = -INFINITY, L = 0.f, S[4] = {0.f, 0.f, 0.f, 0.f};
      for (int c0 = part; c0 < nchunks; c0 += 4 * NB) {
        float pm[NB], ps[NB];
        float4 pa[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          const int cc = min(c0 + 4 * u, nchunks - 1);
          const size_t o = pb + (size_t)cc * m + jc;
          pm[u] = pmax[o];
          ps[u] = psum[o];
          pa[u] = *reinterpret_cast<const float4*>(&pacc[o * D + f0 + 4 * q]);
        }
        float Mb = M;
#pragma unroll
        for (int u = 0; u < NB; ++u)
          if (c0 + 4 * u < nchunks) Mb = fmaxf(Mb, pm[u]);
        // Arguments <= 0; 0 while M = -inf.  Chunks past a sequence's end are
        // empty (max -inf): a batch of only those keeps M = Mb = -inf and must
        // not form -inf - -inf.
        const float a = M == Mb ? 1.f : __builtin_amdgcn_exp2f(M - Mb);
        L *= a;
#pragma unroll
        for (int k = 0; k < 4; ++k) S[k] *= a;
#pragma unroll
        for (int u = 0; u < NB; ++u) {
          if (c0 + 4 * u < nchunks) {
            const float e = pm[u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(pm[u] - Mb);
            L += ps[u] * e;
            S[0] += pa[u].x * e;
            S[1] += pa[u].y * e;
            S[2] += pa[u].z * e;
            S[3] += pa[u].w * e;
          }
        }
        M = Mb;
      }
      // Parts with no chunk (nchunks < 4) keep M = -inf, L = S = 0.
      if (q == 0) {
        red[part][jl][0] = M;
        red[part][jl][1] = L;
      }
      *reinterpret_cast<float4*>(&reds[part][jl][q][0]) = make_float4(S[0], S[1], S[2], S[3]);
      __syncthreads();
      if (part == 0 && j < m) {
        float Mt = -INFINITY;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) Mt = fmaxf(Mt, red[pp][jl][0]);
        float Lt = 0.f, St[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const float e = __builtin_amdgcn_exp2f(red[pp][jl][0] - Mt);  // exp2(-inf) = 0 for empty parts
          Lt += red[pp][jl][1] * e;
#pragma unroll
          for (int k = 0; k < 4; ++k) St[k] += reds[pp][jl][q][k] * e;
        }
        // A sequence with no keys (length 0) has every chunk empty: BV = 0.
        const float inv = Mt == -INFINITY ? 0.f : 1.f / Lt;
        if (Mt == -INFINITY) {
#pragma unroll
          for (int k = 0; k < 4; ++k) St[k] = 0.f;
        }
        float4 v = make_float4(St[0] * inv, St[1] * inv, St[2] * inv, St[3] * inv);
        sbv[j][4 * q] = v.x;
        sbv[j][4 * q + 1] = v.y;
        sbv[j][4 * q + 2] = v.z;
        sbv[j][4 * q + 3] = v.w;
        *reinterpret_cast<float4*>(&BV[((size_t)bh * m + j) * D + f0 + 4 * q]) = v;
      }
      __syncthreads();
    }
  }
  if constexpr (ZLDS) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + 1024 * u;
      if (e < m * m) sz[(e / m) * 68 + e % m] = zv[u];
    }
    __syncthreads();
    // W slice (64 x 16, rows >= m zero) = Z (64 x 64) BV slice (64 x 16): wave
    // ti < 4 computes row tile ti; lane (c, g) ends with W[16ti + 4g + i][f0 + c].
    const int lane = tid & 63, ti = tid >> 6, c = lane & 15, g = lane >> 4;
    if (ti < 4 && 16 * ti < mpa) {
      f32x4_t acc = zero4();
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        float a[8], b[8];
        const int r = 16 * ti + c;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int k = 32 * kc + 8 * g + q;
          a[q] = (r < m && k < m) ? sz[r * 68 + k] : 0.f;
          b[q] = k < m ? sbv[k][c] : 0.f;
        }
        acc = mma_f32<PR>(a, b, acc);
      }
      const int fo = f0 + c;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * ti + 4 * g + i;
        if (r < m) W[((size_t)bh * m + r) * D + fo] = acc[i];
      }
      // Landmarks 16ti + 4g .. +3 sit at positions 32(ti/2) + 8g + 4(ti%2) .. +3.
      const size_t o = ((size_t)bh * D + fo) * mpa + 32 * (ti >> 1) + 8 * g + 4 * (ti & 1);
      uint2 hv, lv;
      split_pair(acc[0], acc[1], hv.x, lv.x);
      split_pair(acc[2], acc[3], hv.y, lv.y);
      *reinterpret_cast<uint2*>(&wt_hi[o]) = hv;
      if constexpr (PR == 6) *reinterpret_cast<uint2*>(&wt_lo[o]) = lv;
    }
    return;
  }
  __syncthreads();
  {
    // W slice (m x 16) = Z (m x m) BV slice (m x 16) on the matrix cores,
    // three-way split (fp32-grade): wave ti computes row tile ti (m <= 256:
    // at most 16 tiles for the 16 waves); lane (c, g) ends with
    // W[16 ti + 4g + i][f0 + c].  Z rows are read from global memory, every
    // chunk's loads issued before the first product; rows and columns past
    // m read as zero.
    const int lane = tid & 63, ti = tid >> 6, c = lane & 15, g = lane >> 4;
    if (16 * ti < m) {
      const int r = 16 * ti + c;
      const bool rin = r < m;
      const bool vec = (m & 3) == 0;
      constexpr int NK = 8;  // 32-wide chunks of m <= 256
      float a[NK][8];
#pragma unroll
      for (int kc = 0; kc < NK; ++kc) {
        const int k0 = 32 * kc + 8 * g;
        if (vec && rin && k0 + 8 <= m) {
          const float4 u0 = *reinterpret_cast<const float4*>(&z[(size_t)r * m + k0]);
          const float4 u1 = *reinterpret_cast<const float4*>(&z[(size_t)r * m + k0 + 4]);
          a[kc][0] = u0.x; a[kc][1] = u0.y; a[kc][2] = u0.z; a[kc][3] = u0.w;
          a[kc][4] = u1.x; a[kc][5] = u1.y; a[kc][6] = u1.z; a[kc][7] = u1.w;
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) a[kc][q] = (rin && k0 + q < m) ? z[(size_t)r * m + k0 + q] : 0.f;
        }
      }
      f32x4_t acc = zero4();
#pragma unroll
      for (int kc = 0; kc < NK; ++kc) {
        if (32 * kc >= m) break;
        float b[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int k = 32 * kc + 8 * g + q;
          b[q] = k < m ? sbv[k][c] : 0.f;
        }
        acc = mma_f32<PR>(a[kc], b, acc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = 16 * ti + 4 * g + i;
        if (rr < m) {
          sw[rr][c] = acc[i];
          W[((size_t)bh * m + rr) * D + f0 + c] = acc[i];
        }
      }
    }
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

template <typename IO, int D, bool SIN>
static void seg_means_k(const Problem& p, const Ws& w, hipStream_t s) {
  using T = typename IO::T;
  const int BH = p.batch * p.heads;
  KernelTimer kt_("segment_mean", s);
  if ((p.n + p.m - 1) / p.m <= 32) {  // segments of at most 32 rows: a wave each (bert 123.3 -> 120.8 us)
    k_segment_mean<IO, D, true, SIN><<<dim3((p.m + 3) / 4, BH, 2), 256, 0, s>>>(
        static_cast<const T*>(p.Q), static_cast<const T*>(p.K), w.Qt, w.Kt, w.kt_hi, w.kt_lo, w.qt_hi, w.qt_lo,
        p.lens, p.heads, p.n, p.m, w.mpa, kLog2e / sqrtf((float)D), w.sync, 2 * BH, in_layout(p));
    return;
  }
  k_segment_mean<IO, D, false, SIN><<<dim3(p.m, BH, 2), 256, 0, s>>>(static_cast<const T*>(p.Q), static_cast<const T*>(p.K),
                                                         w.Qt, w.Kt, w.kt_hi, w.kt_lo, w.qt_hi, w.qt_lo, p.lens,
                                                         p.heads, p.n, p.m, w.mpa, kLog2e / sqrtf((float)D),
                                                         w.sync, 2 * BH, in_layout(p));
}

template <typename IO, int D>
static void seg_means_t(const Problem& p, const Ws& w, hipStream_t s) {
  if (p.in_ld > 0) seg_means_k<IO, D, true>(p, w, s); else seg_means_k<IO, D, false>(p, w, s);
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
    k_pinv_lds<32, PR><<<BH, 64 * kPinvWaves, sizeof(PinvSmem<32>), s>>>(w.Qt, w.Kt, w.A, w.Z, m, D, sl2e, p.iters, p.zsave,
                                                             p.zmp);
  } else if (m <= 64) {
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_pinv_lds<64, PR>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       (int)sizeof(PinvSmem<64>));
    if (attr != hipSuccess) return attr;
    KernelTimer kt_("pinv", s);
    k_pinv_lds<64, PR><<<BH, 64 * kPinvWaves, sizeof(PinvSmem<64>), s>>>(w.Qt, w.Kt, w.A, w.Z, m, D, sl2e, p.iters, p.zsave,
                                                             p.zmp);
  } else {
    {
      KernelTimer kt_("landmark_softmax", s);
      k_landmark_softmax<PR><<<dim3(ceil_div(m, 16), BH), 256, 0, s>>>(w.Qt, w.Kt, w.A, w.colp, w.rsum, m, D, sl2e);
    }
    const hipError_t attr = ensure_dynamic_smem(reinterpret_cast<const void*>(&k_mmr<PR>), kMmrSmem);
    if (attr != hipSuccess) return attr;
    const int T = p.iters, tiles = ceil_div(m, 64);
    // Z_t lives in Zb[t % 2]; the last, Z_T, in Zb[T % 2] = Z.
    float* Zb[2] = {T % 2 == 0 ? w.Z : w.V, T % 2 == 0 ? w.V : w.Z};
    auto launch = [&](int mode, const float* X, const float* Y, float* C, const float* F, float alpha, float beta) {
      MmrArgs ma;
      ma.job.mode = mode;
      ma.job.X = X;
      ma.job.Y = Y;
      ma.job.C = C;
      ma.job.F = F;
      ma.job.alpha = alpha;
      ma.job.beta = beta;
      ma.colp = w.colp;
      ma.rsum = w.rsum;
      ma.m = m;
      ma.nb = ceil_div(m, 16);
      KernelTimer kt_("pinv_mm", s);
      k_mmr<PR><<<tiles * tiles * BH, 512, kMmrSmem, s>>>(ma);
    };
    launch(kMmZ0, w.A, nullptr, Zb[0], nullptr, 0.f, 0.f);
    for (int t = 0; t < T; ++t) {
      float* Zt = Zb[t % 2];
      launch(kMmProduct, w.A, Zt, w.X, nullptr, 1.f, 0.f);                  // X = A Z
      launch(kMmProduct, w.X, w.X, w.T, w.X, -1.f, 7.f);                   // T = 7X - X X
      launch(kMmProduct, w.X, w.T, w.U, w.X, -1.f, 15.f);                  // U = 15X - X T
      launch(kMmProduct, Zt, w.U, Zb[(t + 1) % 2], Zt, -0.25f, 3.25f);     // Z' = (13Z - Z U) / 4
    }
  }
  return hipGetLastError();
}

bool pinv_in_landmark_pass(const Problem& p) { return p.bf16 && p.m <= 64; }

// fp32 I/O: the pseudoinverse in the same launch as the key pass (its LDS
// holds two key groups beside it for d <= 64).
static bool pinv_beside_keys(const Problem& p) { return !p.bf16 && p.m <= 64 && p.d <= 64; }

int forward_partials(const Problem& p, const Ws& w) { return pinv_in_landmark_pass(p) ? w.nchunks / 2 : w.nchunks; }

hipError_t stage_pinv(const Problem& p, const Ws& w, hipStream_t s) {
  if (pinv_in_landmark_pass(p) || pinv_beside_keys(p)) return hipSuccess;
  return p.bf16 ? pinv_t<3>(p, w, s) : pinv_t<6>(p, w, s);
}

static bool conv_uses_ops(const Problem& p) { return p.bf16 && p.conv_w && p.conv_k > 1 && p.conv_k <= 33; }

template <typename IO, int D, int NTW, int PMP, int CPB = 2>
static void landmark_pass_launch(const Problem& p, const Ws& w, hipStream_t s) {
  const int BH = p.batch * p.heads;
  LandmarkPassArgs a;
  a.K = p.K;
  a.V = p.V;
  a.zsave = p.zsave;
  a.zmp = p.zmp;
  a.Qt = w.Qt;
  a.Kt = w.Kt;
  a.qt_hi = w.qt_hi;
  a.qt_lo = w.qt_lo;
  a.kt_hi = w.kt_hi;
  a.kt_lo = w.kt_lo;
  a.A = w.A;
  a.Z = w.Z;
  a.pacc = w.pacc;
  a.pmax = w.pmax;
  a.psum = w.psum;
  a.conv_w = p.conv_w;
  a.cwop = w.cwop;
  a.lens = p.lens;
  a.n = p.n;
  a.heads = p.heads;
  a.m = p.m;
  a.chunk = w.chunk;
  a.nchunks = w.nchunks;
  a.iters = p.iters;
  a.npinv = PMP > 0 ? BH : 0;
  a.conv_total = conv_uses_ops(p) ? p.heads * p.d * 4 * 9 : 0;
  a.nconv = ceil_div(a.conv_total, 512);
  a.conv_k = p.conv_k;
  a.sl2e = kLog2e / sqrtf((float)D);
  a.sync = w.sync;
  a.BV = w.BV;
  a.W = w.W;
  a.wt_hi = w.wt_hi;
  a.bhn = BH;
  a.il = in_layout(p);
  KernelTimer kt_("landmark_pass", s);
  if constexpr (CPB == 1 && PMP == 0 && (IO::kBf16 || D <= 64)) {  // fp32 at d = 128 needs more registers
    a.nconv = ceil_div(a.conv_total, 1024);
    k_key_pass16<IO, D><<<a.nconv + w.nchunks * BH, 1024, 0, s>>>(a);
    return;
  }
  const int grid = a.npinv + a.nconv + (CPB == 2 ? w.nchunks / 2 : w.nchunks) * BH;
  if constexpr (PMP > 0 && CPB == 2 && (D == 32 || D == 64)) {
    if (p.in_ld > 0) {  // K, V read in place (launch_forward admits no other shape)
      k_landmark_pass<IO, D, NTW, PMP, false, CPB, true><<<grid, 512, 0, s>>>(a);
      return;
    }
  }
  if constexpr (PMP > 0) {
    if (p.zsave) {
      k_landmark_pass<IO, D, NTW, PMP, true><<<grid, 512, 0, s>>>(a);
      return;
    }
  }
  k_landmark_pass<IO, D, NTW, PMP, false, CPB><<<grid, 512, 0, s>>>(a);
}


template <int PMP, int D>
static hipError_t landmark_pass_f32_launch(const Problem& p, const Ws& w, hipStream_t s) {
  const int BH = p.batch * p.heads;
  LandmarkPassArgs a{};
  a.K = p.K;
  a.V = p.V;
  a.zsave = p.zsave;
  a.zmp = p.zmp;
  a.Qt = w.Qt;
  a.Kt = w.Kt;
  a.A = w.A;
  a.Z = w.Z;
  a.pacc = w.pacc;
  a.pmax = w.pmax;
  a.psum = w.psum;
  a.lens = p.lens;
  a.n = p.n;
  a.heads = p.heads;
  a.m = p.m;
  a.chunk = w.chunk;
  a.nchunks = w.nchunks;
  a.iters = p.iters;
  a.npinv = BH;
  a.sl2e = kLog2e / sqrtf((float)D);
  a.il = in_layout(p);
  constexpr int SMEM = sizeof(PinvSmem<PMP>) > 2 * sizeof(BvSmem<F32, D>) ? (int)sizeof(PinvSmem<PMP>)
                                                                            : (int)(2 * sizeof(BvSmem<F32, D>));
  auto go = [&](auto kern) -> hipError_t {
    const hipError_t attr = ensure_dynamic_smem(reinterpret_cast<const void*>(kern), SMEM);
    if (attr != hipSuccess) return attr;
    KernelTimer kt_("landmark_pass", s);
    kern<<<BH + (w.nchunks / 2) * BH, 64 * kPinvWaves, SMEM, s>>>(a, kLog2e / sqrtf((float)D));
    return hipSuccess;
  };
  if constexpr (D == 32 || D == 64) {
    if (p.in_ld > 0) return go(&k_landmark_pass_f32<PMP, D, true>);  // K, V read in place
  }
  return go(&k_landmark_pass_f32<PMP, D, false>);
}

template <typename IO, int D>
static void landmark_pass_t(const Problem& p, const Ws& w, hipStream_t s) {
  if constexpr (IO::kBf16) {
    if (p.m <= 32) return landmark_pass_launch<IO, D, 1, 32>(p, w, s);
    if (p.m <= 64) return landmark_pass_launch<IO, D, 1, 64>(p, w, s);
  }
  if (p.m <= 64)
    landmark_pass_launch<IO, D, 1, 0>(p, w, s);
  else if (p.m <= 128)
    landmark_pass_launch<IO, D, 2, 0>(p, w, s);
  else
    landmark_pass_launch<IO, D, 2, 0, 1>(p, w, s);  // 8 waves x 2 landmark tiles per chunk
}

hipError_t stage_landmark_pass(const Problem& p, const Ws& w, hipStream_t s) {
  if (pinv_beside_keys(p)) {
    hipError_t e;
    const bool small = p.m <= 32;
    switch (p.d) {
      case 16: e = small ? landmark_pass_f32_launch<32, 16>(p, w, s) : landmark_pass_f32_launch<64, 16>(p, w, s); break;
      case 32: e = small ? landmark_pass_f32_launch<32, 32>(p, w, s) : landmark_pass_f32_launch<64, 32>(p, w, s); break;
      default: e = small ? landmark_pass_f32_launch<32, 64>(p, w, s) : landmark_pass_f32_launch<64, 64>(p, w, s); break;
    }
    return e != hipSuccess ? e : hipGetLastError();
  }
  switch (p.d) {
    case 16: p.bf16 ? landmark_pass_t<BF16, 16>(p, w, s) : landmark_pass_t<F32, 16>(p, w, s); break;
    case 32: p.bf16 ? landmark_pass_t<BF16, 32>(p, w, s) : landmark_pass_t<F32, 32>(p, w, s); break;
    case 64: p.bf16 ? landmark_pass_t<BF16, 64>(p, w, s) : landmark_pass_t<F32, 64>(p, w, s); break;
    case 128: p.bf16 ? landmark_pass_t<BF16, 128>(p, w, s) : landmark_pass_t<F32, 128>(p, w, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t stage_bv_finish(const Problem& p, const Ws& w, hipStream_t s) {
  if (pinv_in_landmark_pass(p)) return hipSuccess;  // folded into the landmark pass
  const int BH = p.batch * p.heads;
  KernelTimer kt_("bv_finish", s);
  if (p.m <= 64 && p.bf16)
    k_bv_finish<true, 3><<<dim3(p.d / 16, BH), 1024, 0, s>>>(w.pacc, w.pmax, w.psum, w.Z, w.BV, w.W, w.wt_hi,
                                                            w.wt_lo, p.m, p.d, w.nchunks, w.mpa);
  else if (p.m <= 64)
    k_bv_finish<true, 6><<<dim3(p.d / 16, BH), 1024, 0, s>>>(w.pacc, w.pmax, w.psum, w.Z, w.BV, w.W, w.wt_hi,
                                                            w.wt_lo, p.m, p.d, w.nchunks, w.mpa);
  else
    k_bv_finish<false, 6><<<dim3(p.d / 16, BH), 1024, 0, s>>>(w.pacc, w.pmax, w.psum, w.Z, w.BV, w.W, w.wt_hi,
                                                             w.wt_lo, p.m, p.d, w.nchunks, w.mpa);
  return hipGetLastError();
}

}  // namespace nys

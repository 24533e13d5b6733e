// Nyström self-attention forward, landmark side: HIP kernels for gfx950 (CDNA4).
//
// Method: "Nyströmformer: A Nyström-Based Algorithm for Approximating
// Self-Attention" (paper deep-dive page, sec. 3.2 and 3.4).  Per (batch, head):
//   segment means Qt, Kt (Eq. 16)         -> k_segment_mean
//   A = softmax(Qt Kt^T / sqrt d), Z = Lemma-1 iterations from the
//   Pan-Schreiber start                    -> pinv_head inside k_landmark_pass (m <= 64,
//                                             bf16 I/O), k_pinv_lds (m <= 64, fp32 I/O) or
//                                             k_landmark_softmax + k_pinv_start + k_mm chain
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
// Key landmarks are also written, pre-multiplied by log2(e)/sqrt(d), as bf16
// hi/lo planes [bh][mpa][D] (rows m..mpa-1 zero), the operand layout of the
// output stage, whose scores then come out in base-2 units.
template <typename IO, int D>
__global__ __launch_bounds__(256) void k_segment_mean(const typename IO::T* __restrict__ Q,
                                                      const typename IO::T* __restrict__ K,
                                                      float* __restrict__ Qt, float* __restrict__ Kt,
                                                      uint16_t* __restrict__ kt_hi, uint16_t* __restrict__ kt_lo,
                                                      const int* __restrict__ lens, int heads, int n, int m,
                                                      int mpa, float sl2e) {
  using T = typename IO::T;
  constexpr int VEC = 16 / sizeof(T);
  constexpr int SLOTS = D / VEC;   // 16-byte vectors per row
  constexpr int RS = 256 / SLOTS;  // rows covered per pass
  __shared__ float part[4][D];
  const int j = blockIdx.x, bh = blockIdx.y;
  const int nb = seq_rows(lens, bh / heads, n, m);
  const int seg = (nb + m - 1) / m;
  const int rows = max(0, min(seg, nb - j * seg));  // real rows of this segment
  const T* X = (blockIdx.z == 0 ? Q : K) + ((size_t)bh * n + (size_t)j * seg) * D;
  float* out = (blockIdx.z == 0 ? Qt : Kt) + ((size_t)bh * m + j) * D;
  const int slot = threadIdx.x % SLOTS, r0 = threadIdx.x / SLOTS;
  float acc[VEC];
#pragma unroll
  for (int q = 0; q < VEC; ++q) acc[q] = 0.f;
  // 8 independent 16-byte loads in flight per thread, accumulated in row order.
  for (int r = r0; r < rows; r += 8 * RS) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int rr = r + u * RS;
      v[u] = rr < rows ? *reinterpret_cast<const uint4*>(X + (size_t)rr * D + slot * VEC) : make_uint4(0, 0, 0, 0);
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
      split_hi_lo(mean * sl2e, hi, lo);
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
                                                  int d, float sl2e, int iters, float* __restrict__ zsave,
                                                  int zmp) {
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
      load8_masked(kt, rk, m, kc + 8 * g, d, d, a);
      load8_masked(qt, rq, m, kc + 8 * g, d, d, b);
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
    if (zsave) {
      // For the backward pass: Z_k, X_k, T1_k = 15I - U, T2_k = 13I - T
      // ([zmp][zmp] fp32 each, zero beyond m).
      float* zs = zsave + ((size_t)bh * iters + it) * 4 * zmp * zmp;
      for (int e = tid; e < zmp * zmp; e += 256) {
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
  for (int e = tid; e < m * m; e += 256) {
    const int i = e / m, j = e % m;
    ao[e] = sm.A[i][j];
    zo[e] = Z[i][j];
  }
}

// ---------------------------------------------------------------------------
// Pseudoinverse for m <= 64 with bf16x3 products (bf16 I/O).  One block of
// MP/16 waves per head; wave j owns column block j (16 columns, all MP rows)
// of every iterate.  In C = P R the right operand's column block comes from
// the wave's own registers: a result in the matrix-core C layout (lane (c, g)
// holds rows 4g..4g+3 of column c of each 16-row tile) is already a B operand
// once the contraction index of every 32-chunk is taken in the order
//   slot 8g + q  <->  k = 4g + q (q < 4),  16 + 4g + (q - 4) (q >= 4).
// Only the left operands X = A Z and Z, which every wave needs whole, go
// through LDS, as bf16 hi/lo planes, row-major with each row's columns stored
// in that slot order (so a left-operand fragment is one 16-byte read per
// plane).  A stays in registers.  One iteration
//   X = A Z;  T = 7I - X;  T = 15I - X T;  T = 13I - X T;  Z = Z T / 4
// has two barriers: after X is stored, and after every wave has loaded the X
// and Z fragments it needs (before Z is overwritten).
template <int MP>
struct PinvSmem2 {
  static constexpr int LD = MP + 8;  // plane row pitch (bf16): rows stay 16-byte aligned
  static constexpr int PL = MP * LD;
  static constexpr int SP = MP + 4;  // fp32 score row pitch
  __align__(16) uint16_t xp[2][PL];  // X planes [hi, lo]; the fp32 scores alias them before the iterations
  __align__(16) uint16_t zp[2][PL];  // Z planes [hi, lo]
  float colp[4][MP];                 // partial column sums of A
  float rows[MP];                    // row sums of A
  __device__ float* S() { return reinterpret_cast<float*>(&xp[0][0]); }
  static_assert(sizeof(float) * MP * SP <= sizeof(uint16_t) * 2 * PL, "scores do not fit the X planes");
};

// B operand (chunks kc) of this wave's column block j from C-layout tiles v:
// slot q of chunk kc is element q % 4 of tile 2kc + q / 4, as
// scale * v + alpha * (row == column), split into bf16 hi/lo.
template <int MP>
__device__ __forceinline__ void to_bop(const f32x4_t (&v)[MP / 16], float scale, float alpha, int j,
                                       B8 (&bh)[MP / 32], B8 (&bl)[MP / 32]) {
  const int lane = threadIdx.x & 63, c = lane & 15, g = lane >> 4;
  const int col = 16 * j + c;
#pragma unroll
  for (int kc = 0; kc < MP / 32; ++kc)
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int t = 2 * kc + q / 4, i = q % 4;
      const float x = scale * v[t][i] + (16 * t + 4 * g + i == col ? alpha : 0.f);
      split_hi_lo(x, bh[kc].h[q], bl[kc].h[q]);
    }
}

// Stores a column block held as B-operand planes into row-major planes with
// slot-ordered columns (2-byte writes).
template <int MP>
__device__ __forceinline__ void store_bop(uint16_t* h, uint16_t* l, const B8 (&bh)[MP / 32],
                                          const B8 (&bl)[MP / 32], int j) {
  constexpr int LD = PinvSmem2<MP>::LD;
  const int lane = threadIdx.x & 63, c = lane & 15, g = lane >> 4;
  const int slot = 32 * (j >> 1) + 8 * (c >> 2) + 4 * (j & 1) + (c & 3);
#pragma unroll
  for (int kc = 0; kc < MP / 32; ++kc)
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int o = (16 * (2 * kc + q / 4) + 4 * g + q % 4) * LD + slot;
      h[o] = bh[kc].h[q];
      l[o] = bl[kc].h[q];
    }
}

// Left-operand fragments of all row tiles from slot-ordered planes.
template <int MP>
__device__ __forceinline__ void load_aop(const uint16_t* h, const uint16_t* l, B8 (&ah)[MP / 16][MP / 32],
                                         B8 (&al)[MP / 16][MP / 32]) {
  constexpr int LD = PinvSmem2<MP>::LD;
  const int lane = threadIdx.x & 63, c = lane & 15, g = lane >> 4;
#pragma unroll
  for (int t = 0; t < MP / 16; ++t)
#pragma unroll
    for (int kc = 0; kc < MP / 32; ++kc) {
      const int o = (16 * t + c) * LD + 32 * kc + 8 * g;
      ah[t][kc].q = *reinterpret_cast<const uint4*>(h + o);
      al[t][kc].q = *reinterpret_cast<const uint4*>(l + o);
    }
}

// acc[t] = P(t) R for every row tile t (bf16x3).
template <int MP>
__device__ __forceinline__ void chain_mm(const B8 (&ph)[MP / 16][MP / 32], const B8 (&pl)[MP / 16][MP / 32],
                                         const B8 (&rh)[MP / 32], const B8 (&rl)[MP / 32],
                                         f32x4_t (&acc)[MP / 16]) {
#pragma unroll
  for (int t = 0; t < MP / 16; ++t) {
    acc[t] = zero4();
#pragma unroll
    for (int kc = 0; kc < MP / 32; ++kc) acc[t] = mfma3(ph[t][kc], pl[t][kc], rh[kc], rl[kc], acc[t]);
  }
}

// Pseudoinverse of one head, run by a block of 4 * MP threads.  SAVE: also
// write each step's Z_k, X_k, T1_k, T2_k to zsave (for the backward pass);
// the plain forward's kernel is compiled without that code.
template <int MP, int D, bool SAVE>
__device__ __forceinline__ void pinv_head(PinvSmem2<MP>& sm, int bh, const float* __restrict__ Qt,
                                          const float* __restrict__ Kt, float* __restrict__ Aout,
                                          float* __restrict__ Zout, int m, float sl2e, int iters,
                                          float* __restrict__ zsave, int zmp) {
  using SM = PinvSmem2<MP>;
  constexpr int SP = SM::SP, RT = MP / 16, KC = MP / 32, CPT = MP / 4;
  constexpr int KCD = (D + 31) / 32;  // 32-wide chunks of the head dimension
  float* const S = sm.S();
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, c = lane & 15, g = lane >> 4;
  const float* qt = Qt + (size_t)bh * m * D;
  const float* kt = Kt + (size_t)bh * m * D;

  // Scaled scores of row block `wave`, computed transposed ((Kt Qt^T)^T) so
  // that lane (c, g) of tile tj ends with row 16*wave+c, columns 16tj+4g..+3.
  // Every fragment load is issued before the first product (rows and columns
  // are clamped in bounds and masked to zero outside).
  {
    const int rq = 16 * wave + c;
    float4 qv[KCD][2], kv[RT][KCD][2];
#pragma unroll
    for (int kc = 0; kc < KCD; ++kc) {
      const int k0 = min(32 * kc + 8 * g, D - 8);
      const float* src = qt + (size_t)min(rq, m - 1) * D + k0;
      qv[kc][0] = *reinterpret_cast<const float4*>(src);
      qv[kc][1] = *reinterpret_cast<const float4*>(src + 4);
#pragma unroll
      for (int tj = 0; tj < RT; ++tj) {
        const float* ks = kt + (size_t)min(16 * tj + c, m - 1) * D + k0;
        kv[tj][kc][0] = *reinterpret_cast<const float4*>(ks);
        kv[tj][kc][1] = *reinterpret_cast<const float4*>(ks + 4);
      }
    }
    auto frag = [](const float4 (&v)[2], bool ok, B8& h, B8& l) {
      const float x[8] = {v[0].x, v[0].y, v[0].z, v[0].w, v[1].x, v[1].y, v[1].z, v[1].w};
      float y[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) y[q] = ok ? x[q] : 0.f;
      split8(y, h, l);
    };
    B8 qh[KCD], ql[KCD];
#pragma unroll
    for (int kc = 0; kc < KCD; ++kc) frag(qv[kc], rq < m && 32 * kc + 8 * g < D, qh[kc], ql[kc]);
#pragma unroll
    for (int tj = 0; tj < RT; ++tj) {
      f32x4_t acc = zero4();
#pragma unroll
      for (int kc = 0; kc < KCD; ++kc) {
        B8 kh, kl;
        frag(kv[tj][kc], 16 * tj + c < m && 32 * kc + 8 * g < D, kh, kl);
        acc = mfma3(kh, kl, qh[kc], ql[kc], acc);
      }
      *reinterpret_cast<float4*>(&S[rq * SP + 16 * tj + 4 * g]) =
          make_float4(acc[0] * sl2e, acc[1] * sl2e, acc[2] * sl2e, acc[3] * sl2e);
    }
  }
  __syncthreads();

  // Row softmax: four adjacent lanes per row, CPT columns each.  Padded rows
  // and columns become 0.
  {
    const int r = tid >> 2, sub = tid & 3, j0 = sub * CPT;
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
    mx = fmaxf(mx, shfl_xor(mx, 1));
    mx = fmaxf(mx, shfl_xor(mx, 2));
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      a[q] = (r < m && j0 + q < m) ? exp2f(a[q] - mx) : 0.f;
      sum += a[q];
    }
    sum += shfl_xor(sum, 1);
    sum += shfl_xor(sum, 2);
    const float inv = r < m ? 1.f / sum : 0.f;
    float rs = 0.f;
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      a[q] *= inv;
      rs += a[q];
    }
    rs += shfl_xor(rs, 1);
    rs += shfl_xor(rs, 2);
#pragma unroll
    for (int u = 0; u < CPT / 4; ++u)
      *reinterpret_cast<float4*>(&S[r * SP + j0 + 4 * u]) = make_float4(a[4 * u], a[4 * u + 1], a[4 * u + 2], a[4 * u + 3]);
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
  {  // partial column sums over quarters of the rows
    const int col = tid % MP, part = tid / MP;
    float s = 0.f;
#pragma unroll 4
    for (int rr = 0; rr < MP / 4; ++rr) s += S[(part * (MP / 4) + rr) * SP + col];
    sm.colp[part][col] = s;
  }
  __syncthreads();
  // ||A||_1 (max column sum) and ||A||_inf (max row sum; entries are >= 0).
  float cz;
  {
    const int k = lane % MP;
    float cs = sm.colp[0][k] + sm.colp[1][k] + sm.colp[2][k] + sm.colp[3][k];
    float rm = sm.rows[k];
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      cs = fmaxf(cs, shfl_xor(cs, o));
      rm = fmaxf(rm, shfl_xor(rm, o));
    }
    cz = 1.f / (cs * rm);
  }

  // A as register-resident left operand (all row tiles, slot-ordered
  // columns); Z0 = cz A^T, column block `wave` = cz * (row block `wave` of A).
  B8 Ah[RT][KC], Al[RT][KC];
  B8 Zh[KC], Zl[KC];
  f32x4_t zf[RT];
#pragma unroll
  for (int t = 0; t < RT; ++t)
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const float* src = &S[(16 * t + c) * SP + 32 * kc + 4 * g];
      const float4 u0 = *reinterpret_cast<const float4*>(src);
      const float4 u1 = *reinterpret_cast<const float4*>(src + 16);
      const float x[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
      split8(x, Ah[t][kc], Al[t][kc]);
      if (t == wave) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const float z = cz * x[q];
          split_hi_lo(z, Zh[kc].h[q], Zl[kc].h[q]);
          zf[2 * kc + q / 4][q % 4] = z;
        }
      }
    }
  store_bop<MP>(sm.zp[0], sm.zp[1], Zh, Zl, wave);
  __syncthreads();  // every wave has read the scores before X overwrites them

  // For the backward pass: the column block `wave` of Z_k, X_k, T1_k =
  // X_k (7I - X_k) and T2_k = X_k (15I - T1_k), fp32 [zmp][zmp] each.
  auto save = [&](const f32x4_t (&v)[RT], int it, int which) {
    float* zs = zsave + (((size_t)bh * iters + it) * 4 + which) * zmp * zmp;
    const int col = 16 * wave + c;
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * t + 4 * g + i;
        if (row < zmp && col < zmp) zs[(size_t)row * zmp + col] = v[t][i];
      }
  };
  for (int it = 0; it < iters; ++it) {
    f32x4_t acc[RT];
    B8 Th[KC], Tl[KC];
    if constexpr (SAVE) save(zf, it, 0);
    // X = A Z: store X for every wave; keep T1 = 7I - X (own columns).
    chain_mm<MP>(Ah, Al, Zh, Zl, acc);
    if constexpr (SAVE) save(acc, it, 1);
    {
      B8 xh[KC], xl[KC];
      to_bop<MP>(acc, 1.f, 0.f, wave, xh, xl);
      store_bop<MP>(sm.xp[0], sm.xp[1], xh, xl, wave);
    }
    to_bop<MP>(acc, -1.f, 7.f, wave, Th, Tl);
    __syncthreads();
    B8 Ph[RT][KC], Pl[RT][KC], Rh[RT][KC], Rl[RT][KC];
    load_aop<MP>(sm.xp[0], sm.xp[1], Ph, Pl);
    load_aop<MP>(sm.zp[0], sm.zp[1], Rh, Rl);  // in flight during the two X products
    chain_mm<MP>(Ph, Pl, Th, Tl, acc);  // X T1
    if constexpr (SAVE) save(acc, it, 2);
    to_bop<MP>(acc, -1.f, 15.f, wave, Th, Tl);
    chain_mm<MP>(Ph, Pl, Th, Tl, acc);  // X T3
    if constexpr (SAVE) save(acc, it, 3);
    to_bop<MP>(acc, -1.f, 13.f, wave, Th, Tl);
    chain_mm<MP>(Rh, Rl, Th, Tl, acc);  // Z T5
#pragma unroll
    for (int t = 0; t < RT; ++t) zf[t] = acc[t] * 0.25f;
    to_bop<MP>(zf, 1.f, 0.f, wave, Zh, Zl);
    __syncthreads();  // every wave holds its X and Z fragments
    store_bop<MP>(sm.zp[0], sm.zp[1], Zh, Zl, wave);
  }

  // Z in fp32 straight from the last product.
  const int col = 16 * wave + c;
  if (col < m) {
    float* zo = Zout + (size_t)bh * m * m;
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * t + 4 * g + i;
        if (row < m) zo[(size_t)row * m + col] = zf[t][i];
      }
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
template <typename IO, int D, int NTW>
__device__ __forceinline__ void bv_chunk(BvSmem<IO, D>& sm, int ch, int bh, const typename IO::T* __restrict__ Kin,
                                         const typename IO::T* __restrict__ Vin, const float* __restrict__ Qt,
                                         float* __restrict__ pacc, float* __restrict__ pmax,
                                         float* __restrict__ psum, int n, int nb, int m, int chunk, int nchunks,
                                         float sl2e) {
  using T = typename IO::T;
  using SM = BvSmem<IO, D>;
  constexpr int KC = (D + 31) / 32;  // 32-wide k chunks over the head dimension
  constexpr int MD = D / 16;         // 16-row tiles of V^T
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, c = lane & 15, g = lane >> 4;
  // Keys [kbeg, kend) of this chunk; nb <= n is the head's number of real
  // keys (chunks past it are empty and leave max -inf, sum 0).
  const int kbeg = ch * chunk, kend = min(nb, kbeg + chunk);
  const T* Kh = Kin + (size_t)bh * n * D;
  const T* Vh = Vin + (size_t)bh * n * D;
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
  float *A, *Z, *pacc, *pmax, *psum;
  const float* conv_w;
  uint4* cwop;
  const int* lens;  // tokens per sequence, or nullptr
  int n, heads, m, chunk, nchunks, iters, npinv, nconv, conv_total, conv_k;
  float sl2e;
};

template <bool PINV, typename B>
union LandmarkPassSmem {
  PinvSmem2<64> p;
  B b;
};
template <typename B>
union LandmarkPassSmem<false, B> {
  B b;
};

template <typename IO, int D, int NTW, bool PINV, bool SAVE>
__global__ __launch_bounds__(256) void k_landmark_pass(LandmarkPassArgs a) {
  using T = typename IO::T;
  __shared__ LandmarkPassSmem<PINV, BvSmem<IO, D>> sm;
  int blk = blockIdx.x;
  if constexpr (PINV) {
    if (blk < a.npinv) {
      pinv_head<64, D, SAVE>(sm.p, blk, a.Qt, a.Kt, a.A, a.Z, a.m, a.sl2e, a.iters, a.zsave, a.zmp);
      return;
    }
    blk -= a.npinv;
  }
  if (blk < a.nconv) {
    const int idx = blk * 256 + (int)threadIdx.x;
    if (idx < a.conv_total) conv_operand(a.conv_w, a.cwop, idx, a.conv_k);
    return;
  }
  blk -= a.nconv;
  const int bh = blk / a.nchunks;
  bv_chunk<IO, D, NTW>(sm.b, blk % a.nchunks, bh, static_cast<const T*>(a.K), static_cast<const T*>(a.V), a.Qt,
                       a.pacc, a.pmax, a.psum, a.n, seq_rows(a.lens, bh / a.heads, a.n, a.m), a.m, a.chunk,
                       a.nchunks, a.sl2e);
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
  const int f = tid & 15;
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
        const float inv = 1.f / Lt;
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
  for (int i = tid >> 4; i < m; i += 64) {
    // Four interleaved partial sums (fixed order) keep the loads in flight.
    float acc4[4] = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < m; ++k) acc4[k & 3] = fmaf(z[(size_t)i * m + k], sbv[k][f], acc4[k & 3]);
    const float acc = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
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
                                                         w.Qt, w.Kt, w.kt_hi, w.kt_lo, p.lens, p.heads, p.n,
                                                         p.m, w.mpa,
                                                         kLog2e / sqrtf((float)D));
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
    k_pinv_lds<32, PR><<<BH, 256, sizeof(PinvSmem<32>), s>>>(w.Qt, w.Kt, w.A, w.Z, m, D, sl2e, p.iters, p.zsave,
                                                             p.zmp);
  } else if (m <= 64) {
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_pinv_lds<64, PR>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                                       (int)sizeof(PinvSmem<64>));
    if (attr != hipSuccess) return attr;
    KernelTimer kt_("pinv", s);
    k_pinv_lds<64, PR><<<BH, 256, sizeof(PinvSmem<64>), s>>>(w.Qt, w.Kt, w.A, w.Z, m, D, sl2e, p.iters, p.zsave,
                                                             p.zmp);
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

bool pinv_in_landmark_pass(const Problem& p) { return p.bf16 && p.m <= 64; }

hipError_t stage_pinv(const Problem& p, const Ws& w, hipStream_t s) {
  if (pinv_in_landmark_pass(p)) return hipSuccess;
  return p.bf16 ? pinv_t<3>(p, w, s) : pinv_t<6>(p, w, s);
}

static bool conv_uses_ops(const Problem& p) { return p.bf16 && p.conv_w && p.conv_k > 1 && p.conv_k <= 33; }

template <typename IO, int D, int NTW, bool PINV>
static void landmark_pass_launch(const Problem& p, const Ws& w, hipStream_t s) {
  const int BH = p.batch * p.heads;
  LandmarkPassArgs a;
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
  a.conv_w = p.conv_w;
  a.cwop = w.cwop;
  a.lens = p.lens;
  a.n = p.n;
  a.heads = p.heads;
  a.m = p.m;
  a.chunk = w.chunk;
  a.nchunks = w.nchunks;
  a.iters = p.iters;
  a.npinv = PINV ? BH : 0;
  a.conv_total = conv_uses_ops(p) ? p.heads * p.d * 4 * 9 : 0;
  a.nconv = ceil_div(a.conv_total, 256);
  a.conv_k = p.conv_k;
  a.sl2e = kLog2e / sqrtf((float)D);
  const int grid = a.npinv + a.nconv + w.nchunks * BH;
  KernelTimer kt_("landmark_pass", s);
  if constexpr (PINV) {
    if (p.zsave) {
      k_landmark_pass<IO, D, NTW, true, true><<<grid, 256, 0, s>>>(a);
      return;
    }
  }
  k_landmark_pass<IO, D, NTW, PINV, false><<<grid, 256, 0, s>>>(a);
}

template <typename IO, int D>
static void landmark_pass_t(const Problem& p, const Ws& w, hipStream_t s) {
  if constexpr (IO::kBf16) {
    if (p.m <= 64) return landmark_pass_launch<IO, D, 1, true>(p, w, s);
  }
  if (p.m <= 64)
    landmark_pass_launch<IO, D, 1, false>(p, w, s);
  else if (p.m <= 128)
    landmark_pass_launch<IO, D, 2, false>(p, w, s);
  else
    landmark_pass_launch<IO, D, 4, false>(p, w, s);
}

hipError_t stage_landmark_pass(const Problem& p, const Ws& w, hipStream_t s) {
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

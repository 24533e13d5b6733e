// Nyström self-attention forward, output stage (gfx950 / CDNA4):
//   out = softmax(Q Kt^T / sqrt d) W + DConv(V)
// ("Nyströmformer: A Nyström-Based Algorithm for Approximating Self-Attention",
// paper deep-dive page, sec. 3.4 "Putting It Together": Eq. 17 with the
// product taken as F~ (Z (B~ V)) = F~ W, and the depthwise-convolution skip of
// Figure 4).  The same kernel with the attention part switched off is the
// standalone depthwise-conv entry point.
//
// One block = TQ consecutive rows (queries) of one (batch, head), 4 waves:
//   A. stage the V rows the skip needs (tile plus a 16-row halo) in LDS,
//      feature-major (Vt[feature][row]);
//   B. each wave: scores for its queries against all landmarks on the matrix
//      cores, transposed (landmarks x queries) so that a query's scores sit in
//      one lane column; softmax across lanes; then O = F W, whose result tiles
//      give each lane 4 consecutive queries of one feature -> feature-major
//      LDS tile Ot[feature][row] (fp32), one 16-byte write per tile;
//   C. the skip.  bf16 I/O: on the matrix cores with the 16-block 4x4x4
//      instruction, one block per feature: A = a 4 x 4 band of that feature's
//      taps (Toeplitz), B = 4 consecutive V rows, 9 steps of 4 taps cover 33
//      taps for 16 output rows; each lane ends with 4 consecutive rows of one
//      feature and adds them to Ot with one 16-byte read-modify-write.  fp32
//      I/O, or one tap: fp32 FMAs by a register sliding window;
//   D. Ot -> output rows, one 16-byte store per lane, coalesced per row.
#include <math.h>

#include "nys_common.hpp"
#include "nys_internal.hpp"

namespace nys {

namespace {

typedef short bf16x4_t __attribute__((__vector_size__(4 * sizeof(short))));

template <int D>
struct ApplyShape {
  static constexpr int TQ = D >= 128 ? 64 : 128;  // rows per block
  static constexpr int NQ = TQ / 64;              // 16-query tiles per wave
  static constexpr int KC = (D + 31) / 32;        // 32-wide chunks of the head dim
  static constexpr int ND = D / 16;               // 16-feature tiles
};

// KW: 0 = no skip, 1 = one tap, 33 = up to 33 taps (zero-padded, centred),
//     -1 = wider filters (taps and rows read from global memory; slow path).
template <typename IO, int D, int KW>
struct ApplySmem {
  using T = typename IO::T;
  static constexpr int TQ = ApplyShape<D>::TQ;
  static constexpr int HALO = KW == 33 ? 16 : 0;
  static constexpr int VCOLS = TQ + 2 * HALO;
  static constexpr bool STAGE = KW == 1 || KW == 33;
  // Vt row pitch (elements): a multiple of 4 elements for 8/16-byte accesses.
  static constexpr int VP = VCOLS + (IO::kBf16 ? 16 : 4);
  static constexpr int OP = TQ + 4;  // Ot row pitch (floats)
  __align__(16) T vt[STAGE ? D * VP : 4];
  __align__(16) float ot[D * OP];
};

}  // namespace

template <typename IO, int D, int NTM, int KW, bool ATT>
__global__ __launch_bounds__(256) void k_apply(const typename IO::T* __restrict__ Qin,
                                               const typename IO::T* __restrict__ Vin,
                                               const uint16_t* __restrict__ kt_hi,
                                               const uint16_t* __restrict__ kt_lo,
                                               const uint16_t* __restrict__ wt_hi,
                                               const uint16_t* __restrict__ wt_lo,
                                               const float* __restrict__ conv_w, typename IO::T* __restrict__ out,
                                               int n, int m, int mpa, int heads, int conv_k, float sl2e) {
  using T = typename IO::T;
  using S = ApplyShape<D>;
  using SM = ApplySmem<IO, D, KW>;
  constexpr int TQ = S::TQ, NQ = S::NQ, KC = S::KC, ND = S::ND;
  constexpr int HALO = SM::HALO, VP = SM::VP, OP = SM::OP;
  __shared__ SM sm;
  const int bh = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, c = lane & 15, g = lane >> 4;
  const int t0 = blockIdx.x * TQ;
  const int h = bh % heads;
  const T* Vh = Vin + (size_t)bh * n * D;

  // A. V rows [t0 - HALO, t0 + TQ + HALO) -> Vt (feature-major), zero outside [0, n).
  if constexpr (SM::STAGE) {
    if constexpr (IO::kBf16) {
      // Task: 4 rows x 8 features -> 8 writes of 4 rows each.
      constexpr int TASKS = (SM::VCOLS / 4) * (D / 8);
      for (int e = tid; e < TASKS; e += 256) {
        const int rq = e / (D / 8), oc = e % (D / 8);
        uint4 r[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = t0 - HALO + 4 * rq + q;
          r[q] = (row >= 0 && row < n) ? *reinterpret_cast<const uint4*>(Vh + (size_t)row * D + 8 * oc)
                                       : make_uint4(0, 0, 0, 0);
        }
        const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&r[0]);
        const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&r[1]);
        const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&r[2]);
        const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&r[3]);
#pragma unroll
        for (int dw = 0; dw < 4; ++dw) {
          // features 8*oc + 2*dw (low halves) and 8*oc + 2*dw + 1 (high halves)
          const uint2 lo = make_uint2((w0[dw] & 0xffffu) | (w1[dw] << 16), (w2[dw] & 0xffffu) | (w3[dw] << 16));
          const uint2 hi = make_uint2((w0[dw] >> 16) | (w1[dw] & 0xffff0000u), (w2[dw] >> 16) | (w3[dw] & 0xffff0000u));
          *reinterpret_cast<uint2*>(&sm.vt[(8 * oc + 2 * dw) * VP + 4 * rq]) = lo;
          *reinterpret_cast<uint2*>(&sm.vt[(8 * oc + 2 * dw + 1) * VP + 4 * rq]) = hi;
        }
      }
    } else {
      // Task: 4 rows x 4 features -> 4 writes of 4 rows each.
      constexpr int TASKS = (SM::VCOLS / 4) * (D / 4);
      for (int e = tid; e < TASKS; e += 256) {
        const int rq = e / (D / 4), qc = e % (D / 4);
        float4 r[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = t0 - HALO + 4 * rq + q;
          r[q] = (row >= 0 && row < n) ? *reinterpret_cast<const float4*>(Vh + (size_t)row * D + 4 * qc)
                                       : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        *reinterpret_cast<float4*>(&sm.vt[(4 * qc + 0) * VP + 4 * rq]) = make_float4(r[0].x, r[1].x, r[2].x, r[3].x);
        *reinterpret_cast<float4*>(&sm.vt[(4 * qc + 1) * VP + 4 * rq]) = make_float4(r[0].y, r[1].y, r[2].y, r[3].y);
        *reinterpret_cast<float4*>(&sm.vt[(4 * qc + 2) * VP + 4 * rq]) = make_float4(r[0].z, r[1].z, r[2].z, r[3].z);
        *reinterpret_cast<float4*>(&sm.vt[(4 * qc + 3) * VP + 4 * rq]) = make_float4(r[0].w, r[1].w, r[2].w, r[3].w);
      }
    }
  }

  // B. Attention for this wave's NQ x 16 queries -> Ot; or zeros.
  if constexpr (ATT) {
    const T* Qh = Qin + (size_t)bh * n * D;
    const int qw = t0 + wave * 16 * NQ;
    B8 qh[NQ][KC], ql[NQ][KC];
#pragma unroll
    for (int u = 0; u < NQ; ++u)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const int row = qw + 16 * u + c, dd = kc * 32 + 8 * g;
        if constexpr (IO::kBf16) {
          qh[u][kc].q = (row < n && dd < D) ? *reinterpret_cast<const uint4*>(Qh + (size_t)row * D + dd)
                                            : make_uint4(0, 0, 0, 0);
        } else {
          float x[8];
          if (row < n && dd < D) {
            load8f<IO>(Qh + (size_t)row * D + dd, x);
          } else {
#pragma unroll
            for (int q = 0; q < 8; ++q) x[q] = 0.f;
          }
          split8(x, qh[u][kc], ql[u][kc]);
        }
      }

    // S^T (landmarks x queries) = Kt Q^T.
    f32x4_t sc[NQ][NTM];
    const uint16_t* kth = kt_hi + (size_t)bh * mpa * D;
    const uint16_t* ktl = kt_lo + (size_t)bh * mpa * D;
#pragma unroll
    for (int mt = 0; mt < NTM; ++mt) {
#pragma unroll
      for (int u = 0; u < NQ; ++u) sc[u][mt] = zero4();
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const int dd = kc * 32 + 8 * g;
        B8 kh, kl;
        if (dd < D) {
          const size_t o = (size_t)(mt * 16 + c) * D + dd;
          kh.q = *reinterpret_cast<const uint4*>(kth + o);
          kl.q = *reinterpret_cast<const uint4*>(ktl + o);
        } else {
          kh.q = make_uint4(0, 0, 0, 0);
          kl.q = make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < NQ; ++u) {
          if constexpr (IO::kBf16) {
            sc[u][mt] = mfma(kl, qh[u][kc], sc[u][mt]);
            sc[u][mt] = mfma(kh, qh[u][kc], sc[u][mt]);
          } else {
            sc[u][mt] = mfma3(kh, kl, qh[u][kc], ql[u][kc], sc[u][mt]);
          }
        }
      }
    }
    // Softmax over landmarks (lane's query = 16u + c; landmark = mt*16 + 4g + i).
    float inv[NQ];
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < NTM; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int lm = mt * 16 + 4 * g + i;
          sc[u][mt][i] = (lm < m) ? sc[u][mt][i] * sl2e : -INFINITY;
          mx = fmaxf(mx, sc[u][mt][i]);
        }
      mx = max_over_groups(mx);
      float sum = 0.f;
#pragma unroll
      for (int mt = 0; mt < NTM; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sc[u][mt][i] = exp2f(sc[u][mt][i] - mx);
          sum += sc[u][mt][i];
        }
      inv[u] = 1.f / sum_over_groups(sum);
    }

    // O (queries x features) = F W.  The W^T planes hold each 32-landmark chunk
    // in the order {4g..4g+3, 16+4g..16+4g+3}, the order the lanes hold F in.
    f32x4_t o[NQ][ND];
#pragma unroll
    for (int u = 0; u < NQ; ++u)
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) o[u][nd] = zero4();
    const uint16_t* wth = wt_hi + (size_t)bh * D * mpa;
    const uint16_t* wtl = wt_lo + (size_t)bh * D * mpa;
#pragma unroll
    for (int kk = 0; kk < NTM / 2; ++kk) {
      B8 fh[NQ], fl[NQ];
#pragma unroll
      for (int u = 0; u < NQ; ++u) {
        float f[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f[i] = sc[u][2 * kk][i] * inv[u];
          f[4 + i] = sc[u][2 * kk + 1][i] * inv[u];
        }
        split8(f, fh[u], fl[u]);
      }
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) {
        const size_t off = (size_t)(nd * 16 + c) * mpa + kk * 32 + 8 * g;
        B8 wh, wl;
        wh.q = *reinterpret_cast<const uint4*>(wth + off);
        wl.q = *reinterpret_cast<const uint4*>(wtl + off);
#pragma unroll
        for (int u = 0; u < NQ; ++u) o[u][nd] = mfma3(fh[u], fl[u], wh, wl, o[u][nd]);
      }
    }
    // Lane holds O[16u + 4g + i][nd*16 + c]: 4 consecutive rows of one feature.
#pragma unroll
    for (int u = 0; u < NQ; ++u)
#pragma unroll
      for (int nd = 0; nd < ND; ++nd)
        *reinterpret_cast<float4*>(&sm.ot[(nd * 16 + c) * OP + wave * 16 * NQ + 16 * u + 4 * g]) =
            make_float4(o[u][nd][0], o[u][nd][1], o[u][nd][2], o[u][nd][3]);
  } else {
    for (int e = tid; e < D * TQ / 4; e += 256) {
      const int f = e / (TQ / 4), r4 = e % (TQ / 4);
      *reinterpret_cast<float4*>(&sm.ot[f * OP + 4 * r4]) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  __syncthreads();

  // C. The skip, added into Ot.
  if constexpr (KW == 33 && IO::kBf16) {
    constexpr int FG = D / 16, RB = TQ / 16, UPW = FG * RB / 4;
    constexpr int NS = 9;  // 4-tap steps covering 33 taps for 4 rows
    const int b = lane >> 2, q4 = lane & 3;
    const int off = (33 - conv_k) / 2;
#pragma unroll
    for (int seg = 0; seg < (UPW >= RB ? UPW / RB : 1); ++seg) {
      const int u0 = wave * UPW + seg * RB;
      const int fg = u0 / RB;
      const int rb0 = u0 % RB;
      constexpr int NRB = UPW >= RB ? RB : UPW;
      const int f = fg * 16 + b;
      // A_s (hi/lo) for lane row i = q4: taps 4s + k' - i, centred in 33 slots.
      const float* wf = conv_w + ((size_t)h * D + f) * conv_k;
      bf16x4_t ah[NS], al[NS];
#pragma unroll
      for (int st = 0; st < NS; ++st)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int tt = 4 * st + k - q4 - off;
          const float wv = (tt >= 0 && tt < conv_k) ? wf[tt] : 0.f;
          uint16_t hi, lo;
          split_hi_lo(wv, hi, lo);
          ah[st][k] = (short)hi;
          al[st][k] = (short)lo;
        }
      // B_s for lane column j = q4: Vt[f][rb*16 + 4(j + s) .. +3]; consecutive
      // row blocks share 5 of 9 operands.
      const T* vf = &sm.vt[f * VP];
      bf16x4_t bw[NS + 4 * (NRB - 1)];
#pragma unroll
      for (int st = 0; st < NS + 4 * (NRB - 1); ++st) {
        const uint2 v = *reinterpret_cast<const uint2*>(vf + rb0 * 16 + 4 * (q4 + st));
        bw[st] = __builtin_bit_cast(bf16x4_t, v);
      }
#pragma unroll
      for (int r = 0; r < NRB; ++r) {
        f32x4_t acc = zero4();
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          acc = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(al[st], bw[4 * r + st], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(ah[st], bw[4 * r + st], acc, 0, 0, 0);
        }
        float4* dst = reinterpret_cast<float4*>(&sm.ot[f * OP + (rb0 + r) * 16 + 4 * q4]);
        float4 cur = *dst;
        cur.x += acc[0];
        cur.y += acc[1];
        cur.z += acc[2];
        cur.w += acc[3];
        *dst = cur;
      }
    }
  } else if constexpr (KW == 33 || KW == 1) {
    // fp32 sliding window: thread = (feature pair fp, row group rg).
    constexpr int P = D / 2, RG = 256 / P, RPT = TQ / RG;
    constexpr int NT = KW;
    const int rg = tid % RG, fp = tid / RG, r0 = rg * RPT;
    const int off = (NT - conv_k) / 2;
    const float* w0p = conv_w + ((size_t)h * D + 2 * fp) * conv_k;
    const float* w1p = w0p + conv_k;
    float w0[NT], w1[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int tt = t - off;
      const bool in = tt >= 0 && tt < conv_k;
      w0[t] = in ? w0p[tt] : 0.f;
      w1[t] = in ? w1p[tt] : 0.f;
    }
    float a0[RPT], a1[RPT];
#pragma unroll
    for (int r = 0; r < RPT; r += 4) {
      const float4 x0 = *reinterpret_cast<const float4*>(&sm.ot[(2 * fp) * OP + r0 + r]);
      const float4 x1 = *reinterpret_cast<const float4*>(&sm.ot[(2 * fp + 1) * OP + r0 + r]);
      a0[r] = x0.x; a0[r + 1] = x0.y; a0[r + 2] = x0.z; a0[r + 3] = x0.w;
      a1[r] = x1.x; a1[r + 1] = x1.y; a1[r + 2] = x1.z; a1[r + 3] = x1.w;
    }
    const T* v0p = &sm.vt[(2 * fp) * VP + r0];
    const T* v1p = &sm.vt[(2 * fp + 1) * VP + r0];
    // Output row r0 + r reads Vt columns r0 + r + t (t = 0 .. NT-1).
#pragma unroll
    for (int j = 0; j < RPT + NT - 1; ++j) {
      float v0, v1;
      if constexpr (IO::kBf16) {
        v0 = bf16_to_f32(v0p[j]);
        v1 = bf16_to_f32(v1p[j]);
      } else {
        v0 = v0p[j];
        v1 = v1p[j];
      }
#pragma unroll
      for (int r = 0; r < RPT; ++r) {
        const int t = j - r;
        if (t >= 0 && t < NT) {
          a0[r] = fmaf(w0[t], v0, a0[r]);
          a1[r] = fmaf(w1[t], v1, a1[r]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RPT; r += 4) {
      *reinterpret_cast<float4*>(&sm.ot[(2 * fp) * OP + r0 + r]) = make_float4(a0[r], a0[r + 1], a0[r + 2], a0[r + 3]);
      *reinterpret_cast<float4*>(&sm.ot[(2 * fp + 1) * OP + r0 + r]) =
          make_float4(a1[r], a1[r + 1], a1[r + 2], a1[r + 3]);
    }
  }
  if constexpr (KW == 33 || KW == 1) __syncthreads();

  // D. Ot -> output rows: 16 bytes (8 bf16 or 4 fp32 features) per lane.
  constexpr int FPL = IO::kBf16 ? 8 : 4;  // features per lane
  constexpr int GPR = D / FPL;            // lanes per row
  T* oh = out + (size_t)bh * n * D;
  for (int e = tid; e < TQ * GPR; e += 256) {
    const int p = e / GPR, fc = (e % GPR) * FPL;
    const int row = t0 + p;
    if (row >= n) continue;
    float v[FPL];
#pragma unroll
    for (int q = 0; q < FPL; ++q) v[q] = sm.ot[(fc + q) * OP + p];
    if constexpr (KW == -1) {
      const int R = (conv_k - 1) / 2;
      const int tb = max(0, R - row), te = min(conv_k, n - row + R);
#pragma unroll
      for (int q = 0; q < FPL; ++q) {
        const float* wq = conv_w + ((size_t)h * D + fc + q) * conv_k;
        for (int t = tb; t < te; ++t) v[q] = fmaf(wq[t], load_elem<IO>(Vh + (size_t)(row + t - R) * D + fc + q), v[q]);
      }
    }
    if constexpr (IO::kBf16) {
      B8 o8;
#pragma unroll
      for (int q = 0; q < 8; ++q) o8.h[q] = f32_to_bf16(v[q]);
      *reinterpret_cast<uint4*>(oh + (size_t)row * D + fc) = o8.q;
    } else {
      *reinterpret_cast<float4*>(oh + (size_t)row * D + fc) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers.

static int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }

template <typename IO, int D, int NTM, int KW, bool ATT>
static void launch_one(const Problem& p, const Ws* w, hipStream_t s) {
  using T = typename IO::T;
  constexpr int TQ = ApplyShape<D>::TQ;
  const int BH = p.batch * p.heads;
  const dim3 grid(cdiv(p.n, TQ), BH);
  k_apply<IO, D, NTM, KW, ATT><<<grid, 256, 0, s>>>(
      static_cast<const T*>(p.Q), static_cast<const T*>(p.V), w ? w->kt_hi : nullptr, w ? w->kt_lo : nullptr,
      w ? w->wt_hi : nullptr, w ? w->wt_lo : nullptr, p.conv_w, static_cast<T*>(p.out), p.n, p.m,
      w ? w->mpa : 0, p.heads, p.conv_k, kLog2e / sqrtf((float)D));
}

template <typename IO, int D, int NTM, bool ATT>
static void pick_kw(const Problem& p, const Ws* w, hipStream_t s) {
  if (!p.conv_w || p.conv_k <= 0)
    launch_one<IO, D, NTM, 0, ATT>(p, w, s);
  else if (p.conv_k == 1)
    launch_one<IO, D, NTM, 1, ATT>(p, w, s);
  else if (p.conv_k <= 33)
    launch_one<IO, D, NTM, 33, ATT>(p, w, s);
  else
    launch_one<IO, D, NTM, -1, ATT>(p, w, s);
}

template <typename IO, int D>
static void apply_t(const Problem& p, const Ws& w, hipStream_t s) {
  KernelTimer kt_("apply", s);
  switch (w.mpa) {  // landmark tiles of 16 = mpa / 16
    case 32: pick_kw<IO, D, 2, true>(p, &w, s); break;
    case 64: pick_kw<IO, D, 4, true>(p, &w, s); break;
    case 128: pick_kw<IO, D, 8, true>(p, &w, s); break;
    default: pick_kw<IO, D, 16, true>(p, &w, s); break;
  }
}

hipError_t stage_apply(const Problem& p, const Ws& w, hipStream_t s) {
  switch (p.d) {
    case 16: p.bf16 ? apply_t<BF16, 16>(p, w, s) : apply_t<F32, 16>(p, w, s); break;
    case 32: p.bf16 ? apply_t<BF16, 32>(p, w, s) : apply_t<F32, 32>(p, w, s); break;
    case 64: p.bf16 ? apply_t<BF16, 64>(p, w, s) : apply_t<F32, 64>(p, w, s); break;
    case 128: p.bf16 ? apply_t<BF16, 128>(p, w, s) : apply_t<F32, 128>(p, w, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename IO, int D>
static void dconv_t(const Problem& p, hipStream_t s) {
  KernelTimer kt_("dconv", s);
  pick_kw<IO, D, 2, false>(p, nullptr, s);
}

hipError_t launch_dconv(const void* V, const float* conv_w, void* out, int batch, int heads, int n, int d, int k,
                        bool bf16, hipStream_t s) {
  Problem p{nullptr, nullptr, V, conv_w, out, batch, heads, n, d, 1, 0, k, bf16};
  switch (d) {
    case 16: bf16 ? dconv_t<BF16, 16>(p, s) : dconv_t<F32, 16>(p, s); break;
    case 32: bf16 ? dconv_t<BF16, 32>(p, s) : dconv_t<F32, 32>(p, s); break;
    case 64: bf16 ? dconv_t<BF16, 64>(p, s) : dconv_t<F32, 64>(p, s); break;
    case 128: bf16 ? dconv_t<BF16, 128>(p, s) : dconv_t<F32, 128>(p, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace nys

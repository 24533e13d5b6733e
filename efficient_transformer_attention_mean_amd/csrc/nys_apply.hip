// Nyström self-attention forward, output stage (gfx950 / CDNA4):
//   out = softmax(Q Kt^T / sqrt d) W + DConv(V)
// ("Nyströmformer: A Nyström-Based Algorithm for Approximating Self-Attention",
// paper deep-dive page, sec. 3.4 "Putting It Together": Eq. 17 with the
// product taken as F~ (Z (B~ V)) = F~ W, and the depthwise-convolution skip of
// Figure 4).  The same kernel with the attention part switched off is the
// standalone depthwise-conv entry point.
//
// One block = 64 consecutive rows (queries) of one (batch, head), 4 waves.
// Blocks are numbered so that each XCD (block L runs on XCD L % 8) takes a
// contiguous run of tiles: neighbouring tiles share their halo rows and the
// tiles of a head share Kt/W operands through that XCD's L2.
//   0. every global load of the tile is issued first (V rows with a 16-row
//      halo, Q fragments), so that they are in flight during the attention;
//   1. each wave: scores of its 16 queries against all landmarks on the
//      matrix cores, transposed (landmarks x queries), so a query's scores sit
//      in one lane column; softmax across lanes; then O^T = W^T F^T, whose
//      result tiles give each lane 4 consecutive features of one query ->
//      row-major fp32 tile Ot[row][feature], one 16-byte write per tile;
//   2. the V rows -> LDS, feature-major (Vt[feature][row]);
//   3. the skip, added into Ot.  bf16 I/O: on the matrix cores with the
//      16-block 4x4x4 instruction, one block per feature: A = a 4 x 4 band of
//      that feature's taps (Toeplitz; operands prepared once per call in
//      the landmark pass), B = 4 consecutive V rows, 9 steps of 4 taps cover 33 taps
//      for 16 output rows; each lane ends with 4 consecutive rows of one
//      feature.  fp32 I/O, or one tap: fp32 FMAs by a register sliding window;
//   4. Ot -> output rows, one 16-byte store per lane, coalesced per row.
#include <math.h>

#include "nys_common.hpp"
#include "nys_internal.hpp"

namespace nys {

namespace {

typedef short bf16x4_t __attribute__((__vector_size__(4 * sizeof(short))));

constexpr int kTQ = 64;     // rows per tile: 4 waves x 16 queries
constexpr int kConvNS = 9;  // 4-tap steps of the matrix-core skip (33 taps)

// Shared-memory layout (bytes) of one block.
// KW: 0 = no skip, 1 = one tap, 33 = up to 33 taps (zero-padded, centred),
//     -1 = wider filters (taps and rows read from global memory; slow path).
template <typename IO, int D, int NTM, int KW, bool ATT>
struct ApplyLayout {
  using T = typename IO::T;
  static constexpr int MPA = 16 * NTM;
  static constexpr int HALO = KW == 33 ? 16 : 0;
  static constexpr int VCOLS = kTQ + 2 * HALO;
  static constexpr bool STAGE = KW == 1 || KW == 33;  // V rows staged in LDS; the skip goes through Ot
  // Matrix-core skip (bf16, up to 33 taps): row pitch 56 dwords (8 x odd)
  // plus 8 dwords before every group of 8 feature rows (vt_row), so that
  // both the staging writes (8 features 8 apart, 4 row groups per half wave)
  // and the skip's operand reads (8 consecutive features, 4 row groups) hit
  // 64 distinct LDS banks.  Otherwise a plain pitch.
  static constexpr bool PADG = IO::kBf16 && KW == 33;
  static constexpr int VP = PADG ? 112 : VCOLS + 4;  // Vt row pitch (elements; 8/16-byte aligned rows)
  static constexpr int VTE = D * VP + (PADG ? 16 * (D / 8) : 0);  // Vt elements
  static constexpr int OP = D + 4;      // Ot row pitch (floats)
  static constexpr int KP = D + 8;      // Kt plane row pitch (bf16): 16-byte reads of 16 rows hit distinct banks
  static constexpr int WP = MPA + 8;    // W^T plane row pitch (bf16)
  // Operand planes per matrix: bf16 I/O takes single bf16 products with
  // fp32 accumulation (hi plane only), fp32 I/O the three-product split.
  static constexpr int NPL = IO::kBf16 ? 1 : 2;
  // The current head's Kt and W^T planes are kept in LDS when they fit
  // (KWL), else read from global memory: beside the skip's buffers within
  // 72 KB; without them (no skip staged) within the LDS of a CU.
  static constexpr int PLANES = 2 * NPL * (MPA * KP + D * WP);
  static constexpr bool KWL = ATT && PLANES <= (STAGE ? 72 * 1024 : 159 * 1024);
  static constexpr int OT = 0;
  static constexpr int VT = OT + (STAGE ? 4 * kTQ * OP : 0);
  static constexpr int KT = VT + (STAGE ? (int)sizeof(T) * VTE : 0);
  static constexpr int WT = KT + (KWL ? 2 * NPL * MPA * KP : 0);
  static constexpr int BYTES = WT + (KWL ? 2 * NPL * D * WP : 0) + 16;
  // V tile loads: task = 4 rows x one 16-byte chunk.
  static constexpr int FPC = IO::kBf16 ? 8 : 4;  // features per 16-byte chunk
  static constexpr int NCH = D / FPC;
  static constexpr int TASKS = (VCOLS / 4) * NCH;
  static constexpr int NTK = STAGE ? (TASKS + 255) / 256 : 1;
  static constexpr int QW = IO::kBf16 ? 1 : 2;  // 16-byte words per 8 head-dim elements
};

// First element of feature f's Vt row.
template <typename LY>
__device__ __forceinline__ int vt_row(int f) {
  return f * LY::VP + (LY::PADG ? 16 * (f >> 3) : 0);
}

// Issues the loads of the V rows [t0 - HALO, t0 + 64 + HALO) of one head into
// registers; rows outside the head read as zero (buffer range check).  Every
// load is unconditional, so the compiler keeps exact counts of loads in flight.
template <typename LY>
__device__ __forceinline__ void load_v(uint4 (&vr)[LY::NTK][4], __amdgpu_buffer_rsrc_t rs, int t0, int ld) {
  constexpr int ES = 16 / LY::FPC;
#pragma unroll
  for (int k = 0; k < LY::NTK; ++k) {
    const int e = min((int)threadIdx.x + 256 * k, LY::TASKS - 1);
    const int rq = e / LY::NCH, oc = e % LY::NCH;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // Each row's offset stays in the address register: the range check
      // then sees the row itself (a row past the end inside a group of four
      // must not be reached through the instruction's immediate offset).
      int off = ((t0 - LY::HALO + 4 * rq + q) * ld + LY::FPC * oc) * ES;
      asm volatile("" : "+v"(off));
      vr[k][q] = buf_load16(rs, off);
    }
  }
}

// Issues the loads of this lane's query fragments (row qrow, head-dim
// elements 32kc + 8g .. +7 for every chunk kc); rows past the end read as zero.
// Rows are ld elements apart.
template <typename LY, int D>
__device__ __forceinline__ void load_q(uint4 (&qr)[(D + 31) / 32][LY::QW], __amdgpu_buffer_rsrc_t rs, int qrow,
                                       int ld) {
  constexpr int ES = 16 / LY::FPC;
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int kc = 0; kc < (D + 31) / 32; ++kc) {
    const int dd = min(kc * 32 + 8 * g, D - 8);
#pragma unroll
    for (int w = 0; w < LY::QW; ++w) qr[kc][w] = buf_load16(rs, (qrow * ld + dd) * ES + 16 * w);
  }
}

}  // namespace

// Persistent blocks: block `rank` (XCD-contiguous numbering) processes the
// run of 64-row tiles [rank * total / G, (rank + 1) * total / G) of the
// (batch*head)-major tile list.  Per tile, between two barriers:
//   region 1 (after the first barrier): the skip of the tile from the
//     feature-major V rows in LDS -> Ot (fp32, row-major), and, independent
//     of it, each wave's attention for its 16 queries into registers, so the
//     two interleave;
//   region 2 (after the second barrier): each lane adds its Ot values to its
//     attention values and stores them; then the next tile's V rows (loaded
//     two tiles ahead) go to LDS and the loads for the tile after next are
//     issued.
// The Q fragments of a tile are likewise loaded two tiles ahead.
// WPE: waves per SIMD the register allocation is held to (1 = no limit).
// ACC: add the attention to what `out` holds (the skip, written by an
// earlier launch) instead of overwriting it.
// NWV: waves per block, 16 rows each (tiles of 16 NWV rows).  Without the
// skip's staging the waves share only the head's planes, so when those fill
// the LDS a block of more waves hides more latency per CU; the tile's
// barriers are then needed only where a block moves to another head.
// SIN: Q and V rows where il says (the layer's QKV product); otherwise the
// [batch][heads][n][d] layout with its strides known at compile time.
template <typename IO, int D, int NTM, int KW, bool ATT, int WPE, bool ACC, int NWV = 4, bool SIN = false>
__global__ __launch_bounds__(64 * NWV) __attribute__((amdgpu_waves_per_eu(WPE))) void k_apply(const typename IO::T* __restrict__ Qin,
                                               const typename IO::T* __restrict__ Vin,
                                               const uint16_t* __restrict__ kt_hi,
                                               const uint16_t* __restrict__ kt_lo,
                                               const uint16_t* __restrict__ wt_hi,
                                               const uint16_t* __restrict__ wt_lo,
                                               const float* __restrict__ conv_w, const uint4* __restrict__ cwop,
                                               typename IO::T* __restrict__ out,
                                               const int* __restrict__ lens, int n, int m, int heads,
                                               int conv_k, int ntile, long long ntotal, int out_ld,
                                               long long out_hs, long long out_bs, InLayout il) {
  using T = typename IO::T;
  using LY = ApplyLayout<IO, D, NTM, KW, ATT>;
  static_assert(NWV == 4 || !LY::STAGE, "the staged skip is laid out for 4 waves");
  constexpr int TQ = 16 * NWV, NTH = 64 * NWV;  // rows per tile, threads per block
  constexpr int KC = (D + 31) / 32;  // 32-wide chunks of the head dimension
  constexpr int ND = D / 16;         // 16-feature tiles
  constexpr int FPG = D / 4;         // output features per lane (lane group g owns [g FPG, (g+1) FPG))
  constexpr bool KFULL = D % 32 == 0;
  constexpr int ES = sizeof(T);
  constexpr int MPA = LY::MPA, VP = LY::VP, OP = LY::OP, KP = LY::KP, WP = LY::WP;
  constexpr int NCH = LY::NCH, TASKS = LY::TASKS, NTK = LY::NTK;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  float* ot = reinterpret_cast<float*>(smem_raw + LY::OT);
  T* vt = reinterpret_cast<T*>(smem_raw + LY::VT);
  uint16_t* kp = reinterpret_cast<uint16_t*>(smem_raw + LY::KT);  // [hi (, lo)][MPA][KP]
  uint16_t* wp = reinterpret_cast<uint16_t*>(smem_raw + LY::WT);  // [hi (, lo)][D][WP]
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, c = lane & 15, g = lane >> 4;
  // Bytes of head bh's rows that hold tokens (the row pitch of a head is n
  // rows; with per-sequence lengths only the first ones are real): Q and V
  // rows past them read as zero through the range check.
  // Q and V: head bh's first element, and the bytes from there to the end
  // of its last token row (rows il.ld elements apart).
  const int ild = SIN ? il.ld : D;
  auto in_off = [&](int bh) -> long long {
    if constexpr (SIN) return (bh / heads) * il.bs + (bh % heads) * il.hs; else return (long long)bh * n * D;
  };
  auto token_bytes = [&](int bh) {
    const int nb = seq_rows(lens, bh / heads, n);
    if constexpr (SIN) return nb > 0 ? ((nb - 1) * il.ld + D) * ES : 0; else return nb * (D * ES);
  };

  // Run of tiles of this block.
  const long long G = gridDim.x, L = blockIdx.x;
  const long long xcd = L & 7, per = G >> 3, rem = G & 7;
  const long long rank = xcd * per + (xcd < rem ? xcd : rem) + (L >> 3);
  const long long tbeg = rank * ntotal / G, tend = (rank + 1) * ntotal / G;
  if (tbeg >= tend) return;

  // Skip filter operands (matrix-core path): one 16-feature group per
  // segment; kept in registers across tiles of one head when a wave has a
  // single segment, or (no attention part, registers to spare) for all of
  // its segments.
  constexpr int FG = D / 16, RB = kTQ / 16, UPW = FG * RB / 4;
  constexpr int NRB = UPW >= RB ? RB : UPW;  // consecutive row blocks per segment
  constexpr int NSEG = UPW / NRB;
  constexpr bool MMCONV = KW == 33 && IO::kBf16;
  constexpr int NSR = (MMCONV && NSEG > 1 && !ATT) ? NSEG : 1;  // operand sets held
  bf16x4_t ah[NSR][kConvNS], al[NSR][kConvNS];
  auto conv_operands = [&](int h, int seg, int slot) {
    const int b = lane >> 2, q4 = lane & 3;
    const int f = ((wave * UPW + seg * NRB) / RB) * 16 + b;
    if constexpr (ATT) {
      const uint4* src = cwop + ((size_t)(h * D + f) * 4 + q4) * kConvNS;
#pragma unroll
      for (int st = 0; st < kConvNS; ++st) {
        const uint4 v = src[st];
        ah[slot][st] = __builtin_bit_cast(bf16x4_t, make_uint2(v.x, v.y));
        al[slot][st] = __builtin_bit_cast(bf16x4_t, make_uint2(v.z, v.w));
      }
    } else {
      const int off = (33 - conv_k) / 2;
      const float* wf = conv_w + ((size_t)h * D + f) * conv_k;
#pragma unroll
      for (int st = 0; st < kConvNS; ++st)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int tt = 4 * st + k - q4 - off;
          const float wl = wf[min(max(tt, 0), conv_k - 1)];  // clamped: no branch per load
          const float wv = (tt >= 0 && tt < conv_k) ? wl : 0.f;
          uint16_t hi, lo;
          split_hi_lo(wv, hi, lo);
          ah[slot][st][k] = (short)hi;
          al[slot][st][k] = (short)lo;
        }
    }
  };

  // Two register sets of tile inputs, each two tiles ahead of its use.
  uint4 vra[NTK][4], vrb[NTK][4];
  uint4 qra[KC][LY::QW], qrb[KC][LY::QW];
  // Tile positions: (batch*head, tile within the head), stepped without division.
  struct Pos {
    int bh, ti;
  };
  auto step = [&](Pos q) {
    if (++q.ti == ntile) {
      q.ti = 0;
      ++q.bh;
    }
    return q;
  };
  const Pos pfirst{(int)(tbeg / ntile), (int)(tbeg % ntile)};
  const Pos plast{(int)((tend - 1) / ntile), (int)((tend - 1) % ntile)};
  const int count = (int)(tend - tbeg);  // tiles of this block
  // Position of the block's tile i + k, or its last tile past the end (loads
  // stay unconditional).  Positions are wave-uniform; readfirstlane says so
  // to the compiler, so buffer descriptors built from them stay scalar.
  auto ahead = [&](int i, Pos q, int k) {
    if (i + k >= count) return plast;
    for (int j = 0; j < k; ++j) q = step(q);
    return Pos{__builtin_amdgcn_readfirstlane(q.bh), __builtin_amdgcn_readfirstlane(q.ti)};
  };
  auto issue_v = [&](Pos q, uint4 (&vr)[NTK][4]) {
    if constexpr (LY::STAGE) load_v<LY>(vr, head_rsrc(Vin + in_off(q.bh), token_bytes(q.bh)), q.ti * kTQ, ild);
  };
  auto issue_q = [&](Pos q, uint4 (&qr)[KC][LY::QW]) {
    if constexpr (ATT)
      load_q<LY, D>(qr, head_rsrc(Qin + in_off(q.bh), token_bytes(q.bh)), q.ti * TQ + 16 * wave + c, ild);
  };

  // V rows (registers) -> Vt[feature][row].
  auto stage = [&](uint4 (&vr)[NTK][4]) {
    if constexpr (LY::STAGE) {
#pragma unroll
      for (int k = 0; k < NTK; ++k) {
        const int e = tid + 256 * k;
        if (e >= TASKS) continue;
        const int rq = e / NCH, oc = e % NCH;
        if constexpr (IO::kBf16) {
          const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vr[k][0]);
          const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vr[k][1]);
          const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vr[k][2]);
          const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vr[k][3]);
#pragma unroll
          for (int dw = 0; dw < 4; ++dw) {
            // features 8*oc + 2*dw (low halves) and 8*oc + 2*dw + 1 (high halves);
            // byte selects: 0x05040100 = {b.lo16, a.lo16}, 0x07060302 = {b.hi16, a.hi16}.
            const uint2 lo = make_uint2(__builtin_amdgcn_perm(w1[dw], w0[dw], 0x05040100u),
                                        __builtin_amdgcn_perm(w3[dw], w2[dw], 0x05040100u));
            const uint2 hi = make_uint2(__builtin_amdgcn_perm(w1[dw], w0[dw], 0x07060302u),
                                        __builtin_amdgcn_perm(w3[dw], w2[dw], 0x07060302u));
            const int f = 8 * oc + 2 * dw;
            *reinterpret_cast<uint2*>(&vt[vt_row<LY>(f) + 4 * rq]) = lo;
            *reinterpret_cast<uint2*>(&vt[vt_row<LY>(f + 1) + 4 * rq]) = hi;
          }
        } else {
          const float4 r0 = __builtin_bit_cast(float4, vr[k][0]), r1 = __builtin_bit_cast(float4, vr[k][1]);
          const float4 r2 = __builtin_bit_cast(float4, vr[k][2]), r3 = __builtin_bit_cast(float4, vr[k][3]);
          *reinterpret_cast<float4*>(&vt[(4 * oc + 0) * VP + 4 * rq]) = make_float4(r0.x, r1.x, r2.x, r3.x);
          *reinterpret_cast<float4*>(&vt[(4 * oc + 1) * VP + 4 * rq]) = make_float4(r0.y, r1.y, r2.y, r3.y);
          *reinterpret_cast<float4*>(&vt[(4 * oc + 2) * VP + 4 * rq]) = make_float4(r0.z, r1.z, r2.z, r3.z);
          *reinterpret_cast<float4*>(&vt[(4 * oc + 3) * VP + 4 * rq]) = make_float4(r0.w, r1.w, r2.w, r3.w);
        }
      }
    }
  };

  // The skip of the staged tile -> Ot (plain stores).
  auto skip = [&](int h) {
    if constexpr (MMCONV) {
      // bf16: on the matrix cores with the 16-block 4x4x4 instruction, one
      // block per feature: A = a 4 x 4 band of that feature's taps
      // (Toeplitz), B = 4 consecutive V rows; 9 steps of 4 taps cover 33 taps
      // for 16 output rows, and each lane ends with 4 consecutive rows of
      // one feature.  hi and lo tap planes accumulate separately.
      const int b = lane >> 2, q4 = lane & 3;
#pragma unroll
      for (int seg = 0; seg < NSEG; ++seg) {
        if constexpr (NSEG > 1 && NSR == 1) conv_operands(h, seg, 0);
        const int sl = NSR > 1 ? seg : 0;
        const int u0 = wave * UPW + seg * NRB;
        const int fg = u0 / RB, rb0 = u0 % RB;
        const int f = fg * 16 + b;
        // B_s for lane column j = q4: Vt[f][rb*16 + 4(j + s) .. +3];
        // consecutive row blocks share 5 of 9 operands.
        const T* vf = &vt[vt_row<LY>(f)];
        bf16x4_t bw[kConvNS + 4 * (NRB - 1)];
#pragma unroll
        for (int st = 0; st < kConvNS + 4 * (NRB - 1); ++st)
          bw[st] = __builtin_bit_cast(bf16x4_t, *reinterpret_cast<const uint2*>(vf + rb0 * 16 + 4 * (q4 + st)));
#pragma unroll
        for (int r = 0; r < NRB; ++r) {
          f32x4_t acc = zero4();
#pragma unroll
          for (int st = 0; st < kConvNS; ++st) {
            acc = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(al[sl][st], bw[4 * r + st], acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(ah[sl][st], bw[4 * r + st], acc, 0, 0, 0);
          }
          // Lane (b, q4) holds rows (rb0 + r)*16 + 4*q4 + i of feature f.
          float* dst = &ot[((rb0 + r) * 16 + 4 * q4) * OP + f];
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[i * OP] = acc[i];
        }
      }
    } else if constexpr (KW == 33 || KW == 1) {
      // fp32 sliding window: thread = (feature pair fp, row group rg).
      constexpr int P = D / 2, RG = 256 / P, RPT = kTQ / RG;
      constexpr int NT = KW;
      const int rg = tid % RG, fp = tid / RG, r0 = rg * RPT;
      const int off = (NT - conv_k) / 2;
      const float* w0p = conv_w + ((size_t)h * D + 2 * fp) * conv_k;
      const float* w1p = w0p + conv_k;
      float w0[NT], w1[NT];
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        const int ti = tt - off;
        const bool in = ti >= 0 && ti < conv_k;
        w0[tt] = in ? w0p[ti] : 0.f;
        w1[tt] = in ? w1p[ti] : 0.f;
      }
      float a0[RPT], a1[RPT];
#pragma unroll
      for (int r = 0; r < RPT; ++r) a0[r] = a1[r] = 0.f;
      const T* v0p = &vt[(2 * fp) * VP + r0];
      const T* v1p = &vt[(2 * fp + 1) * VP + r0];
      // Output row r0 + r reads Vt columns r0 + r + tt (tt = 0 .. NT-1).
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
          const int tt = j - r;
          if (tt >= 0 && tt < NT) {
            a0[r] = fmaf(w0[tt], v0, a0[r]);
            a1[r] = fmaf(w1[tt], v1, a1[r]);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < RPT; ++r) *reinterpret_cast<float2*>(&ot[(r0 + r) * OP + 2 * fp]) = make_float2(a0[r], a1[r]);
    }
  };

  // Attention of this wave's 16 queries: lane (c, g) ends with query
  // 16*wave + c, features g*FPG + 4*nd + i in o[nd][i].  Issues the Q loads
  // of tile `pq` once its own fragments are consumed.
  auto attention = [&](int bh, int t0, Pos pq, uint4 (&qr)[KC][LY::QW], f32x4_t (&o)[ND]) {
    B8 qh[KC], ql[KC];
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const bool ok = KFULL || kc * 32 + 8 * g < D;
      if constexpr (IO::kBf16) {
        qh[kc].q = ok ? qr[kc][0] : make_uint4(0, 0, 0, 0);
      } else {
        const float4 a = __builtin_bit_cast(float4, qr[kc][0]), b = __builtin_bit_cast(float4, qr[kc][LY::QW - 1]);
        float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int q = 0; q < 8; ++q) x[q] = ok ? x[q] : 0.f;
        split8(x, qh[kc], ql[kc]);
      }
    }
    // S^T (landmarks x queries) = Kt Q^T from the Kt planes.
    const uint16_t* kth = LY::KWL ? kp : kt_hi + (size_t)bh * MPA * D;
    const uint16_t* ktl = LY::KWL ? kp + MPA * KP : kt_lo + (size_t)bh * MPA * D;
    constexpr int KPI = LY::KWL ? KP : D;
    f32x4_t sc[NTM];
#pragma unroll
    for (int mt = 0; mt < NTM; ++mt) {
      sc[mt] = zero4();
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const int dd = kc * 32 + 8 * g;
        B8 kh, kl;
        const int o_ = (mt * 16 + c) * KPI + (KFULL ? dd : min(dd, D - 8));
        kh.q = *reinterpret_cast<const uint4*>(kth + o_);
        if constexpr (!IO::kBf16) kl.q = *reinterpret_cast<const uint4*>(ktl + o_);
        if (!KFULL && dd >= D) {
          kh.q = make_uint4(0, 0, 0, 0);
          kl.q = make_uint4(0, 0, 0, 0);
        }
        if constexpr (IO::kBf16) {
          sc[mt] = mfma(kh, qh[kc], sc[mt]);
        } else {
          sc[mt] = mfma3(kh, kl, qh[kc], ql[kc], sc[mt]);
        }
      }
    }
    issue_q(pq, qr);
    // Softmax over landmarks (lane's query = c; landmark = mt*16 + 4g + i).
    // Scores are already in base-2 units (the Kt planes carry log2(e)/sqrt(d)).
    if (m < MPA) {
#pragma unroll
      for (int mt = 0; mt < NTM; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (mt * 16 + 4 * g + i >= m) sc[mt][i] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < NTM; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[mt][i]);
    mx = max_over_groups(mx);
    float sum = 0.f;
#pragma unroll
    for (int mt = 0; mt < NTM; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sc[mt][i] = __builtin_amdgcn_exp2f(sc[mt][i] - mx);  // arguments <= 0; exp2(-inf) = 0
        sum += sc[mt][i];
      }
    const float inv = __builtin_amdgcn_rcpf(sum_over_groups(sum));  // sum >= 1 (the max term is 1)

    // O^T (features x queries) = W^T F^T.  The W^T planes hold each
    // 32-landmark chunk in the order {4g..4g+3, 16+4g..16+4g+3}, the order
    // this lane holds its query's probabilities in.  Row c of tile nd is
    // feature (c/4)*FPG + 4nd + c%4, so that a lane's output features are
    // contiguous; in LDS that feature's row is 16 nd + c.
    const uint16_t* wth = LY::KWL ? wp : wt_hi + (size_t)bh * D * MPA;
    const uint16_t* wtl = LY::KWL ? wp + D * WP : wt_lo + (size_t)bh * D * MPA;
    constexpr int WPI = LY::KWL ? WP : MPA;
#pragma unroll
    for (int nd = 0; nd < ND; ++nd) o[nd] = zero4();
#pragma unroll
    for (int kk = 0; kk < NTM / 2; ++kk) {
      B8 fh, fl;
      {
        float f[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f[i] = sc[2 * kk][i] * inv;
          f[4 + i] = sc[2 * kk + 1][i] * inv;
        }
        if constexpr (IO::kBf16) round8(f, fh); else split8(f, fh, fl);
      }
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) {
        const int frow = LY::KWL ? 16 * nd + c : (c >> 2) * FPG + 4 * nd + (c & 3);
        const int off = frow * WPI + kk * 32 + 8 * g;
        B8 wh, wl;
        wh.q = *reinterpret_cast<const uint4*>(wth + off);
        if constexpr (IO::kBf16) {
          o[nd] = mfma(wh, fh, o[nd]);
        } else {
          wl.q = *reinterpret_cast<const uint4*>(wtl + off);
          o[nd] = mfma3(wh, wl, fh, fl, o[nd]);
        }
      }
    }
  };

  // Attention + Ot (+ wide-filter skip) -> output row 16*wave + c of the
  // tile, features g*FPG .. +FPG-1: 16-byte stores (8-byte for bf16 at
  // d = 16); rows past the end are dropped by the range check, rows of a
  // sequence's padding (nb <= row < n) are written as zero.
  auto epilogue = [&](int bh, int h, int t0, int nb, const f32x4_t (&o)[ND]) {
    const int p = 16 * wave + c, row = t0 + p, f0 = g * FPG;
    float v[FPG];
#pragma unroll
    for (int nd = 0; nd < ND; ++nd)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (ATT) v[4 * nd + i] = o[nd][i]; else v[4 * nd + i] = 0.f;
      }
    if constexpr (LY::STAGE) {
#pragma unroll
      for (int nd = 0; nd < ND; ++nd) {
        const float4 x = *reinterpret_cast<const float4*>(&ot[p * OP + f0 + 4 * nd]);
        v[4 * nd] += x.x;
        v[4 * nd + 1] += x.y;
        v[4 * nd + 2] += x.z;
        v[4 * nd + 3] += x.w;
      }
    }
    if constexpr (KW == -1) {
      if (row < nb) {
        const T* Vh = Vin + in_off(bh);
        const int R = (conv_k - 1) / 2;
        const int tb = max(0, R - row), te = min(conv_k, nb - row + R);
        for (int q = 0; q < FPG; ++q) {
          const float* wq = conv_w + ((size_t)h * D + f0 + q) * conv_k;
          float s = 0.f;
          for (int tt = tb; tt < te; ++tt) s = fmaf(wq[tt], load_elem<IO>(Vh + (size_t)(row + tt - R) * ild + f0 + q), s);
          v[q] += s;
        }
      }
    }
    if (row >= nb) {
#pragma unroll
      for (int q = 0; q < FPG; ++q) v[q] = 0.f;
    }
    // Head bh's rows in `out`: out_ld elements apart; the range check ends
    // after the last row's d elements (rows past n are dropped).
    const __amdgpu_buffer_rsrc_t ro = head_rsrc(out + (bh / heads) * out_bs + (bh % heads) * out_hs,
                                                ((n - 1) * out_ld + D) * ES);
    const int base = (row * out_ld + f0) * ES;
    if constexpr (ACC) {
      // Rows past the tokens stay zero; rows past n read zero (range check).
      if (row < nb) {
        if constexpr (IO::kBf16) {
          if constexpr (FPG >= 8) {
#pragma unroll
            for (int j = 0; j < FPG / 8; ++j) {
              B8 o8;
              o8.q = buf_load16(ro, base + 16 * j);
#pragma unroll
              for (int q = 0; q < 8; ++q) v[8 * j + q] += bf16_to_f32(o8.h[q]);
            }
          } else {
            const uint2 x = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(ro, (unsigned)base, 0, 0));
            v[0] += __uint_as_float(x.x << 16);
            v[1] += __uint_as_float(x.x & 0xffff0000u);
            v[2] += __uint_as_float(x.y << 16);
            v[3] += __uint_as_float(x.y & 0xffff0000u);
          }
        } else {
#pragma unroll
          for (int j = 0; j < FPG / 4; ++j) {
            const float4 x = __builtin_bit_cast(float4, buf_load16(ro, base + 16 * j));
            v[4 * j] += x.x;
            v[4 * j + 1] += x.y;
            v[4 * j + 2] += x.z;
            v[4 * j + 3] += x.w;
          }
        }
      }
    }
    if constexpr (IO::kBf16) {
      if constexpr (FPG >= 8) {
#pragma unroll
        for (int j = 0; j < FPG / 8; ++j) {
          B8 o8;
#pragma unroll
          for (int q = 0; q < 4; ++q) o8.u[q] = pack_bf16x2(v[8 * j + 2 * q], v[8 * j + 2 * q + 1]);
          buf_store16(ro, base + 16 * j, o8.q);
        }
      } else {
        buf_store8(ro, base, make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])));
      }
    } else {
#pragma unroll
      for (int j = 0; j < FPG / 4; ++j)
        buf_store16(ro, base + 16 * j,
                    __builtin_bit_cast(uint4, make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3])));
    }
  };

  int cur = -1;
  // Tile t at `pos`: Q fragments in qr (two tiles ahead); vn holds the V rows
  // of tile t + 1, staged at the end, then refilled with tile t + 3's.
  auto tile = [&](int t, Pos pos, uint4 (&qr)[KC][LY::QW], uint4 (&vn)[NTK][4]) {
    const int bh = pos.bh, t0 = pos.ti * TQ, h = bh % heads;
    const bool fresh = bh != cur;  // block-uniform
    if (fresh) {
      // New head: its Kt / W^T planes -> LDS (the previous tile's readers
      // are past its second barrier, or past this one without the skip's
      // staging), filter operands.
      if constexpr (!LY::STAGE && LY::KWL) __syncthreads();
      if constexpr (LY::KWL) {
        const uint4* sk[2] = {reinterpret_cast<const uint4*>(kt_hi + (size_t)bh * MPA * D),
                              reinterpret_cast<const uint4*>(kt_lo + (size_t)bh * MPA * D)};
        for (int e = tid; e < LY::NPL * MPA * D / 8; e += NTH) {
          const int pl = e / (MPA * D / 8), r = (e % (MPA * D / 8)) / (D / 8), cc = e % (D / 8);
          *reinterpret_cast<uint4*>(kp + (pl * MPA + r) * KP + 8 * cc) = sk[pl][r * (D / 8) + cc];
        }
        const uint4* sw[2] = {reinterpret_cast<const uint4*>(wt_hi + (size_t)bh * D * MPA),
                              reinterpret_cast<const uint4*>(wt_lo + (size_t)bh * D * MPA)};
        for (int e = tid; e < LY::NPL * D * MPA / 8; e += NTH) {
          const int pl = e / (D * MPA / 8), r = (e % (D * MPA / 8)) / (MPA / 8), cc = e % (MPA / 8);
          // Feature r = a FPG + 4 nd + b sits in row 16 nd + 4a + b, so that the
          // 16 rows one product step reads are consecutive (distinct banks).
          const int rr = 16 * ((r % FPG) >> 2) + 4 * (r / FPG) + (r & 3);
          *reinterpret_cast<uint4*>(wp + (pl * D + rr) * WP + 8 * cc) = sw[pl][r * (MPA / 8) + cc];
        }
      }
      if constexpr (MMCONV && (NSEG == 1 || NSR > 1)) {
#pragma unroll
        for (int sg = 0; sg < NSR; ++sg) conv_operands(h, sg, sg);
      }
      cur = bh;
      // Rare path: settle its loads here so that the counts of the tile loads
      // in flight stay exact past the merge.
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    }
    // Vt of this tile and the planes visible; the previous epilogue's Ot reads done.
    if (LY::STAGE || fresh) __syncthreads();

    // A tile wholly inside a sequence's padding only writes zeros (its loads
    // past the tokens read zeros and move no data).
    const int nb = seq_rows(lens, bh / heads, n);
    const bool live = t0 < nb;
    if (live) skip(h);
    f32x4_t o[ND];
    if constexpr (ATT) {
      if (live) {
        attention(bh, t0, ahead(t, pos, 2), qr, o);
      } else {
        issue_q(ahead(t, pos, 2), qr);
#pragma unroll
        for (int nd = 0; nd < ND; ++nd) o[nd] = zero4();
      }
    }
    if constexpr (LY::STAGE) __syncthreads();  // Ot visible; the skip's Vt reads and the attention's plane reads done

    epilogue(bh, h, t0, nb, o);
    if constexpr (LY::STAGE) {
      stage(vn);
      issue_v(ahead(t, pos, 3), vn);
    }
  };

  issue_v(pfirst, vra);
  issue_q(pfirst, qra);
  const Pos p1 = ahead(0, pfirst, 1);
  issue_v(p1, vrb);
  issue_q(p1, qrb);
  stage(vra);
  issue_v(ahead(0, pfirst, 2), vra);
  int t = 0;
  Pos pos = pfirst;
  for (; t + 1 < count; t += 2) {
    tile(t, pos, qra, vrb);
    pos = step(pos);
    tile(t + 1, pos, qrb, vra);
    pos = step(pos);
  }
  if (t < count) tile(t, pos, qra, vrb);
}

// ---------------------------------------------------------------------------
// Launchers.

static int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }

// Blocks per CU the persistent grid is sized for (LDS and registers allow it
// for the common shapes; more resident blocks only queue).
static int multiprocessors() {
  static const int cus = [] {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 256;
    return v > 0 ? v : 256;
  }();
  return cus;
}

template <typename IO, int D, int NTM, int KW, bool ATT, bool ACC, bool SIN>
static hipError_t launch_one_k(const Problem& p, const Ws* w, hipStream_t s) {
  using T = typename IO::T;
  using LY = ApplyLayout<IO, D, NTM, KW, ATT>;
  // bf16 with the matrix-core skip at d <= 64, m <= 64 fits three blocks per
  // CU (LDS ~48 KB) when the registers are held to 168 per lane, without
  // spills; other instantiations keep the compiler's choice.
  constexpr int WPE = (IO::kBf16 && KW == 33 && ATT && D <= 64 && NTM <= 4) ? 3 : 1;
  // Without the skip, planes that leave room for at most one block per CU
  // get blocks of as many waves as the registers allow: 12 (three per SIMD)
  // for bf16 I/O, 8 for fp32 (stress shape: 767 -> 701 -> 690 us per call
  // for 4, 8 and 12 waves).
  constexpr int NWV = (KW == 0 && LY::KWL && LY::BYTES > 80 * 1024) ? (IO::kBf16 ? 12 : 8) : 4;
  constexpr int NTH = 64 * NWV;
  auto kern = &k_apply<IO, D, NTM, KW, ATT, WPE, ACC, NWV, SIN>;
  static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, LY::BYTES);
  if (attr != hipSuccess) return attr;
  static const int per_cu = [&] {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void*>(kern), NTH, LY::BYTES) !=
            hipSuccess ||
        nb < 1)
      nb = 1;
    return nb;
  }();
  const int ntile = cdiv(p.n, 16 * NWV);
  const long long total = (long long)ntile * p.batch * p.heads;
  const long long want = (long long)per_cu * multiprocessors();
  const int grid = (int)(total < want ? total : want);
  kern<<<grid, NTH, LY::BYTES, s>>>(static_cast<const T*>(p.Q), static_cast<const T*>(p.V), w ? w->kt_hi : nullptr,
                                    w ? w->kt_lo : nullptr, w ? w->wt_hi : nullptr, w ? w->wt_lo : nullptr, p.conv_w,
                                    w ? w->cwop : nullptr, static_cast<T*>(p.out), p.lens, p.n, p.m, p.heads, p.conv_k,
                                    ntile, total, p.out_merged ? p.heads * D : D,
                                    p.out_merged ? (long long)D : (long long)p.n * D,
                                    (long long)p.n * p.heads * D, in_layout(p));
  return hipSuccess;
}

// Q, K, V read in place from another layout (in_ld > 0) are compiled for the
// layer's common shapes only (apply_in_place); elsewhere the strides stay
// compile-time constants.
template <typename IO, int D, int NTM, int KW, bool ATT, bool ACC = false>
static hipError_t launch_one(const Problem& p, const Ws* w, hipStream_t s) {
  if (p.in_ld > 0) {
    if constexpr (ATT && !ACC && (KW == 0 || KW == 33) && (D == 32 || D == 64) && NTM <= 4)
      return launch_one_k<IO, D, NTM, KW, ATT, ACC, true>(p, w, s);
    else
      return hipErrorInvalidValue;
  }
  return launch_one_k<IO, D, NTM, KW, ATT, ACC, false>(p, w, s);
}

bool apply_in_place(const Problem& p) {
  return (p.d == 32 || p.d == 64) && p.m <= 64 && (!p.conv_w || p.conv_k <= 0 || (p.conv_k > 1 && p.conv_k <= 33));
}

template <typename IO, int D, int NTM, bool ATT>
static hipError_t pick_kw(const Problem& p, const Ws* w, hipStream_t s) {
  if (!p.conv_w || p.conv_k <= 0) return launch_one<IO, D, NTM, 0, ATT>(p, w, s);
  if (p.conv_k == 1) return launch_one<IO, D, NTM, 1, ATT>(p, w, s);
  if (p.conv_k <= 33) return launch_one<IO, D, NTM, 33, ATT>(p, w, s);
  return launch_one<IO, D, NTM, -1, ATT>(p, w, s);
}

// With a skip of up to 33 taps whose fused kernel cannot keep the head's
// Kt and W^T planes in LDS (they do not fit beside the skip's buffers) but
// whose attention-only kernel can, the skip runs first as the standalone
// convolution (out = DConv(V)) and the attention pass adds into out: two
// more passes over rows of out, against re-reading every plane from L2 for
// each 64-row tile.
template <typename IO, int D, int NTM>
static hipError_t apply_m(const Problem& p, const Ws& w, hipStream_t s) {
  if constexpr (!ApplyLayout<IO, D, NTM, 33, true>::KWL && ApplyLayout<IO, D, NTM, 0, true>::KWL) {
    if (p.conv_w && p.conv_k > 1 && p.conv_k <= 33) {
      hipError_t e;
      {
        KernelTimer kt_("dconv", s);
        e = launch_one<IO, D, 2, 33, false>(p, nullptr, s);
      }
      if (e != hipSuccess) return e;
      KernelTimer kt_("apply", s);
      return launch_one<IO, D, NTM, 0, true, true>(p, &w, s);
    }
  }
  KernelTimer kt_("apply", s);
  return pick_kw<IO, D, NTM, true>(p, &w, s);
}

template <typename IO, int D>
static hipError_t apply_t(const Problem& p, const Ws& w, hipStream_t s) {
  switch (w.mpa) {  // landmark tiles of 16 = mpa / 16
    case 32: return apply_m<IO, D, 2>(p, w, s);
    case 64: return apply_m<IO, D, 4>(p, w, s);
    case 128: return apply_m<IO, D, 8>(p, w, s);
    default: return apply_m<IO, D, 16>(p, w, s);
  }
}

hipError_t stage_apply(const Problem& p, const Ws& w, hipStream_t s) {
  hipError_t e;
  switch (p.d) {
    case 16: e = p.bf16 ? apply_t<BF16, 16>(p, w, s) : apply_t<F32, 16>(p, w, s); break;
    case 32: e = p.bf16 ? apply_t<BF16, 32>(p, w, s) : apply_t<F32, 32>(p, w, s); break;
    case 64: e = p.bf16 ? apply_t<BF16, 64>(p, w, s) : apply_t<F32, 64>(p, w, s); break;
    case 128: e = p.bf16 ? apply_t<BF16, 128>(p, w, s) : apply_t<F32, 128>(p, w, s); break;
    default: return hipErrorInvalidValue;
  }
  return e != hipSuccess ? e : hipGetLastError();
}

template <typename IO, int D>
static hipError_t dconv_t(const Problem& p, hipStream_t s) {
  KernelTimer kt_("dconv", s);
  return pick_kw<IO, D, 2, false>(p, nullptr, s);
}

hipError_t launch_dconv(const void* V, const float* conv_w, void* out, int batch, int heads, int n, int d, int k,
                        bool bf16, hipStream_t s, const int* lens) {
  Problem p{nullptr, nullptr, V, conv_w, out, batch, heads, n, d, 1, 0, k, bf16};
  p.lens = lens;
  hipError_t e;
  switch (d) {
    case 16: e = bf16 ? dconv_t<BF16, 16>(p, s) : dconv_t<F32, 16>(p, s); break;
    case 32: e = bf16 ? dconv_t<BF16, 32>(p, s) : dconv_t<F32, 32>(p, s); break;
    case 64: e = bf16 ? dconv_t<BF16, 64>(p, s) : dconv_t<F32, 64>(p, s); break;
    case 128: e = bf16 ? dconv_t<BF16, 128>(p, s) : dconv_t<F32, 128>(p, s); break;
    default: return hipErrorInvalidValue;
  }
  return e != hipSuccess ? e : hipGetLastError();
}

}  // namespace nys

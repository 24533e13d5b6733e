// Device helpers shared by the Nyström attention kernels (gfx950 / CDNA4).
//
// Matrix-core convention used throughout: v_mfma_f32_16x16x32_bf16, one wave
// (64 lanes), lane l = 16*g + c with g = l >> 4 (0..3), c = l & 15:
//   A operand (16 x 32, row-major M x K): lane holds A[c][8g .. 8g+7]
//   B operand (32 x 16, K x N):          lane holds B[8g .. 8g+7][c]
//   C / D     (16 x 16):                 lane holds D[4g .. 4g+3][c]
// A contraction only needs A's k-slot q and B's k-slot q to name the same
// index, so kernels may feed a permuted k order to both operands.
//
// Extra precision ("bf16x3"): an fp32 value x is split into hi = bf16(x) and
// lo = bf16(x - hi), so x = hi + lo up to about 2^-16 |x|; a product is then
// hi*hi + hi*lo + lo*hi on the matrix cores with fp32 accumulation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nys {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));

union B8 {
  bf16x8_t v;
  uint32_t u[4];
  uint16_t h[8];
  uint4 q;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// Round to nearest even (gfx950 has a hardware conversion; the cast uses it).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ void split_hi_lo(float x, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_bf16(x);
  lo = f32_to_bf16(x - bf16_to_f32(hi));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two values rounded to bf16 (RNE) in one packed conversion: x0 in the low half.
__device__ __forceinline__ uint32_t pack_bf16x2(float x0, float x1) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){x0, x1}, bf16x2_t));
}

// split_hi_lo for a pair, on packed conversions.
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(x0, x1);
  lo = pack_bf16x2(x0 - __uint_as_float(hi << 16), x1 - __uint_as_float(hi & 0xffff0000u));
}

__device__ __forceinline__ void split8(const float (&x)[8], B8& hi, B8& lo) {
#pragma unroll
  for (int q = 0; q < 4; ++q) split_pair(x[2 * q], x[2 * q + 1], hi.u[q], lo.u[q]);
}

__device__ __forceinline__ void round8(const float (&x)[8], B8& hi) {
#pragma unroll
  for (int q = 0; q < 4; ++q) hi.u[q] = pack_bf16x2(x[2 * q], x[2 * q + 1]);
}

__device__ __forceinline__ f32x4_t mfma(const B8& a, const B8& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}

// acc += (ah + al)(bh + bl) without the lo*lo term.
__device__ __forceinline__ f32x4_t mfma3(const B8& ah, const B8& al, const B8& bh, const B8& bl, f32x4_t c) {
  c = mfma(al, bh, c);
  c = mfma(ah, bl, c);
  return mfma(ah, bh, c);
}

__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }

// Three-way split x = hi + mid + lo (each bf16; both differences are exact in
// fp32), leaving about 2^-24 |x|: fp32-grade products from six bf16 products.
// Pairs of elements per packed conversion (the same RNE values as one at a time).
__device__ __forceinline__ void split8x3(const float (&x)[8], B8& hi, B8& mid, B8& lo) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float x0 = x[2 * q], x1 = x[2 * q + 1];
    const uint32_t h = pack_bf16x2(x0, x1);
    const float r0 = x0 - __uint_as_float(h << 16), r1 = x1 - __uint_as_float(h & 0xffff0000u);
    const uint32_t md = pack_bf16x2(r0, r1);
    const float s0 = r0 - __uint_as_float(md << 16), s1 = r1 - __uint_as_float(md & 0xffff0000u);
    hi.u[q] = h;
    mid.u[q] = md;
    lo.u[q] = pack_bf16x2(s0, s1);
  }
}

// acc += a b for 8-element fp32 fragments (A: 16 x 32 row slice, B: 32 x 16).
// P = 3: bf16x3 (about 2^-17 relative per product); P = 6: three-way split,
// terms of order 2^-16 and above kept (about 2^-24).
template <int P>
__device__ __forceinline__ f32x4_t mma_f32(const float (&a)[8], const float (&b)[8], f32x4_t acc) {
  if constexpr (P == 3) {
    B8 ah, al, bh, bl;
    split8(a, ah, al);
    split8(b, bh, bl);
    return mfma3(ah, al, bh, bl, acc);
  } else {
    B8 ah, am, al, bh, bm, bl;
    split8x3(a, ah, am, al);
    split8x3(b, bh, bm, bl);
    acc = mfma(al, bh, acc);
    acc = mfma(ah, bl, acc);
    acc = mfma(am, bm, acc);
    acc = mfma(am, bh, acc);
    acc = mfma(ah, bm, acc);
    return mfma(ah, bh, acc);
  }
}

// Element types at the boundary.
struct F32 {
  using T = float;
  static constexpr bool kBf16 = false;
};
struct BF16 {
  using T = uint16_t;
  static constexpr bool kBf16 = true;
};

template <typename IO>
__device__ __forceinline__ float load_elem(const typename IO::T* p) {
  if constexpr (IO::kBf16) return bf16_to_f32(*p); else return *p;
}

template <typename IO>
__device__ __forceinline__ void store_elem(typename IO::T* p, float v) {
  if constexpr (IO::kBf16) *p = f32_to_bf16(v); else *p = v;
}

// Load 8 consecutive elements (16-byte aligned for bf16, 32-byte for fp32) as floats.
template <typename IO>
__device__ __forceinline__ void load8f(const typename IO::T* p, float (&x)[8]) {
  if constexpr (IO::kBf16) {
    B8 b;
    b.q = *reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int q = 0; q < 8; ++q) x[q] = bf16_to_f32(b.h[q]);
  } else {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 c = *reinterpret_cast<const float4*>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = c.x; x[5] = c.y; x[6] = c.z; x[7] = c.w;
  }
}

// x = base[row][col0 .. col0+7] (row pitch ld), zero where row >= rows or
// col0 >= cols; cols and col0 are multiples of 8.  Both 16-byte loads are
// issued from clamped, in-bounds addresses without a branch, so the loads of
// several calls are in flight together.
__device__ __forceinline__ void load8_masked(const float* __restrict__ base, int row, int rows, int col0, int cols,
                                             int ld, float (&x)[8]) {
  const float* src = base + (size_t)min(row, rows - 1) * ld + min(col0, cols - 8);
  const float4 u0 = *reinterpret_cast<const float4*>(src);
  const float4 u1 = *reinterpret_cast<const float4*>(src + 4);
  const bool ok = row < rows && col0 < cols;
  const float v[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
  for (int q = 0; q < 8; ++q) x[q] = ok ? v[q] : 0.f;
}

// Cross-lane helpers within a wave of 64.
__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Reductions over lanes c, c+16, c+32, c+48 with gfx950's row swaps
// (v_permlane16_swap / v_permlane32_swap, no LDS round trip).  With both
// operands equal, the 16-swap returns {rows 0,0,2,2} and {rows 1,1,3,3} and
// the 32-swap {low half twice} and {high half twice}; every lane of a group
// ends with the same bits ((x0 op x1) op (x2 op x3)).
__device__ __forceinline__ float max_over_groups(float v) {
  const uint32_t b = __float_as_uint(v);
  const auto p = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  v = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const uint32_t b2 = __float_as_uint(v);
  const auto q = __builtin_amdgcn_permlane32_swap(b2, b2, false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}
__device__ __forceinline__ float sum_over_groups(float v) {
  const uint32_t b = __float_as_uint(v);
  const auto p = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const uint32_t b2 = __float_as_uint(v);
  const auto q = __builtin_amdgcn_permlane32_swap(b2, b2, false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// Buffer resource over `bytes` bytes from `base`: 32-bit byte offsets, range
// checked by the hardware (loads at offsets >= `bytes` return zero, stores
// there are dropped; a negative offset reads as a huge unsigned one).  The
// third word sets a 32-bit data format, under which untyped dword accesses
// are range checked.
constexpr int kRawBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kRawBufferWord3);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (unsigned)off, 0, 0));
}

__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, int off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, (unsigned)off, 0, 0);
}

__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, int off, uint2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, v), r, (unsigned)off, 0, 0);
}

// Device-coherent accesses: the cache policy that agent-scope atomic loads
// and stores carry (the sc1 scope bit, 16 in the buffer instructions' aux
// operand).  The L2 of each XCD is not coherent with the others; with these,
// a block reads what another block of the same launch wrote, on any XCD,
// once the writer's stores have completed (wait_stores) before it signals
// through an agent-scope atomic, with no L2 writeback or invalidation.
constexpr int kDeviceCoherent = 16;

__device__ __forceinline__ void st_coh(__amdgpu_buffer_rsrc_t r, int off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (unsigned)off, 0, kDeviceCoherent);
}
__device__ __forceinline__ void st_coh4(__amdgpu_buffer_rsrc_t r, int off, float4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, (unsigned)off, 0, kDeviceCoherent);
}
__device__ __forceinline__ float ld_coh(__amdgpu_buffer_rsrc_t r, int off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (unsigned)off, 0, kDeviceCoherent));
}
__device__ __forceinline__ float4 ld_coh4(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, (unsigned)off, 0, kDeviceCoherent));
}

// Waits until every memory access this lane issued has completed.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

constexpr float kLog2e = 1.4426950408889634f;

// Rows of batch entry b that are tokens: lens[b] clamped to [0, n] for a
// batch of right-padded sequences, n without lengths (lens == nullptr).
__device__ __forceinline__ int seq_rows(const int* __restrict__ lens, int b, int n) {
  return lens ? min(max(lens[b], 0), n) : n;
}

}  // namespace nys

// Device-side helpers shared by the gfx950 kernels of libpsa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace psa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D(32x32, f32) += A(32x16, bf16) * B(16x32, bf16) on the matrix cores.
// Lane l supplies A[l%32][8*(l/32) + j] and B[8*(l/32) + j][l%32] for j = 0..7,
// and holds D[8*(r/4) + 4*(l/32) + r%4][l%32] in accumulator element r.
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(16x16, f32) += A(16x32, bf16) * B(32x16, bf16). Lane l supplies
// A[l%16][8*(l/16) + j] and B[8*(l/16) + j][l%16] for j = 0..7, and holds
// D[4*(l/16) + r][l%16] in accumulator element r (checked on gfx950).
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
  return __builtin_bit_cast(float, static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bf16 bit pattern (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// 8 bf16 values p[0], p[stride], ..., p[7*stride], zero where idx0 + e >= limit.
__device__ __forceinline__ u32x4 gather8(const uint16_t* p, int64_t stride, int idx0, int limit) {
  u32x4 r;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t lo = (idx0 + 2 * w < limit) ? p[(2 * w) * stride] : 0u;
    const uint32_t hi = (idx0 + 2 * w + 1 < limit) ? p[(2 * w + 1) * stride] : 0u;
    r[w] = lo | (hi << 16);
  }
  return r;
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// One MFMA operand (8 values along LDS rows) from two ds_read_b64_tr_b16: each
// reads 8 bytes per lane, and inside each 16-lane group output lane i receives
// element i%4 of the 8 bytes addressed by lane 4r + i/4 (r = 0..3), a 4x16
// transpose. The second read is 4 rows (`row` elements per row) further on.
__device__ __forceinline__ bf16x8 lds_read_tr8(const uint16_t* p, int row) {
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 4 * row));
  const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  return as_bf16x8(u32x4{a[0], a[1], b[0], b[1]});
}

// The same operand with the two reads' addresses given separately (tiles
// whose rows are swizzled differently).
__device__ __forceinline__ bf16x8 lds_read_tr8_2(const uint16_t* p_lo, const uint16_t* p_hi) {
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p_lo));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p_hi));
  const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  return as_bf16x8(u32x4{a[0], a[1], b[0], b[1]});
}

// Index held by row rho (0..31) of a 32-row accumulator block whose A operand
// was read with tr_key_col: 8h + 4g + e -> 8g + 4h + e inside each 16-row half.
// Accumulator element r of lane group g then holds index 16*(r/8) + 8g + r%8:
// 8 consecutive indices per 8 elements, ready to be a B operand over them.
__device__ __forceinline__ int key_of_row(int rho) {
  return (rho & 16) | ((rho & 4) << 1) | ((rho & 8) >> 1) | (rho & 3);
}

// Column offset a 16-lane group's source lane s supplies for a transposed
// read, so that output lane i receives index key_of_row(i).
__device__ __forceinline__ int tr_key_col(int s) { return ((s & 1) << 3) | ((s & 2) << 1); }

// Position of 16-byte chunk c of row `row` in an unpadded LDS tile of 64
// bf16 columns: an XOR swizzle with x = (row >> 1) & 7 mapped to
// ((x & 1) << 2) | (x >> 1). The map is a bijection of 0..7, so the 16 rows
// one 16-byte-per-lane instruction reads together fall on 16 different bank
// groups; and rows 4k + 2, 4k + 3 flip chunk bit 2 against rows 4k, 4k + 1, so
// a transposed read of chunks 4j..4j+3 of four consecutive rows (one 32-lane
// half of ds_read_b64_tr_b16) covers all 64 banks once.
__device__ __forceinline__ int tile_chunk_pos(int row, int c) {
  const int x = (row >> 1) & 7;
  return c ^ (((x & 1) << 2) | (x >> 1));
}

// Position of 16-byte chunk c of row `row` in an unpadded tile of packed rows
// of D columns (D/8 chunks per row): an XOR swizzle chosen so that neither the
// 16-byte operand reads (rows in key_of_row order) nor the transposed 8-byte
// operand reads (rows r and r + 4) of one instruction meet twice on a bank.
// Both attention directions read their packed row tiles in these two ways.
template <int D>
__device__ __forceinline__ int packed_chunk_pos(int row, int c) {
  static_assert(D == 32 || D == 64 || D == 128, "packed direct staging");
  if constexpr (D == 32) return c ^ ((row >> 2) & 3);
  if constexpr (D == 64)
    return c ^ (((row >> 1) & 1) | (((row >> 2) & 1) << 1) | ((((row >> 1) ^ (row >> 3)) & 1) << 2));
  return c ^ ((row & 1) | (((row >> 1) & 1) << 1) | (((row ^ (row >> 2)) & 1) << 2) |
              ((((row >> 1) ^ (row >> 3)) & 1) << 3));
}

// Word 3 of a gfx9 buffer resource for raw (untyped, unswizzled) byte-offset
// loads: data format 32 so the hardware does not treat the buffer as invalid.
constexpr int kBufferWord3 = 0x00020000;

template <typename T>
__device__ __forceinline__ T ldg_nt(const T* p) { return __builtin_nontemporal_load(p); }
template <typename T>
__device__ __forceinline__ void stg_nt(T* p, T v) { __builtin_nontemporal_store(v, p); }

// Moves E float32 values per thread between global memory and LDS (or from
// one global buffer to another) for the one-thread-per-row float32 kernels:
// the loads of each batch of up to 8 are issued before the batch's stores, so
// a thread waits for memory once per batch rather than once per value (a load
// followed by a store that may alias the next load would otherwise be waited
// for one at a time). load(i) returns the thread's i-th value, store(i, x)
// writes it.
template <int E, typename Load, typename Store>
__device__ __forceinline__ void move_batched(Load&& load, Store&& store) {
  constexpr int kB = E < 8 ? E : 8;
  static_assert(E % kB == 0, "whole batches");
#pragma unroll
  for (int i0 = 0; i0 < E; i0 += kB) {
    float t[kB];
#pragma unroll
    for (int i = 0; i < kB; ++i) t[i] = load(i0 + i);
#pragma unroll
    for (int i = 0; i < kB; ++i) store(i0 + i, t[i]);
  }
}

// Dot product of two float32 rows of D values as four partial sums (by d mod
// 4): four independent chains of multiply-adds instead of one.
template <int D>
__device__ __forceinline__ float dot_f32(const float* x, const float* y) {
  float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int d = 0; d < D; ++d) s[d & 3] = fmaf(x[d], y[d], s[d & 3]);
  return (s[0] + s[1]) + (s[2] + s[3]);
}

}  // namespace psa

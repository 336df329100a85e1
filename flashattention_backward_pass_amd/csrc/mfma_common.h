// Building blocks shared by the gfx950 matrix-core kernels: the bf16 MFMA,
// the transposing LDS read and the row swizzle of bf16 tiles in LDS.
#pragma once

#include "fabwd_device.h"

namespace fabwd {

typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// D (32x32 fp32) += A (32x16 bf16) * B (16x32 bf16).
// Lane l: A row l%32 and B column l%32 hold k = 8(l/32) .. 8(l/32)+7 (any
// permutation of k works as long as A and B agree); accumulator register r
// holds row 8(r/4) + 4(l/32) + r%4 of column l%32.
__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group, lane
// x supplies the address of 4 consecutive bf16 (8 bytes); lane j receives
// element j%4 of the rows supplied by lanes j/4, j/4+4, j/4+8, j/4+12.  With
// lane x pointing at row r0 + x/4, columns c0 + 4(x%4) .. +3 of a row-major
// tile, lane j receives rows r0 .. r0+3 of column c0 + j.
__device__ __forceinline__ bf16x4_t lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p));
}

// Lanes l and l ^ 32 hold the two halves of one accumulator column: combine
// their values with one gfx950 v_permlane32_swap (no LDS round trip).  The
// instruction exchanges lanes 32-63 of its first operand with lanes 0-31 of
// its second; with v in both, lane l < 32 receives (v[l], v[l + 32]) and
// lane l >= 32 receives (v[l - 32], v[l]).  (The two results are copied to
// scalars before the bit cast: a bit cast of a vector element reads the
// vector's first element.)
__device__ __forceinline__ void lane_pair32(float v, float& a, float& b) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned r0 = r[0], r1 = r[1];
  a = __builtin_bit_cast(float, r0);
  b = __builtin_bit_cast(float, r1);
}
__device__ __forceinline__ float max_lane_pair32(float v) {
  float a, b;
  lane_pair32(v, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum_lane_pair32(float v) {
  float a, b;
  lane_pair32(v, a, b);
  return a + b;
}

__device__ __forceinline__ bf16x8_t cat8(bf16x4_t a, bf16x4_t b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x8_t load_bf16x8(const bf16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(p));
}

__device__ __forceinline__ bf16x8_t pack_bf16x8(const f32x16_t& v, int base) {
  bf16x8_t r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)v[base + e];
  return r;
}

// Bf16 tiles of D columns live in LDS with unpadded rows whose 16-byte chunks
// are XOR-swizzled by row.  Two access patterns must stay free of bank
// conflicts (64 banks of 4 bytes; a 16-byte read is served 16 lanes at a time,
// an 8-byte read 32 lanes at a time):
//  * row reads: 16 lanes read the same logical chunk of 16 consecutive rows,
//    so over 16 aligned rows the swizzle must be a permutation;
//  * transposing reads: 32 lanes read an aligned group of 4 chunks (64 bytes)
//    in each of 4 aligned consecutive rows, so those 4 rows must move the
//    group to 4 different positions.
// d = 128 (16 chunks per 256-byte row): swz = 4 (r % 4) + (r / 4) % 4.
// d = 64 (8 chunks per 128-byte row, two rows per bank window):
// swz = 4 ((r / 2) % 2) + (r / 4) % 4.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

// Element offset of (row, 16-byte chunk, element within chunk) in a swizzled tile.
template <int D>
__device__ __forceinline__ int swz_off(int row, int chunk, int sub) {
  return row * D + 8 * (chunk ^ swz<D>(row)) + sub;
}

}  // namespace fabwd

namespace fabwd {

// Epilogue staging.  A wave's 32 x (32 NT) fp32 accumulator block (acc[n],
// register r: row row0 + 8(r/4) + 4(lane/32) + r%4, column 32n + lane%32) is
// scaled by `mul`, converted to T and written into a row-major LDS tile of
// COLS elements per row; stage_copy_rows then moves whole rows to global
// memory with 16-byte accesses (a 2-byte store per lane and element would
// touch 64 scattered bytes per instruction).
template <typename T, int NT, int COLS>
__device__ __forceinline__ void stage_acc(T* tile, int row0, const f32x16_t* acc, float mul, int lane) {
  const int l32 = lane & 31, g = lane >> 5;
#pragma unroll
  for (int n = 0; n < NT; ++n) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = row0 + 8 * (r >> 2) + 4 * g + (r & 3);
      const float v = acc[n][r] * mul;
      if constexpr (sizeof(T) == 2) {
        reinterpret_cast<uint16_t*>(tile)[row * COLS + 32 * n + l32] = __builtin_bit_cast(uint16_t, (__bf16)v);
      } else {
        reinterpret_cast<float*>(tile)[row * COLS + 32 * n + l32] = v;
      }
    }
  }
}

// Rows [0, rows) of a row-major LDS tile of COLS elements of T per row go to
// dst + row * COLS; rows at or past `valid` are skipped.  All NTHREADS
// threads of the workgroup take part.
template <typename T, int COLS, int NTHREADS>
__device__ __forceinline__ void stage_copy_rows(T* __restrict__ dst, const T* tile, int rows, int valid, int tid) {
  constexpr int kPerChunk = 16 / sizeof(T);
  constexpr int kChunks = COLS / kPerChunk;  // 16-byte chunks per row
  for (int i = tid; i < rows * kChunks; i += NTHREADS) {
    const int row = i / kChunks, c = i % kChunks;
    if (row < valid)
      *reinterpret_cast<u32x4_t*>(dst + int64_t(row) * COLS + c * kPerChunk) =
          *reinterpret_cast<const u32x4_t*>(tile + row * COLS + c * kPerChunk);
  }
}

}  // namespace fabwd

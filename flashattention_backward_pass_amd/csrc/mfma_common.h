// Building blocks shared by the gfx950 matrix-core kernels: the bf16 MFMA,
// the transposing LDS read, the row swizzle of bf16 tiles in LDS and the
// asynchronous global -> LDS copies.
#pragma once

#include "fabwd_device.h"

namespace fabwd {

typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
typedef __attribute__((address_space(1))) void global_void_t;
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

// Asynchronous copy global -> LDS (global_load_lds): the 64 lanes of the wave
// fill 64 * bytes of LDS starting at the wave-uniform `lds_base`, lane L at
// lds_base + bytes * L, each lane reading its own global address.  Completion
// is tracked by vmcnt.
__device__ __forceinline__ void dma16(const void* gsrc, void* lds_base) {
  __builtin_amdgcn_global_load_lds((global_void_t*)(gsrc), (lds_void_t*)(lds_base), 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* gsrc, void* lds_base) {
  __builtin_amdgcn_global_load_lds((global_void_t*)(gsrc), (lds_void_t*)(lds_base), 4, 0, 0);
}

// Copies `rows` rows (multiple of 1024 / (2 D)) of a row-major bf16 matrix into
// a swizzled LDS tile with the 4 waves of a 256-thread workgroup.  Source rows
// at or past `n_valid` read row n_valid - 1 instead (always in bounds).
template <int D, int ROWS>
__device__ __forceinline__ void dma_tile(const bf16_t* src_row0, int n_valid, uint16_t* tile, int lane, int w) {
  constexpr int kRowsPerSlab = 1024 / (2 * D);
  constexpr int kSlabs = ROWS / kRowsPerSlab;
  static_assert(kSlabs % 4 == 0, "tile must split evenly over 4 waves");
#pragma unroll
  for (int s = 0; s < kSlabs / 4; ++s) {
    const int I = s * 4 + w;
    const int row = I * kRowsPerSlab + lane / (D / 8);
    const int chunk = (lane % (D / 8)) ^ swz<D>(row);
    dma16(src_row0 + int64_t(min(row, n_valid - 1)) * D + 8 * chunk, tile + I * 512);
  }
}

}  // namespace fabwd

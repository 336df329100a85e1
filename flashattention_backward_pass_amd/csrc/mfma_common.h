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

// The handoff of a split work unit's output tile between its two halves.
// The partial goes through memory with agent-coherent (sc1) 16-byte buffer
// accesses, the cache policy the memory model gives relaxed agent-scope
// atomics: no L2 write-back or invalidation is needed (an acquire/release
// pair would flush and invalidate the whole L2 of both XCDs for every
// handoff, which measured far slower).  The order is kept by waits: the
// first half's stores complete (vmcnt 0, then a barrier) before its counter
// update is issued, and the second half issues its loads only after reading
// the final count.
constexpr int kAgentCoherent = 16;  // buffer-access aux bits: sc1

// Rows [0, rows) of a row-major fp32 LDS tile (COLS per row) to dst + row *
// COLS with agent-coherent 16-byte stores; rows at or past `valid` skipped.
template <int COLS, int NTHREADS>
__device__ __forceinline__ void stage_store_rows_coherent(float* dst, const float* tile, int rows, int valid,
                                                          int tid) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(dst, 0, rows * COLS * 4, 0x00020000);
  constexpr int kChunks = COLS / 4;
  for (int i = tid; i < rows * kChunks; i += NTHREADS) {
    const int row = i / kChunks, c = i % kChunks;
    if (row < valid) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(tile + row * COLS + 4 * c);
      __builtin_amdgcn_raw_buffer_store_b128(v, r, (row * COLS + 4 * c) * 4, 0, kAgentCoherent);
    }
  }
}

// Rows [0, rows) of the fp32 LDS tile plus the same rows of `other` (read
// with agent-coherent loads; row-major, COLS per row), times mul, rounded to
// bf16 (RNE) and stored to dst + row * COLS with 16-byte stores; rows at or
// past `valid` are skipped.  The sum is tile + other in fp32, the same value
// as other + tile.
template <int COLS, int NTHREADS>
__device__ __forceinline__ void stage_add_rows(bf16_t* __restrict__ dst, const float* tile, const float* other,
                                               int rows, int valid, float mul, int tid) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(other), 0, rows * COLS * 4, 0x00020000);
  constexpr int kChunks = COLS / 8;  // 8 elements: one 16-byte bf16 store
  for (int i = tid; i < rows * kChunks; i += NTHREADS) {
    const int row = i / kChunks, c = i % kChunks;
    if (row < valid) {
      const f32x4_t a0 = *reinterpret_cast<const f32x4_t*>(tile + row * COLS + 8 * c);
      const f32x4_t a1 = *reinterpret_cast<const f32x4_t*>(tile + row * COLS + 8 * c + 4);
      const f32x4_t b0 = __builtin_bit_cast(
          f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (row * COLS + 8 * c) * 4, 0, kAgentCoherent));
      const f32x4_t b1 = __builtin_bit_cast(
          f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (row * COLS + 8 * c + 4) * 4, 0, kAgentCoherent));
      u32x4_t o;
      o[0] = pack_bf16x2(mul * (a0[0] + b0[0]), mul * (a0[1] + b0[1]));
      o[1] = pack_bf16x2(mul * (a0[2] + b0[2]), mul * (a0[3] + b0[3]));
      o[2] = pack_bf16x2(mul * (a1[0] + b1[0]), mul * (a1[1] + b1[1]));
      o[3] = pack_bf16x2(mul * (a1[2] + b1[2]), mul * (a1[3] + b1[3]));
      *reinterpret_cast<u32x4_t*>(dst + int64_t(row) * COLS + 8 * c) = o;
    }
  }
}

// A counter (zero before the launch) counts the halves' arrivals: the first
// to arrive writes its fp32 partial (stage_store_rows_coherent), then
// split_publish raises the counter to 3 once the other has arrived too
// (2 + 1), or to 2 before (1 + 1, and the other's arrival makes it 3); the
// second waits in split_wait for 3, adds the partial to its own
// (stage_add_rows) and writes the result.  Nobody waits for a workgroup that
// has not yet arrived, so the handoff cannot deadlock whatever the order of
// dispatch.  The bounded wait is a safety net only (its limit, about a
// second, is far beyond the partial write it waits for).
__device__ __forceinline__ bool split_arrive_first(unsigned* counter, unsigned* lds_word, int tid) {
  if (tid == 0) *lds_word = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  return *lds_word == 0u;
}
__device__ __forceinline__ void split_publish(unsigned* counter, int tid) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();  // every thread's partial stores have completed
  if (tid == 0) __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void split_wait(unsigned* counter, int tid) {
  if (tid == 0) {
    for (int it = 0; it < (1 << 22); ++it) {
      if (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 3u) break;
      __builtin_amdgcn_s_sleep(8);
    }
    // Zero again for the next launch (the preprocess zeroes it too).
    __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

}  // namespace fabwd

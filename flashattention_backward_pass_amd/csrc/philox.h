// Dropout mask replay on the device: the Philox4x32-10 counter-based
// generator and the keep test built on it.
//
// "解析 FlashAttention（3）：FlashAttention-v1 反向传播", section 3.3 and the
// dropout lines of Algorithm 4: the backward pass regenerates, tile by tile,
// the mask Z the forward pass drew, from the saved generator state, instead
// of storing it.  Z is 1/(1-p) where an element is kept and 0 elsewhere.
//
// Generator: Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel
// Random Numbers: As Easy as 1, 2, 3", SC'11, section 3).  A round multiplies
// counter words 0 and 2 by two fixed odd constants, keeps both halves of each
// 64-bit product, xors the high halves with words 3 / 1 and the round key,
// and permutes; the key advances by two Weyl constants between rounds.
//
// Element (query head bh, query q, key k): the call with counter
// (k >> 1, q >> 2, bh, offset) and key (seed_lo, seed_hi) yields words
// x0..x3; the element's 16-bit value is half (k & 1) of word x[q & 3], and the
// element is kept iff that value is below keep_t.  One call thus covers 4
// query rows x 2 keys.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fabwd {

// Generator state and keep threshold, passed to kernels by value.
struct Dropout {
  int enabled;       // 0: no dropout (every other field unused)
  uint32_t keep_t;   // kept iff the 16-bit value < keep_t (65536 keeps all)
  uint32_t seed_lo;  // key word 0
  uint32_t seed_hi;  // key word 1
  uint32_t offset;   // counter word 3
  float scale;       // 1 / (1 - p), applied to kept elements
};

constexpr uint32_t kPhiloxMulA = 0xD2511F53u;  // multiplies counter word 0
constexpr uint32_t kPhiloxMulB = 0xCD9E8D57u;  // multiplies counter word 2
constexpr uint32_t kPhiloxWeylA = 0x9E3779B9u;  // key word 0 increment
constexpr uint32_t kPhiloxWeylB = 0xBB67AE85u;  // key word 1 increment

// A Philox4x32 evaluation that can be advanced a few rounds at a time, so a
// kernel can spread the 10 rounds over the gaps between matrix instructions.
struct PhiloxState {
  uint32_t x0, x1, x2, x3;  // counter, then output
  uint32_t k0, k1;          // current round key

  __device__ __forceinline__ void init(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, const Dropout& d) {
    x0 = c0;
    x1 = c1;
    x2 = c2;
    x3 = c3;
    k0 = d.seed_lo;
    k1 = d.seed_hi;
  }
  __device__ __forceinline__ void round() {
    const uint64_t pa = uint64_t(kPhiloxMulA) * x0;
    const uint64_t pb = uint64_t(kPhiloxMulB) * x2;
    const uint32_t y0 = uint32_t(pb >> 32) ^ x1 ^ k0;
    const uint32_t y2 = uint32_t(pa >> 32) ^ x3 ^ k1;
    x0 = y0;
    x1 = uint32_t(pb);
    x2 = y2;
    x3 = uint32_t(pa);
    k0 += kPhiloxWeylA;
    k1 += kPhiloxWeylB;
  }
  // Rounds [r0, r1) of the 10 (the key schedule only depends on how many ran).
  __device__ __forceinline__ void rounds(int r0, int r1) {
#pragma unroll
    for (int r = r0; r < r1; ++r) round();
  }
  __device__ __forceinline__ uint32_t word(int i) const {
    return i == 0 ? x0 : i == 1 ? x1 : i == 2 ? x2 : x3;
  }
};

// Keep test of one element (any layout; one full generator call).
__device__ __forceinline__ bool dropout_keep(const Dropout& d, uint32_t bh, uint32_t q, uint32_t k) {
  PhiloxState s;
  s.init(k >> 1, q >> 2, bh, d.offset, d);
  s.rounds(0, 10);
  const uint32_t w = s.word(int(q & 3));
  const uint32_t u = (w >> (16 * (k & 1))) & 0xFFFFu;
  return u < d.keep_t;
}

// Packed 16-bit values of one 32x32 tile of a 32x32x16 matrix-instruction
// accumulator (register r of lane l: row 8(r/4) + 4(l/32) + r%4, column
// l%32).  Word w holds the values of registers 2w (low half) and 2w+1 (high
// half).
struct DropBits {
  uint32_t w[8];
  __device__ __forceinline__ bool keep(int r, uint32_t keep_t) const {
    return ((w[r >> 1] >> (16 * (r & 1))) & 0xFFFFu) < keep_t;
  }
};

// DPP lane swaps inside groups of 4 lanes (quad_perm [1,0,3,2] and [2,3,0,1]).
__device__ __forceinline__ uint32_t swap_lane1(uint32_t v) {
  return uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t swap_lane2(uint32_t v) {
  return uint32_t(__builtin_amdgcn_mov_dpp(int(v), 0x4E, 0xF, 0xF, false));
}

// Layout "key per lane": accumulator rows are queries q_row0 + row, the lane's
// column is key `key` (lanes l and l^1 hold keys 2c and 2c+1).  Each 4-row run
// of a lane (registers 4m .. 4m+3, rows 8m + 4(l/32) + 0..3) is one half of
// one generator call, shared with lane l^1.  The lane pair evaluates the four
// calls of its runs two each (lane parity e takes runs m = e and m = 2 + e),
// then swaps the halves the other lane needs.
struct DropKeyLane {
  PhiloxState c[2];
  __device__ __forceinline__ void init(const Dropout& d, uint32_t bh, int q_row0, int key, int lane) {
    const int e = lane & 1, g = (lane >> 5) & 1;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int q = q_row0 + 8 * (2 * j + e) + 4 * g;
      c[j].init(uint32_t(key) >> 1, uint32_t(q) >> 2, bh, d.offset, d);
    }
  }
  __device__ __forceinline__ void rounds(int r0, int r1) {
#pragma unroll
    for (int r = r0; r < r1; ++r) {
      c[0].round();
      c[1].round();
    }
  }
  // After all 10 rounds: the packed values of this lane's 16 registers.
  __device__ __forceinline__ DropBits finish(int lane) const {
    const bool odd = lane & 1;
    DropBits b;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const PhiloxState& s = c[j];
      // Halves of words r = 0..3 for keys 2c (low) and 2c+1 (high).
      const uint32_t lo01 = (s.x0 & 0xFFFFu) | (s.x1 << 16), hi01 = (s.x0 >> 16) | (s.x1 & 0xFFFF0000u);
      const uint32_t lo23 = (s.x2 & 0xFFFFu) | (s.x3 << 16), hi23 = (s.x2 >> 16) | (s.x3 & 0xFFFF0000u);
      const uint32_t own01 = odd ? hi01 : lo01, own23 = odd ? hi23 : lo23;
      const uint32_t got01 = swap_lane1(odd ? lo01 : hi01), got23 = swap_lane1(odd ? lo23 : hi23);
      // Run 2j + parity is this lane's own call, run 2j + 1 - parity the partner's.
      b.w[2 * (2 * j)] = odd ? got01 : own01;
      b.w[2 * (2 * j) + 1] = odd ? got23 : own23;
      b.w[2 * (2 * j + 1)] = odd ? own01 : got01;
      b.w[2 * (2 * j + 1) + 1] = odd ? own23 : got23;
    }
    return b;
  }
};

// Layout "query per lane": accumulator rows are keys k_row0 + row, the lane's
// column is query `q` (lanes 4a .. 4a+3 hold queries 4c .. 4c+3).  A 4-key run
// (registers 4m .. 4m+3) needs word q&3 of two calls (key pairs 2m' and
// 2m'+1 of the run); the four lanes of a quad need the same eight calls, so
// lane j of the quad evaluates the two calls of run m = j and a 4x4 transpose
// of words across the quad (two DPP butterfly stages) hands each lane its word.
struct DropQueryLane {
  PhiloxState c[2];
  __device__ __forceinline__ void init(const Dropout& d, uint32_t bh, int k_row0, int q, int lane) {
    const int m = lane & 3, g = (lane >> 5) & 1;
    const int k = k_row0 + 8 * m + 4 * g;
#pragma unroll
    for (int j = 0; j < 2; ++j) c[j].init((uint32_t(k) >> 1) + uint32_t(j), uint32_t(q) >> 2, bh, d.offset, d);
  }
  __device__ __forceinline__ void rounds(int r0, int r1) {
#pragma unroll
    for (int r = r0; r < r1; ++r) {
      c[0].round();
      c[1].round();
    }
  }
  // 4x4 transpose of words across the quad: a[i] = word i of this lane's
  // call (run lane&3) becomes a[m] = word (lane&3) of run m's call.
  static __device__ __forceinline__ void quad_transpose(uint32_t (&a)[4], int lane) {
    const bool b0 = lane & 1, b1 = lane & 2;
    // Stage 1: swap 2x2 blocks across lanes l ^ 2.
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t r = swap_lane2(b1 ? a[i] : a[i + 2]);
      a[i] = b1 ? r : a[i];
      a[i + 2] = b1 ? a[i + 2] : r;
    }
    // Stage 2: swap elements across lanes l ^ 1.
#pragma unroll
    for (int i = 0; i < 4; i += 2) {
      const uint32_t r = swap_lane1(b0 ? a[i] : a[i + 1]);
      a[i] = b0 ? r : a[i];
      a[i + 1] = b0 ? a[i + 1] : r;
    }
  }
  __device__ __forceinline__ DropBits finish(int lane) const {
    DropBits out;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t a[4] = {c[j].x0, c[j].x1, c[j].x2, c[j].x3};
      quad_transpose(a, lane);
#pragma unroll
      for (int m = 0; m < 4; ++m) out.w[2 * m + j] = a[m];
    }
    return out;
  }
  // The same bits as init + rounds(0, 10) + finish, one call at a time: one
  // generator state live instead of two.
  static __device__ __forceinline__ DropBits sequential(const Dropout& d, uint32_t bh, int k_row0, int q, int lane) {
    const int m = lane & 3, g = (lane >> 5) & 1;
    const int k = k_row0 + 8 * m + 4 * g;
    DropBits out;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      PhiloxState s;
      s.init((uint32_t(k) >> 1) + uint32_t(j), uint32_t(q) >> 2, bh, d.offset, d);
      s.rounds(0, 10);
      uint32_t a[4] = {s.x0, s.x1, s.x2, s.x3};
      quad_transpose(a, lane);
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) out.w[2 * mm + j] = a[mm];
    }
    return out;
  }
};

}  // namespace fabwd

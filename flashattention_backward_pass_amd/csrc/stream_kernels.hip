// Bandwidth-bound kernels of the backward pass:
//   bwd_preprocess : D_i = sum_k dO_ik O_ik in fp32, and dQaccum <- 0 for the
//                    fp32 path (whose backward adds into dQaccum); for bf16,
//                    the handoff counters of split units in the combined
//                    launch (a few words of dQaccum) <- 0
//                    ("解析 FlashAttention（3）：FlashAttention-v1 反向传播", eq (6);
//                     Inference Cookbook "反向传播算法详解" section 2.1, dPsum
//                     computed before the backward kernel);
//   bwd_dq_convert : dQ = scale * dQaccum rounded to the output dtype
//                    (FlashAttention-v1 backward page, eq (7) carries the scale).
//
// Both stream each byte once with 16-byte accesses.  A row of d elements is
// covered by L = d*sizeof(T)/16 consecutive lanes; the row dot product is a
// fixed-order xor-shuffle tree, so D is bitwise reproducible.
#include "fabwd_device.h"
#include "fabwd_launch.h"

namespace fabwd {

namespace {

constexpr int kThreads = 256;

template <typename T>
__device__ __forceinline__ void load16(const T* p, float* out);

template <>
__device__ __forceinline__ void load16<float>(const float* p, float* out) {
  f32x4_t v = *reinterpret_cast<const f32x4_t*>(p);
  out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
}
template <>
__device__ __forceinline__ void load16<bf16_t>(const bf16_t* p, float* out) {
  u32x4_t v = *reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(v[i] << 16);
    out[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
}

// One lane handles 16 bytes of a row of O and dO, for kUnroll row groups at a
// time (all loads issued before any arithmetic, so more bytes are in flight).
// Grid-stride over row groups.
constexpr int kUnroll = 4;

template <typename T, int D, bool ZERO_ACC>
__global__ __launch_bounds__(kThreads) void preprocess_kernel(const T* __restrict__ O, const T* __restrict__ dO,
                                                              float* __restrict__ Dout,
                                                              float* __restrict__ dQacc, int64_t rows,
                                                              unsigned* __restrict__ zero_words, int n_zero) {
  for (int i = blockIdx.x * kThreads + threadIdx.x; i < n_zero; i += gridDim.x * kThreads) zero_words[i] = 0u;
  constexpr int kPerLane = 16 / sizeof(T);      // elements per 16-byte access
  constexpr int L = D / kPerLane;                // lanes per row
  constexpr int kRowsPerGroup = kThreads / L;    // rows covered by the block at once
  constexpr int kZeroPerLane = (D / 4) / L;      // float4 zero stores per lane
  static_assert(L >= 1 && L <= 64 && (L & (L - 1)) == 0, "row must map to a power-of-two lane group");
  const int lane_in_row = threadIdx.x % L;
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  for (int64_t row0 = int64_t(blockIdx.x) * kRowsPerGroup * kUnroll; row0 < rows;
       row0 += int64_t(gridDim.x) * kRowsPerGroup * kUnroll) {
    u32x4_t ob[kUnroll], gb[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t row = row0 + u * kRowsPerGroup + threadIdx.x / L;
      const int64_t off = min(row, rows - 1) * D + int64_t(lane_in_row) * kPerLane;
      // Non-temporal: O and dO are read once here (9.95 against 11.3 us back to
      // back on the long causal workload, 85 % of the 8 TB/s HBM peak).
      ob[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(O + off));
      gb[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(dO + off));
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t row = row0 + u * kRowsPerGroup + threadIdx.x / L;
      float o[kPerLane], g[kPerLane], acc = 0.f;
      load16<T>(reinterpret_cast<const T*>(&ob[u]), o);
      load16<T>(reinterpret_cast<const T*>(&gb[u]), g);
#pragma unroll
      for (int e = 0; e < kPerLane; ++e) acc = fmaf(o[e], g[e], acc);
      acc = wave_xor_sum(acc, L);
      if (row < rows) {
        if (lane_in_row == 0) Dout[row] = acc;
        if (ZERO_ACC) {
          f32x4_t* z = reinterpret_cast<f32x4_t*>(dQacc + row * D) + lane_in_row * kZeroPerLane;
#pragma unroll
          for (int e = 0; e < kZeroPerLane; ++e) z[e] = zero;
        }
      }
    }
  }
}

// dQ = scale * dQaccum.  Each lane converts 8 floats (bf16 output: one 16-byte
// store) or 4 floats (fp32 output).
template <typename T>
__global__ __launch_bounds__(kThreads) void dq_convert_kernel(const float* __restrict__ acc, T* __restrict__ dQ,
                                                              float scale, int64_t n);

template <>
__global__ __launch_bounds__(kThreads) void dq_convert_kernel<bf16_t>(const float* __restrict__ acc,
                                                                      bf16_t* __restrict__ dQ, float scale,
                                                                      int64_t n) {
  const int64_t groups = n / 8;
  for (int64_t gi = int64_t(blockIdx.x) * kThreads + threadIdx.x; gi < groups;
       gi += int64_t(gridDim.x) * kThreads) {
    const f32x4_t a = reinterpret_cast<const f32x4_t*>(acc)[2 * gi];
    const f32x4_t b = reinterpret_cast<const f32x4_t*>(acc)[2 * gi + 1];
    u32x4_t out;
    out[0] = pack_bf16x2(scale * a[0], scale * a[1]);
    out[1] = pack_bf16x2(scale * a[2], scale * a[3]);
    out[2] = pack_bf16x2(scale * b[0], scale * b[1]);
    out[3] = pack_bf16x2(scale * b[2], scale * b[3]);
    reinterpret_cast<u32x4_t*>(dQ)[gi] = out;
  }
}

template <>
__global__ __launch_bounds__(kThreads) void dq_convert_kernel<float>(const float* __restrict__ acc,
                                                                     float* __restrict__ dQ, float scale,
                                                                     int64_t n) {
  const int64_t groups = n / 4;
  for (int64_t gi = int64_t(blockIdx.x) * kThreads + threadIdx.x; gi < groups;
       gi += int64_t(gridDim.x) * kThreads) {
    f32x4_t a = reinterpret_cast<const f32x4_t*>(acc)[gi];
    a *= scale;
    reinterpret_cast<f32x4_t*>(dQ)[gi] = a;
  }
}

// Enough blocks to cover the work, capped so a grid-stride loop takes over
// for very large tensors (2048 blocks = 8 per CU on 256 CUs, 8 resident waves).
unsigned grid_for(int64_t work_items, int64_t per_block) {
  int64_t g = (work_items + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > 16384) g = 16384;
  return unsigned(g);
}

template <typename T, int D>
hipError_t preprocess_t(const Problem& p, const void* O, const void* dO, float* Dv, float* dQacc, hipStream_t s) {
  constexpr int L = D / (16 / sizeof(T));
  const int64_t rows = p.q_rows();
  constexpr bool kZero = sizeof(T) == 4;  // only the fp32 backward accumulates into dQaccum
  const FusedSplit sp = kZero ? FusedSplit{} : fused_split(p, true);
  unsigned* zero_words = sp.counters > 0 ? reinterpret_cast<unsigned*>(dQacc + sp.counter_off) : nullptr;
  hipLaunchKernelGGL((preprocess_kernel<T, D, kZero>), dim3(grid_for(rows, kThreads / L * kUnroll)), dim3(kThreads),
                     0, s,
                     static_cast<const T*>(O), static_cast<const T*>(dO), Dv, dQacc, rows, zero_words, sp.counters);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_preprocess(const Problem& p, const void* O, const void* dO, float* D, float* dQacc,
                                 hipStream_t s) {
  (void)hipGetLastError();
  if (p.dtype == 1) {
    return p.d == 64 ? preprocess_t<bf16_t, 64>(p, O, dO, D, dQacc, s)
                     : preprocess_t<bf16_t, 128>(p, O, dO, D, dQacc, s);
  }
  return p.d == 64 ? preprocess_t<float, 64>(p, O, dO, D, dQacc, s)
                   : preprocess_t<float, 128>(p, O, dO, D, dQacc, s);
}

hipError_t launch_bwd_dq_convert(const Problem& p, const float* dQacc, void* dQ, hipStream_t s) {
  (void)hipGetLastError();
  const int64_t n = p.q_elems();
  if (p.dtype == 1) {
    hipLaunchKernelGGL(dq_convert_kernel<bf16_t>, dim3(grid_for(n / 8, kThreads)), dim3(kThreads), 0, s, dQacc,
                       static_cast<bf16_t*>(dQ), p.scale, n);
  } else {
    hipLaunchKernelGGL(dq_convert_kernel<float>, dim3(grid_for(n / 4, kThreads)), dim3(kThreads), 0, s, dQacc,
                       static_cast<float*>(dQ), p.scale, n);
  }
  return hipGetLastError();
}

}  // namespace fabwd

// dQ-accumulation traffic probe (HIP, gfx950): replays the dQaccum updates
// that a key-block-outer backward would make on the long causal workload
// (B = 1, H = 8, N = 16384, d = 128; key blocks of 128, query tiles of 64 rows)
// without any matrix work, once as fp32 atomic adds (device scope) and once as
// plain stores of the same bytes.  Each (query tile, key block) pair with the
// tile inside the causal range writes 64 x 128 floats; 4 waves per workgroup
// each cover a 32-column slice, each lane 32 floats.  Prints one JSON line per
// mode: milliseconds per launch and the update rate.
//
// The point of comparison is the Inference Cookbook page "反向传播算法详解",
// section 6.2 (dQ accumulated with atomics into a global fp32 buffer).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

namespace {

constexpr int kH = 8, kN = 16384, kD = 128, kBC = 128, kBR = 64;

template <bool ATOMIC>
__global__ __launch_bounds__(256, 1) void dq_updates(float* __restrict__ acc) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int h = blockIdx.x % kH, j = blockIdx.x / kH;  // head fastest: one head per XCD
  const float v = 1.0f + float(lane) * 0.001f;
  const int i_lo = (j * kBC) / kBR, n_tiles = kN / kBR;
  for (int i = n_tiles - 1; i >= i_lo; --i) {
    float* tile = acc + (int64_t(h) * kN + int64_t(i) * kBR) * kD;
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      // accumulator layout of a 32x32 matrix instruction: row 8(r/4) + 4(lane/32) + r%4 of
      // the slice's two 32-row halves, column lane % 32
      const int row = 32 * (r >> 4) + 8 * ((r & 15) >> 2) + 4 * (lane >> 5) + (r & 3);
      float* p = tile + row * kD + 32 * w + (lane & 31);
      if (ATOMIC)
        __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        *p = v;
    }
  }
}

void check(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    std::exit(1);
  }
}

template <bool ATOMIC>
void run(float* acc, const char* name) {
  const dim3 grid(kH * (kN / kBC)), block(256);
  hipEvent_t a, b;
  check(hipEventCreate(&a), "hipEventCreate");
  check(hipEventCreate(&b), "hipEventCreate");
  for (int it = 0; it < 2; ++it) hipLaunchKernelGGL(dq_updates<ATOMIC>, grid, block, 0, nullptr, acc);
  check(hipEventRecord(a, nullptr), "hipEventRecord");
  const int iters = 5;
  for (int it = 0; it < iters; ++it) hipLaunchKernelGGL(dq_updates<ATOMIC>, grid, block, 0, nullptr, acc);
  check(hipEventRecord(b, nullptr), "hipEventRecord");
  check(hipEventSynchronize(b), "hipEventSynchronize");
  check(hipGetLastError(), "launch");
  float ms = 0.f;
  check(hipEventElapsedTime(&ms, a, b), "hipEventElapsedTime");
  ms /= iters;
  // (query tile, key block) pairs per head: sum over key blocks j of (N/BR - 2j)
  double pairs = 0;
  for (int j = 0; j < kN / kBC; ++j) pairs += kN / kBR - (j * kBC) / kBR;
  const double bytes = pairs * kH * kBR * kD * 4.0;
  std::printf("{\"mode\": \"%s\", \"ms_per_launch\": %.4f, \"update_bytes\": %.0f, \"GBs\": %.1f}\n", name, ms, bytes,
              bytes / (ms * 1e-3) / 1e9);
  check(hipEventDestroy(a), "hipEventDestroy");
  check(hipEventDestroy(b), "hipEventDestroy");
}

}  // namespace

int main() {
  float* acc = nullptr;
  const size_t bytes = size_t(kH) * kN * kD * sizeof(float);
  check(hipMalloc(&acc, bytes), "hipMalloc");
  check(hipMemset(acc, 0, bytes), "hipMemset");
  run<true>(acc, "fp32_atomic_add_agent_scope");
  run<false>(acc, "plain_store");
  check(hipFree(acc), "hipFree");
  return 0;
}

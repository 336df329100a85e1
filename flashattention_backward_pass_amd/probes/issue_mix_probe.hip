// Issue-mix probe (HIP, gfx950): how much VALU and LDS work one wave can
// issue beside its matrix instructions.  Per slot: two independent
// v_mfma_f32_32x32x16_bf16 (rotating over four accumulators), R transposing
// LDS reads (ds_read_b64_tr_b16, issued one slot ahead of their use), V
// full-rate fp32 FMAs and E v_exp_f32 on registers the MFMAs do not touch.
// 256 workgroups of four waves, one per SIMD (or only wave 0 of each
// workgroup); each wave times its loop with s_memtime.  Prints one JSON line
// per mix: cycles per slot.  The mixes bracket the slots of the dK/dV work
// unit (bwd_dkdv_block.h), about 4 reads, 4 VALU and 1 exp per MFMA pair.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <vector>
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) bf16x4_t lds4;
__device__ inline f32x16_t mf(bf16x8_t a, bf16x8_t b, f32x16_t c) { return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0); }

template <int R, int V, int E>
__global__ __launch_bounds__(256, 1) void k(float* out, long long* cyc, int iters, int nw) {
  __shared__ __attribute__((aligned(1024))) uint16_t t[32768];
  for (int i = threadIdx.x; i < 32768; i += 256) t[i] = (uint16_t)(i * 7);
  __syncthreads();
  const int w = threadIdx.x / 64, lane = threadIdx.x & 63;
  if (w >= nw) return;
  bf16x8_t a;
  for (int e = 0; e < 8; ++e) a[e] = (__bf16)(0.001f * (lane + e));
  f32x16_t acc[8];
  for (int c = 0; c < 8; ++c) acc[c] = f32x16_t{};
  float vv[16];
  for (int e = 0; e < 16; ++e) vv[e] = 0.5f + 0.01f * (lane + e);
  auto rd = [&](int i, int j) -> bf16x8_t {
    const int o2 = (w * 4096 + lane * 4 + ((i * 4 + j) & 7) * 512) & 32767;
    bf16x4_t p = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds4*)(&t[o2]));
    bf16x4_t q = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds4*)(&t[(o2 + 256) & 32767]));
    return __builtin_shufflevector(p, q, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  bf16x8_t op[2][4];
#pragma unroll
  for (int j = 0; j < R / 2; ++j) op[0][j] = rd(0, j);
  long long t0 = __builtin_amdgcn_s_memtime();
  for (int i = 0; i < iters; i += 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int j = 0; j < R / 2; ++j) op[1 - h][j] = rd(i + h + 1, j);
      acc[(2 * h) & 7] = mf(a, R ? op[h][0] : a, acc[(2 * h) & 7]);
      acc[(2 * h + 1) & 7] = mf(a, R > 2 ? op[h][1] : a, acc[(2 * h + 1) & 7]);
#pragma unroll
      for (int e = 0; e < V; ++e) vv[e & 15] = vv[e & 15] * 0.999f + 0.001f;
#pragma unroll
      for (int e = 0; e < E; ++e) vv[(e + 8) & 15] = __builtin_amdgcn_exp2f(vv[(e + 8) & 15] * -0.01f);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  long long t1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
  for (int c = 0; c < 8; ++c) s += acc[c][0];
  for (int e = 0; e < 16; ++e) s += vv[e];
  out[blockIdx.x * 256 + threadIdx.x] = s;
  if (lane == 0) cyc[blockIdx.x * 4 + w] = t1 - t0;
}
template <int R, int V, int E>
void run(float* out, long long* cyc, int nw) {
  const int blocks = 256, iters = 2048;
  hipLaunchKernelGGL((k<R, V, E>), dim3(blocks), dim3(256), 0, 0, out, cyc, iters, nw);
  (void)hipDeviceSynchronize();
  hipLaunchKernelGGL((k<R, V, E>), dim3(blocks), dim3(256), 0, 0, out, cyc, iters, nw);
  std::vector<long long> h(blocks * 4);
  (void)hipMemcpy(h.data(), cyc, h.size() * 8, hipMemcpyDeviceToHost);
  double s = 0; int n = 0;
  for (int b = 0; b < blocks; ++b) for (int w = 0; w < nw; ++w) { s += h[b * 4 + w]; ++n; }
  printf("{\"reads\": %d, \"valu\": %d, \"exp\": %d, \"waves\": %d, \"cycles_per_slot\": %.1f}\n", R, V, E, nw, s / n / iters);
}
int main() {
  float* out; long long* cyc;
  if (hipMalloc(&out, 256 * 256 * 4) != hipSuccess || hipMalloc(&cyc, 256 * 4 * 8) != hipSuccess) return 1;
  run<0, 0, 0>(out, cyc, 4); run<4, 0, 0>(out, cyc, 4);
  run<0, 4, 0>(out, cyc, 4); run<0, 8, 0>(out, cyc, 4); run<0, 12, 0>(out, cyc, 4);
  run<0, 0, 2>(out, cyc, 4); run<0, 0, 4>(out, cyc, 4);
  run<0, 4, 2>(out, cyc, 4); run<0, 6, 2>(out, cyc, 4);
  run<4, 4, 2>(out, cyc, 4); run<4, 6, 2>(out, cyc, 4); run<4, 8, 2>(out, cyc, 4);
  run<4, 6, 2>(out, cyc, 1);
  hipError_t e = hipDeviceSynchronize();
  printf("{\"status\": \"%s\"}\n", hipGetErrorString(e));
  return e == hipSuccess ? 0 : 1;
}

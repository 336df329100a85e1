// bf16 dK / dV kernel: one workgroup per work unit of dkdv_block
// (bwd_dkdv_block.h), plus the fixed-order sum of head-split partials.
#include "bwd_dkdv_block.h"

namespace fabwd {

namespace {

using dkdv::BC;
using dkdv::kThreads;

template <int D, bool SOFTCAP, bool DROPOUT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(
    dkdv::kWavesPerSimd<D, SOFTCAP, DROPOUT>, dkdv::kWavesPerSimd<D, SOFTCAP, DROPOUT>))) void bwd_dkdv_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const bf16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    bf16_t* __restrict__ dK, bf16_t* __restrict__ dV, int H, int H_kv, int N, int BH, float scale,
    float softcap, int wl, int wr, int n_split, float* __restrict__ part, Dropout drop) {
  dkdv::dkdv_block<D, SOFTCAP, DROPOUT>(Q, K, V, dO, LSE, Dv, dK, dV, H, H_kv, N, BH, scale, softcap, wl, wr, n_split,
                                        part, drop, blockIdx.x);
}

// Sums the head-split partials in a fixed order and rounds: dK = -tau * sum,
// dV = sum (8 elements per thread; `elems` = B*H_kv*N*D is a multiple of 8).
__global__ __launch_bounds__(256) void dkdv_split_sum_kernel(const float* __restrict__ part, int n_split,
                                                             int64_t elems, bf16_t* __restrict__ dK,
                                                             bf16_t* __restrict__ dV, float scale) {
  const int64_t i = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 8;
  if (i >= elems) return;
  dkdv::split_sum8(part, n_split, elems, i, dK, dV, scale);
}

}  // namespace

int dkdv_split_count(const Problem& p, bool have_scratch) {
  const int64_t units = int64_t(p.B) * p.H_kv * ((p.N + BC - 1) / BC);
  return (have_scratch && p.H / p.H_kv >= 4 && units < 1024) ? 2 : 1;
}

namespace {

template <int D, bool SOFTCAP, bool DROPOUT>
hipError_t dkdv_t(const Problem& p, const void* Q, const void* K, const void* V, const void* dO, const float* LSE,
                  const float* Dv, void* dK, void* dV, float* scratch, bool sum_later, hipStream_t s) {
  const int BH = p.B * p.H_kv;
  const int n_kblk = (p.N + BC - 1) / BC;
  // Grouped-query heads with few work units: the heaviest (first causal)
  // key blocks would run G times every query tile in one workgroup.  Share
  // the heads out over two workgroups; their fp32 partials fit in `scratch`
  // (B*H*N*d floats) because 2 splits x (dK, dV) x B*H_kv*N*d <= B*H*N*d
  // when G >= 4.
  const int n_split = dkdv_split_count(p, scratch != nullptr);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, SOFTCAP, DROPOUT>), dim3(unsigned(BH) * unsigned(n_kblk) * unsigned(n_split)),
                     dim3(kThreads), 0, s, static_cast<const bf16_t*>(Q), static_cast<const bf16_t*>(K),
                     static_cast<const bf16_t*>(V), static_cast<const bf16_t*>(dO), LSE, Dv,
                     static_cast<bf16_t*>(dK), static_cast<bf16_t*>(dV), p.H, p.H_kv, p.N, BH, p.scale, p.softcap,
                     p.wl, p.wr, n_split, n_split > 1 ? scratch : nullptr, p.drop());
  if (n_split == 1 || sum_later) return hipGetLastError();
  const int64_t elems = int64_t(BH) * p.N * D;
  const unsigned blocks = unsigned((elems / 8 + 255) / 256);
  hipLaunchKernelGGL(dkdv_split_sum_kernel, dim3(blocks), dim3(256), 0, s, static_cast<const float*>(scratch),
                     n_split, elems, static_cast<bf16_t*>(dK), static_cast<bf16_t*>(dV), p.scale);
  return hipGetLastError();
}

template <int D>
hipError_t dkdv_d(const Problem& p, const void* Q, const void* K, const void* V, const void* dO, const float* LSE,
                  const float* Dv, void* dK, void* dV, float* scratch, bool sum_later, hipStream_t s) {
  if (p.dropout)
    return p.softcap > 0.f ? dkdv_t<D, true, true>(p, Q, K, V, dO, LSE, Dv, dK, dV, scratch, sum_later, s)
                           : dkdv_t<D, false, true>(p, Q, K, V, dO, LSE, Dv, dK, dV, scratch, sum_later, s);
  return p.softcap > 0.f ? dkdv_t<D, true, false>(p, Q, K, V, dO, LSE, Dv, dK, dV, scratch, sum_later, s)
                         : dkdv_t<D, false, false>(p, Q, K, V, dO, LSE, Dv, dK, dV, scratch, sum_later, s);
}

}  // namespace

hipError_t launch_bwd_dkdv_mfma(const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                                const float* LSE, const float* Dv, void* dK, void* dV, float* scratch,
                                bool sum_later, hipStream_t s) {
  return p.d == 64 ? dkdv_d<64>(p, Q, K, V, dO, LSE, Dv, dK, dV, scratch, sum_later, s)
                   : dkdv_d<128>(p, Q, K, V, dO, LSE, Dv, dK, dV, scratch, sum_later, s);
}

}  // namespace fabwd

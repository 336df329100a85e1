// bf16 dQ kernel: one workgroup per work unit of dq_block (bwd_dq_block.h).
#include "bwd_dq_block.h"

namespace fabwd {

namespace {

using dq::BQ;
using dq::kThreads;

template <int D, bool SOFTCAP, bool DROPOUT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_dq_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const bf16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    float* __restrict__ dQacc, bf16_t* __restrict__ dQout, int H, int H_kv, int N, int BHq, float scale,
    float softcap, int wl, int wr, Dropout drop) {
  dq::dq_block<D, SOFTCAP, DROPOUT>(Q, K, V, dO, LSE, Dv, dQacc, dQout, H, H_kv, N, BHq, scale, softcap, wl, wr, drop,
                                    blockIdx.x);
}

template <int D, bool SOFTCAP, bool DROPOUT>
hipError_t dq_t(const Problem& p, const void* Q, const void* K, const void* V, const void* dO, const float* LSE,
                const float* Dv, float* dQacc, void* dQout, hipStream_t s) {
  const int BHq = p.B * p.H;
  const int n_qblk = (p.N + BQ - 1) / BQ;
  hipLaunchKernelGGL((bwd_dq_kernel<D, SOFTCAP, DROPOUT>), dim3(unsigned(BHq) * unsigned(n_qblk)), dim3(kThreads), 0, s,
                     static_cast<const bf16_t*>(Q), static_cast<const bf16_t*>(K), static_cast<const bf16_t*>(V),
                     static_cast<const bf16_t*>(dO), LSE, Dv, dQacc, static_cast<bf16_t*>(dQout), p.H, p.H_kv, p.N, BHq, p.scale, p.softcap,
                     p.wl, p.wr, p.drop());
  return hipGetLastError();
}

template <int D>
hipError_t dq_d(const Problem& p, const void* Q, const void* K, const void* V, const void* dO, const float* LSE,
                const float* Dv, float* dQacc, void* dQout, hipStream_t s) {
  if (p.dropout)
    return p.softcap > 0.f ? dq_t<D, true, true>(p, Q, K, V, dO, LSE, Dv, dQacc, dQout, s)
                           : dq_t<D, false, true>(p, Q, K, V, dO, LSE, Dv, dQacc, dQout, s);
  return p.softcap > 0.f ? dq_t<D, true, false>(p, Q, K, V, dO, LSE, Dv, dQacc, dQout, s)
                         : dq_t<D, false, false>(p, Q, K, V, dO, LSE, Dv, dQacc, dQout, s);
}

}  // namespace

hipError_t launch_bwd_dq_mfma(const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                              const float* LSE, const float* Dv, float* dQacc, void* dQout, hipStream_t s) {
  return p.d == 64 ? dq_d<64>(p, Q, K, V, dO, LSE, Dv, dQacc, dQout, s)
                   : dq_d<128>(p, Q, K, V, dO, LSE, Dv, dQacc, dQout, s);
}

}  // namespace fabwd

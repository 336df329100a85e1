// bf16 dQ kernel: one workgroup per work unit of dq_block (bwd_dq_block.h).
// Given dQ and head-split dK/dV partials (sum_elems > 0), its workgroups
// also add those partials, each a contiguous share, before their own unit:
// the dK/dV kernel has finished (same stream) and the dQ kernel, writing bf16
// dQ, leaves the partials in dQaccum alone, so the separate sum launch goes.
#include "bwd_dkdv_block.h"
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
    float softcap, int wl, int wr, Dropout drop, int n_split, int64_t sum_elems, bf16_t* __restrict__ dK,
    bf16_t* __restrict__ dV) {
  if (sum_elems > 0) {
    const int64_t groups = sum_elems / 8;
    const int64_t per = (groups + gridDim.x - 1) / gridDim.x;
    const int64_t g_end = min(groups, (int64_t(blockIdx.x) + 1) * per);
    for (int64_t gi = int64_t(blockIdx.x) * per + threadIdx.x; gi < g_end; gi += kThreads)
      dkdv::split_sum8(dQacc, n_split, sum_elems, gi * 8, dK, dV, scale);
  }
  dq::dq_block<D, SOFTCAP, DROPOUT>(Q, K, V, dO, LSE, Dv, dQacc, dQout, H, H_kv, N, BHq, scale, softcap, wl, wr, drop,
                                    blockIdx.x);
}

template <int D, bool SOFTCAP, bool DROPOUT>
hipError_t dq_t(const Problem& p, const void* Q, const void* K, const void* V, const void* dO, const float* LSE,
                const float* Dv, float* dQacc, void* dQout, void* dK, void* dV, hipStream_t s) {
  const int BHq = p.B * p.H;
  const int n_qblk = (p.N + BQ - 1) / BQ;
  // Head-split partials to add (only given dQ, see above).
  const int n_split = dK ? dkdv_split_count(p, true) : 1;
  const int64_t sum_elems = n_split > 1 ? int64_t(p.B) * p.H_kv * p.N * D : 0;
  hipLaunchKernelGGL((bwd_dq_kernel<D, SOFTCAP, DROPOUT>), dim3(unsigned(BHq) * unsigned(n_qblk)), dim3(kThreads), 0, s,
                     static_cast<const bf16_t*>(Q), static_cast<const bf16_t*>(K), static_cast<const bf16_t*>(V),
                     static_cast<const bf16_t*>(dO), LSE, Dv, dQacc, static_cast<bf16_t*>(dQout), p.H, p.H_kv, p.N,
                     BHq, p.scale, p.softcap, p.wl, p.wr, p.drop(), n_split, sum_elems, static_cast<bf16_t*>(dK),
                     static_cast<bf16_t*>(dV));
  return hipGetLastError();
}

template <int D>
hipError_t dq_d(const Problem& p, const void* Q, const void* K, const void* V, const void* dO, const float* LSE,
                const float* Dv, float* dQacc, void* dQout, void* dK, void* dV, hipStream_t s) {
  if (p.dropout)
    return p.softcap > 0.f ? dq_t<D, true, true>(p, Q, K, V, dO, LSE, Dv, dQacc, dQout, dK, dV, s)
                           : dq_t<D, false, true>(p, Q, K, V, dO, LSE, Dv, dQacc, dQout, dK, dV, s);
  return p.softcap > 0.f ? dq_t<D, true, false>(p, Q, K, V, dO, LSE, Dv, dQacc, dQout, dK, dV, s)
                         : dq_t<D, false, false>(p, Q, K, V, dO, LSE, Dv, dQacc, dQout, dK, dV, s);
}

}  // namespace

hipError_t launch_bwd_dq_mfma(const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                              const float* LSE, const float* Dv, float* dQacc, void* dQout, void* dK, void* dV,
                              hipStream_t s) {
  return p.d == 64 ? dq_d<64>(p, Q, K, V, dO, LSE, Dv, dQacc, dQout, dK, dV, s)
                   : dq_d<128>(p, Q, K, V, dO, LSE, Dv, dQacc, dQout, dK, dV, s);
}

}  // namespace fabwd

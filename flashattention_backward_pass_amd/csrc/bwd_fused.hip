// The dK/dV and dQ work units of the bf16 backward in one launch.
//
// The two kernels are independent: both read Q, K, V, dO, LSE and D; the
// dK/dV units write dK and dV, the dQ units write dQaccum (as long as the
// dK/dV units do not borrow dQaccum for head-split partials, which the
// dispatch rules out).  A problem with few units, such as one head at full
// length (128 key blocks and 128 query blocks of N = 16384 for 256 compute
// units), leaves half the chip idle in each kernel when they run one after
// the other, and each kernel's time is set by its heaviest (first causal)
// unit.  Here the workgroups of one grid take either kind of unit, the
// heaviest of each kind first and the two kinds interleaved, so both run at
// once.  The grid runs at one wave per SIMD, as the dK/dV units need.
#include "bwd_dkdv_block.h"
#include "bwd_dq_block.h"

namespace fabwd {

namespace {

static_assert(dkdv::kThreads == dq::kThreads, "one workgroup size for both kinds of unit");
constexpr int kThreads = dkdv::kThreads;
// Grids of at most this many workgroups (four per compute unit) take the
// combined launch: measured faster up to 1024 (6-19 % at 1024 workgroups),
// slower at 2048 (5-10 %, where the dQ units lose their second wave per SIMD).
constexpr int64_t kFusedMaxBlocks = 1024;

template <int D, bool SOFTCAP, bool DROPOUT>
__global__ __launch_bounds__(kThreads, 1) void bwd_fused_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const bf16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    bf16_t* __restrict__ dK, bf16_t* __restrict__ dV, float* __restrict__ dQacc, bf16_t* __restrict__ dQout, int H,
    int H_kv, int N,
    int BH_kv, int BH_q, float scale, float softcap, int wl, int wr, Dropout drop, unsigned n_dkdv, unsigned n_dq) {
  // Blocks 0 .. 2m-1 alternate between the two kinds (m = the smaller
  // count); the rest belong to the larger kind.
  const unsigned m = min(n_dkdv, n_dq);
  const unsigned b = blockIdx.x;
  bool dq_unit;
  unsigned unit;
  if (b < 2 * m) {
    dq_unit = (b & 1u) != 0;
    unit = b >> 1;
  } else {
    dq_unit = n_dq > n_dkdv;
    unit = b - m;
  }
  if (dq_unit)
    dq::dq_block<D, SOFTCAP, DROPOUT>(Q, K, V, dO, LSE, Dv, dQacc, dQout, H, H_kv, N, BH_q, scale, softcap, wl, wr,
                                      drop, unit);
  else
    dkdv::dkdv_block<D, SOFTCAP, DROPOUT>(Q, K, V, dO, LSE, Dv, dK, dV, H, H_kv, N, BH_kv, scale, softcap, wl, wr,
                                          1, nullptr, drop, unit);
}

unsigned dkdv_units(const Problem& p) {
  return unsigned(p.B * p.H_kv) * unsigned((p.N + dkdv::BC - 1) / dkdv::BC);
}
unsigned dq_units(const Problem& p) { return unsigned(p.B * p.H) * unsigned((p.N + dq::BQ - 1) / dq::BQ); }

template <int D, bool SOFTCAP, bool DROPOUT>
hipError_t fused_t(const Problem& p, const void* Q, const void* K, const void* V, const void* dO, const float* LSE,
                   const float* Dv, void* dK, void* dV, float* dQacc, void* dQout, hipStream_t s) {
  const unsigned n1 = dkdv_units(p), n2 = dq_units(p);
  hipLaunchKernelGGL((bwd_fused_kernel<D, SOFTCAP, DROPOUT>), dim3(n1 + n2), dim3(kThreads), 0, s,
                     static_cast<const bf16_t*>(Q), static_cast<const bf16_t*>(K), static_cast<const bf16_t*>(V),
                     static_cast<const bf16_t*>(dO), LSE, Dv, static_cast<bf16_t*>(dK), static_cast<bf16_t*>(dV),
                     dQacc, static_cast<bf16_t*>(dQout), p.H, p.H_kv, p.N, p.B * p.H_kv, p.B * p.H, p.scale, p.softcap, p.wl, p.wr, p.drop(), n1,
                     n2);
  return hipGetLastError();
}

template <int D>
hipError_t fused_d(const Problem& p, const void* Q, const void* K, const void* V, const void* dO, const float* LSE,
                   const float* Dv, void* dK, void* dV, float* dQacc, void* dQout, hipStream_t s) {
  if (p.dropout)
    return p.softcap > 0.f ? fused_t<D, true, true>(p, Q, K, V, dO, LSE, Dv, dK, dV, dQacc, dQout, s)
                           : fused_t<D, false, true>(p, Q, K, V, dO, LSE, Dv, dK, dV, dQacc, dQout, s);
  return p.softcap > 0.f ? fused_t<D, true, false>(p, Q, K, V, dO, LSE, Dv, dK, dV, dQacc, dQout, s)
                         : fused_t<D, false, false>(p, Q, K, V, dO, LSE, Dv, dK, dV, dQacc, dQout, s);
}

}  // namespace

bool bwd_fused_fits(const Problem& p) {
  return p.dtype == 1 && dkdv_split_count(p, true) == 1 &&
         int64_t(dkdv_units(p)) + int64_t(dq_units(p)) <= kFusedMaxBlocks;
}

hipError_t launch_bwd_fused_mfma(const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                                 const float* LSE, const float* Dv, void* dK, void* dV, float* dQacc,
                                 void* dQout, hipStream_t s) {
  if (!bwd_fused_fits(p)) return hipErrorInvalidValue;
  return p.d == 64 ? fused_d<64>(p, Q, K, V, dO, LSE, Dv, dK, dV, dQacc, dQout, s)
                   : fused_d<128>(p, Q, K, V, dO, LSE, Dv, dK, dV, dQacc, dQout, s);
}

}  // namespace fabwd

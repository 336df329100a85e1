// Chooses the kernel family for each entry point.
#include "fabwd_launch.h"

namespace fabwd {

hipError_t launch_fwd_stats(const Problem& p, const void* Q, const void* K, const void* V, void* O, float* LSE,
                            hipStream_t s) {
  (void)hipGetLastError();
  // bf16: matrix-core kernel; fp32: vector-ALU kernel.
  if (p.dtype == 1) return launch_fwd_mfma(p, Q, K, V, O, LSE, s);
  return launch_fwd_simple(p, Q, K, V, O, LSE, s);
}

const char* bwd_kernels(const Problem& p, bool with_dq) {
  if (p.dtype == 1) {
    if (bwd_fused_fits(p))
      return fused_split(p, with_dq).floats > 0 ? "bwd_fused_kernel:split" : "bwd_fused_kernel";
    // Given dQ, the dQ kernel also adds the head-split partials.
    return dkdv_split_count(p, true) > 1 && !with_dq ? "bwd_dkdv_kernel+dkdv_split_sum_kernel+bwd_dq_kernel"
                                                     : "bwd_dkdv_kernel+bwd_dq_kernel";
  }
  if (p.deterministic)
    return with_dq ? "bwd_simple_kernel+bwd_dq_simple_kernel+dq_convert_kernel"
                   : "bwd_simple_kernel+bwd_dq_simple_kernel";
  return with_dq ? "bwd_simple_kernel+dq_convert_kernel" : "bwd_simple_kernel";
}

hipError_t launch_bwd(const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                      const float* LSE, const float* D, float* dQacc, void* dK, void* dV, void* dQ,
                      hipStream_t s) {
  (void)hipGetLastError();
  // bf16: matrix-core kernels; fp32: vector-ALU kernel (same fp32 peak on MI355X).
  if (p.dtype == 1) {
    // Few work units: both kinds in one launch, so that they share the chip.
    // Given dQ, the dQ work units write it directly (the same bits as
    // dq_convert of their dQaccum rows).
    if (bwd_fused_fits(p)) return launch_bwd_fused_mfma(p, Q, K, V, dO, LSE, D, dK, dV, dQacc, dQ, s);
    // dQaccum is overwritten by the dQ kernel afterwards (or no longer
    // needed): until then the dK/dV kernel may keep partial sums in it.
    // Given dQ, the dQ kernel leaves dQaccum alone, so it can also add the
    // head-split partials (no separate sum launch).
    const bool sum_in_dq = dQ != nullptr && dkdv_split_count(p, true) > 1;
    hipError_t e = launch_bwd_dkdv_mfma(p, Q, K, V, dO, LSE, D, dK, dV, dQacc, sum_in_dq, s);
    if (e != hipSuccess) return e;
    return launch_bwd_dq_mfma(p, Q, K, V, dO, LSE, D, dQacc, dQ, sum_in_dq ? dK : nullptr,
                              sum_in_dq ? dV : nullptr, s);
  }
  // fp32: dQ partials added with atomics (the pages' scheme), or, in
  // deterministic mode, dK/dV alone plus a query-block-outer dQ kernel.
  hipError_t e = launch_bwd_simple(p, Q, K, V, dO, LSE, D, dQacc, dK, dV, s);
  if (e == hipSuccess && p.deterministic) e = launch_bwd_dq_simple(p, Q, K, V, dO, LSE, D, dQacc, s);
  if (e != hipSuccess || !dQ) return e;
  return launch_bwd_dq_convert(p, dQacc, dQ, s);
}

}  // namespace fabwd

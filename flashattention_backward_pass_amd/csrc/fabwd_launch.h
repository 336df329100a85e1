// Host-side launchers of the gfx950 kernels.  The C ABI (api.cpp) validates
// arguments and then calls exactly one launcher per entry point.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "philox.h"

namespace fabwd {

// Problem description shared by the launchers (already validated).
struct Problem {
  int B, H, H_kv, N, d;
  int dtype;  // 0 fp32, 1 bf16
  bool causal;
  float scale;
  float softcap;
  bool deterministic = false;  // fp32: no atomics (query-block-outer dQ kernel)
  // Visible band: key k is visible to query q iff q - wl <= k <= q + wr (and
  // k < N).  Causal gives wr = 0; an unbounded side is N.
  int wl = 0, wr = 0;
  // Dropout: kept iff the element's 16-bit Philox value is below keep_t;
  // kept elements are scaled by drop_scale = 1 / (1 - p).
  bool dropout = false;
  uint32_t keep_t = 65536;
  float drop_scale = 1.f;
  uint32_t seed_lo = 0, seed_hi = 0, rng_offset = 0;
  int group() const { return H / H_kv; }
  int64_t q_rows() const { return int64_t(B) * H * N; }
  int64_t q_elems() const { return q_rows() * d; }
  Dropout drop() const { return Dropout{dropout ? 1 : 0, keep_t, seed_lo, seed_hi, rng_offset, drop_scale}; }
};

hipError_t launch_fwd_stats(const Problem& p, const void* Q, const void* K, const void* V, void* O, float* LSE,
                            hipStream_t s);
hipError_t launch_bwd_preprocess(const Problem& p, const void* O, const void* dO, float* D, float* dQacc,
                                 hipStream_t s);
// dQ (dtype) non-null: dQ = scale * dQaccum is written as well (bf16: by
// the dQ kernel itself, and dQaccum is then only scratch).
hipError_t launch_bwd(const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                      const float* LSE, const float* D, float* dQacc, void* dK, void* dV, void* dQ,
                      hipStream_t s);
hipError_t launch_bwd_dq_convert(const Problem& p, const float* dQacc, void* dQ, hipStream_t s);
// The allocation-free step (noalloc.cpp): preprocess + backward with every
// scratch buffer in the library's own device array.  noalloc_scratch_floats:
// what p needs; noalloc_scratch_capacity: what the array holds.
int64_t noalloc_scratch_floats(const Problem& p);
int64_t noalloc_scratch_capacity();
hipError_t launch_bwd_noalloc(const Problem& p, const void* Q, const void* K, const void* V, const void* O,
                              const void* dO, const float* LSE, void* dQ, void* dK, void* dV, hipStream_t s);
// Names of the kernels launch_bwd runs for p (with or without dQ), in launch
// order, '+'-separated (static strings; the same decisions as launch_bwd).
const char* bwd_kernels(const Problem& p, bool with_dq);

// Kernel families behind launch_fwd_stats / launch_bwd (dispatch.cpp picks
// one): the *_simple launchers are the fp32 vector kernels (fp32 only; they
// return hipErrorInvalidValue for bf16), the *_mfma launchers the bf16
// matrix-core kernels.
hipError_t launch_fwd_simple(const Problem& p, const void* Q, const void* K, const void* V, void* O, float* LSE,
                             hipStream_t s);
hipError_t launch_fwd_mfma(const Problem& p, const void* Q, const void* K, const void* V, void* O, float* LSE,
                           hipStream_t s);
hipError_t launch_bwd_simple(const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                             const float* LSE, const float* D, float* dQacc, void* dK, void* dV, hipStream_t s);
hipError_t launch_bwd_dq_simple(const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                                const float* LSE, const float* Dv, float* dQacc, hipStream_t s);
// bf16 matrix-core backward: dK/dV kernel (key blocks outer) and dQ kernel
// (query blocks outer); the dQ kernel overwrites dQaccum, or, given dQout,
// writes dQ = scale * acc in bf16 instead and leaves dQaccum alone.
// scratch: B*H*N*d floats the kernel may use for partial sums before the
// dQ kernel overwrites them (dQaccum), or nullptr.  With sum_later the
// head-split partials are left for the dQ kernel to add (given dQout, pass
// dK and dV to launch_bwd_dq_mfma then).
hipError_t launch_bwd_dkdv_mfma(const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                                const float* LSE, const float* Dv, void* dK, void* dV, float* scratch,
                                bool sum_later, hipStream_t s);
// dK, dV: non-null (with dQout) when the dK/dV launch left head-split
// partials in dQacc for this kernel to add; else nullptr.
hipError_t launch_bwd_dq_mfma(const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                              const float* LSE, const float* D, float* dQacc, void* dQout, void* dK, void* dV,
                              hipStream_t s);
// Workgroups sharing each (b, kv head, key block) unit of the dK/dV kernel:
// 2 for grouped heads (G >= 4) with few units, whose fp32 partials then use
// the scratch space (dQaccum) before the dQ kernel overwrites it; else 1.
int dkdv_split_count(const Problem& p, bool have_scratch);
// Both kernels' work units in one launch, for problems too small to fill
// the chip with either kernel alone (bwd_fused_fits).  Requires
// dkdv_split_count(p, true) == 1.
bool bwd_fused_fits(const Problem& p);
// Units the combined launch splits in two when dQ is given (its heaviest
// units under a causal or windowed mask): the first `kv` key blocks of every
// kv head (dK/dV by query range) and the last `q` query blocks of every query
// head (dQ by key range).  Their handoff slots and then `counters` counter
// words (from float offset counter_off, which the preprocess zeroes) take the
// first `floats` floats of dQaccum.  All zero when no split is predicted to
// pay.
struct FusedSplit {
  int kv = 0, q = 0;
  int64_t floats = 0;
  int64_t counter_off = 0;
  int counters = 0;
};
FusedSplit fused_split(const Problem& p, bool with_dq);
hipError_t launch_bwd_fused_mfma(const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                                 const float* LSE, const float* D, void* dK, void* dV, float* dQacc, void* dQout,
                                 hipStream_t s);

}  // namespace fabwd

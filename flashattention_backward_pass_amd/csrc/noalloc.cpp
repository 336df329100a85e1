// attn_bwd_with_dq_noalloc: the backward step (D = rowsum(dO o O), then dK,
// dV and dQ) for callers that cannot allocate device memory.  Every scratch
// buffer of the step lives in one file-scope device array, `scratch`:
//   [0, B*H*N)                      D (fp32)
//   [B*H*N, B*H*N + extra)          fp32: dQaccum (B*H*N*d, zeroed by the
//                                   preprocess kernel); bf16 with the grouped-
//                                   head split: the dK/dV partials
//                                   (4*B*H_kv*N*d); bf16 with split units in
//                                   the combined launch: their partials (at
//                                   most B*H*N*d); otherwise nothing.
// Each device holds its own copy of the array until the process ends; its
// device address is looked up once per device (hipGetSymbolAddress) and only
// that address is handed to kernels.  Calls that overlap on one device share
// the array and race.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "../../include/fabwd.h"
#include "fabwd_launch.h"

namespace {

constexpr int64_t kScratchFloats = int64_t(1) << 24;  // 64 MiB
static __device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
float* g_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, or nullptr.
float* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_ptr[dev] = static_cast<float*>(p);
  }
  return g_ptr[dev];
}

}  // namespace

namespace fabwd {

// Floats of scratch the step needs (see the layout above).
int64_t noalloc_scratch_floats(const Problem& p) {
  const int64_t rows = int64_t(p.B) * p.H * p.N;
  if (p.dtype == 0) return rows + rows * p.d;
  if (dkdv_split_count(p, true) > 1) return rows + 4 * int64_t(p.B) * p.H_kv * p.N * p.d;
  return rows + fused_split(p, true).floats;
}

int64_t noalloc_scratch_capacity() { return kScratchFloats; }

hipError_t launch_bwd_noalloc(const Problem& p, const void* Q, const void* K, const void* V, const void* O,
                              const void* dO, const float* LSE, void* dQ, void* dK, void* dV, hipStream_t s) {
  float* base = scratch_ptr();
  if (!base) return hipErrorInvalidDevicePointer;
  const int64_t rows = int64_t(p.B) * p.H * p.N;
  float* D = base;
  float* extra = base + rows;
  hipError_t e = launch_bwd_preprocess(p, O, dO, D, extra, s);
  if (e != hipSuccess) return e;
  return launch_bwd(p, Q, K, V, dO, LSE, D, extra, dK, dV, dQ, s);
}

}  // namespace fabwd

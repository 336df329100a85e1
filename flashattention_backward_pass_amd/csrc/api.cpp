// C ABI of the backward library: argument validation and dispatch.
// Declarations and the contract of every entry point: include/fabwd.h.
#include "../../include/fabwd.h"

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "fabwd_launch.h"

namespace {

// 2^36 elements per tensor is more than device memory holds.
constexpr int64_t kMaxElems = int64_t(1) << 36;
constexpr int kMaxN = 1 << 24;
// A dispatch counts its work-items in 32 bits.  The matrix-core kernels launch
// at most 2 * B * H * ceil(N / 128) workgroups of 256 work-items (2: the
// grouped-head split of the dK/dV kernel), so short sequences with very many
// heads are the case this bounds.  The fp32 kernels put H (or H_kv) and B in
// the second and third grid dimensions, each at most 65535 blocks.
constexpr int64_t kMaxWorkItems = (int64_t(1) << 32) - 1;
constexpr int kMaxGridYZ = 65535;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validates the sizes and scalars of `p`.  On success fills `out` and sets
// `empty` when there is nothing to compute (B == 0 or N == 0).
int check_params(const attn_params* p, fabwd::Problem* out, bool* empty) {
  if (!p) return ATTN_ERR_INVALID_ARG;
  if (p->B < 0 || p->N < 0 || p->H <= 0 || p->H_kv <= 0 || p->d <= 0) return ATTN_ERR_INVALID_ARG;
  if (p->H % p->H_kv != 0) return ATTN_ERR_INVALID_ARG;
  if (p->dtype != ATTN_FP32 && p->dtype != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
  if (p->causal != 0 && p->causal != 1) return ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(p->scale) || !(p->scale > 0.0f)) return ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(p->softcap) || p->softcap < 0.0f) return ATTN_ERR_INVALID_ARG;
  if (p->deterministic != 0 && p->deterministic != 1) return ATTN_ERR_INVALID_ARG;
  if (p->window_left < -1 || p->window_right < -1) return ATTN_ERR_INVALID_ARG;
  if (!std::isfinite(p->dropout_p) || p->dropout_p < 0.0f || p->dropout_p >= 1.0f) return ATTN_ERR_INVALID_ARG;
  if (p->d != 64 && p->d != 128) return ATTN_ERR_UNSUPPORTED;
  if (p->N > kMaxN) return ATTN_ERR_INVALID_ARG;
  const int64_t elems = int64_t(p->B) * p->H * p->N * p->d;
  if (elems > kMaxElems) return ATTN_ERR_INVALID_ARG;
  const int64_t max_blocks = 2 * int64_t(p->B) * p->H * ((int64_t(p->N) + 127) / 128);
  if (max_blocks * 256 > kMaxWorkItems) return ATTN_ERR_INVALID_ARG;
  if (p->dtype == ATTN_FP32 && (p->B > kMaxGridYZ || p->H > kMaxGridYZ)) return ATTN_ERR_INVALID_ARG;
  out->B = p->B;
  out->H = p->H;
  out->H_kv = p->H_kv;
  out->N = p->N;
  out->d = p->d;
  out->dtype = p->dtype;
  out->causal = p->causal != 0;
  out->scale = p->scale;
  out->softcap = p->softcap;
  out->deterministic = p->deterministic != 0;
  {
    const int n = p->N;
    out->wl = p->window_left < 0 ? n : std::min(p->window_left, n);
    int wr = p->window_right < 0 ? n : std::min(p->window_right, n);
    if (p->causal) wr = std::min(wr, 0);
    out->wr = wr;
  }
  if (p->dropout_p > 0.0f) {
    const double keep = std::floor((1.0 - double(p->dropout_p)) * 65536.0 + 0.5);
    out->dropout = true;
    out->keep_t = uint32_t(std::min(keep, 65536.0));
    out->drop_scale = 1.0f / (1.0f - p->dropout_p);
    out->seed_lo = p->rng_seed_lo;
    out->seed_hi = p->rng_seed_hi;
    out->rng_offset = p->rng_offset;
  }
  *empty = (p->B == 0 || p->N == 0);
  return ATTN_OK;
}

int check_ptrs(std::initializer_list<const void*> ptrs) {
  for (const void* q : ptrs)
    if (!q) return ATTN_ERR_INVALID_ARG;
  for (const void* q : ptrs)
    if (!aligned16(q)) return ATTN_ERR_MISALIGNED;
  return ATTN_OK;
}

int finish(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

}  // namespace

extern "C" {

int attn_fwd_stats(const attn_params* p, const void* Q, const void* K, const void* V, void* O, float* LSE,
                   void* stream) {
  fabwd::Problem pr;
  bool empty = false;
  int rc = check_params(p, &pr, &empty);
  if (rc != ATTN_OK || empty) return rc;
  if ((rc = check_ptrs({Q, K, V, O, LSE})) != ATTN_OK) return rc;
  return finish(fabwd::launch_fwd_stats(pr, Q, K, V, O, LSE, static_cast<hipStream_t>(stream)));
}

int attn_bwd_preprocess(const attn_params* p, const void* O, const void* dO, float* D, float* dQaccum,
                        void* stream) {
  fabwd::Problem pr;
  bool empty = false;
  int rc = check_params(p, &pr, &empty);
  if (rc != ATTN_OK || empty) return rc;
  if ((rc = check_ptrs({O, dO, D, dQaccum})) != ATTN_OK) return rc;
  return finish(fabwd::launch_bwd_preprocess(pr, O, dO, D, dQaccum, static_cast<hipStream_t>(stream)));
}

int attn_bwd(const attn_params* p, const void* Q, const void* K, const void* V, const void* dO, const float* LSE,
             const float* D, float* dQaccum, void* dK, void* dV, void* stream) {
  fabwd::Problem pr;
  bool empty = false;
  int rc = check_params(p, &pr, &empty);
  if (rc != ATTN_OK || empty) return rc;
  if ((rc = check_ptrs({Q, K, V, dO, LSE, D, dQaccum, dK, dV})) != ATTN_OK) return rc;
  return finish(
      fabwd::launch_bwd(pr, Q, K, V, dO, LSE, D, dQaccum, dK, dV, nullptr, static_cast<hipStream_t>(stream)));
}

int attn_bwd_with_dq(const attn_params* p, const void* Q, const void* K, const void* V, const void* dO,
                     const float* LSE, const float* D, float* dQaccum, void* dQ, void* dK, void* dV, void* stream) {
  fabwd::Problem pr;
  bool empty = false;
  int rc = check_params(p, &pr, &empty);
  if (rc != ATTN_OK || empty) return rc;
  if ((rc = check_ptrs({Q, K, V, dO, LSE, D, dQaccum, dQ, dK, dV})) != ATTN_OK) return rc;
  return finish(
      fabwd::launch_bwd(pr, Q, K, V, dO, LSE, D, dQaccum, dK, dV, dQ, static_cast<hipStream_t>(stream)));
}

int attn_bwd_dq_convert(const attn_params* p, const float* dQaccum, void* dQ, void* stream) {
  fabwd::Problem pr;
  bool empty = false;
  int rc = check_params(p, &pr, &empty);
  if (rc != ATTN_OK || empty) return rc;
  if ((rc = check_ptrs({dQaccum, dQ})) != ATTN_OK) return rc;
  return finish(fabwd::launch_bwd_dq_convert(pr, dQaccum, dQ, static_cast<hipStream_t>(stream)));
}

int attn_bwd_with_dq_noalloc(const attn_params* p, const void* Q, const void* K, const void* V, const void* O,
                             const void* dO, const float* LSE, void* dQ, void* dK, void* dV, void* stream) {
  fabwd::Problem pr;
  bool empty = false;
  int rc = check_params(p, &pr, &empty);
  if (rc != ATTN_OK || empty) return rc;
  if (fabwd::noalloc_scratch_floats(pr) > fabwd::noalloc_scratch_capacity()) return ATTN_ERR_INVALID_ARG;
  if ((rc = check_ptrs({Q, K, V, O, dO, LSE, dQ, dK, dV})) != ATTN_OK) return rc;
  return finish(fabwd::launch_bwd_noalloc(pr, Q, K, V, O, dO, LSE, dQ, dK, dV, static_cast<hipStream_t>(stream)));
}

const char* attn_bwd_kernels(const attn_params* p, int with_dq) {
  fabwd::Problem pr;
  bool empty = false;
  if (check_params(p, &pr, &empty) != ATTN_OK || (with_dq != 0 && with_dq != 1)) return nullptr;
  if (empty) return "";
  return fabwd::bwd_kernels(pr, with_dq != 0);
}

const char* attn_status_str(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_INVALID_ARG: return "ATTN_ERR_INVALID_ARG: invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED: no kernel for this configuration";
    case ATTN_ERR_MISALIGNED: return "ATTN_ERR_MISALIGNED: pointer not 16-byte aligned";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP: HIP runtime error at launch";
    default: return "unknown attn_status";
  }
}

const char* attn_version(void) { return "fabwd 0.1 gfx950"; }

}  // extern "C"

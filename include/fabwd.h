/*
 * fabwd.h - C ABI of the MI355X (gfx950) FlashAttention backward library.
 *
 * Sources cited in this header:
 *   [CB]  Inference Cookbook, "反向传播算法详解" (FlashAttention backward pass
 *         explained): section 1.2 (recompute P from the saved LSE), 1.3 (what
 *         the forward saves), 2.1 (the five gradients, dPsum, softcap chain,
 *         dK scaled by the softmax scale), 3.1 (KV-block-outer loop), 6.2 (dQ
 *         accumulated with atomics into an fp32 dQaccum buffer), 8.5 (GQA).
 *   [FA1] "解析 FlashAttention（3）：FlashAttention-v1 反向传播" (FlashAttention-v1
 *         backward): equations (1)-(16), section 3.3 (dropout replay) and
 *         Algorithm 4 (section 4).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or synchronises; it only enqueues kernels.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls are asynchronous and ordered only by that stream.  Kernel faults
 *    surface on a later synchronisation of that stream, as with any launch.
 *  - Layouts are contiguous row-major with the head dimension d fastest:
 *      Q, O, dO, dQ : [B, H,    N, d]
 *      K, V, dK, dV : [B, H_kv, N, d]
 *      LSE, D       : [B, H, N]       float32
 *      dQaccum      : [B, H, N, d]    float32
 *    Element type of Q, K, V, O, dO, dQ, dK, dV is `dtype` (fp32 or bf16).
 *  - Grouped-query attention: H must be a multiple of H_kv; query head h uses
 *    key/value head h / (H / H_kv), and dK, dV of a key/value head are the sum
 *    over its query heads ([CB] 8.5).
 *  - Scores: R = Q K^T (raw).  With softcap c > 0 the logits are
 *    Z = scale * c * tanh(R / c), otherwise Z = scale * R ([CB] 2.1: the cap
 *    acts on the raw scores; the softmax scale multiplies the capped value).
 *    Causal: key j is masked for query i when j > i (the diagonal is kept).
 *    Local window ([CB] 3.4 names a masking phase for a local window's
 *    boundary; the band below is this library's reading): with
 *    window_left >= 0, key j is masked for query i when j < i - window_left;
 *    with window_right >= 0, when j > i + window_right.  Both combine with
 *    the causal mask; -1 leaves a side unbounded, so (-1, -1) is no window.
 *  - Dropout ([FA1] 3.3 and the dropout lines of Algorithm 4): with
 *    dropout_p > 0 the forward multiplies P by a mask Z before P V, and the
 *    backward regenerates the same Z from (rng_seed, rng_offset) instead of
 *    storing it.  Z_ij = 1 / (1 - dropout_p) when element (i, j) is kept,
 *    else 0.  The pages fix no generator; this library's is Philox4x32-10
 *    (Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11):
 *    for query head bh = b * H + h, query i and key j, one call with
 *      counter = (j >> 1, i >> 2, bh, rng_offset),
 *      key     = (rng_seed_lo, rng_seed_hi)
 *    gives words x0..x3; u = bits [16 (j & 1), 16 (j & 1) + 16) of word
 *    x[i & 3]; the element is kept iff u < t, t = floor((1 - p) 65536 + 1/2)
 *    computed in double from the float dropout_p.  LSE is that of the
 *    undropped P.  The same (seed, offset, dropout_p) must be passed to
 *    attn_fwd_stats and attn_bwd; callers advance rng_offset (or the seed)
 *    between layers and steps.
 *  - Every pointer must be 16-byte aligned.  Sizes are rejected
 *    (ATTN_ERR_INVALID_ARG) when B*H*N*d exceeds 2^36 elements (more than
 *    device memory holds), when N exceeds 2^24, when 2*B*H*ceil(N/128)*256
 *    reaches 2^32 (a kernel grid would exceed the work-item count of one
 *    dispatch: very many heads of short sequences), or, for fp32, when B or
 *    H exceeds 65535.  N = 0 or B = 0 is a valid empty problem: the call
 *    validates its arguments and enqueues nothing.
 *  - Return value: ATTN_OK (0) or one of the ATTN_ERR_* codes below.  On an
 *    error nothing is enqueued.  No exception crosses this interface.
 */
#ifndef FABWD_H
#define FABWD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1, /* null pointer, bad size, H % H_kv != 0, scale <= 0, softcap < 0, window < -1,
                               dropout_p outside [0, 1), ... */
  ATTN_ERR_UNSUPPORTED = 2, /* no kernel instance for this (dtype, d) */
  ATTN_ERR_MISALIGNED = 3,  /* a pointer is not 16-byte aligned */
  ATTN_ERR_HIP = 4          /* the HIP runtime reported an error at launch */
};

enum attn_dtype { ATTN_FP32 = 0, ATTN_BF16 = 1 };

typedef struct attn_params {
  int32_t B, H, H_kv, N, d; /* batch, query heads, key/value heads, sequence length, head dim */
  int32_t dtype;            /* enum attn_dtype */
  int32_t causal;           /* 0 or 1 */
  float scale;              /* softmax scale tau, finite and > 0 (usually 1/sqrt(d)) */
  float softcap;            /* c > 0 enables the tanh cap, 0 disables it */
  int32_t deterministic;    /* 0 or 1; see attn_bwd */
  int32_t window_left;      /* local mask: key j hidden from query i when j < i - window_left; -1 = off */
  int32_t window_right;     /* local mask: key j hidden from query i when j > i + window_right; -1 = off */
  float dropout_p;          /* dropout probability in [0, 1); 0 = no dropout */
  uint32_t rng_seed_lo;     /* dropout generator key, low word */
  uint32_t rng_seed_hi;     /* dropout generator key, high word */
  uint32_t rng_offset;      /* dropout generator counter word 3 (per call site / step) */
} attn_params;

/* Supported head dimensions: d = 64 and d = 128, for both dtypes. */

/*
 * attn_fwd_stats - forward pass producing what the backward needs ([CB] 1.3).
 *   O[b,h,i,:]  = sum_j P_ij Zd_ij V[b,g,j,:],  P_i = softmax_j(Z_ij)   (dtype)
 *   LSE[b,h,i]  = ln sum_j exp(Z_ij)                             (float32, natural log)
 * Zd is the dropout mask (all ones when dropout_p = 0).
 * Reads Q, K, V; writes O and LSE.
 */
int attn_fwd_stats(const attn_params* p, const void* Q, const void* K, const void* V,
                   void* O, float* LSE, void* stream);

/*
 * attn_bwd_preprocess - D = rowsum(dO o O) ([FA1] eq (6); [CB] 2.1 dPsum),
 * accumulated in float32 in a fixed order (bitwise reproducible).
 * Reads O, dO; writes D [B,H,N].  For fp32 inputs it also zeroes dQaccum
 * [B,H,N,d] (the fp32 backward adds into it); for bf16 inputs it zeroes at
 * most one word per work unit of dQaccum when attn_bwd_with_dq splits work
 * units for these parameters (the split units' handoff counters; that call
 * must get the same dQaccum) and leaves the rest alone (the bf16 backward
 * overwrites it).
 */
int attn_bwd_preprocess(const attn_params* p, const void* O, const void* dO,
                        float* D, float* dQaccum, void* stream);

/*
 * attn_bwd - the recompute-based backward ([FA1] Algorithm 4; [CB] 3.1, 5.2).
 * For every key/value block j (outer) and query block i (inner):
 *   P   = exp(Z - LSE)                ([CB] 1.2)
 *   dV += (P o Zd)^T dO               ([FA1] eq (10))
 *   dP  = (dO V^T) o Zd               ([FA1] eqs (11), (12))
 *   dS  = P o (dP - D), times (1 - tanh^2(R/c)) with a cap   ([FA1] eq (14); [CB] 2.1)
 *   dK += dS^T Q, scaled by `scale` once at the end            ([FA1] eq (16); [CB] 2.1)
 *   dQaccum += dS K (unscaled)                                 ([FA1] eq (15))
 * Zd is the dropout mask regenerated from the generator state in `p` (all
 * ones when dropout_p = 0); it must be the state attn_fwd_stats used.
 * Inputs: Q, K, V, dO (dtype), LSE from attn_fwd_stats, D from
 * attn_bwd_preprocess on the same stream.  dK and dV are overwritten (not
 * accumulated into).  dQaccum receives sum_j dS_ij K_j without the scale;
 * attn_bwd_dq_convert applies it.
 *   bf16: dK/dV come from a key-block-outer kernel and dQaccum from a
 *         query-block-outer kernel that recomputes S and dP and keeps dQ in
 *         registers; every row of dQaccum is overwritten with plain stores,
 *         so the result is bitwise reproducible (no atomics).  With grouped
 *         query heads (H / H_kv >= 4) and few key blocks, the dK/dV kernel
 *         shares each group's heads over two workgroups and keeps their fp32
 *         partial sums in dQaccum until a fixed-order sum writes dK, dV; the
 *         dQ kernel then overwrites dQaccum.  Problems with few work units
 *         (no head split, at most 1024 workgroups for both kernels at
 *         d = 128, 2048 at d = 64) run both
 *         kinds of work unit in one launch; the results are the same bits.
 *   fp32, deterministic = 0: one kernel adds the dQ partials of each key
 *         block into the zeroed dQaccum with fp32 atomics ([CB] 6.2); the
 *         order of those additions is not fixed, so the low bits of dQ may
 *         differ between runs.
 *   fp32, deterministic = 1: the deterministic mode of [CB] 6.4: dK/dV from
 *         the same kernel without the atomics, and dQaccum overwritten by a
 *         query-block-outer kernel that sums in a fixed order; bitwise
 *         reproducible.
 * The bf16 path is reproducible for either value of `deterministic`.
 * Errors: ATTN_ERR_INVALID_ARG for deterministic other than 0 or 1.
 */
int attn_bwd(const attn_params* p, const void* Q, const void* K, const void* V,
             const void* dO, const float* LSE, const float* D,
             float* dQaccum, void* dK, void* dV, void* stream);

/*
 * attn_bwd_dq_convert - dQ = scale * dQaccum, rounded to dtype
 * (round-to-nearest-even for bf16) ([FA1] eq (7): dQ carries the scale).
 */
int attn_bwd_dq_convert(const attn_params* p, const float* dQaccum, void* dQ, void* stream);

/*
 * attn_bwd_with_dq - attn_bwd and attn_bwd_dq_convert in one call: dK, dV
 * and dQ = scale * sum_j dS_ij K_j ([FA1] eqs (15), (16) with the scale of
 * eq (7)) in dtype, [B, H, N, d] row-major, overwritten.  dQ gets the same
 * bits as attn_bwd followed by attn_bwd_dq_convert, and dK, dV those of
 * attn_bwd, except for split units (below).
 *   bf16: the query-block-outer dQ work units round their fp32 sums and
 *         store dQ directly (no convert launch, no fp32 dQ round trip);
 *         dQaccum is still required as scratch (the grouped-head split of
 *         the dK/dV work keeps partial sums there) and its contents are
 *         unspecified afterwards.  Small causal or windowed problems whose
 *         heaviest work units outweigh the rest take the combined launch
 *         with those units split in two (dK/dV of the first key blocks by
 *         query range, dQ of the last query blocks by key range); the
 *         second half of a unit to finish adds the first's fp32 partial,
 *         handed over in dQaccum with a counter that attn_bwd_preprocess
 *         zeroed (attn_bwd_kernels then returns "bwd_fused_kernel:split").
 *         Those rows add two fp32 halves before rounding and may differ from
 *         attn_bwd's in the last bit; they are still the same from run to
 *         run (the addition is commutative).
 *   fp32: attn_bwd, then the convert kernel; dQaccum holds the unscaled
 *         sums afterwards, as with attn_bwd.
 * dQ must not overlap any other buffer.  Inputs, D (from
 * attn_bwd_preprocess on the same stream), errors and the deterministic
 * flag as for attn_bwd.
 */
int attn_bwd_with_dq(const attn_params* p, const void* Q, const void* K, const void* V,
                     const void* dO, const float* LSE, const float* D,
                     float* dQaccum, void* dQ, void* dK, void* dV, void* stream);

/*
 * attn_bwd_with_dq_noalloc - the whole backward step, attn_bwd_preprocess
 * followed by attn_bwd_with_dq, with no caller-provided scratch and no
 * allocation of any kind: for callers that cannot allocate device memory
 * (code under stream capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Inputs Q, K, V, O, dO, LSE and outputs dQ, dK, dV as for
 * attn_bwd_with_dq (same layouts, dtype and overwrite semantics; the results
 * equal those of attn_bwd_preprocess + attn_bwd_with_dq on the same inputs).
 * D and every scratch buffer of the step (fp32: the dQaccum sums; bf16 with
 * the grouped-head split: the dK/dV partial sums) live in one static device
 * array of 64 MiB that the library holds on each device it runs on until the
 * process ends; calls that overlap on one device share it and race.
 * Errors: as attn_bwd_with_dq, plus ATTN_ERR_INVALID_ARG when the step needs
 * more than 2^24 floats of scratch: B*H*N (D) plus, for fp32, B*H*N*d, or,
 * for bf16 when H / H_kv >= 4 and B*H_kv*ceil(N/128) < 1024, 4*B*H_kv*N*d,
 * or, for bf16 with split units in the combined launch, at most B*H*N*d.
 */
int attn_bwd_with_dq_noalloc(const attn_params* p, const void* Q, const void* K, const void* V,
                             const void* O, const void* dO, const float* LSE,
                             void* dQ, void* dK, void* dV, void* stream);

/*
 * attn_bwd_kernels - the kernels that attn_bwd (with_dq = 0) or
 * attn_bwd_with_dq (with_dq = 1) launches for these parameters on the
 * current device, in launch order, separated by '+' (static storage; ""
 * for an empty problem; NULL when the parameters are invalid or with_dq is
 * not 0 or 1).  A name may carry a ":split" suffix: the combined launch
 * with split work units (see attn_bwd_with_dq).  Enqueues nothing.  For
 * tests and tools that need to know which path a shape takes.
 */
const char* attn_bwd_kernels(const attn_params* p, int with_dq);

/* Human-readable name of a status code (static storage; never NULL). */
const char* attn_status_str(int status);

/* Library version string (static storage). */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FABWD_H */

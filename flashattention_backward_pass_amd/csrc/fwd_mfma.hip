// bf16 forward (O and LSE) on gfx950 matrix cores: query blocks outer, key
// blocks inner, online softmax (Inference Cookbook page "反向传播算法详解",
// section 3.1; the LSE it saves is section 1.3 of that page).
//
// Per workgroup: 128 query rows of one query head, wave w owning rows
// 32w .. 32w+31; key blocks of 64 stream through double-buffered LDS tiles in
// two halves of 32 keys.  Per half:
//   S^T  = K Q^T           (keys x queries: one query per lane, so the row
//                           max and row sum are per-lane register reductions
//                           plus one exchange with the partner lane that
//                           holds the other keys of the same query)
//   P^T  = exp2(S' tau log2e - m)            (m: running max, log2 units)
//   O^T += V^T P^T         (d x queries: P^T is the S^T accumulator packed
//                           to bf16, V^T is read transposed from the
//                           row-major V tile)
// Keeping O transposed makes the online-softmax rescale a per-lane scalar.
// The running max is raised lazily: only when a new score exceeds it by more
// than 8 (log2 units) are O and the row sum rescaled, so P <= 2^8 and the
// rescale is rare; O / l and LSE = (m + log2 l) ln 2 at the end are exact
// whatever max was used.
// Dropout (FlashAttention-v1 page, section 3.3): P^T is multiplied by the
// mask Z before it enters O^T (the row sum keeps the undropped P); the mask
// is regenerated per 32-key half from the generator state (philox.h), and
// the 1 / (1 - p) of the kept elements is applied with the final 1 / l.
#include <type_traits>

#include "fabwd_launch.h"
#include "mfma_common.h"

namespace fabwd {

namespace {

constexpr int kThreads = 256;
constexpr int BQ = 128;  // query rows per workgroup
constexpr int BK = 64;   // keys per LDS block
constexpr float kLazy = 8.f;
constexpr float kLn2 = 0.6931471805599453f;

// Key k is visible to query q iff q - wl <= k <= q + wr and k < N (causal:
// wr = 0; an unbounded side is N).
template <int D, bool SOFTCAP, bool DROPOUT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_mfma_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    bf16_t* __restrict__ O, float* __restrict__ LSE, int H, int H_kv, int N, int BHq, float scale, float softcap,
    int wl, int wr, Dropout drop) {
  constexpr int KC = D / 16;
  constexpr int NT = D / 32;
  // Double buffers as separate variables (own alias scopes: reads of one
  // buffer do not wait for copies landing in the other).
  __shared__ __attribute__((aligned(1024))) uint16_t sK0[BK * D], sK1[BK * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sV0[BK * D], sV1[BK * D];
  auto bufsel = [](auto bufc, auto* a0, auto* a1) {
    if constexpr (decltype(bufc)::value == 0) return a0;
    else return a1;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int j16 = lane & 15, h16 = (lane >> 4) & 1;

  // Work unit: the key/value head varies fastest, so that with the
  // round-robin placement of workgroups on the 8 XCDs the query heads of one
  // group share an XCD (and its L2 holds their K, V); then the query head in
  // the group; query blocks vary slowest, last (heaviest under a causal
  // mask) first.
  const int n_qblk = (N + BQ - 1) / BQ;
  const int G = H / H_kv;
  const int BHkv = BHq / G;
  const int kvu = int(blockIdx.x % unsigned(BHkv));
  const int rest = int(blockIdx.x / unsigned(BHkv));
  const int b = kvu / H_kv, hk = kvu % H_kv;
  const int h = hk * G + rest % G;
  const int bhq = b * H + h;
  const int iblk = n_qblk - 1 - rest / G;
  const int q0 = iblk * BQ;
  const int64_t q_off = (int64_t(b) * H + h) * N;
  const int64_t kv_off = (int64_t(b) * H_kv + hk) * N;
  const int my_q = q0 + 32 * w + l32;  // query of this lane
  const int qc = min(my_q, N - 1);
  // Keys k that my_q sees form one range (my_q - wl <= k <= my_q + wr, k < N):
  // one unsigned compare per element on masked blocks.
  const int vk_lo = max(0, my_q - wl);
  const int vk_len = max(0, min(N - 1, my_q + wr) - vk_lo + 1);

  // Q row of this lane: B operand of S^T = K Q^T (k = d).
  bf16x8_t qreg[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) qreg[c] = load_bf16x8(Q + (q_off + qc) * D + 16 * c + 8 * g);
  const float zs = scale * kLog2e;
  const float cap_k = SOFTCAP ? 2.f * kLog2e / softcap : 0.f;  // tanh(x / c) = tanh_scaled(x, cap_k)
  const float cap_zs = softcap * zs;

  f32x16_t o_acc[NT];  // O^T: register r of tile n = d index 32n + 8(r/4) + 4g + r%4
#pragma unroll
  for (int n = 0; n < NT; ++n) o_acc[n] = f32x16_t{};
  float m = -__builtin_inff();  // running max of S' tau log2e for this query
  float l = 0.f;                // this lane's share of the row sum (its keys)

  // Key blocks seen by some row of this block: [s_lo, s_hi).  Blocks in
  // [p_lo, p_hi) are visible to every row (no mask); the others are partly
  // masked (left window edge, diagonal / right edge, ragged end).
  const int q_hi = min(q0 + BQ, N) - 1;  // last valid row
  const int s_lo = max(0, q0 - wl) / BK;
  const int s_hi = (min(N, q_hi + wr + 1) + BK - 1) / BK;
  const int p_lo = min(s_hi, max(s_lo, (max(0, q_hi - wl) + BK - 1) / BK));
  const int p_hi = max(p_lo, min(s_hi, min((q0 + wr + 1) / BK, N / BK)));
  const int n_steps = s_hi - s_lo;
  // Position -> key block: the unmasked blocks first, then the masked ones.
  auto block_at = [&](int pos) {
    const int n_plain = p_hi - p_lo, n_pre = p_lo - s_lo;
    if (pos < n_plain) return p_lo + pos;
    if (pos < n_plain + n_pre) return s_lo + (pos - n_plain);
    return p_hi + (pos - n_plain - n_pre);
  };

  // K/V block copies (buffer loads that write LDS); descriptors span the
  // block's valid rows, reads past N return zeros and the tiles start zeroed.
  constexpr int RPS = 1024 / (2 * D);
  constexpr int NSLAB = BK / RPS / 4;
  int voff[NSLAB];
#pragma unroll
  for (int s = 0; s < NSLAB; ++s) {
    const int row = (s * 4 + w) * RPS + lane / (D / 8);
    voff[s] = (row * D + 8 * ((lane % (D / 8)) ^ swz<D>(row))) * 2;
  }
  auto issue = [&](auto bufc, int blk) {
    const int kb = blk * BK;
    const int rows = min(BK, N - kb);
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(K + (kv_off + kb) * D), 0, rows * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)(V + (kv_off + kb) * D), 0, rows * D * 2, 0x00020000);
#pragma unroll
    for (int s = 0; s < NSLAB; ++s) {
      const int vo = voff[s];  // a plain local: see the dQ kernel's note on buffer builtins
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)&bufsel(bufc, sK0, sK1)[(s * 4 + w) * 512], 16, vo,
                                               0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)&bufsel(bufc, sV0, sV1)[(s * 4 + w) * 512], 16, vo,
                                               0, 0, 0);
    }
  };

  // Per-lane LDS offsets: row reads of K (A operand of S^T: row l32, chunk
  // 2c + g) and transposing reads of V (A operand V^T of O^T: rows 4g + j16/4
  // (+8), chunk 4n + 2 h16 + (j16 % 4)/2, element 4 (j16 % 2)).
  int off_a[KC], off_t[NT][2];
#pragma unroll
  for (int c = 0; c < KC; ++c) off_a[c] = swz_off<D>(l32, 2 * c + g, 0);
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int ch = 4 * n + 2 * h16 + ((j16 & 3) >> 1);
#pragma unroll
    for (int v = 0; v < 2; ++v) off_t[n][v] = swz_off<D>(4 * g + (j16 >> 2) + 8 * v, ch, 4 * (j16 & 1));
  }

  // One half (32 keys, kb .. kb+31) of the block in buffer BUF.
  auto half = [&](auto bufc, auto maskc, int kb, int s) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(maskc)::value;
    const uint16_t* sk = bufsel(bufc, sK0, sK1);
    const uint16_t* sv = bufsel(bufc, sV0, sV1);
    // S^T: register r = key kb + 32s + 8(r/4) + 4g + r%4, lane = query.
    f32x16_t st = {};
    if (MASKED) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb + 32 * s + 8 * (r >> 2) + 4 * g + (r & 3);
        st[r] = unsigned(key - vk_lo) < unsigned(vk_len) ? 0.f : -__builtin_inff();
      }
    }
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int c = 0; c < KC; ++c)
      st = mfma32(*reinterpret_cast<const bf16x8_t*>(&sk[off_a[c] + 32 * s * D]), qreg[c], st);
    // Phases (S chain | softmax | O chain) stay in order: bounded live ranges.
    __builtin_amdgcn_sched_barrier(0);
    // The softmax phase issues at a higher priority than the matrix chains,
    // so it completes under the other wave's matrix instructions.
    __builtin_amdgcn_s_setprio(2);
    // Mask bits of this half (the other wave's matrix instructions overlap).
    DropBits keep;
    if (DROPOUT) keep = DropQueryLane::sequential(drop, uint32_t(bhq), kb + 32 * s, my_q, lane);
    // New max (log2 units) over these keys and the partner lane's.  With a
    // cap, st becomes the capped score in log2 units; without one st stays
    // the raw score (tau > 0 keeps the order), the max is scaled once, and
    // the scale folds into the exponent below.
    float mx = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (SOFTCAP) {
        // The cap would turn a masked -inf into a finite -c: keep it -inf.
        const float z = (MASKED && st[r] == -__builtin_inff()) ? st[r] : cap_zs * tanh_scaled(st[r], cap_k);
        st[r] = z;
      }
      mx = fmaxf(mx, st[r]);
    }
    if (!SOFTCAP) mx *= zs;  // -inf stays -inf
    mx = max_lane_pair32(mx);
    // Lazy rescale: raise m only when a score exceeds it by more than kLazy.
    if (__builtin_amdgcn_ballot_w64(mx > m + kLazy) != 0) {
      const float m_new = mx > m + kLazy ? mx : m;
      const float alpha = m_new == m ? 1.f : fast_exp2(m - m_new);  // 0 when m was -inf
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) o_acc[n][r] *= alpha;
    }
    // P^T = exp2(z - m), row-sum share, bf16 B operand of O^T.  (While no
    // key of the row has been seen, m = -inf and every z is -inf: use 0.)
    const float mu = m == -__builtin_inff() ? 0.f : m;
    bf16x8_t pf[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      u32x4_t pw;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float p0 = fast_exp2(SOFTCAP ? st[8 * u + 2 * k] - mu : fmaf(st[8 * u + 2 * k], zs, -mu));
        const float p1 = fast_exp2(SOFTCAP ? st[8 * u + 2 * k + 1] - mu : fmaf(st[8 * u + 2 * k + 1], zs, -mu));
        l += p0 + p1;
        if (DROPOUT)
          pw[k] = pack_bf16x2(keep.keep(8 * u + 2 * k, drop.keep_t) ? p0 : 0.f,
                              keep.keep(8 * u + 2 * k + 1, drop.keep_t) ? p1 : 0.f);
        else
          pw[k] = pack_bf16x2(p0, p1);
      }
      pf[u] = __builtin_bit_cast(bf16x8_t, pw);
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    // O^T += V^T P^T: k = keys 32s + 16u + (accumulator row order), d on lanes.
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int base = (32 * s + 16 * u) * D;
        const bf16x8_t va = cat8(lds_read_tr(&sv[off_t[n][0] + base]), lds_read_tr(&sv[off_t[n][1] + base]));
        o_acc[n] = mfma32(va, pf[u], o_acc[n]);
      }
  };

  // Zero the tiles once, so rows past N (never copied) hold finite values.
  {
    const u32x4_t z = {0u, 0u, 0u, 0u};
    for (int i = tid; i < BK * D / 8; i += kThreads) {
      reinterpret_cast<u32x4_t*>(sK0)[i] = z;
      reinterpret_cast<u32x4_t*>(sK1)[i] = z;
      reinterpret_cast<u32x4_t*>(sV0)[i] = z;
      reinterpret_cast<u32x4_t*>(sV1)[i] = z;
    }
    __syncthreads();
  }
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  auto step_fn = [&](auto bufc, auto maskc, int pos) __attribute__((always_inline)) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // block at `pos` in this buffer; the other buffer no longer read
    if (pos + 1 < n_steps) issue(std::integral_constant<int, 1 - decltype(bufc)::value>{}, block_at(pos + 1));
    const int kb = block_at(pos) * BK;
    half(bufc, maskc, kb, 0);
    half(bufc, maskc, kb, 1);
  };
  if (n_steps > 0) issue(B0{}, block_at(0));
  const int n_plain = p_hi - p_lo;
  int pos = 0;
  for (; pos + 2 <= n_plain; pos += 2) {
    step_fn(B0{}, std::false_type{}, pos);
    step_fn(B1{}, std::false_type{}, pos + 1);
  }
  if (pos < n_plain) {
    step_fn(B0{}, std::false_type{}, pos);
    ++pos;
  }
  for (; pos < n_steps; ++pos) {
    if (pos & 1)
      step_fn(B1{}, std::true_type{}, pos);
    else
      step_fn(B0{}, std::true_type{}, pos);
  }

  // Epilogue: l over both key groups; O = O^T / l (4 consecutive d per
  // register group), LSE = (m + log2 l) ln 2.
  l = sum_lane_pair32(l);
  if (my_q < N) {
    const float inv = (DROPOUT ? drop.scale : 1.f) / l;
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int mq = 0; mq < 4; ++mq) {
        u32x2_t v;
        v[0] = pack_bf16x2(o_acc[n][4 * mq] * inv, o_acc[n][4 * mq + 1] * inv);
        v[1] = pack_bf16x2(o_acc[n][4 * mq + 2] * inv, o_acc[n][4 * mq + 3] * inv);
        *reinterpret_cast<u32x2_t*>(O + (q_off + my_q) * D + 32 * n + 8 * mq + 4 * g) = v;
      }
    if (g == 0) LSE[q_off + my_q] = (m + __builtin_log2f(l)) * kLn2;
  }
}

template <int D, bool SOFTCAP, bool DROPOUT>
hipError_t fwd_t(const Problem& p, const void* Q, const void* K, const void* V, void* O, float* LSE, hipStream_t s) {
  const int BHq = p.B * p.H;
  const int n_qblk = (p.N + BQ - 1) / BQ;
  hipLaunchKernelGGL((fwd_mfma_kernel<D, SOFTCAP, DROPOUT>), dim3(unsigned(BHq) * unsigned(n_qblk)), dim3(kThreads),
                     0, s, static_cast<const bf16_t*>(Q), static_cast<const bf16_t*>(K),
                     static_cast<const bf16_t*>(V), static_cast<bf16_t*>(O), LSE, p.H, p.H_kv, p.N, BHq, p.scale,
                     p.softcap, p.wl, p.wr, p.drop());
  return hipGetLastError();
}

template <int D>
hipError_t fwd_d(const Problem& p, const void* Q, const void* K, const void* V, void* O, float* LSE, hipStream_t s) {
  if (p.dropout)
    return p.softcap > 0.f ? fwd_t<D, true, true>(p, Q, K, V, O, LSE, s) : fwd_t<D, false, true>(p, Q, K, V, O, LSE, s);
  return p.softcap > 0.f ? fwd_t<D, true, false>(p, Q, K, V, O, LSE, s) : fwd_t<D, false, false>(p, Q, K, V, O, LSE, s);
}

}  // namespace

hipError_t launch_fwd_mfma(const Problem& p, const void* Q, const void* K, const void* V, void* O, float* LSE,
                           hipStream_t s) {
  return p.d == 64 ? fwd_d<64>(p, Q, K, V, O, LSE, s) : fwd_d<128>(p, Q, K, V, O, LSE, s);
}

}  // namespace fabwd

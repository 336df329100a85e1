// bf16 dQ work unit on gfx950 matrix cores: query blocks outer, key blocks
// inner.  The body of bwd_dq_kernel (bwd_dq.hip); `block` plays the role of
// the block index.
//
// dQ_i = sum_j dS_ij K_j ("解析 FlashAttention（3）：FlashAttention-v1 反向传播",
// eq (15), without the scale tau, which the convert kernel applies).  The
// pages accumulate dQ across key blocks with fp32 atomics into a global
// buffer (Inference Cookbook "反向传播算法详解", section 6.2).  On MI355X every
// global float atomic is executed at the memory side rather than in L2, which
// caps that path near 1.3 TB/s of update traffic; this kernel instead gives
// each workgroup a whole block of query rows, recomputes S and dP for them
// (P from the saved LSE, section 1.2 of the Cookbook page), and keeps dQ in
// registers over all key blocks, so dQaccum is written once with plain
// stores and the result does not depend on any summation order across
// workgroups.
//
// Per workgroup: 128 query rows of one query head (wave w owns rows
// 32w..32w+31), key blocks of 64 streamed through double-buffered LDS tiles.
// Per key block and 32-key half:
//   S^T  = K Q^T      (keys x queries; Q rows of this wave in registers)
//   dP^T = V dO^T
//   P = exp2(S' tau log2e - LSE log2e), dS = P o (dP - D) [o (1 - tanh^2)]
//   dQ  += dS K       (dS^T accumulator layout = A operand with queries on
//                      lanes; K^T read transposed from the row-major K tile)
// Computing S^T rather than S puts one query per lane, so LSE and D are one
// register each.  Wave priorities: S/dP chain 0, softmax 2, dQ chain 1.
// Dropout (FlashAttention-v1 page, eq (12)): dP^T is multiplied by the
// replayed mask Z before dS; the quad of lanes holding 4 consecutive queries
// evaluates the 8 generator calls of a 32-key half together (philox.h).
#pragma once

#include <type_traits>

#include "fabwd_launch.h"
#include "mfma_common.h"

namespace fabwd {
namespace dq {

constexpr int kThreads = 256;
constexpr int kPF = 2;   // matrix steps (S/dP and dQ chains) whose operand reads run ahead
constexpr int BQ = 128;  // query rows per workgroup
constexpr int BK = 64;   // keys per inner step

// Key k is visible to query q iff q - wl <= k <= q + wr and k < N (causal:
// wr = 0; an unbounded side is N).
template <int D, bool SOFTCAP, bool DROPOUT>
__device__ __forceinline__ void dq_block(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const bf16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    float* __restrict__ dQacc, bf16_t* __restrict__ dQout, int H, int H_kv, int N, int BHq, float scale,
    float softcap, int wl, int wr, Dropout drop, unsigned block, int khalf = -1, int qq = 0,
    float* __restrict__ part = nullptr, unsigned* counters = nullptr) {
  constexpr int KC = D / 16;
  constexpr int NT = D / 32;
  // Double buffers as separate variables: the compiler gives each LDS
  // variable its own alias scope, so reads of one buffer do not wait for the
  // asynchronous copies still landing in the other.
  // K and V of one buffer share a variable (copied and read together): a V
  // address is then the K address plus an immediate offset.
  __shared__ __attribute__((aligned(1024))) uint16_t sKV0[2 * BK * D], sKV1[2 * BK * D];
  uint16_t* const sK0 = sKV0;
  uint16_t* const sK1 = sKV1;
  uint16_t* const sV0 = sKV0 + BK * D;
  uint16_t* const sV1 = sKV1 + BK * D;
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
  const int kvu = int(block % unsigned(BHkv));
  const int rest = int(block / unsigned(BHkv));
  const int b = kvu / H_kv, hk = kvu % H_kv;
  const int h = hk * G + rest % G;
  const int bhq = b * H + h;
  const int iblk = n_qblk - 1 - rest / G;
  const int q0 = iblk * BQ;
  const int64_t q_off = (int64_t(b) * H + h) * N;
  const int64_t kv_off = (int64_t(b) * H_kv + hk) * N;
  const int my_q = q0 + 32 * w + l32;  // query row owned by this lane
  const int my_qc = min(my_q, N - 1);
  // Keys k that my_q sees form one range: my_q - wl <= k <= my_q + wr, k < N
  // (one unsigned compare per element in the mask pass).
  const int vk_lo = max(0, my_q - wl);
  const int vk_len = max(0, min(N - 1, my_q + wr) - vk_lo + 1);

  // Q and dO rows of this lane (B operands of S^T and dP^T), LSE and D.
  bf16x8_t qreg[KC], doreg[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    qreg[c] = load_bf16x8(Q + (q_off + my_qc) * D + 16 * c + 8 * g);
    doreg[c] = load_bf16x8(dO + (q_off + my_qc) * D + 16 * c + 8 * g);
  }
  const float nl2 = -LSE[q_off + my_qc] * kLog2e;
  const float dval = Dv[q_off + my_qc];
  const float zs = scale * kLog2e;
  const float cap_k = SOFTCAP ? 2.f * kLog2e / softcap : 0.f;  // tanh(x / c) = tanh_scaled(x, cap_k)
  const float cap_zs = softcap * zs;

  // -D_q in every register: without dropout the first dP^T instruction of a
  // key block takes it as the accumulator input, so the chain ends with
  // dP - D (this lane's query, and so D, is the same for every key) and the
  // softmax step saves a subtraction per element.
  f32x16_t neg_d;
#pragma unroll
  for (int r = 0; r < 16; ++r) neg_d[r] = -dval;

  f32x16_t dq_acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) dq_acc[n] = f32x16_t{};

  // LDS element offsets of this lane's operand reads within a K or V block.
  // The swizzle depends on the row mod 16 only, so rows 32 s + l32 (row
  // reads) and 32 s + 16 u + 4 g + j16/4 (+ 8) (transposed reads) are these
  // offsets plus a multiple of 16 D.  The empty asm hides their bits from the
  // compiler: otherwise it forms the V and second-buffer addresses with a
  // bitwise or, which an LDS instruction cannot take as its immediate offset,
  // and keeps a register for every (buffer, tensor, half) variant.
  int roff[KC], toff[NT][2];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    roff[c] = swz_off<D>(l32, 2 * c + g, 0);
    asm volatile("" : "+v"(roff[c]));
  }
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int ch = 4 * n + 2 * h16 + ((j16 & 3) >> 1);
    const int sub = 4 * (j16 & 1);
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      toff[n][v] = swz_off<D>(4 * g + (j16 >> 2) + 8 * v, ch, sub);
      asm volatile("" : "+v"(toff[n][v]));
    }
  }

  // Key blocks [s_lo, s_hi) hold every key that some row of this block sees.
  // With khalf >= 0 (combined launch) this workgroup takes half khalf of them
  // (0: the later ones, 1: the earlier ones); the two halves hand the tile
  // over through slot bhq * qq + (n_qblk - 1 - iblk) of `part` (BQ x D
  // floats) and the counter of the same index (split_arrive_first).
  const int q_hi = min(q0 + BQ, N) - 1;  // last valid row
  int s_lo = max(0, q0 - wl) / BK;
  int s_hi = (min(N, q_hi + wr + 1) + BK - 1) / BK;
  if (khalf >= 0) {
    const int mid = (s_lo + s_hi + 1) / 2;
    if (khalf == 0) s_lo = mid;
    else s_hi = mid;
  }

  // Per-lane byte offsets of the K/V block copies: slab I = s*4 + w covers
  // rows I*RPS ..; lane L fills physical chunk L % (D/8) of row I*RPS + L/(D/8),
  // i.e. logical chunk (L % (D/8)) ^ swz(row).
  constexpr int RPS = 1024 / (2 * D);
  constexpr int NSLAB = BK / RPS / 4;
  int dma_voff[NSLAB];
#pragma unroll
  for (int s = 0; s < NSLAB; ++s) {
    const int row = (s * 4 + w) * RPS + lane / (D / 8);
    dma_voff[s] = (row * D + 8 * ((lane % (D / 8)) ^ swz<D>(row))) * 2;
  }
  // Copy key/value block `step` into LDS buffer step%2 with buffer loads that
  // write LDS directly (scalar base per block; a ragged block clamps its rows
  // to the last valid key).
  auto issue = [&](auto bufc, int step) {
    const int kb = step * BK;
    const int rows = min(BK, N - kb);
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)(K + (kv_off + kb) * D), 0, rows * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc((void*)(V + (kv_off + kb) * D), 0, rows * D * 2, 0x00020000);
#pragma unroll
    for (int s = 0; s < NSLAB; ++s) {
      int voff = dma_voff[s];
      if (rows < BK) {
        const int row = min((s * 4 + w) * RPS + lane / (D / 8), rows - 1);
        voff = (row * D + 8 * ((lane % (D / 8)) ^ swz<D>((s * 4 + w) * RPS + lane / (D / 8)))) * 2;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)&bufsel(bufc, sK0, sK1)[(s * 4 + w) * 512], 16, voff,
                                               0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)&bufsel(bufc, sV0, sV1)[(s * 4 + w) * 512], 16, voff,
                                               0, 0, 0);
    }
  };

  // One key block in buffer BUF (the loop below alternates the buffers with
  // compile-time selection, so every LDS access names one variable).
  auto body = [&](auto bufc, int step) __attribute__((always_inline)) {
    using NB = std::integral_constant<int, 1 - decltype(bufc)::value>;
    const uint16_t* sk = bufsel(bufc, sK0, sK1);
    const uint16_t* sv = bufsel(bufc, sV0, sV1);
    const int kb = step * BK;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // block `step` in this buffer; the other buffer no longer read
    if (step + 1 < s_hi) issue(NB{}, step + 1);
    // Unmasked: every key of the block is visible to every row of this block.
    const bool masked = kb + BK > N || kb < q_hi - wl || kb + BK - 1 > q0 + wr;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      // S^T, dP^T for keys kb + 32 s .. + 31 (rows) x this wave's 32 queries (columns).
      f32x16_t st = {}, dpt = DROPOUT ? f32x16_t{} : neg_d;
      __builtin_amdgcn_s_setprio(0);
      // The reads of step c + kPF are issued before the matrix instructions of
      // step c (the fences keep the scheduler from sinking them to their use).
      bf16x8_t kop[KC], vop[KC];
      auto read_ops = [&](int c) {
        kop[c] = *reinterpret_cast<const bf16x8_t*>(&sk[roff[c] + 32 * s * D]);
        vop[c] = *reinterpret_cast<const bf16x8_t*>(&sv[roff[c] + 32 * s * D]);
      };
#pragma unroll
      for (int c = 0; c < kPF; ++c) read_ops(c);
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        if (c + kPF < KC) read_ops(c + kPF);
        __builtin_amdgcn_sched_barrier(0);
        st = mfma32(kop[c], qreg[c], st);
        dpt = mfma32(vop[c], doreg[c], dpt);
        __builtin_amdgcn_sched_barrier(0);
      }
      // The two waves of a SIMD overlap one's softmax with the other's matrix
      // instructions; the softmax phase (mask generator included) issues at
      // the higher priority so it finishes while the matrix core is busy.
      __builtin_amdgcn_s_setprio(2);
      DropBits keep;
      if (DROPOUT) {
        DropQueryLane gen;
        gen.init(drop, uint32_t(bhq), kb + 32 * s, my_q, lane);
        gen.rounds(0, 10);
        keep = gen.finish(lane);
      }
      // Register r: key kb + 32 s + 8(r/4) + 4g + r%4, query my_q.  dS is
      // computed for every key, then masked keys are set to 0 in one pass
      // under a single uniform branch (a test inside this loop becomes a
      // branch per element).  The select discards whatever a masked key
      // produced, inf or NaN included.
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float dt = 1.f;
        float p;
        if (SOFTCAP) {
          const float th = tanh_scaled(st[r], cap_k);
          dt = fmaf(-th, th, 1.f);
          p = fast_exp2(fmaf(th, cap_zs, nl2));
        } else {
          p = fast_exp2(fmaf(st[r], zs, nl2));
        }
        // dP - D: the accumulator holds it already without dropout; with
        // dropout the mask and 1/(1-p) apply to dP alone.
        float dpd = dpt[r];
        if (DROPOUT) dpd = (keep.keep(r, drop.keep_t) ? dpd * drop.scale : 0.f) - dval;
        float ds = p * dpd;
        if (SOFTCAP) ds *= dt;
        st[r] = ds;
      }
      if (masked) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb + 32 * s + 8 * (r >> 2) + 4 * g + (r & 3);
          st[r] = unsigned(key - vk_lo) < unsigned(vk_len) ? st[r] : 0.f;
        }
      }
      bf16x8_t dsf[2];
      dsf[0] = pack_bf16x8(st, 0);
      dsf[1] = pack_bf16x8(st, 8);
      __builtin_amdgcn_s_setprio(1);
      // dQ += dS K over these 32 keys: K operand rows 32 s + 16u + 4g + (0..3)
      // and +8; step i = 2n + u, its operand read kPF steps ahead.
      bf16x8_t kt[2 * NT];
      auto read_kt = [&](int i) {
        const int rb = (32 * s + 16 * (i & 1)) * D;
        kt[i] = cat8(lds_read_tr(&sk[toff[i >> 1][0] + rb]), lds_read_tr(&sk[toff[i >> 1][1] + rb]));
      };
#pragma unroll
      for (int i = 0; i < kPF; ++i) read_kt(i);
#pragma unroll
      for (int i = 0; i < 2 * NT; ++i) {
        if (i + kPF < 2 * NT) read_kt(i + kPF);
        __builtin_amdgcn_sched_barrier(0);
        dq_acc[i >> 1] = mfma32(dsf[i & 1], kt[i], dq_acc[i >> 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  if (s_lo < s_hi) issue(B0{}, s_lo);
  for (int step = s_lo; step < s_hi; step += 2) {
    body(B0{}, step);
    if (step + 1 < s_hi) body(B1{}, step + 1);
  }

  // Rows of this wave, register r: row 32w + 8(r/4) + 4g + r%4.  Either
  // dQaccum (unscaled fp32) or, given dQout, dQ itself: the same fp32 product
  // scale * acc and round-to-nearest-even as the convert kernel, so the bits
  // equal those of the two-step path.  Staged through the idle K/V tiles so
  // that the global writes are 16-byte row chunks; rows past N are skipped.
  const int valid = min(BQ, N - q0);
  // The last tile's copies (into the idle buffer) must land before the tiles are reused.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();  // every wave is done with the K/V tiles
  if (dQout && khalf < 0) {
    bf16_t* t = reinterpret_cast<bf16_t*>(sKV0);  // BQ x D bf16 = one buffer
    stage_acc<bf16_t, NT, D>(t, 32 * w, dq_acc, scale, lane);
    __syncthreads();
    stage_copy_rows<bf16_t, D, kThreads>(dQout + (q_off + q0) * D, t, BQ, valid, tid);
  } else {
    // BQ x D fp32 = both buffers: rows 0-63 in buffer 0, rows 64-127 in buffer 1.
    float* t0 = reinterpret_cast<float*>(sKV0);
    float* t1 = reinterpret_cast<float*>(sKV1);
    // Key-range split: the first half to finish writes its fp32 sum to the
    // unit's slot, the second adds it to its own and writes dQ.
    __shared__ unsigned s_arrival;
    const int64_t slot = int64_t(bhq) * qq + (n_qblk - 1 - iblk);
    const bool to_part = khalf < 0 || split_arrive_first(counters + slot, &s_arrival, tid);
    float* dst = khalf >= 0 ? part + slot * (BQ * D) : dQacc + (q_off + q0) * D;
    stage_acc<float, NT, D>(w < 2 ? t0 : t1, 32 * w - (w < 2 ? 0 : BQ / 2), dq_acc, 1.f, lane);
    if (!to_part) split_wait(counters + slot, tid);
    __syncthreads();
    if (to_part && khalf < 0) {
      stage_copy_rows<float, D, kThreads>(dst, t0, BQ / 2, valid, tid);
      stage_copy_rows<float, D, kThreads>(dst + (BQ / 2) * D, t1, BQ / 2, valid - BQ / 2, tid);
    } else if (to_part) {
      stage_store_rows_coherent<D, kThreads>(dst, t0, BQ / 2, valid, tid);
      stage_store_rows_coherent<D, kThreads>(dst + (BQ / 2) * D, t1, BQ / 2, valid - BQ / 2, tid);
      split_publish(counters + slot, tid);
    } else {
      bf16_t* out = dQout + (q_off + q0) * D;
      stage_add_rows<D, kThreads>(out, t0, dst, BQ / 2, valid, scale, tid);
      stage_add_rows<D, kThreads>(out + (BQ / 2) * D, t1, dst + (BQ / 2) * D, BQ / 2, valid - BQ / 2, scale, tid);
    }
  }
}

}  // namespace dq
}  // namespace fabwd

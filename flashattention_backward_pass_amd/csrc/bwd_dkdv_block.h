// bf16 dK / dV work unit on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16):
// the body of bwd_dkdv_kernel (bwd_dkdv.hip); `block` plays the role of the
// block index.
//
// Algorithm: "解析 FlashAttention（3）：FlashAttention-v1 反向传播", section 4
// (Algorithm 4) and the Inference Cookbook page "反向传播算法详解", sections
// 3.1 and 5.2: one workgroup owns a block of 128 keys of one key/value head
// (K_j, V_j stay in registers for the whole loop, dK_j and dV_j accumulate in
// fp32 registers), and loops over the query heads of its GQA group and over
// query blocks of 64 rows.  Per (query block i, key block j):
//   S  = Q_i K_j^T                      (GEMM 1)
//   dP = dO_i V_j^T                     (GEMM 2)
//   P  = exp2(S' tau log2e - LSE log2e), S' = c tanh(S/c) with a cap
//   dS = P o (dP - D) [o (1 - tanh^2)]  rounded to bf16, P rounded to bf16
//   dV += P^T dO_i                      (GEMM 3, FlashAttention-v1 page eq (10))
//   dK += dS^T Q_i                      (GEMM 4, FlashAttention-v1 page eq (16))
// dK is multiplied by tau once in the epilogue (Cookbook 2.1).  dQ is
// produced by the query-block-outer kernel in bwd_dq.hip.
//
// Wave layout (4 waves, wave w owns keys 32w..32w+31 of the block):
//  * GEMM 1/2 produce S, dP with keys on the 32 lanes and queries on the
//    accumulator registers, so that P and dS are already the A operand of
//    GEMM 3/4 (keys x queries) without leaving registers.  The k index of
//    those GEMMs (queries) follows the accumulator's row order; the matching
//    B operand (dO_i, Q_i with queries along k) is read from the row-major
//    LDS tile with the transposing read ds_read_b64_tr_b16.
//  * The S and dP accumulators start from values read out of LDS instead of
//    zero.  S starts at -LSE/tau, so P = exp2(tau log2e * S_acc).  The V
//    slice is held negated and dP starts at +D, so the dP accumulator ends at
//    D - dP and P * acc = -dS; the sign is folded into dK's epilogue scale.
//    Masked positions start S at -inf.  The softmax gradient is one
//    multiply, one exp2 and one multiply per element.
//  * All matrix instructions use VGPR accumulators (the file is built with
//    -mllvm -amdgpu-mfma-vgpr-form); the K_j, V_j slices, only ever read as
//    matrix operands, are pinned to AGPRs.
//
// Pipeline (one barrier per tile of 64 query rows, two LDS buffers):
//   tile t: A(0) | A(1) + B(0) | C(0) + B(1) | C(1)   (see do_tile)
//   the copies of tile t+1 (Q, dO, LSE, D; buffer loads that write LDS
//   directly) are issued between the matrix instructions of A(0); wave 0
//   rescales the LSE of tile t+1 in LDS during C(1); then wait + barrier.
// The loop is unrolled over the two buffers so every LDS offset is a
// compile-time immediate.
//
// Dropout (FlashAttention-v1 page, section 3.3, eqs (10)-(12)): the mask of
// each 32-query half is regenerated during its A stage (the 10 generator
// rounds are spread over the slots; lanes l and l^1 share the calls, see
// philox.h).  The dP accumulator then starts at 0 (acc = -dP~, dP~ = dO V^T),
// and -dS = P (D + Z acc) with Z = 1/(1-p) or 0, D read from LDS one step
// ahead; dV accumulates (P o keep)^T dO and takes the 1/(1-p) in the
// epilogue.
#pragma once

#include <type_traits>

#include "fabwd_launch.h"
#include "mfma_common.h"

namespace fabwd {
namespace dkdv {

constexpr int kThreads = 256;
constexpr int BC = 128;  // keys per workgroup
constexpr int BR = 64;   // query rows per inner iteration

// Waves per SIMD of the kernels that run this work unit.  d = 128 needs the
// whole register file of a SIMD lane (one wave); at d = 64 two workgroups
// share a CU, each wave within 256 registers (all VGPRs: the K, V slices are
// not pinned to AGPRs there), except with both soft cap and dropout, which
// would spill.
template <int D, bool SOFTCAP, bool DROPOUT>
constexpr int kWavesPerSimd = (D == 64 && !(SOFTCAP && DROPOUT)) ? 2 : 1;

// Position in the sequence of query tiles of a workgroup.
struct Cursor {
  int q0;        // first row of the query block
  int64_t row0;  // (b*H + h)*N, row offset of the query head
  int bh;        // b*H + h, the query head (dropout generator counter)
};

// Eight elements (from element i, a multiple of 8) of the head-split sum:
// dK = -tau * sum_sp partial_k[sp], dV = sum_sp partial_v[sp], added in split
// order and rounded to bf16.  The partials are [2][n_split][elems] floats
// (dK planes, then dV planes), elems = B*H_kv*N*D.
__device__ __forceinline__ void split_sum8(const float* __restrict__ part, int n_split, int64_t elems, int64_t i,
                                           bf16_t* __restrict__ dK, bf16_t* __restrict__ dV, float scale) {
  float k[8], v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) k[e] = v[e] = 0.f;
  for (int sp = 0; sp < n_split; ++sp) {
    const f32x4_t* pk = reinterpret_cast<const f32x4_t*>(part + sp * elems + i);
    const f32x4_t* pv = reinterpret_cast<const f32x4_t*>(part + (n_split + sp) * elems + i);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4_t a = pk[h], c = pv[h];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        k[4 * h + e] += a[e];
        v[4 * h + e] += c[e];
      }
    }
  }
  u32x4_t ko, vo;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ko[e] = pack_bf16x2(k[2 * e] * -scale, k[2 * e + 1] * -scale);
    vo[e] = pack_bf16x2(v[2 * e], v[2 * e + 1]);
  }
  *reinterpret_cast<u32x4_t*>(dK + i) = ko;
  *reinterpret_cast<u32x4_t*>(dV + i) = vo;
}

// Key k is visible to query q iff q - wl <= k <= q + wr and k < N (causal:
// wr = 0; an unbounded side is N).
template <int D, bool SOFTCAP, bool DROPOUT>
__device__ __forceinline__ void dkdv_block(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K,
                                           const bf16_t* __restrict__ V, const bf16_t* __restrict__ dO,
                                           const float* __restrict__ LSE, const float* __restrict__ Dv,
                                           bf16_t* __restrict__ dK, bf16_t* __restrict__ dV, int H, int H_kv, int N,
                                           int BH, float scale, float softcap, int wl, int wr, int n_split,
                                           float* __restrict__ part, Dropout drop, unsigned block,
                                           int qhalf = -1, int qblocks = 0, unsigned* counters = nullptr) {
  constexpr int KC = D / 16;  // 16-wide k chunks over d
  constexpr int NT = D / 32;  // 32-wide column tiles over d
  // Double buffers as separate variables: the compiler gives each LDS
  // variable its own alias scope, so reads of one buffer do not wait for the
  // asynchronous copies still landing in the other.  Q and dO of one buffer
  // share a variable (copied and read together): a dO address is then the Q
  // address plus an immediate offset, not a register of its own.
  __shared__ __attribute__((aligned(1024))) uint16_t sQO0[2 * BR * D], sQO1[2 * BR * D];
  uint16_t* const sQ0 = sQO0;
  uint16_t* const sQ1 = sQO1;
  uint16_t* const sdO0 = sQO0 + BR * D;
  uint16_t* const sdO1 = sQO1 + BR * D;
  __shared__ __attribute__((aligned(256))) float sL0[BR], sL1[BR];
  __shared__ __attribute__((aligned(256))) float sD0[BR], sD1[BR];
  __shared__ float sX[4][BR];  // rows rescaled by waves 1-3 in place of the LSE
  auto bufsel = [](auto bufc, auto* a0, auto* a1) {
    if constexpr (decltype(bufc)::value == 0) return a0;
    else return a1;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;  // accumulator column / row group
  const int j16 = lane & 15, h16 = (lane >> 4) & 1;

  // Work unit: (batch*kv-head, key block, head subset).  Key blocks vary
  // slowest so that the heaviest causal blocks (small j) are dispatched first.
  // With n_split > 1 the G query heads of the group are shared out over
  // n_split workgroups, which write fp32 partial sums to `part`.  With
  // qhalf >= 0 (combined launch, n_split == 1) the caller has
  // decoded the unit: `block` is bh + BH * jblk and this workgroup takes half
  // qhalf of the key block's query tiles (0: the later ones, 1: the earlier
  // ones); the two halves hand the tile over through slot bh * qblocks + jblk
  // of `part` (dK then dV, BC x D floats each) and the counter of the same
  // index (split_arrive_first).
  const int unit = block % (BH * n_split);
  const int bh = unit % BH, split = unit / BH;
  const int jblk = block / (BH * n_split);
  const int b = bh / H_kv, hk = bh % H_kv;
  // Query heads [g_lo, g_hi) of the group (of G_full = H / H_kv) belong to
  // this workgroup; with an odd group the later split takes one head more.
  const int G_full = H / H_kv;
  const int g_lo = split * G_full / n_split, g_hi = (split + 1) * G_full / n_split;
  const int G = g_hi - g_lo;  // query heads of this workgroup
  const int k0 = jblk * BC;
  const int64_t kv_off = (int64_t(b) * H_kv + hk) * N;  // row offset of this kv head
  const int kw = w * 32;                                 // this wave's first key in the block
  const int my_key = k0 + kw + l32;                      // key owned by this lane in GEMM 1/2
  // Queries q that see my_key: q - wl <= my_key <= q + wr, q < N, my_key < N.
  const int vq_lo = max(0, my_key - wr);
  const int vq_len = my_key < N ? max(0, min(N - 1, my_key + wl) - vq_lo + 1) : 0;

  // K_j and -V_j slices: B operands of GEMM 1/2, resident for the whole loop.
  // Keys past N read row N-1: their P is masked to 0, so they contribute nothing.
  bf16x8_t kreg[KC], vreg[KC];
  {
    const int64_t row = (kv_off + min(my_key, N - 1)) * D;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      kreg[c] = load_bf16x8(K + row + 16 * c + 8 * g);
      const u32x4_t vb = *reinterpret_cast<const u32x4_t*>(V + row + 16 * c + 8 * g);
      vreg[c] = __builtin_bit_cast(bf16x8_t, vb ^ 0x80008000u);
      // Only matrix instructions read them: keep them in AGPRs (d = 128).
      if (D == 128) {
        asm volatile("" : "+a"(kreg[c]));
        asm volatile("" : "+a"(vreg[c]));
      }
    }
  }

  f32x16_t dk_acc[NT], dv_acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    dk_acc[n] = f32x16_t{};
    dv_acc[n] = f32x16_t{};
  }

  const float zs = scale * kLog2e;
  const float lse_mul = SOFTCAP ? kLog2e : -1.f / scale;
  const float cap_k = SOFTCAP ? 2.f * kLog2e / softcap : 0.f;  // tanh(x / c) = tanh_scaled(x, cap_k)
  const float cap_zs = softcap * zs;
  // Query blocks [i_lo, i_hi) hold every row that sees a key of this block.
  const int k_end = min(k0 + BC, N);
  int i_lo = max(0, k0 - wr) / BR;
  int i_hi = (min(N, k_end + wl) + BR - 1) / BR;
  if (qhalf >= 0) {
    const int mid = (i_lo + i_hi + 1) / 2;
    if (qhalf == 0) i_lo = mid;
    else i_hi = mid;
  }
  const int n_iter = (i_hi - i_lo) * G;
  const bool ragged_keys = k0 + BC > N;
  const int q_last = (i_hi - 1) * BR;  // first row of the last query block visited

  // Tiles run over the query heads of the group and, within a head, over the
  // query blocks from the last one down (concurrent workgroups of a head sweep
  // the same rows together).  A cursor steps through that sequence without
  // divisions; one cursor feeds the copies, one the compute.
  const int64_t head0 = (int64_t(b) * H + hk * G_full + g_lo) * N;
  auto advance = [&](Cursor& c) {
    if (c.q0 == i_lo * BR) {
      c.q0 = q_last;
      c.row0 += N;
      ++c.bh;
    } else {
      c.q0 -= BR;
    }
  };

  // Per-lane byte offsets of the tile copy: slab I = s*4 + w covers rows
  // I*RPS .. I*RPS + RPS - 1; lane L fills physical chunk L % (D/8) of row
  // I*RPS + L / (D/8), i.e. logical chunk (L % (D/8)) ^ swz(row).  Each copy's
  // buffer descriptor spans only the tile's valid rows: reads past N return
  // zeros (rows that are masked anyway), and the LDS tiles start zeroed.
  constexpr int RPS = 1024 / (2 * D);  // rows per 1 KB slab
  constexpr int NSLAB = BR / RPS / 4;  // slabs per wave and tensor
  constexpr int NDMA = 2 * NSLAB + 1;  // copies per wave and tile (Q, dO, LSE or D)
  int voff[NSLAB];
#pragma unroll
  for (int s = 0; s < NSLAB; ++s) {
    const int row = (s * 4 + w) * RPS + lane / (D / 8);
    voff[s] = (row * D + 8 * ((lane % (D / 8)) ^ swz<D>(row))) * 2;
  }

  // Copy k (0 .. NDMA-1) of the tile at cursor c into buffer BUF.  Each
  // buffer descriptor spans the tile's valid rows of Q, dO, and LSE (wave 0)
  // or D (wave 1).  (The buffer builtins get plain local values: an array
  // element written directly as an argument makes the host compilation
  // silently drop the kernel.)
  auto copy_one = [&](auto bufc, const Cursor& c, int k) {
    const int rows = min(BR, N - c.q0);
    const int64_t r0 = c.row0 + c.q0;
    if (k < 2 * NSLAB) {
      const int s = k % NSLAB;
      const int vo = voff[s];
      const bf16_t* src = k < NSLAB ? Q : dO;
      uint16_t* dst = k < NSLAB ? bufsel(bufc, sQ0, sQ1) : bufsel(bufc, sdO0, sdO1);
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)(src + r0 * D), 0, rows * D * 2, 0x00020000);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)&dst[(s * 4 + w) * 512], 16, vo, 0, 0, 0);
    } else if (w < 2) {
      const __amdgpu_buffer_rsrc_t r =
          __builtin_amdgcn_make_buffer_rsrc((void*)((w == 0 ? LSE : Dv) + r0), 0, rows * 4, 0x00020000);
      float* dst = w == 0 ? bufsel(bufc, sL0, sL1) : bufsel(bufc, sD0, sD1);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)dst, 4, lane * 4, 0, 0, 0);
    }
  };
  // Once its copy of the LSE into buffer BUF has landed, wave 0 turns it into
  // -LSE/tau in place (LSE log2e with a soft cap), published by the next
  // barrier.  Waves 1-3 run the same instructions on a row of their own, so
  // there is no branch.
  auto prescale = [&](auto bufc) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    float* l = w == 0 ? bufsel(bufc, sL0, sL1) : &sX[w][0];
    l[lane] *= lse_mul;
  };

  // Per-lane LDS offsets (elements), fixed for the whole loop; the half,
  // the buffer and the 16-row step add compile-time constants.
  //  * row reads (A operand of S, dP): row l32, logical chunk 2c + g;
  //  * transposing reads (B operand of dV, dK): row 4g + j16/4 (+8), logical
  //    chunk 4n + 2 h16 + (j16 % 4)/2, element 4 (j16 % 2) within the chunk.
  // The swizzle only depends on the row modulo 16, so rows +16 and +32 share it.
  int off_a[KC], off_t[NT][2];
#pragma unroll
  for (int c = 0; c < KC; ++c) off_a[c] = swz_off<D>(l32, 2 * c + g, 0);
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int ch = 4 * n + 2 * h16 + ((j16 & 3) >> 1);
#pragma unroll
    for (int v = 0; v < 2; ++v) off_t[n][v] = swz_off<D>(4 * g + (j16 >> 2) + 8 * v, ch, 4 * (j16 & 1));
  }

  // One tile of 64 query rows in two halves h = 0, 1 of 32 rows:
  //   A(h): S_h, dP_h accumulate over d (2 MFMAs per 16-wide chunk of d)
  //   B(h): P and dS of half h, packed to bf16 (VALU)
  //   C(h): dV += P_h^T dO_h, dK += dS_h^T Q_h (2 MFMAs per (u, n) step)
  // issued as A(0) | A(1) + B(0) | C(0) + B(1) | C(1), so the softmax
  // gradient of one half runs under the matrix instructions of the other.
  // Each stage is a fixed sequence of slots (2 MFMAs, the LDS reads for a
  // later slot, a share of the other work) separated by scheduling barriers,
  // so the compiler keeps this order and its register use stays bounded.
  // `next` is the tile whose copies go out during A(0), into the other buffer.
  auto do_tile = [&](auto bufc, int q0, int bh, bool masked, const Cursor& next) {
    using NB = std::integral_constant<int, 1 - decltype(bufc)::value>;
    const uint16_t* tq_ = bufsel(bufc, sQ0, sQ1);
    const uint16_t* to_ = bufsel(bufc, sdO0, sdO1);
    const float* sl_ = bufsel(bufc, sL0, sL1);
    const float* sd_ = bufsel(bufc, sD0, sD1);
    auto rowop = [&](const uint16_t* t, int h, int c) {
      return *reinterpret_cast<const bf16x8_t*>(&t[off_a[c] + 32 * h * D]);
    };
    auto trop = [&](const uint16_t* t, int h, int u, int n) {
      return cat8(lds_read_tr(&t[off_t[n][0] + (32 * h + 16 * u) * D]),
                  lds_read_tr(&t[off_t[n][1] + (32 * h + 16 * u) * D]));
    };
    auto acc_init = [&](const float* src, int h) {
      f32x16_t a;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(&src[32 * h + 8 * m + 4 * g]);
        a[4 * m] = v[0];
        a[4 * m + 1] = v[1];
        a[4 * m + 2] = v[2];
        a[4 * m + 3] = v[3];
      }
      return a;
    };
    // Masked tiles: positions outside the causal triangle or past N start S
    // at -inf (so P = exp2(-inf) = 0 and dS = 0); with a soft cap the
    // subtracted LSE becomes +inf instead.  Applied to the initial values only.
    // The queries that see this lane's key form one range [vq_lo, vq_lo +
    // vq_len) (empty past N), so the test is one unsigned compare per element
    // (a chain of compares was compiled into a branch per element).
    auto mask_init = [&](f32x16_t& a, int h) {
      const float fill = SOFTCAP ? __builtin_inff() : -__builtin_inff();
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qg = q0 + 32 * h + 8 * (r >> 2) + 4 * g + (r & 3);
        a[r] = unsigned(qg - vq_lo) < unsigned(vq_len) ? a[r] : fill;
      }
    };
    // The softmax gradient of one element in three steps, software-pipelined
    // over the slots of a stage (slot i runs step 1 of its elements, step 2 of
    // the previous slot's and step 3 of the one before), so consecutive VALU
    // instructions are independent.
    //   1: t = S_acc * tau log2e  (cap: t = c tanh(S/c) tau log2e - LSE log2e)
    //   2: P = exp2(t)
    //   3: -dS = P * dP_acc [* (1 - tanh^2)]; bf16 pairs packed
    auto step1 = [&](f32x16_t& sa, f32x16_t& la, int r) {
      if (SOFTCAP) {
        const float th = tanh_scaled(sa[r], cap_k);
        sa[r] = fmaf(cap_zs, th, -la[r]);
        la[r] = fmaf(-th, th, 1.f);
      } else {
        sa[r] = sa[r] * zs;
      }
    };
    // With dropout, step 2 also fetches D of the element's query row.
    auto step2 = [&](f32x16_t& sa, f32x16_t& dd, int h, int r) {
      sa[r] = fast_exp2(sa[r]);
      if (DROPOUT) dd[r] = sd_[32 * h + 8 * (r >> 2) + 4 * g + (r & 3)];
    };
    auto step3 = [&](f32x16_t& sa, f32x16_t& da, const f32x16_t& la, const f32x16_t& dd, const DropBits& kb,
                     u32x4_t* pw, u32x4_t* dw, int r) {
      float ds;
      if (DROPOUT) {
        const bool kp = kb.keep(r, drop.keep_t);
        ds = sa[r] * fmaf(kp ? drop.scale : 0.f, da[r], dd[r]);
        sa[r] = kp ? sa[r] : 0.f;
      } else {
        ds = sa[r] * da[r];
      }
      if (SOFTCAP) ds *= la[r];
      da[r] = ds;
      if (r & 1) {
        pw[r >> 3][(r & 7) >> 1] = pack_bf16x2(sa[r - 1], sa[r]);
        dw[r >> 3][(r & 7) >> 1] = pack_bf16x2(da[r - 1], ds);
      }
    };
    // Pipeline position `slot` of a stage with E elements per slot; slots past
    // the stage's own (16 / E) only drain steps 2 and 3.
    auto sm_slot = [&](f32x16_t& sa, f32x16_t& da, f32x16_t& la, f32x16_t& dd, const DropBits& kb, int h,
                       u32x4_t* pw, u32x4_t* dw, int E, int slot) {
      const int ns = 16 / E;
      if (slot < ns)
        for (int e = 0; e < E; ++e) step1(sa, la, E * slot + e);
      if (slot >= 1 && slot - 1 < ns)
        for (int e = 0; e < E; ++e) step2(sa, dd, h, E * (slot - 1) + e);
      if (slot >= 2 && slot - 2 < ns)
        for (int e = 0; e < E; ++e) step3(sa, da, la, dd, kb, pw, dw, E * (slot - 2) + e);
    };
    // Mask generator of one half: init, then rounds spread over the KC slots
    // of its A stage, then the lane-pair exchange.
    DropKeyLane gen;
    DropBits kb0, kb1;
    f32x16_t dd0, dd1;
    auto gen_slot = [&](int c) {
      if (DROPOUT) gen.rounds(10 * c / KC, 10 * (c + 1) / KC);
    };

    constexpr int PF = 2;              // row-operand prefetch distance (chunks)
    constexpr int EA = 16 / KC;        // softmax elements per A slot
    constexpr int EC = 16 / (2 * NT);  // softmax elements per C slot
    f32x16_t s0, d0, s1, d1, l0 = {}, l1 = {};
    u32x4_t pw0[2], dw0[2], pw1[2], dw1[2];
    bf16x8_t qa[KC], oa[KC];

    // ---- A(0), with the copies of the next tile ----
    s0 = SOFTCAP ? f32x16_t{} : acc_init(sl_, 0);
    if (SOFTCAP) l0 = acc_init(sl_, 0);
    d0 = DROPOUT ? f32x16_t{} : acc_init(sd_, 0);
    if (DROPOUT) gen.init(drop, uint32_t(bh), q0, my_key, lane);
    if (masked) mask_init(SOFTCAP ? l0 : s0, 0);
#pragma unroll
    for (int c = 0; c < PF; ++c) {
      qa[c] = rowop(tq_, 0, c);
      oa[c] = rowop(to_, 0, c);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      if (c + PF < KC) {
        qa[c + PF] = rowop(tq_, 0, c + PF);
        oa[c + PF] = rowop(to_, 0, c + PF);
      } else {
        // The first chunks of half 1.
        const int c1 = c + PF - KC;
        qa[c1] = rowop(tq_, 1, c1);
        oa[c1] = rowop(to_, 1, c1);
      }
      s0 = mfma32(qa[c], kreg[c], s0);
      d0 = mfma32(oa[c], vreg[c], d0);
#pragma unroll
      for (int k = c; k < NDMA; k += KC) copy_one(NB{}, next, k);
      gen_slot(c);
      __builtin_amdgcn_sched_barrier(0);
    }
    s1 = SOFTCAP ? f32x16_t{} : acc_init(sl_, 1);
    if (SOFTCAP) l1 = acc_init(sl_, 1);
    d1 = DROPOUT ? f32x16_t{} : acc_init(sd_, 1);
    if (masked) mask_init(SOFTCAP ? l1 : s1, 1);
    __builtin_amdgcn_sched_barrier(0);

    // ---- A(1) + B(0) ----
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      if (c + PF < KC) {
        qa[c + PF] = rowop(tq_, 1, c + PF);
        oa[c + PF] = rowop(to_, 1, c + PF);
      }
      s1 = mfma32(qa[c], kreg[c], s1);
      d1 = mfma32(oa[c], vreg[c], d1);
      if (DROPOUT && c == 0) {
        kb0 = gen.finish(lane);
        gen.init(drop, uint32_t(bh), q0 + 32, my_key, lane);
      }
      gen_slot(c);
      sm_slot(s0, d0, l0, dd0, kb0, 0, pw0, dw0, EA, c);
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- C(0) + B(1) ----  slot i: u = i / NT, n = i % NT
    bf16x8_t ob[2], qb[2];
    ob[0] = trop(to_, 0, 0, 0);
    qb[0] = trop(tq_, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 2 * NT; ++i) {
      const int u = i / NT, n = i % NT;
      if (i + 1 < 2 * NT) {
        ob[(i + 1) & 1] = trop(to_, 0, (i + 1) / NT, (i + 1) % NT);
        qb[(i + 1) & 1] = trop(tq_, 0, (i + 1) / NT, (i + 1) % NT);
      } else {
        ob[(i + 1) & 1] = trop(to_, 1, 0, 0);
        qb[(i + 1) & 1] = trop(tq_, 1, 0, 0);
      }
      dv_acc[n] = mfma32(__builtin_bit_cast(bf16x8_t, pw0[u]), ob[i & 1], dv_acc[n]);
      dk_acc[n] = mfma32(__builtin_bit_cast(bf16x8_t, dw0[u]), qb[i & 1], dk_acc[n]);
      // Drain B(0) in the first two slots; B(1) runs alongside.
      if (DROPOUT && i == 0) kb1 = gen.finish(lane);
      if (i < 2) sm_slot(s0, d0, l0, dd0, kb0, 0, pw0, dw0, EA, KC + i);
      sm_slot(s1, d1, l1, dd1, kb1, 1, pw1, dw1, EC, i);
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- C(1) ----  (2 NT is even: slot i reads buffer i & 1 again)
#pragma unroll
    for (int i = 0; i < 2 * NT; ++i) {
      const int u = i / NT, n = i % NT;
      if (i + 1 < 2 * NT) {
        ob[(i + 1) & 1] = trop(to_, 1, (i + 1) / NT, (i + 1) % NT);
        qb[(i + 1) & 1] = trop(tq_, 1, (i + 1) / NT, (i + 1) % NT);
      }
      dv_acc[n] = mfma32(__builtin_bit_cast(bf16x8_t, pw1[u]), ob[i & 1], dv_acc[n]);
      dk_acc[n] = mfma32(__builtin_bit_cast(bf16x8_t, dw1[u]), qb[i & 1], dk_acc[n]);
      if (i < 2) sm_slot(s1, d1, l1, dd1, kb1, 1, pw1, dw1, EC, 2 * NT + i);
      if (i == 2) prescale(NB{});
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  // Zero the tiles once, so rows past N (never copied) hold finite values.
  {
    const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = tid; i < BR * D / 8; i += kThreads) {
      reinterpret_cast<u32x4_t*>(sQ0)[i] = z;
      reinterpret_cast<u32x4_t*>(sQ1)[i] = z;
      reinterpret_cast<u32x4_t*>(sdO0)[i] = z;
      reinterpret_cast<u32x4_t*>(sdO1)[i] = z;
    }
    if (tid < BR) {
      sL0[tid] = sL1[tid] = sD0[tid] = sD1[tid] = 0.f;
    }
    __syncthreads();
  }
  Cursor cc{q_last, head0, int(b) * H + hk * G_full + g_lo};  // tile being computed
  Cursor ci = cc;            // tile being copied
  if (n_iter > 0) {
#pragma unroll
    for (int k = 0; k < NDMA; ++k) copy_one(B0{}, ci, k);
    prescale(B0{});
  }
  advance(ci);
  auto tile = [&](auto bufc, int t) {
    // Unmasked: every key of the block is visible to every row of the tile.
    const bool masked = ragged_keys || cc.q0 + BR > N || k0 < cc.q0 + BR - 1 - wl || k0 + BC - 1 > cc.q0 + wr;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // tile t in this buffer; the other buffer no longer read
    // After the last tile the copy repeats the current tile into the idle
    // buffer, which nothing reads: no branch around the copies.
    do_tile(bufc, cc.q0, cc.bh, masked, t + 1 < n_iter ? ci : cc);
    advance(ci);
    advance(cc);
  };
  for (int t = 0; t < n_iter; t += 2) {
    tile(B0{}, t);
    if (t + 1 < n_iter) tile(B1{}, t + 1);
  }

  // Epilogue: dK = -tau * dK_acc (the accumulator holds -dS^T Q), dV = dV_acc
  // (rows = keys, columns = d), staged through the idle Q/dO tiles so that the
  // global writes are 16-byte row chunks.  With a head split the raw fp32
  // accumulators go to `part` ([2][n_split][B*H_kv*N][D]: dK partials, then dV
  // partials), one tensor at a time (a 128 x D fp32 tile fills both buffers).
  // Rows past N are not written.
  const int64_t plane = int64_t(BH) * N * D;
  const float v_scale = DROPOUT ? drop.scale : 1.f;  // dV sums P o keep; Z = keep / (1 - p)
  const int valid = min(BC, N - k0);
  // The last tile's copies (into the idle buffer) must land before the tiles are reused.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();  // every wave is done with the Q/dO tiles
  if (n_split == 1 && qhalf < 0) {
    bf16_t* tk = reinterpret_cast<bf16_t*>(sQO0);  // BC x D bf16 = the size of one buffer
    bf16_t* tv = reinterpret_cast<bf16_t*>(sQO1);
    stage_acc<bf16_t, NT, D>(tk, kw, dk_acc, -scale, lane);
    stage_acc<bf16_t, NT, D>(tv, kw, dv_acc, v_scale, lane);
    __syncthreads();
    stage_copy_rows<bf16_t, D, kThreads>(dK + (kv_off + k0) * D, tk, BC, valid, tid);
    stage_copy_rows<bf16_t, D, kThreads>(dV + (kv_off + k0) * D, tv, BC, valid, tid);
  } else {
    // 128 x D fp32 = both buffers: rows 0-63 in buffer 0, rows 64-127 in buffer 1.
    float* t0 = reinterpret_cast<float*>(sQO0);
    float* t1 = reinterpret_cast<float*>(sQO1);
    float* tw = w < 2 ? t0 : t1;
    const int row0 = kw - (w < 2 ? 0 : BC / 2);
    // Head split: the raw partials go to their planes.  Query-range split:
    // the first half to finish writes its partials to the unit's slot, the
    // second adds them to its own and writes dK, dV.
    __shared__ unsigned s_arrival;
    const int64_t slot = int64_t(bh) * qblocks + jblk;
    const bool to_part = qhalf < 0 || split_arrive_first(counters + slot, &s_arrival, tid);
    float* dst_k;
    float* dst_v;
    if (qhalf >= 0) {
      dst_k = part + slot * (2 * BC * D);
      dst_v = dst_k + BC * D;
      if (!to_part) split_wait(counters + slot, tid);
    } else {
      dst_k = part + split * plane + (kv_off + k0) * D;
      dst_v = part + (n_split + split) * plane + (kv_off + k0) * D;
    }
#pragma unroll
    for (int tensor = 0; tensor < 2; ++tensor) {
      stage_acc<float, NT, D>(tw, row0, tensor == 0 ? dk_acc : dv_acc, tensor == 0 ? 1.f : v_scale, lane);
      __syncthreads();
      float* dst = tensor == 0 ? dst_k : dst_v;
      if (to_part && qhalf < 0) {
        stage_copy_rows<float, D, kThreads>(dst, t0, BC / 2, valid, tid);
        stage_copy_rows<float, D, kThreads>(dst + (BC / 2) * D, t1, BC / 2, valid - BC / 2, tid);
      } else if (to_part) {
        stage_store_rows_coherent<D, kThreads>(dst, t0, BC / 2, valid, tid);
        stage_store_rows_coherent<D, kThreads>(dst + (BC / 2) * D, t1, BC / 2, valid - BC / 2, tid);
      } else {
        bf16_t* out = (tensor == 0 ? dK : dV) + (kv_off + k0) * D;
        const float mul = tensor == 0 ? -scale : 1.f;
        stage_add_rows<D, kThreads>(out, t0, dst, BC / 2, valid, mul, tid);
        stage_add_rows<D, kThreads>(out + (BC / 2) * D, t1, dst + (BC / 2) * D, BC / 2, valid - BC / 2, mul, tid);
      }
      __syncthreads();
    }
    if (qhalf >= 0 && to_part) split_publish(counters + slot, tid);
  }
}

}  // namespace dkdv
}  // namespace fabwd

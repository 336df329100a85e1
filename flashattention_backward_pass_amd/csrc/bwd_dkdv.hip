// bf16 dK / dV kernel on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
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
//  * GEMM 1-4 run in two halves of 32 queries, so that only one 32x32 S and
//    dP accumulator pair is live at a time.
//  * K_j, V_j and the dK, dV accumulators are pinned to AGPRs (empty asm
//    statements with an AGPR constraint): only matrix instructions touch them,
//    and the VGPRs stay free for the softmax-gradient work without spills.
//
// Pipeline (one barrier per tile of 64 query rows):
//   wait for tile t in LDS buffer t%2; barrier
//   copy tile t+1 (Q, dO, LSE, D) global -> LDS buffer (t+1)%2 with buffer
//   loads that write LDS directly (scalar tile offsets, no address VALU work)
//   GEMM 1/2, softmax gradient, GEMM 3/4 of tile t
//   wave 0 rescales the LSE of tile t+1 by log2(e) in LDS once it has landed
// The loop is unrolled over the two buffers so every LDS offset is a
// compile-time immediate.
#include <type_traits>

#include "fabwd_launch.h"
#include "mfma_common.h"

namespace fabwd {

namespace {

constexpr int kThreads = 256;
constexpr int BC = 128;  // keys per workgroup
constexpr int BR = 64;   // query rows per inner iteration

template <int D, bool CAUSAL, bool SOFTCAP>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const bf16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    bf16_t* __restrict__ dK, bf16_t* __restrict__ dV, int H, int H_kv, int N, int BH, float scale,
    float softcap) {
  constexpr int KC = D / 16;  // 16-wide k chunks over d
  constexpr int NT = D / 32;  // 32-wide column tiles over d
  __shared__ __attribute__((aligned(1024))) uint16_t sQ[2][BR * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sdO[2][BR * D];
  __shared__ __attribute__((aligned(256))) float sL[2][BR];
  __shared__ __attribute__((aligned(256))) float sD[2][BR];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;  // accumulator column / row group
  const int j16 = lane & 15, h16 = (lane >> 4) & 1;

  // Work unit: (batch*kv-head, key block).  Key blocks vary slowest so that
  // the heaviest causal blocks (small j) are dispatched first.
  const int bh = blockIdx.x % BH;
  const int jblk = blockIdx.x / BH;
  const int b = bh / H_kv, hk = bh % H_kv;
  const int G = H / H_kv;
  const int k0 = jblk * BC;
  const int64_t kv_off = (int64_t(b) * H_kv + hk) * N;  // row offset of this kv head
  const int kw = w * 32;                                 // this wave's first key in the block
  const int my_key = k0 + kw + l32;                      // key owned by this lane in GEMM 1/2

  // K_j, V_j slices: B operands of GEMM 1/2, resident for the whole loop.
  // Keys past N read row N-1: their P is masked to 0, so they contribute nothing.
  bf16x8_t kreg[KC], vreg[KC];
  {
    const int64_t row = (kv_off + min(my_key, N - 1)) * D;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      kreg[c] = load_bf16x8(K + row + 16 * c + 8 * g);
      vreg[c] = load_bf16x8(V + row + 16 * c + 8 * g);
      // Only matrix instructions read K_j and V_j: keep them in AGPRs.
      asm volatile("" : "+a"(kreg[c]));
      asm volatile("" : "+a"(vreg[c]));
    }
  }

  f32x16_t dk_acc[NT], dv_acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    dk_acc[n] = f32x16_t{};
    dv_acc[n] = f32x16_t{};
    // dK, dV accumulate in AGPRs, leaving the VGPRs to the softmax-gradient work.
    asm volatile("" : "+a"(dk_acc[n]));
    asm volatile("" : "+a"(dv_acc[n]));
  }

  const float zs = scale * kLog2e;
  const int n_qblk = (N + BR - 1) / BR;
  const int i_first = CAUSAL ? (k0 / BR) : 0;
  const int per_head = n_qblk - i_first;
  const int n_iter = per_head * G;
  const bool ragged_keys = k0 + BC > N;

  // Tile t of the flattened (query head, query block) sequence; query blocks
  // run from the last one down, so concurrent workgroups of a head sweep the
  // same rows together.
  auto tile_q0 = [&](int t) { return (n_qblk - 1 - t % per_head) * BR; };
  auto tile_qoff = [&](int t) { return (int64_t(b) * H + hk * G + t / per_head) * N; };

  // Per-lane byte offsets of the tile copy: slab I = s*4 + w covers rows
  // I*RPS .. I*RPS + RPS - 1; lane L fills physical chunk L % (D/8) of row
  // I*RPS + L / (D/8), i.e. logical chunk (L % (D/8)) ^ swz(row).
  constexpr int RPS = 1024 / (2 * D);          // rows per 1 KB slab
  constexpr int NSLAB = BR / RPS / 4;          // slabs per wave
  int dma_row[NSLAB], dma_col[NSLAB];
#pragma unroll
  for (int s = 0; s < NSLAB; ++s) {
    const int row = (s * 4 + w) * RPS + lane / (D / 8);
    dma_row[s] = row;
    dma_col[s] = 8 * ((lane % (D / 8)) ^ swz<D>(row));
  }

  auto issue_tile = [&](auto bufc, int t) {
    constexpr int buf = decltype(bufc)::value;
    const int q0 = tile_q0(t);
    const int64_t qoff = tile_qoff(t);
    const int rows = min(BR, N - q0);
    // Buffer resources over this tile's rows only; a ragged tile clamps its
    // rows to the last valid one so every read stays inside the tensor.
    const __amdgpu_buffer_rsrc_t rq =
        __builtin_amdgcn_make_buffer_rsrc((void*)(Q + (qoff + q0) * D), 0, rows * D * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t ro =
        __builtin_amdgcn_make_buffer_rsrc((void*)(dO + (qoff + q0) * D), 0, rows * D * 2, 0x00020000);
#pragma unroll
    for (int s = 0; s < NSLAB; ++s) {
      const int row = rows == BR ? dma_row[s] : min(dma_row[s], rows - 1);
      const int voff = (row * D + dma_col[s]) * 2;
      lds_void_t* dq = (lds_void_t*)&sQ[buf][(s * 4 + w) * 512];
      lds_void_t* dd = (lds_void_t*)&sdO[buf][(s * 4 + w) * 512];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, dq, 16, voff, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ro, dd, 16, voff, 0, 0, 0);
    }
    if (w < 2) {
      const float* src = (w == 0 ? LSE : Dv) + qoff + q0;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, rows * 4, 0x00020000);
      lds_void_t* dst = (lds_void_t*)(w == 0 ? &sL[buf][0] : &sD[buf][0]);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 4, min(lane, rows - 1) * 4, 0, 0, 0);
    }
  };
  // Wave 0: once the LSE of buffer BUF has landed, turn it into LSE * log2(e)
  // in place (published to the other waves by the next barrier).
  auto prescale_lse = [&](auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    if (w == 0) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      sL[buf][lane] *= kLog2e;
    }
  };

  // Softmax gradient of 32 queries (rows qbase..qbase+31 of the tile):
  // s_acc <- P, dp_acc <- dS (both fp32).
  auto softmax_grad = [&](f32x16_t& s_acc, f32x16_t& dp_acc, int buf, int q0, int qbase, bool masked) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int qr = qbase + 8 * m + 4 * g;
      const f32x4_t l4 = *reinterpret_cast<const f32x4_t*>(&sL[buf][qr]);
      const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(&sD[buf][qr]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * m + e;
        float s = s_acc[r];
        float dt = 1.f;
        if (SOFTCAP) {
          const float th = tanh_f32(s / softcap);
          s = softcap * th;
          dt = 1.f - th * th;
        }
        float p = fast_exp2(fmaf(s, zs, -l4[e]));
        if (masked) {
          const int qg = q0 + qr + e;
          if (my_key >= N || qg >= N || (CAUSAL && my_key > qg)) p = 0.f;
        }
        s_acc[r] = p;
        float ds = p * (dp_acc[r] - d4[e]);
        if (SOFTCAP) ds *= dt;
        dp_acc[r] = ds;
      }
    }
  };

  auto do_tile = [&](auto bufc, int t) {
    constexpr int buf = decltype(bufc)::value;
    const int q0 = tile_q0(t);
    const bool masked = (CAUSAL && q0 < k0 + BC) || ragged_keys || q0 + BR > N;
#pragma unroll
    for (int tq = 0; tq < 2; ++tq) {
      // GEMM 1, 2: S and dP for queries 32 tq .. 32 tq + 31 x this wave's 32 keys.
      f32x16_t s_acc = {}, dp_acc = {};
      const int row = 32 * tq + l32;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const int off = swz_off<D>(row, 2 * c + g, 0);
        const bf16x8_t qa = *reinterpret_cast<const bf16x8_t*>(&sQ[buf][off]);
        const bf16x8_t oa = *reinterpret_cast<const bf16x8_t*>(&sdO[buf][off]);
        s_acc = mfma32(qa, kreg[c], s_acc);
        dp_acc = mfma32(oa, vreg[c], dp_acc);
      }
      // P and dS.  Accumulator register r holds query 32 tq + 8(r/4) + 4g + r%4, key my_key.
      if (masked)
        softmax_grad(s_acc, dp_acc, buf, q0, 32 * tq, true);
      else
        softmax_grad(s_acc, dp_acc, buf, q0, 32 * tq, false);
      // bf16 A operands: chunk u (16 queries) = registers 8u..8u+7.
      bf16x8_t pf[2], dsf[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        pf[u] = pack_bf16x8(s_acc, 8 * u);
        dsf[u] = pack_bf16x8(dp_acc, 8 * u);
      }
      // GEMM 3, 4: dV += P^T dO_i, dK += dS^T Q_i over these 32 queries.
      // B operand rows (queries) 32 tq + 16u + 4g + (0..3) and +8, read transposed.
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const int ch = 4 * n + 2 * h16 + ((j16 & 3) >> 1);
        const int sub = 4 * (j16 & 1);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int r0 = 32 * tq + 16 * u + 4 * g + (j16 >> 2);
          const int o0 = swz_off<D>(r0, ch, sub), o1 = swz_off<D>(r0 + 8, ch, sub);
          const bf16x8_t ob = cat8(lds_read_tr(&sdO[buf][o0]), lds_read_tr(&sdO[buf][o1]));
          const bf16x8_t qb = cat8(lds_read_tr(&sQ[buf][o0]), lds_read_tr(&sQ[buf][o1]));
          dv_acc[n] = mfma32(pf[u], ob, dv_acc[n]);
          dk_acc[n] = mfma32(dsf[u], qb, dk_acc[n]);
        }
        asm volatile("" : "+a"(dv_acc[n]));
        asm volatile("" : "+a"(dk_acc[n]));
      }
    }
  };

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  issue_tile(B0{}, 0);
  prescale_lse(B0{});
  for (int t = 0; t < n_iter; t += 2) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // tile t in buffer 0; buffer 1 no longer read
    if (t + 1 < n_iter) issue_tile(B1{}, t + 1);
    do_tile(B0{}, t);
    if (t + 1 < n_iter) {
      prescale_lse(B1{});
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();  // tile t+1 in buffer 1; buffer 0 no longer read
      if (t + 2 < n_iter) issue_tile(B0{}, t + 2);
      do_tile(B1{}, t + 1);
      if (t + 2 < n_iter) prescale_lse(B0{});
    }
  }

  // Epilogue: dK = tau * dK_acc, dV = dV_acc (rows = keys, lanes = d).
#pragma unroll
  for (int n = 0; n < NT; ++n) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + kw + 8 * (r >> 2) + 4 * g + (r & 3);
      if (key < N) {
        const int64_t off = (kv_off + key) * D + 32 * n + l32;
        dK[off].bits = f32_to_bf16(dk_acc[n][r] * scale);
        dV[off].bits = f32_to_bf16(dv_acc[n][r]);
      }
    }
  }
}

template <int D, bool CAUSAL, bool SOFTCAP>
hipError_t dkdv_t(const Problem& p, const void* Q, const void* K, const void* V, const void* dO, const float* LSE,
                  const float* Dv, void* dK, void* dV, hipStream_t s) {
  const int BH = p.B * p.H_kv;
  const int n_kblk = (p.N + BC - 1) / BC;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, SOFTCAP>), dim3(unsigned(BH) * unsigned(n_kblk)), dim3(kThreads),
                     0, s, static_cast<const bf16_t*>(Q), static_cast<const bf16_t*>(K),
                     static_cast<const bf16_t*>(V), static_cast<const bf16_t*>(dO), LSE, Dv,
                     static_cast<bf16_t*>(dK), static_cast<bf16_t*>(dV), p.H, p.H_kv, p.N, BH, p.scale, p.softcap);
  return hipGetLastError();
}

template <int D>
hipError_t dkdv_d(const Problem& p, const void* Q, const void* K, const void* V, const void* dO, const float* LSE,
                  const float* Dv, void* dK, void* dV, hipStream_t s) {
  const bool sc = p.softcap > 0.f;
  if (p.causal) return sc ? dkdv_t<D, true, true>(p, Q, K, V, dO, LSE, Dv, dK, dV, s)
                          : dkdv_t<D, true, false>(p, Q, K, V, dO, LSE, Dv, dK, dV, s);
  return sc ? dkdv_t<D, false, true>(p, Q, K, V, dO, LSE, Dv, dK, dV, s)
            : dkdv_t<D, false, false>(p, Q, K, V, dO, LSE, Dv, dK, dV, s);
}

}  // namespace

hipError_t launch_bwd_dkdv_mfma(const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                                const float* LSE, const float* Dv, void* dK, void* dV, hipStream_t s) {
  return p.d == 64 ? dkdv_d<64>(p, Q, K, V, dO, LSE, Dv, dK, dV, s)
                   : dkdv_d<128>(p, Q, K, V, dO, LSE, Dv, dK, dV, s);
}

}  // namespace fabwd

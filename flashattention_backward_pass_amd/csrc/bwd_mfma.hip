// bf16 backward kernel on gfx950 matrix cores (v_mfma_f32_32x32x16_bf16).
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
//   dV += P^T dO_i                      (GEMM 3)
//   dK += dS^T Q_i                      (GEMM 4)
//   dQaccum[i] += dS K_j                (GEMM 5, fp32 atomics; Cookbook 6.2)
// dK is multiplied by tau once in the epilogue (Cookbook 2.1); dQ's tau is
// applied by the convert kernel.
//
// Wave layout (4 waves, wave w owns keys 32w..32w+31 of the block):
//  * GEMM 1/2 produce S, dP with keys on the 32 lanes and queries on the
//    accumulator registers, so that P and dS are already the A operand of
//    GEMM 3/4 (keys x queries) without leaving registers.  The k index of
//    those GEMMs (queries) follows the accumulator's row order; the matching
//    B operand (dO_i, Q_i with queries along k) is read from the row-major
//    LDS tile with the gfx950 transposing read ds_read_b64_tr_b16.
//  * GEMM 5 needs dS with queries on lanes: dS is written to LDS transposed
//    (keys x queries, 8-byte writes from the accumulator layout) and read back
//    with the transposing read.  Wave w computes dQ columns 32w..32w+31
//    (d = 128) or one 32x32 quadrant (d = 64) over all 128 keys; its slice of
//    K^T is held in registers for the whole loop.
#include "fabwd_device.h"
#include "fabwd_launch.h"

namespace fabwd {

namespace {

typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

constexpr int kThreads = 256;
constexpr int BC = 128;  // keys per workgroup
constexpr int BR = 64;   // query rows per inner iteration

template <int D>
struct Cfg {
  static constexpr int QP = D + 8;   // LDS row pitch (elements) of the Q and dO tiles
  static constexpr int SP = BR + 8;  // LDS row pitch (elements) of the transposed dS tile
  static constexpr int KC = D / 16;  // 16-wide k chunks over d
  static constexpr int NT = D / 32;  // 32-wide column tiles over d
  static constexpr int QT = D == 128 ? 2 : 1;  // dQ row tiles per wave
};

__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Transposing LDS read: within each 16-lane group, lane x supplies the address
// of 4 consecutive bf16 (8 bytes); lane j receives element j%4 of the rows
// supplied by lanes j/4, j/4+4, j/4+8, j/4+12.
__device__ __forceinline__ bf16x4_t lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p));
}

__device__ __forceinline__ bf16x8_t cat(bf16x4_t a, bf16x4_t b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x8_t load_bf16x8(const bf16_t* p) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(p));
}

__device__ __forceinline__ bf16x8_t pack8(const f32x16_t& v, int base) {
  bf16x8_t r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)v[base + e];
  return r;
}

template <int D, bool CAUSAL, bool SOFTCAP>
__global__ __launch_bounds__(kThreads, 1) void bwd_mfma_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const bf16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    float* __restrict__ dQacc, bf16_t* __restrict__ dK, bf16_t* __restrict__ dV, int H, int H_kv, int N,
    int BH, float scale, float softcap) {
  using C = Cfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t sQ[BR * C::QP];
  __shared__ __attribute__((aligned(16))) uint16_t sdO[BR * C::QP];
  __shared__ __attribute__((aligned(16))) uint16_t sdST[BC * C::SP];
  __shared__ __attribute__((aligned(16))) float sL[BR];
  __shared__ __attribute__((aligned(16))) float sD[BR];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;     // accumulator column / row-group
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

  // ---- registers resident for the whole loop: K_j, V_j slices (B operands of
  // GEMM 1/2) and the K^T slice of GEMM 5.
  bf16x8_t kreg[C::KC], vreg[C::KC], ktreg[BC / 16];
  {
    const bool ok = my_key < N;
    const int64_t row = (kv_off + (ok ? my_key : 0)) * D;
#pragma unroll
    for (int c = 0; c < C::KC; ++c) {
      const int col = 16 * c + 8 * g;
      bf16x8_t z = {};
      kreg[c] = ok ? load_bf16x8(K + row + col) : z;
      vreg[c] = ok ? load_bf16x8(V + row + col) : z;
    }
    const int n_dq = D == 128 ? w : (w & 1);  // dQ column tile of this wave
#pragma unroll
    for (int v = 0; v < BC / 16; ++v) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = k0 + 16 * v + 8 * g + e;
        ktreg[v][e] = key < N ? __builtin_bit_cast(__bf16, K[(kv_off + key) * D + 32 * n_dq + l32].bits)
                              : (__bf16)0.0f;
      }
    }
  }

  f32x16_t dk_acc[C::NT], dv_acc[C::NT];
#pragma unroll
  for (int n = 0; n < C::NT; ++n) {
    dk_acc[n] = f32x16_t{};
    dv_acc[n] = f32x16_t{};
  }

  const float zs = scale * kLog2e;
  const int n_qblk = (N + BR - 1) / BR;
  const int i_first = CAUSAL ? (k0 / BR) : 0;
  const bool ragged_keys = k0 + BC > N;
  const int dq_n = D == 128 ? w : (w & 1);
  const int dq_t0 = D == 128 ? 0 : (w >> 1);

  for (int hg = 0; hg < G; ++hg) {
    const int h = hk * G + hg;
    const int64_t q_off = (int64_t(b) * H + h) * N;
    for (int i = n_qblk - 1; i >= i_first; --i) {
      const int q0 = i * BR;
      __syncthreads();  // previous iteration finished with sQ, sdO, sdST, sL, sD
      // ---- stage Q_i, dO_i (row-major, padded rows), LSE*log2e and D.
#pragma unroll
      for (int it = 0; it < (BR * D / 8) / kThreads; ++it) {
        const int idx = tid + it * kThreads;
        const int r = idx / (D / 8), ch = idx % (D / 8);
        u32x4_t qv = {0, 0, 0, 0}, ov = {0, 0, 0, 0};
        if (q0 + r < N) {
          const int64_t off = (q_off + q0 + r) * D + 8 * ch;
          qv = *reinterpret_cast<const u32x4_t*>(Q + off);
          ov = *reinterpret_cast<const u32x4_t*>(dO + off);
        }
        *reinterpret_cast<u32x4_t*>(&sQ[r * C::QP + 8 * ch]) = qv;
        *reinterpret_cast<u32x4_t*>(&sdO[r * C::QP + 8 * ch]) = ov;
      }
      if (tid < BR) {
        const bool ok = q0 + tid < N;
        sL[tid] = ok ? LSE[q_off + q0 + tid] * kLog2e : INFINITY;
      } else if (tid < 2 * BR) {
        const int r = tid - BR;
        sD[r] = q0 + r < N ? Dv[q_off + q0 + r] : 0.f;
      }
      __syncthreads();

      // ---- GEMM 1, 2: S and dP for 64 queries x this wave's 32 keys.
      f32x16_t s_acc[2], dp_acc[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        s_acc[t] = f32x16_t{};
        dp_acc[t] = f32x16_t{};
        const int row = 32 * t + l32;
#pragma unroll
        for (int c = 0; c < C::KC; ++c) {
          const int col = 16 * c + 8 * g;
          const bf16x8_t qa = *reinterpret_cast<const bf16x8_t*>(&sQ[row * C::QP + col]);
          const bf16x8_t oa = *reinterpret_cast<const bf16x8_t*>(&sdO[row * C::QP + col]);
          s_acc[t] = mfma(qa, kreg[c], s_acc[t]);
          dp_acc[t] = mfma(oa, vreg[c], dp_acc[t]);
        }
      }

      // ---- P and dS.  Accumulator register r of tile t holds query
      // 32t + 8(r/4) + 4g + r%4 and key my_key.
      const bool masked = (CAUSAL && q0 < k0 + BC) || ragged_keys;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int qr = 32 * t + 8 * m + 4 * g;
          const f32x4_t l4 = *reinterpret_cast<const f32x4_t*>(&sL[qr]);
          const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(&sD[qr]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * m + e;
            float s = s_acc[t][r];
            float dt = 1.f;
            if (SOFTCAP) {
              const float th = tanh_f32(s / softcap);
              s = softcap * th;
              dt = 1.f - th * th;
            }
            float p = fast_exp2(s * zs - l4[e]);
            if (masked) {
              const int qg = q0 + qr + e;
              if (my_key >= N || (CAUSAL && my_key > qg)) p = 0.f;
            }
            s_acc[t][r] = p;
            dp_acc[t][r] = p * (dp_acc[t][r] - d4[e]) * dt;
          }
        }
      }
      // bf16 operands: chunk u (16 queries) = registers 8(u%2)..8(u%2)+7 of tile u/2.
      bf16x8_t pf[4], dsf[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        pf[u] = pack8(s_acc[u >> 1], 8 * (u & 1));
        dsf[u] = pack8(dp_acc[u >> 1], 8 * (u & 1));
      }
      // dS^T to LDS: key row kw + l32, queries 16u + 4g + (0..3) and 16u + 8 + 4g + (0..3).
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        uint16_t* dst = &sdST[(kw + l32) * C::SP + 16 * u + 4 * g];
        *reinterpret_cast<bf16x4_t*>(dst) = __builtin_shufflevector(dsf[u], dsf[u], 0, 1, 2, 3);
        *reinterpret_cast<bf16x4_t*>(dst + 8) = __builtin_shufflevector(dsf[u], dsf[u], 4, 5, 6, 7);
      }

      // ---- GEMM 3, 4: dV += P^T dO_i, dK += dS^T Q_i.  B operand rows
      // (queries) 16u + 4g + (0..3) and +8, read transposed from LDS.
#pragma unroll
      for (int n = 0; n < C::NT; ++n) {
        const int col = 32 * n + 16 * h16 + 4 * (j16 & 3);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int row = 16 * u + 4 * g + (j16 >> 2);
          const bf16x8_t ob = cat(lds_read_tr(&sdO[row * C::QP + col]), lds_read_tr(&sdO[(row + 8) * C::QP + col]));
          const bf16x8_t qb = cat(lds_read_tr(&sQ[row * C::QP + col]), lds_read_tr(&sQ[(row + 8) * C::QP + col]));
          dv_acc[n] = mfma(pf[u], ob, dv_acc[n]);
          dk_acc[n] = mfma(dsf[u], qb, dk_acc[n]);
        }
      }
      __syncthreads();  // dS^T complete

      // ---- GEMM 5: dQ partial (queries x d) = dS K_j over all 128 keys.
#pragma unroll
      for (int tt = 0; tt < C::QT; ++tt) {
        const int t = dq_t0 + tt;
        f32x16_t dq = {};
        const int qcol = 32 * t + 16 * h16 + 4 * (j16 & 3);
#pragma unroll
        for (int v = 0; v < BC / 16; ++v) {
          const int key = 16 * v + 8 * g + (j16 >> 2);
          const bf16x8_t a = cat(lds_read_tr(&sdST[key * C::SP + qcol]), lds_read_tr(&sdST[(key + 4) * C::SP + qcol]));
          dq = mfma(a, ktreg[v], dq);
        }
        float* dst = dQacc + (q_off + q0) * D + 32 * dq_n + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qr = 32 * t + 8 * (r >> 2) + 4 * g + (r & 3);
          if (q0 + qr < N) atomic_add_f32(dst + int64_t(qr) * D, dq[r]);
        }
      }
    }
  }

  // ---- epilogue: dK = tau * dK_acc, dV = dV_acc (rows = keys, lanes = d).
#pragma unroll
  for (int n = 0; n < C::NT; ++n) {
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
hipError_t bwd_mfma_t(const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                      const float* LSE, const float* Dv, float* dQacc, void* dK, void* dV, hipStream_t s) {
  const int BH = p.B * p.H_kv;
  const int n_kblk = (p.N + BC - 1) / BC;
  hipLaunchKernelGGL((bwd_mfma_kernel<D, CAUSAL, SOFTCAP>), dim3(unsigned(BH) * unsigned(n_kblk)), dim3(kThreads),
                     0, s, static_cast<const bf16_t*>(Q), static_cast<const bf16_t*>(K),
                     static_cast<const bf16_t*>(V), static_cast<const bf16_t*>(dO), LSE, Dv, dQacc,
                     static_cast<bf16_t*>(dK), static_cast<bf16_t*>(dV), p.H, p.H_kv, p.N, BH, p.scale,
                     p.softcap);
  return hipGetLastError();
}

template <int D>
hipError_t bwd_mfma_d(const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                      const float* LSE, const float* Dv, float* dQacc, void* dK, void* dV, hipStream_t s) {
  const bool sc = p.softcap > 0.f;
  if (p.causal) return sc ? bwd_mfma_t<D, true, true>(p, Q, K, V, dO, LSE, Dv, dQacc, dK, dV, s)
                          : bwd_mfma_t<D, true, false>(p, Q, K, V, dO, LSE, Dv, dQacc, dK, dV, s);
  return sc ? bwd_mfma_t<D, false, true>(p, Q, K, V, dO, LSE, Dv, dQacc, dK, dV, s)
            : bwd_mfma_t<D, false, false>(p, Q, K, V, dO, LSE, Dv, dQacc, dK, dV, s);
}

}  // namespace

hipError_t launch_bwd_mfma(const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                           const float* LSE, const float* Dv, float* dQacc, void* dK, void* dV, hipStream_t s) {
  return p.d == 64 ? bwd_mfma_d<64>(p, Q, K, V, dO, LSE, Dv, dQacc, dK, dV, s)
                   : bwd_mfma_d<128>(p, Q, K, V, dO, LSE, Dv, dQacc, dK, dV, s);
}

}  // namespace fabwd

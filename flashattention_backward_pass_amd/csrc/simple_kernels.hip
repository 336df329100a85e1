// Vector-ALU (fp32 FMA) forward and backward kernels.
//
// These serve the fp32 workloads (on MI355X the fp32 vector and fp32 matrix
// peaks are the same, 157.3 TFLOP/s); bf16 runs on the matrix-core kernels.  They follow the tiling of
// "解析 FlashAttention（3）：FlashAttention-v1 反向传播", section 4 (Algorithm 4):
// key/value blocks outer, query blocks inner, P recomputed per tile from the
// saved LSE (Inference Cookbook "反向传播算法详解", section 1.2), dK and dV kept
// on chip, dQ partials added into an fp32 buffer (section 6.2 of the latter),
// or, in deterministic mode, dQ from a query-block-outer kernel.
//
// Arithmetic: inputs are widened to fp32, every product and sum is fp32, and
// exponentials are hardware exp2 with the log2(e) factor folded into the
// scale.  The forward is the online-softmax loop of the Cookbook page,
// section 3.1 (query blocks outer, key blocks inner).
//
// Dropout (FlashAttention-v1 page, section 3.3 and eqs (10)-(12)): each
// element's keep bit is regenerated from the generator state (philox.h);
// the forward accumulates P o Z into O while the row sum uses P, and the
// backward uses P o Z for dV and (dO V^T) o Z for dP.
#include "fabwd_device.h"
#include "fabwd_launch.h"

namespace fabwd {

namespace {

constexpr int kThreads = 256;

// ----------------------------------------------------------------- forward
// One workgroup per (query block of 32 rows, head, batch); 8 lanes per row.
// Key k is visible to query q iff q - wl <= k <= q + wr and k < N (causal:
// wr = 0; an unbounded side is N).
template <typename T, int D, bool SOFTCAP>
__global__ __launch_bounds__(kThreads) void fwd_simple_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                              const T* __restrict__ V, T* __restrict__ O,
                                                              float* __restrict__ LSE, int H, int H_kv, int N,
                                                              float scale, float softcap, int wl, int wr,
                                                              Dropout drop) {
  constexpr int BQ = 32, BK = 64, DX = D / 8;
  __shared__ float sQ[BQ][D];
  __shared__ float sK[BK][D + 1];
  __shared__ float sV[BK][D];
  __shared__ float sP[BQ][BK + 1];

  const int t = threadIdx.x, r = t >> 3, sub = t & 7;
  const int q0 = blockIdx.x * BQ, h = blockIdx.y, b = blockIdx.z;
  const int hk = h / (H / H_kv);
  const T* q_base = Q + (int64_t(b) * H + h) * N * D;
  const T* k_base = K + (int64_t(b) * H_kv + hk) * N * D;
  const T* v_base = V + (int64_t(b) * H_kv + hk) * N * D;

  for (int idx = t; idx < BQ * D; idx += kThreads) {
    const int rr = idx / D, x = idx % D;
    sQ[rr][x] = (q0 + rr < N) ? Elem<T>::load(q_base, int64_t(q0 + rr) * D + x) : 0.f;
  }
  const int row = q0 + r;
  float m_run = -INFINITY, l_run = 0.f;
  float acc[DX];
#pragma unroll
  for (int k = 0; k < DX; ++k) acc[k] = 0.f;

  // Keys visible to some row of the block.
  const int kv_begin = max(0, q0 - wl) / BK * BK;
  const int kv_end = min(N, min(q0 + BQ, N) + wr);
  const float zscale = scale * kLog2e;
  const float cap_k = SOFTCAP ? 2.f * kLog2e / softcap : 0.f;  // tanh(x / c) = tanh_scaled(x, cap_k)
  for (int k0 = kv_begin; k0 < kv_end; k0 += BK) {
    __syncthreads();
    for (int idx = t; idx < BK * D; idx += kThreads) {
      const int kk = idx / D, x = idx % D;
      const bool ok = k0 + kk < N;
      sK[kk][x] = ok ? Elem<T>::load(k_base, int64_t(k0 + kk) * D + x) : 0.f;
      sV[kk][x] = ok ? Elem<T>::load(v_base, int64_t(k0 + kk) * D + x) : 0.f;
    }
    __syncthreads();
    float z[BK / 8];
    float bmax = -INFINITY;
#pragma unroll
    for (int m = 0; m < BK / 8; ++m) {
      const int c = sub + 8 * m, key = k0 + c;
      float s = 0.f;
#pragma unroll 8
      for (int x = 0; x < D; ++x) s = fmaf(sQ[r][x], sK[c][x], s);
      if (SOFTCAP) s = softcap * tanh_scaled(s, cap_k);
      float zz = s * zscale;
      if (key >= N || key > row + wr || key < row - wl) zz = -INFINITY;
      z[m] = zz;
      bmax = fmaxf(bmax, zz);
    }
    bmax = wave_xor_max(bmax, 8);
    const float m_new = fmaxf(m_run, bmax);
    const float base = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - base);
    float psum = 0.f;
#pragma unroll
    for (int m = 0; m < BK / 8; ++m) {
      const float p = fast_exp2(z[m] - base);
      psum += p;
      float pd = p;
      if (drop.enabled)
        pd = dropout_keep(drop, uint32_t(b * H + h), uint32_t(row), uint32_t(k0 + sub + 8 * m)) ? p * drop.scale : 0.f;
      sP[r][sub + 8 * m] = pd;
    }
    psum = wave_xor_sum(psum, 8);
    l_run = l_run * alpha + psum;
    m_run = m_new;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < DX; ++k) acc[k] *= alpha;
#pragma unroll 2
    for (int c = 0; c < BK; ++c) {
      const float pv = sP[r][c];
#pragma unroll
      for (int k = 0; k < DX; ++k) acc[k] = fmaf(pv, sV[c][sub + 8 * k], acc[k]);
    }
  }
  if (row < N) {
    const float inv_l = 1.0f / l_run;
    T* o_row = O + ((int64_t(b) * H + h) * N + row) * D;
#pragma unroll
    for (int k = 0; k < DX; ++k) Elem<T>::store(o_row, sub + 8 * k, acc[k] * inv_l);
    if (sub == 0) LSE[(int64_t(b) * H + h) * N + row] = (m_run + __log2f(l_run)) * kLn2;
  }
}

// ----------------------------------------------------------------- backward
// One workgroup per (key block of 32 keys, key/value head, batch); it loops
// over the query heads of its group and over query blocks of 32 rows.
template <typename T, int D, bool SOFTCAP, bool ATOMIC_DQ>
__global__ __launch_bounds__(kThreads) void bwd_simple_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                              const T* __restrict__ V, const T* __restrict__ dO,
                                                              const float* __restrict__ LSE,
                                                              const float* __restrict__ Dv,
                                                              float* __restrict__ dQacc, T* __restrict__ dK,
                                                              T* __restrict__ dV, int H, int H_kv, int N,
                                                              float scale, float softcap, int wl, int wr,
                                                              Dropout drop) {
  constexpr int BK = 32, BQ = 32, DX = D / 8;
  __shared__ float sK[BK][D + 1];
  __shared__ float sV[BK][D + 1];
  __shared__ float sQ[BQ][D + 1];
  __shared__ float sdO[BQ][D + 1];
  __shared__ float sP[BQ][BK + 1];
  __shared__ float sdS[BQ][BK + 1];
  __shared__ float sL[BQ];
  __shared__ float sD[BQ];

  const int t = threadIdx.x, r = t >> 3, sub = t & 7;
  const int k0 = blockIdx.x * BK, hk = blockIdx.y, b = blockIdx.z;
  const int G = H / H_kv;
  const int64_t kv_off = (int64_t(b) * H_kv + hk) * N * D;

  for (int idx = t; idx < BK * D; idx += kThreads) {
    const int kk = idx / D, x = idx % D;
    const bool ok = k0 + kk < N;
    sK[kk][x] = ok ? Elem<T>::load(K + kv_off, int64_t(k0 + kk) * D + x) : 0.f;
    sV[kk][x] = ok ? Elem<T>::load(V + kv_off, int64_t(k0 + kk) * D + x) : 0.f;
  }
  float acc_dk[DX], acc_dv[DX];
#pragma unroll
  for (int k = 0; k < DX; ++k) acc_dk[k] = acc_dv[k] = 0.f;

  const float zscale = scale * kLog2e;
  const float cap_k = SOFTCAP ? 2.f * kLog2e / softcap : 0.f;  // tanh(x / c) = tanh_scaled(x, cap_k)
  // Query rows that see some key of the block.
  const int q_begin = max(0, k0 - wr) / BQ * BQ;
  const int q_end = min(N, min(k0 + BK, N) + wl);
  for (int hg = 0; hg < G; ++hg) {
    const int h = hk * G + hg;
    const int64_t q_off = (int64_t(b) * H + h) * N;
    for (int q0 = q_begin; q0 < q_end; q0 += BQ) {
      __syncthreads();
      for (int idx = t; idx < BQ * D; idx += kThreads) {
        const int rr = idx / D, x = idx % D;
        const bool ok = q0 + rr < N;
        sQ[rr][x] = ok ? Elem<T>::load(Q, (q_off + q0 + rr) * D + x) : 0.f;
        sdO[rr][x] = ok ? Elem<T>::load(dO, (q_off + q0 + rr) * D + x) : 0.f;
      }
      if (t < BQ) {
        const bool ok = q0 + t < N;
        sL[t] = ok ? LSE[q_off + q0 + t] * kLog2e : INFINITY;
        sD[t] = ok ? Dv[q_off + q0 + t] : 0.f;
      }
      __syncthreads();
      const int row = q0 + r;
#pragma unroll
      for (int m = 0; m < BK / 8; ++m) {
        const int c = sub + 8 * m, key = k0 + c;
        float s = 0.f, dp = 0.f;
#pragma unroll 8
        for (int x = 0; x < D; ++x) {
          s = fmaf(sQ[r][x], sK[c][x], s);
          dp = fmaf(sdO[r][x], sV[c][x], dp);
        }
        float dtanh = 1.f;
        if (SOFTCAP) {
          const float th = tanh_scaled(s, cap_k);
          s = softcap * th;
          dtanh = 1.f - th * th;
        }
        const bool masked = key >= N || row >= N || key > row + wr || key < row - wl;
        const float p = masked ? 0.f : fast_exp2(s * zscale - sL[r]);
        float zd = 1.f;  // dropout multiplier Z of this element
        if (drop.enabled)
          zd = dropout_keep(drop, uint32_t(b * H + h), uint32_t(row), uint32_t(key)) ? drop.scale : 0.f;
        sP[r][c] = p * zd;
        sdS[r][c] = p * (dp * zd - sD[r]) * dtanh;
      }
      __syncthreads();
      // dV += P^T dO and dK += dS^T Q for key r (this thread's key row),
      // query rows outer.
#pragma unroll 2
      for (int rr = 0; rr < BQ; ++rr) {
        const float pv = sP[rr][r], dsv = sdS[rr][r];
#pragma unroll
        for (int k = 0; k < DX; ++k) {
          acc_dv[k] = fmaf(pv, sdO[rr][sub + 8 * k], acc_dv[k]);
          acc_dk[k] = fmaf(dsv, sQ[rr][sub + 8 * k], acc_dk[k]);
        }
      }
      // dQ partial of this (query block, key block) pair, unscaled: keys
      // outer, so only this lane's DX partial sums are live.
      if (ATOMIC_DQ && row < N) {
        float a[DX];
#pragma unroll
        for (int k = 0; k < DX; ++k) a[k] = 0.f;
#pragma unroll 4
        for (int c = 0; c < BK; ++c) {
          const float ds = sdS[r][c];
#pragma unroll
          for (int k = 0; k < DX; ++k) a[k] = fmaf(ds, sK[c][sub + 8 * k], a[k]);
        }
#pragma unroll
        for (int k = 0; k < DX; ++k) atomic_add_f32(dQacc + (q_off + row) * D + sub + 8 * k, a[k]);
      }
    }
  }
  const int key = k0 + r;
  if (key < N) {
#pragma unroll
    for (int k = 0; k < DX; ++k) {
      const int x = sub + 8 * k;
      Elem<T>::store(dK + kv_off, int64_t(key) * D + x, acc_dk[k] * scale);
      Elem<T>::store(dV + kv_off, int64_t(key) * D + x, acc_dv[k]);
    }
  }
}

// ------------------------------------------------------- deterministic dQ
// dQ_i = sum_j dS_ij K_j ("解析 FlashAttention（3）：FlashAttention-v1 反向传播",
// eq (15), unscaled) with query blocks outer and key blocks inner: one
// workgroup per (query block of 32 rows, head, batch) recomputes P and dS for
// its rows and keeps dQ in registers; every sum runs in a fixed order and
// dQaccum is written once with plain stores, so the result is bitwise
// reproducible.  8 lanes per row, lane `sub` owns columns sub + 8k.
template <typename T, int D, bool SOFTCAP>
__global__ __launch_bounds__(kThreads) void bwd_dq_simple_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, const T* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Dv, float* __restrict__ dQacc, int H, int H_kv, int N,
    float scale, float softcap, int wl, int wr, Dropout drop) {
  constexpr int BQ = 32, BK = 32, DX = D / 8;
  __shared__ float sQ[BQ][D + 1];
  __shared__ float sdO[BQ][D + 1];
  __shared__ float sK[BK][D + 1];
  __shared__ float sV[BK][D + 1];
  __shared__ float sdS[BQ][BK + 1];

  const int t = threadIdx.x, r = t >> 3, sub = t & 7;
  const int q0 = blockIdx.x * BQ, h = blockIdx.y, b = blockIdx.z;
  const int hk = h / (H / H_kv);
  const int64_t q_off = (int64_t(b) * H + h) * N;
  const int64_t kv_off = (int64_t(b) * H_kv + hk) * N * D;
  const int row = q0 + r;

  for (int idx = t; idx < BQ * D; idx += kThreads) {
    const int rr = idx / D, x = idx % D;
    const bool ok = q0 + rr < N;
    sQ[rr][x] = ok ? Elem<T>::load(Q, (q_off + q0 + rr) * D + x) : 0.f;
    sdO[rr][x] = ok ? Elem<T>::load(dO, (q_off + q0 + rr) * D + x) : 0.f;
  }
  const float lse2 = row < N ? LSE[q_off + row] * kLog2e : INFINITY;
  const float dval = row < N ? Dv[q_off + row] : 0.f;
  const float zscale = scale * kLog2e;
  const float cap_k = SOFTCAP ? 2.f * kLog2e / softcap : 0.f;  // tanh(x / c) = tanh_scaled(x, cap_k)
  float acc[DX];
#pragma unroll
  for (int k = 0; k < DX; ++k) acc[k] = 0.f;

  const int kv_begin = max(0, q0 - wl) / BK * BK;
  const int kv_end = min(N, min(q0 + BQ, N) + wr);
  for (int k0 = kv_begin; k0 < kv_end; k0 += BK) {
    __syncthreads();
    for (int idx = t; idx < BK * D; idx += kThreads) {
      const int kk = idx / D, x = idx % D;
      const bool ok = k0 + kk < N;
      sK[kk][x] = ok ? Elem<T>::load(K + kv_off, int64_t(k0 + kk) * D + x) : 0.f;
      sV[kk][x] = ok ? Elem<T>::load(V + kv_off, int64_t(k0 + kk) * D + x) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < BK / 8; ++m) {
      const int c = sub + 8 * m, key = k0 + c;
      float s = 0.f, dp = 0.f;
#pragma unroll 8
      for (int x = 0; x < D; ++x) {
        s = fmaf(sQ[r][x], sK[c][x], s);
        dp = fmaf(sdO[r][x], sV[c][x], dp);
      }
      float dtanh = 1.f;
      if (SOFTCAP) {
        const float th = tanh_scaled(s, cap_k);
        s = softcap * th;
        dtanh = 1.f - th * th;
      }
      const bool masked = key >= N || row >= N || key > row + wr || key < row - wl;
      const float p = masked ? 0.f : fast_exp2(s * zscale - lse2);
      float zd = 1.f;
      if (drop.enabled) zd = dropout_keep(drop, uint32_t(b * H + h), uint32_t(row), uint32_t(key)) ? drop.scale : 0.f;
      sdS[r][c] = p * (dp * zd - dval) * dtanh;
    }
    __syncthreads();
#pragma unroll 2
    for (int c = 0; c < BK; ++c) {
      const float dsv = sdS[r][c];
#pragma unroll
      for (int k = 0; k < DX; ++k) acc[k] = fmaf(dsv, sK[c][sub + 8 * k], acc[k]);
    }
  }
  if (row < N) {
#pragma unroll
    for (int k = 0; k < DX; ++k) dQacc[(q_off + row) * D + sub + 8 * k] = acc[k];
  }
}

template <typename T, int D, bool S>
hipError_t fwd_simple_t(const Problem& p, const void* Q, const void* K, const void* V, void* O, float* LSE,
                        hipStream_t s) {
  dim3 grid((p.N + 31) / 32, p.H, p.B);
  hipLaunchKernelGGL((fwd_simple_kernel<T, D, S>), grid, dim3(kThreads), 0, s, static_cast<const T*>(Q),
                     static_cast<const T*>(K), static_cast<const T*>(V), static_cast<T*>(O), LSE, p.H, p.H_kv,
                     p.N, p.scale, p.softcap, p.wl, p.wr, p.drop());
  return hipGetLastError();
}

template <typename T, int D, bool S>
hipError_t bwd_simple_t(const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                        const float* LSE, const float* Dv, float* dQacc, void* dK, void* dV, hipStream_t s) {
  dim3 grid((p.N + 31) / 32, p.H_kv, p.B);
  auto kern = p.deterministic ? bwd_simple_kernel<T, D, S, false> : bwd_simple_kernel<T, D, S, true>;
  hipLaunchKernelGGL(kern, grid, dim3(kThreads), 0, s, static_cast<const T*>(Q), static_cast<const T*>(K),
                     static_cast<const T*>(V), static_cast<const T*>(dO), LSE, Dv, dQacc, static_cast<T*>(dK),
                     static_cast<T*>(dV), p.H, p.H_kv, p.N, p.scale, p.softcap, p.wl, p.wr, p.drop());
  return hipGetLastError();
}

template <typename T, int D, bool S>
hipError_t bwd_dq_simple_t(const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                           const float* LSE, const float* Dv, float* dQacc, hipStream_t s) {
  dim3 grid((p.N + 31) / 32, p.H, p.B);
  hipLaunchKernelGGL((bwd_dq_simple_kernel<T, D, S>), grid, dim3(kThreads), 0, s, static_cast<const T*>(Q),
                     static_cast<const T*>(K), static_cast<const T*>(V), static_cast<const T*>(dO), LSE, Dv,
                     dQacc, p.H, p.H_kv, p.N, p.scale, p.softcap, p.wl, p.wr, p.drop());
  return hipGetLastError();
}

template <typename T, int D>
hipError_t fwd_simple_d(const Problem& p, const void* Q, const void* K, const void* V, void* O, float* LSE,
                        hipStream_t s) {
  return p.softcap > 0.f ? fwd_simple_t<T, D, true>(p, Q, K, V, O, LSE, s)
                         : fwd_simple_t<T, D, false>(p, Q, K, V, O, LSE, s);
}

template <typename T, int D>
hipError_t bwd_simple_d(const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                        const float* LSE, const float* Dv, float* dQacc, void* dK, void* dV, hipStream_t s) {
  return p.softcap > 0.f ? bwd_simple_t<T, D, true>(p, Q, K, V, dO, LSE, Dv, dQacc, dK, dV, s)
                         : bwd_simple_t<T, D, false>(p, Q, K, V, dO, LSE, Dv, dQacc, dK, dV, s);
}

template <typename T, int D>
hipError_t bwd_dq_simple_d(const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                           const float* LSE, const float* Dv, float* dQacc, hipStream_t s) {
  return p.softcap > 0.f ? bwd_dq_simple_t<T, D, true>(p, Q, K, V, dO, LSE, Dv, dQacc, s)
                         : bwd_dq_simple_t<T, D, false>(p, Q, K, V, dO, LSE, Dv, dQacc, s);
}

}  // namespace

hipError_t launch_fwd_simple(const Problem& p, const void* Q, const void* K, const void* V, void* O, float* LSE,
                             hipStream_t s) {
  if (p.dtype != 0) return hipErrorInvalidValue;
  return p.d == 64 ? fwd_simple_d<float, 64>(p, Q, K, V, O, LSE, s)
                   : fwd_simple_d<float, 128>(p, Q, K, V, O, LSE, s);
}

hipError_t launch_bwd_simple(const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                             const float* LSE, const float* Dv, float* dQacc, void* dK, void* dV, hipStream_t s) {
  if (p.dtype != 0) return hipErrorInvalidValue;
  return p.d == 64 ? bwd_simple_d<float, 64>(p, Q, K, V, dO, LSE, Dv, dQacc, dK, dV, s)
                   : bwd_simple_d<float, 128>(p, Q, K, V, dO, LSE, Dv, dQacc, dK, dV, s);
}

}  // namespace fabwd

namespace fabwd {

hipError_t launch_bwd_dq_simple(const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                                const float* LSE, const float* Dv, float* dQacc, hipStream_t s) {
  if (p.dtype != 0) return hipErrorInvalidValue;
  return p.d == 64 ? bwd_dq_simple_d<float, 64>(p, Q, K, V, dO, LSE, Dv, dQacc, s)
                   : bwd_dq_simple_d<float, 128>(p, Q, K, V, dO, LSE, Dv, dQacc, s);
}

}  // namespace fabwd

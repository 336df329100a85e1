// The dK/dV and dQ work units of the bf16 backward in one launch.
//
// The two kernels are independent: both read Q, K, V, dO, LSE and D; the
// dK/dV units write dK and dV, the dQ units write dQaccum (as long as the
// dK/dV units do not borrow dQaccum for head-split partials, which the
// dispatch rules out).  A problem with few units, such as one head at full
// length (128 key blocks and 128 query blocks of N = 16384 for 256 compute
// units), leaves half the chip idle in each kernel when they run one after
// the other, and each kernel's time is set by its heaviest (first causal)
// unit.  Here the workgroups of one grid take either kind of unit, the
// heaviest of each kind first and the two kinds interleaved, so both run at
// once.  The grid runs at one wave per SIMD, as the dK/dV units need.
#include "bwd_dkdv_block.h"
#include "bwd_dq_block.h"

#include <algorithm>

namespace fabwd {

namespace {

static_assert(dkdv::kThreads == dq::kThreads, "one workgroup size for both kinds of unit");
constexpr int kThreads = dkdv::kThreads;
// Grids of at most this many workgroups take the combined launch.  d = 128
// (one workgroup per CU): measured faster up to 1024 (6-19 % at 1024
// workgroups), slower at 2048 (5-10 %, where the dQ units lose their second
// wave per SIMD).  d = 64 (two workgroups per CU, like the dQ kernel):
// faster up to 2048 (0.3-5.5 %).
constexpr int64_t kFusedMaxBlocks = 2048;
constexpr int64_t fused_max_blocks(int d) { return d == 64 ? kFusedMaxBlocks : kFusedMaxBlocks / 2; }

// With dQ given, dQaccum is free for partial sums: the heaviest units of a
// causal (or windowed) problem, the first `qblocks` key blocks of every kv
// head and the last `qq` query blocks of every query head, are each split in
// two, dK/dV units by query range and dQ units by key range, whose fp32
// partial tiles go to dQaccum (dK/dV tiles first, then dQ tiles);
// fused_partial_sum_kernel adds the halves after the launch.  Units of each
// kind are numbered split halves first ((block i, half h, head x) at
// 2 BH i + BH h + x), then the unsplit blocks.
template <int D, bool SOFTCAP, bool DROPOUT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(
    dkdv::kWavesPerSimd<D, SOFTCAP, DROPOUT>, dkdv::kWavesPerSimd<D, SOFTCAP, DROPOUT>))) void bwd_fused_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const bf16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    bf16_t* __restrict__ dK, bf16_t* __restrict__ dV, float* __restrict__ dQacc, bf16_t* __restrict__ dQout, int H,
    int H_kv, int N,
    int BH_kv, int BH_q, float scale, float softcap, int wl, int wr, Dropout drop, unsigned n_dkdv, unsigned n_dq,
    int qblocks, int qq) {
  // Blocks 0 .. 2m-1 alternate between the two kinds (m = the smaller
  // count); the rest belong to the larger kind.
  const unsigned m = min(n_dkdv, n_dq);
  const unsigned b = blockIdx.x;
  bool dq_unit;
  unsigned unit;
  if (b < 2 * m) {
    dq_unit = (b & 1u) != 0;
    unit = b >> 1;
  } else {
    dq_unit = n_dq > n_dkdv;
    unit = b - m;
  }
  if (dq_unit) {
    const unsigned n_half = 2u * unsigned(BH_q) * unsigned(qq);
    int khalf = -1;
    unsigned u;
    if (unit < n_half) {
      khalf = int((unit / unsigned(BH_q)) & 1u);
      u = unit % unsigned(BH_q) + unsigned(BH_q) * (unit / (2u * unsigned(BH_q)));
    } else {
      u = unit - n_half + unsigned(BH_q) * unsigned(qq);
    }
    float* qpart = dQacc + 4 * int64_t(BH_kv) * qblocks * (dkdv::BC * D);
    dq::dq_block<D, SOFTCAP, DROPOUT>(Q, K, V, dO, LSE, Dv, dQacc, dQout, H, H_kv, N, BH_q, scale, softcap, wl, wr,
                                      drop, u, khalf, qq, qpart);
  } else {
    const unsigned n_half = 2u * unsigned(BH_kv) * unsigned(qblocks);
    int qhalf = -1;
    unsigned u = unit;
    if (unit < n_half) {
      const unsigned bh = unit % unsigned(BH_kv), j = unit / (2u * unsigned(BH_kv));
      qhalf = int((unit / unsigned(BH_kv)) & 1u);
      u = bh + unsigned(BH_kv) * j;
    } else {
      u = unit - n_half + unsigned(BH_kv) * unsigned(qblocks);
    }
    dkdv::dkdv_block<D, SOFTCAP, DROPOUT>(Q, K, V, dO, LSE, Dv, dK, dV, H, H_kv, N, BH_kv, scale, softcap, wl, wr,
                                          1, qhalf >= 0 ? dQacc : nullptr, drop, u, qhalf, qblocks);
  }
}

// Sums the partial tiles of the split units (fixed order; layout as
// bwd_fused_kernel writes them): elements [0, BH_kv qblocks BC D) are dK/dV
// tiles, dK = -tau (p0 + p1) and dV = p0 + p1; the rest are dQ tiles,
// dQ = tau (p0 + p1), the product and rounding of the convert kernel.
// 8 elements per thread; rows past N skipped.
template <int D>
__global__ __launch_bounds__(256) void fused_partial_sum_kernel(const float* __restrict__ part, int BH_kv,
                                                                int qblocks, int BH_q, int qq, int N,
                                                                bf16_t* __restrict__ dK, bf16_t* __restrict__ dV,
                                                                bf16_t* __restrict__ dQ, float scale) {
  constexpr int BC = dkdv::BC, BQ = dq::BQ;
  const int64_t kv_tiles = int64_t(BH_kv) * qblocks, q_tiles = int64_t(BH_q) * qq;
  const int64_t kv_elems = kv_tiles * BC * D;
  int64_t i = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 8;
  u32x4_t o0, o1;
  if (i < kv_elems) {
    const int64_t t = i / (BC * D);
    const int within = int(i % (BC * D));
    const int bh = int(t / qblocks), j = int(t % qblocks);
    const int key = j * BC + within / D;
    if (key >= N) return;
    const int64_t out = (int64_t(bh) * N + key) * D + within % D;
    const float* pk0 = part + i;
    const float* pv0 = pk0 + kv_elems;
    const float* pk1 = pv0 + kv_elems;
    const float* pv1 = pk1 + kv_elems;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o0[e] = pack_bf16x2(-scale * (pk0[2 * e] + pk1[2 * e]), -scale * (pk0[2 * e + 1] + pk1[2 * e + 1]));
      o1[e] = pack_bf16x2(pv0[2 * e] + pv1[2 * e], pv0[2 * e + 1] + pv1[2 * e + 1]);
    }
    *reinterpret_cast<u32x4_t*>(dK + out) = o0;
    *reinterpret_cast<u32x4_t*>(dV + out) = o1;
    return;
  }
  i -= kv_elems;
  if (i >= q_tiles * BQ * D) return;
  const int64_t t = i / (BQ * D);
  const int within = int(i % (BQ * D));
  const int bh = int(t / qq), iq = int(t % qq);
  const int row = ((N + BQ - 1) / BQ - 1 - iq) * BQ + within / D;
  if (row >= N) return;
  const int64_t out = (int64_t(bh) * N + row) * D + within % D;
  const float* p0 = part + 4 * kv_elems + i;
  const float* p1 = p0 + q_tiles * BQ * D;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    o0[e] = pack_bf16x2(scale * (p0[2 * e] + p1[2 * e]), scale * (p0[2 * e + 1] + p1[2 * e + 1]));
  *reinterpret_cast<u32x4_t*>(dQ + out) = o0;
}

unsigned dkdv_units(const Problem& p) {
  return unsigned(p.B * p.H_kv) * unsigned((p.N + dkdv::BC - 1) / dkdv::BC);
}

// Query tiles (of dkdv::BR rows, per query head) that key block j visits.
int kblock_tiles(const Problem& p, int j) {
  const int k0 = j * dkdv::BC, k_end = std::min(k0 + dkdv::BC, p.N);
  const int i_lo = std::max(0, k0 - p.wr) / dkdv::BR;
  const int i_hi = (std::min(p.N, k_end + p.wl) + dkdv::BR - 1) / dkdv::BR;
  return i_hi - i_lo;
}
// Key steps (of dq::BK keys) that query block i visits.
int qblock_steps(const Problem& p, int i) {
  const int q0 = i * dq::BQ, q_hi = std::min(q0 + dq::BQ, p.N) - 1;
  const int s_lo = std::max(0, q0 - p.wl) / dq::BK;
  const int s_hi = (std::min(p.N, q_hi + p.wr + 1) + dq::BK - 1) / dq::BK;
  return s_hi - s_lo;
}
unsigned dq_units(const Problem& p) { return unsigned(p.B * p.H) * unsigned((p.N + dq::BQ - 1) / dq::BQ); }

template <int D, bool SOFTCAP, bool DROPOUT>
hipError_t fused_t(const Problem& p, const void* Q, const void* K, const void* V, const void* dO, const float* LSE,
                   const float* Dv, void* dK, void* dV, float* dQacc, void* dQout, hipStream_t s) {
  const FusedSplit sp = fused_split(p, dQout != nullptr);
  const int BH = p.B * p.H_kv, BHq = p.B * p.H;
  const unsigned n1 = dkdv_units(p) + unsigned(BH) * unsigned(sp.kv), n2 = dq_units(p) + unsigned(BHq) * unsigned(sp.q);
  hipLaunchKernelGGL((bwd_fused_kernel<D, SOFTCAP, DROPOUT>), dim3(n1 + n2), dim3(kThreads), 0, s,
                     static_cast<const bf16_t*>(Q), static_cast<const bf16_t*>(K), static_cast<const bf16_t*>(V),
                     static_cast<const bf16_t*>(dO), LSE, Dv, static_cast<bf16_t*>(dK), static_cast<bf16_t*>(dV),
                     dQacc, static_cast<bf16_t*>(dQout), p.H, p.H_kv, p.N, BH, BHq, p.scale, p.softcap, p.wl,
                     p.wr, p.drop(), n1, n2, sp.kv, sp.q);
  if (sp.kv + sp.q == 0) return hipGetLastError();
  const int64_t elems = (int64_t(BH) * sp.kv * dkdv::BC + int64_t(BHq) * sp.q * dq::BQ) * D;
  hipLaunchKernelGGL(fused_partial_sum_kernel<D>, dim3(unsigned((elems / 8 + 255) / 256)), dim3(256), 0, s,
                     static_cast<const float*>(dQacc), BH, sp.kv, BHq, sp.q, p.N, static_cast<bf16_t*>(dK),
                     static_cast<bf16_t*>(dV), static_cast<bf16_t*>(dQout), p.scale);
  return hipGetLastError();
}

template <int D>
hipError_t fused_d(const Problem& p, const void* Q, const void* K, const void* V, const void* dO, const float* LSE,
                   const float* Dv, void* dK, void* dV, float* dQacc, void* dQout, hipStream_t s) {
  if (p.dropout)
    return p.softcap > 0.f ? fused_t<D, true, true>(p, Q, K, V, dO, LSE, Dv, dK, dV, dQacc, dQout, s)
                           : fused_t<D, false, true>(p, Q, K, V, dO, LSE, Dv, dK, dV, dQacc, dQout, s);
  return p.softcap > 0.f ? fused_t<D, true, false>(p, Q, K, V, dO, LSE, Dv, dK, dV, dQacc, dQout, s)
                         : fused_t<D, false, false>(p, Q, K, V, dO, LSE, Dv, dK, dV, dQacc, dQout, s);
}

}  // namespace

// Which units to split.  A unit's cost is counted in matrix steps of about
// equal time: a dK/dV tile (dkdv::BR query rows x BC keys, four products) per
// query head of the group, or a dQ step (BQ rows x BK keys, three products)
// (both near 1.4 us at d = 128 on one compute unit, measured).  The launch
// takes about max(heaviest unit, total / compute units); splitting the
// leading units of a kind (the heaviest under a causal mask) halves them,
// costs a summing launch of about kSumCost steps and is limited by the
// room in dQaccum.  The split with the least predicted time is taken when it
// beats the unsplit launch.
FusedSplit fused_split(const Problem& p, bool with_dq) {
  FusedSplit r;
  if (!with_dq || p.dtype != 1 || !bwd_fused_fits(p)) return r;
  constexpr int64_t kComputeUnits = 256;
  const int64_t kSumCost = p.d == 128 ? 3 : 6;
  const int G = p.H / p.H_kv;
  const int n_kb = (p.N + dkdv::BC - 1) / dkdv::BC, n_qb = (p.N + dq::BQ - 1) / dq::BQ;
  const int64_t BHkv = int64_t(p.B) * p.H_kv, BHq = int64_t(p.B) * p.H;
  // Unit weights in dispatch order (key blocks from the first, query blocks
  // from the last) and their suffix maxima, in fixed arrays (no allocation:
  // the combined launch has at most kFusedMaxBlocks units of each kind, so
  // at most that many blocks per head).
  int kv[kFusedMaxBlocks], q[kFusedMaxBlocks], kv_suf[kFusedMaxBlocks + 1], q_suf[kFusedMaxBlocks + 1];
  if (n_kb > kFusedMaxBlocks || n_qb > kFusedMaxBlocks) return r;
  kv_suf[n_kb] = q_suf[n_qb] = 0;
  int64_t total = 0;
  for (int j = 0; j < n_kb; ++j) total += BHkv * (kv[j] = G * kblock_tiles(p, j));
  for (int i = 0; i < n_qb; ++i) total += BHq * (q[i] = qblock_steps(p, n_qb - 1 - i));
  for (int j = n_kb - 1; j >= 0; --j) kv_suf[j] = std::max(kv_suf[j + 1], kv[j]);
  for (int i = n_qb - 1; i >= 0; --i) q_suf[i] = std::max(q_suf[i + 1], q[i]);
  const int64_t avg = (total + kComputeUnits - 1) / kComputeUnits;
  const int64_t before = std::max<int64_t>({kv_suf[0], q_suf[0], avg});
  if (std::max(kv_suf[0], q_suf[0]) <= avg) return r;
  // Room: B*H*N*d floats; a split key block takes 4 BC x d tiles per kv head,
  // a split query block 2 BQ x d tiles per query head.
  const int64_t room = BHq * p.N * p.d;
  const int64_t kv_tile = 4 * BHkv * dkdv::BC * p.d, q_tile = 2 * BHq * dq::BQ * p.d;
  // best_q[c]: the least heaviest-dQ weight with at most c query blocks split
  // (each split block must keep a step in both halves), and its count.
  int best_q[kFusedMaxBlocks + 1], best_qn[kFusedMaxBlocks + 1];
  int q_half = 0;
  bool q_ok = true;
  for (int c = 0; c <= n_qb; ++c) {
    const int w = std::max(q_half, q_suf[c]);
    if (c == 0 || w < best_q[c - 1]) { best_q[c] = w; best_qn[c] = c; }
    else { best_q[c] = best_q[c - 1]; best_qn[c] = best_qn[c - 1]; }
    if (c < n_qb) {
      q_ok = q_ok && q[c] >= 2;
      if (q_ok) q_half = std::max(q_half, (q[c] + 1) / 2);
      else { for (int e = c + 1; e <= n_qb; ++e) { best_q[e] = best_q[c]; best_qn[e] = best_qn[c]; } break; }
    }
  }
  int64_t best = before;
  int kv_half = 0;
  for (int a = 0; a <= n_kb; ++a) {
    if (a * kv_tile > room) break;
    const int c = int(std::min<int64_t>(n_qb, (room - a * kv_tile) / q_tile));
    const int64_t cost = std::max<int64_t>({kv_half, kv_suf[a], best_q[c], avg}) + ((a + best_qn[c]) > 0 ? kSumCost : 0);
    if (cost < best) { best = cost; r.kv = a; r.q = best_qn[c]; }
    if (a == n_kb || kblock_tiles(p, a) < 2) break;
    kv_half = std::max(kv_half, G * ((kblock_tiles(p, a) + 1) / 2));
  }
  r.floats = r.kv * kv_tile + r.q * q_tile;
  return r;
}

bool bwd_fused_fits(const Problem& p) {
  return p.dtype == 1 && dkdv_split_count(p, true) == 1 &&
         int64_t(dkdv_units(p)) + int64_t(dq_units(p)) <= fused_max_blocks(p.d);
}

hipError_t launch_bwd_fused_mfma(const Problem& p, const void* Q, const void* K, const void* V, const void* dO,
                                 const float* LSE, const float* Dv, void* dK, void* dV, float* dQacc,
                                 void* dQout, hipStream_t s) {
  if (!bwd_fused_fits(p)) return hipErrorInvalidValue;
  return p.d == 64 ? fused_d<64>(p, Q, K, V, dO, LSE, Dv, dK, dV, dQacc, dQout, s)
                   : fused_d<128>(p, Q, K, V, dO, LSE, Dv, dK, dV, dQacc, dQout, s);
}

}  // namespace fabwd

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
#include <mutex>

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
// two, dK/dV units by query range and dQ units by key range.  The two halves
// of a unit hand the output tile over through dQaccum: the first to finish
// writes an fp32 partial, the second adds it and writes the result
// (split_arrive_first).  dQaccum holds the dK/dV slots (2 BC x D floats each),
// then the dQ slots (BQ x D), then one counter word per split unit, zeroed
// by the preprocess.  Units of each kind are numbered split halves first
// ((block i, half h, head x) at 2 BH i + BH h + x), then the unsplit blocks.
template <int D, bool SOFTCAP, bool DROPOUT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(
    dkdv::kWavesPerSimd<D, SOFTCAP, DROPOUT>, dkdv::kWavesPerSimd<D, SOFTCAP, DROPOUT>))) void bwd_fused_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    const bf16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dv,
    bf16_t* __restrict__ dK, bf16_t* __restrict__ dV, float* __restrict__ dQacc, bf16_t* __restrict__ dQout, int H,
    int H_kv, int N,
    int BH_kv, int BH_q, float scale, float softcap, int wl, int wr, Dropout drop, unsigned n_dkdv, unsigned n_dq,
    int qblocks, int qq) {
  // Blocks 0 .. 2m-1 interleave the two kinds (m = the smaller count) in
  // runs of 8: blocks 16g .. 16g+7 take dK/dV units 8g .. 8g+7, blocks
  // 16g+8 .. 16g+15 dQ units 8g .. 8g+7.  The hardware places block b on XCD
  // b % 8, so every XCD gets both kinds, and unit u of either kind lands on
  // XCD u % 8: a key/value head's dK/dV and dQ units share an XCD and its L2.
  // Past the last full run the kinds alternate; the rest of the blocks
  // belong to the larger kind.
  const unsigned m = min(n_dkdv, n_dq), m8 = m & ~7u;
  const unsigned b = blockIdx.x;
  bool dq_unit;
  unsigned unit;
  if (b < 2 * m8) {
    dq_unit = ((b >> 3) & 1u) != 0;
    unit = ((b >> 4) << 3) | (b & 7u);
  } else if (b < 2 * m) {
    dq_unit = ((b - 2 * m8) & 1u) != 0;
    unit = m8 + ((b - 2 * m8) >> 1);
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
    const int64_t kv_floats = 2 * int64_t(BH_kv) * qblocks * (dkdv::BC * D);
    float* qpart = dQacc + kv_floats;
    unsigned* qcnt = reinterpret_cast<unsigned*>(qpart + int64_t(BH_q) * qq * (dq::BQ * D)) + BH_kv * qblocks;
    dq::dq_block<D, SOFTCAP, DROPOUT>(Q, K, V, dO, LSE, Dv, dQacc, dQout, H, H_kv, N, BH_q, scale, softcap, wl, wr,
                                      drop, u, khalf, qq, qpart, qcnt);
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
    const int64_t kv_floats = 2 * int64_t(BH_kv) * qblocks * (dkdv::BC * D);
    unsigned* kcnt = reinterpret_cast<unsigned*>(dQacc + kv_floats + int64_t(BH_q) * qq * (dq::BQ * D));
    dkdv::dkdv_block<D, SOFTCAP, DROPOUT>(Q, K, V, dO, LSE, Dv, dK, dV, H, H_kv, N, BH_kv, scale, softcap, wl, wr,
                                          1, qhalf >= 0 ? dQacc : nullptr, drop, u, qhalf, qblocks, kcnt);
  }
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
// costs a handoff of about kSplitCost steps and is limited by the room in
// dQaccum.  The split with the least predicted time is taken when it beats
// the unsplit launch.
// Makespan, in matrix steps, of the combined launch's units in dispatch
// order (as bwd_fused_kernel numbers them) when each goes to the workgroup
// slot that frees first, with key blocks [0, a) and the last c query blocks
// split in two.  A binary heap of slot finish times in a fixed array.
int64_t fused_makespan(const Problem& p, int a, int c) {
  // Workgroup slots: 256 CUs times the workgroups each holds (two at d = 64,
  // except with soft cap and dropout together).
  const int slots = p.d == 64 && !(p.softcap > 0.f && p.dropout) ? 512 : 256;
  const int G = p.H / p.H_kv;
  const int n_kb = (p.N + dkdv::BC - 1) / dkdv::BC, n_qb = (p.N + dq::BQ - 1) / dq::BQ;
  const int64_t BHkv = int64_t(p.B) * p.H_kv, BHq = int64_t(p.B) * p.H;
  const int64_t n1 = BHkv * (n_kb + a), n2 = BHq * (n_qb + c);
  auto halves = [](int lo, int hi, int h) { const int mid = (lo + hi + 1) / 2; return h == 0 ? hi - mid : mid - lo; };
  auto kv_weight = [&](int64_t u) -> int64_t {
    if (u < 2 * BHkv * a) {
      const int j = int(u / (2 * BHkv)), h = int((u / BHkv) & 1);
      const int k0 = j * dkdv::BC, k_end = std::min(k0 + dkdv::BC, p.N);
      return int64_t(G) * halves(std::max(0, k0 - p.wr) / dkdv::BR,
                                 (std::min(p.N, k_end + p.wl) + dkdv::BR - 1) / dkdv::BR, h);
    }
    return int64_t(G) * kblock_tiles(p, int((u - 2 * BHkv * a) / BHkv) + a);
  };
  auto q_weight = [&](int64_t u) -> int64_t {
    if (u < 2 * BHq * c) {
      const int i = n_qb - 1 - int(u / (2 * BHq)), h = int((u / BHq) & 1);
      const int q0 = i * dq::BQ, q_hi = std::min(q0 + dq::BQ, p.N) - 1;
      return halves(std::max(0, q0 - p.wl) / dq::BK, (std::min(p.N, q_hi + p.wr + 1) + dq::BK - 1) / dq::BK, h);
    }
    return qblock_steps(p, n_qb - 1 - (int((u - 2 * BHq * c) / BHq) + c));
  };
  int64_t heap[512];
  for (int k = 0; k < slots; ++k) heap[k] = 0;
  auto place = [&](int64_t w) {  // replace the minimum (root) by root + w, sift down
    int64_t v = heap[0] + w;
    int k = 0;
    for (;;) {
      int l = 2 * k + 1, m = k;
      if (l < slots && heap[l] < v) m = l;
      if (l + 1 < slots && heap[l + 1] < (m == k ? v : heap[m])) m = l + 1;
      if (m == k) break;
      heap[k] = heap[m];
      k = m;
    }
    heap[k] = v;
  };
  // The dispatch order of bwd_fused_kernel: runs of 8 of each kind, then
  // alternating, then the rest of the larger kind.
  const int64_t m = std::min(n1, n2), m8 = m & ~int64_t(7);
  for (int64_t u0 = 0; u0 < m8; u0 += 8) {
    for (int64_t u = u0; u < u0 + 8; ++u) place(kv_weight(u));
    for (int64_t u = u0; u < u0 + 8; ++u) place(q_weight(u));
  }
  for (int64_t u = m8; u < m; ++u) {
    place(kv_weight(u));
    place(q_weight(u));
  }
  for (int64_t u = m; u < n1; ++u) place(kv_weight(u));
  for (int64_t u = m; u < n2; ++u) place(q_weight(u));
  int64_t span = 0;
  for (int k = 0; k < slots; ++k) span = std::max(span, heap[k]);
  return span;
}

FusedSplit fused_split_choice(const Problem& p) {
  FusedSplit r;
  constexpr int64_t kComputeUnits = 256;
  const int64_t kSplitCost = p.d == 128 ? 2 : 4;
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
  // Room: B*H*N*d floats; a split key block takes a slot of 2 BC x d floats
  // and a counter word per kv head, a split query block a slot of BQ x d
  // floats and a counter per query head.
  const int64_t room = BHq * p.N * p.d;
  const int64_t kv_tile = BHkv * (2 * dkdv::BC * p.d + 1), q_tile = BHq * (int64_t(dq::BQ) * p.d + 1);
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
    const int64_t cost = std::max<int64_t>({kv_half, kv_suf[a], best_q[c], avg}) + ((a + best_qn[c]) > 0 ? kSplitCost : 0);
    if (cost < best) { best = cost; r.kv = a; r.q = best_qn[c]; }
    if (a == n_kb || kblock_tiles(p, a) < 2) break;
    kv_half = std::max(kv_half, G * ((kblock_tiles(p, a) + 1) / 2));
  }
  if (r.kv + r.q == 0) return r;
  // The bound above misses how whole units pack onto the compute units, and
  // the chip runs idle units' neighbours faster (it is power-limited), so a
  // split pays less than the critical path alone says: keep it only if the
  // list-scheduled makespan drops to kKeepRatio or less (measured: the
  // splits that paid predicted 0.67-0.69, those that lost 0.75 and 0.90).
  constexpr int64_t kKeepNum = 72, kKeepDen = 100;
  if (fused_makespan(p, r.kv, r.q) * kKeepDen > fused_makespan(p, 0, 0) * kKeepNum) return FusedSplit{};
  r.counter_off = BHkv * r.kv * 2 * dkdv::BC * p.d + BHq * r.q * int64_t(dq::BQ) * p.d;
  r.counters = int(BHkv * r.kv + BHq * r.q);
  r.floats = r.counter_off + r.counters;
  return r;
}

// The choice depends only on the shape and band; a few recent ones are kept
// (fixed table, no allocation), since every launch and its preprocess ask.
FusedSplit fused_split(const Problem& p, bool with_dq) {
  if (!with_dq || p.dtype != 1 || !bwd_fused_fits(p)) return FusedSplit{};
  struct Entry {
    int B = -1, H, H_kv, N, d, wl, wr;
    bool narrow;  // one workgroup per CU at d = 64 (soft cap with dropout)
    FusedSplit v;
  };
  const bool narrow = p.softcap > 0.f && p.dropout;
  static Entry cache[16];
  static std::mutex mu;
  const unsigned slot = (unsigned(p.B) * 131u + unsigned(p.H) * 31u + unsigned(p.H_kv) * 7u + unsigned(p.N) * 3u +
                         unsigned(p.d) + unsigned(p.wl) * 17u + unsigned(p.wr) * 13u) % 16u;
  {
    std::lock_guard<std::mutex> lock(mu);
    const Entry& e = cache[slot];
    if (e.B == p.B && e.H == p.H && e.H_kv == p.H_kv && e.N == p.N && e.d == p.d && e.wl == p.wl && e.wr == p.wr &&
        e.narrow == narrow)
      return e.v;
  }
  const FusedSplit v = fused_split_choice(p);
  std::lock_guard<std::mutex> lock(mu);
  Entry& e = cache[slot];
  e.B = p.B; e.H = p.H; e.H_kv = p.H_kv; e.N = p.N; e.d = p.d; e.wl = p.wl; e.wr = p.wr;
  e.narrow = narrow;
  e.v = v;
  return v;
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

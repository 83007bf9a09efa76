// Kernel launch helpers, one explicit instantiation per (dtype, op) in the
// launch_<dtype>_<op>.hip translation units (compiled in parallel).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>

#include "kernels.h"

namespace ar {

// Optional caller events recorded at a launch's own start and end.
struct Evs {
  hipEvent_t start = nullptr, stop = nullptr;
};

// Leaf batch for P leaves per tree: the size in [2, 8] that leaves the fewest
// empty slots in the last batch (larger on ties); 1 for single-leaf trees.
inline int leaf_batch(int P) {
  if (P <= 1) return 1;  // single-leaf trees (all-gather copies): one load, no clamped repeats
  int best = 8, waste = 1 << 30;
  for (int b = 8; b >= 2; --b) {
    int w = (P + b - 1) / b * b - P;
    if (w < waste) { waste = w; best = b; }
  }
  return best;
}

// P: ranks (LDS staging); leaves: the most leaves of one tree (leaf batch).
template <int DT, int OPK>
hipError_t launch_fused_t(int D, int TM, int P, int leaves, int64_t nitems, const RankPtrs& ptrs, const Item* items,
                          const int32_t* prog, hipStream_t st, Evs ev, bool ordered = false);
template <int DT, int OPK>
hipError_t launch_fused_strided_t(int D, int TM, int64_t nitems, const RankPtrs& ptrs, const SItem* items,
                                  const int32_t* prog, int64_t stride, hipStream_t st, Evs ev);
template <int DT, int OPK>
hipError_t launch_fused_rows_t(int D, int TM, const RankPtrs& ptrs, const int32_t* prog, const uint8_t* tab,
                               int64_t first, int64_t total, int n, int R, int P, int iters, int64_t max_blocks,
                               hipStream_t st, Evs ev);
// chain: the reference tree is a chain of combinations (D is then ignored).
template <int DT, int OPK>
hipError_t launch_fused_rows_vec_t(int D, bool chain, const RankPtrs& ptrs, const int32_t* prog, const uint8_t* tab,
                                   int64_t nvec, int n, int R, int P, int64_t max_blocks, hipStream_t st, Evs ev);
template <int DT, int OPK>
hipError_t launch_fused_multi_t(int nl, int64_t nitems, const MultiPtrs& mp, const Item* items, const int32_t* tab,
                                hipStream_t st, Evs ev);
template <int DT, int OPK>
hipError_t launch_fused_fixed_t(int shape, int nl, int M, int64_t nitems, const RankPtrs& ptrs, const Item* items,
                                const RankTab& tab, hipStream_t st, Evs ev);
template <int DT, int OPK>
hipError_t launch_literal_t(int64_t nwork, const RankPtrs& ptrs, const WsDesc& ws, const LitWork* work,
                            const LitWork* packed, hipStream_t st, Evs ev);
// shared: one program for every range (blocks of kDagLanes elements over [0, total));
// otherwise nitems work items. threads: 256 or 1024; lds: dynamic LDS bytes.
template <int DT, int OPK>
hipError_t launch_fused_dag_t(bool shared, int threads, size_t lds, int64_t nitems, const RankPtrs& ptrs,
                              const Item* items, const int32_t* prog, const uint8_t* tab, int64_t total, int n,
                              int P, int vals_words, int tab_rows, int64_t max_blocks, hipStream_t st, Evs ev);
template <int DT, int OPK>
hipError_t launch_direct_t(bool vec, const RankPtrs& ptrs, int P, int64_t total, int64_t max_blocks, hipStream_t st,
                           Evs ev);

// Compute units of the current device (cached per device; 256 when HIP cannot tell).
inline int device_cus() {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  cache[dev] = cus;
  return cus;
}

// Whether `blocks` workgroups of four vectors per thread fill whole rounds of
// the compute units well enough: launches of a few hundred workgroups run as
// long as their busiest compute unit, so a last round of a few workgroups
// (259 for 256 units: 6 ranks x 10^4 x 106 fp32) costs nearly a whole one;
// twice the workgroups of two vectors then spread evenly (12.2 -> 10.1 us).
inline bool four_vectors_fit(int64_t blocks, int cus) {
  const int64_t rest = blocks % cus;
  return blocks <= cus || rest == 0 || rest >= cus / 2;
}

#ifdef AR_LAUNCH_DEFINITIONS
// Launches go through hipExtLaunchKernelGGL so that optional caller events can
// be recorded at the kernel's own start and end.

// Leaf batch for P leaves per tree: the size in [2, 8] that leaves the fewest
// empty slots in the last batch (larger on ties); 1 for single-leaf trees. Single-tree programs are
// compiled for the (stack depth, batch) pairs that occur; others use 8.

template <int DT, int OPK, int D, int B, bool IDL = false>
void fused1(const dim3& g, const dim3& b, hipStream_t st, Evs ev, const RankPtrs& ptrs, const Item* items,
            const int32_t* prog) {
  hipExtLaunchKernelGGL((k_fused<DT, OPK, D, 1, B, IDL>), g, b, 0, st, ev.start, ev.stop, 0, ptrs, items, prog);
}

// One tree over at most 32 ranks with the buffers passed in leaf order, then
// output order (`ordered`): the leaves' ranks need no program read.
template <int DT, int OPK>
void fused_ordered(int D, int B, const dim3& g, const dim3& b, hipStream_t st, Evs ev, const RankPtrs& ptrs,
                   const Item* items, const int32_t* prog) {
  if (D == 2) {
    switch (B) {
      case 1: fused1<DT, OPK, 2, 1, true>(g, b, st, ev, ptrs, items, prog); break;
      case 2: fused1<DT, OPK, 2, 2, true>(g, b, st, ev, ptrs, items, prog); break;
      case 3: fused1<DT, OPK, 2, 3, true>(g, b, st, ev, ptrs, items, prog); break;
      case 4: fused1<DT, OPK, 2, 4, true>(g, b, st, ev, ptrs, items, prog); break;
      case 5: fused1<DT, OPK, 2, 5, true>(g, b, st, ev, ptrs, items, prog); break;
      case 6: fused1<DT, OPK, 2, 6, true>(g, b, st, ev, ptrs, items, prog); break;
      case 7: fused1<DT, OPK, 2, 7, true>(g, b, st, ev, ptrs, items, prog); break;
      default: fused1<DT, OPK, 2, 8, true>(g, b, st, ev, ptrs, items, prog); break;
    }
  } else if (D == 4) {
    switch (B) {
      case 3: fused1<DT, OPK, 4, 3, true>(g, b, st, ev, ptrs, items, prog); break;
      case 4: fused1<DT, OPK, 4, 4, true>(g, b, st, ev, ptrs, items, prog); break;
      case 5: fused1<DT, OPK, 4, 5, true>(g, b, st, ev, ptrs, items, prog); break;
      case 6: fused1<DT, OPK, 4, 6, true>(g, b, st, ev, ptrs, items, prog); break;
      case 7: fused1<DT, OPK, 4, 7, true>(g, b, st, ev, ptrs, items, prog); break;
      default: fused1<DT, OPK, 4, 8, true>(g, b, st, ev, ptrs, items, prog); break;
    }
  } else if (D == 6) {
    switch (B) {
      case 5: fused1<DT, OPK, 6, 5, true>(g, b, st, ev, ptrs, items, prog); break;
      case 6: fused1<DT, OPK, 6, 6, true>(g, b, st, ev, ptrs, items, prog); break;
      case 7: fused1<DT, OPK, 6, 7, true>(g, b, st, ev, ptrs, items, prog); break;
      default: fused1<DT, OPK, 6, 8, true>(g, b, st, ev, ptrs, items, prog); break;
    }
  } else {
    switch (B) {
      case 5: fused1<DT, OPK, 8, 5, true>(g, b, st, ev, ptrs, items, prog); break;
      case 6: fused1<DT, OPK, 8, 6, true>(g, b, st, ev, ptrs, items, prog); break;
      case 7: fused1<DT, OPK, 8, 7, true>(g, b, st, ev, ptrs, items, prog); break;
      default: fused1<DT, OPK, 8, 8, true>(g, b, st, ev, ptrs, items, prog); break;
    }
  }
}

template <int DT, int OPK>
hipError_t launch_fused_t(int D, int TM, int P, int leaves, int64_t nitems, const RankPtrs& ptrs, const Item* items,
                          const int32_t* prog, hipStream_t st, Evs ev, bool ordered) {
  const dim3 g{unsigned(nitems), 1, 1};
  const dim3 b{unsigned(kThreads), 1, 1};
  if (TM == 1 && ordered && D <= 8) {
    fused_ordered<DT, OPK>(D, leaf_batch(std::min(P, leaves)), g, b, st, ev, ptrs, items, prog);
    return hipGetLastError();
  }
  if (TM == 1) {
    const int B = leaf_batch(std::min(P, leaves));
    if (D == 2) {
      switch (B) {
        case 1: fused1<DT, OPK, 2, 1>(g, b, st, ev, ptrs, items, prog); break;
        case 2: fused1<DT, OPK, 2, 2>(g, b, st, ev, ptrs, items, prog); break;
        case 3: fused1<DT, OPK, 2, 3>(g, b, st, ev, ptrs, items, prog); break;
        case 4: fused1<DT, OPK, 2, 4>(g, b, st, ev, ptrs, items, prog); break;
        case 5: fused1<DT, OPK, 2, 5>(g, b, st, ev, ptrs, items, prog); break;
        case 6: fused1<DT, OPK, 2, 6>(g, b, st, ev, ptrs, items, prog); break;
        case 7: fused1<DT, OPK, 2, 7>(g, b, st, ev, ptrs, items, prog); break;
        default: fused1<DT, OPK, 2, 8>(g, b, st, ev, ptrs, items, prog); break;
      }
    } else if (D == 4) {
      switch (B) {
        case 3: fused1<DT, OPK, 4, 3>(g, b, st, ev, ptrs, items, prog); break;
        case 4: fused1<DT, OPK, 4, 4>(g, b, st, ev, ptrs, items, prog); break;
        case 5: fused1<DT, OPK, 4, 5>(g, b, st, ev, ptrs, items, prog); break;
        case 6: fused1<DT, OPK, 4, 6>(g, b, st, ev, ptrs, items, prog); break;
        case 7: fused1<DT, OPK, 4, 7>(g, b, st, ev, ptrs, items, prog); break;
        default: fused1<DT, OPK, 4, 8>(g, b, st, ev, ptrs, items, prog); break;
      }
    } else if (D == 8) {
      switch (B) {
        case 5: fused1<DT, OPK, 8, 5>(g, b, st, ev, ptrs, items, prog); break;
        case 6: fused1<DT, OPK, 8, 6>(g, b, st, ev, ptrs, items, prog); break;
        case 7: fused1<DT, OPK, 8, 7>(g, b, st, ev, ptrs, items, prog); break;
        default: fused1<DT, OPK, 8, 8>(g, b, st, ev, ptrs, items, prog); break;
      }
    } else {
      fused1<DT, OPK, 16, 8>(g, b, st, ev, ptrs, items, prog);
    }
  } else if (P <= kMaxStagedRanks) {
    const uint32_t lds = uint32_t(P) * kThreads * sizeof(u32x4);
    switch (D) {
      case 2: hipExtLaunchKernelGGL((k_fused_staged<DT, OPK, 2>), g, b, lds, st, ev.start, ev.stop, 0, ptrs, items, prog, P); break;
      case 4: hipExtLaunchKernelGGL((k_fused_staged<DT, OPK, 4>), g, b, lds, st, ev.start, ev.stop, 0, ptrs, items, prog, P); break;
      default: hipExtLaunchKernelGGL((k_fused_staged<DT, OPK, 8>), g, b, lds, st, ev.start, ev.stop, 0, ptrs, items, prog, P); break;
    }
  } else {
    switch (D) {
      case 2: hipExtLaunchKernelGGL((k_fused<DT, OPK, 2, kMaxFusedTrees, 8>), g, b, 0, st, ev.start, ev.stop, 0, ptrs, items, prog); break;
      case 4: hipExtLaunchKernelGGL((k_fused<DT, OPK, 4, kMaxFusedTrees, 8>), g, b, 0, st, ev.start, ev.stop, 0, ptrs, items, prog); break;
      default: hipExtLaunchKernelGGL((k_fused<DT, OPK, 8, kMaxFusedTrees, 8>), g, b, 0, st, ev.start, ev.stop, 0, ptrs, items, prog); break;
    }
  }
  return hipGetLastError();
}

// shape: SH_BALANCED (nl = 4 or 8), SH_CHAIN (nl = 1..8) or SH_STACK (nl =
// 3..8) leaves per tree; M = 2 or 4 vectors per thread.
template <int DT, int OPK>
hipError_t launch_fused_fixed_t(int shape, int nl, int M, int64_t nitems, const RankPtrs& ptrs, const Item* items,
                                const RankTab& tab, hipStream_t st, Evs ev) {
  const dim3 g{unsigned(nitems), 1, 1};
  const dim3 b{unsigned(kThreads), 1, 1};
  FixPtrs fp;
  std::memset(&fp, 0, sizeof(fp));
  for (int r = 0; r < kMaxTabRanges; ++r) {
    for (int k = 0; k < 8; ++k) {
      fp.leaf[r][k] = ptrs.p[tab.leaf[r][k]];
      fp.out[r][k] = ptrs.p[tab.out[r][k]];
    }
    fp.nouts[r] = tab.nouts[r];
  }
  for (int k = 0; k < 8; ++k) fp.nc[k] = tab.nc[k];
  fp.div = ptrs.div;
  fp.xcd = ptrs.xcd;
#define AR_FIX(SH_, M_, NL_) \
  hipExtLaunchKernelGGL((k_fused_fixed<DT, OPK, SH_, M_, NL_>), g, b, 0, st, ev.start, ev.stop, 0, fp, items)
#define AR_CHAIN(M_)                                       \
  switch (nl) {                                            \
    case 1: AR_FIX(SH_CHAIN, M_, 1); break;                \
    case 2: AR_FIX(SH_CHAIN, M_, 2); break;                \
    case 3: AR_FIX(SH_CHAIN, M_, 3); break;                \
    case 4: AR_FIX(SH_CHAIN, M_, 4); break;                \
    case 5: AR_FIX(SH_CHAIN, M_, 5); break;                \
    case 6: AR_FIX(SH_CHAIN, M_, 6); break;                \
    case 7: AR_FIX(SH_CHAIN, M_, 7); break;                \
    default: AR_FIX(SH_CHAIN, M_, 8); break;               \
  }
#define AR_STK(M_)                                         \
  switch (nl) {                                            \
    case 3: AR_FIX(SH_STACK, M_, 3); break;                \
    case 4: AR_FIX(SH_STACK, M_, 4); break;                \
    case 5: AR_FIX(SH_STACK, M_, 5); break;                \
    case 6: AR_FIX(SH_STACK, M_, 6); break;                \
    case 7: AR_FIX(SH_STACK, M_, 7); break;                \
    default: AR_FIX(SH_STACK, M_, 8); break;               \
  }
  if (shape == SH_STACK) {
    if (M == 4) { AR_STK(4) } else { AR_STK(2) }
  } else if (shape == SH_BALANCED) {
    if (M == 4) {
      if (nl == 4) AR_FIX(SH_BALANCED, 4, 4); else AR_FIX(SH_BALANCED, 4, 8);
    } else {
      if (nl == 4) AR_FIX(SH_BALANCED, 2, 4); else AR_FIX(SH_BALANCED, 2, 8);
    }
  } else {
    if (M == 4) { AR_CHAIN(4) } else { AR_CHAIN(2) }
  }
#undef AR_STK
#undef AR_CHAIN
#undef AR_FIX
  return hipGetLastError();
}

template <int DT, int OPK>
hipError_t launch_fused_multi_t(int nl, int64_t nitems, const MultiPtrs& mp, const Item* items, const int32_t* tab,
                                hipStream_t st, Evs ev) {
  const dim3 g{unsigned(nitems), 1, 1};
  const dim3 b{unsigned(kThreads), 1, 1};
  const uint32_t lds = uint32_t(nl) * kThreads * sizeof(u32x4);
#define AR_MT(NL_) hipExtLaunchKernelGGL((k_fused_multi<DT, OPK, NL_>), g, b, lds, st, ev.start, ev.stop, 0, mp, items, tab)
  switch (nl) {
    case 3: AR_MT(3); break;
    case 4: AR_MT(4); break;
    case 5: AR_MT(5); break;
    case 6: AR_MT(6); break;
    case 7: AR_MT(7); break;
    default: AR_MT(8); break;
  }
#undef AR_MT
  return hipGetLastError();
}

template <int DT, int OPK, int D, int TM>
hipError_t rows_d(const RankPtrs& ptrs, const int32_t* prog, const uint8_t* tab, int64_t first, int64_t total, int n,
                  int R, int P, int iters, int64_t max_blocks, hipStream_t st, Evs ev) {
  const int64_t unit = int64_t(iters) * kThreads;  // elements per workgroup
  const int64_t blocks = (total - first + unit - 1) / unit;
  const size_t lds = size_t(R * (P | 1) + P) * sizeof(void*) + size_t(n);
  for (int64_t b0 = 0; b0 < blocks; b0 += max_blocks) {  // workgroups are independent
    const int64_t cnt = std::min(max_blocks, blocks - b0);
    const Evs ei{b0 == 0 ? ev.start : nullptr, b0 + cnt >= blocks ? ev.stop : nullptr};
    hipExtLaunchKernelGGL((k_fused_rows<DT, OPK, D, TM, kLeafBatch>), dim3(unsigned(cnt)), dim3(kThreads), lds, st,
                          ei.start, ei.stop, 0, ptrs, prog, tab, first + b0 * unit, total, int32_t(n), int32_t(R),
                          int32_t(P), int32_t(iters));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Workgroups of `fn` (with `lds` bytes of dynamic LDS) that the current device
// holds at once: compute units x resident workgroups per unit, cached per
// kernel, LDS size and device. 0 when HIP cannot tell.
inline int64_t resident_blocks(const void* fn, int threads, size_t lds) {
  static std::mutex mu;
  static std::map<std::tuple<const void*, int, size_t, int>, int64_t> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lk(mu);
  const auto key = std::make_tuple(fn, threads, lds, dev);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int cus = 0, per = 0;
  int64_t v = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fn, threads, lds) == hipSuccess)
    v = int64_t(cus) * per;
  cache[key] = v;
  return v;
}

template <int DT, int OPK, int D, int K, int G, bool REG, bool CHAIN>
hipError_t rows_vec_d(const RankPtrs& ptrs, const int32_t* prog, const uint8_t* tab, int64_t nvec, int n, int R, int P,
                      int64_t max_blocks, hipStream_t st, Evs ev) {
  const int64_t npos = (nvec + 16 * K - 1) / (16 * K);
  // one launch: each wave walks its positions (16 K vectors) with the stride of
  // every wave of the grid, which holds at most what the device keeps resident.
  // Four waves per workgroup share the tables; when the device holds more than
  // half the positions at once, single-wave workgroups spread them evenly.
  const void* fn = reinterpret_cast<const void*>(&k_fused_rows_vec<DT, OPK, D, kLeafBatch, K, G, REG, CHAIN>);
  auto lds_of = [&](int waves) {
    if (REG) return size_t(n + 1) / 2 * 8;  // the packed leaf ranks of each offset
    return size_t(waves) * (P + 1) * 64 * K * sizeof(uint32_t) + size_t(K == 1 ? 4 * G : 0) * sizeof(void*) +
           size_t((n + 7) / 8 * 8 + R * P + 7) / 8 * 8;
  };
  int waves = 4;
  int64_t res = resident_blocks(fn, 64 * waves, lds_of(waves));
  if (res > 0 && npos < 2 * res * waves) {
    waves = 1;
    res = resident_blocks(fn, 64, lds_of(1));
  }
  int64_t blocks = (npos + waves - 1) / waves;
  if (res > 0) blocks = std::min(blocks, res);
  blocks = std::max<int64_t>(1, std::min(blocks, max_blocks));
  hipExtLaunchKernelGGL((k_fused_rows_vec<DT, OPK, D, kLeafBatch, K, G, REG, CHAIN>), dim3(unsigned(blocks)), dim3(64 * waves),
                        lds_of(waves), st, ev.start, ev.stop, 0, ptrs, prog, tab, nvec, int32_t(n), int32_t(R),
                        int32_t(P));
  return hipGetLastError();
}

// At most 8 ranks: four elements per lane, one load per rank (G = P), in
// registers up to kRowsRegMaxRanks ranks, else staged; 9..32 ranks: one element
// per lane, G = ceil(P / 4) loads of four ranks each.
template <int DT, int OPK, int D, int G, bool CHAIN>
hipError_t rows_vec_few(const RankPtrs& ptrs, const int32_t* prog, const uint8_t* tab, int64_t nvec, int n, int R, int P,
                        int64_t max_blocks, hipStream_t st, Evs ev) {
  constexpr bool reg = G <= kRowsRegMaxRanks;
  return rows_vec_d<DT, OPK, D, 4, G, reg, CHAIN && !reg>(ptrs, prog, tab, nvec, n, R, P, max_blocks, st, ev);
}
// CHAIN: the reference tree is a chain (evaluated without the register stack
// in the staged forms; D is then 2)
template <int DT, int OPK, int D, bool CHAIN>
hipError_t rows_vec_g(const RankPtrs& ptrs, const int32_t* prog, const uint8_t* tab, int64_t nvec, int n, int R, int P,
                      int64_t max_blocks, hipStream_t st, Evs ev) {
#define AR_RF(G_) return rows_vec_few<DT, OPK, D, G_, CHAIN>(ptrs, prog, tab, nvec, n, R, P, max_blocks, st, ev)
#define AR_RV(G_) return rows_vec_d<DT, OPK, D, 1, G_, false, CHAIN>(ptrs, prog, tab, nvec, n, R, P, max_blocks, st, ev)
  switch (P) {
    case 1: AR_RF(1);
    case 2: AR_RF(2);
    case 3: AR_RF(3);
    case 4: AR_RF(4);
    case 5: AR_RF(5);
    case 6: AR_RF(6);
    case 7: AR_RF(7);
    case 8: AR_RF(8);
    default: break;
  }
  switch ((P + 3) / 4) {
    case 3: AR_RV(3);
    case 4: AR_RV(4);
    case 5: AR_RV(5);
    case 6: AR_RV(6);
    case 7: AR_RV(7);
    default: AR_RV(8);
  }
#undef AR_RF
#undef AR_RV
}

template <int DT, int OPK>
hipError_t launch_fused_rows_vec_t(int D, bool chain, const RankPtrs& ptrs, const int32_t* prog, const uint8_t* tab,
                                   int64_t nvec, int n, int R, int P, int64_t max_blocks, hipStream_t st, Evs ev) {
  if constexpr (TT<DT>::V != 4) {
    return hipErrorInvalidValue;  // 4-byte elements only
  } else {
    if (P < 1 || P > 32) return hipErrorInvalidValue;
    if (chain) return rows_vec_g<DT, OPK, 2, true>(ptrs, prog, tab, nvec, n, R, P, max_blocks, st, ev);
    switch (D) {
      case 2: return rows_vec_g<DT, OPK, 2, false>(ptrs, prog, tab, nvec, n, R, P, max_blocks, st, ev);
      case 4: return rows_vec_g<DT, OPK, 4, false>(ptrs, prog, tab, nvec, n, R, P, max_blocks, st, ev);
      case 6: return rows_vec_g<DT, OPK, 6, false>(ptrs, prog, tab, nvec, n, R, P, max_blocks, st, ev);
      case 8: return rows_vec_g<DT, OPK, 8, false>(ptrs, prog, tab, nvec, n, R, P, max_blocks, st, ev);
      default: return rows_vec_g<DT, OPK, 16, false>(ptrs, prog, tab, nvec, n, R, P, max_blocks, st, ev);
    }
  }
}

template <int DT, int OPK>
hipError_t launch_fused_rows_t(int D, int TM, const RankPtrs& ptrs, const int32_t* prog, const uint8_t* tab,
                               int64_t first, int64_t total, int n, int R, int P, int iters, int64_t max_blocks,
                               hipStream_t st, Evs ev) {
#define AR_ROWS(DD, TT_) \
  return rows_d<DT, OPK, DD, TT_>(ptrs, prog, tab, first, total, n, R, P, iters, max_blocks, st, ev)
  if (TM == 1) {
    switch (D) {
      case 2: AR_ROWS(2, 1);
      case 4: AR_ROWS(4, 1);
      case 8: AR_ROWS(8, 1);
      default: AR_ROWS(16, 1);
    }
  }
  switch (D) {
    case 2: AR_ROWS(2, kMaxFusedTrees);
    case 4: AR_ROWS(4, kMaxFusedTrees);
    default: AR_ROWS(8, kMaxFusedTrees);
  }
#undef AR_ROWS
}

template <int DT, int OPK>
hipError_t launch_fused_strided_t(int D, int TM, int64_t nitems, const RankPtrs& ptrs, const SItem* items,
                                  const int32_t* prog, int64_t stride, hipStream_t st, Evs ev) {
  const dim3 g{unsigned(nitems), 1, 1};
  const dim3 b{unsigned(kThreads), 1, 1};
#define AR_STRIDED(DD, TT_) \
  hipExtLaunchKernelGGL((k_fused_strided<DT, OPK, DD, TT_, kLeafBatch>), g, b, 0, st, ev.start, ev.stop, 0, ptrs, \
                        items, prog, stride)
  if (TM == 1) {
    switch (D) {
      case 2: AR_STRIDED(2, 1); break;
      case 4: AR_STRIDED(4, 1); break;
      case 8: AR_STRIDED(8, 1); break;
      default: AR_STRIDED(16, 1); break;
    }
  } else {
    switch (D) {
      case 2: AR_STRIDED(2, kMaxFusedTrees); break;
      case 4: AR_STRIDED(4, kMaxFusedTrees); break;
      default: AR_STRIDED(8, kMaxFusedTrees); break;
    }
  }
#undef AR_STRIDED
  return hipGetLastError();
}

template <int DT, int OPK>
hipError_t launch_literal_t(int64_t nwork, const RankPtrs& ptrs, const WsDesc& ws, const LitWork* work,
                            const LitWork* packed, hipStream_t st, Evs ev) {
  hipExtLaunchKernelGGL((k_literal<DT, OPK>), dim3(unsigned(nwork)), dim3(kThreads), 0, st, ev.start, ev.stop, 0,
                        ptrs, ws, work, packed);
  return hipGetLastError();
}

template <int DT, int OPK, bool SH>
hipError_t dag_d(int threads, size_t lds, int64_t nitems, const RankPtrs& ptrs, const Item* items,
                 const int32_t* prog, const uint8_t* tab, int64_t total, int n, int P, int vals_words,
                 int tab_rows, int64_t max_blocks, hipStream_t st, Evs ev) {
  static bool raised = false;  // LDS beyond 64 KB per workgroup needs the kernel's attribute raised once
  if (lds > 65536 && !raised) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_fused_dag<DT, OPK, SH>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
    raised = true;
  }
  const int64_t blocks = SH ? (total + kDagLanes - 1) / kDagLanes : nitems;
  for (int64_t b0 = 0; b0 < blocks; b0 += max_blocks) {  // workgroups are independent
    const int64_t cnt = std::min(max_blocks, blocks - b0);
    const Evs ei{b0 == 0 ? ev.start : nullptr, b0 + cnt >= blocks ? ev.stop : nullptr};
    hipExtLaunchKernelGGL((k_fused_dag<DT, OPK, SH>), dim3(unsigned(cnt)), dim3(unsigned(threads)), uint32_t(lds), st,
                          ei.start, ei.stop, 0, ptrs, SH ? items : items + b0, prog, tab, b0 * kDagLanes, total,
                          int32_t(n), int32_t(P), int32_t(vals_words), int32_t(tab_rows));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int DT, int OPK>
hipError_t launch_fused_dag_t(bool shared, int threads, size_t lds, int64_t nitems, const RankPtrs& ptrs,
                              const Item* items, const int32_t* prog, const uint8_t* tab, int64_t total, int n,
                              int P, int vals_words, int tab_rows, int64_t max_blocks, hipStream_t st, Evs ev) {
  if (shared)
    return dag_d<DT, OPK, true>(threads, lds, nitems, ptrs, items, prog, tab, total, n, P, vals_words, tab_rows,
                                max_blocks, st, ev);
  return dag_d<DT, OPK, false>(threads, lds, nitems, ptrs, items, prog, tab, total, n, P, vals_words, tab_rows,
                               max_blocks, st, ev);
}

// One launch per run of at most max_blocks workgroups; each launch gets the
// rank pointers advanced to its first element. The vector path's element tail
// (past the last whole vector) goes to block 0 of the last launch.
template <int DT, int OPK, int B, int MD>
hipError_t direct_b(bool vec, const RankPtrs& ptrs, int P, int64_t total, int64_t max_blocks, hipStream_t st,
                    Evs ev) {
  constexpr int V = TT<DT>::V;
  constexpr int64_t elt = sizeof(typename TT<DT>::S);
  const int64_t whole = vec ? total / V * V : total;  // elements the workgroups cover
  // vectors per workgroup: kThreads x MD, or, for a launch of a few rounds of
  // workgroups over the compute units, the smallest multiple of 16 that needs
  // no more rounds, so that every unit gets the same count (6 ranks x 10^4 x
  // 106 fp32: 4.33 -> 5.59 TB/s; 24 ranks: 5.19 -> 5.51)
  int64_t per_block = int64_t(kThreads) * MD;
  if (vec) {
    const int64_t nvec = whole / V, full = (nvec + per_block - 1) / per_block;
    if (full > 0 && full <= max_blocks) {
      const int64_t cus = device_cus(), cap = (full + cus - 1) / cus * cus;
      per_block = std::min(per_block, std::max<int64_t>(64, ((nvec + cap - 1) / cap + 15) / 16 * 16));
    }
  }
  const int64_t unit = vec ? per_block * V : int64_t(kThreads);  // elements per workgroup
  const int64_t per = max_blocks * unit;
  RankPtrs pp = ptrs;
  int64_t done = 0;
  do {
    const int64_t len = std::min(per, whole - done);
    const bool last = done + len >= whole;
    for (int p = 0; p < P; ++p) pp.p[p] = static_cast<char*>(ptrs.p[p]) + done * elt;
    const Evs ei{done == 0 ? ev.start : nullptr, last ? ev.stop : nullptr};
    const int64_t blocks = std::max<int64_t>(1, (len + unit - 1) / unit);
    if (vec) {
      hipExtLaunchKernelGGL((k_direct<DT, OPK, true, B, MD>), dim3(unsigned(blocks)), dim3(kThreads), 0, st,
                            ei.start, ei.stop, 0, pp, P, len / V, last ? total - done : len, int(per_block));
    } else {
      hipExtLaunchKernelGGL((k_direct<DT, OPK, false, B>), dim3(unsigned(blocks)), dim3(kThreads), 0, st, ei.start,
                            ei.stop, 0, pp, P, int64_t(0), len, kThreads);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    done += len;
  } while (done < whole);
  return hipSuccess;
}

template <int DT, int OPK, int MD>
hipError_t direct_m(bool vec, const RankPtrs& ptrs, int P, int64_t total, int64_t max_blocks, hipStream_t st,
                    Evs ev) {
  switch (leaf_batch(P)) {
    case 2: return direct_b<DT, OPK, 2, MD>(vec, ptrs, P, total, max_blocks, st, ev);
    case 3: return direct_b<DT, OPK, 3, MD>(vec, ptrs, P, total, max_blocks, st, ev);
    case 4: return direct_b<DT, OPK, 4, MD>(vec, ptrs, P, total, max_blocks, st, ev);
    case 5: return direct_b<DT, OPK, 5, MD>(vec, ptrs, P, total, max_blocks, st, ev);
    case 6: return direct_b<DT, OPK, 6, MD>(vec, ptrs, P, total, max_blocks, st, ev);
    case 7: return direct_b<DT, OPK, 7, MD>(vec, ptrs, P, total, max_blocks, st, ev);
    default: return direct_b<DT, OPK, 8, MD>(vec, ptrs, P, total, max_blocks, st, ev);
  }
}

// Four vectors per thread for launches of at most 2^19 vectors (a few hundred
// workgroups) with at most 8 ranks; one with 9..32 ranks; two otherwise. Latency-bound launches
// (at most 2^14 elements) with 9..32 ranks fetch every rank in one batch
// instead of rounds of 8, each of which waits on memory.
template <int DT, int OPK>
hipError_t launch_direct_t(bool vec, const RankPtrs& ptrs, int P, int64_t total, int64_t max_blocks, hipStream_t st,
                           Evs ev) {
  if (P > 8 && P <= 32 && total <= (int64_t(1) << 14)) {
    if (P <= 16) return direct_b<DT, OPK, 16, 1>(vec, ptrs, P, total, max_blocks, st, ev);
    return direct_b<DT, OPK, 32, 1>(vec, ptrs, P, total, max_blocks, st, ev);
  }
  if (vec && P <= 8 && total / TT<DT>::V <= (int64_t(1) << 19) &&
      four_vectors_fit((total / TT<DT>::V + 4 * kThreads - 1) / (4 * kThreads), device_cus()))
    return direct_m<DT, OPK, 4>(vec, ptrs, P, total, max_blocks, st, ev);
  // 9..32 ranks: one vector per thread, twice the workgroups (24 ranks x 1.06M
  // fp32: 41.3 -> 39.1 us); many more ranks keep two (192 ranks: 137 vs 147 us)
  if (P > 8 && P <= 32) return direct_m<DT, OPK, 1>(vec, ptrs, P, total, max_blocks, st, ev);
  return direct_m<DT, OPK, kDirectM>(vec, ptrs, P, total, max_blocks, st, ev);
}


#define AR_INSTANTIATE_LAUNCHES(DT, OPK)                                                                    \
  template hipError_t launch_fused_t<DT, OPK>(int, int, int, int, int64_t, const RankPtrs&, const Item*,    \
                                              const int32_t*, hipStream_t, Evs, bool);                      \
  template hipError_t launch_fused_fixed_t<DT, OPK>(int, int, int, int64_t, const RankPtrs&, const Item*,   \
                                                    const RankTab&, hipStream_t, Evs);                      \
  template hipError_t launch_fused_multi_t<DT, OPK>(int, int64_t, const MultiPtrs&, const Item*,          \
                                                    const int32_t*, hipStream_t, Evs);                      \
  template hipError_t launch_fused_rows_t<DT, OPK>(int, int, const RankPtrs&, const int32_t*, const uint8_t*, \
                                                   int64_t, int64_t, int, int, int, int, int64_t, hipStream_t,  \
                                                   Evs);                                                        \
  template hipError_t launch_fused_rows_vec_t<DT, OPK>(int, bool, const RankPtrs&, const int32_t*,           \
                                                       const uint8_t*, int64_t, int, int, int, int64_t,        \
                                                       hipStream_t, Evs);                                       \
  template hipError_t launch_fused_strided_t<DT, OPK>(int, int, int64_t, const RankPtrs&, const SItem*,     \
                                                      const int32_t*, int64_t, hipStream_t, Evs);          \
  template hipError_t launch_literal_t<DT, OPK>(int64_t, const RankPtrs&, const WsDesc&, const LitWork*,    \
                                                const LitWork*, hipStream_t, Evs);                          \
  template hipError_t launch_fused_dag_t<DT, OPK>(bool, int, size_t, int64_t, const RankPtrs&, const Item*,  \
                                                  const int32_t*, const uint8_t*, int64_t, int, int, int, int,\
                                                  int64_t, hipStream_t, Evs);                                 \
  template hipError_t launch_direct_t<DT, OPK>(bool, const RankPtrs&, int, int64_t, int64_t, hipStream_t, Evs);
#endif  // AR_LAUNCH_DEFINITIONS

}  // namespace ar

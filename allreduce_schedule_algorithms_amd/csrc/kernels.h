// Device code for gfx950: work-item and operand layouts, fragments of 128-bit
// loads and stores, the fused replay, literal step and direct kernels.
// Included by exec.hip; nothing here runs on the host.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "sched.h"

namespace ar {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct RankPtrs {
  void* p[kMaxRanks];
  float div;    // O_AVG: the complete sum is divided by this (P), once, before the store
  int32_t xcd;  // fused replay: give each XCD a contiguous run of work items (item_index)
};

// MI355X dispatches workgroup b to XCD b % 8, and each XCD has its own L2.
// With a large fused program (many ranges with long programs, as in AHC), a
// contiguous run of items per XCD keeps each XCD's share of the program
// words in its caches; with small programs the plain order streams better.
constexpr unsigned kXcds = 8;
__device__ __forceinline__ unsigned item_index(int32_t xcd) {
  if (!xcd) return blockIdx.x;
  const unsigned nb = gridDim.x, per = (nb + kXcds - 1) / kXcds, x = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const unsigned full = nb % kXcds == 0 ? kXcds : nb % kXcds;  // XCDs that receive 'per' workgroups
  return x < full ? x * per + slot : full * per + (x - full) * (per - 1) + slot;
}

// Program words stay unchanged for the whole launch. Reading them through the
// constant address space lets the compiler use scalar loads for them even after
// the kernel's own stores, which it cannot otherwise prove leave them alone;
// they are then read in whole runs of kLeafBatch words (merged scalar loads; the
// uploaded program is padded past its last tree). Replays with several trees per
// range read their words this way (measured 40% faster at seven trees). The
// single-tree replay keeps plain pointers and per-word loads, which measured
// 3-6% faster on its 12 us launches.
typedef const __attribute__((address_space(4))) int32_t* ProgPtr;
__device__ __forceinline__ ProgPtr as_prog(const int32_t* p) { return (ProgPtr)p; }
template <typename WP> constexpr bool word_runs() { return std::is_same<WP, ProgPtr>::value; }
template <int TM> __device__ __forceinline__ auto prog_words(const int32_t* prog, int32_t tag) {
  if constexpr (TM == 1) return prog + tag;
  else return as_prog(prog) + tag;
}

// Work item: `count` > 0 is a run of vectors, < 0 a run of -count single elements;
// `start` is the element offset of its first element in every rank buffer.
struct Item {
  int64_t start;
  int32_t count;
  int32_t tag;  // program word offset (fused) or op index (literal)
};

// A vector item of the program-driven replay may cover partial vectors at a
// range's ends: its count then holds the vectors in bits 0..15, the elements
// before the range in bits 16..23 and those past it in bits 24..27 (neither is
// loaded for the range's sake nor stored).
__host__ __device__ constexpr int32_t item_count(int64_t vectors, int64_t skip, int64_t trim) {
  return int32_t(vectors | (skip << 16) | (trim << 24));
}
constexpr int32_t kItemVectorsMask = 0xffff;

constexpr int kThreads = 256;
constexpr int kLeafBatch = 8;
constexpr int kMaxFusedTrees = 8;  // distinct result trees per range the fused replay keeps in registers
constexpr int kMaxStagedRanks = 16;  // ranks whose fragments fit the LDS staging of multi-tree ranges

// ----------------------------------------------------------------------------
// element types
// ----------------------------------------------------------------------------
template <int DT> struct TT;
template <> struct TT<D_INT32> { using S = int32_t;  using A = uint32_t; static constexpr int V = 4; };
template <> struct TT<D_FP32>  { using S = float;    using A = float;    static constexpr int V = 4; };
template <> struct TT<D_BF16>  { using S = uint16_t; using A = float;    static constexpr int V = 8; };

__device__ __forceinline__ float as_f(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u(float f) { return __float_as_uint(f); }
__device__ __forceinline__ uint32_t as_u(uint32_t u) { return u; }
__device__ __forceinline__ void from_u(uint32_t u, float& f) { f = __uint_as_float(u); }
__device__ __forceinline__ void from_u(uint32_t u, uint32_t& v) { v = u; }

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs)
__device__ __forceinline__ uint32_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int OPK> __device__ __forceinline__ float cmb(float a, float b) {
  if constexpr (OPK == O_SUM || OPK == O_AVG) {
    return a + b;
  } else {
    // total order on non-NaN floats with -0 < +0: IEEE 754-2019 maximum, one
    // v_maximum3_f32 on gfx950 (denormals are kept, so they compare exactly)
    return __builtin_elementwise_maximum(a, b);
  }
}
template <int OPK> __device__ __forceinline__ uint32_t cmb(uint32_t a, uint32_t b) {
  if constexpr (OPK == O_SUM) return a + b;  // wraps modulo 2^32
  else return int32_t(b) > int32_t(a) ? b : a;
}

// ----------------------------------------------------------------------------
// fragments: what one thread moves per rank
// ----------------------------------------------------------------------------
// A fragment is M 16-byte vectors (M >= 1) at element offsets e, e + kThreads*V,
// ... (the vectors of a block interleave so that every load instruction of a
// wave covers 1 KB of contiguous memory), or a single element (M == 0, used at
// ragged range edges and for buffers that are not 16-byte aligned). Loads and
// stores carry the non-temporal hint: every byte is touched once per call.
template <int M> constexpr int mm() { return M ? M : 1; }
template <int DT, int M> constexpr int nvals() { return M ? M * TT<DT>::V : 1; }

// Raw bits of one fragment of the caller's dtype. NT = non-temporal hint; it is
// dropped where a program loads the same leaf again (several result trees).
template <typename T, bool NT>
__device__ __forceinline__ T ld(const T* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

template <int DT, int M, bool NT = true>
__device__ __forceinline__ void ld_user(const void* base, int64_t e, const bool (&ok)[mm<M>()],
                                        u32x4 (&r)[mm<M>()]) {
  using S = typename TT<DT>::S;
  if constexpr (M == 0) {
    if (ok[0]) {
      if constexpr (DT == D_BF16) r[0][0] = uint32_t(ld<uint16_t, NT>(reinterpret_cast<const uint16_t*>(base) + e));
      else r[0][0] = ld<uint32_t, NT>(reinterpret_cast<const uint32_t*>(base) + e);
    }
  } else {
#pragma unroll
    for (int j = 0; j < M; ++j)
      if (ok[j])
        r[j] = ld<u32x4, NT>(
            reinterpret_cast<const u32x4*>(reinterpret_cast<const S*>(base) + e + int64_t(j) * kThreads * TT<DT>::V));
  }
}

// Widen raw bits to the accumulation type (bf16 -> fp32 is exact).
template <int DT, int M>
__device__ __forceinline__ void widen(const u32x4 (&r)[mm<M>()], typename TT<DT>::A (&out)[nvals<DT, M>()]) {
  if constexpr (M == 0) {
    if constexpr (DT == D_BF16) out[0] = as_f(r[0][0] << 16);
    else from_u(r[0][0], out[0]);
  } else {
#pragma unroll
    for (int j = 0; j < M; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (DT == D_BF16) {
          out[8 * j + 2 * i] = as_f(r[j][i] << 16);
          out[8 * j + 2 * i + 1] = as_f(r[j][i] & 0xffff0000u);
        } else {
          from_u(r[j][i], out[4 * j + i]);
        }
      }
  }
}

// Store a fragment in the caller's dtype (bf16: one round to nearest even).
// NT = non-temporal hint; single elements that other workgroups complete into
// whole lines (strided items) are stored cacheable, so L2 merges the lines.
template <typename T, bool NT>
__device__ __forceinline__ void st1(T v, T* p) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

template <int DT, int M, bool NT = true>
__device__ __forceinline__ void st_user(void* base, int64_t e, const bool (&ok)[mm<M>()],
                                        const typename TT<DT>::A (&v)[nvals<DT, M>()]) {
  using S = typename TT<DT>::S;
  if constexpr (M == 0) {
    if (ok[0]) {
      if constexpr (DT == D_BF16) st1<uint16_t, NT>(uint16_t(to_bf16(v[0])), reinterpret_cast<uint16_t*>(base) + e);
      else st1<uint32_t, NT>(as_u(v[0]), reinterpret_cast<uint32_t*>(base) + e);
    }
  } else {
#pragma unroll
    for (int j = 0; j < M; ++j) {
      u32x4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (DT == D_BF16) r[i] = to_bf16(v[8 * j + 2 * i]) | (to_bf16(v[8 * j + 2 * i + 1]) << 16);
        else r[i] = as_u(v[4 * j + i]);
      }
      if (ok[j])
        __builtin_nontemporal_store(
            r, reinterpret_cast<u32x4*>(reinterpret_cast<S*>(base) + e + int64_t(j) * kThreads * TT<DT>::V));
    }
  }
}

// st_user for a fragment of vectors of which those not wholly inside [lo, hi)
// (the partial vectors at a range's ends) store only their elements inside it.
template <int DT, int M, bool NT = true>
__device__ __forceinline__ void st_user_edge(void* base, int64_t e, const bool (&ok)[mm<M>()],
                                             const typename TT<DT>::A (&v)[nvals<DT, M>()], int64_t lo, int64_t hi) {
  static_assert(M > 0, "vector fragments");
  using S = typename TT<DT>::S;
  constexpr int V = TT<DT>::V;
#pragma unroll
  for (int j = 0; j < M; ++j) {
    if (!ok[j]) continue;
    const int64_t ej = e + int64_t(j) * kThreads * V;
    if (ej >= lo && ej + V <= hi) {
      u32x4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (DT == D_BF16) r[i] = to_bf16(v[8 * j + 2 * i]) | (to_bf16(v[8 * j + 2 * i + 1]) << 16);
        else r[i] = as_u(v[4 * j + i]);
      }
      st1<u32x4, NT>(r, reinterpret_cast<u32x4*>(reinterpret_cast<S*>(base) + ej));
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i)
        if (ej + i >= lo && ej + i < hi) {
          if constexpr (DT == D_BF16) *(reinterpret_cast<uint16_t*>(base) + ej + i) = uint16_t(to_bf16(v[V * j + i]));
          else *(reinterpret_cast<uint32_t*>(base) + ej + i) = as_u(v[V * j + i]);
        }
    }
  }
}

// Store one fragment to `cnt` ranks: rank_of(i) gives the i-th destination.
// Destinations go 8 at a time so their pointer lookups (scalar loads) overlap.
// RUNS: rank_of may be read for whole runs of kLeafBatch indices (it reads
// padded program words) and is clamped by value past cnt; otherwise only
// indices below cnt are read.
template <int DT, int M, bool RUNS = false, bool NT = true, bool EDGE = false, typename RankOf>
__device__ __forceinline__ void st_user_all(const RankPtrs& ptrs, int cnt, RankOf&& rank_of, int64_t e,
                                            const bool (&ok)[mm<M>()],
                                            const typename TT<DT>::A (&v)[nvals<DT, M>()], int64_t lo = 0,
                                            int64_t hi = 0) {
  for (int b = 0; b < cnt; b += kLeafBatch) {
    void* pp[kLeafBatch];
    if constexpr (RUNS) {
      int rk[kLeafBatch];
#pragma unroll
      for (int k = 0; k < kLeafBatch; ++k) rk[k] = rank_of(b + k);
#pragma unroll
      for (int k = 1; k < kLeafBatch; ++k) rk[k] = b + k < cnt ? rk[k] : rk[0];
#pragma unroll
      for (int k = 0; k < kLeafBatch; ++k) pp[k] = ptrs.p[rk[k]];
    } else {
#pragma unroll
      for (int k = 0; k < kLeafBatch; ++k) pp[k] = ptrs.p[rank_of(b + k < cnt ? b + k : b)];
    }
#pragma unroll
    for (int k = 0; k < kLeafBatch; ++k)
      if (b + k < cnt) {
        if constexpr (EDGE) st_user_edge<DT, M, NT>(pp[k], e, ok, v, lo, hi);
        else st_user<DT, M, NT>(pp[k], e, ok, v);
      }
  }
}

// Workspace slots hold the accumulation type (4 bytes per element).
template <int DT, int M>
__device__ __forceinline__ void ld_acc(const void* base, int64_t e, const bool (&ok)[mm<M>()],
                                       typename TT<DT>::A (&out)[nvals<DT, M>()]) {
  const uint32_t* p = reinterpret_cast<const uint32_t*>(base) + e;
  if constexpr (M == 0) {
    if (ok[0]) from_u(__builtin_nontemporal_load(p), out[0]);
  } else {
    constexpr int V = TT<DT>::V;
#pragma unroll
    for (int j = 0; j < M; ++j)
#pragma unroll
      for (int q = 0; q < V / 4; ++q) {
        u32x4 r = {0, 0, 0, 0};
        if (ok[j]) r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + int64_t(j) * kThreads * V) + q);
#pragma unroll
        for (int i = 0; i < 4; ++i) from_u(r[i], out[V * j + 4 * q + i]);
      }
  }
}

template <int DT, int M>
__device__ __forceinline__ void st_acc(void* base, int64_t e, const bool (&ok)[mm<M>()],
                                       const typename TT<DT>::A (&v)[nvals<DT, M>()]) {
  uint32_t* p = reinterpret_cast<uint32_t*>(base) + e;
  if constexpr (M == 0) {
    if (ok[0]) __builtin_nontemporal_store(as_u(v[0]), p);
  } else {
    constexpr int V = TT<DT>::V;
#pragma unroll
    for (int j = 0; j < M; ++j)
#pragma unroll
      for (int q = 0; q < V / 4; ++q) {
        u32x4 r;
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = as_u(v[V * j + 4 * q + i]);
        if (ok[j]) __builtin_nontemporal_store(r, reinterpret_cast<u32x4*>(p + int64_t(j) * kThreads * V) + q);
      }
  }
}

// Iterate over the fragments of one work item: f(e, ok) for every fragment of
// this thread. Vector items hold `count` vectors; element items -count elements.
template <int M, typename F>
__device__ __forceinline__ void for_fragments(const Item& it, int V, F&& f) {
  if constexpr (M == 0) {
    const int cnt = -it.count;
    for (int v = threadIdx.x; v < cnt; v += kThreads) {
      const bool ok[1] = {true};
      f(it.start + v, ok);
    }
  } else {
    for (int v0 = 0; v0 < it.count; v0 += kThreads * M) {
      const int vb = v0 + int(threadIdx.x);
      bool ok[M];
#pragma unroll
      for (int j = 0; j < M; ++j) ok[j] = vb + j * kThreads < it.count;
      if (ok[0]) f(it.start + int64_t(vb) * V, ok);
    }
  }
}

// ----------------------------------------------------------------------------
// fused per-element replay
// ----------------------------------------------------------------------------
// Program words of one range: ntrees, then per tree: nleaves, nouts,
// leaf rank[nleaves] (postfix order), ncomb[nleaves] (combinations that follow
// each leaf), out rank[nouts]. Every tree reads the values from before the
// call, so all trees of a range are evaluated before any result is stored
// (results stay in registers; TM bounds the trees per range).
// Evaluate one tree's postfix program on a register stack of depth D. `leaf_at`
// fetches the raw bits of a leaf rank's fragment (from HBM, or from LDS where
// a range's leaves were staged once for several trees).
// Leaves are fetched B at a time with unconditional loads, so a batch is one
// clause of loads in flight. The host picks B from the leaf count so that the
// last batch is full where it can (B = 7 for seven leaves); otherwise the
// missing slots repeat the batch's first leaf.
// IDL: the leaves are ranks 0, 1, ... in postfix order (the caller passes
// the buffers in that order), so their ranks need no program read.
template <int DT, int OPK, int D, int M, int B, bool IDL = false, typename WP, typename LeafAt>
__device__ __forceinline__ void eval_one(WP __restrict__ w, LeafAt&& leaf_at,
                                         typename TT<DT>::A (&res)[nvals<DT, M>()]) {
  using A = typename TT<DT>::A;
  constexpr int N = nvals<DT, M>();
  const int nl = w[0];
  const WP __restrict__ leaf = w + 2;
  const WP __restrict__ nc = leaf + nl;
  A st[D][N];
#pragma unroll
  for (int d = 0; d < D; ++d)
#pragma unroll
    for (int i = 0; i < N; ++i) st[d][i] = A(0);
  for (int base = 0; base < nl; base += B) {
    u32x4 raw[B][mm<M>()];
    int cnt[B];
    if constexpr (IDL) {
#pragma unroll
      for (int k = 0; k < B; ++k) {
        leaf_at(base + k < nl ? base + k : base, raw[k]);
        if constexpr (word_runs<WP>()) cnt[k] = nc[base + k];
      }
    } else if constexpr (word_runs<WP>()) {  // whole runs of B words, clamped by value past the end
      int rk[B];
#pragma unroll
      for (int k = 0; k < B; ++k) {
        rk[k] = leaf[base + k];
        cnt[k] = nc[base + k];
      }
#pragma unroll
      for (int k = 1; k < B; ++k) rk[k] = base + k < nl ? rk[k] : rk[0];
#pragma unroll
      for (int k = 0; k < B; ++k) leaf_at(rk[k], raw[k]);
    } else {
#pragma unroll
      for (int k = 0; k < B; ++k) leaf_at(leaf[base + k < nl ? base + k : base], raw[k]);
    }
#pragma unroll
    for (int k = 0; k < B; ++k) {
      if (base + k < nl) {
        // push: shift the stack down by one (static register moves), widen the leaf on top
#pragma unroll
        for (int d = D - 1; d > 0; --d)
#pragma unroll
          for (int i = 0; i < N; ++i) st[d][i] = st[d - 1][i];
        widen<DT, M>(raw[k], st[0]);
        // each combination folds the top two entries and shifts the rest up
        for (int c = word_runs<WP>() ? cnt[k] : nc[base + k]; c > 0; --c) {
#pragma unroll
          for (int i = 0; i < N; ++i) st[0][i] = cmb<OPK>(st[1][i], st[0][i]);
#pragma unroll
          for (int d = 1; d < D - 1; ++d)
#pragma unroll
            for (int i = 0; i < N; ++i) st[d][i] = st[d + 1][i];
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < N; ++i) res[i] = st[0][i];
}

// A chain (every leaf after the first followed by one combination) needs no
// stack: res = combine(res, leaf) in leaf order, the operations the register
// stack performs on it, with the same operands in the same order. Leaf ranks
// are read in runs of B words like eval_one's (the host pads the program).
template <int DT, int OPK, int M, int B, typename WP, typename LeafAt>
__device__ __forceinline__ void eval_chain(WP __restrict__ w, LeafAt&& leaf_at,
                                           typename TT<DT>::A (&res)[nvals<DT, M>()]) {
  using A = typename TT<DT>::A;
  constexpr int N = nvals<DT, M>();
  const int nl = w[0];
  const WP __restrict__ leaf = w + 2;
  for (int base = 0; base < nl; base += B) {
    int rk[B];
#pragma unroll
    for (int k = 0; k < B; ++k) rk[k] = leaf[base + k];
#pragma unroll
    for (int k = 1; k < B; ++k) rk[k] = base + k < nl ? rk[k] : rk[0];
    u32x4 raw[B][mm<M>()];
#pragma unroll
    for (int k = 0; k < B; ++k) leaf_at(rk[k], raw[k]);
#pragma unroll
    for (int k = 0; k < B; ++k) {
      if (base + k < nl) {
        A x[N];
        widen<DT, M>(raw[k], x);
#pragma unroll
        for (int i = 0; i < N; ++i) res[i] = base + k == 0 ? x[i] : cmb<OPK>(res[i], x[i]);
      }
    }
  }
}

// IDL (one tree): leaves are ranks 0 .. nl - 1 and outputs nl, nl + 1, ... of
// ptrs, which the caller orders so.
template <int DT, int OPK, int D, int TM, int M, int B, bool NTS = true, bool EDGE = false, bool IDL = false,
          typename WP, typename LeafAt>
__device__ __forceinline__ void replay(const RankPtrs& ptrs, WP __restrict__ w, int64_t e,
                                       const bool (&ok)[mm<M>()], LeafAt&& leaf_at, int64_t lo = 0, int64_t hi = 0) {
  static_assert(!IDL || TM == 1, "ordered buffers for one tree");
  using A = typename TT<DT>::A;
  const int ntrees = w[0];
  w += 1;
  A res[TM][nvals<DT, M>()];
  WP outs[TM];
  int nouts[TM], nls[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    if (t < ntrees) {
      const int nl = w[0];
      nls[t] = nl;
      nouts[t] = w[1];
      outs[t] = w + 2 + 2 * nl;
      eval_one<DT, OPK, D, M, B, IDL>(w, leaf_at, res[t]);
      w = outs[t] + nouts[t];
    }
  }
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    if (t < ntrees) {
      const WP ot = outs[t];
      if constexpr (OPK == O_AVG) {
#pragma unroll
        for (int i = 0; i < nvals<DT, M>(); ++i) res[t][i] = res[t][i] / ptrs.div;
      }
      if constexpr (IDL) {
        const int first = nls[t];
        st_user_all<DT, M, false, NTS, EDGE>(ptrs, nouts[t], [&](int i) { return first + i; }, e, ok, res[t], lo, hi);
      } else {
        st_user_all<DT, M, word_runs<WP>(), NTS, EDGE>(ptrs, nouts[t], [&](int i) { return ot[i]; }, e, ok, res[t],
                                                       lo, hi);
      }
    }
  }
}

// Register fragments per thread of the program-driven replay. Its work items
// hold one vector per thread, so the second fragment of a two-fragment form
// stays idle; yet for single-tree programs with a stack of 4 to 8 (bf16: 4)
// that read their leaf ranks from the program, that form measured faster
// (interleaved runs: AHC 5.96 vs 5.87 TB/s; 24-rank binomial 5.18 vs 5.00 TB/s
// before single-range programs took the ordered form below, which keeps one).
// Chains (a stack of 2) take one fragment: the idle one's arithmetic cost the
// 192-rank bf16 ring 8% (4.42 vs 4.79 TB/s).
template <int DT, int D, int TM> constexpr int fused_m() {
  return (TM == 1 && D > 2 && D <= (DT == D_BF16 ? 4 : 8)) ? 2 : 1;
}

// With the buffers in leaf order (IDL) the replay takes one fragment at every
// stack depth: the loads no longer wait on rank reads from the program, and
// the smaller register footprint (fp32: 96 VGPRs at a stack of 6, 112 at 8,
// against 114-162 with two fragments) keeps more waves resident (interleaved
// runs, 10^4 x 106 fp32: 24-rank recursive doubling and binomial +3%, 12-rank
// +1-2%).
template <int DT, int OPK, int D, int TM, int B, bool IDL = false>
__global__ __launch_bounds__(kThreads) void k_fused(RankPtrs ptrs, const Item* __restrict__ items,
                                                    const int32_t* __restrict__ prog) {
  constexpr int V = TT<DT>::V;
  constexpr int M = IDL ? 1 : fused_m<DT, D, TM>();
  constexpr bool NT = TM == 1;  // several trees re-read their leaves: keep them cacheable
  const Item it = items[item_index(ptrs.xcd)];
  const auto w = prog_words<TM>(prog, it.tag);
  if (TM == 1 && it.count > kItemVectorsMask) {
    // partial vectors at the range's ends (single-tree programs): load them
    // whole (in the buffer), store only the range's elements; vectors wholly
    // before the range stay idle
    Item jt = it;
    jt.count = it.count & kItemVectorsMask;
    const int64_t lo = it.start + ((it.count >> 16) & 0xff);
    const int64_t hi = it.start + int64_t(jt.count) * V - ((it.count >> 24) & 0xf);
    // program words through the constant address space: the element stores
    // would otherwise make the compiler fetch every later word with a vector load
    const ProgPtr wc = as_prog(prog) + it.tag;
    for_fragments<M>(jt, V, [&](int64_t e, const bool (&ok0)[M]) {
      bool ok[M];
#pragma unroll
      for (int j = 0; j < M; ++j) ok[j] = ok0[j] && e + int64_t(j) * kThreads * V + V > lo;
      replay<DT, OPK, D, TM, M, B, true, true, IDL>(
          ptrs, wc, e, ok, [&](int rank, u32x4(&r)[M]) { ld_user<DT, M, NT>(ptrs.p[rank], e, ok, r); }, lo, hi);
    });
  } else if (it.count > 0) {
    for_fragments<M>(it, V, [&](int64_t e, const bool (&ok)[M]) {
      replay<DT, OPK, D, TM, M, B, true, false, IDL>(
          ptrs, w, e, ok, [&](int rank, u32x4(&r)[M]) { ld_user<DT, M, NT>(ptrs.p[rank], e, ok, r); });
    });
  } else {
    for_fragments<0>(it, V, [&](int64_t e, const bool (&ok)[1]) {
      replay<DT, OPK, D, TM, 0, B, true, false, IDL>(
          ptrs, w, e, ok, [&](int rank, u32x4(&r)[1]) { ld_user<DT, 0, NT>(ptrs.p[rank], e, ok, r); });
    });
  }
}

// Single-tree programs of at most kMaxTabRanges ranges in which every tree has
// one fixed shape of at most 8 leaves run with their leaves loaded at once:
//  - SH_BALANCED: a perfect binary tree of NL = 4 or 8 leaves, combined level
//    by level (recursive halving and doubling, the generalized algorithm over
//    Z_2^k give these);
//  - SH_CHAIN: ((l0 + l1) + l2) + ... over NL = 1..8 leaves (the ring and the
//    pipelined chain give these; one leaf is the all-gather's copy);
//  - SH_STACK: any other tree of NL = 3..8 leaves, the same shape in every
//    range (the generalized algorithm over Z_P, halving and doubling with
//    fold-in, the binomial tree): the register stack (depth 4 holds every such
//    tree in the program's Sethi-Ullman order) driven by the combination
//    counts in the kernel argument.
// The host checks each tree's combination counts against the shape and passes,
// per call, the buffer pointers of every range's leaves (postfix order) and
// outputs as a kernel argument: the data loads then wait on no program read and
// no rank lookup (measured on 8 x 2^20 fp32 halving + doubling: 12.2 us with
// the ranks read from the program words, 11.9 with a rank table, 11.6 with the
// pointers). cmb(left, right) keeps the operands of the postfix fold.
constexpr int kMaxTabRanges = 8;
enum : int { SH_NONE = 0, SH_BALANCED = 1, SH_CHAIN = 2, SH_STACK = 3 };
struct RankTab {  // host side: ranks per range, turned into FixPtrs per call
  uint8_t leaf[kMaxTabRanges][8];
  uint8_t out[kMaxTabRanges][8];
  uint8_t nouts[kMaxTabRanges];
  uint8_t nc[8];  // SH_STACK: combinations after each leaf (every range alike)
};
struct FixPtrs {
  void* leaf[kMaxTabRanges][8];  // range r's leaf buffers, postfix order
  void* out[kMaxTabRanges][8];   // its output buffers
  uint8_t nouts[kMaxTabRanges];
  uint8_t nc[8];                 // SH_STACK
  float div;                     // O_AVG: divide the complete sum by this (P)
  int32_t xcd;                   // as RankPtrs::xcd
};

template <int DT, int OPK, int SH, int M, int NL>
__device__ __forceinline__ void fixed_one(const FixPtrs& fp, int r, int64_t e, const bool (&ok)[mm<M>()]) {
  using A = typename TT<DT>::A;
  constexpr int N = nvals<DT, M>();
  u32x4 raw[NL][mm<M>()];
#pragma unroll
  for (int k = 0; k < NL; ++k) ld_user<DT, M>(fp.leaf[r][k], e, ok, raw[k]);
  A v[NL][N];
#pragma unroll
  for (int k = 0; k < NL; ++k) widen<DT, M>(raw[k], v[k]);
  if constexpr (SH == SH_STACK) {
    // as eval_one with the leaves already loaded: a push shifts the stack down
    // (static moves); each combination folds the top two entries, cmb(deeper,
    // top), and shifts the rest up
    constexpr int D = 4;
    A st[D][N];
#pragma unroll
    for (int d = 0; d < D; ++d)
#pragma unroll
      for (int j = 0; j < N; ++j) st[d][j] = A(0);
#pragma unroll
    for (int k = 0; k < NL; ++k) {
#pragma unroll
      for (int d = D - 1; d > 0; --d)
#pragma unroll
        for (int j = 0; j < N; ++j) st[d][j] = st[d - 1][j];
#pragma unroll
      for (int j = 0; j < N; ++j) st[0][j] = v[k][j];
      const int c = fp.nc[k];
#pragma unroll
      for (int q = 0; q < D - 1; ++q) {
        if (q < c) {
#pragma unroll
          for (int j = 0; j < N; ++j) st[0][j] = cmb<OPK>(st[1][j], st[0][j]);
#pragma unroll
          for (int d = 1; d < D - 1; ++d)
#pragma unroll
            for (int j = 0; j < N; ++j) st[d][j] = st[d + 1][j];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < N; ++j) v[0][j] = st[0][j];
  } else if constexpr (SH == SH_BALANCED) {
    // level by level: v[i] = v[2i] + v[2i+1]; reads never trail the writes
#pragma unroll
    for (int h = NL / 2; h >= 1; h /= 2)
#pragma unroll
      for (int i = 0; i < h; ++i)
#pragma unroll
        for (int j = 0; j < N; ++j) v[i][j] = cmb<OPK>(v[2 * i][j], v[2 * i + 1][j]);
  } else {
#pragma unroll
    for (int k = 1; k < NL; ++k)
#pragma unroll
      for (int j = 0; j < N; ++j) v[0][j] = cmb<OPK>(v[0][j], v[k][j]);
  }
  if constexpr (OPK == O_AVG) {
#pragma unroll
    for (int j = 0; j < N; ++j) v[0][j] = v[0][j] / fp.div;
  }
  const int no = fp.nouts[r];
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if (k < no) st_user<DT, M>(fp.out[r][k], e, ok, v[0]);
}

// NL leaves per tree; M vectors per thread on the vector path (the items hold
// kThreads * M vectors); an item's tag is its range's index.
template <int DT, int OPK, int SH, int M, int NL>
__global__ __launch_bounds__(kThreads) void k_fused_fixed(FixPtrs fp, const Item* __restrict__ items) {
  constexpr int V = TT<DT>::V;
  const Item it = items[item_index(fp.xcd)];
  if (it.count > 0) {
    for_fragments<M>(it, V, [&](int64_t e, const bool (&ok)[M]) { fixed_one<DT, OPK, SH, M, NL>(fp, it.tag, e, ok); });
  } else {
    for_fragments<0>(it, V, [&](int64_t e, const bool (&ok)[1]) { fixed_one<DT, OPK, SH, 0, NL>(fp, it.tag, e, ok); });
  }
}

// Several trees per range, all of one shape of NL = P <= 8 leaves, at most 8
// ranges of 8 trees (the generalized algorithm with r > 0 on up to 8 ranks):
// every rank's fragment is staged in LDS once, as in k_fused_staged, and each
// tree's leaf ranks, output ranks and the shared combination counts come from
// a fixed-stride table of scalar words, with the leaf count known at compile
// time (measured on 7 x 2^24 fp32: r = 3 218 -> 204 us, r = 2 193 -> 189 us
// against k_fused_staged). Reading the ranks as bytes of a kernel argument
// instead made the compiler copy the argument to scratch (4x slower).
struct MultiTab {  // host side: per range, ntrees; per tree leaf[8], nouts, out[8]
  uint8_t leaf[8][8][8];
  uint8_t out[8][8][8];
  uint8_t nouts[8][8];
  uint8_t ntrees[8];
  uint8_t nc[8];
};
// device table (int32 words, read as scalars): nc[8], then per range r at
// 8 + r * kMultiRangeWords: ntrees, then per tree t at + 1 + t * 17:
// leaf[8], nouts, out[8]
constexpr int kMultiRangeWords = 1 + 8 * 17;
struct MultiPtrs {
  void* p[8];
  float div;
  int32_t xcd;
};

template <int DT, int OPK, int NL, int M>
__device__ __forceinline__ void multi_one(const MultiPtrs& mp, ProgPtr tab, int r, int64_t e,
                                          const bool (&ok)[mm<M>()], u32x4* stage) {
  using A = typename TT<DT>::A;
  constexpr int N = nvals<DT, M>();
  constexpr int D = 4;
  {
    u32x4 raw[NL][mm<M>()];
#pragma unroll
    for (int k = 0; k < NL; ++k) ld_user<DT, M>(mp.p[k], e, ok, raw[k]);
#pragma unroll
    for (int k = 0; k < NL; ++k) stage[k * kThreads + threadIdx.x] = raw[k][0];
  }
  int nc[NL];
#pragma unroll
  for (int k = 0; k < NL; ++k) nc[k] = tab[k];
  const ProgPtr rt = tab + 8 + r * kMultiRangeWords;
  const int nt = rt[0];
  A res[kMaxFusedTrees][N];
#pragma unroll
  for (int t = 0; t < kMaxFusedTrees; ++t) {
    if (t < nt) {
      const ProgPtr tw = rt + 1 + t * 17;
      int lr[NL];
#pragma unroll
      for (int k = 0; k < NL; ++k) lr[k] = tw[k];
      A st[D][N];
#pragma unroll
      for (int d = 0; d < D; ++d)
#pragma unroll
        for (int j = 0; j < N; ++j) st[d][j] = A(0);
#pragma unroll
      for (int k = 0; k < NL; ++k) {
        u32x4 raw[1];
        raw[0] = stage[lr[k] * kThreads + threadIdx.x];
#pragma unroll
        for (int d = D - 1; d > 0; --d)
#pragma unroll
          for (int j = 0; j < N; ++j) st[d][j] = st[d - 1][j];
        widen<DT, M>(raw, st[0]);
#pragma unroll
        for (int q = 0; q < D - 1; ++q) {
          if (q < nc[k]) {
#pragma unroll
            for (int j = 0; j < N; ++j) st[0][j] = cmb<OPK>(st[1][j], st[0][j]);
#pragma unroll
            for (int d = 1; d < D - 1; ++d)
#pragma unroll
              for (int j = 0; j < N; ++j) st[d][j] = st[d + 1][j];
          }
        }
      }
#pragma unroll
      for (int j = 0; j < N; ++j) res[t][j] = st[0][j];
    }
  }
#pragma unroll
  for (int t = 0; t < kMaxFusedTrees; ++t) {
    if (t < nt) {
      if constexpr (OPK == O_AVG) {
#pragma unroll
        for (int j = 0; j < N; ++j) res[t][j] = res[t][j] / mp.div;
      }
      const ProgPtr tw = rt + 1 + t * 17;
      const int no = tw[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j < no) st_user<DT, M>(mp.p[tw[9 + j]], e, ok, res[t]);
    }
  }
}

template <int DT, int OPK, int NL>
__global__ __launch_bounds__(kThreads) void k_fused_multi(MultiPtrs mp, const Item* __restrict__ items,
                                                          const int32_t* __restrict__ tab) {
  constexpr int V = TT<DT>::V;
  extern __shared__ u32x4 stage[];
  const Item it = items[item_index(mp.xcd)];
  const ProgPtr t = as_prog(tab);
  if (it.count > 0) {
    for_fragments<1>(it, V, [&](int64_t e, const bool (&ok)[1]) { multi_one<DT, OPK, NL, 1>(mp, t, it.tag, e, ok, stage); });
  } else {
    for_fragments<0>(it, V, [&](int64_t e, const bool (&ok)[1]) { multi_one<DT, OPK, NL, 0>(mp, t, it.tag, e, ok, stage); });
  }
}

// Batches of short instances: a strided item covers one range of `len`
// elements (the same offsets in every instance) across `nb` consecutive
// instances `stride` elements apart, one element per thread: instance v / len,
// offset v % len. Per-instance items would give a workgroup a handful of
// elements each.
struct SItem {
  int64_t start;  // the range's first element in the item's first instance
  int32_t tag;    // program word offset
  int32_t len;    // elements of the range in one instance
  int32_t nb;     // instances
  int32_t pad;
};

template <int DT, int OPK, int D, int TM, int B>
__global__ __launch_bounds__(kThreads) void k_fused_strided(RankPtrs ptrs, const SItem* __restrict__ items,
                                                            const int32_t* __restrict__ prog, int64_t stride) {
  const SItem it = items[item_index(ptrs.xcd)];
  const auto w = prog_words<TM>(prog, it.tag);
  const int total = it.len * it.nb;
  for (int v = threadIdx.x; v < total; v += kThreads) {
    const int b = v / it.len;
    const int64_t e = it.start + int64_t(b) * stride + (v - b * it.len);
    const bool ok[1] = {true};
    // neighbouring ranges of the same instances run in neighbouring items and
    // share cache lines: cacheable loads and stores
    replay<DT, OPK, D, TM, 0, B, false>(ptrs, w, e, ok,
                                        [&](int rank, u32x4(&r)[1]) { ld_user<DT, 0, false>(ptrs.p[rank], e, ok, r); });
  }
}

// Batches of short instances whose ranges all run one program up to a renaming
// of leaf ranks (the pieces of a vector of ~100 elements split over many ranks
// by reduce-scatter/all-gather style schedules). A workgroup takes `iters` x
// kThreads consecutive elements of the whole batch, one per thread per step, so
// every cache line is fetched once, by one workgroup. Each thread looks up its
// element's range in LDS and evaluates the reference range's program, reading
// leaf `rank` from the buffer that the range's row names. `tab` holds the range
// of each of the n offsets of an instance (padded to 8 bytes), then the renaming
// as map[rank][range]: R bytes per leaf rank of the reference range. The evaluation order is the reference program's, so the
// bits equal those of the replay over per-range items.
template <int DT, int OPK, int D, int TM, int B>
__global__ __launch_bounds__(kThreads) void k_fused_rows(RankPtrs ptrs, const int32_t* __restrict__ prog,
                                                         const uint8_t* __restrict__ tab, int64_t first,
                                                         int64_t total, int32_t n, int32_t R, int32_t P,
                                                         int32_t iters) {
  extern __shared__ uint64_t rows_lds[];
  // rows of Q = P | 1 pointers: an odd stride of 8-byte entries puts the rows
  // that one load's lanes read in distinct LDS banks
  const int Q = P | 1;
  void** row_ptr = reinterpret_cast<void**>(rows_lds);         // R x Q buffers
  void** base = row_ptr + R * Q;                               // P buffers
  uint8_t* range_of = reinterpret_cast<uint8_t*>(base + P);    // n ranges
  if (threadIdx.x == 0)
    for (int x = 0; x < P; ++x) base[x] = ptrs.p[x];
  for (int o = threadIdx.x; o < n; o += kThreads) range_of[o] = tab[o];
  __syncthreads();
  const int moff = (n + 7) / 8 * 8;
  // the table holds map[rank][range]
  for (int i = threadIdx.x; i < R * P; i += kThreads) row_ptr[(i % R) * Q + i / R] = base[tab[moff + i]];
  __syncthreads();
  const auto w = prog_words<TM>(prog, 0);
  const int64_t v0 = first + int64_t(blockIdx.x) * iters * kThreads;  // the workgroup's first element
  int64_t v = v0 + threadIdx.x;
  int o = int(v0 % n) + int(threadIdx.x);  // one wide division per workgroup, a narrow one per thread
  o = o % n;
  const int step = kThreads % n;
  for (int i = 0; i < iters; ++i) {
    const bool ok[1] = {v < total};
    void* const* row = row_ptr + range_of[o] * Q;
    // a line of one rank is read by the several loads whose ranges it spans:
    // cacheable loads
    replay<DT, OPK, D, TM, 0, B>(ptrs, w, v, ok,
                                 [&](int rank, u32x4(&r)[1]) { ld_user<DT, 0, false>(row[rank], v, ok, r); });
    v += kThreads;
    o += step;
    if (o >= n) o -= n;
  }
}

// The same batches with 4-byte elements, 16-byte aligned buffers and at most
// 32 ranks, whose reference tree stores to all P ranks. Each wave works on
// positions of 64 K consecutive elements (16 K vectors) and walks the
// positions of the launch with a stride of all its waves; the grid holds what
// the device keeps resident. The loads of a wave's next position are issued
// before the current one is evaluated, and its first position is loaded before
// the tables are copied, so that memory round trip overlaps theirs (with one
// position per wave, as on 3 or 6 ranks x 10^4 x 106 elements, it is the
// wave's whole life). Three forms:
//  - at most kRowsRegMaxRanks ranks (REG, K = 4): lane L loads vector L of
//    every rank (G = P non-temporal 16-byte loads, 1 KB runs) and evaluates
//    the reference range's program for its own four elements in registers.
//    Leaf `rank` of an element is the loaded value of the rank that the
//    element's range renames it to, picked by selects among the G loads; one
//    LDS word per offset of an instance holds those ranks for every leaf
//    (4 bits each). The results go straight from registers to the outputs.
//    The selects grow as P^2 per element; past a few ranks the staged form
//    below is faster.
//  - staged, K = 4 (up to 8 ranks): lane L loads vector L of every rank
//    (G = P loads) into the wave's own LDS stage, [rank][element];
//  - staged, K = 1 (9..32 ranks): the P x 16 vectors are spread over the
//    lanes, lane L loading vector L % 16 of ranks L / 16, L / 16 + 4, ...
//    (G = ceil(P / 4) loads per lane; one instruction covers four 256-byte
//    runs, which measured as fast as 1 KB runs of one rank), each line once.
//  In the staged forms lane L evaluates the reference range's program for
//  elements L, L + 64, ..., reading leaf `rank` from the stage row of the rank
//  its element's range renames it to (map[rank][range]: the lanes of one read
//  hit consecutive bytes; stage reads hit consecutive words). A chain (the
//  ring's trees; CHAIN) is folded leaf by leaf without the register stack.
//  The results go through LDS once more, so that each lane stores whole
//  vectors to the program's output ranks. Only the wave reads what it wrote
//  to its stage; wave-scope fences order those LDS accesses.
// The waves of a workgroup share one copy of the tables (those of k_fused_rows,
// then the packed leaf ranks for at most kRowsRegMaxRanks ranks, each padded
// to a multiple of 8 bytes) and, with one element per lane, of the output
// buffer table.
constexpr int kRowsVecThreads = 256;  // at most; the host picks 1 or 4 waves per workgroup
constexpr int kRowsRegMaxRanks = 3;   // ranks up to which the register form runs (even at 4, slower from 5)
constexpr int kRowsTableRegs = 4;     // register form: table words per thread loaded ahead of the data
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
template <int DT, int OPK, int D, int B, int K, int G, bool REG, bool CHAIN>
__global__ __launch_bounds__(kRowsVecThreads) void k_fused_rows_vec(RankPtrs ptrs, const int32_t* __restrict__ prog,
                                                                    const uint8_t* __restrict__ tab, int64_t nvec,
                                                                    int32_t n, int32_t R, int32_t P) {
  static_assert(TT<DT>::V == 4, "four 4-byte elements per vector");
  static_assert(K == 1 || K == 4, "one or four elements per lane");
  static_assert(!REG || (K == 4 && G <= kRowsRegMaxRanks), "the register form: one vector per lane and rank");
  static_assert(!(REG && CHAIN), "chains are evaluated apart in the staged forms");
  using A = typename TT<DT>::A;
  constexpr int E = 64 * K, NV = 16 * K;  // elements and vectors of a position
  extern __shared__ uint32_t rows_vec_lds[];
  const int lane = int(threadIdx.x) & 63, waves = int(blockDim.x) >> 6;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
  const int64_t npos = (nvec + NV - 1) / NV;
  const int64_t stride = int64_t(gridDim.x) * waves;
  int64_t pos = int64_t(blockIdx.x) * waves + wave;
  const ProgPtr tree = as_prog(prog) + 1;  // the reference range's single tree, P outputs
  const ProgPtr outs = tree + 2 + 2 * tree[0];
  const int moff = (n + 7) / 8 * 8;
  const int ostep = int((stride * E) % n);
  const int b0 = int(pos * E % n);  // the offset of the position's first element in its instance
  if constexpr (REG) {
    const u32x4* src[G];
    u32x4* dst[G];
#pragma unroll
    for (int i = 0; i < G; ++i) src[i] = static_cast<const u32x4*>(ptrs.p[i]);
    // the last position may be partial: its lanes past the end repeat the
    // last vector and store nothing
    auto load = [&](int64_t ps, u32x4(&r)[G]) {
      const int64_t g = ps * NV + lane < nvec ? ps * NV + lane : nvec - 1;
#pragma unroll
      for (int i = 0; i < G; ++i) r[i] = __builtin_nontemporal_load(src[i] + g);
    };
    // the table's first words are loaded ahead of the data, so that the wait
    // before their LDS copy covers them alone (loads retire in order) and the
    // lookups of the first position run while its data is in flight. The data
    // loads read memory nothing has stored to yet, which the compiler may
    // place anywhere: scheduling barriers keep them after the table loads and
    // ahead of the table's copy and the workgroup barrier. Unconditional,
    // clamped loads leave no branch between a load and its wait.
    const uint32_t* lsrc = reinterpret_cast<const uint32_t*>(tab) + (moff + R * P + 7) / 8 * 2;
    uint32_t tw[kRowsTableRegs];
#pragma unroll
    for (int r = 0; r < kRowsTableRegs; ++r) {
      const int i = int(threadIdx.x) + r * int(blockDim.x);
      tw[r] = lsrc[i < n ? i : n - 1];
    }
    __builtin_amdgcn_sched_barrier(0);
    u32x4 ra[G], rb[G];
    load(pos, ra);  // past the end (an idle wave) the last vector, unused
    __builtin_amdgcn_sched_barrier(0);
    uint32_t* lrank = rows_vec_lds;  // per offset: the rank each leaf reads, 4 bits per leaf rank
#pragma unroll
    for (int r = 0; r < kRowsTableRegs; ++r) {
      const int i = int(threadIdx.x) + r * int(blockDim.x);
      if (i < n) lrank[i] = tw[r];
    }
    for (int i = int(threadIdx.x) + kRowsTableRegs * int(blockDim.x); i < n; i += int(blockDim.x)) lrank[i] = lsrc[i];
#pragma unroll
    for (int i = 0; i < G; ++i) dst[i] = static_cast<u32x4*>(ptrs.p[outs[i]]);
    int o[4];  // offsets of the lane's elements in their instances
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = int(unsigned(b0 + 4 * lane + c) % unsigned(n));
    __syncthreads();
    if (pos >= npos) return;
    // evaluate the position in `cur` (loads of the next one into `nxt` first)
    auto step = [&](u32x4(&cur)[G], u32x4(&nxt)[G], bool more) {
      if (more) load(pos + stride, nxt);
      uint32_t pk[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) pk[c] = lrank[o[c]];
      A res[nvals<DT, 1>()];
      eval_one<DT, OPK, D, 1, B>(tree, [&](int rank, u32x4(&x)[1]) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t row = (pk[c] >> (4 * rank)) & 15u;
          uint32_t y = cur[0][c];
#pragma unroll
          for (int i = 1; i < G; ++i) y = row == uint32_t(i) ? cur[i][c] : y;
          x[0][c] = y;
        }
      }, res);
      u32x4 rv;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if constexpr (OPK == O_AVG) res[c] = res[c] / ptrs.div;
        rv[c] = as_u(res[c]);
      }
      const int64_t g = pos * NV + lane;
      if (g < nvec)
#pragma unroll
        for (int i = 0; i < G; ++i) __builtin_nontemporal_store(rv, dst[i] + g);
    };
    auto advance = [&] {
      pos += stride;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        o[c] += ostep;
        if (o[c] >= n) o[c] -= n;
      }
    };
    // two register sets in turn, so that no loaded value is moved while its
    // load may be in flight
    for (;;) {
      bool more = pos + stride < npos;
      step(ra, rb, more);
      if (!more) break;
      advance();
      more = pos + stride < npos;
      step(rb, ra, more);
      if (!more) break;
      advance();
    }
  } else {
    uint32_t* stage = rows_vec_lds + wave * (P + 1) * E;  // P rows of E words, then the E results
    uint32_t* outw = stage + P * E;
    const int q = K == 1 ? lane & 15 : lane, y0 = K == 1 ? lane >> 4 : 0;  // vector in the position, lane group
    // the buffer of each load: K = 4, rank i; K = 1, rank 4 i + y0, and past
    // the last rank the last rank again (the same vector from the same lane
    // slot within one instruction: one request and one line, written to the
    // same stage word with the same value). Chosen from the kernel argument by
    // uniform selects at constant indices, once.
    const u32x4* src[G];
    if constexpr (K == 4) {
#pragma unroll
      for (int i = 0; i < G; ++i) src[i] = static_cast<const u32x4*>(ptrs.p[i]);
    } else {
      const int lk = P - 1 - 4 * (G - 1);  // the last rank's place in the last group of four
      void* const last = lk == 0 ? ptrs.p[4 * G - 4] : lk == 1 ? ptrs.p[4 * G - 3] : lk == 2 ? ptrs.p[4 * G - 2]
                                                                                              : ptrs.p[4 * G - 1];
#pragma unroll
      for (int i = 0; i < G; ++i) {
        void* c[4];
#pragma unroll
        for (int y = 0; y < 4; ++y) c[y] = 4 * i + y < P ? ptrs.p[4 * i + y] : last;
        src[i] = static_cast<const u32x4*>(y0 == 0 ? c[0] : y0 == 1 ? c[1] : y0 == 2 ? c[2] : c[3]);
      }
    }
    u32x4 cur[G];
    // the last position may be partial: its lanes past the end repeat the last
    // vector (within the instruction) and store nothing
    auto load = [&](int64_t ps) {
      const int64_t g = ps * NV + q < nvec ? ps * NV + q : nvec - 1;
#pragma unroll
      for (int i = 0; i < G; ++i) cur[i] = __builtin_nontemporal_load(src[i] + g);
    };
    // TF (9..12 ranks): like the register form, a word of the table per
    // thread is loaded ahead of the data, the output table is written from
    // scalar reads, and each position's range lookup precedes its stage
    // writes, so the first position's lookups run while its data is in flight
    // (measured +3-4.5% at 12 ranks; at 24 ranks, with more positions per
    // wave, 1% slower)
    constexpr bool TF = K == 1 && G <= 3;
    const uint32_t* tsrc = reinterpret_cast<const uint32_t*>(tab);
    const int words = (moff + R * P + 7) / 8 * 2;
    uint32_t tw0 = 0;
    if constexpr (TF) {
      tw0 = tsrc[int(threadIdx.x) < words ? int(threadIdx.x) : words - 1];
      __builtin_amdgcn_sched_barrier(0);
      load(pos);  // past the end (an idle wave) the last vector, unused
      __builtin_amdgcn_sched_barrier(0);
    } else {
      if (pos < npos) load(pos);
    }
    // K = 1: the output table, entry 4 i + y the output lane group y stores to
    // in its i-th store (past the last output the last one again)
    u32x4** ptab = reinterpret_cast<u32x4**>(rows_vec_lds + waves * (P + 1) * E);
    uint32_t* tabw = reinterpret_cast<uint32_t*>(ptab + (K == 1 ? 4 * G : 0));
    auto cl = [P](int k) { return k < P ? k : P - 1; };
    if constexpr (TF) {
      if (threadIdx.x == 0)
#pragma unroll
        for (int e = 0; e < 4 * G; ++e) ptab[e] = static_cast<u32x4*>(ptrs.p[outs[cl(e)]]);
      if (int(threadIdx.x) < words) tabw[threadIdx.x] = tw0;
      for (int i = int(threadIdx.x + blockDim.x); i < words; i += int(blockDim.x)) tabw[i] = tsrc[i];
    } else {
      if constexpr (K == 1) {
        if (threadIdx.x < 4 * G) ptab[threadIdx.x] = static_cast<u32x4*>(ptrs.p[outs[cl(int(threadIdx.x))]]);
      }
      for (int i = threadIdx.x; i < words; i += blockDim.x) tabw[i] = tsrc[i];
    }
    int o[K];  // offsets of the lane's elements in their instances
#pragma unroll
    for (int j = 0; j < K; ++j) o[j] = int(unsigned(b0 + 64 * j + lane) % unsigned(n));
    __syncthreads();
    if (pos >= npos) return;
    const uint8_t* range_of = reinterpret_cast<const uint8_t*>(tabw);
    const uint8_t* map = range_of + moff;  // [rank][range]
    // stage the loaded position, evaluate, store; `next` issues the following
    // position's loads between the stage writes and the evaluation. Only a
    // wave's last position can be partial.
    auto step = [&](auto next, bool last) {
      int rr[K];
      if constexpr (TF) rr[0] = range_of[o[0]];  // before the stage writes, which wait for the loads
#pragma unroll
      for (int i = 0; i < G; ++i)
        *reinterpret_cast<u32x4*>(stage + (K == 1 ? cl(4 * i + y0) : i) * E + q * 4) = cur[i];
      next();
      wave_lds_sync();
      if constexpr (!TF)
#pragma unroll
        for (int j = 0; j < K; ++j) rr[j] = range_of[o[j]];
      constexpr int M = K == 1 ? 0 : 1;
      A res[nvals<DT, M>()];
      auto leaf = [&](int rank, u32x4(&v)[1]) {
#pragma unroll
        for (int j = 0; j < K; ++j) v[0][j] = stage[map[rank * R + rr[j]] * E + 64 * j + lane];
      };
      if constexpr (CHAIN) eval_chain<DT, OPK, M, B>(tree, leaf, res);
      else eval_one<DT, OPK, D, M, B>(tree, leaf, res);
#pragma unroll
      for (int j = 0; j < K; ++j) {
        if constexpr (OPK == O_AVG) res[j] = res[j] / ptrs.div;
        outw[64 * j + lane] = as_u(res[j]);
      }
      wave_lds_sync();
      const u32x4 rv = *reinterpret_cast<const u32x4*>(outw + q * 4);
      if (!last || pos * NV + q < nvec)
#pragma unroll
        for (int i = 0; i < G; ++i) {
          u32x4* d = K == 1 ? ptab[4 * i + y0] : static_cast<u32x4*>(ptrs.p[outs[i]]);
          __builtin_nontemporal_store(rv, d + pos * NV + q);
        }
      wave_lds_sync();  // the next position's stage writes follow this one's reads
    };
    auto advance = [&] {
      pos += stride;
#pragma unroll
      for (int j = 0; j < K; ++j) {
        o[j] += ostep;
        if (o[j] >= n) o[j] -= n;
      }
    };
    if (pos + stride < npos) {
      // the first position apart, so that the loop is entered, like its back
      // edge, with a position's loads and stores in flight (the compiler then
      // waits for the loads alone)
      step([&] { load(pos + stride); }, false);  // in flight while this position is evaluated
      advance();
      for (; pos + stride < npos; advance()) step([&] { load(pos + stride); }, false);
    }
    step([] {}, true);
  }
}

// Several result trees per range and few ranks: each thread loads its fragment of
// every rank once (non-temporal) into its own LDS slots, then evaluates every tree
// from LDS. Dynamic LDS holds P x kThreads 16-byte entries; each thread touches
// only its own entries, so no barrier is needed.
template <int DT, int OPK, int D>
__global__ __launch_bounds__(kThreads) void k_fused_staged(RankPtrs ptrs, const Item* __restrict__ items,
                                                           const int32_t* __restrict__ prog, int P) {
  constexpr int V = TT<DT>::V;
  extern __shared__ u32x4 stage[];
  const Item it = items[item_index(ptrs.xcd)];
  const ProgPtr w = as_prog(prog) + it.tag;
  if (it.count > 0) {
    for_fragments<1>(it, V, [&](int64_t e, const bool (&ok)[1]) {
      for (int base = 0; base < P; base += kLeafBatch) {
        u32x4 raw[kLeafBatch][1];
#pragma unroll
        for (int k = 0; k < kLeafBatch; ++k)
          if (base + k < P) ld_user<DT, 1, true>(ptrs.p[base + k], e, ok, raw[k]);
#pragma unroll
        for (int k = 0; k < kLeafBatch; ++k)
          if (base + k < P) stage[(base + k) * kThreads + threadIdx.x] = raw[k][0];
      }
      replay<DT, OPK, D, kMaxFusedTrees, 1, kLeafBatch>(ptrs, w, e, ok, [&](int rank, u32x4(&r)[1]) {
        r[0] = stage[rank * kThreads + threadIdx.x];
      });
    });
  } else {
    for_fragments<0>(it, V, [&](int64_t e, const bool (&ok)[1]) {
      for (int rank = 0; rank < P; ++rank) {
        u32x4 raw[1] = {u32x4{0, 0, 0, 0}};
        ld_user<DT, 0, true>(ptrs.p[rank], e, ok, raw);
        stage[rank * kThreads + threadIdx.x] = raw[0];
      }
      replay<DT, OPK, D, kMaxFusedTrees, 0, kLeafBatch>(ptrs, w, e, ok, [&](int rank, u32x4(&r)[1]) {
        r[0] = stage[rank * kThreads + threadIdx.x];
      });
    });
  }
}

// ----------------------------------------------------------------------------
// DAG replay: every distinct combination of a range's result trees once
// ----------------------------------------------------------------------------
// A program (words as DagProgram::words on the host: S, nleaf, nlevel, ninstr,
// nout, leaf ranks, level starts, instructions, outputs) evaluates the result
// trees of a range as a DAG in which each distinct combination appears once,
// grouped in levels of independent combinations. A workgroup takes up to
// kDagLanes positions, one per lane (a position is one element, or VW = 4
// consecutive elements), and keeps every value in LDS, [slot][lane] of VW
// words. Its waves share the work of each phase: a wave loads the leaves k =
// wave, wave + waves, ... (four loads in flight), runs the combinations of a
// level the same way (instruction words are wave-uniform: scalar loads; four
// independent combinations per round), and after the last level stores the
// outputs. Barriers separate the phases and the levels; a slot is reused only
// in a later level than its value's last read, or by the one combination that
// reads it last, which reads both operands before it writes. Every store
// follows every load of the workgroup's positions, and no other workgroup
// touches them, so in-place buffers are safe.
constexpr int kDagLanes = 64;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// VW elements at element e of a rank buffer, as accumulation-type bits
template <int DT, int VW>
__device__ __forceinline__ void dag_ld(const void* base, int64_t e, uint32_t (&v)[VW]) {
  if constexpr (VW == 4) {
    if constexpr (DT == D_BF16) {
      const u32x2 r = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(base) + e));
      v[0] = r[0] << 16;
      v[1] = r[0] & 0xffff0000u;
      v[2] = r[1] << 16;
      v[3] = r[1] & 0xffff0000u;
    } else {
      const u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const uint32_t*>(base) + e));
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = r[j];
    }
  } else {
    if constexpr (DT == D_BF16) v[0] = uint32_t(__builtin_nontemporal_load(static_cast<const uint16_t*>(base) + e)) << 16;
    else v[0] = __builtin_nontemporal_load(static_cast<const uint32_t*>(base) + e);
  }
}

template <int DT, int OPK>
__device__ __forceinline__ uint32_t dag_cmb(uint32_t a, uint32_t b) {
  if constexpr (DT == D_INT32) return cmb<OPK>(a, b);
  else return as_u(cmb<OPK>(as_f(a), as_f(b)));
}

// a complete result: O_AVG divides by P, bf16 rounds once to nearest even
template <int DT, int OPK, int VW>
__device__ __forceinline__ void dag_st(void* base, int64_t e, const uint32_t (&v)[VW], float div) {
  uint32_t r[VW];
#pragma unroll
  for (int j = 0; j < VW; ++j) r[j] = OPK == O_AVG ? as_u(as_f(v[j]) / div) : v[j];
  if constexpr (VW == 4) {
    if constexpr (DT == D_BF16) {
      const u32x2 q = {to_bf16(as_f(r[0])) | (to_bf16(as_f(r[1])) << 16),
                       to_bf16(as_f(r[2])) | (to_bf16(as_f(r[3])) << 16)};
      __builtin_nontemporal_store(q, reinterpret_cast<u32x2*>(static_cast<uint16_t*>(base) + e));
    } else {
      const u32x4 q = {r[0], r[1], r[2], r[3]};
      __builtin_nontemporal_store(q, reinterpret_cast<u32x4*>(static_cast<uint32_t*>(base) + e));
    }
  } else {
    if constexpr (DT == D_BF16) __builtin_nontemporal_store(uint16_t(to_bf16(as_f(r[0]))), static_cast<uint16_t*>(base) + e);
    else __builtin_nontemporal_store(r[0], static_cast<uint32_t*>(base) + e);
  }
}

template <int VW>
__device__ __forceinline__ void dag_get(const uint32_t* vals, int slot, int lane, uint32_t (&v)[VW]) {
  if constexpr (VW == 4) {
    const u32x4 q = reinterpret_cast<const u32x4*>(vals)[slot * kDagLanes + lane];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = q[j];
  } else {
    v[0] = vals[slot * kDagLanes + lane];
  }
}
template <int VW>
__device__ __forceinline__ void dag_put(uint32_t* vals, int slot, int lane, const uint32_t (&v)[VW]) {
  if constexpr (VW == 4) reinterpret_cast<u32x4*>(vals)[slot * kDagLanes + lane] = u32x4{v[0], v[1], v[2], v[3]};
  else vals[slot * kDagLanes + lane] = v[0];
}

// The contiguous block [*b0, *b1) of n units that wave `wave` of NW takes (the
// units of a phase split evenly: consecutive program words per wave).
__device__ __forceinline__ void wave_block(int n, int wave, int NW, int* b0, int* b1) {
  const int per = (n + NW - 1) / NW;
  *b0 = min(n, wave * per);
  *b1 = min(n, *b0 + per);
}

// One workgroup's positions [start, start + cnt * VW). `w` is the program (its
// words are read as scalars; each wave reads a contiguous block of each phase,
// so its words share scalar cache lines). SHARED: the program's ranks are
// renamed per lane through `row` (the lane's range's row of the renaming table)
// and the buffers come from the LDS pointer table `lptr`.
template <int DT, int OPK, int VW, bool SHARED>
__device__ __forceinline__ void dag_body(const RankPtrs& ptrs, ProgPtr w, int64_t start, int cnt, void* const* lptr,
                                         const uint8_t* row, uint32_t* vals) {
  const int lane = int(threadIdx.x) & (kDagLanes - 1);
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) / kDagLanes);
  const int NW = int(blockDim.x) / kDagLanes;
  const bool act = lane < cnt;
  const int64_t e = start + int64_t(lane) * VW;
  const int nleaf = w[1], nlev = w[2], ninstr = w[3], nout = w[4];
  const ProgPtr leaves = w + 5;
  const ProgPtr lv = leaves + nleaf;
  const ProgPtr ins = lv + nlev + 1;
  const ProgPtr outs = ins + ninstr;
  auto buf = [&](int rank) -> void* {
    if constexpr (SHARED) return lptr[row[rank]];
    else return ptrs.p[rank];
  };
  // The combinations below are branch-free over the unrolled units, so their
  // LDS accesses overlap. Lanes past `cnt` compute on their own LDS column and
  // skip only the global accesses. Global loads and stores past a block are
  // skipped by wave-uniform (scalar) branches: a repeated non-temporal access
  // would move its line through HBM again.
  int b0, b1;
  wave_block(nleaf, wave, NW, &b0, &b1);
  for (int k0 = b0; k0 < b1; k0 += 8) {  // up to eight loads in flight per lane
    uint32_t v[8][VW];
    if (act) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (k0 + u < b1) dag_ld<DT, VW>(buf(leaves[k0 + u]), e, v[u]);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (k0 + u < b1) dag_put<VW>(vals, k0 + u, lane, v[u]);
  }
  __syncthreads();
  for (int l = 0; l < nlev; ++l) {
    wave_block(lv[l + 1] - lv[l], wave, NW, &b0, &b1);
    b0 += lv[l];
    b1 += lv[l];
    // whole groups of four (their eight operand reads in flight together), then
    // the block's remainder one combination at a time
    int i = b0;
    for (; i + 4 <= b1; i += 4) {
      uint32_t iw[4], a[4][VW], b[4][VW];
#pragma unroll
      for (int u = 0; u < 4; ++u) iw[u] = uint32_t(ins[i + u]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        dag_get<VW>(vals, int((iw[u] >> 10) & 1023u), lane, a[u]);
        dag_get<VW>(vals, int(iw[u] >> 20), lane, b[u]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
#pragma unroll
        for (int j = 0; j < VW; ++j) a[u][j] = dag_cmb<DT, OPK>(a[u][j], b[u][j]);
        dag_put<VW>(vals, int(iw[u] & 1023u), lane, a[u]);
      }
    }
    for (; i < b1; ++i) {
      const uint32_t iw = uint32_t(ins[i]);
      uint32_t a[VW], b[VW];
      dag_get<VW>(vals, int((iw >> 10) & 1023u), lane, a);
      dag_get<VW>(vals, int(iw >> 20), lane, b);
#pragma unroll
      for (int j = 0; j < VW; ++j) a[j] = dag_cmb<DT, OPK>(a[j], b[j]);
      dag_put<VW>(vals, int(iw & 1023u), lane, a);
    }
    __syncthreads();
  }
  wave_block(nout, wave, NW, &b0, &b1);
  for (int o0 = b0; o0 < b1; o0 += 8) {
    int ow[8];
    uint32_t v[8][VW];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      ow[u] = outs[min(o0 + u, b1 - 1)];
      dag_get<VW>(vals, ow[u] >> 16, lane, v[u]);
    }
    if (act) {
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (o0 + u < b1) dag_st<DT, OPK, VW>(buf(ow[u] & 0xffff), e, v[u], ptrs.div);
    }
  }
}

// Per-range programs (SHARED false): one work item per workgroup, `count` > 0
// positions of 4 elements (16-byte aligned vectors; 8-byte for bf16), < 0 single
// elements, at most kDagLanes, all in one range; the item's tag is its program's
// offset. One program for every range (SHARED): workgroup b takes elements
// first + b * kDagLanes onward, one per lane; `tab` holds the range of each of
// the n offsets of an instance (padded to 8 bytes), then per range a row of P
// bytes renaming the program's ranks to the range's (tab_rows rows; the table is
// padded to a multiple of 4 bytes). LDS: S slots of kDagLanes values (of 4
// words if any item has vectors; `vals_words` words in all), then (SHARED) the
// P buffer pointers and the table.
template <int DT, int OPK, bool SHARED>
__global__ __launch_bounds__(1024) void k_fused_dag(RankPtrs ptrs, const Item* __restrict__ items,
                                                    const int32_t* __restrict__ prog, const uint8_t* __restrict__ tab,
                                                    int64_t first, int64_t total, int32_t n, int32_t P,
                                                    int32_t vals_words, int32_t tab_rows) {
  extern __shared__ u32x4 dag_lds[];
  uint32_t* vals = reinterpret_cast<uint32_t*>(dag_lds);
  if constexpr (SHARED) {
    // the buffer pointers and the renaming table (range of each offset, then
    // the rows) copied to LDS once: a lane's rank lookups are LDS reads
    void** lptr = reinterpret_cast<void**>(vals + vals_words);
    uint8_t* ltab = reinterpret_cast<uint8_t*>(lptr + P);
    const int tab_words = ((n + 7) / 8 * 8 + tab_rows * P + 3) / 4;
    if (threadIdx.x == 0)
      for (int x = 0; x < P; ++x) lptr[x] = ptrs.p[x];
    for (int i = int(threadIdx.x); i < tab_words; i += int(blockDim.x))
      reinterpret_cast<uint32_t*>(ltab)[i] = reinterpret_cast<const uint32_t*>(tab)[i];
    __syncthreads();
    const int64_t pos0 = first + int64_t(blockIdx.x) * kDagLanes;
    const int64_t left = total - pos0;
    const int cnt = int(left < kDagLanes ? left : kDagLanes);
    const int lane = int(threadIdx.x) & (kDagLanes - 1);
    const uint8_t* row = ltab;
    if (lane < cnt) {
      const int o = int((pos0 + lane) % n);
      row = ltab + (n + 7) / 8 * 8 + int(ltab[o]) * P;
    }
    dag_body<DT, OPK, 1, true>(ptrs, as_prog(prog), pos0, cnt, lptr, row, vals);
  } else {
    const Item it = items[item_index(ptrs.xcd)];
    const ProgPtr w = as_prog(prog) + it.tag;
    if (it.count > 0) dag_body<DT, OPK, 4, false>(ptrs, w, it.start, it.count, nullptr, nullptr, vals);
    else dag_body<DT, OPK, 1, false>(ptrs, w, it.start, -it.count, nullptr, nullptr, vals);
  }
}

// ----------------------------------------------------------------------------
// literal step execution
// ----------------------------------------------------------------------------
struct WsDesc {
  char* base;
  int64_t slot_bytes;  // bytes of one (slot, rank) workspace buffer
  int32_t P;
};

__device__ __forceinline__ void* slot_ptr(const RankPtrs& ptrs, const WsDesc& ws, int rank, int slot) {
  return slot == 0 ? ptrs.p[rank] : ws.base + (int64_t(slot - 1) * ws.P + rank) * ws.slot_bytes;
}

template <int DT, int M>
__device__ __forceinline__ void ld_slot(const RankPtrs& ptrs, const WsDesc& ws, int rank, int slot, int64_t e,
                                        const bool (&ok)[mm<M>()], typename TT<DT>::A (&out)[nvals<DT, M>()]) {
  if (slot == 0) {
    u32x4 r[mm<M>()];
#pragma unroll
    for (int j = 0; j < mm<M>(); ++j) r[j] = u32x4{0, 0, 0, 0};
    ld_user<DT, M>(ptrs.p[rank], e, ok, r);
    widen<DT, M>(r, out);
  } else {
    ld_acc<DT, M>(slot_ptr(ptrs, ws, rank, slot), e, ok, out);
  }
}

template <int DT, int M>
__device__ __forceinline__ void st_slot(const RankPtrs& ptrs, const WsDesc& ws, int rank, int slot, int64_t e,
                                        const bool (&ok)[mm<M>()], const typename TT<DT>::A (&v)[nvals<DT, M>()]) {
  if (slot == 0) st_user<DT, M>(ptrs.p[rank], e, ok, v);
  else st_acc<DT, M>(slot_ptr(ptrs, ws, rank, slot), e, ok, v);
}


// Literal work records. A workgroup either runs one chunk (count != 0) or a
// packed group of up to kThreads / S small chunks, S threads each (S a power of
// two >= the chunk's units; a unit is one vector of a vector chunk or one
// element of an element chunk). The op travels inside the record, so a
// workgroup reaches its data after one metadata load (two when packed): a step
// made of thousands of tiny chunks then neither pays one workgroup per chunk
// nor a chain of dependent table lookups.
struct LitCode {
  uint8_t kind;  // bit 0: copy (else combine into dst); bit 1: second destination
  uint8_t src_rank, src_slot, own_slot, dst_rank, dst_slot, dst2_rank, dst2_slot;
};
enum : uint8_t { kLitCopy = 1, kLitDst2 = 2, kLitAvg = 4 };  // kLitAvg: the combination completes an average
struct LitWork {
  int64_t start;  // first element of the chunk, or first packed chunk (count == 0)
  int32_t count;  // > 0 vectors, < 0 elements, 0 packed group
  int32_t pack;   // packed group: (chunks << 8) | log2 S
  LitCode code;
};
constexpr int kPackSmall = 64;  // chunks of fewer units are packed

template <int DT, int OPK, int M>
__device__ __forceinline__ void literal_one(const RankPtrs& ptrs, const WsDesc& ws, const LitCode& c, int64_t e,
                                            const bool (&ok)[mm<M>()]) {
  using A = typename TT<DT>::A;
  constexpr int N = nvals<DT, M>();
  A s[N], r[N];
  ld_slot<DT, M>(ptrs, ws, c.src_rank, c.src_slot, e, ok, s);
  if (!(c.kind & kLitCopy)) {
    A o[N];
    ld_slot<DT, M>(ptrs, ws, c.dst_rank, c.own_slot, e, ok, o);
#pragma unroll
    for (int i = 0; i < N; ++i) r[i] = cmb<OPK>(o[i], s[i]);
    if constexpr (OPK == O_AVG) {
      if (c.kind & kLitAvg) {
#pragma unroll
        for (int i = 0; i < N; ++i) r[i] = r[i] / ptrs.div;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) r[i] = s[i];
  }
  st_slot<DT, M>(ptrs, ws, c.dst_rank, c.dst_slot, e, ok, r);
  if (c.kind & kLitDst2) st_slot<DT, M>(ptrs, ws, c.dst2_rank, c.dst2_slot, e, ok, r);
}

template <int DT, int OPK>
__global__ __launch_bounds__(kThreads) void k_literal(RankPtrs ptrs, WsDesc ws, const LitWork* __restrict__ work,
                                                      const LitWork* __restrict__ packed) {
  constexpr int V = TT<DT>::V;
  constexpr int M = 2;
  const LitWork w = work[blockIdx.x];
  if (w.count != 0) {
    const Item it{w.start, w.count, 0};
    if (it.count > 0) {
      for_fragments<M>(it, V, [&](int64_t e, const bool (&ok)[M]) { literal_one<DT, OPK, M>(ptrs, ws, w.code, e, ok); });
    } else {
      for_fragments<0>(it, V, [&](int64_t e, const bool (&ok)[1]) { literal_one<DT, OPK, 0>(ptrs, ws, w.code, e, ok); });
    }
    return;
  }
  const int lg = w.pack & 0xff;
  const int chunks = w.pack >> 8;
  const int c = int(threadIdx.x) >> lg;
  const int k = int(threadIdx.x) & ((1 << lg) - 1);
  if (c >= chunks) return;
  const LitWork x = packed[w.start + c];
  const bool ok[1] = {true};
  if (x.count > 0) {
    if (k < x.count) literal_one<DT, OPK, 1>(ptrs, ws, x.code, x.start + int64_t(k) * V, ok);
  } else if (k < -x.count) {
    literal_one<DT, OPK, 0>(ptrs, ws, x.code, x.start + k, ok);
  }
}

// ----------------------------------------------------------------------------
// direct: read all P, fold left to right, write all P
// ----------------------------------------------------------------------------
template <int DT, int OPK, int M, int B>
__device__ __forceinline__ void direct_one(const RankPtrs& ptrs, int P, int64_t e, const bool (&ok)[mm<M>()]) {
  using A = typename TT<DT>::A;
  constexpr int N = nvals<DT, M>();
  A acc[N];
  for (int base = 0; base < P; base += B) {
    u32x4 raw[B][mm<M>()];
#pragma unroll
    for (int k = 0; k < B; ++k) ld_user<DT, M>(ptrs.p[base + k < P ? base + k : base], e, ok, raw[k]);
#pragma unroll
    for (int k = 0; k < B; ++k) {
      if (base + k == 0) {
        widen<DT, M>(raw[0], acc);
      } else if (base + k < P) {
        A l[N];
        widen<DT, M>(raw[k], l);
#pragma unroll
        for (int i = 0; i < N; ++i) acc[i] = cmb<OPK>(acc[i], l[i]);
      }
    }
  }
  if constexpr (OPK == O_AVG) {
#pragma unroll
    for (int i = 0; i < N; ++i) acc[i] = acc[i] / ptrs.div;
  }
  st_user_all<DT, M>(ptrs, P, [](int i) { return i; }, e, ok, acc);
}

// Vectors per thread and rank of the direct kernel: 2, or 4 for launches of a
// few hundred workgroups with few ranks (the launcher decides), where the
// wider fragment keeps more loads in flight (8 x 2^20 fp32: 12.8 -> 11.1 us;
// 2 stays faster at 7 x 2^24 fp32 and at 192 ranks).
constexpr int kDirectM = 2;

// A workgroup takes `per` vectors (at most kThreads x MD): thread t the
// vectors t, t + kThreads, ... below per.
template <int DT, int OPK, bool VEC, int B, int MD = kDirectM>
__global__ __launch_bounds__(kThreads) void k_direct(RankPtrs ptrs, int P, int64_t nvec, int64_t total, int per) {
  constexpr int V = TT<DT>::V;
  if constexpr (VEC) {
    const int64_t vb = int64_t(blockIdx.x) * per + threadIdx.x;
    bool ok[MD];
#pragma unroll
    for (int j = 0; j < MD; ++j) ok[j] = int(threadIdx.x) + j * kThreads < per && vb + j * kThreads < nvec;
    if (ok[0]) direct_one<DT, OPK, MD, B>(ptrs, P, vb * V, ok);
    // the elements past the last whole vector: the last block's highest
    // threads, which a short launch leaves without vectors, so the tail does
    // not add a round of loads after the vectors
    if (blockIdx.x == gridDim.x - 1) {
      const bool one[1] = {true};
      for (int64_t e = nvec * V + (kThreads - 1 - int(threadIdx.x)); e < total; e += kThreads)
        direct_one<DT, OPK, 0, B>(ptrs, P, e, one);
    }
  } else {
    const int64_t g = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    const bool one[1] = {true};
    if (g < total) direct_one<DT, OPK, 0, B>(ptrs, P, g, one);
  }
}

}  // namespace ar

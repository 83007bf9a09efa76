// HIP kernels for gfx950 and the executor that launches them.
//
// Three kernels, all streaming and HBM-bound (no contraction, so no MFMA):
//  * k_fused   -- fused per-element replay. A block takes one work item (a run of
//                 16-byte vectors, or of single elements at ragged range edges)
//                 inside one range of the schedule's fused program. Each thread
//                 evaluates the range's result trees for its vector on a small
//                 register stack in the program's postfix order: leaves are
//                 loaded 8 at a time (128-bit loads), combined in exactly the
//                 order the step list combines them, and the root is written to
//                 every rank listed for that tree. bf16 is widened to fp32 on
//                 load and rounded once on store.
//  * k_literal -- one launch per schedule step: for every op of the step, over
//                 its chunk, dst = own (+) src (REDUCE) or dst = src (COPY/MOVE),
//                 operands in the caller's buffers (slot 0) or in fp32/int32
//                 workspace slots. A pair of mirrored REDUCEs (recursive
//                 doubling's exchange) runs as one op that reads both operands
//                 before writing both results.
//  * k_direct  -- the one-pass direct Allreduce: read P, fold left to right,
//                 write P. It is the HBM-roofline reference: 2 P n elt bytes.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <sstream>
#include <vector>

#include "exec.h"

namespace ar {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct RankPtrs {
  void* p[kMaxRanks];
};

// Work item: `count` > 0 is a run of vectors, < 0 a run of -count single elements;
// `start` is the element offset of its first element in every rank buffer.
struct Item {
  int64_t start;
  int32_t count;
  int32_t tag;  // program word offset (fused) or op index (literal)
};

struct LitOp {
  int32_t kind, src_rank, src_slot, own_slot, dst_rank, dst_slot, dst2_rank, dst2_slot;
};

constexpr int kThreads = 256;
constexpr int kLeafBatch = 8;
constexpr int kMaxFusedTrees = 8;  // distinct result trees per range the fused replay keeps in registers

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
  if constexpr (OPK == O_SUM) {
    return a + b;
  } else {
    // total order on non-NaN floats with -0 < +0: flip the magnitude bits of negatives
    int ia = __float_as_int(a), ib = __float_as_int(b);
    int ka = ia ^ ((ia >> 31) & 0x7fffffff), kb = ib ^ ((ib >> 31) & 0x7fffffff);
    return kb > ka ? b : a;
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
template <int DT, int M>
__device__ __forceinline__ void st_user(void* base, int64_t e, const bool (&ok)[mm<M>()],
                                        const typename TT<DT>::A (&v)[nvals<DT, M>()]) {
  using S = typename TT<DT>::S;
  if constexpr (M == 0) {
    if (ok[0]) {
      if constexpr (DT == D_BF16) __builtin_nontemporal_store(uint16_t(to_bf16(v[0])), reinterpret_cast<uint16_t*>(base) + e);
      else __builtin_nontemporal_store(as_u(v[0]), reinterpret_cast<uint32_t*>(base) + e);
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
template <int DT, int OPK, int D, int M, bool NT>
__device__ __forceinline__ void eval_one(const RankPtrs& ptrs, const int32_t* __restrict__ w, int64_t e,
                                         const bool (&ok)[mm<M>()], typename TT<DT>::A (&res)[nvals<DT, M>()]) {
  using A = typename TT<DT>::A;
  constexpr int N = nvals<DT, M>();
  const int nl = w[0];
  const int32_t* __restrict__ leaf = w + 2;
  const int32_t* __restrict__ nc = leaf + nl;
  A st[D][N];
#pragma unroll
  for (int d = 0; d < D; ++d)
#pragma unroll
    for (int i = 0; i < N; ++i) st[d][i] = A(0);
  for (int base = 0; base < nl; base += kLeafBatch) {
    u32x4 raw[kLeafBatch][mm<M>()];
#pragma unroll
    for (int k = 0; k < kLeafBatch; ++k) {
      const int idx = base + k < nl ? base + k : base;
      ld_user<DT, M, NT>(ptrs.p[leaf[idx]], e, ok, raw[k]);
    }
#pragma unroll
    for (int k = 0; k < kLeafBatch; ++k) {
      if (base + k < nl) {
#pragma unroll
        for (int d = D - 1; d > 0; --d)
#pragma unroll
          for (int i = 0; i < N; ++i) st[d][i] = st[d - 1][i];
        widen<DT, M>(raw[k], st[0]);
        for (int c = nc[base + k]; c > 0; --c) {
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

template <int DT, int OPK, int D, int TM, int M>
__device__ __forceinline__ void replay(const RankPtrs& ptrs, const int32_t* __restrict__ w, int64_t e,
                                       const bool (&ok)[mm<M>()]) {
  using A = typename TT<DT>::A;
  const int ntrees = w[0];
  w += 1;
  A res[TM][nvals<DT, M>()];
  const int32_t* outs[TM];
  int nouts[TM];
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    if (t < ntrees) {
      const int nl = w[0];
      nouts[t] = w[1];
      outs[t] = w + 2 + 2 * nl;
      eval_one<DT, OPK, D, M, TM == 1>(ptrs, w, e, ok, res[t]);
      w = outs[t] + nouts[t];
    }
  }
#pragma unroll
  for (int t = 0; t < TM; ++t) {
    if (t < ntrees) {
      for (int o = 0; o < nouts[t]; ++o) st_user<DT, M>(ptrs.p[outs[t][o]], e, ok, res[t]);
    }
  }
}

// Vectors per thread of the fused replay: two for shallow single-tree
// programs, one where the register stack or several results need the room.
template <int DT, int D, int TM> constexpr int fused_m() { return (TM == 1 && D <= 4) ? 2 : 1; }

template <int DT, int OPK, int D, int TM>
__global__ __launch_bounds__(kThreads) void k_fused(RankPtrs ptrs, const Item* __restrict__ items,
                                                    const int32_t* __restrict__ prog) {
  constexpr int V = TT<DT>::V;
  constexpr int M = fused_m<DT, D, TM>();
  const Item it = items[blockIdx.x];
  const int32_t* w = prog + it.tag;
  if (it.count > 0) {
    for_fragments<M>(it, V, [&](int64_t e, const bool (&ok)[M]) { replay<DT, OPK, D, TM, M>(ptrs, w, e, ok); });
  } else {
    for_fragments<0>(it, V, [&](int64_t e, const bool (&ok)[1]) { replay<DT, OPK, D, TM, 0>(ptrs, w, e, ok); });
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

template <int DT, int OPK, int M>
__device__ __forceinline__ void literal_one(const RankPtrs& ptrs, const WsDesc& ws, const LitOp& op, int64_t e,
                                            const bool (&ok)[mm<M>()]) {
  using A = typename TT<DT>::A;
  constexpr int N = nvals<DT, M>();
  A s[N], r[N];
  ld_slot<DT, M>(ptrs, ws, op.src_rank, op.src_slot, e, ok, s);
  if (op.kind == K_REDUCE) {
    A o[N];
    ld_slot<DT, M>(ptrs, ws, op.dst_rank, op.own_slot, e, ok, o);
#pragma unroll
    for (int i = 0; i < N; ++i) r[i] = cmb<OPK>(o[i], s[i]);
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) r[i] = s[i];
  }
  st_slot<DT, M>(ptrs, ws, op.dst_rank, op.dst_slot, e, ok, r);
  if (op.dst2_rank >= 0) st_slot<DT, M>(ptrs, ws, op.dst2_rank, op.dst2_slot, e, ok, r);
}

template <int DT, int OPK>
__global__ __launch_bounds__(kThreads) void k_literal(RankPtrs ptrs, WsDesc ws, const Item* __restrict__ items,
                                                      const LitOp* __restrict__ ops) {
  constexpr int V = TT<DT>::V;
  constexpr int M = 2;
  const Item it = items[blockIdx.x];
  const LitOp op = ops[it.tag];
  if (it.count > 0) {
    for_fragments<M>(it, V, [&](int64_t e, const bool (&ok)[M]) { literal_one<DT, OPK, M>(ptrs, ws, op, e, ok); });
  } else {
    for_fragments<0>(it, V, [&](int64_t e, const bool (&ok)[1]) { literal_one<DT, OPK, 0>(ptrs, ws, op, e, ok); });
  }
}

// ----------------------------------------------------------------------------
// direct: read all P, fold left to right, write all P
// ----------------------------------------------------------------------------
template <int DT, int OPK, int M>
__device__ __forceinline__ void direct_one(const RankPtrs& ptrs, int P, int64_t e, const bool (&ok)[mm<M>()]) {
  using A = typename TT<DT>::A;
  constexpr int N = nvals<DT, M>();
  A acc[N];
  for (int base = 0; base < P; base += kLeafBatch) {
    u32x4 raw[kLeafBatch][mm<M>()];
#pragma unroll
    for (int k = 0; k < kLeafBatch; ++k) {
      const int r = base + k < P ? base + k : base;
      ld_user<DT, M>(ptrs.p[r], e, ok, raw[k]);
    }
#pragma unroll
    for (int k = 0; k < kLeafBatch; ++k) {
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
  for (int p = 0; p < P; ++p) st_user<DT, M>(ptrs.p[p], e, ok, acc);
}

constexpr int kDirectM = 2;

template <int DT, int OPK, bool VEC>
__global__ __launch_bounds__(kThreads) void k_direct(RankPtrs ptrs, int P, int64_t nvec, int64_t total) {
  constexpr int V = TT<DT>::V;
  if constexpr (VEC) {
    const int64_t vb = int64_t(blockIdx.x) * kThreads * kDirectM + threadIdx.x;
    bool ok[kDirectM];
#pragma unroll
    for (int j = 0; j < kDirectM; ++j) ok[j] = vb + j * kThreads < nvec;
    if (ok[0]) direct_one<DT, OPK, kDirectM>(ptrs, P, vb * V, ok);
    if (blockIdx.x == 0) {
      const bool one[1] = {true};
      for (int64_t e = nvec * V + threadIdx.x; e < total; e += kThreads) direct_one<DT, OPK, 0>(ptrs, P, e, one);
    }
  } else {
    const int64_t g = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    const bool one[1] = {true};
    if (g < total) direct_one<DT, OPK, 0>(ptrs, P, g, one);
  }
}

// ----------------------------------------------------------------------------
// host side: plans, caches, launches
// ----------------------------------------------------------------------------
namespace {

std::mutex g_mu;

std::string spec_key(const Spec& s) {
  std::ostringstream k;
  k << s.P << ',' << s.n << ',' << s.batch << ',' << s.dtype << ',' << s.op << ',' << s.algo << ',' << s.knob << ':';
  for (int g : s.groups) k << g << '.';
  return k.str();
}

std::map<std::string, std::unique_ptr<Schedule>>& sched_cache() {
  static std::map<std::string, std::unique_ptr<Schedule>> m;
  return m;
}

const Schedule* schedule_locked(const Spec& spec, std::string* err) {
  auto& m = sched_cache();
  std::string k = spec_key(spec);
  auto it = m.find(k);
  if (it != m.end()) return it->second.get();
  if (m.size() > 512) m.clear();
  Schedule* s = build_schedule(spec, err);
  if (!s) return nullptr;
  auto* raw = s;
  m.emplace(k, std::unique_ptr<Schedule>(s));
  return raw;
}

int64_t env_int(const char* name, int64_t dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  long long x = std::atoll(v);
  return x > 0 ? x : dflt;
}

void add_segment(std::vector<Item>& out, int64_t s0, int64_t len, int32_t tag, int V, bool vec) {
  static const int64_t item_vec = env_int("AR_ITEM_VECTORS", 2 * kThreads);
  const int64_t item_sc = kThreads;
  if (len <= 0) return;
  if (!vec) {
    for (int64_t off = 0; off < len; off += item_sc) out.push_back({s0 + off, -int32_t(std::min(item_sc, len - off)), tag});
    return;
  }
  int64_t head = (V - s0 % V) % V;
  head = std::min(head, len);
  if (head) out.push_back({s0, -int32_t(head), tag});
  const int64_t b0 = s0 + head;
  const int64_t nv = (len - head) / V;
  for (int64_t off = 0; off < nv; off += item_vec) out.push_back({b0 + off * V, int32_t(std::min(item_vec, nv - off)), tag});
  const int64_t t0 = b0 + nv * V;
  if (s0 + len > t0) out.push_back({t0, -int32_t(s0 + len - t0), tag});
}

struct DevBuf {
  void* p = nullptr;
  ~DevBuf() { if (p) (void)hipFree(p); }
};

struct Plan {
  const Schedule* s = nullptr;
  int exec = E_FUSED;
  int D = 2;
  DevBuf prog, lops;
  DevBuf items[2];  // [vector mode, scalar mode]
  int64_t nitems[2] = {0, 0};
  bool built[2] = {false, false};
  // literal: per launch (step or finalize), range of items
  std::vector<std::pair<int64_t, int64_t>> launches[2];
  int64_t slot_bytes = 0;
  size_t ws_bytes = 0;
};

std::map<std::string, std::unique_ptr<Plan>>& plan_cache() {
  static std::map<std::string, std::unique_ptr<Plan>> m;
  return m;
}

struct Workspace {
  void* p = nullptr;
  size_t bytes = 0;
};
std::map<int, Workspace>& ws_cache() {
  static std::map<int, Workspace> m;
  return m;
}

RunResult hip_fail(hipError_t e, const char* what) {
  RunResult r;
  r.status = 4;  // AR_HIP_ERROR
  r.hip_error = int(e);
  r.message = std::string(what) + ": " + hipGetErrorString(e);
  return r;
}

template <typename T>
hipError_t upload(DevBuf& b, const std::vector<T>& v) {
  if (v.empty()) return hipSuccess;
  hipError_t e = hipMalloc(&b.p, v.size() * sizeof(T));
  if (e != hipSuccess) { b.p = nullptr; return e; }
  return hipMemcpy(b.p, v.data(), v.size() * sizeof(T), hipMemcpyHostToDevice);
}

int vec_width(int dtype) { return dtype == D_BF16 ? 8 : 4; }

// Build the fused or literal item tables for one alignment mode.
RunResult build_items(Plan& pl, bool vec) {
  const Schedule& s = *pl.s;
  const Spec& sp = s.spec;
  const int V = vec_width(sp.dtype);
  const int mode = vec ? 0 : 1;
  std::vector<Item> items;
  if (pl.exec == E_LITERAL) {
    // joint ops per launch
    std::vector<LitOp> lops;
    std::vector<std::pair<int64_t, int64_t>> launches;
    for (int st = 0; st <= s.nsteps; ++st) {
      int64_t first = int64_t(items.size());
      for (int32_t i = s.steps_begin[st]; i < s.steps_begin[st + 1]; ++i) {
        const OpRec& o = s.ops[i];
        if (o.pair >= 0 && o.pair < i) continue;  // executed with its partner
        LitOp lo{o.kind, o.src_rank, o.src_slot, o.own_slot, o.dst_rank, o.dst_slot, -1, -1};
        if (o.pair >= 0) {
          lo.dst2_rank = s.ops[o.pair].dst_rank;
          lo.dst2_slot = s.ops[o.pair].dst_slot;
        }
        int32_t tag = int32_t(lops.size());
        lops.push_back(lo);
        if (sp.batch > 1 && o.offset == 0 && o.length == sp.n) {
          add_segment(items, 0, sp.n * sp.batch, tag, V, vec);
        } else {
          for (int64_t b = 0; b < sp.batch; ++b) add_segment(items, b * sp.n + o.offset, o.length, tag, V, vec);
        }
      }
      if (int64_t(items.size()) > first) launches.push_back({first, int64_t(items.size()) - first});
    }
    if (!pl.lops.p) {
      hipError_t e = upload(pl.lops, lops);
      if (e != hipSuccess) return hip_fail(e, "uploading literal ops");
    }
    pl.launches[mode] = launches;
  } else {
    const bool flat = s.ranges.size() == 1 && s.ranges[0].start == 0 && s.ranges[0].len == sp.n;
    if (sp.batch == 1 || flat) {
      const int64_t mult = flat ? sp.batch : 1;
      for (const FusedRange& r : s.ranges) add_segment(items, r.start, r.len * mult, r.prog, V, vec);
    } else {
      for (int64_t b = 0; b < sp.batch; ++b)
        for (const FusedRange& r : s.ranges) add_segment(items, b * sp.n + r.start, r.len, r.prog, V, vec);
    }
    if (!pl.prog.p) {
      hipError_t e = upload(pl.prog, s.prog);
      if (e != hipSuccess) return hip_fail(e, "uploading the fused program");
    }
  }
  hipError_t e = upload(pl.items[mode], items);
  if (e != hipSuccess) return hip_fail(e, "uploading work items");
  pl.nitems[mode] = int64_t(items.size());
  pl.built[mode] = true;
  return RunResult{};
}

RunResult get_plan(const Spec& spec, int exec, int device, Plan** out) {
  std::string k = spec_key(spec) + "|" + std::to_string(exec) + "|" + std::to_string(device);
  auto& m = plan_cache();
  auto it = m.find(k);
  if (it != m.end()) { *out = it->second.get(); return RunResult{}; }
  std::string err;
  const Schedule* s = schedule_locked(spec, &err);
  if (!s) { RunResult r; r.status = 1; r.message = err; return r; }
  auto pl = std::make_unique<Plan>();
  pl->s = s;
  pl->exec = exec;
  pl->D = s->max_need <= 2 ? 2 : s->max_need <= 4 ? 4 : s->max_need <= 8 ? 8 : 16;
  int64_t slot = spec.n * spec.batch * int64_t(acc_bytes(spec.dtype));
  pl->slot_bytes = (slot + 255) / 256 * 256;
  pl->ws_bytes = size_t(s->nslots - 1) * size_t(spec.P) * size_t(pl->slot_bytes);
  if (m.size() > 256) {
    (void)hipDeviceSynchronize();
    m.clear();
  }
  *out = pl.get();
  m.emplace(k, std::move(pl));
  return RunResult{};
}

// ---- kernel dispatch ----
template <int DT, int OPK>
hipError_t launch_fused_t(int D, int TM, int64_t nitems, const RankPtrs& ptrs, const Item* items, const int32_t* prog,
                          hipStream_t st) {
  const dim3 g{unsigned(nitems), 1, 1};
  const dim3 b{unsigned(kThreads), 1, 1};
  if (TM == 1) {
    switch (D) {
      case 2: hipLaunchKernelGGL((k_fused<DT, OPK, 2, 1>), g, b, 0, st, ptrs, items, prog); break;
      case 4: hipLaunchKernelGGL((k_fused<DT, OPK, 4, 1>), g, b, 0, st, ptrs, items, prog); break;
      case 8: hipLaunchKernelGGL((k_fused<DT, OPK, 8, 1>), g, b, 0, st, ptrs, items, prog); break;
      default: hipLaunchKernelGGL((k_fused<DT, OPK, 16, 1>), g, b, 0, st, ptrs, items, prog); break;
    }
  } else {
    switch (D) {
      case 2: hipLaunchKernelGGL((k_fused<DT, OPK, 2, kMaxFusedTrees>), g, b, 0, st, ptrs, items, prog); break;
      case 4: hipLaunchKernelGGL((k_fused<DT, OPK, 4, kMaxFusedTrees>), g, b, 0, st, ptrs, items, prog); break;
      default: hipLaunchKernelGGL((k_fused<DT, OPK, 8, kMaxFusedTrees>), g, b, 0, st, ptrs, items, prog); break;
    }
  }
  return hipGetLastError();
}

template <int DT, int OPK>
hipError_t launch_literal_t(int64_t nitems, const RankPtrs& ptrs, const WsDesc& ws, const Item* items,
                            const LitOp* ops, hipStream_t st) {
  hipLaunchKernelGGL((k_literal<DT, OPK>), dim3(unsigned(nitems)), dim3(kThreads), 0, st, ptrs, ws, items, ops);
  return hipGetLastError();
}

template <int DT, int OPK>
hipError_t launch_direct_t(bool vec, const RankPtrs& ptrs, int P, int64_t total, hipStream_t st) {
  constexpr int V = TT<DT>::V;
  if (vec) {
    int64_t nvec = total / V;
    int64_t blocks = std::max<int64_t>(1, (nvec + kThreads * kDirectM - 1) / (kThreads * kDirectM));
    hipLaunchKernelGGL((k_direct<DT, OPK, true>), dim3(unsigned(blocks)), dim3(kThreads), 0, st, ptrs, P, nvec, total);
  } else {
    int64_t blocks = std::max<int64_t>(1, (total + kThreads - 1) / kThreads);
    hipLaunchKernelGGL((k_direct<DT, OPK, false>), dim3(unsigned(blocks)), dim3(kThreads), 0, st, ptrs, P, int64_t(0), total);
  }
  return hipGetLastError();
}

#define AR_DISPATCH(DTV, OPV, CALL)                                      \
  do {                                                                    \
    if ((DTV) == D_INT32 && (OPV) == O_SUM) { constexpr int DT = D_INT32, OPK = O_SUM; CALL; } \
    else if ((DTV) == D_INT32) { constexpr int DT = D_INT32, OPK = O_MAX; CALL; }              \
    else if ((DTV) == D_FP32 && (OPV) == O_SUM) { constexpr int DT = D_FP32, OPK = O_SUM; CALL; } \
    else if ((DTV) == D_FP32) { constexpr int DT = D_FP32, OPK = O_MAX; CALL; }                \
    else if ((OPV) == O_SUM) { constexpr int DT = D_BF16, OPK = O_SUM; CALL; }                 \
    else { constexpr int DT = D_BF16, OPK = O_MAX; CALL; }                                     \
  } while (0)

}  // namespace

const Schedule* cached_schedule(const Spec& spec, std::string* err) {
  std::lock_guard<std::mutex> lk(g_mu);
  return schedule_locked(spec, err);
}

RunResult literal_workspace_bytes(const Spec& spec, size_t* bytes) {
  std::string err;
  const Schedule* s = cached_schedule(spec, &err);
  if (!s) { RunResult r; r.status = 1; r.message = err; return r; }
  int64_t slot = (spec.n * spec.batch * int64_t(acc_bytes(spec.dtype)) + 255) / 256 * 256;
  *bytes = size_t(s->nslots - 1) * size_t(spec.P) * size_t(slot);
  return RunResult{};
}

RunResult run_allreduce(void* const* bufs, const Spec& spec, int exec, void* workspace, size_t workspace_bytes,
                        void* stream) {
  RunResult res;
  if (spec.P <= 1 || spec.n == 0) return res;  // nothing to combine
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int V = vec_width(spec.dtype);
  bool vec = true;
  RankPtrs ptrs;
  std::memset(&ptrs, 0, sizeof(ptrs));
  for (int p = 0; p < spec.P; ++p) {
    ptrs.p[p] = bufs[p];
    if (reinterpret_cast<uintptr_t>(bufs[p]) % 16) vec = false;
  }
  const int64_t total = spec.n * spec.batch;
  if (exec == E_FUSED && spec.algo == A_DIRECT) {
    hipError_t e = hipSuccess;
    AR_DISPATCH(spec.dtype, spec.op, (e = launch_direct_t<DT, OPK>(vec, ptrs, spec.P, total, st)));
    if (e != hipSuccess) return hip_fail(e, "launching the direct kernel");
    return res;
  }
  Plan* pl = nullptr;
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    res = get_plan(spec, exec == E_LITERAL ? E_LITERAL : E_FUSED, device, &pl);
    if (res.status) return res;
    const int mode = vec ? 0 : 1;
    if (!pl->built[mode]) {
      if (pl->exec != E_LITERAL && !pl->s->fused_ok) {
        res.status = 5;
        res.message = "fused replay program unavailable: " + pl->s->fused_error;
        return res;
      }
      if (pl->exec != E_LITERAL && (pl->s->max_trees > kMaxFusedTrees || (pl->s->max_trees > 1 && pl->D > 8))) {
        res.status = 2;
        res.message = "fused replay keeps at most " + std::to_string(kMaxFusedTrees) +
                      " distinct result trees of stack depth <= 8 per range in registers; this schedule has " +
                      std::to_string(pl->s->max_trees) + " (use AR_EXEC_LITERAL)";
        return res;
      }
      res = build_items(*pl, vec);
      if (res.status) return res;
    }
    if (pl->exec == E_LITERAL && pl->ws_bytes) {
      if (workspace) {
        if (workspace_bytes < pl->ws_bytes) {
          res.status = 3;
          res.message = "workspace too small: need " + std::to_string(pl->ws_bytes) + " bytes";
          return res;
        }
        ws = workspace;
      } else {
        Workspace& w = ws_cache()[device];
        if (w.bytes < pl->ws_bytes) {
          if (w.p) {
            e = hipDeviceSynchronize();
            if (e != hipSuccess) return hip_fail(e, "synchronizing before growing the workspace");
            (void)hipFree(w.p);
            w.p = nullptr;
            w.bytes = 0;
          }
          e = hipMalloc(&w.p, pl->ws_bytes);
          if (e != hipSuccess) { w.p = nullptr; return hip_fail(e, "allocating the literal workspace"); }
          w.bytes = pl->ws_bytes;
        }
        ws = w.p;
      }
    }
  }
  const int mode = vec ? 0 : 1;
  if (pl->exec == E_LITERAL) {
    WsDesc wd{reinterpret_cast<char*>(ws), pl->slot_bytes, spec.P};
    const Item* items = reinterpret_cast<const Item*>(pl->items[mode].p);
    const LitOp* lops = reinterpret_cast<const LitOp*>(pl->lops.p);
    for (auto& ln : pl->launches[mode]) {
      AR_DISPATCH(spec.dtype, spec.op, (e = launch_literal_t<DT, OPK>(ln.second, ptrs, wd, items + ln.first, lops, st)));
      if (e != hipSuccess) return hip_fail(e, "launching a literal step");
    }
  } else {
    if (pl->nitems[mode] == 0) return res;
    const Item* items = reinterpret_cast<const Item*>(pl->items[mode].p);
    const int32_t* prog = reinterpret_cast<const int32_t*>(pl->prog.p);
    AR_DISPATCH(spec.dtype, spec.op,
                (e = launch_fused_t<DT, OPK>(pl->D, pl->s->max_trees > 1 ? kMaxFusedTrees : 1, pl->nitems[mode], ptrs,
                                             items, prog, st)));
    if (e != hipSuccess) return hip_fail(e, "launching the fused replay");
  }
  (void)V;
  return res;
}

}  // namespace ar

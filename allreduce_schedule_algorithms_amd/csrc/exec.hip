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
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <limits>
#include <map>
#include <memory>
#include <mutex>
#include <sstream>
#include <vector>

#include "exec.h"
#include "jit.h"
#include "launch.h"

namespace ar {

// ----------------------------------------------------------------------------
// host side: plans, caches, launches
// ----------------------------------------------------------------------------
namespace {

std::mutex g_mu;

std::string spec_key(const Spec& s) {
  std::ostringstream k;
  k << s.P << ',' << s.n << ',' << s.batch << ',' << s.dtype << ',' << s.op << ',' << s.algo << ',' << s.knob << ','
    << s.coll << ',' << s.steps << ':';
  for (int g : s.groups) k << g << '.';
  return k.str();
}

// Schedules are shared: a plan keeps its schedule alive even after the
// schedule cache has been cleared.
std::map<std::string, std::shared_ptr<const Schedule>>& sched_cache() {
  static std::map<std::string, std::shared_ptr<const Schedule>> m;
  return m;
}

std::shared_ptr<const Schedule> schedule_locked(const Spec& spec, std::string* err) {
  auto& m = sched_cache();
  std::string k = spec_key(spec);
  auto it = m.find(k);
  if (it != m.end()) return it->second;
  if (m.size() > 512) m.clear();
  std::shared_ptr<const Schedule> s(build_schedule(spec, err));
  if (!s) return nullptr;
  m.emplace(k, s);
  return s;
}

int64_t env_int(const char* name, int64_t dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  long long x = std::atoll(v);
  return x > 0 ? x : dflt;
}

// Buffers in leaf order for one-tree replay over at most 32 ranks (AR_ORDERED=0
// keeps the rank lookups from the program, for comparisons).
bool ordered_enabled() {
  static const bool on = env_int("AR_ORDERED", 1) != 0;
  return on;
}

// Vectors per work item of the program-driven replay (k_fused, k_fused_staged):
// one per thread (measured 2-3% faster than two on the 24-rank batch and on
// AHC's 192 ranks; the literal steps keep two).
int64_t replay_item_vectors() {
  static const int64_t v = env_int("AR_ITEM_VECTORS", kThreads);
  return v;
}

// With `edges` (the program-driven replay, k_fused), the partial vectors at a
// range's ends run in its vector items instead of in element items: the run
// starts at the 256-byte boundary at or before s0 and ends on the vector that
// holds the range's last element, and each item carries in its count the
// elements to skip before s0 (first item) and past the end (last item). Only
// where that last vector would reach past the buffer (`limit` elements) does
// a tail element item remain.
void add_segment(std::vector<Item>& out, int64_t s0, int64_t len, int32_t tag, int V, bool vec,
                 int64_t vectors = 0, int64_t limit = -1) {
  const int64_t item_vec = vectors > 0 ? vectors : 2 * kThreads;
  const int64_t item_sc = kThreads;
  if (len <= 0) return;
  if (!vec) {
    for (int64_t off = 0; off < len; off += item_sc) out.push_back({s0 + off, -int32_t(std::min(item_sc, len - off)), tag});
    return;
  }
  if (limit >= 0) {
    const int64_t A = int64_t(V) * 16, a0 = s0 / A * A, end = s0 + len;
    int64_t t1 = (end + V - 1) / V * V;
    if (t1 > limit) t1 = end / V * V;
    if (t1 > s0) {  // at least one whole vector in the buffer holds range elements
      const int64_t nv = (t1 - a0) / V;
      for (int64_t off = 0; off < nv; off += item_vec) {
        const int64_t cnt = std::min(item_vec, nv - off);
        const int64_t b = a0 + off * V, skip = std::max<int64_t>(0, s0 - b), trim = std::max<int64_t>(0, b + cnt * V - end);
        if (skip >= cnt * V) continue;  // no range element in this item (a head run longer than an item)
        out.push_back({b, item_count(cnt, skip, trim), tag});
      }
      if (end > t1) out.push_back({t1, -int32_t(end - t1), tag});
      return;
    }
  }
  // Vector runs start on a 256-byte boundary (16 vectors of V elements): a wave's
  // 1 KB access then covers whole 128-byte lines instead of splitting one line
  // with the neighbouring wave. The peeled head goes through the element path.
  const int64_t A = int64_t(V) * 16;
  int64_t head = (A - s0 % A) % A;
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
  std::shared_ptr<const Schedule> s;
  int exec = E_FUSED;
  int device = 0;  // the device holding the plan's buffers
  int D = 2;
  DevBuf prog;
  DevBuf items[2];  // [vector mode, scalar mode]
  int64_t nitems[2] = {0, 0};
  bool built[2] = {false, false};
  // literal: per launch (step or finalize), range of work records; packed
  // small chunks
  std::vector<std::pair<int64_t, int64_t>> launches[2];
  DevBuf packed[2];
  std::vector<LitWork> lit_work[2], lit_packed[2];  // literal: the records on the host
  bool host_built[2] = {false, false};
  bool strided = false;  // fused: items are SItem (batches of short ranges)
  // k_fused on one range of one tree over at most 32 ranks: the buffers go to
  // the kernel in leaf order, then output order (these ranks)
  bool ordered = false;
  std::vector<int32_t> ordered_ranks;
  bool rows = false;      // fused: k_fused_rows (strided batches of one program shape)
  int rows_ref = 0;       // its reference range
  bool rows_chain = false;  // whose tree is a chain (each leaf after the first followed by one combination)
  int64_t rows_n = 0;     // the instance length its table describes (1: one range, identity renaming)
  std::vector<uint8_t> rows_tab;  // its range and rank tables
  DevBuf rtab;            // the same on the device
  int shape = SH_NONE;    // fused: every tree of this fixed shape (k_fused_fixed)
  int shape_nl = 0;       // its leaves per tree
  RankTab tab;            // k_fused_fixed: leaf and output ranks per range
  int multi = 0;          // fused: k_fused_multi with this many leaves per tree
  MultiTab mt;            // its ranks
  DevBuf mtab;            // the same as device words
  int md = 2;             // k_fused_fixed: vectors per thread (items of kThreads * md vectors)
  int64_t slot_bytes = 0;
  size_t ws_bytes = 0;
  bool dag = false;         // fused: k_fused_dag
  bool dag_shared = false;  // one program for every range, ranks renamed per lane
  DagPlan dp;               // its programs
  std::vector<uint8_t> dag_tab;  // shared: range of each offset, then the renaming rows
  DevBuf dtab;
  size_t dag_lds[2] = {0, 0};    // per alignment mode: dynamic LDS bytes
  int dag_vals[2] = {0, 0};      // per alignment mode: LDS words of the values
  int dag_words = 0;             // longest program, in words
  size_t lds_limit = 0;
  int kernel = K_NONE;     // the kernel family the plan launches (ar_kernel)
  std::string fallback;   // why a fused call runs the literal steps (empty otherwise)
  size_t device_bytes = 0;  // device memory the plan's tables hold
  // K_JIT: the register DAG kernel compiled for this schedule; loaded on the
  // plan's device at its first launch, unloaded with the plan
  std::vector<char> jit_code;
  int jit_vectors = 2;     // 16-byte vectors per thread (items of kThreads * jit_vectors vectors)
  std::string jit_note;    // why a multi-tree program does not run compiled (empty otherwise)
  bool jit_table = false;  // the table form: one tree shape for every range, ranks from jtab
  std::vector<int32_t> jit_tab;
  int jit_w = 0;           // words per range in jit_tab
  DevBuf jtab;
  struct JitModule {
    JitKernel k;
    ~JitModule() { jit_unload(&k); }
  } jit;
};

// Plans hold device tables that enqueued launches and captured HIP graphs keep
// as kernel arguments, so none is freed while the process may still use it:
// when the cache is full its plans move to the retired list, which keeps them
// (and their device buffers) until ar_release_cached().
std::map<std::string, std::unique_ptr<Plan>>& plan_cache() {
  static std::map<std::string, std::unique_ptr<Plan>> m;
  return m;
}
std::vector<std::unique_ptr<Plan>>& retired_plans() {
  static std::vector<std::unique_ptr<Plan>> v;
  return v;
}
constexpr size_t kMaxLivePlans = 256;

// Literal workspace for calls that bring none: one per (device, stream), so
// calls on different streams never share partials. A workspace that has to
// grow is retired (kept, like a plan) rather than freed, because launches
// still in flight or captured earlier may use it.
struct Workspace {
  void* p = nullptr;
  size_t bytes = 0;
};
std::map<std::pair<int, uintptr_t>, Workspace>& ws_cache() {
  static std::map<std::pair<int, uintptr_t>, Workspace> m;
  return m;
}
std::vector<Workspace>& retired_ws() {
  static std::vector<Workspace> v;
  return v;
}

RunResult hip_fail(hipError_t e, const char* what) {
  RunResult r;
  r.status = 4;  // AR_HIP_ERROR
  r.hip_error = int(e);
  r.message = std::string(what) + ": " + hipGetErrorString(e);
  return r;
}

// Device copy of a host table. The copy is synchronous, so a plan is complete
// before its first launch is enqueued; run_allreduce refuses to build one while
// the caller's stream is capturing.
size_t* g_upload_bytes = nullptr;  // the plan being built counts its bytes here (under g_mu)
template <typename T>
hipError_t upload(DevBuf& b, const std::vector<T>& v) {
  if (v.empty()) return hipSuccess;
  hipError_t e = hipMalloc(&b.p, v.size() * sizeof(T));
  if (e != hipSuccess) { b.p = nullptr; return e; }
  if (g_upload_bytes) *g_upload_bytes += v.size() * sizeof(T);
  return hipMemcpy(b.p, v.data(), v.size() * sizeof(T), hipMemcpyHostToDevice);
}

int vec_width(int dtype) { return dtype == D_BF16 ? 8 : 4; }

// Fused programs above this size run with one contiguous run of items per XCD
// (measured: AHC's 300 KB program +3.4%; programs of a few hundred bytes lose 2-6%).
constexpr size_t kXcdProgramBytes = 64 * 1024;

// Batched calls whose ranges are all shorter than this many elements use
// strided items (one element per thread across instances) instead of one item
// per instance and range.
constexpr int64_t kStridedMaxLen = 64;

// Calls of at most this many elements (n x batch) run the fused replay's
// element path (see run_allreduce).
constexpr int64_t kTinyElements = 4096;

// Whether every range of a single-tree program of at most kMaxTabRanges ranges
// has a tree of the same shape, 1..8 leaves and at most 8 outputs, and which:
//  - SH_BALANCED: a perfect binary tree of 4 or 8 leaves (after leaf k, as many
//    combinations as k + 1 has trailing zero bits);
//  - SH_CHAIN: one combination after every leaf but the first (one leaf: the
//    all-gather's copies);
//  - SH_STACK: any other shape of 3..8 leaves whose stack stays within 4.
// Returns the shape (leaf count in *nl, ranks and counts in *tab), or SH_NONE.
// Unused table entries stay rank 0, a valid buffer the kernel never touches
// for them.
int fixed_shape(const Schedule& s, RankTab* tab, int* nl_out) {
  if (s.max_trees != 1 || s.ranges.empty() || s.ranges.size() > size_t(kMaxTabRanges)) return SH_NONE;
  std::memset(tab, 0, sizeof(*tab));
  const int32_t* nc0 = nullptr;
  int nl0 = 0;
  for (size_t i = 0; i < s.ranges.size(); ++i) {
    const int32_t* w = s.prog.data() + s.ranges[i].prog;
    if (w[0] != 1) return SH_NONE;
    const int nl = w[1], nouts = w[2];
    if (nl < 1 || nl > 8 || nouts < 1 || nouts > 8 || (i > 0 && nl != nl0)) return SH_NONE;
    const int32_t* leaf = w + 3;
    const int32_t* nc = leaf + nl;
    const int32_t* outs = nc + nl;
    if (i == 0) { nc0 = nc; nl0 = nl; }
    for (int k = 0; k < nl; ++k) {
      if (nc[k] != nc0[k]) return SH_NONE;
      tab->leaf[i][k] = uint8_t(leaf[k]);
    }
    for (int k = 0; k < nouts; ++k) tab->out[i][k] = uint8_t(outs[k]);
    tab->nouts[i] = uint8_t(nouts);
  }
  bool chain = nc0[0] == 0, bal = nl0 == 4 || nl0 == 8;
  int depth = 0, most = 0;
  for (int k = 0; k < nl0; ++k) {
    chain = chain && (k == 0 || nc0[k] == 1);
    bal = bal && nc0[k] == __builtin_ctz(unsigned(k + 1));
    depth += 1;
    most = std::max(most, depth);
    depth -= nc0[k];
    tab->nc[k] = uint8_t(nc0[k]);
  }
  *nl_out = nl0;
  if (bal) return SH_BALANCED;
  if (chain) return SH_CHAIN;
  return nl0 >= 3 && most <= 4 && depth == 1 ? SH_STACK : SH_NONE;
}

// Whether a program of several trees per range fits k_fused_multi: at most 8
// ranges of at most 8 trees, every tree with the same combination counts over
// all P = 3..8 leaves and at most 8 outputs. Fills the ranks of *mt.
int multi_shape(const Schedule& s, MultiTab* mt) {
  const int P = s.spec.P;
  if (s.max_trees <= 1 || P < 3 || P > 8 || s.ranges.empty() || s.ranges.size() > 8) return 0;
  std::memset(mt, 0, sizeof(*mt));
  const int32_t* nc0 = nullptr;
  for (size_t i = 0; i < s.ranges.size(); ++i) {
    const int32_t* w = s.prog.data() + s.ranges[i].prog;
    const int nt = w[0];
    if (nt < 1 || nt > 8) return 0;
    mt->ntrees[i] = uint8_t(nt);
    w += 1;
    for (int t = 0; t < nt; ++t) {
      const int nl = w[0], nouts = w[1];
      if (nl != P || nouts < 1 || nouts > 8) return 0;
      const int32_t* leaf = w + 2;
      const int32_t* nc = leaf + nl;
      const int32_t* outs = nc + nl;
      if (!nc0) nc0 = nc;
      for (int k = 0; k < nl; ++k) {
        if (nc[k] != nc0[k]) return 0;
        mt->leaf[i][t][k] = uint8_t(leaf[k]);
      }
      for (int j = 0; j < nouts; ++j) mt->out[i][t][j] = uint8_t(outs[j]);
      mt->nouts[i][t] = uint8_t(nouts);
      w = outs + nouts;
    }
  }
  int depth = 0, most = 0;
  for (int k = 0; k < P; ++k) {
    depth += 1;
    most = std::max(most, depth);
    depth -= nc0[k];
    mt->nc[k] = uint8_t(nc0[k]);
  }
  return most <= 4 && depth == 1 ? P : 0;
}

// Whether a batched call's fused replay uses strided items: several ranges,
// all shorter than kStridedMaxLen elements.
bool strided_items(const Schedule& s) {
  const Spec& sp = s.spec;
  const bool flat = s.ranges.size() == 1 && s.ranges[0].start == 0 && s.ranges[0].len == sp.n;
  if (sp.batch <= 1 || flat) return false;
  int64_t max_len = 0;
  for (const FusedRange& r : s.ranges) max_len = std::max(max_len, r.len);
  return max_len < kStridedMaxLen;
}

// Whether a batched call with strided items can run k_fused_rows instead:
// one tree per range, and every range's program is the reference range's (the
// first non-empty one) with its leaf ranks renamed, with the same combination
// counts and the same output ranks. Fills *t
// with the range of each offset of an instance (n bytes, padded to 8), then the
// renaming map[rank][range] (R bytes per leaf rank of the reference range: the
// rank it stands for in each range; the lanes of one lookup read neighbouring
// bytes), and *ref with the reference range's index.
constexpr int64_t kRowsMaxTable = 4096;  // limit on R x (P | 1) and on n (LDS)
bool rows_table(const Schedule& s, std::vector<uint8_t>* t, int* ref) {
  const Spec& sp = s.spec;
  const int64_t R = int64_t(s.ranges.size()), P = sp.P;
  if (!strided_items(s) || s.max_trees != 1 || R > 255 || R * (P | 1) > kRowsMaxTable || sp.n > kRowsMaxTable)
    return false;
  const int64_t moff = (sp.n + 7) / 8 * 8;
  t->assign(size_t(moff + R * P), 0);
  std::vector<int> cover(size_t(sp.n), -1);
  *ref = -1;
  for (int64_t r = 0; r < R; ++r) {
    const FusedRange& fr = s.ranges[size_t(r)];
    if (fr.len > 0 && *ref < 0) *ref = int(r);
    for (int64_t o = fr.start; o < fr.start + fr.len; ++o) {
      if (o < 0 || o >= sp.n || cover[size_t(o)] >= 0) return false;
      cover[size_t(o)] = int(r);
    }
  }
  for (int64_t o = 0; o < sp.n; ++o) {
    if (cover[size_t(o)] < 0) return false;
    (*t)[size_t(o)] = uint8_t(cover[size_t(o)]);
  }
  const int32_t* w0 = s.prog.data() + s.ranges[size_t(*ref)].prog;
  for (int64_t r = 0; r < R; ++r) {
    if (s.ranges[size_t(r)].len == 0) continue;
    std::vector<int> map(size_t(P), -1);
    const int32_t* a = w0;
    const int32_t* b = s.prog.data() + s.ranges[size_t(r)].prog;
    if (a[0] != b[0]) return false;
    const int nt = a[0];
    ++a;
    ++b;
    for (int q = 0; q < nt; ++q) {
      const int nl = a[0], no = a[1];
      if (b[0] != nl || b[1] != no) return false;
      for (int k = 0; k < nl; ++k) {
        if (a[2 + nl + k] != b[2 + nl + k]) return false;  // combination counts
        int& m = map[size_t(a[2 + k])];
        if (m < 0) m = b[2 + k];
        else if (m != b[2 + k]) return false;
      }
      std::vector<int32_t> oa(a + 2 + 2 * nl, a + 2 + 2 * nl + no), ob(b + 2 + 2 * nl, b + 2 + 2 * nl + no);
      std::sort(oa.begin(), oa.end());
      std::sort(ob.begin(), ob.end());
      if (oa != ob) return false;
      a += 2 + 2 * nl + no;
      b += 2 + 2 * nl + no;
    }
    for (int64_t x = 0; x < P; ++x) (*t)[size_t(moff + x * R + r)] = uint8_t(map[size_t(x)] < 0 ? 0 : map[size_t(x)]);
  }
  t->resize((t->size() + 7) / 8 * 8, 0);  // k_fused_rows_vec copies it in 8-byte runs
  if (P <= kRowsRegMaxRanks) {
    // k_fused_rows_vec in registers: per offset o, one word whose bits
    // 4 x .. 4 x + 3 hold the rank that reference leaf rank x reads at o
    const size_t loff = t->size();
    t->resize(loff + 4 * size_t(sp.n), 0);
    for (int64_t o = 0; o < sp.n; ++o) {
      uint32_t w = 0;
      for (int64_t x = 0; x < P; ++x) w |= uint32_t((*t)[size_t(moff + x * R + cover[size_t(o)])]) << (4 * x);
      std::memcpy(t->data() + loff + 4 * size_t(o), &w, sizeof w);
    }
  }
  return true;
}

// Whether range `ref`'s program is one tree that is a chain: at least two
// leaves, each after the first followed by exactly one combination.
bool chain_tree(const Schedule& s, int ref) {
  if (ref < 0) return false;
  const int32_t* w = s.prog.data() + s.ranges[size_t(ref)].prog;
  if (w[0] != 1 || w[1] < 2) return false;
  const int nl = w[1];
  const int32_t* nc = w + 3 + nl;
  for (int k = 0; k < nl; ++k)
    if (nc[k] != (k == 0 ? 0 : 1)) return false;
  return true;
}

// Whether a k_fused_rows call runs k_fused_rows_vec for its whole vectors:
// 4-byte elements, at most 32 ranks, aligned buffers, more than
// kTinyElements elements, and a reference tree whose result goes to all P ranks
// (an Allreduce's).
constexpr int kRowsVecMaxRanks = 32;
bool rows_vec(const Schedule& s, int ref) {
  const Spec& sp = s.spec;
  if (vec_width(sp.dtype) != 4 || sp.P > kRowsVecMaxRanks || sp.n * sp.batch <= kTinyElements || ref < 0) return false;
  const int32_t* w = s.prog.data() + s.ranges[size_t(ref)].prog;
  return w[0] == 1 && w[2] == sp.P;
}

// LDS one workgroup may allocate on a device (gfx950: 160 KB); host-only plans
// assume the gfx950 figure.
size_t lds_limit(int device) {
  static std::map<int, size_t> m;
  auto it = m.find(device);
  if (it != m.end()) return it->second;
  int v = 0;
  size_t lim = 160 * 1024;
  if (device >= 0 && hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, device) == hipSuccess && v > 0)
    lim = size_t(v);
  m[device] = lim;
  return lim;
}

bool dag_forced() {
  static const bool on = [] {
    const char* v = std::getenv("AR_DAG");  // "1": the DAG replay for every program with several trees per range
    return v && v[0] == '1';
  }();
  return on;
}

// Renaming table of a shared DAG program (the layout of rows_table): the range
// of each offset of an instance, padded to 8 bytes, then per range the P bytes
// of its renaming. False when the ranges do not cover every offset once.
bool dag_table(const Schedule& s, const DagPlan& d, std::vector<uint8_t>* t) {
  const Spec& sp = s.spec;
  const int64_t R = int64_t(s.ranges.size());
  if (R > 256 || !d.shared) return false;
  const int64_t moff = (sp.n + 7) / 8 * 8;
  t->assign(size_t(moff + R * sp.P), 0);
  std::vector<char> seen(size_t(sp.n), 0);
  for (int64_t r = 0; r < R; ++r) {
    const FusedRange& fr = s.ranges[size_t(r)];
    for (int64_t o = fr.start; o < fr.start + fr.len; ++o) {
      if (o < 0 || o >= sp.n || seen[size_t(o)]) return false;
      seen[size_t(o)] = 1;
      (*t)[size_t(o)] = uint8_t(r);
    }
  }
  for (int64_t o = 0; o < sp.n; ++o)
    if (!seen[size_t(o)]) return false;
  std::memcpy(t->data() + moff, d.maps.data(), size_t(R * sp.P));
  t->resize((t->size() + 3) / 4 * 4, 0);  // the kernel copies it to LDS in 4-byte words
  return true;
}

// Work items of the DAG replay: at most kDagLanes positions each, all in one
// range; vec4: runs of 4-element vectors starting on 64-element boundaries,
// the ragged head and tail as single elements.
void dag_segment(std::vector<Item>& out, int64_t s0, int64_t len, int32_t tag, bool vec4) {
  if (len <= 0) return;
  if (!vec4) {
    for (int64_t off = 0; off < len; off += kDagLanes)
      out.push_back({s0 + off, -int32_t(std::min<int64_t>(kDagLanes, len - off)), tag});
    return;
  }
  const int64_t head = std::min<int64_t>((kDagLanes - s0 % kDagLanes) % kDagLanes, len);
  if (head) out.push_back({s0, -int32_t(head), tag});
  const int64_t b0 = s0 + head, nv = (len - head) / 4;
  for (int64_t off = 0; off < nv; off += kDagLanes)
    out.push_back({b0 + off * 4, int32_t(std::min<int64_t>(kDagLanes, nv - off)), tag});
  const int64_t t0 = b0 + nv * 4;
  if (s0 + len > t0) out.push_back({t0, -int32_t(s0 + len - t0), tag});
}

bool fixed_shapes_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("AR_FUSED_SHAPES");  // "0": no shape-specialised kernel (for comparisons)
    return !(v && v[0] == '0');
  }();
  return on;
}

// The literal executor's work records for one alignment mode, on the host.
RunResult literal_tables(Plan& pl, bool vec) {
  const Schedule& s = *pl.s;
  const Spec& sp = s.spec;
  const int V = vec_width(sp.dtype);
  const int mode = vec ? 0 : 1;
  {
    // per launch (schedule step, then the finalize moves): the step's chunks,
    // each joint op with its op code inline
    if (s.nslots > 255) return RunResult{2, 0, "literal execution supports at most 255 slots"};
    std::vector<LitWork> work, packed;
    std::vector<std::pair<int64_t, int64_t>> launches;
    std::vector<Item> chunks;
    std::vector<LitCode> codes;
    for (int st = 0; st <= s.nsteps; ++st) {
      chunks.clear();
      codes.clear();
      for (int32_t i = s.steps_begin[st]; i < s.steps_begin[st + 1]; ++i) {
        const OpRec& o = s.ops[i];
        if (o.pair >= 0 && o.pair < i) continue;  // executed with its partner
        LitCode c{uint8_t(o.kind == K_REDUCE ? 0 : kLitCopy), uint8_t(o.src_rank), uint8_t(o.src_slot),
                  uint8_t(o.own_slot < 0 ? 0 : o.own_slot), uint8_t(o.dst_rank), uint8_t(o.dst_slot), 0, 0};
        if (o.pair >= 0) {
          c.kind |= kLitDst2;
          c.dst2_rank = uint8_t(s.ops[o.pair].dst_rank);
          c.dst2_slot = uint8_t(s.ops[o.pair].dst_slot);
        }
        if (sp.op == O_AVG && s.completes[i]) c.kind |= kLitAvg;
        const int32_t tag = int32_t(codes.size());
        codes.push_back(c);
        if (sp.batch > 1 && o.offset == 0 && o.length == sp.n) {
          add_segment(chunks, 0, sp.n * sp.batch, tag, V, vec);
        } else {
          for (int64_t b = 0; b < sp.batch; ++b) add_segment(chunks, b * sp.n + o.offset, o.length, tag, V, vec);
        }
      }
      if (chunks.empty()) continue;
      // chunks of kPackSmall units or more get a workgroup each; smaller ones
      // are packed, S threads per chunk, kThreads / S chunks per workgroup
      const int64_t w0 = int64_t(work.size());
      size_t i = 0;
      while (i < chunks.size()) {
        const int32_t u0 = chunks[i].count > 0 ? chunks[i].count : -chunks[i].count;
        if (u0 >= kPackSmall) {
          work.push_back({chunks[i].start, chunks[i].count, 0, codes[chunks[i].tag]});
          ++i;
          continue;
        }
        size_t j = i;
        int lg = 0;
        while (j < chunks.size()) {
          const int32_t u = chunks[j].count > 0 ? chunks[j].count : -chunks[j].count;
          if (u >= kPackSmall) break;
          int l2 = lg;
          while ((1 << l2) < u) ++l2;
          if (int64_t(j - i + 1) << l2 > kThreads) break;
          lg = l2;
          ++j;
        }
        if (j - i == 1) {
          work.push_back({chunks[i].start, chunks[i].count, 0, codes[chunks[i].tag]});
        } else {
          work.push_back({int64_t(packed.size()), 0, int32_t((j - i) << 8) | lg, LitCode{}});
          for (size_t q = i; q < j; ++q) packed.push_back({chunks[q].start, chunks[q].count, 0, codes[chunks[q].tag]});
        }
        i = j;
      }
      launches.push_back({w0, int64_t(work.size()) - w0});
    }
    pl.lit_work[mode] = std::move(work);
    pl.lit_packed[mode] = std::move(packed);
    pl.launches[mode] = std::move(launches);
    pl.host_built[mode] = true;
  }
  return RunResult{};
}

// Build the fused or literal item tables for one alignment mode.
bool trace_enabled();

RunResult build_items(Plan& pl, bool vec) {
  int64_t item_vectors_traced = 0;
  const Schedule& s = *pl.s;
  const Spec& sp = s.spec;
  const int V = vec_width(sp.dtype);
  const int mode = vec ? 0 : 1;
  std::vector<Item> items;
  if (pl.exec == E_LITERAL) {
    if (!pl.host_built[mode]) {
      RunResult r = literal_tables(pl, vec);
      if (r.status) return r;
    }
    const std::vector<LitWork>& work = pl.lit_work[mode];
    const std::vector<LitWork>& packed = pl.lit_packed[mode];
    hipError_t e = upload(pl.items[mode], work);
    if (e == hipSuccess) e = upload(pl.packed[mode], packed);
    if (e != hipSuccess) return hip_fail(e, "uploading literal work");
    pl.nitems[mode] = int64_t(work.size());
    pl.built[mode] = true;
    return RunResult{};
  } else if (pl.dag) {
    if (!pl.prog.p) {
      hipError_t e = upload(pl.prog, pl.dp.words);
      if (e != hipSuccess) return hip_fail(e, "uploading the DAG program");
    }
    const size_t vals1 = size_t(pl.dp.S) * kDagLanes * 4;
    const size_t progb = 0;  // the program is read from global memory (scalar loads)
    if (pl.dag_shared) {
      if (!pl.dtab.p) {
        hipError_t e = upload(pl.dtab, pl.dag_tab);
        if (e != hipSuccess) return hip_fail(e, "uploading the renaming table");
      }
      pl.dag_vals[mode] = int(vals1 / 4);
      pl.dag_lds[mode] = vals1 + progb + size_t(sp.P) * sizeof(void*) + pl.dag_tab.size();
      pl.nitems[mode] = 1;  // launched by element count
      pl.built[mode] = true;
      return RunResult{};
    }
    // vectors of 4 elements where the buffers are aligned and four times the values fit the LDS
    const bool vec4 = vec && 4 * vals1 + progb <= pl.lds_limit;
    const bool flat = s.ranges.size() == 1 && s.ranges[0].start == 0 && s.ranges[0].len == sp.n;
    if (sp.batch == 1 || flat) {
      const int64_t mult = flat ? sp.batch : 1;
      for (size_t i = 0; i < s.ranges.size(); ++i)
        dag_segment(items, s.ranges[i].start, s.ranges[i].len * mult, pl.dp.offsets[i], vec4);
    } else {
      for (int64_t b = 0; b < sp.batch; ++b)
        for (size_t i = 0; i < s.ranges.size(); ++i)
          dag_segment(items, b * sp.n + s.ranges[i].start, s.ranges[i].len, pl.dp.offsets[i], vec4);
    }
    pl.dag_vals[mode] = int((vec4 ? 4 * vals1 : vals1) / 4);
    pl.dag_lds[mode] = (vec4 ? 4 * vals1 : vals1) + progb;
  } else {
    const bool flat = s.ranges.size() == 1 && s.ranges[0].start == 0 && s.ranges[0].len == sp.n;
    int64_t max_len = 0;
    for (const FusedRange& r : s.ranges) max_len = std::max(max_len, r.len);
    std::vector<SItem> sitems;
    const bool strided = strided_items(s);
    // the fixed-shape and compiled kernels find a range by its index
    const bool jit = pl.kernel == K_JIT;
    const bool fixed = jit || pl.shape != SH_NONE || pl.multi;
    // k_fused_multi: one vector per thread per item (2-5% faster than two on 7 ranks, r = 1..3)
    int64_t iv = jit ? int64_t(pl.jit_table ? 64 : kThreads) * pl.jit_vectors
                           : pl.multi ? int64_t(kThreads) : fixed ? int64_t(kThreads) * pl.md : replay_item_vectors();
    auto tag_of = [&](size_t i) { return fixed ? int32_t(i) : s.ranges[i].prog; };
    // the program-driven replay of single-tree programs takes the partial
    // vectors at range ends in its vector items
    const int64_t limit = (pl.kernel == K_REPLAY && s.max_trees == 1) || pl.jit_table ? sp.n * sp.batch : -1;
    if (pl.shape != SH_NONE && pl.md == 4 && vec && (sp.batch == 1 || flat)) {
      // four vectors per thread only where their items fill whole rounds of the compute units
      std::vector<Item> probe;
      for (size_t i = 0; i < s.ranges.size(); ++i)
        add_segment(probe, s.ranges[i].start, s.ranges[i].len * (flat ? sp.batch : 1), tag_of(i), V, vec, iv, limit);
      if (!probe.empty() && !four_vectors_fit(int64_t(probe.size()), device_cus())) {
        pl.md = 2;
        iv = int64_t(kThreads) * pl.md;
      }
    }
    if (vec && (sp.batch == 1 || flat) && !strided &&
        (pl.kernel == K_REPLAY || pl.shape != SH_NONE || (pl.kernel == K_JIT && !pl.jit_table && pl.jit_vectors == 1))) {
      // the fewest rounds of workgroups over the compute units that full items
      // need, shared out evenly (the smallest items that still need no more
      // rounds), in whole 256-byte runs so that no two items split a cache line
      auto count = [&](int64_t S) {
        std::vector<Item> probe;
        for (size_t i = 0; i < s.ranges.size(); ++i)
          add_segment(probe, s.ranges[i].start, s.ranges[i].len * (flat ? sp.batch : 1), tag_of(i), V, vec, S, limit);
        return int64_t(probe.size());
      };
      const int64_t cus = device_cus(), most = count(iv);
      const int64_t cap = (most + cus - 1) / cus * cus;
      int64_t lo = kThreads / 64, hi = iv / 16;  // in runs of 16 vectors; count(16 hi) <= cap
      while (lo < hi) {
        const int64_t mid = (lo + hi) / 2;
        if (count(16 * mid) <= cap) hi = mid;
        else lo = mid + 1;
      }
      iv = 16 * hi;
    }
    item_vectors_traced = iv;
    if (sp.batch == 1 || flat) {
      const int64_t mult = flat ? sp.batch : 1;
      for (size_t i = 0; i < s.ranges.size(); ++i)
        add_segment(items, s.ranges[i].start, s.ranges[i].len * mult, tag_of(i), V, vec, iv, limit);
    } else if (strided) {
      // short ranges in many instances: one strided item per range and block
      // of instances; the items of one block sit next to each other, so the
      // ranges sharing its cache lines run together
      const int64_t nb = std::max<int64_t>(1, kThreads / max_len);
      for (int64_t b0 = 0; b0 < sp.batch; b0 += nb)
        for (const FusedRange& r : s.ranges)
          if (r.len > 0)
            sitems.push_back({b0 * sp.n + r.start, r.prog, int32_t(r.len), int32_t(std::min(nb, sp.batch - b0)), 0});
    } else {
      for (int64_t b = 0; b < sp.batch; ++b)
        for (size_t i = 0; i < s.ranges.size(); ++i)
          add_segment(items, b * sp.n + s.ranges[i].start, s.ranges[i].len, tag_of(i), V, vec, iv, limit);
    }
    if (pl.rows) {
      if (!pl.rtab.p) {
        hipError_t e = upload(pl.rtab, pl.rows_tab);
        if (e != hipSuccess) return hip_fail(e, "uploading the range table");
      }
      sitems.clear();
    }
    if (pl.jit_table && !pl.jtab.p) {
      hipError_t e = upload(pl.jtab, pl.jit_tab);
      if (e != hipSuccess) return hip_fail(e, "uploading the rank table");
    }
    if (pl.multi && !pl.mtab.p) {
      std::vector<int32_t> t(8 + 8 * kMultiRangeWords + 16, 0);
      for (int k = 0; k < 8; ++k) t[k] = pl.mt.nc[k];
      for (int r = 0; r < 8; ++r) {
        int32_t* rw = t.data() + 8 + r * kMultiRangeWords;
        rw[0] = pl.mt.ntrees[r];
        for (int q = 0; q < 8; ++q) {
          int32_t* tw = rw + 1 + q * 17;
          for (int k = 0; k < 8; ++k) tw[k] = pl.mt.leaf[r][q][k];
          tw[8] = pl.mt.nouts[r][q];
          for (int k = 0; k < 8; ++k) tw[9 + k] = pl.mt.out[r][q][k];
        }
      }
      hipError_t e = upload(pl.mtab, t);
      if (e != hipSuccess) return hip_fail(e, "uploading the multi-tree table");
    }
    if (!pl.prog.p) {
      // the replay reads each batch's leaf ranks and combination counts as whole
      // runs of kLeafBatch words, so the last tree's runs may reach past its end
      std::vector<int32_t> words(s.prog);
      words.resize(words.size() + 2 * kLeafBatch, 0);
      hipError_t e = upload(pl.prog, words);
      if (e != hipSuccess) return hip_fail(e, "uploading the fused program");
    }
    if (pl.rows) {
      pl.nitems[mode] = 1;  // launched by element count (run_allreduce)
      pl.built[mode] = true;
      return RunResult{};
    }
    if (!sitems.empty()) {
      hipError_t e = upload(pl.items[mode], sitems);
      if (e != hipSuccess) return hip_fail(e, "uploading work items");
      pl.nitems[mode] = int64_t(sitems.size());
      pl.strided = true;
      pl.built[mode] = true;
      return RunResult{};
    }
  }
  if (pl.jit_table) {
    // element items of at most one element per lane (64), then four wave
    // items per workgroup: pad with empty ones
    std::vector<Item> w;
    w.reserve(items.size() + 8);
    for (const Item& x : items) {
      if (x.count >= 0) { w.push_back(x); continue; }
      for (int32_t k = 0; k < -x.count; k += 64) w.push_back(Item{x.start + k, -std::min(64, -x.count - k), x.tag});
    }
    while (w.size() % 4) w.push_back(Item{0, 0, 0});
    items.swap(w);
  }
  if (trace_enabled())
    std::fprintf(stderr, "ar: plan P=%d n=%lld: %zu work items (%s buffers, vector items of at most %lld vectors)\n",
                 sp.P, (long long)sp.n, items.size(), vec ? "aligned" : "unaligned", (long long)item_vectors_traced);
  hipError_t e = upload(pl.items[mode], items);
  if (e != hipSuccess) return hip_fail(e, "uploading work items");
  pl.nitems[mode] = int64_t(items.size());
  pl.built[mode] = true;
  return RunResult{};
}

bool same_spec(const Spec& a, const Spec& b) {
  return a.P == b.P && a.n == b.n && a.batch == b.batch && a.dtype == b.dtype && a.op == b.op && a.algo == b.algo &&
         a.knob == b.knob && a.coll == b.coll && a.steps == b.steps && a.groups == b.groups;
}

// Whether the fused replay can run a schedule: at most kMaxFusedTrees result
// trees per range, and several trees only with a stack of depth <= 8.
bool fused_runs(const Schedule& s) {
  const int D = s.max_need <= 2 ? 2 : s.max_need <= 4 ? 4 : s.max_need <= 8 ? 8 : 16;
  return s.max_trees <= kMaxFusedTrees && !(s.max_trees > 1 && D > 8);
}

const char* kernel_name(int k) {
  static const char* names[] = {"none", "k_direct", "k_literal", "k_fused", "k_fused_staged", "k_fused_strided",
                                "k_fused_fixed (chain)", "k_fused_fixed (balanced)", "k_fused_fixed (stack)",
                                "k_fused_multi", "k_fused_rows", "k_fused_rows_vec", "k_fused_dag", "ar_jit"};
  return k >= 0 && k < int(sizeof(names) / sizeof(names[0])) ? names[k] : "?";
}

// The kernel family a fused plan launches, in the order run_allreduce tries
// them; K_LITERAL (with the reason in pl.fallback) when no replay holds the
// program.
bool jit_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("AR_JIT");  // "0": no run-time compiled kernels (for comparisons)
    return !(v && v[0] == '0');
  }();
  return on;
}

// The compiled register DAG kernel of s: generated, then compiled once per
// distinct source (schedules of one shape at other sizes share it). False and
// *why when it is not available.
bool jit_code_for(const Schedule& s, std::vector<char>* code, int* vectors, std::string* why) {
  static std::mutex mu;
  static std::map<std::string, std::pair<std::vector<char>, int>> cache;
  if (!jit_available(why)) return false;
  // two vectors per thread (measured 23% faster than one on 7 x 2^24 fp32)
  // where that still leaves at least 2048 workgroups; shorter calls keep the
  // workgroups (6 ranks x 10^4 x 106 fp32, r = 3: one vector per thread)
  const int64_t call_vectors = s.spec.n * s.spec.batch / vec_width(s.spec.dtype);
  const int max_vectors = call_vectors >= (int64_t(1) << 20) ? 2 : 1;
  std::string src;
  int v = 0;
  if (!jit_source(s, s.spec.dtype, s.spec.op, max_vectors, &src, &v, why)) return false;
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find(src);
  if (it == cache.end()) {
    std::vector<char> c;
    if (!jit_compile(src, &c, why)) return false;
    it = cache.emplace(src, std::make_pair(std::move(c), v)).first;
  }
  *code = it->second.first;
  *vectors = it->second.second;
  return true;
}

// The table-form kernel of s (jit.h), compiled once per distinct source.
bool jit_table_code_for(const Schedule& s, Plan& pl, std::string* why) {
  static std::mutex mu;
  static std::map<std::string, std::pair<std::vector<char>, int>> cache;
  if (!jit_available(why)) return false;
  std::string src;
  int vectors = 0;
  if (!jit_table_source(s, s.spec.dtype, s.spec.op, 2, &src, &pl.jit_tab, &pl.jit_w, &vectors, why)) return false;
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find(src);
  if (it == cache.end()) {
    std::vector<char> c;
    if (!jit_compile(src, &c, why)) return false;
    it = cache.emplace(src, std::make_pair(std::move(c), vectors)).first;
  }
  pl.jit_code = it->second.first;
  pl.jit_vectors = it->second.second;
  pl.jit_table = true;
  return true;
}

void choose_kernel(Plan& pl) {
  const Schedule& s = *pl.s;
  if (pl.exec == E_LITERAL) { pl.kernel = K_LITERAL; return; }
  if (!s.fused_ok) {
    pl.kernel = K_LITERAL;
    pl.fallback = "no replay program (" + s.fused_error + ")";
    return;
  }
  // Several result trees per range, or a latency-bound call over more than 8
  // ranks, with few ranks and ranges: the range's DAG as straight-line register
  // code, compiled for the schedule (jit.h), where hipRTC is there to compile
  // it; otherwise the kernels below.
  const bool jit_tiny = s.spec.n * s.spec.batch <= kTinyElements && s.spec.P > 8;
  // One range of single-tree programs over more than 32 ranks (halving and
  // doubling, recursive doubling, the binomial tree, the pipelined chain): the
  // tree shape compiled with a rank table, in wave-sized work items.
  if (pl.exec == E_FUSED && fixed_shapes_enabled() && jit_enabled() && s.max_trees == 1 && s.ranges.size() == 1 &&
      s.spec.P > kJitMaxRanks && !jit_tiny && !strided_items(s) && !pl.rows && pl.shape == SH_NONE) {
    if (jit_table_code_for(s, pl, &pl.jit_note)) {
      pl.kernel = K_JIT;
      return;
    }
  }
  if (pl.exec == E_FUSED && fixed_shapes_enabled() && jit_enabled() && (s.max_trees > 1 || jit_tiny) &&
      !strided_items(s) && s.spec.P <= kJitMaxRanks && int(s.ranges.size()) <= kJitMaxRanges) {
    if (jit_code_for(s, &pl.jit_code, &pl.jit_vectors, &pl.jit_note)) {
      pl.kernel = K_JIT;
      return;
    }
  }
  // The DAG replay (each distinct combination once, values in LDS) takes:
  // programs with more result trees than the register replays hold; other
  // programs of several trees per range except those k_fused_multi holds and
  // batches of short ranges of several shapes (strided items); and
  // latency-bound calls over many ranks whose trees are shallow (one element
  // per lane, every rank loaded at once instead of in rounds of eight).
  const bool tiny = s.spec.n * s.spec.batch <= kTinyElements;
  const bool many = s.max_trees > 1 && !pl.multi && !strided_items(s);
  const bool wide = s.max_trees == 1 && tiny && s.spec.P >= 16;
  if (pl.exec == E_DAG || (s.max_trees > 1 && (!fused_runs(s) || dag_forced())) ||
      (pl.exec == E_FUSED && fixed_shapes_enabled() && (many || wide))) {
    std::string err;
    if (!dag_plan(s, &pl.dp, &err)) {
      pl.kernel = K_LITERAL;
      pl.fallback = "no DAG program (" + err + ")";
      return;
    }
    if (pl.exec == E_FUSED && fused_runs(s) && !dag_forced() && wide && !many &&
        pl.dp.levels > 2 * ceil_log2(s.spec.P)) {
      pl.dp = DagPlan{};  // a deep tree (a chain): one barrier per level would not pay
      goto registers;
    }
    int64_t max_len = 0;
    for (const FusedRange& r : s.ranges) max_len = std::max(max_len, r.len);
    // the renaming table goes to LDS: only short instances (n <= 4096) share one program
    pl.dag_shared = pl.dp.shared && s.ranges.size() > 1 && max_len < 4 * kDagLanes && s.spec.n <= 4096 &&
                    dag_table(s, pl.dp, &pl.dag_tab);
    if (pl.dp.shared && s.ranges.size() > 1 && !pl.dag_shared && !dag_plan(s, &pl.dp, &err, false)) {
      // long ranges run per-range work items, each with its own range's program
      pl.kernel = K_LITERAL;
      pl.fallback = "no DAG program (" + err + ")";
      return;
    }
    pl.dag_words = 0;
    for (size_t r = 0; r < pl.dp.offsets.size(); ++r) {
      const int32_t* w = pl.dp.words.data() + pl.dp.offsets[r];
      pl.dag_words = std::max(pl.dag_words, 5 + w[1] + w[2] + 1 + w[3] + w[4]);
    }
    const size_t need = size_t(pl.dp.S) * kDagLanes * 4 +
                        (pl.dag_shared ? size_t(s.spec.P) * sizeof(void*) + pl.dag_tab.size() : 0);
    if (need > pl.lds_limit) {
      pl.kernel = K_LITERAL;
      pl.fallback = "the DAG replay needs " + std::to_string(need) + " bytes of LDS per workgroup (" +
                    std::to_string(pl.dp.S) + " values per element, a program of " + std::to_string(pl.dag_words) +
                    " words); the device allows " + std::to_string(pl.lds_limit);
      return;
    }
    pl.dag = true;
    pl.kernel = K_DAG;
    return;
  }
registers:
  if (!fused_runs(s)) {
    pl.kernel = K_LITERAL;
    pl.fallback = std::to_string(s.max_trees) + " result trees per range with a stack of " +
                  std::to_string(s.max_need) + " (the replay keeps at most " + std::to_string(kMaxFusedTrees) +
                  " trees, with a stack of at most 8)";
    return;
  }
  if (pl.rows) pl.kernel = rows_vec(s, pl.rows_ref) ? K_ROWS_VEC : K_ROWS;
  else if (strided_items(s)) pl.kernel = K_STRIDED;
  else if (pl.shape == SH_CHAIN) pl.kernel = K_FIXED_CHAIN;
  else if (pl.shape == SH_BALANCED) pl.kernel = K_FIXED_BALANCED;
  else if (pl.shape == SH_STACK) pl.kernel = K_FIXED_STACK;
  else if (pl.multi) pl.kernel = K_MULTI;
  else if (s.max_trees > 1 && s.spec.P <= kMaxStagedRanks) pl.kernel = K_STAGED;
  else pl.kernel = K_REPLAY;
  if (pl.kernel == K_REPLAY && s.max_trees == 1 && s.ranges.size() == 1 && s.spec.P <= 32 && pl.D <= 8 &&
      ordered_enabled()) {
    const int32_t* w = s.prog.data() + s.ranges[0].prog;  // ntrees, leaves, outputs, ranks, counts, outputs
    const int nl = w[1], no = w[2];
    if (nl + no <= kMaxRanks) {
      pl.ordered_ranks.assign(w + 3, w + 3 + nl);
      pl.ordered_ranks.insert(pl.ordered_ranks.end(), w + 3 + 2 * nl, w + 3 + 2 * nl + no);
      pl.ordered = true;
    }
  }
}

bool trace_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("AR_TRACE");  // "1": one line per plan on stderr
    return v && v[0] && v[0] != '0';
  }();
  return on;
}

void trace_plan(const Plan& pl) {
  static const char* dt[] = {"int32", "fp32", "bf16"};
  static const char* op[] = {"sum", "max", "avg"};
  static const char* coll[] = {"allreduce", "reduce_scatter", "all_gather"};
  static const char* algo[] = {"direct", "ring", "rh_rd", "rd", "binomial", "generalized", "generalized_xor", "ahc",
                               "chain"};
  const Schedule& s = *pl.s;
  const Spec& sp = s.spec;
  std::ostringstream o;
  o << "ar: plan P=" << sp.P << " n=" << sp.n << " batch=" << sp.batch << ' ' << dt[sp.dtype] << ' ' << op[sp.op]
    << ' ' << algo[sp.algo] << " knob=" << sp.knob << " steps=" << sp.steps << ' ' << coll[sp.coll];
  if (!sp.groups.empty()) {
    o << " groups=";
    for (size_t i = 0; i < sp.groups.size(); ++i) o << (i ? "," : "") << sp.groups[i];
  }
  static const char* ex[] = {"fused", "literal", "replay", "dag"};
  o << " exec=" << ex[pl.exec] << " device=" << pl.device << ": kernel "
    << kernel_name(pl.kernel) << " (method steps " << s.nsteps << ", slots " << s.nslots << ", ranges "
    << s.ranges.size() << ", most trees " << s.max_trees << ", stack " << s.max_need << ", most leaves "
    << s.max_leaves << ", program words " << s.prog.size() << ")";
  if (pl.kernel == K_DAG)
    o << "; DAG " << (pl.dag_shared ? "shared by every range" : pl.dp.shared ? "one program" : "per range")
      << ": " << pl.dp.instr << " combinations per element in " << pl.dp.levels << " levels, " << pl.dp.S << " slots";
  if (pl.kernel == K_LITERAL) o << "; " << s.nsteps << " step launches" << (s.finalize_ops ? " + 1 finalize" : "");
  if (pl.kernel == K_JIT)
    o << "; compiled " << (pl.jit_table ? "tree shape with a rank table, wave items" : "register DAG")
      << ", " << pl.jit_vectors << " vectors per thread, code object " << pl.jit_code.size()
      << " bytes";
  if (!pl.jit_note.empty()) o << "; not compiled: " << pl.jit_note;
  if (!pl.fallback.empty()) o << "; literal fallback: " << pl.fallback;
  std::fprintf(stderr, "%s\n", o.str().c_str());
}

// The plan kind of an execution mode: AR_EXEC_REPLAY shares the fused plans
// (it only differs for AR_DIRECT, which then replays instead of the direct kernel).
int plan_exec(int exec) { return exec == E_REPLAY ? E_FUSED : exec; }

// Repeated calls with one spec (a training loop's buckets, the unbatched
// small-message case) skip building the cache key: the last plan found on
// this thread is reused while the plan cache has not been emptied since.
uint64_t g_plan_generation = 0;  // bumped whenever the plan cache is emptied (under g_mu)
struct LastPlan {
  Spec spec;
  int exec = -1, device = -2;
  uint64_t generation = 0;
  Plan* plan = nullptr;
};
thread_local LastPlan t_last;

// Device -1 builds a host-only plan (kernel choice, sizes; no device tables).
RunResult get_plan(const Spec& spec, int exec, int device, Plan** out) {
  if (t_last.plan && t_last.generation == g_plan_generation && t_last.exec == exec && t_last.device == device &&
      same_spec(t_last.spec, spec)) {
    *out = t_last.plan;
    return RunResult{};
  }
  auto remember = [&](Plan* p) {
    t_last.spec = spec;
    t_last.exec = exec;
    t_last.device = device;
    t_last.generation = g_plan_generation;
    t_last.plan = p;
  };
  std::string k = spec_key(spec) + "|" + std::to_string(exec) + "|" + std::to_string(device);
  auto& m = plan_cache();
  auto it = m.find(k);
  if (it != m.end()) {
    *out = it->second.get();
    remember(*out);
    return RunResult{};
  }
  std::string err;
  std::shared_ptr<const Schedule> s = schedule_locked(spec, &err);
  if (!s) { RunResult r; r.status = 1; r.message = err; return r; }
  auto pl = std::make_unique<Plan>();
  pl->s = s;
  pl->exec = exec;
  pl->device = device;
  if (exec == E_FUSED && s->fused_ok && fixed_shapes_enabled()) {
    pl->shape = fixed_shape(*s, &pl->tab, &pl->shape_nl);
    if (pl->shape == SH_NONE) pl->multi = multi_shape(*s, &pl->mt);
    pl->rows = rows_table(*s, &pl->rows_tab, &pl->rows_ref);
    if (pl->rows) pl->rows_chain = chain_tree(*s, pl->rows_ref);
    pl->rows_n = spec.n;
    // four vectors per thread for short launches with few ranks, as the direct kernel
    pl->md = spec.P <= 8 && spec.n * spec.batch / vec_width(spec.dtype) <= (int64_t(1) << 19) ? 4 : 2;
  }
  pl->D = s->max_need <= 2 ? 2 : s->max_need <= 4 ? 4 : s->max_need <= 8 ? 8 : 16;
  int64_t slot = spec.n * spec.batch * int64_t(acc_bytes(spec.dtype));
  pl->slot_bytes = (slot + 255) / 256 * 256;
  pl->ws_bytes = size_t(s->nslots - 1) * size_t(spec.P) * size_t(pl->slot_bytes);
  pl->lds_limit = lds_limit(device);
  choose_kernel(*pl);
  if (trace_enabled()) trace_plan(*pl);
  if (m.size() >= kMaxLivePlans) {
    // retire, never free: launches in flight and captured graphs keep their tables
    for (auto& kv : m) retired_plans().push_back(std::move(kv.second));
    m.clear();
    ++g_plan_generation;
  }
  *out = pl.get();
  m.emplace(k, std::move(pl));
  remember(*out);
  return RunResult{};
}

// ---- kernel dispatch ----
#define AR_DISPATCH(DTV, OPV, CALL)                                      \
  do {                                                                    \
    if ((DTV) == D_INT32 && (OPV) == O_SUM) { constexpr int DT = D_INT32, OPK = O_SUM; CALL; } \
    else if ((DTV) == D_INT32) { constexpr int DT = D_INT32, OPK = O_MAX; CALL; }              \
    else if ((DTV) == D_FP32 && (OPV) == O_SUM) { constexpr int DT = D_FP32, OPK = O_SUM; CALL; } \
    else if ((DTV) == D_FP32 && (OPV) == O_AVG) { constexpr int DT = D_FP32, OPK = O_AVG; CALL; } \
    else if ((DTV) == D_FP32) { constexpr int DT = D_FP32, OPK = O_MAX; CALL; }                \
    else if ((OPV) == O_SUM) { constexpr int DT = D_BF16, OPK = O_SUM; CALL; }                 \
    else if ((OPV) == O_AVG) { constexpr int DT = D_BF16, OPK = O_AVG; CALL; }                 \
    else { constexpr int DT = D_BF16, OPK = O_MAX; CALL; }                                     \
  } while (0)

}  // namespace

std::shared_ptr<const Schedule> cached_schedule(const Spec& spec, std::string* err) {
  std::lock_guard<std::mutex> lk(g_mu);
  return schedule_locked(spec, err);
}

// The dispatch packet counts a grid's work-items in 32 bits, so one launch holds
// at most kMaxLaunchBlocks workgroups of kThreads; longer work is split into
// consecutive launches on the same stream. The limit can be lowered.
static_assert(kThreads == 256, "kMaxLaunchBlocks assumes 256-thread workgroups");
static std::atomic<int64_t> g_launch_blocks{kMaxLaunchBlocks};

int64_t launch_blocks() { return g_launch_blocks.load(std::memory_order_relaxed); }

bool set_launch_blocks(int64_t blocks, int64_t* previous) {
  if (blocks < 1 || blocks > kMaxLaunchBlocks) return false;
  const int64_t old = g_launch_blocks.exchange(blocks);
  if (previous) *previous = old;
  return true;
}

RunResult workspace_bytes(const Spec& spec, int exec, size_t* bytes) {
  std::lock_guard<std::mutex> lk(g_mu);
  Plan* pl = nullptr;
  RunResult r = get_plan(spec, plan_exec(exec), -1, &pl);
  if (r.status) return r;
  // the replays keep partials in registers or LDS; the literal steps need the slots
  *bytes = pl->kernel == K_LITERAL ? pl->ws_bytes : 0;
  return RunResult{};
}

RunResult kernel_of(const Spec& spec, int exec, int* kernel) {
  *kernel = K_NONE;
  if (spec.P <= 1 || spec.n == 0) return RunResult{};
  if (exec == E_LITERAL) { *kernel = K_LITERAL; return RunResult{}; }
  if (exec == E_FUSED && spec.algo == A_DIRECT && spec.coll == C_ALLREDUCE) { *kernel = K_DIRECT; return RunResult{}; }
  std::lock_guard<std::mutex> lk(g_mu);
  Plan* pl = nullptr;
  RunResult r = get_plan(spec, plan_exec(exec), -1, &pl);  // the launch's own choice, on a host-only plan
  if (r.status) return r;
  *kernel = pl->kernel;
  return RunResult{};
}

CacheStats cache_stats() {
  std::lock_guard<std::mutex> lk(g_mu);
  CacheStats c;
  for (const auto& kv : plan_cache()) {
    ++c.live_plans;
    c.plan_device_bytes += int64_t(kv.second->device_bytes);
  }
  for (const auto& p : retired_plans()) {
    ++c.retired_plans;
    c.plan_device_bytes += int64_t(p->device_bytes);
  }
  for (const auto& kv : ws_cache()) {
    ++c.workspaces;
    c.workspace_device_bytes += int64_t(kv.second.bytes);
  }
  for (const auto& w : retired_ws()) {
    ++c.retired_workspaces;
    c.workspace_device_bytes += int64_t(w.bytes);
  }
  return c;
}

RunResult release_cached() {
  std::lock_guard<std::mutex> lk(g_mu);
  int cur = -1;
  const bool have_cur = hipGetDevice(&cur) == hipSuccess;
  std::vector<int> devs;
  auto note = [&](int d) {
    if (d >= 0 && std::find(devs.begin(), devs.end(), d) == devs.end()) devs.push_back(d);
  };
  for (const auto& kv : plan_cache()) note(kv.second->device);
  for (const auto& p : retired_plans()) note(p->device);
  for (const auto& kv : ws_cache()) note(kv.first.first);
  RunResult res;
  // every launch that may read a table or workspace ends before it is freed
  for (int d : devs) {
    hipError_t e = hipSetDevice(d);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess && !res.status) res = hip_fail(e, "synchronizing before the release");
  }
  if (res.status) {
    if (have_cur) (void)hipSetDevice(cur);
    return res;
  }
  plan_cache().clear();
  retired_plans().clear();
  for (auto& kv : ws_cache())
    if (kv.second.p) (void)hipFree(kv.second.p);
  for (auto& w : retired_ws())
    if (w.p) (void)hipFree(w.p);
  ws_cache().clear();
  retired_ws().clear();
  sched_cache().clear();
  ++g_plan_generation;
  if (have_cur) (void)hipSetDevice(cur);
  return res;
}

// One launch per literal step (a long step is cut into launches of at most
// launch_blocks() records: a step's records are independent).
static RunResult literal_launches(const Plan& pl, int mode, const RankPtrs& ptrs, const WsDesc& wd,
                                  const LitWork* work, const LitWork* packed, hipStream_t st, const Evs& ev) {
  const Spec& spec = pl.s->spec;
  const auto& lns = pl.launches[mode];
  const int64_t cap = launch_blocks();
  hipError_t e = hipSuccess;
  for (size_t i = 0; i < lns.size(); ++i) {
    for (int64_t off = 0; off < lns[i].second; off += cap) {
      const bool last = i + 1 == lns.size() && off + cap >= lns[i].second;
      const Evs ei{i == 0 && off == 0 ? ev.start : nullptr, last ? ev.stop : nullptr};
      const int64_t cnt = std::min(cap, lns[i].second - off);
      AR_DISPATCH(spec.dtype, spec.op,
                  (e = launch_literal_t<DT, OPK>(cnt, ptrs, wd, work + lns[i].first + off, packed, st, ei)));
      if (e != hipSuccess) return hip_fail(e, "launching a literal step");
    }
  }
  return RunResult{};
}

RunResult run_allreduce(void* const* bufs, const Spec& spec, int exec, void* workspace, size_t workspace_bytes,
                        void* stream, void* start_event, void* stop_event) {
  RunResult res;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const Evs ev{reinterpret_cast<hipEvent_t>(start_event), reinterpret_cast<hipEvent_t>(stop_event)};
  auto mark_empty = [&]() -> RunResult {  // no kernel: both events mark the same point of the stream
    RunResult r;
    hipError_t e = hipSuccess;
    if (ev.start) e = hipEventRecord(ev.start, st);
    if (e == hipSuccess && ev.stop) e = hipEventRecord(ev.stop, st);
    return e == hipSuccess ? r : hip_fail(e, "recording events");
  };
  if (spec.P <= 1 || spec.n == 0) return mark_empty();  // nothing to combine
  const int V = vec_width(spec.dtype);
  bool vec = true;
  RankPtrs ptrs;
  std::memset(&ptrs, 0, sizeof(ptrs));
  for (int p = 0; p < spec.P; ++p) {
    ptrs.p[p] = bufs[p];
    if (reinterpret_cast<uintptr_t>(bufs[p]) % 16) vec = false;
  }
  ptrs.div = float(spec.P);
  const int64_t total = spec.n * spec.batch;
  if (exec == E_FUSED && spec.algo == A_DIRECT && spec.coll == C_ALLREDUCE) {
    hipError_t e = hipSuccess;
    AR_DISPATCH(spec.dtype, spec.op,
                (e = launch_direct_t<DT, OPK>(vec, ptrs, spec.P, total, launch_blocks(), st, ev)));
    if (e != hipSuccess) return hip_fail(e, "launching the direct kernel");
    return res;
  }
  // Latency-bound calls (at most kTinyElements elements) replay one element per
  // thread: a thread's register stack then holds one value per entry instead
  // of a vector's, and its serial chain of moves and combinations is 4-8x
  // shorter (24 ranks x 106 fp32, recursive doubling: 8.3 -> 7.1 us per call).
  if (total <= kTinyElements) vec = false;
  Plan* pl = nullptr;
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  // building device tables (first call of a schedule, size and alignment) or a
  // workspace allocates and copies synchronously, which a stream capture cannot hold
  auto capturing = [&]() {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(st, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone;
  };
  auto refuse_capture = [&](const char* what) {
    RunResult r;
    r.status = 2;  // AR_UNSUPPORTED
    r.message = std::string(what) + " cannot be built while the stream is capturing: make one call with this "
                "schedule, size and buffer alignment before the capture";
    return r;
  };
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    res = get_plan(spec, plan_exec(exec), device, &pl);
    if (res.status) return res;
    if (pl->kernel == K_LITERAL && pl->exec != E_LITERAL) {
      // no replay holds the program: the step-by-step kernels compute the same bits
      res = get_plan(spec, E_LITERAL, device, &pl);
      if (res.status) return res;
    }
    const int mode = vec ? 0 : 1;
    if (!pl->built[mode]) {
      if (capturing()) return refuse_capture("the call's device tables");
      g_upload_bytes = &pl->device_bytes;
      res = build_items(*pl, vec);
      g_upload_bytes = nullptr;
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
        Workspace& w = ws_cache()[{device, reinterpret_cast<uintptr_t>(st)}];
        if (w.bytes < pl->ws_bytes) {
          if (capturing()) return refuse_capture("the literal workspace");
          void* p = nullptr;
          e = hipMalloc(&p, pl->ws_bytes);
          if (e != hipSuccess) return hip_fail(e, "allocating the literal workspace");
          if (w.p) retired_ws().push_back(w);  // earlier launches on this stream may still use it
          w.p = p;
          w.bytes = pl->ws_bytes;
        }
        ws = w.p;
      }
    }
  }
  const int mode = vec ? 0 : 1;
  if (pl->exec == E_LITERAL) {
    WsDesc wd{reinterpret_cast<char*>(ws), pl->slot_bytes, spec.P};
    const LitWork* work = reinterpret_cast<const LitWork*>(pl->items[mode].p);
    const LitWork* packed = reinterpret_cast<const LitWork*>(pl->packed[mode].p);
    if (pl->launches[mode].empty()) return mark_empty();
    return literal_launches(*pl, mode, ptrs, wd, work, packed, st, ev);
  } else {
    if (pl->nitems[mode] == 0) return mark_empty();
    const Item* items = reinterpret_cast<const Item*>(pl->items[mode].p);
    const int32_t* prog = reinterpret_cast<const int32_t*>(pl->prog.p);
    // strided items of one block of instances share cache lines: keeping
    // neighbouring items on one XCD keeps those lines in one L2
    ptrs.xcd = pl->strided || pl->s->prog.size() * sizeof(int32_t) > kXcdProgramBytes ? 1 : 0;
    const int64_t nit = pl->nitems[mode], cap = launch_blocks();
    const int TM = pl->s->max_trees > 1 ? kMaxFusedTrees : 1;
    if (pl->dag) {
      // few workgroups (a latency-bound call): 16 waves each share the levels' combinations
      const int64_t total = spec.n * spec.batch;
      const int64_t blocks = pl->dag_shared ? (total + kDagLanes - 1) / kDagLanes : nit;
      const int threads = blocks <= 512 ? 1024 : 256;
      const Item* ditems = pl->dag_shared ? nullptr : items;
      AR_DISPATCH(spec.dtype, spec.op,
                  (e = launch_fused_dag_t<DT, OPK>(pl->dag_shared, threads, pl->dag_lds[mode], nit, ptrs, ditems, prog,
                                                   reinterpret_cast<const uint8_t*>(pl->dtab.p), total, int(spec.n),
                                                   spec.P, pl->dag_vals[mode], int(pl->s->ranges.size()), cap, st,
                                                   ev)));
      if (e != hipSuccess) return hip_fail(e, "launching the DAG replay");
      return res;
    }
    if (pl->rows) {
      // whole vectors in k_fused_rows_vec where it applies, the rest (or all)
      // in k_fused_rows; each launcher splits its launch by the block limit
      const int64_t total = spec.n * spec.batch;
      const int32_t* ref = prog + pl->s->ranges[size_t(pl->rows_ref)].prog;
      const uint8_t* rt = reinterpret_cast<const uint8_t*>(pl->rtab.p);
      const int R = int(pl->s->ranges.size());
      const int64_t nvec = vec && rows_vec(*pl->s, pl->rows_ref) ? total / 4 : 0;
      if (nvec > 0) {
        const Evs ev1{ev.start, nvec * 4 == total ? ev.stop : nullptr};
        // a stack of 6 for trees that need 5 or 6 (each push shifts the whole
        // stack; measured 5% faster than 8 on 24-rank trees of three results)
        const int dv = pl->D == 8 && pl->s->max_need <= 6 ? 6 : pl->D;
        AR_DISPATCH(spec.dtype, spec.op,
                    (e = launch_fused_rows_vec_t<DT, OPK>(dv, pl->rows_chain, ptrs, ref, rt, nvec, int(pl->rows_n), R,
                                                          spec.P, cap, st, ev1)));
        if (e != hipSuccess) return hip_fail(e, "launching the fused replay");
      }
      if (nvec * 4 < total) {
        const int iters = int(std::clamp<int64_t>(total / (int64_t(kThreads) * 16384), 1, 8));
        const Evs ev2{nvec > 0 ? nullptr : ev.start, ev.stop};
        AR_DISPATCH(spec.dtype, spec.op,
                    (e = launch_fused_rows_t<DT, OPK>(pl->D, TM, ptrs, ref, rt, nvec * 4, total, int(pl->rows_n), R,
                                                      spec.P, iters, cap, st, ev2)));
        if (e != hipSuccess) return hip_fail(e, "launching the fused replay");
      }
      return res;
    }
    if (pl->kernel == K_JIT && !pl->jit.k.fn) {
      std::string err;
      if (!jit_load(pl->jit_code, &pl->jit.k, &err)) {
        RunResult r;
        r.status = 4;  // AR_HIP_ERROR
        r.message = "loading the compiled replay: " + err;
        return r;
      }
    }
    const int64_t per = pl->jit_table ? 4 : 1;  // work items per workgroup
    for (int64_t off = 0; off < nit; off += cap * per) {  // work items are independent
      const Evs ei{off == 0 ? ev.start : nullptr, off + cap * per >= nit ? ev.stop : nullptr};
      const int64_t cnt = std::min(cap * per, nit - off) / per;
      if (pl->kernel == K_JIT && pl->jit_table) {
        JitTabArgs ja;
        std::memset(&ja, 0, sizeof(ja));
        for (int q = 0; q < spec.P; ++q) ja.p[q] = ptrs.p[q];
        ja.items = items + off;
        ja.tab = pl->jtab.p;
        ja.div = ptrs.div;
        ja.w = pl->jit_w;
        void* params[] = {&ja};
        e = hipExtModuleLaunchKernel(static_cast<hipFunction_t>(pl->jit.k.fn), uint32_t(cnt * kThreads), 1, 1,
                                     kThreads, 1, 1, 0, st, params, nullptr, ei.start, ei.stop, 0);
      } else if (pl->kernel == K_JIT) {
        JitArgs ja;
        std::memset(&ja, 0, sizeof(ja));
        for (int q = 0; q < spec.P; ++q) ja.p[q] = ptrs.p[q];
        ja.items = items + off;
        ja.div = ptrs.div;
        void* params[] = {&ja};
        e = hipExtModuleLaunchKernel(static_cast<hipFunction_t>(pl->jit.k.fn), uint32_t(cnt * kThreads), 1, 1,
                                     kThreads, 1, 1, 0, st, params, nullptr, ei.start, ei.stop, 0);
      } else if (pl->strided) {
        const SItem* sit = reinterpret_cast<const SItem*>(pl->items[mode].p) + off;
        AR_DISPATCH(spec.dtype, spec.op,
                    (e = launch_fused_strided_t<DT, OPK>(pl->D, TM, cnt, ptrs, sit, prog, spec.n, st, ei)));
      } else if (pl->multi) {
        MultiPtrs mp;
        std::memset(&mp, 0, sizeof(mp));
        for (int q = 0; q < spec.P; ++q) mp.p[q] = ptrs.p[q];
        mp.div = ptrs.div;
        mp.xcd = ptrs.xcd;
        AR_DISPATCH(spec.dtype, spec.op,
                    (e = launch_fused_multi_t<DT, OPK>(pl->multi, cnt, mp, items + off,
                                                       reinterpret_cast<const int32_t*>(pl->mtab.p), st, ei)));
      } else if (pl->shape != SH_NONE) {
        AR_DISPATCH(spec.dtype, spec.op,
                    (e = launch_fused_fixed_t<DT, OPK>(pl->shape, pl->shape_nl, pl->md, cnt, ptrs, items + off,
                                                       pl->tab, st, ei)));
      } else if (pl->ordered) {
        RankPtrs op = ptrs;  // leaf buffers in postfix order, then the output buffers
        for (size_t q = 0; q < pl->ordered_ranks.size(); ++q) op.p[q] = ptrs.p[pl->ordered_ranks[q]];
        const int dv = pl->D == 8 && pl->s->max_need <= 6 ? 6 : pl->D;  // a stack of 6 where it suffices
        AR_DISPATCH(spec.dtype, spec.op,
                    (e = launch_fused_t<DT, OPK>(dv, TM, spec.P, pl->s->max_leaves, cnt, op, items + off, prog, st,
                                                 ei, true)));
      } else {
        AR_DISPATCH(spec.dtype, spec.op,
                    (e = launch_fused_t<DT, OPK>(pl->D, TM, spec.P, pl->s->max_leaves, cnt, ptrs, items + off, prog,
                                                 st, ei)));
      }
      if (e != hipSuccess) return hip_fail(e, "launching the fused replay");
    }
  }
  (void)V;
  return res;
}

// ----------------------------------------------------------------------------
// allocation-free literal execution
// ----------------------------------------------------------------------------
// Device memory the allocation-free entry point uses in place of allocations:
// one call's literal work records and its workspace slots. Every device holds
// its own copy of the array from the library's load until the process ends;
// host code reaches it only through the address hipGetSymbolAddress returns on
// that device (the array's name is not a device address in host code).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::map<int, char*>& scratch_ptrs() {
  static std::map<int, char*> m;
  return m;
}
}  // namespace

RunResult run_noalloc(void* const* bufs, const Spec& spec, void* stream, void* start_event, void* stop_event) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const Evs ev{reinterpret_cast<hipEvent_t>(start_event), reinterpret_cast<hipEvent_t>(stop_event)};
  auto mark_empty = [&]() -> RunResult {
    hipError_t e = hipSuccess;
    if (ev.start) e = hipEventRecord(ev.start, st);
    if (e == hipSuccess && ev.stop) e = hipEventRecord(ev.stop, st);
    return e == hipSuccess ? RunResult{} : hip_fail(e, "recording events");
  };
  if (spec.P <= 1 || spec.n == 0) return mark_empty();
  RankPtrs ptrs;
  std::memset(&ptrs, 0, sizeof(ptrs));
  bool vec = true;
  for (int p = 0; p < spec.P; ++p) {
    ptrs.p[p] = bufs[p];
    if (reinterpret_cast<uintptr_t>(bufs[p]) % 16) vec = false;
  }
  ptrs.div = float(spec.P);
  const int mode = vec ? 0 : 1;
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  Plan* pl = nullptr;
  char* base = nullptr;
  size_t off_packed = 0, off_ws = 0;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    // the device's copy of the array: its address, taken once with the device current
    auto it = scratch_ptrs().find(device);
    if (it == scratch_ptrs().end()) {
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress");
      it = scratch_ptrs().emplace(device, static_cast<char*>(p)).first;
    }
    base = it->second;
    // a plan's host tables only: no device tables, no workspace allocation
    RunResult res = get_plan(spec, E_LITERAL, device, &pl);
    if (res.status) return res;
    if (!pl->host_built[mode]) {
      res = literal_tables(*pl, vec);
      if (res.status) return res;
    }
    const size_t wb = pl->lit_work[mode].size() * sizeof(LitWork);
    const size_t pb = pl->lit_packed[mode].size() * sizeof(LitWork);
    off_packed = (wb + 255) / 256 * 256;
    off_ws = off_packed + (pb + 255) / 256 * 256;
    const size_t need = off_ws + pl->ws_bytes;
    if (need > kScratchBytes) {
      RunResult r;
      r.status = 2;  // AR_UNSUPPORTED
      r.message = "the call needs " + std::to_string(need) + " bytes of device scratch (work records and workspace "
                  "slots); the allocation-free entry point holds at most " + std::to_string(kScratchBytes);
      return r;
    }
  }
  if (pl->launches[mode].empty()) return mark_empty();
  // this call's records, ordered on the stream before its launches (the array
  // keeps whatever the previous call on this device left; every workspace slot
  // element is written by a step before any step reads it)
  const auto& work = pl->lit_work[mode];
  const auto& packed = pl->lit_packed[mode];
  e = hipMemcpyAsync(base, work.data(), work.size() * sizeof(LitWork), hipMemcpyHostToDevice, st);
  if (e == hipSuccess && !packed.empty())
    e = hipMemcpyAsync(base + off_packed, packed.data(), packed.size() * sizeof(LitWork), hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return hip_fail(e, "copying the work records to the scratch array");
  WsDesc wd{base + off_ws, pl->slot_bytes, spec.P};
  return literal_launches(*pl, mode, ptrs, wd, reinterpret_cast<const LitWork*>(base),
                          reinterpret_cast<const LitWork*>(base + off_packed), st, ev);
}

}  // namespace ar

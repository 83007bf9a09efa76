// Register DAG kernels compiled at run time (jit.h).
#include "jit.h"

#include <dlfcn.h>
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <sstream>

namespace ar {
namespace {

// Device code shared by every generated kernel. AR_DT / AR_OP select the
// element type and operation (the values of Dtype and Op). A thread takes one
// element (element items: ragged range edges, unaligned buffers) or AR_M (one
// or two) 16-byte vectors 256 vectors apart (vector items of up to 256 AR_M
// vectors), and a fragment Fr<F> holds its F values in the accumulation type:
// fp32 for fp32 and bf16 (widened exactly), 32-bit two's complement for int32.
const char* kPrelude = R"(
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
struct Item { long long start; int count; int tag; };
#if AR_DT == 0
typedef unsigned A;
#define AR_V 4
#elif AR_DT == 1
typedef float A;
#define AR_V 4
#else
typedef float A;
#define AR_V 8
#endif
template <int F> struct Fr { A v[F]; };
__device__ __forceinline__ A cmb(A a, A b) {
#if AR_OP == 1
#if AR_DT == 0
  return (int)b > (int)a ? b : a;
#else
  return __builtin_elementwise_maximum(a, b);  // -0 < +0 on non-NaN values
#endif
#else
  return a + b;
#endif
}
template <int F> __device__ __forceinline__ Fr<F> add(const Fr<F>& x, const Fr<F>& y) {
  Fr<F> r;
#pragma unroll
  for (int i = 0; i < F; ++i) r.v[i] = cmb(x.v[i], y.v[i]);
  return r;
}
__device__ __forceinline__ A fin(A x, float div) {
#if AR_OP == 2
  return x / div;
#else
  return x;
#endif
}
__device__ __forceinline__ unsigned bits(A x) { return __builtin_bit_cast(unsigned, x); }
__device__ __forceinline__ A val(unsigned u) { return __builtin_bit_cast(A, u); }
// fp32 -> bf16 bits, nearest even (finite values)
__device__ __forceinline__ unsigned to_bf16(A x) {
  const unsigned u = bits(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
// one 16-byte vector at element e into v[o .. o + AR_V)
template <int F> __device__ __forceinline__ void ldv(const void* base, long long e, Fr<F>& f, int o) {
#if AR_DT == 2
  const u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const unsigned short*>(base) + e));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f.v[o + 2 * i] = val(r[i] << 16);
    f.v[o + 2 * i + 1] = val(r[i] & 0xffff0000u);
  }
#else
  const u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(static_cast<const unsigned*>(base) + e));
#pragma unroll
  for (int i = 0; i < 4; ++i) f.v[o + i] = val(r[i]);
#endif
}
template <int F> __device__ __forceinline__ void stv(void* base, long long e, const Fr<F>& f, int o, float div) {
  u32x4 r;
#if AR_DT == 2
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = to_bf16(fin(f.v[o + 2 * i], div)) | (to_bf16(fin(f.v[o + 2 * i + 1], div)) << 16);
  __builtin_nontemporal_store(r, reinterpret_cast<u32x4*>(static_cast<unsigned short*>(base) + e));
#else
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = bits(fin(f.v[o + i], div));
  __builtin_nontemporal_store(r, reinterpret_cast<u32x4*>(static_cast<unsigned*>(base) + e));
#endif
}
__device__ __forceinline__ A ld1(const void* base, long long e) {
#if AR_DT == 2
  return val(unsigned(__builtin_nontemporal_load(static_cast<const unsigned short*>(base) + e)) << 16);
#else
  return val(__builtin_nontemporal_load(static_cast<const unsigned*>(base) + e));
#endif
}
__device__ __forceinline__ void st1(void* base, long long e, A x, float div) {
#if AR_DT == 2
  __builtin_nontemporal_store((unsigned short)to_bf16(fin(x, div)), static_cast<unsigned short*>(base) + e);
#else
  __builtin_nontemporal_store(bits(fin(x, div)), static_cast<unsigned*>(base) + e);
#endif
}
)";

// The kernel body: one work item per workgroup of 256 threads; the range's
// function is picked by the item's tag (uniform).
const char* kKernelHead = R"(
struct Args { void* p[32]; const Item* items; float div; int pad; };
extern "C" __global__ __launch_bounds__(256) void ar_jit(Args a) {
  const Item it = a.items[blockIdx.x];
  if (it.count > 0) {
    // up to AR_M vectors per thread, 256 vectors apart
    const int vb = threadIdx.x;
    if (vb >= it.count) return;
    const bool two = AR_M == 2 && vb + 256 < it.count;
    const long long e0 = it.start + (long long)vb * AR_V, e1 = e0 + 256LL * AR_V;
    auto ld = [&](int rank) {
      Fr<AR_M * AR_V> f;
      ldv(a.p[rank], e0, f, 0);
      if (two) ldv(a.p[rank], e1, f, AR_V);
      return f;
    };
    auto st = [&](int rank, const Fr<AR_M * AR_V>& f) {
      stv(a.p[rank], e0, f, 0, a.div);
      if (two) stv(a.p[rank], e1, f, AR_V, a.div);
    };
    switch (it.tag) {
)";

const char* kKernelMid = R"(
    }
  } else {
    for (int v = threadIdx.x; v < -it.count; v += 256) {
      const long long e = it.start + v;
      auto ld = [&](int rank) { Fr<1> f; f.v[0] = ld1(a.p[rank], e); return f; };
      auto st = [&](int rank, const Fr<1>& f) { st1(a.p[rank], e, f.v[0], a.div); };
      switch (it.tag) {
)";

const char* kKernelTail = R"(
      }
    }
  }
}
)";

// Device code of the table form: raw 16-byte vectors (or single elements) as
// loaded, widened where a leaf is pushed; T points at the item's range row of
// the rank table (leaves, then outputs), read through the constant address
// space so that its words are scalar loads even after the kernel's stores.
const char* kTabPrelude = R"(
struct TArgs { void* p[256]; const Item* items; const int* tab; float div; int w; };
typedef const __attribute__((address_space(4))) int* CI;
template <int F> struct Raw { u32x4 q[F / AR_V]; };
template <> struct Raw<1> { unsigned u; };
template <int F> __device__ __forceinline__ Fr<F> wid(const Raw<F>& r) {
  Fr<F> f;
#pragma unroll
  for (int j = 0; j < F / AR_V; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#if AR_DT == 2
      f.v[j * 8 + 2 * i] = val(r.q[j][i] << 16);
      f.v[j * 8 + 2 * i + 1] = val(r.q[j][i] & 0xffff0000u);
#else
      f.v[j * 4 + i] = val(r.q[j][i]);
#endif
    }
  return f;
}
__device__ __forceinline__ Fr<1> wid(const Raw<1>& r) {
  Fr<1> f;
#if AR_DT == 2
  f.v[0] = val(r.u << 16);
#else
  f.v[0] = val(r.u);
#endif
  return f;
}
// Loads and stores at a byte offset (32 bits) from a base the work item has
// advanced to its first element (a scalar): the instructions then take the base
// in scalar registers and one offset register for every leaf.
#if AR_DT == 2
typedef unsigned short S;
#else
typedef unsigned S;
#endif
__device__ __forceinline__ u32x4 ldq(const char* base, unsigned off) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + off));
}
__device__ __forceinline__ unsigned ldu(const char* base, unsigned off) {
  return __builtin_nontemporal_load(reinterpret_cast<const S*>(base + off));
}
template <int F> __device__ __forceinline__ void stq(char* base, unsigned off, const Fr<F>& f, int o, float div) {
  u32x4 r;
#if AR_DT == 2
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = to_bf16(fin(f.v[o + 2 * i], div)) | (to_bf16(fin(f.v[o + 2 * i + 1], div)) << 16);
#else
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = bits(fin(f.v[o + i], div));
#endif
  __builtin_nontemporal_store(r, reinterpret_cast<u32x4*>(base + off));
}
__device__ __forceinline__ void stu(char* base, unsigned off, A x, float div) {
#if AR_DT == 2
  __builtin_nontemporal_store((S)to_bf16(fin(x, div)), reinterpret_cast<S*>(base + off));
#else
  __builtin_nontemporal_store(bits(fin(x, div)), reinterpret_cast<S*>(base + off));
#endif
}
// a vector partly inside the range (its element indices [lo, hi) relative to
// the item's first element): its elements inside, one at a time
template <int F>
__device__ __forceinline__ void stq_part(char* base, int e, const Fr<F>& f, int o, float div, int lo, int hi) {
#pragma unroll
  for (int i = 0; i < AR_V; ++i)
    if (e + i >= lo && e + i < hi) stu(base, unsigned(e + i) * sizeof(S), f.v[o + i], div);
}
#define SB __builtin_amdgcn_sched_barrier(0)
)";

// The table-form kernel: one work item per wave, four per workgroup; a vector
// item's count holds its vectors in bits 0..15 and, at a range's ends, the
// elements before the range (bits 16..23) and past it (bits 24..27), which are
// loaded with their vector but not stored; element items take one element per
// lane.
const char* kTabKernel = R"(
extern "C" __global__ __launch_bounds__(256) void ar_jit(TArgs a) {
  // TArgs is the only argument: its rank pointers are read in place, from the
  // kernel argument segment, so that indexing them by a table value needs no
  // private copy of the argument
  typedef char* Ptr;
  typedef const __attribute__((address_space(4))) Ptr* CP;
  typedef const __attribute__((address_space(4))) Item* CIt;
  const CP P = (CP)__builtin_amdgcn_kernarg_segment_ptr();
  // one work item per wave, four per workgroup (the wave index made scalar:
  // items and table rows are then scalar loads)
  const int lane = threadIdx.x & 63;
  const Item it = ((CIt)a.items)[blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)];
  const float div = a.div;
  const long long base = it.start * (long long)sizeof(S);  // the item's first element, in bytes
  if (it.count > 0) {
    const CI T = (CI)a.tab + (long long)it.tag * a.w;
    const int nv = it.count & 0xffff;
    if (lane >= nv) return;
    const bool two = AR_M == 2 && lane + 64 < nv;
    const unsigned o0 = unsigned(lane) * 16u, o1 = two ? o0 + 1024u : o0;
    auto ld = [&](int k) {
      const char* b = P[T[k]] + base;
      Raw<AR_M * AR_V> r;
      r.q[0] = ldq(b, o0);
      if (AR_M == 2) r.q[AR_M - 1] = ldq(b, o1);
      return r;
    };
    const Fr<AR_M * AR_V> x = shape<AR_M * AR_V>(ld);
    // whole vectors inside the range are stored whole; a vector across one of
    // its ends, element by element (only the items at a range's ends hold one)
    const int lo = (it.count >> 16) & 0xff, hi = nv * AR_V - ((it.count >> 24) & 0xf);
    const int e0 = lane * AR_V, e1 = e0 + 64 * AR_V;
    const bool w0 = e0 >= lo && e0 + AR_V <= hi, w1 = e1 >= lo && e1 + AR_V <= hi;
    const bool p0 = !w0 && e0 < hi && e0 + AR_V > lo, p1 = two && !w1 && e1 < hi && e1 + AR_V > lo;
#pragma unroll 8
    for (int j = 0; j < AR_NO; ++j) {
      char* b = P[T[AR_NL + j]] + base;
      if (w0) stq(b, o0, x, 0, div);
      else if (p0) stq_part(b, e0, x, 0, div, lo, hi);
      if (two) {
        if (w1) stq(b, o1, x, AR_V, div);
        else if (p1) stq_part(b, e1, x, AR_V, div, lo, hi);
      }
    }
  } else if (lane < -it.count) {
    // element items (at most 64 elements): one element per lane. Their table
    // row is read through an offset the compiler cannot equate with the vector
    // path's, so that it does not merge the two paths' table reads and hoist
    // all of them above the branch.
    const CI Te = (CI)a.tab + __builtin_amdgcn_readfirstlane(it.tag * a.w);
    const unsigned o = unsigned(lane) * sizeof(S);
    auto ld = [&](int k) { Raw<1> r; r.u = ldu(P[Te[k]] + base, o); return r; };
    const Fr<1> x = shape<1>(ld);
#pragma unroll 8
    for (int j = 0; j < AR_NO; ++j) stu(P[Te[AR_NL + j]] + base, o, x.v[0], div);
  }
}
)";

// Most values of one range's straight-line code live at once: every leaf from
// the start to its last read, every combination from its instruction to its
// last read (outputs are read at the end).
int max_live(const DagProgram& d) {
  const int nl = int(d.leaves.size()), ni = int(d.instr.size()), end = ni;
  std::vector<int> slot_val(size_t(d.S), -1), last(size_t(nl + ni), -1);
  for (int k = 0; k < nl; ++k) slot_val[size_t(k)] = k;
  for (int i = 0; i < ni; ++i) {
    const uint32_t w = d.instr[size_t(i)];
    const int a = slot_val[(w >> 10) & 1023u], b = slot_val[(w >> 20) & 1023u];
    if (a >= 0) last[size_t(a)] = i;
    if (b >= 0) last[size_t(b)] = i;
    slot_val[w & 1023u] = nl + i;
  }
  for (int32_t w : d.outs) {
    const int v = slot_val[uint32_t(w) >> 16];
    if (v >= 0) last[size_t(v)] = end;
  }
  int live = nl, most = nl;  // all leaves are loaded first
  for (int i = 0; i < ni; ++i) {
    ++live;  // the combination's value
    most = std::max(most, live);
    for (int v = 0; v < nl + i; ++v)
      if (last[size_t(v)] == i) --live;
  }
  return most;
}

// One range's DAG as straight-line code over fragments: leaves loaded once,
// each combination a new value named after its instruction, outputs stored.
bool range_function(const DagProgram& d, int r, std::ostringstream& o, std::string* why) {
  const int nl = int(d.leaves.size());
  if (int(d.instr.size()) > kJitMaxNodes) {
    *why = "range " + std::to_string(r) + " has " + std::to_string(d.instr.size()) + " distinct combinations";
    return false;
  }
  o << "template <int F, typename LD, typename ST> __device__ __forceinline__ void range" << r
    << "(LD& ld, ST& st) {\n";
  std::vector<std::string> cur(size_t(d.S));
  for (int k = 0; k < nl; ++k) {
    o << "  const Fr<F> x" << k << " = ld(" << d.leaves[size_t(k)] << ");\n";
    cur[size_t(k)] = "x" + std::to_string(k);
  }
  for (size_t i = 0; i < d.instr.size(); ++i) {
    const uint32_t w = d.instr[i];
    const uint32_t dst = w & 1023u, a = (w >> 10) & 1023u, b = (w >> 20) & 1023u;
    if (cur[a].empty() || cur[b].empty()) {
      *why = "range " + std::to_string(r) + ": an instruction reads an empty slot";
      return false;
    }
    o << "  const Fr<F> n" << i << " = add(" << cur[a] << ", " << cur[b] << ");\n";
    cur[dst] = "n" + std::to_string(i);
  }
  for (int32_t w : d.outs) {
    const uint32_t slot = uint32_t(w) >> 16;
    if (cur[slot].empty()) {
      *why = "range " + std::to_string(r) + ": an output reads an empty slot";
      return false;
    }
    o << "  st(" << (w & 0xffff) << ", " << cur[slot] << ");\n";
  }
  o << "}\n";
  return true;
}

// hipRTC entry points, resolved at run time.
struct Rtc {
  void* h = nullptr;
  int (*create)(void**, const char*, const char*, int, const char**, const char**) = nullptr;
  int (*compile)(void*, int, const char**) = nullptr;
  int (*log_size)(void*, size_t*) = nullptr;
  int (*log)(void*, char*) = nullptr;
  int (*code_size)(void*, size_t*) = nullptr;
  int (*code)(void*, char*) = nullptr;
  int (*destroy)(void**) = nullptr;
  std::string why;
};

Rtc* rtc() {
  static Rtc r;
  static std::once_flag once;
  std::call_once(once, [] {
    // the hipRTC beside the HIP runtime that is in use, else ROCm's
    std::vector<std::string> paths;
    Dl_info info;
    if (dladdr(reinterpret_cast<void*>(&hipGetDevice), &info) && info.dli_fname) {
      std::string f(info.dli_fname);
      const size_t sl = f.rfind('/');
      if (sl != std::string::npos) paths.push_back(f.substr(0, sl + 1) + "libhiprtc.so");
    }
    paths.push_back("libhiprtc.so.7");
    paths.push_back("/opt/rocm/lib/libhiprtc.so.7");
    for (const std::string& p : paths) {
      r.h = dlopen(p.c_str(), RTLD_NOW | RTLD_LOCAL);
      if (r.h) break;
    }
    if (!r.h) {
      r.why = "hipRTC not found";
      return;
    }
    auto sym = [&](const char* n) { return dlsym(r.h, n); };
    r.create = reinterpret_cast<decltype(r.create)>(sym("hiprtcCreateProgram"));
    r.compile = reinterpret_cast<decltype(r.compile)>(sym("hiprtcCompileProgram"));
    r.log_size = reinterpret_cast<decltype(r.log_size)>(sym("hiprtcGetProgramLogSize"));
    r.log = reinterpret_cast<decltype(r.log)>(sym("hiprtcGetProgramLog"));
    r.code_size = reinterpret_cast<decltype(r.code_size)>(sym("hiprtcGetCodeSize"));
    r.code = reinterpret_cast<decltype(r.code)>(sym("hiprtcGetCode"));
    r.destroy = reinterpret_cast<decltype(r.destroy)>(sym("hiprtcDestroyProgram"));
    if (!r.create || !r.compile || !r.log_size || !r.log || !r.code_size || !r.code || !r.destroy) {
      r.why = "hipRTC lacks an entry point";
      r.h = nullptr;
    }
  });
  return &r;
}

}  // namespace

bool jit_available(std::string* why) {
  Rtc* r = rtc();
  if (!r->h && why) *why = r->why;
  return r->h != nullptr;
}

bool jit_source(const Schedule& s, int dtype, int op, int max_vectors, std::string* src, int* vectors,
                std::string* why) {
  const Spec& sp = s.spec;
  if (sp.P > kJitMaxRanks) {
    *why = "more than " + std::to_string(kJitMaxRanks) + " ranks";
    return false;
  }
  if (int(s.ranges.size()) > kJitMaxRanges) {
    *why = "more than " + std::to_string(kJitMaxRanges) + " ranges";
    return false;
  }
  std::vector<DagProgram> progs(s.ranges.size());
  int live = 0;
  for (size_t r = 0; r < s.ranges.size(); ++r) {
    std::string err;
    if (!compile_dag(s.prog.data() + s.ranges[r].prog, sp.P, &progs[r], &err)) {
      *why = "range " + std::to_string(r) + ": " + err;
      return false;
    }
    live = std::max(live, max_live(progs[r]));
  }
  // two vectors per thread where the live values fit the register budget
  // (measured 23% faster than one on 7 x 2^24 fp32), else one
  const int per_vector = dtype == D_BF16 ? 8 : 4;
  *vectors = max_vectors >= 2 && live * 2 * per_vector <= kJitRegisterBudget ? 2
             : live * per_vector <= kJitRegisterBudget                       ? 1
                                                                             : 0;
  if (!*vectors) {
    *why = std::to_string(live) + " values live at once exceed the register budget";
    return false;
  }
  std::ostringstream o;
  o << "#define AR_DT " << dtype << "\n#define AR_OP " << op << "\n#define AR_M " << *vectors << "\n" << kPrelude;
  for (size_t r = 0; r < s.ranges.size(); ++r)
    if (!range_function(progs[r], int(r), o, why)) return false;
  o << kKernelHead;
  for (size_t r = 0; r < s.ranges.size(); ++r)
    o << "      case " << r << ": range" << r << "<AR_M * AR_V>(ld, st); break;\n";
  o << kKernelMid;
  for (size_t r = 0; r < s.ranges.size(); ++r) o << "        case " << r << ": range" << r << "<1>(ld, st); break;\n";
  o << kKernelTail;
  *src = o.str();
  return true;
}

bool jit_table_source(const Schedule& s, int dtype, int op, int max_vectors, std::string* src, std::vector<int32_t>* tab,
                      int* w, int* vectors, std::string* why) {
  const Spec& sp = s.spec;
  if (sp.P > kJitTabRanks) {
    *why = "more than " + std::to_string(kJitTabRanks) + " ranks";
    return false;
  }
  if (s.max_trees != 1 || s.ranges.empty()) {
    *why = "not one result tree per range";
    return false;
  }
  // the shape of the first range; every other range must repeat it
  const int32_t* w0 = s.prog.data() + s.ranges[0].prog;
  const int nl = w0[1], no = w0[2];
  if (w0[0] != 1 || nl < 1 || no < 1 || nl > 1024) {
    *why = "a tree of " + std::to_string(nl) + " leaves";
    return false;
  }
  const int32_t* nc0 = w0 + 3 + nl;
  *w = nl + no;
  tab->assign(s.ranges.size() * size_t(*w), 0);
  for (size_t r = 0; r < s.ranges.size(); ++r) {
    const int32_t* x = s.prog.data() + s.ranges[r].prog;
    if (x[0] != 1 || x[1] != nl || x[2] != no || !std::equal(nc0, nc0 + nl, x + 3 + nl)) {
      *why = "range " + std::to_string(r) + " has another tree shape than range 0";
      return false;
    }
    int32_t* row = tab->data() + r * size_t(*w);
    std::copy(x + 3, x + 3 + nl, row);                   // leaf ranks, postfix order
    std::copy(x + 3 + 2 * nl, x + 3 + 2 * nl + no, row + nl);  // output ranks
  }
  // the postfix program on a stack of value names: every combination pops two
  std::ostringstream body;
  std::vector<std::string> stk;
  int most = 0, ci = 0;
  const int batch = kJitTableBatch, ahead = 1;
  const int nb = (nl + batch - 1) / batch;
  auto loads = [&](int b) {
    for (int k = b * batch; k < std::min(nl, (b + 1) * batch); ++k)
      body << "  const Raw<F> r" << k << " = ld(" << k << ");\n";
  };
  for (int b = 0; b <= ahead && b < nb; ++b) loads(b);
  for (int b = 0; b < nb; ++b) {
    body << "  SB;\n";
    for (int k = b * batch; k < std::min(nl, (b + 1) * batch); ++k) {
      body << "  const Fr<F> w" << k << " = wid(r" << k << ");\n";
      stk.push_back("w" + std::to_string(k));
      most = std::max(most, int(stk.size()));
      for (int c = 0; c < nc0[k]; ++c) {
        if (stk.size() < 2) {
          *why = "a combination with fewer than two values on the stack";
          return false;
        }
        const std::string right = stk.back();
        stk.pop_back();
        const std::string left = stk.back();
        stk.pop_back();
        body << "  const Fr<F> c" << ci << " = add(" << left << ", " << right << ");\n";
        stk.push_back("c" + std::to_string(ci++));
      }
    }
    if (b + ahead + 1 < nb) {
      body << "  SB;\n";
      loads(b + ahead + 1);
    }
  }
  if (stk.size() != 1) {
    *why = "the tree leaves " + std::to_string(stk.size()) + " values";
    return false;
  }
  body << "  SB;\n  return " << stk.back() << ";\n";
  // registers per thread: raw vectors in flight, values on the stack; two
  // vectors per lane where they fit
  const int per_vector = dtype == D_BF16 ? 8 : 4;
  auto regs = [&](int v) { return (ahead + 1) * batch * v * 4 + most * v * per_vector; };
  *vectors = max_vectors >= 2 && regs(2) <= kJitTableRegisters ? 2 : regs(1) <= kJitTableRegisters ? 1 : 0;
  if (!*vectors) {
    *why = std::to_string(regs(1)) + " registers per thread for loads in flight and stack values";
    return false;
  }
  std::ostringstream o;
  o << "#define AR_DT " << dtype << "\n#define AR_OP " << op << "\n#define AR_M " << *vectors << "\n#define AR_NL "
    << nl << "\n#define AR_NO " << no << "\n"
    << kPrelude << kTabPrelude
    << "template <int F, typename LD> __device__ __forceinline__ Fr<F> shape(LD& ld) {\n"
    << body.str() << "}\n"
    << kTabKernel;
  *src = o.str();
  return true;
}

bool jit_compile(const std::string& src, std::vector<char>* code, std::string* err) {
  Rtc* r = rtc();
  if (!r->h) {
    *err = r->why;
    return false;
  }
  if (const char* dir = std::getenv("AR_JIT_SOURCE")) {  // a directory: keep each compiled source there
    static int seq = 0;
    const std::string path = std::string(dir) + "/ar_jit_" + std::to_string(seq++) + ".hip";
    if (FILE* f = std::fopen(path.c_str(), "w")) {
      std::fwrite(src.data(), 1, src.size(), f);
      std::fclose(f);
    }
  }
  void* prog = nullptr;
  if (r->create(&prog, src.c_str(), "ar_jit.hip", 0, nullptr, nullptr) != 0) {
    *err = "hiprtcCreateProgram failed";
    return false;
  }
  const char* opts[] = {"--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
                        "-fno-gpu-flush-denormals-to-zero", "-fno-fast-math", "-Xclang", "-target-feature",
                        "-Xclang", "-packed-fp32-ops"};
  const int rc = r->compile(prog, int(sizeof(opts) / sizeof(opts[0])), opts);
  if (rc != 0) {
    size_t n = 0;
    r->log_size(prog, &n);
    std::string log(n, '\0');
    if (n) r->log(prog, &log[0]);
    *err = "hipRTC compile failed: " + log.substr(0, 2000);
    r->destroy(&prog);
    return false;
  }
  size_t n = 0;
  r->code_size(prog, &n);
  code->assign(n, 0);
  r->code(prog, code->data());
  r->destroy(&prog);
  return n > 0;
}

bool jit_load(const std::vector<char>& code, JitKernel* k, std::string* err) {
  hipModule_t m = nullptr;
  hipError_t e = hipModuleLoadData(&m, code.data());
  if (e != hipSuccess) {
    *err = std::string("hipModuleLoadData: ") + hipGetErrorString(e);
    return false;
  }
  hipFunction_t f = nullptr;
  e = hipModuleGetFunction(&f, m, "ar_jit");
  if (e != hipSuccess) {
    (void)hipModuleUnload(m);
    *err = std::string("hipModuleGetFunction: ") + hipGetErrorString(e);
    return false;
  }
  k->module = m;
  k->fn = f;
  return true;
}

void jit_unload(JitKernel* k) {
  if (k->module) (void)hipModuleUnload(static_cast<hipModule_t>(k->module));
  k->module = nullptr;
  k->fn = nullptr;
}

}  // namespace ar

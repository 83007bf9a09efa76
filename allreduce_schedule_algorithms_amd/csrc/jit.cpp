// Register DAG kernels compiled at run time (jit.h).
#include "jit.h"

#include <dlfcn.h>
#include <hip/hip_runtime_api.h>

#include <algorithm>
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
struct Args { void* p[32]; const Item* items; float div; int pad; };
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

bool jit_compile(const std::string& src, std::vector<char>* code, std::string* err) {
  Rtc* r = rtc();
  if (!r->h) {
    *err = r->why;
    return false;
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

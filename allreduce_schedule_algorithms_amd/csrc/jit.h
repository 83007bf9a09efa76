// Register DAG kernels compiled at run time (hipRTC) for one fused program.
//
// The DAG replay keeps every value of a range's result trees in LDS and reads
// its combinations from a program at run time. For programs with few ranks and
// few ranges that indirection costs more than the arithmetic: the same DAG
// written out as straight-line code keeps every value in registers and every
// operand a compile-time register. This module writes that code for the ranges
// of one schedule (one C++ function per range, each distinct combination once,
// in the DAG's level order) and compiles it for gfx950 with hipRTC on the plan's
// first call. The bits equal the other replays': the same combinations of the
// same operands, and IEEE addition and the maximum are commutative.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "sched.h"

namespace ar {

// One compiled module: its code object and, once loaded on a device, the
// kernel. Modules are loaded on the device current at jit_load.
struct JitKernel {
  void* module = nullptr;  // hipModule_t
  void* fn = nullptr;      // hipFunction_t
};

// Limits of the register form: ranks (buffer pointers in the kernel argument),
// ranges (one function each), distinct combinations per range.
constexpr int kJitMaxRanks = 32;
constexpr int kJitMaxRanges = 16;
constexpr int kJitMaxNodes = 256;
// 32-bit registers per thread for values live at once (fragments of one or two
// 16-byte vectors per value, widened to fp32 for bf16)
constexpr int kJitRegisterBudget = 192;

// Work item of the compiled kernel: the fused replay's Item (start, count,
// range index as tag); its kernel argument.
struct JitArgs {
  void* p[kJitMaxRanks];
  const void* items;
  float div;  // avg: complete results are divided by this (P)
  int32_t pad;
};

// Source of the kernel `ar_jit` for schedule s with the given element type and
// operation (Dtype, Op of sched.h); *vectors is the 16-byte vectors a thread
// takes per item (at most max_vectors, 1 or 2; work items then hold 256 x
// *vectors vectors). False (and *why) when a range's program exceeds the
// limits above.
bool jit_source(const Schedule& s, int dtype, int op, int max_vectors, std::string* src, int* vectors,
                std::string* why);

// Table form, for programs of one result tree per range in which every
// range's tree has one shape (leaf count, combinations after each leaf, output
// count) and only the ranks differ: the shape is compiled once as straight-line
// code, and each work item reads its range's leaf and output ranks from a
// table (kJitTabRanks buffer pointers in the kernel argument). A work item is
// one wave's (64 lanes x *vectors 16-byte vectors, or up to 64 single
// elements), four per workgroup. Leaves are loaded in batches of
// kJitTableBatch, the next batch in flight while one is combined.
constexpr int kJitTabRanks = 256;
constexpr int kJitTableBatch = 8;
constexpr int kJitTableRegisters = 256;  // loads in flight and stack values, 32-bit registers per lane
struct JitTabArgs {
  void* p[kJitTabRanks];
  const void* items;
  const void* tab;  // int32 ranks: per range, its leaves (postfix order), then its outputs
  float div;
  int32_t w;        // words per range in tab
};
// *tab, *w: the rank table; *vectors: 16-byte vectors per lane (at most
// max_vectors). False (and *why) when the ranges differ in shape or the
// program exceeds the limits.
bool jit_table_source(const Schedule& s, int dtype, int op, int max_vectors, std::string* src, std::vector<int32_t>* tab,
                      int* w, int* vectors, std::string* why);

// Compile src for gfx950 (no packed fp32, no contraction, IEEE denormals).
bool jit_compile(const std::string& src, std::vector<char>* code, std::string* err);

// Load a code object on the current device; unload frees it.
bool jit_load(const std::vector<char>& code, JitKernel* k, std::string* err);
void jit_unload(JitKernel* k);

// Whether hipRTC could be loaded (the library looks next to the HIP runtime in
// use, then in the ROCm installation); *why says what failed.
bool jit_available(std::string* why);

}  // namespace ar

// libar_probe.so: streaming kernels that move the bytes of an Allreduce over P
// rank buffers with no arithmetic (include/ar_probe.h). They bound what a
// one-pass Allreduce kernel can reach on the same buffers.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "../../include/ar_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kMaxRanks = 256;
constexpr int kBatch = 8;  // ranks loaded before their stores, as the direct kernel's leaf batch

struct Bufs {
  u32x4* p[kMaxRanks];
};

thread_local int32_t t_hip = 0;

// M 16-byte vectors per thread and rank at vector offsets v, v + kThreads, ...
// inside the block's run of kThreads * M vectors (every wave-level access is
// 1 KB contiguous). NP > 0: compiled for exactly NP ranks, every rank loaded
// before any store (the direct kernel's order); NP == 0: any P, ranks kBatch
// at a time, the loads of a batch issued before its stores.
// `key` is 0 at run time; the stores write the loaded data XOR key, so the
// compiler cannot drop them as stores of the value just loaded from the same
// address.
template <int M, int NP>
__global__ __launch_bounds__(kThreads) void k_probe_streams(Bufs b, int P, int64_t nvec, uint32_t key) {
  const int64_t v0 = int64_t(blockIdx.x) * kThreads * M + threadIdx.x;
  bool ok[M];
#pragma unroll
  for (int j = 0; j < M; ++j) ok[j] = v0 + int64_t(j) * kThreads < nvec;
  if constexpr (NP > 0) {
    u32x4 r[NP][M];
#pragma unroll
    for (int k = 0; k < NP; ++k)
#pragma unroll
      for (int j = 0; j < M; ++j)
        if (ok[j]) r[k][j] = __builtin_nontemporal_load(b.p[k] + v0 + int64_t(j) * kThreads);
#pragma unroll
    for (int k = 0; k < NP; ++k)
#pragma unroll
      for (int j = 0; j < M; ++j)
        if (ok[j]) __builtin_nontemporal_store(r[k][j] ^ key, b.p[k] + v0 + int64_t(j) * kThreads);
    return;
  }
  for (int base = 0; base < P; base += kBatch) {
    u32x4 r[kBatch][M];
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
#pragma unroll
      for (int j = 0; j < M; ++j)
        if (base + k < P && ok[j]) r[k][j] = __builtin_nontemporal_load(b.p[base + k] + v0 + int64_t(j) * kThreads);
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
#pragma unroll
      for (int j = 0; j < M; ++j)
        if (base + k < P && ok[j])
          __builtin_nontemporal_store(r[k][j] ^ key, b.p[base + k] + v0 + int64_t(j) * kThreads);
  }
}

// The smallest one-pass Allreduce kernel: fp32 sum of NP ranks (compiled for
// 7 or 8), written back to every rank; M vectors per thread and rank laid out
// as above, all loads before any store, no work items, no rank table.
template <int M, int NP>
__global__ __launch_bounds__(kThreads) void k_probe_fold(Bufs b, int64_t nvec) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int64_t v0 = int64_t(blockIdx.x) * kThreads * M + threadIdx.x;
  bool ok[M];
#pragma unroll
  for (int j = 0; j < M; ++j) ok[j] = v0 + int64_t(j) * kThreads < nvec;
  f32x4 x[NP][M];
#pragma unroll
  for (int k = 0; k < NP; ++k)
#pragma unroll
    for (int j = 0; j < M; ++j)
      if (ok[j]) x[k][j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(b.p[k] + v0 + int64_t(j) * kThreads));
  f32x4 acc[M];
#pragma unroll
  for (int j = 0; j < M; ++j) acc[j] = x[0][j];
#pragma unroll
  for (int k = 1; k < NP; ++k)
#pragma unroll
    for (int j = 0; j < M; ++j) acc[j] = acc[j] + x[k][j];
#pragma unroll
  for (int k = 0; k < NP; ++k)
#pragma unroll
    for (int j = 0; j < M; ++j)
      if (ok[j]) __builtin_nontemporal_store(acc[j], reinterpret_cast<f32x4*>(b.p[k] + v0 + int64_t(j) * kThreads));
}

template <int M>
__global__ __launch_bounds__(kThreads) void k_probe_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                         int64_t nvec, uint32_t key) {
  const int64_t v0 = int64_t(blockIdx.x) * kThreads * M + threadIdx.x;
  u32x4 r[M];
#pragma unroll
  for (int j = 0; j < M; ++j)
    if (v0 + int64_t(j) * kThreads < nvec) r[j] = __builtin_nontemporal_load(src + v0 + int64_t(j) * kThreads);
#pragma unroll
  for (int j = 0; j < M; ++j)
    if (v0 + int64_t(j) * kThreads < nvec) __builtin_nontemporal_store(r[j] ^ key, dst + v0 + int64_t(j) * kThreads);
}

template <int M, int NP>
void streams(const Bufs& b, int P, int64_t nvec, int64_t blocks, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  hipExtLaunchKernelGGL((k_probe_streams<M, NP>), dim3(unsigned(blocks)), dim3(kThreads), 0, st, e0, e1, 0, b, P, nvec,
                        0u);
}

template <int M>
hipError_t launch(const Bufs& b, int P, int64_t nvec, int kind, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  const int64_t blocks = (nvec + int64_t(kThreads) * M - 1) / (int64_t(kThreads) * M);
  if (blocks > (int64_t(1) << 24) - 1) return hipErrorInvalidValue;
  if (kind == AR_PROBE_STREAMS) {
    switch (P) {  // the rank counts of the large workloads, compiled exactly
      case 7: streams<M, 7>(b, P, nvec, blocks, st, e0, e1); break;
      case 8: streams<M, 8>(b, P, nvec, blocks, st, e0, e1); break;
      default: streams<M, 0>(b, P, nvec, blocks, st, e0, e1); break;
    }
  } else if (kind == AR_PROBE_FOLD) {
    if (P == 7)
      hipExtLaunchKernelGGL((k_probe_fold<M, 7>), dim3(unsigned(blocks)), dim3(kThreads), 0, st, e0, e1, 0, b, nvec);
    else
      hipExtLaunchKernelGGL((k_probe_fold<M, 8>), dim3(unsigned(blocks)), dim3(kThreads), 0, st, e0, e1, 0, b, nvec);
  } else
    hipExtLaunchKernelGGL((k_probe_copy<M>), dim3(unsigned(blocks)), dim3(kThreads), 0, st, e0, e1, 0, b.p[0], b.p[1],
                          nvec, 0u);
  return hipGetLastError();
}

}  // namespace

extern "C" {

int32_t ar_probe_stream(void* const* bufs, int32_t P, int64_t bytes, int32_t kind, int32_t vectors_per_thread,
                        void* stream, void* start_event, void* stop_event) {
  if (!bufs || P < 1 || P > kMaxRanks || bytes <= 0 || bytes % 16) return 1;
  if (kind != AR_PROBE_STREAMS && kind != AR_PROBE_COPY && kind != AR_PROBE_FOLD) return 1;
  if (kind == AR_PROBE_COPY && P != 2) return 1;
  if (kind == AR_PROBE_FOLD && P != 7 && P != 8) return 1;
  Bufs b;
  std::memset(&b, 0, sizeof(b));
  for (int p = 0; p < P; ++p) {
    if (!bufs[p] || reinterpret_cast<uintptr_t>(bufs[p]) % 16) return 1;
    b.p[p] = static_cast<u32x4*>(bufs[p]);
  }
  const int64_t nvec = bytes / 16;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipEvent_t e0 = static_cast<hipEvent_t>(start_event), e1 = static_cast<hipEvent_t>(stop_event);
  hipError_t e;
  switch (vectors_per_thread) {
    case 1: e = launch<1>(b, P, nvec, kind, st, e0, e1); break;
    case 2: e = launch<2>(b, P, nvec, kind, st, e0, e1); break;
    case 4: e = launch<4>(b, P, nvec, kind, st, e0, e1); break;
    default: return 1;
  }
  t_hip = int32_t(e);
  return e == hipSuccess ? 0 : 2;
}

int32_t ar_probe_last_hip_error(void) { return t_hip; }

}  // extern "C"

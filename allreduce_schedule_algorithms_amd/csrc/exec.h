// Device executor interface (implemented in exec.hip).
#pragma once

#include <cstddef>
#include <cstdint>
#include <memory>
#include <string>

#include "sched.h"

namespace ar {

enum Exec : int32_t { E_FUSED = 0, E_LITERAL = 1, E_REPLAY = 2, E_DAG = 3 };

struct RunResult {
  int status = 0;     // ar_status value
  int hip_error = 0;  // hipError_t when status == AR_HIP_ERROR
  std::string message;
};

// Enqueue one Allreduce on `stream`. Arguments have been validated.
RunResult run_allreduce(void* const* bufs, const Spec& spec, int exec, void* workspace,
                        size_t workspace_bytes, void* stream, void* start_event = nullptr,
                        void* stop_event = nullptr);

// The allocation-free variant of run_allreduce's literal execution: the
// call's work records and workspace slots live in a static device array of
// kScratchBytes per device (no allocation, no device tables). Calls on one
// device share the array: overlapping calls race.
constexpr size_t kScratchBytes = size_t(64) << 20;
RunResult run_noalloc(void* const* bufs, const Spec& spec, void* stream, void* start_event = nullptr,
                      void* stop_event = nullptr);

// Workspace a call needs (builds the schedule): the literal executor's slots
// for AR_EXEC_LITERAL, and for fused calls whose replay does not fit (they run
// the literal steps); 0 otherwise.
RunResult workspace_bytes(const Spec& spec, int exec, size_t* bytes);

// Workgroups one kernel launch may hold: 2^32 work-items at most (32-bit grid
// size in the dispatch packet), 256 per workgroup.
constexpr int64_t kMaxLaunchBlocks = (int64_t(1) << 32) / 256 - 1;

// Current per-launch workgroup limit; longer work is split into several launches.
int64_t launch_blocks();
// Set the limit (1..kMaxLaunchBlocks; false otherwise); the old value goes to *previous.
bool set_launch_blocks(int64_t blocks, int64_t* previous);

// Which kernel family a call runs (host only; builds the schedule). Values as
// ar_kernel in include/ar.h.
enum Kernel : int32_t {
  K_NONE = 0, K_DIRECT = 1, K_LITERAL = 2, K_REPLAY = 3, K_STAGED = 4, K_STRIDED = 5,
  K_FIXED_CHAIN = 6, K_FIXED_BALANCED = 7, K_FIXED_STACK = 8, K_MULTI = 9, K_ROWS = 10, K_ROWS_VEC = 11,
  K_DAG = 12, K_JIT = 13
};
RunResult kernel_of(const Spec& spec, int exec, int* kernel);

// Plans (device tables per schedule and size) and literal workspaces held by
// the library; retired ones stay allocated until release_cached().
struct CacheStats {
  int64_t live_plans = 0, retired_plans = 0, workspaces = 0, retired_workspaces = 0;
  int64_t plan_device_bytes = 0, workspace_device_bytes = 0;
};
CacheStats cache_stats();
// Synchronize every device the caches touch, then free every plan, workspace
// and cached schedule.
RunResult release_cached();

// Cached host schedule for a spec (shared with the executor's plan cache).
std::shared_ptr<const Schedule> cached_schedule(const Spec& spec, std::string* err);

}  // namespace ar

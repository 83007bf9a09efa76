/*
 * ar.h -- C ABI of the MI355X Allreduce schedule library (libar_mi355x.so).
 *
 * One call combines P rank buffers that live in the HBM of one GPU into their
 * elementwise reduction and writes that result back into every buffer, the
 * Allreduce operation defined in the introduction of "A Generalization of the
 * Allreduce Operation" (vectors owned by the processes are combined into a
 * result that is distributed back to all of them; the elementwise combine is
 * the vector operator of the "Reduction Operator" page). Each schedule named
 * below is executed as its own step list; a call never falls back to a
 * different schedule or to the CPU.
 *
 * Conventions shared by every entry point
 *  - Buffers: bufs[p] is rank p's buffer, caller-owned device memory holding
 *    batch * n elements of the call's dtype (instance b at element b * n).
 *    The call is in place: bufs[p] is input and output, as an in-place
 *    ncclAllReduce (all-reduce blog page, "The APIs"). The library never frees
 *    or keeps the pointers; the host array bufs is read before the call returns.
 *    16-byte aligned buffers use 128-bit accesses; other alignments are
 *    accepted and take a per-element path.
 *  - Stream: `stream` is a hipStream_t (NULL = the default stream). Work is
 *    enqueued and the call returns without waiting, like ncclAllReduce
 *    (all-reduce blog page, "The APIs"). Kernel faults surface at the caller's
 *    next synchronization.
 *  - Errors: arguments are validated on the host before any device work; on
 *    a non-AR_OK return no buffer has been touched. AR_HIP_ERROR carries the
 *    HIP code in ar_last_hip_error(); ar_last_error_message() gives text.
 *  - Precision: int32 sums wrap modulo 2^32; fp32 sums round to nearest even
 *    at every combination, in the schedule's order; bf16 inputs are widened
 *    exactly to fp32, every partial that crosses a step stays fp32, and each
 *    complete result is rounded to bf16 once (all-reduce blog page, "Numerics
 *    and reproducibility"). max uses the total order with -0 < +0; inputs must
 *    be NaN-free.
 *  - Threading: calls are thread-safe; calls on one stream run in order.
 *    Calls that overlap on different streams must not share buffers. A call
 *    that brings no workspace and runs the literal steps uses a workspace the
 *    library keeps per (device, stream), so such calls on different streams
 *    never share partial results.
 *  - Device tables and HIP graphs: the first call of a given schedule, size
 *    and buffer alignment on a device builds device tables (a synchronous
 *    allocation and copy); literal calls without a workspace may also allocate
 *    one. Neither can happen while the stream is being captured: such a call
 *    returns AR_UNSUPPORTED and enqueues nothing, so make one call outside the
 *    capture first. The library never frees a table or workspace that an
 *    enqueued or captured call may use: tables and workspaces it replaces are
 *    retired and kept until ar_release_cached(), so a captured graph stays
 *    valid however many other calls follow.
 *  - Limits: 1 <= P <= 256 (AR_MAX_RANKS).
 */
#ifndef AR_MI355X_H
#define AR_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AR_MAX_RANKS 256

typedef enum {
  AR_OK = 0,
  AR_INVALID_ARGUMENT = 1,
  AR_UNSUPPORTED = 2,
  AR_WORKSPACE_TOO_SMALL = 3,
  AR_HIP_ERROR = 4,
  AR_INTERNAL = 5
} ar_status;

typedef enum { AR_INT32 = 0, AR_FP32 = 1, AR_BF16 = 2 } ar_dtype;
/* AR_AVG (fp32, bf16): the sum, in the accumulation type (fp32), divided by P once when it is
 * complete, then rounded once to the caller's type (all-reduce blog page, "The APIs": the
 * average is taken inside the collective). The division is IEEE (correctly rounded). */
typedef enum { AR_SUM = 0, AR_MAX = 1, AR_AVG = 2 } ar_op;

/* The collective a call runs. Parts are the ceil split of the n elements of an instance into
 * P parts (part q = [q c, (q + 1) c) cut to n, c = ceil(n / P)); the blog page's FSDP/ZeRO
 * paragraph ("The APIs") splits the Allreduce into these two halves.
 *  AR_ALLREDUCE       every rank ends with the reduction of all P buffers.
 *  AR_REDUCE_SCATTER  rank q ends with the reduction of part q, in place at part q's offsets.
 *                     Other elements: untouched by AR_EXEC_FUSED; the step-by-step executor may
 *                     leave partial results there. op as for the Allreduce.
 *  AR_ALL_GATHER      rank q contributes its part q (its other elements are ignored); every
 *                     rank ends with every part. op is ignored (copies only).
 * Halves exist for AR_DIRECT, AR_RING, AR_RH_RD (P a power of two), AR_GENERALIZED and
 * AR_GENERALIZED_XOR (knob 0: the reduction phase, or the distribution phase, of the
 * bandwidth-optimal version), and AR_AUTO among those. */
typedef enum { AR_ALLREDUCE = 0, AR_REDUCE_SCATTER = 1, AR_ALL_GATHER = 2 } ar_collective;

/* Schedules (the pages that define each one):
 *  AR_DIRECT          one root gathers, combines in rank order, broadcasts (all-reduce blog
 *                     page, cost-model section, the naive approach); 2(P-1) steps.
 *  AR_RING            ring reduce-scatter + all-gather, 2(P-1) steps (blog page, "The ring
 *                     algorithm"; generalized-Allreduce paper, eqs. (14)-(16), Fig. 5).
 *  AR_RH_RD           recursive halving reduce-scatter + recursive doubling all-gather,
 *                     2 log2 P' steps, plus fold-in/out steps when P is not a power of two
 *                     (generalized-Allreduce paper, introduction and related work).
 *  AR_RD              recursive doubling, log2 P' steps (+2 with fold-in) (same paper).
 *  AR_BINOMIAL        binomial-tree reduce + broadcast, 2 ceil(log2 P) steps ("Reduction
 *                     Operator" page).
 *  AR_GENERALIZED     group-theoretic generalized Allreduce over the cyclic group Z_P, any P,
 *                     2 ceil(log2 P) - knob steps (generalized-Allreduce paper, eqs. (17)-(44),
 *                     Figs. 5-6).
 *                     With ar_call.steps = S > ceil(log2 P) (the paper's conclusion names such a
 *                     version, up to 2(P-1) steps, without defining it): the same base step
 *                     moving fewer vectors, h_i = max(ceil((N_i - 1) / (S - i)),
 *                     N_i - 2^(S-i-1)), N_{i+1} = N_i - h_i.
 *  AR_GENERALIZED_XOR the same over the self-inverse group of Table 1.b (P a power of two).
 *  AR_AHC             asymmetric hierarchical Allreduce over contiguous groups (HCCL "AHC"
 *                     page, Description), 2(max g - 1) + 2(G - 1) steps.
 *  AR_CHAIN           pipelined chain reduce to rank 0 + pipelined chain broadcast ("Reduction
 *                     Operator" page, pipelined algorithm): knob = m pieces (1..4096, ceil
 *                     split); in reduce step t rank i passes piece t - (P-1-i) to i - 1, which
 *                     combines it; 2(P + m - 2) steps. AR_KNOB_AUTO takes the floor or ceiling
 *                     of the page's optimum m. */
typedef enum {
  AR_DIRECT = 0,
  AR_RING = 1,
  AR_RH_RD = 2,
  AR_RD = 3,
  AR_BINOMIAL = 4,
  AR_GENERALIZED = 5,
  AR_GENERALIZED_XOR = 6,
  AR_AHC = 7,
  AR_CHAIN = 8,
  AR_AUTO = -1             /* let the cost model pick (see ar_select) */
} ar_algo;

/* ar_call.knob with AR_GENERALIZED / AR_GENERALIZED_XOR: let the cost model pick r. */
#define AR_KNOB_AUTO (-1)

/* Execution of a schedule on the GPU.
 *  AR_EXEC_FUSED    default. An AR_DIRECT Allreduce runs the one-pass direct kernel (read all
 *                   P, combine left to right, write all P); every other schedule and collective
 *                   runs its fused per-element replay: one launch evaluates, per element,
 *                   exactly the combination trees the step list builds, in registers, or for
 *                   ranges with more than 8 result trees (or several trees with a stack deeper
 *                   than 8) in the DAG replay, with the values in LDS. A schedule neither can
 *                   hold (a rounded partial combined again, or a DAG whose values exceed the
 *                   workgroup's LDS) runs the literal steps instead, with the same bits, and
 *                   then uses a workspace like AR_EXEC_LITERAL (ar_workspace_bytes says how
 *                   much).
 *  AR_EXEC_LITERAL  one launch per schedule step (chunk REDUCE / COPY kernels), partials
 *                   through HBM workspace slots; a last launch moves results that ended in
 *                   a workspace slot into the caller's buffer.
 *  AR_EXEC_REPLAY   the fused replay kernel for every schedule, AR_DIRECT included.
 *  AR_EXEC_DAG      the DAG replay (AR_KERNEL_DAG) for every schedule, AR_DIRECT included:
 *                   each distinct combination of a range's result trees is evaluated once, in
 *                   levels, with the values in LDS (see ar_schedule_dag_export). AR_EXEC_FUSED
 *                   runs it for programs with more result trees per range than the register
 *                   replays hold.
 * All three give bit-identical results for the same schedule. */
typedef enum { AR_EXEC_FUSED = 0, AR_EXEC_LITERAL = 1, AR_EXEC_REPLAY = 2, AR_EXEC_DAG = 3 } ar_exec;

/* Full description of one call. */
typedef struct ar_call {
  int32_t P;               /* ranks, 1..AR_MAX_RANKS */
  int32_t dtype;           /* ar_dtype */
  int32_t op;              /* ar_op */
  int32_t algo;            /* ar_algo; AR_AUTO lets the cost model choose */
  int32_t knob;            /* AR_GENERALIZED*: r = distribution steps removed, 0..ceil(log2 P) (or
                              0..steps), or AR_KNOB_AUTO; AR_CHAIN: pieces m >= 1, or
                              AR_KNOB_AUTO; ignored otherwise */
  int32_t exec;            /* ar_exec */
  int64_t n;               /* elements per instance (>= 0) */
  int64_t batch;           /* independent instances per buffer (>= 1); 0 is read as 1 */
  int32_t ngroups;         /* AR_AHC: number of groups G (>= 1); with AR_AUTO, optional (0 leaves
                              AHC out of the candidates); AR_GENERALIZED: optional, the number
                              of factors t (<= 8) of its group */
  const int32_t* groups;   /* AR_AHC: G group sizes summing to P, ranks assigned in order.
                              AR_GENERALIZED: factors m_1..m_t (each >= 2, product P) of the
                              group T_P = Z_m1 x ... x Z_mt, element k being the mixed-radix number
                              with digits k mod m_1, (k / m_1) mod m_2, ...; none: Z_P. (P) is the
                              cyclic group, (2, ..., 2) the self-inverse one of AR_GENERALIZED_XOR.
                              Other factorizations change which ranks talk in a step; a step can
                              then have a rank talk to several peers (ar_schedule_info.single_port).
                              Ignored by the other algorithms. */
  void* workspace;         /* calls that run the literal steps: device scratch of
                              ar_workspace_bytes() bytes, or
                              NULL to let the library allocate and cache one per device */
  size_t workspace_bytes;
  void* start_event;       /* optional hipEvent_t (created by the caller): recorded when the
                              call's first kernel starts */
  void* stop_event;        /* optional hipEvent_t: recorded when the call's last kernel ends.
                              With both set, hipEventElapsedTime gives the device time of the
                              call's kernels without the launch latency in front of them */
  int32_t collective;      /* ar_collective; 0 (AR_ALLREDUCE) for a zeroed call */
  int32_t steps;           /* AR_GENERALIZED: reduction steps S, ceil(log2 P) <= S <= P - 1, or 0
                              for ceil(log2 P). More steps move smaller pieces (S = P - 1: one part
                              per step, a ring-shaped chain); the call takes 2S - knob steps and
                              knob ranges over 0..S. Must be 0 for other algorithms. See the
                              schedule notes above. */
} ar_call;

/* Plain Allreduce: fused execution, batch 1, no groups (AR_AHC needs ar_allreduce_ex).
 * bufs: host array of P device pointers, each to n elements. */
ar_status ar_allreduce(void* const* bufs, int32_t P, int64_t n, int32_t dtype, int32_t op,
                       int32_t algo, int32_t knob, void* stream);

/* Reduce-scatter and all-gather halves: fused execution, batch 1, no groups (see
 * ar_collective). bufs: host array of P device pointers, each to n elements. */
ar_status ar_reduce_scatter(void* const* bufs, int32_t P, int64_t n, int32_t dtype, int32_t op,
                            int32_t algo, void* stream);
ar_status ar_all_gather(void* const* bufs, int32_t P, int64_t n, int32_t dtype, int32_t algo,
                        void* stream);

/* The collective of call->collective (an Allreduce by default) with every option of ar_call. */
ar_status ar_allreduce_ex(void* const* bufs, const ar_call* call, void* stream);

/* Allocation-free variant of ar_allreduce_ex, for callers that cannot allocate device memory
 * (tight serving loops, harnesses that forbid allocation). The call runs its schedule step by
 * step as AR_EXEC_LITERAL does, with the same kernels and bits, but its work records and
 * workspace slots live in a device array the library declares statically: 64 MiB
 * (AR_NOALLOC_SCRATCH_BYTES) per device, held from the library's load until the process ends.
 * The call allocates nothing and builds no device tables: it copies the call's work records
 * (host tables built on its first use) into the array with hipMemcpyAsync on `stream`, then
 * enqueues the step launches. No element of the array needs clearing: each step writes a slot
 * before any step reads it.
 * Requirements: call->exec must be AR_EXEC_LITERAL and call->workspace NULL; the records and
 * slots must fit the array (ar_workspace_bytes gives the slots' share), else AR_UNSUPPORTED and
 * nothing is enqueued. Every call on one device shares that device's array, which keeps the last
 * call's contents: calls that overlap on one device (different streams, or threads) race and
 * corrupt each other's results; serialize them. Not meant for stream capture (the copies read
 * host memory). Other arguments, events and errors as ar_allreduce_ex. */
#define AR_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
ar_status ar_allreduce_noalloc(void* const* bufs, const ar_call* call, void* stream);

/* Workspace bytes a call needs: the literal workspace slots for AR_EXEC_LITERAL, and for
 * AR_EXEC_FUSED calls whose schedule runs the literal steps (see ar_exec); 0 otherwise.
 * Builds (and caches) the schedule; returns its validation error for invalid calls. */
ar_status ar_workspace_bytes(const ar_call* call, size_t* bytes);

/* The kernel family a call runs on the GPU (host only: builds and caches the schedule, like
 * ar_workspace_bytes). Fused execution picks one replay kernel per schedule and size; all
 * compute the same combination trees:
 *  AR_KERNEL_NONE            no launch (P = 1 or n = 0)
 *  AR_KERNEL_DIRECT          the one-pass direct kernel (AR_DIRECT Allreduce, AR_EXEC_FUSED)
 *  AR_KERNEL_LITERAL         one launch per schedule step (AR_EXEC_LITERAL, and fused calls the
 *                            replay cannot hold; see ar_exec)
 *  AR_KERNEL_REPLAY          the register-stack replay of the fused program
 *  AR_KERNEL_STAGED          the same with several result trees per range and P <= 16: every
 *                            rank's fragment is loaded once into LDS
 *  AR_KERNEL_STRIDED         batches whose ranges are all shorter than 64 elements: one element
 *                            per thread across a block of instances
 *  AR_KERNEL_FIXED_CHAIN     single-tree programs of at most 8 ranges whose trees are all chains
 *                            of 1..8 leaves ((x + y) + z ..., the ring, the pipelined chain)
 *  AR_KERNEL_FIXED_BALANCED  ... all perfect binary trees of 4 or 8 leaves (halving + doubling)
 *  AR_KERNEL_FIXED_STACK     ... all one other shape of 3..8 leaves (the generalized algorithm
 *                            over Z_P for small P); the fixed kinds take the ranges' buffer
 *                            pointers as a kernel argument
 *  AR_KERNEL_MULTI           several trees per range, all of one shape over P = 3..8 leaves, at
 *                            most 8 ranges of 8 trees (the generalized algorithm with r > 0 on
 *                            up to 8 ranks): ranks staged in LDS once, the trees' ranks read
 *                            from a fixed-stride table.
 *  AR_KERNEL_ROWS            batches whose ranges are all shorter than 64 elements and all run one
 *                            program up to a renaming of leaf ranks (the ring and the generalized
 *                            algorithm's pieces of a short vector): one element per thread over
 *                            consecutive elements of the batch, each thread's range and its
 *                            buffers looked up in LDS.
 *  AR_KERNEL_ROWS_VEC        the same batches with 4-byte elements, one tree per range, at most 32
 *                            ranks and more than 4096 elements (16-byte aligned buffers; otherwise
 *                            AR_KERNEL_ROWS runs): every rank's vectors loaded once, and the leaves
 *                            read in each range's order from registers (at most 3 ranks) or from
 *                            an LDS stage.
 *  AR_KERNEL_DAG             the DAG replay: more than 8 result trees per range (the generalized
 *                            algorithm with large r at large P), and every call under
 *                            AR_EXEC_DAG; each distinct combination once, values in LDS.
 *  AR_KERNEL_JIT             several result trees per range, or a call of at most 4096 elements
 *                            over more than 8 ranks, with at most 32 ranks and 16 ranges (the
 *                            generalized algorithm with r > 0; latency-bound calls), not short
 *                            ranges of a batch: each range's DAG written out as straight-line
 *                            register code and compiled for the schedule with hipRTC on the
 *                            plan's first call (one compile per distinct program, kept for the
 *                            process), loaded on the device at its first launch. Where hipRTC
 *                            is missing or the program exceeds the register budget, the
 *                            kernels above run instead (AR_TRACE=1 says why); AR_JIT=0 turns it
 *                            off. It also runs one range of one result tree over more than 32
 *                            ranks (halving and doubling, recursive doubling, the binomial tree,
 *                            the pipelined chain at large P): the tree's shape compiled once,
 *                            the leaf and output ranks read from a table, one work item per
 *                            wave. */
typedef enum {
  AR_KERNEL_NONE = 0,
  AR_KERNEL_DIRECT = 1,
  AR_KERNEL_LITERAL = 2,
  AR_KERNEL_REPLAY = 3,
  AR_KERNEL_STAGED = 4,
  AR_KERNEL_STRIDED = 5,
  AR_KERNEL_FIXED_CHAIN = 6,
  AR_KERNEL_FIXED_BALANCED = 7,
  AR_KERNEL_FIXED_STACK = 8,
  AR_KERNEL_MULTI = 9,
  AR_KERNEL_ROWS = 10,
  AR_KERNEL_ROWS_VEC = 11,
  AR_KERNEL_DAG = 12,
  AR_KERNEL_JIT = 13
} ar_kernel;
ar_status ar_kernel_of(const ar_call* call, int32_t* kernel);

/* Device memory the library holds between calls: plans (the device tables of one
 * schedule, size and alignment per device) and literal workspaces (one per device and
 * stream, for calls that bring none). Live ones serve new calls; retired ones were
 * replaced (the plan cache holds at most 256 plans; a workspace that had to grow) and
 * are kept because enqueued or captured calls may still use them. */
typedef struct ar_cache_stats {
  int64_t live_plans, retired_plans;
  int64_t workspaces, retired_workspaces;
  int64_t plan_device_bytes;       /* tables of live and retired plans */
  int64_t workspace_device_bytes;  /* live and retired workspaces */
} ar_cache_stats;
ar_status ar_cache_stats_get(ar_cache_stats* out);
/* Free every plan, workspace and cached schedule the library holds (live and retired).
 * It first synchronizes every device they belong to, so launches already enqueued end
 * before their memory is freed. The caller must ensure that no call runs concurrently
 * on another thread and that no HIP graph captured before this call, containing calls
 * of this library, is launched afterwards: its kernels would read freed tables.
 * Returns AR_HIP_ERROR (nothing freed) if a synchronization fails. */
ar_status ar_release_cached(void);

/* Largest grid, in 256-thread workgroups, of one kernel launch. A call whose work needs
 * more (misaligned buffers of 2^32 elements or more, or about 2^35 aligned ones) runs as
 * several consecutive launches on the caller's stream with the same results; events of
 * ar_call then mark the first launch's start and the last one's end. The default and
 * maximum, 2^24 - 1, is what the 32-bit grid size of a dispatch holds. Process-wide; calls
 * enqueued afterwards use the new value. max_blocks outside [1, 2^24 - 1] returns
 * AR_INVALID_ARGUMENT and changes nothing. previous (may be NULL) receives the old value. */
ar_status ar_set_launch_blocks(int64_t max_blocks, int64_t* previous);

/* ---- schedules on the host (no GPU needed) ---- */
typedef struct ar_schedule ar_schedule;

typedef struct ar_oprec {
  int32_t step;      /* method step; finalize moves carry step == steps */
  int32_t kind;      /* 0 REDUCE: dst = own (+) src; 1 COPY: dst = src; 2 MOVE: same-rank slot
                        move after the last step */
  int32_t src_rank, src_slot;
  int32_t dst_rank, dst_slot;
  int32_t own_slot;  /* REDUCE: slot of dst_rank's own operand; -1 otherwise */
  int32_t pair;      /* index of the REDUCE executed jointly with this one (both read before
                        either writes), or -1 */
  int64_t offset;    /* first element, within one instance */
  int64_t length;    /* elements */
} ar_oprec;
/* Slot 0 is the caller's buffer; slot s >= 1 is a workspace buffer of the accumulation
 * type (int32 / fp32 / fp32 for int32 / fp32 / bf16). */

typedef struct ar_schedule_info {
  int32_t steps;         /* method steps */
  int32_t slots;         /* slots per rank including the caller's buffer */
  int32_t atoms;         /* chunks of the schedule's partition */
  int32_t single_port;   /* 1 if in every step each rank sends to <= 1 rank and receives from
                            <= 1 rank (the generalized paper's cost-model assumption) */
  int64_t ops;           /* exported records, finalize moves included */
  int64_t finalize_ops;
  int32_t fused_ok;      /* 1 if the fused replay program exists */
  int32_t ranges;        /* ranges of the fused program (per instance) */
  int32_t max_trees;     /* most distinct result trees in one range */
  int32_t max_need;      /* deepest evaluation stack of the fused program */
  int32_t max_leaves;
  int32_t program_words;
} ar_schedule_info;

/* Build (and validate) the step table of a call; host only. *out must be freed
 * with ar_schedule_free. */
ar_status ar_schedule_build(const ar_call* call, ar_schedule** out);
ar_status ar_schedule_info_get(const ar_schedule* s, ar_schedule_info* info);
/* Copy up to cap records into ops; *count receives the total number. */
ar_status ar_schedule_export(const ar_schedule* s, ar_oprec* ops, size_t cap, size_t* count);
/* Fused replay program. Per range r: starts[r], lens[r] (elements within an instance) and
 * offsets[r] into the int32 word stream. Words of a range: ntrees, then per tree
 * nleaves, nouts, nleaves leaf ranks (postfix order), nleaves counts of combinations that
 * follow each leaf, nouts destination ranks. Any pointer may be NULL to query sizes. */
ar_status ar_schedule_fused_export(const ar_schedule* s, int64_t* starts, int64_t* lens,
                                   int32_t* offsets, size_t range_cap, int32_t* words,
                                   size_t word_cap, size_t* nranges, size_t* nwords);
/* DAG form of the fused program, the one AR_KERNEL_DAG runs. Every distinct combination of a
 * range's result trees (a node identified by its unordered operands) is evaluated once, grouped
 * in levels of independent combinations, with values in numbered slots; a slot is reused only in
 * a level after its value's last read. Words of one program:
 *   S, nleaf, nlevel, ninstr, nout, then nleaf leaf ranks (leaf k in slot k), nlevel + 1
 *   instruction offsets (level l runs instructions [lv[l], lv[l + 1])), ninstr instructions
 *   (dst | a << 10 | b << 20: slot dst = slot a (+) slot b), nout outputs (slot << 16 | rank:
 *   the rank's result is the slot's value after the last level).
 * *shared = 1: one program serves every range; maps holds P bytes per range mapping the
 * program's ranks to the range's (offsets are all 0). *shared = 0: range r's program starts at
 * words[offsets[r]]. Ranges are those of ar_schedule_fused_export. Any pointer may be NULL to
 * query sizes (*nmaps = bytes of maps). */
ar_status ar_schedule_dag_export(const ar_schedule* s, int32_t* shared, int32_t* offsets, size_t range_cap,
                                 uint8_t* maps, size_t map_cap, int32_t* words, size_t word_cap, size_t* nranges,
                                 size_t* nmaps, size_t* nwords);
void ar_schedule_free(ar_schedule* s);

/* Validate any table (for example a modified export): snapshot hazards inside a step,
 * complete results in every rank's slot 0 (symbolic replay), single-port property.
 * Returns AR_OK when the table is a correct Allreduce, AR_INVALID_ARGUMENT otherwise;
 * ar_last_error_message() says why. */
ar_status ar_table_check(int32_t P, int64_t n, int32_t dtype, const ar_oprec* ops,
                         size_t count, int32_t* single_port);
/* The same for any collective: P, n, dtype and collective are taken from call (its other
 * fields are ignored). A reduce-scatter table must leave the complete part q in rank q's slot
 * 0; an all-gather table must leave the owner's part in every rank's slot 0. */
ar_status ar_table_check_ex(const ar_call* call, const ar_oprec* ops, size_t count,
                            int32_t* single_port);

/* ---- alpha-beta-gamma cost report ----
 * A step costs alpha + (bytes sent or received by the busiest rank) * beta + (bytes
 * combined by the busiest rank) * gamma (generalized-Allreduce paper,
 * cost-model paragraph; all-reduce blog page, "A cost model for collectives").
 * closed_form_seconds evaluates the pages' printed closed form for the schedule (eqs.
 * (15), (25), (36), (44) of the generalized paper; NaN for AHC, whose formula the page
 * truncates). Elements are per call (all instances). */
typedef struct ar_cost {
  int32_t steps;
  int64_t sent_busiest, recv_busiest, reduced_busiest; /* per instance, sum over steps of the
                                                          per-step maximum over ranks */
  int64_t sent_total, reduced_total;                   /* per instance, all ranks */
  int64_t max_rank_sent, max_rank_reduced;             /* per instance, busiest rank overall */
  double predicted_seconds;
  double closed_form_seconds;
  double literal_hbm_bytes;  /* bytes AR_EXEC_LITERAL moves through HBM per call */
  double fused_hbm_bytes;    /* bytes the fused replay requests per call */
  double essential_bytes;    /* every input read once, every output written once, per call: 2 P n
                                batch elt (Allreduce), (P + 1) n batch elt (reduce-scatter),
                                P n batch elt (all-gather) */
} ar_cost;
ar_status ar_cost_report(const ar_schedule* s, double alpha, double beta, double gamma,
                         ar_cost* out);
/* Per-step, per-rank element counts (steps x P, row-major, per instance). */
ar_status ar_cost_steps(const ar_schedule* s, int64_t* sent, int64_t* recv, int64_t* reduced);

/* ---- model-driven choice of schedule ----
 * The generalized-Allreduce paper picks its step count r from measured alpha (latency),
 * beta (transfer time per byte) and gamma (combination time per byte) by minimising the
 * cost of eq. (36) (section "Intermediate version" and eq. (37)); the all-reduce blog page
 * describes a library that picks algorithm and protocol per call from a tuning model
 * ("Protocols: Simple, LL and LL128"). Here the model time of a schedule is
 *   alpha * steps + beta * B_sent + gamma * B_combined
 * with the bytes taken from the schedule's exact per-step, per-rank counts (the counts
 * ar_cost_steps returns, times the element size and batch):
 *   AR_COST_BUSIEST_RANK  per step the busiest rank (max of sent and received bytes, and of
 *                         combined bytes), summed over steps: ranks on separate links, the
 *                         paper's model.
 *   AR_COST_ALL_RANKS     every rank's bytes summed: all ranks share one memory, as in this
 *                         library's step-by-step executor (AR_EXEC_LITERAL) on one device.
 * AR_AUTO enumerates AR_DIRECT, AR_RING, AR_RH_RD, AR_RD, AR_BINOMIAL, AR_GENERALIZED r = 0..
 * ceil(log2 P), AR_GENERALIZED_XOR r = 0..ceil(log2 P) when P is a power of two, AR_AHC when
 * groups are given, and AR_CHAIN with the floor and the ceiling of the "Reduction Operator"
 * page's optimal piece count, m* = sqrt(M (P - 2)(2 beta + gamma) / (2 alpha)) for M bytes per
 * rank (clamped to 1..min(4096, n)); AR_KNOB_AUTO enumerates r (or those m) for the given
 * algorithm. The least model time
 * wins; ties go to fewer steps, then to the earlier candidate in that order. The choice
 * depends only on (P, n, batch, dtype, groups) and the model, never on timing. The default
 * model is a least-squares fit of AR_EXEC_LITERAL fp32 calls measured on MI355X, form
 * AR_COST_ALL_RANKS (values via ar_get_cost_model). */
typedef enum { AR_COST_BUSIEST_RANK = 0, AR_COST_ALL_RANKS = 1 } ar_cost_form;
typedef struct ar_cost_model {
  double alpha;  /* seconds per step */
  double beta;   /* seconds per byte sent */
  double gamma;  /* seconds per byte combined */
  int32_t form;  /* ar_cost_form */
  int32_t reserved;
} ar_cost_model;
/* Replace the process-wide model (NULL restores the default). Parameters must be finite and
 * >= 0. Calls already resolved keep no stale choice: the selection cache is cleared. Not
 * meant to race with calls on other threads that use AR_AUTO / AR_KNOB_AUTO. */
ar_status ar_set_cost_model(const ar_cost_model* model);
ar_status ar_get_cost_model(ar_cost_model* model);
/* Resolve a call's schedule as ar_allreduce_ex would: *algo and *knob receive the schedule
 * that runs (unchanged for explicit calls), *predicted_seconds its model time under the
 * current model. Any output pointer may be NULL. Host only. */
ar_status ar_select(const ar_call* call, int32_t* algo, int32_t* knob, double* predicted_seconds);

const char* ar_status_string(ar_status st);
int32_t ar_last_hip_error(void);
const char* ar_last_error_message(void);
/* Library version string. */
const char* ar_version(void);

#ifdef __cplusplus
}
#endif
#endif /* AR_MI355X_H */

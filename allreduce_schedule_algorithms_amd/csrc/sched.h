// Host schedule layer: step-table generators for every Allreduce schedule,
// slot realization with snapshot semantics, a hazard / port checker, the
// fused per-element replay planner and the alpha-beta-gamma cost walk.
//
// A schedule is a list of steps; a step is a set of operations that all read
// the state from before the step. An operation moves a range of elements
// from (src rank, src slot) to (dst rank, dst slot), either combining it with
// the destination rank's own operand (REDUCE) or overwriting (COPY). Every
// operation touches the same element offsets in both ranks: the rows of the
// generalized-Allreduce paper's data matrix gather one element index across all
// processes, and ring and AHC chunks are cut at the same offsets on every
// device. Slot 0 of a rank is the caller's buffer; slots >= 1 are workspace
// buffers of the accumulation type.
#pragma once

#include <array>
#include <cstdint>
#include <string>
#include <unordered_map>
#include <vector>

namespace ar {

enum Kind : int32_t { K_REDUCE = 0, K_COPY = 1, K_MOVE = 2 };
enum Algo : int32_t {
  A_DIRECT = 0, A_RING = 1, A_RH_RD = 2, A_RD = 3, A_BINOMIAL = 4,
  A_GENERALIZED = 5, A_GENERALIZED_XOR = 6, A_AHC = 7, A_CHAIN = 8, A_NUM_ALGOS = 9
};
enum Dtype : int32_t { D_INT32 = 0, D_FP32 = 1, D_BF16 = 2 };
// O_AVG combines as a sum; the complete result is divided by P once.
enum Op : int32_t { O_SUM = 0, O_MAX = 1, O_AVG = 2 };
// Collective: the Allreduce, or one of its halves over the ceil split into P
// parts (reduce-scatter: rank q ends with the reduced part q; all-gather: rank
// q contributes its part q and every rank ends with all parts).
enum Coll : int32_t { C_ALLREDUCE = 0, C_REDUCE_SCATTER = 1, C_ALL_GATHER = 2 };

constexpr int kMaxRanks = 256;
constexpr int kMaxChainPieces = 4096;

struct Spec {
  int P = 0;
  int64_t n = 0;       // elements per instance
  int64_t batch = 1;   // instances per rank buffer, contiguous (instance b at b * n)
  int dtype = D_FP32;
  int op = O_SUM;
  int algo = A_RING;
  int knob = 0;
  std::vector<int> groups;  // AHC group sizes (contiguous ranks)
  int coll = C_ALLREDUCE;
  int steps = 0;  // generalized (cyclic): reduction steps, 0 = ceil(log2 P)
};

// Hash-consed commutative expression DAG over rank leaves 0..P-1.
class Exprs {
 public:
  explicit Exprs(int P);
  int combine(int a, int b);
  bool is_leaf(int id) const { return id < P_; }
  int left(int id) const { return a_[id - P_]; }
  int right(int id) const { return b_[id - P_]; }
  bool complete(int id) const;   // every rank exactly once
  int leaves(int id) const { return id < P_ ? 1 : cnt_[id - P_]; }
  int P() const { return P_; }

 private:
  using Mask = std::array<uint64_t, kMaxRanks / 64>;
  const Mask& mask(int id) const { return id < P_ ? leafmask_[id] : mask_[id - P_]; }
  int P_;
  std::vector<int> a_, b_, cnt_;
  std::vector<Mask> mask_;
  std::vector<Mask> leafmask_;
  Mask full_{};
  std::unordered_map<uint64_t, int> ids_;
};

// One logical operation on one atom (chunk) of the algorithm's partition.
struct LOp {
  int kind, src, dst, atom;
  int src_val, own_val, out_val;
};

// Realized table record (also the exported C record layout).
struct OpRec {
  int32_t step, kind;
  int32_t src_rank, src_slot;
  int32_t dst_rank, dst_slot;
  int32_t own_slot;  // REDUCE: slot of the destination rank's own operand
  int32_t pair;      // index of the op executed jointly with this one, or -1
  int64_t offset, length;  // element range within one instance
};

struct FusedRange {
  int64_t start, len;   // element range within one instance
  int32_t prog;         // offset of its program in the word stream
  int32_t ntrees;
  int32_t need;         // evaluation stack depth
};

struct Schedule {
  Spec spec;
  int nsteps = 0;
  int nslots = 1;
  int C = 1;  // atoms
  std::vector<std::pair<int64_t, int64_t>> atoms;  // element range per atom
  std::vector<OpRec> ops;  // sorted by step; MOVE ops (step == nsteps) restore slot 0
  std::vector<uint8_t> completes;  // per op: a REDUCE whose result is a complete reduction
  std::vector<int32_t> steps_begin;  // ops index where each step starts (nsteps + 2 entries)
  int64_t finalize_ops = 0;
  bool single_port = true;
  // fused replay program (per instance)
  bool fused_ok = false;
  std::string fused_error;
  std::vector<int32_t> prog;
  std::vector<FusedRange> ranges;
  int max_need = 0, max_trees = 0, max_leaves = 0;
};

// DAG form of one range's fused program (its words in Schedule::prog). The
// range's result trees share sub-trees (the generalized algorithm's shifted
// schedules combine the same partial sums), so every distinct combination --
// a node identified by its unordered pair of operands, itself hash-consed --
// is evaluated once. Nodes are grouped in levels (a node's level is one more
// than its deeper operand's); the combinations of one level are independent.
// Values live in numbered slots: leaf k (k-th distinct leaf rank in postfix
// order) in slot k, and each node in a slot freed by a value whose last use
// lies in an earlier level, so no slot is read and written within one level.
// A combination keeps the operand order in which the postfix program first
// builds it. Outputs are read after the last level. Programs of ranges whose
// trees are equal up to a renaming of ranks differ only in leaf and output ranks.
struct DagProgram {
  int32_t S = 0;                     // slots
  std::vector<int32_t> leaves;       // rank of the leaf in slot k
  std::vector<int32_t> level_start;  // levels + 1 offsets into instr
  std::vector<uint32_t> instr;       // dst | a << 10 | b << 20: slot dst = slot a (+) slot b
  std::vector<int32_t> outs;         // slot << 16 | rank: rank's result is slot's value
  // serialized: S, leaves, levels, instructions, outputs, then the arrays
  std::vector<int32_t> words() const;
};
constexpr int kDagMaxSlots = 1024;
bool compile_dag(const int32_t* range_words, int P, DagProgram* out, std::string* err);
// Whether b equals a with every leaf and output rank renamed (leaves in order;
// outputs as a set of (slot, rank)): fills map with a's rank -> b's rank (ranks
// a does not use map to themselves if free, else to an unused rank) so that map
// is a permutation.
bool dag_renaming(const DagProgram& a, const DagProgram& b, int P, std::vector<int>* map);

// DAG programs of a whole fused program. Shared: every range's program is the
// reference range's with ranks renamed, so one program serves all ranges and
// maps holds, per range, P bytes (reference rank -> the range's rank); otherwise
// one program per range, at offsets into words.
struct DagPlan {
  bool shared = false;
  int ref = 0;                   // shared: the reference range
  std::vector<int32_t> words;    // serialized programs (DagProgram::words)
  std::vector<int32_t> offsets;  // per range: its program's offset in words (shared: 0)
  std::vector<uint8_t> maps;     // shared: ranges x P renaming rows
  int S = 0;                     // most slots of any program
  int levels = 0;                // most levels
  int64_t instr = 0;             // combinations per element, most of any range
};
// allow_shared false: one program per range even where they differ only by a renaming.
bool dag_plan(const Schedule& s, DagPlan* out, std::string* err, bool allow_shared = true);

// Generate + realize + plan. Returns nullptr and sets *err on invalid input.
Schedule* build_schedule(const Spec& spec, std::string* err);

// Validate a spec without building (cheap argument checks).
bool validate_spec(const Spec& spec, std::string* err);

// Check an arbitrary exported table: snapshot hazards inside each step, that
// every final value in slot 0 is a complete reduction (symbolic replay), and
// the single-port property. Returns true when the table is a correct Allreduce.
struct TableCheck {
  bool ok = false;
  bool single_port = true;
  int nslots = 0;
  std::string message;
};
TableCheck check_table(int P, int64_t n, int dtype, const OpRec* ops, size_t count, int coll = C_ALLREDUCE);

// Whether a schedule has a reduce-scatter / all-gather half here.
bool half_supported(int algo);

struct CostOut {
  int32_t steps;
  int64_t sent_busiest, recv_busiest, reduced_busiest;  // elements, summed over steps of the per-step max
  int64_t sent_total, reduced_total;                      // elements, all ranks, all steps
  int64_t max_rank_sent, max_rank_reduced;                // elements, the busiest rank over the whole run
  double predicted_seconds;
  double closed_form_seconds;  // NaN when the pages give none
  double literal_hbm_bytes;    // bytes the literal executor moves through HBM per call
  double fused_hbm_bytes;      // bytes the fused replay requests per call
  double essential_bytes;      // 2 P n elt per call
};
CostOut cost_walk(const Schedule& s, double alpha, double beta, double gamma);
// per-step, per-rank element counters (steps x P, row-major)
void cost_steps(const Schedule& s, int64_t* sent, int64_t* recv, int64_t* reduced);

// Per-step, per-rank element counts straight from the generator's logical
// operations (no realization, no fused planning): the same counts as
// cost_steps on the realized table, at a fraction of the build cost. A
// message is one (src rank, src value, dst rank, atom) per step. With n == 0
// or P == 1 nothing moves and there are no steps.
struct StepCounts {
  int nsteps = 0;
  std::vector<int64_t> sent, recv, reduced;  // nsteps x P, row-major, per instance
};
bool step_counts(const Spec& spec, StepCounts* out, std::string* err);

// Model-driven choice of schedule (generalized-Allreduce paper: the optimal
// step count follows from the measured alpha, beta, gamma; all-reduce blog
// page: the library picks an algorithm per call from a cost model).
enum CostForm : int32_t { F_BUSIEST = 0, F_ALL_RANKS = 1 };
struct CostModel {
  double alpha = 0, beta = 0, gamma = 0;
  int form = F_BUSIEST;
};
constexpr int kAutoAlgo = -1;
constexpr int kAutoKnob = -1;
// Model time of a schedule from its step counts: alpha per step plus beta per
// byte moved and gamma per byte combined, where the bytes are the per-step
// maxima over ranks (F_BUSIEST) or the sums over ranks (F_ALL_RANKS).
double model_seconds(const StepCounts& c, const Spec& spec, const CostModel& m);
// Resolve kAutoAlgo / kAutoKnob in `in` to the candidate of least model time
// (ties: fewer steps, then the earlier candidate). Other specs pass through.
bool select_spec(const Spec& in, const CostModel& m, Spec* out, double* seconds, std::string* err);
bool is_auto(const Spec& s);
std::vector<int> chain_pieces(const Spec& s, const CostModel& m);

int elt_bytes(int dtype);
int acc_bytes(int dtype);
int ceil_log2(int P);

}  // namespace ar

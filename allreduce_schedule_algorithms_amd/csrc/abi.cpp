// extern "C" entry points declared in include/ar.h.
#include "../../include/ar.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "exec.h"
#include "sched.h"

static_assert(sizeof(ar_oprec) == sizeof(ar::OpRec), "ar_oprec layout");

namespace {

thread_local std::string t_msg;
thread_local int32_t t_hip = 0;

ar_status fail(ar_status st, const std::string& m) {
  t_msg = m;
  return st;
}

// Process-wide cost model for AR_AUTO / AR_KNOB_AUTO and the choices made under it.
// Default: least-squares fit of AR_EXEC_LITERAL fp32 calls on MI355X (P = 7 and 8,
// 2^10..2^22 elements, every schedule and r), one launch per step, all ranks'
// bytes through one HBM.
constexpr ar::CostModel kDefaultModel{3.52e-6, 2.10e-13, 2.07e-13, ar::F_ALL_RANKS};
std::mutex g_model_mu;
ar::CostModel g_model = kDefaultModel;
std::map<std::string, std::pair<ar::Spec, double>> g_choices;

std::string choice_key(const ar::Spec& s) {
  std::string k = std::to_string(s.P) + "/" + std::to_string(s.n) + "/" + std::to_string(s.batch) + "/" +
                  std::to_string(s.dtype) + "/" + std::to_string(s.op) + "/" + std::to_string(s.algo) + "/" +
                  std::to_string(s.knob) + "/" + std::to_string(s.coll) + "/" + std::to_string(s.steps) + "/";
  for (int g : s.groups) k += std::to_string(g) + ",";
  return k;
}

// Replace an AR_AUTO / AR_KNOB_AUTO spec by the model's choice (cached per spec).
bool resolve(ar::Spec* s, double* seconds, std::string* err) {
  std::lock_guard<std::mutex> lk(g_model_mu);
  const std::string key = choice_key(*s);
  auto it = g_choices.find(key);
  if (it == g_choices.end()) {
    ar::Spec out;
    double t = 0;
    if (!ar::select_spec(*s, g_model, &out, &t, err)) return false;
    if (g_choices.size() > 4096) g_choices.clear();
    it = g_choices.emplace(key, std::make_pair(out, t)).first;
  }
  *s = it->second.first;
  if (seconds) *seconds = it->second.second;
  return true;
}

bool to_spec(const ar_call* c, ar::Spec* s, std::string* err) {
  if (!c) { *err = "call is NULL"; return false; }
  s->P = c->P;
  s->n = c->n;
  s->batch = c->batch == 0 ? 1 : c->batch;
  s->dtype = c->dtype;
  s->op = c->op;
  s->algo = c->algo;
  s->knob = (c->algo == AR_GENERALIZED || c->algo == AR_GENERALIZED_XOR || c->algo == AR_CHAIN) ? c->knob : 0;
  s->steps = c->steps;
  s->groups.clear();
  if (c->algo == AR_AHC) {
    if (c->ngroups < 1 || !c->groups) { *err = "AHC needs ngroups >= 1 and a groups array"; return false; }
    if (c->ngroups > AR_MAX_RANKS) { *err = "too many AHC groups"; return false; }
    s->groups.assign(c->groups, c->groups + c->ngroups);
  } else if (c->algo == AR_GENERALIZED && c->ngroups != 0) {
    if (c->ngroups < 0 || !c->groups) { *err = "ngroups > 0 needs a groups array"; return false; }
    if (c->ngroups > 8) { *err = "at most 8 group factors"; return false; }
    s->groups.assign(c->groups, c->groups + c->ngroups);
  } else if (c->algo == AR_AUTO && c->ngroups != 0) {
    if (c->ngroups < 0 || !c->groups) { *err = "ngroups > 0 needs a groups array"; return false; }
    if (c->ngroups > AR_MAX_RANKS) { *err = "too many AHC groups"; return false; }
    s->groups.assign(c->groups, c->groups + c->ngroups);
    ar::Spec probe = *s;
    probe.algo = ar::A_AHC;
    if (!ar::validate_spec(probe, err)) return false;
  }
  if (c->exec < AR_EXEC_FUSED || c->exec > AR_EXEC_DAG) { *err = "unknown exec mode"; return false; }
  if (c->collective < AR_ALLREDUCE || c->collective > AR_ALL_GATHER) { *err = "unknown collective"; return false; }
  s->coll = c->collective;
  if (s->coll == AR_ALL_GATHER) s->op = ar::O_SUM;  // copies only: the op plays no part
  if (ar::is_auto(*s)) return resolve(s, nullptr, err);
  return ar::validate_spec(*s, err);
}

ar_status check_bufs(void* const* bufs, int P) {
  if (!bufs) return fail(AR_INVALID_ARGUMENT, "bufs is NULL");
  uintptr_t v[AR_MAX_RANKS];  // P was validated: 1..AR_MAX_RANKS
  for (int p = 0; p < P; ++p) {
    if (!bufs[p]) return fail(AR_INVALID_ARGUMENT, "bufs[" + std::to_string(p) + "] is NULL");
    v[p] = reinterpret_cast<uintptr_t>(bufs[p]);
  }
  std::sort(v, v + P);
  for (int p = 1; p < P; ++p)
    if (v[p] == v[p - 1]) return fail(AR_INVALID_ARGUMENT, "two ranks share one buffer");
  return AR_OK;
}

}  // namespace

extern "C" {

ar_status ar_set_cost_model(const ar_cost_model* m) {
  ar::CostModel cm = kDefaultModel;
  if (m) {
    if (!(std::isfinite(m->alpha) && std::isfinite(m->beta) && std::isfinite(m->gamma)) || m->alpha < 0 ||
        m->beta < 0 || m->gamma < 0)
      return fail(AR_INVALID_ARGUMENT, "alpha, beta, gamma must be finite and >= 0");
    if (m->form != AR_COST_BUSIEST_RANK && m->form != AR_COST_ALL_RANKS)
      return fail(AR_INVALID_ARGUMENT, "unknown cost form");
    cm = ar::CostModel{m->alpha, m->beta, m->gamma, m->form};
  }
  std::lock_guard<std::mutex> lk(g_model_mu);
  g_model = cm;
  g_choices.clear();
  return AR_OK;
}

ar_status ar_set_launch_blocks(int64_t max_blocks, int64_t* previous) {
  if (!ar::set_launch_blocks(max_blocks, previous))
    return fail(AR_INVALID_ARGUMENT, "max_blocks must be in [1, " + std::to_string(ar::kMaxLaunchBlocks) + "]");
  return AR_OK;
}

ar_status ar_get_cost_model(ar_cost_model* m) {
  if (!m) return fail(AR_INVALID_ARGUMENT, "model is NULL");
  std::lock_guard<std::mutex> lk(g_model_mu);
  m->alpha = g_model.alpha;
  m->beta = g_model.beta;
  m->gamma = g_model.gamma;
  m->form = g_model.form;
  m->reserved = 0;
  return AR_OK;
}

ar_status ar_select(const ar_call* call, int32_t* algo, int32_t* knob, double* predicted_seconds) {
  std::string err;
  ar::Spec spec;
  if (!to_spec(call, &spec, &err)) return fail(AR_INVALID_ARGUMENT, err);
  double t = 0;
  if (predicted_seconds) {
    ar::CostModel cm;
    {
      std::lock_guard<std::mutex> lk(g_model_mu);
      cm = g_model;
    }
    if (!ar::select_spec(spec, cm, &spec, &t, &err)) return fail(AR_INVALID_ARGUMENT, err);
    *predicted_seconds = t;
  }
  if (algo) *algo = spec.algo;
  if (knob) *knob = spec.knob;
  return AR_OK;
}

const char* ar_status_string(ar_status st) {
  switch (st) {
    case AR_OK: return "AR_OK";
    case AR_INVALID_ARGUMENT: return "AR_INVALID_ARGUMENT";
    case AR_UNSUPPORTED: return "AR_UNSUPPORTED";
    case AR_WORKSPACE_TOO_SMALL: return "AR_WORKSPACE_TOO_SMALL";
    case AR_HIP_ERROR: return "AR_HIP_ERROR";
    case AR_INTERNAL: return "AR_INTERNAL";
  }
  return "unknown status";
}

int32_t ar_last_hip_error(void) { return t_hip; }
const char* ar_last_error_message(void) { return t_msg.c_str(); }
const char* ar_version(void) { return "allreduce-schedules-mi355x 0.1 (gfx950)"; }

ar_status ar_allreduce_ex(void* const* bufs, const ar_call* call, void* stream) {
  std::string err;
  ar::Spec spec;
  if (!to_spec(call, &spec, &err)) return fail(AR_INVALID_ARGUMENT, err);
  ar_status st = check_bufs(bufs, spec.P);
  if (st != AR_OK) return st;
  ar::RunResult r = ar::run_allreduce(bufs, spec, call->exec, call->workspace, call->workspace_bytes, stream,
                                      call->start_event, call->stop_event);
  t_hip = r.hip_error;
  if (r.status) return fail(ar_status(r.status), r.message);
  t_msg.clear();
  return AR_OK;
}

ar_status ar_allreduce(void* const* bufs, int32_t P, int64_t n, int32_t dtype, int32_t op, int32_t algo,
                       int32_t knob, void* stream) {
  if (algo == AR_AHC) return fail(AR_INVALID_ARGUMENT, "AR_AHC needs group sizes: use ar_allreduce_ex");
  ar_call c;
  std::memset(&c, 0, sizeof(c));
  c.P = P;
  c.n = n;
  c.batch = 1;
  c.dtype = dtype;
  c.op = op;
  c.algo = algo;
  c.knob = knob;
  c.exec = AR_EXEC_FUSED;
  return ar_allreduce_ex(bufs, &c, stream);
}

static_assert(AR_NOALLOC_SCRATCH_BYTES == ar::kScratchBytes, "scratch size");

ar_status ar_allreduce_noalloc(void* const* bufs, const ar_call* call, void* stream) {
  std::string err;
  ar::Spec spec;
  if (!to_spec(call, &spec, &err)) return fail(AR_INVALID_ARGUMENT, err);
  if (call->exec != AR_EXEC_LITERAL)
    return fail(AR_INVALID_ARGUMENT, "the allocation-free entry point runs the literal steps: exec must be AR_EXEC_LITERAL");
  if (call->workspace) return fail(AR_INVALID_ARGUMENT, "the allocation-free entry point takes no workspace");
  ar_status st = check_bufs(bufs, spec.P);
  if (st != AR_OK) return st;
  ar::RunResult r = ar::run_noalloc(bufs, spec, stream, call->start_event, call->stop_event);
  t_hip = r.hip_error;
  if (r.status) return fail(ar_status(r.status), r.message);
  t_msg.clear();
  return AR_OK;
}

ar_status ar_reduce_scatter(void* const* bufs, int32_t P, int64_t n, int32_t dtype, int32_t op, int32_t algo,
                            void* stream) {
  if (algo == AR_AHC) return fail(AR_INVALID_ARGUMENT, "AR_AHC has no reduce-scatter half here");
  ar_call c;
  std::memset(&c, 0, sizeof(c));
  c.P = P;
  c.n = n;
  c.batch = 1;
  c.dtype = dtype;
  c.op = op;
  c.algo = algo;
  c.exec = AR_EXEC_FUSED;
  c.collective = AR_REDUCE_SCATTER;
  return ar_allreduce_ex(bufs, &c, stream);
}

ar_status ar_all_gather(void* const* bufs, int32_t P, int64_t n, int32_t dtype, int32_t algo, void* stream) {
  if (algo == AR_AHC) return fail(AR_INVALID_ARGUMENT, "AR_AHC has no all-gather half here");
  ar_call c;
  std::memset(&c, 0, sizeof(c));
  c.P = P;
  c.n = n;
  c.batch = 1;
  c.dtype = dtype;
  c.op = AR_SUM;
  c.algo = algo;
  c.exec = AR_EXEC_FUSED;
  c.collective = AR_ALL_GATHER;
  return ar_allreduce_ex(bufs, &c, stream);
}

ar_status ar_workspace_bytes(const ar_call* call, size_t* bytes) {
  std::string err;
  ar::Spec spec;
  if (!bytes) return fail(AR_INVALID_ARGUMENT, "bytes is NULL");
  if (!to_spec(call, &spec, &err)) return fail(AR_INVALID_ARGUMENT, err);
  *bytes = 0;
  if ((call->exec == AR_EXEC_FUSED && spec.algo == AR_DIRECT && spec.coll == AR_ALLREDUCE) || spec.P <= 1 ||
      spec.n == 0)
    return AR_OK;
  ar::RunResult r = ar::workspace_bytes(spec, call->exec, bytes);
  if (r.status) return fail(ar_status(r.status), r.message);
  return AR_OK;
}

ar_status ar_kernel_of(const ar_call* call, int32_t* kernel) {
  std::string err;
  ar::Spec spec;
  if (!kernel) return fail(AR_INVALID_ARGUMENT, "kernel is NULL");
  if (!to_spec(call, &spec, &err)) return fail(AR_INVALID_ARGUMENT, err);
  int k = 0;
  ar::RunResult r = ar::kernel_of(spec, call->exec, &k);
  if (r.status) return fail(ar_status(r.status), r.message);
  *kernel = k;
  return AR_OK;
}

ar_status ar_cache_stats_get(ar_cache_stats* out) {
  if (!out) return fail(AR_INVALID_ARGUMENT, "out is NULL");
  const ar::CacheStats c = ar::cache_stats();
  out->live_plans = c.live_plans;
  out->retired_plans = c.retired_plans;
  out->workspaces = c.workspaces;
  out->retired_workspaces = c.retired_workspaces;
  out->plan_device_bytes = c.plan_device_bytes;
  out->workspace_device_bytes = c.workspace_device_bytes;
  return AR_OK;
}

ar_status ar_release_cached(void) {
  ar::RunResult r = ar::release_cached();
  if (r.status) {
    t_hip = r.hip_error;
    return fail(ar_status(r.status), r.message);
  }
  return AR_OK;
}

ar_status ar_schedule_build(const ar_call* call, ar_schedule** out) {
  std::string err;
  ar::Spec spec;
  if (!out) return fail(AR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  if (!to_spec(call, &spec, &err)) return fail(AR_INVALID_ARGUMENT, err);
  ar::Schedule* s = ar::build_schedule(spec, &err);
  if (!s) return fail(AR_INTERNAL, err);
  *out = reinterpret_cast<ar_schedule*>(s);
  return AR_OK;
}

ar_status ar_schedule_dag_export(const ar_schedule* sh, int32_t* shared, int32_t* offsets, size_t range_cap,
                                 uint8_t* maps, size_t map_cap, int32_t* words, size_t word_cap, size_t* nranges,
                                 size_t* nmaps, size_t* nwords) {
  if (!sh) return fail(AR_INVALID_ARGUMENT, "NULL schedule");
  const ar::Schedule& s = *reinterpret_cast<const ar::Schedule*>(sh);
  if (!s.fused_ok) return fail(AR_UNSUPPORTED, "no fused program: " + s.fused_error);
  ar::DagPlan d;
  std::string err;
  if (!ar::dag_plan(s, &d, &err)) return fail(AR_UNSUPPORTED, err);
  if (shared) *shared = d.shared ? 1 : 0;
  if (nranges) *nranges = d.offsets.size();
  if (nmaps) *nmaps = d.maps.size();
  if (nwords) *nwords = d.words.size();
  if (offsets) std::memcpy(offsets, d.offsets.data(), std::min(range_cap, d.offsets.size()) * sizeof(int32_t));
  if (maps && !d.maps.empty()) std::memcpy(maps, d.maps.data(), std::min(map_cap, d.maps.size()));
  if (words) std::memcpy(words, d.words.data(), std::min(word_cap, d.words.size()) * sizeof(int32_t));
  return AR_OK;
}

void ar_schedule_free(ar_schedule* s) { delete reinterpret_cast<ar::Schedule*>(s); }

ar_status ar_schedule_info_get(const ar_schedule* sh, ar_schedule_info* info) {
  if (!sh || !info) return fail(AR_INVALID_ARGUMENT, "NULL argument");
  const ar::Schedule& s = *reinterpret_cast<const ar::Schedule*>(sh);
  info->steps = s.nsteps;
  info->slots = s.nslots;
  info->atoms = s.C;
  info->single_port = s.single_port ? 1 : 0;
  info->ops = int64_t(s.ops.size());
  info->finalize_ops = s.finalize_ops;
  info->fused_ok = s.fused_ok ? 1 : 0;
  info->ranges = int32_t(s.ranges.size());
  info->max_trees = s.max_trees;
  info->max_need = s.max_need;
  info->max_leaves = s.max_leaves;
  info->program_words = int32_t(s.prog.size());
  return AR_OK;
}

ar_status ar_schedule_export(const ar_schedule* sh, ar_oprec* ops, size_t cap, size_t* count) {
  if (!sh) return fail(AR_INVALID_ARGUMENT, "NULL schedule");
  const ar::Schedule& s = *reinterpret_cast<const ar::Schedule*>(sh);
  if (count) *count = s.ops.size();
  if (ops) std::memcpy(ops, s.ops.data(), std::min(cap, s.ops.size()) * sizeof(ar_oprec));
  return AR_OK;
}

ar_status ar_schedule_fused_export(const ar_schedule* sh, int64_t* starts, int64_t* lens, int32_t* offsets,
                                   size_t range_cap, int32_t* words, size_t word_cap, size_t* nranges,
                                   size_t* nwords) {
  if (!sh) return fail(AR_INVALID_ARGUMENT, "NULL schedule");
  const ar::Schedule& s = *reinterpret_cast<const ar::Schedule*>(sh);
  if (!s.fused_ok) return fail(AR_UNSUPPORTED, "no fused program: " + s.fused_error);
  if (nranges) *nranges = s.ranges.size();
  if (nwords) *nwords = s.prog.size();
  for (size_t r = 0; r < std::min(range_cap, s.ranges.size()); ++r) {
    if (starts) starts[r] = s.ranges[r].start;
    if (lens) lens[r] = s.ranges[r].len;
    if (offsets) offsets[r] = s.ranges[r].prog;
  }
  if (words) std::memcpy(words, s.prog.data(), std::min(word_cap, s.prog.size()) * sizeof(int32_t));
  return AR_OK;
}

ar_status ar_table_check(int32_t P, int64_t n, int32_t dtype, const ar_oprec* ops, size_t count,
                         int32_t* single_port) {
  if (!ops && count) return fail(AR_INVALID_ARGUMENT, "ops is NULL");
  if (dtype < AR_INT32 || dtype > AR_BF16) return fail(AR_INVALID_ARGUMENT, "unknown dtype");
  ar::TableCheck tc = ar::check_table(P, n, dtype, reinterpret_cast<const ar::OpRec*>(ops), count);
  if (single_port) *single_port = tc.single_port ? 1 : 0;
  if (!tc.ok) return fail(AR_INVALID_ARGUMENT, tc.message);
  return AR_OK;
}

ar_status ar_table_check_ex(const ar_call* call, const ar_oprec* ops, size_t count, int32_t* single_port) {
  if (!call) return fail(AR_INVALID_ARGUMENT, "call is NULL");
  if (!ops && count) return fail(AR_INVALID_ARGUMENT, "ops is NULL");
  if (call->dtype < AR_INT32 || call->dtype > AR_BF16) return fail(AR_INVALID_ARGUMENT, "unknown dtype");
  if (call->collective < AR_ALLREDUCE || call->collective > AR_ALL_GATHER)
    return fail(AR_INVALID_ARGUMENT, "unknown collective");
  if (call->n < 0) return fail(AR_INVALID_ARGUMENT, "n must be >= 0");
  ar::TableCheck tc = ar::check_table(call->P, call->n, call->dtype, reinterpret_cast<const ar::OpRec*>(ops),
                                      count, call->collective);
  if (single_port) *single_port = tc.single_port ? 1 : 0;
  if (!tc.ok) return fail(AR_INVALID_ARGUMENT, tc.message);
  return AR_OK;
}

ar_status ar_cost_report(const ar_schedule* sh, double alpha, double beta, double gamma, ar_cost* out) {
  if (!sh || !out) return fail(AR_INVALID_ARGUMENT, "NULL argument");
  const ar::Schedule& s = *reinterpret_cast<const ar::Schedule*>(sh);
  ar::CostOut c = ar::cost_walk(s, alpha, beta, gamma);
  out->steps = c.steps;
  out->sent_busiest = c.sent_busiest;
  out->recv_busiest = c.recv_busiest;
  out->reduced_busiest = c.reduced_busiest;
  out->sent_total = c.sent_total;
  out->reduced_total = c.reduced_total;
  out->max_rank_sent = c.max_rank_sent;
  out->max_rank_reduced = c.max_rank_reduced;
  out->predicted_seconds = c.predicted_seconds;
  out->closed_form_seconds = c.closed_form_seconds;
  out->literal_hbm_bytes = c.literal_hbm_bytes;
  out->fused_hbm_bytes = c.fused_hbm_bytes;
  out->essential_bytes = c.essential_bytes;
  return AR_OK;
}

ar_status ar_cost_steps(const ar_schedule* sh, int64_t* sent, int64_t* recv, int64_t* reduced) {
  if (!sh || !sent || !recv || !reduced) return fail(AR_INVALID_ARGUMENT, "NULL argument");
  ar::cost_steps(*reinterpret_cast<const ar::Schedule*>(sh), sent, recv, reduced);
  return AR_OK;
}

}  // extern "C"

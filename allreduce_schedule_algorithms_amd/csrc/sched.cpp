// Schedule generators, slot realizer, table checker, fused planner, cost walk.
#include "sched.h"

#include <algorithm>
#include <cmath>
#include <functional>
#include <memory>
#include <tuple>
#include <limits>
#include <map>
#include <numeric>
#include <set>
#include <sstream>
#include <unordered_set>

namespace ar {

int ceil_log2(int P) {
  int L = 0;
  while ((1 << L) < P) ++L;
  return L;
}
int elt_bytes(int dtype) { return dtype == D_BF16 ? 2 : 4; }
int acc_bytes(int) { return 4; }

static int pow2_floor(int P) {
  int p = 1;
  while (p * 2 <= P) p *= 2;
  return p;
}

// Ceil split of [0, n) into C parts (the all-reduce blog page's split():
// chunk length ceil(n / C), the last parts short or empty).
static std::vector<std::pair<int64_t, int64_t>> partition(int64_t n, int C) {
  std::vector<std::pair<int64_t, int64_t>> out(C);
  int64_t c = C > 0 ? (n + C - 1) / C : 0;
  for (int k = 0; k < C; ++k) out[k] = {std::min<int64_t>(k * c, n), std::min<int64_t>((k + 1) * c, n)};
  return out;
}

static int64_t lcm_of(const std::vector<int>& g) {
  int64_t l = 1;
  for (int v : g) {
    l = l / std::gcd<int64_t>(l, v) * v;
    if (l > (1 << 20)) return l;
  }
  return l;
}

// ----------------------------------------------------------------------------
// expression DAG
// ----------------------------------------------------------------------------
Exprs::Exprs(int P) : P_(P) {
  leafmask_.resize(P);
  for (int p = 0; p < P; ++p) {
    leafmask_[p].fill(0);
    leafmask_[p][p / 64] |= uint64_t(1) << (p % 64);
    full_[p / 64] |= uint64_t(1) << (p % 64);
  }
}

int Exprs::combine(int a, int b) {
  if (a > b) std::swap(a, b);
  uint64_t key = (uint64_t(uint32_t(a)) << 32) | uint32_t(b);
  auto it = ids_.find(key);
  if (it != ids_.end()) return it->second;
  int id = P_ + int(a_.size());
  a_.push_back(a);
  b_.push_back(b);
  cnt_.push_back(leaves(a) + leaves(b));
  Mask m;
  const Mask& ma = mask(a);
  const Mask& mb = mask(b);
  for (size_t w = 0; w < m.size(); ++w) m[w] = ma[w] | mb[w];
  mask_.push_back(m);
  ids_.emplace(key, id);
  return id;
}

bool Exprs::complete(int id) const { return leaves(id) == P_ && mask(id) == full_; }

// ----------------------------------------------------------------------------
// generators: logical step lists over atoms
// ----------------------------------------------------------------------------
struct Logical {
  int C = 1;
  std::vector<std::vector<LOp>> steps;
};

// Helper for schedules in which every rank holds one current value per atom.
struct BufGen {
  int P, C;
  Exprs& ex;
  Logical& lg;
  std::vector<int> cur;
  std::vector<std::pair<int, int>> staged;
  BufGen(int P_, int C_, Exprs& e, Logical& l) : P(P_), C(C_), ex(e), lg(l), cur(size_t(P_) * C_) {
    lg.C = C_;
    for (int p = 0; p < P; ++p)
      for (int a = 0; a < C; ++a) cur[size_t(p) * C + a] = p;
  }
  void begin() { lg.steps.emplace_back(); }
  void msg(int kind, int src, int dst, int a0, int a1) {
    for (int a = a0; a < a1; ++a) {
      int sv = cur[size_t(src) * C + a];
      int ov = cur[size_t(dst) * C + a];
      int out = kind == K_REDUCE ? ex.combine(ov, sv) : sv;
      lg.steps.back().push_back({kind, src, dst, a, sv, kind == K_REDUCE ? ov : -1, out});
      staged.push_back({dst * C + a, out});
    }
  }
  void end() {
    for (auto& s : staged) cur[s.first] = s.second;
    staged.clear();
  }
};

// Naive one-root schedule (all-reduce blog page, cost-model section): the root
// folds ranks 1..P-1 in rank order, one per step, then sends the result back.
static void gen_direct(int P, Exprs& ex, Logical& lg) {
  BufGen g(P, 1, ex, lg);
  for (int s = 1; s < P; ++s) { g.begin(); g.msg(K_REDUCE, s, 0, 0, 1); g.end(); }
  for (int s = 1; s < P; ++s) { g.begin(); g.msg(K_COPY, 0, s, 0, 1); g.end(); }
}

// Ring reduce-scatter + all-gather (all-reduce blog page, "The ring
// algorithm"; generalized-Allreduce paper eqs. (14)-(16)). P parts, each
// making two laps of the ring, one hop r -> r + 1 per step for all parts at
// once: on the combining lap part k starts at rank k and every rank it reaches
// adds its own copy, so after P - 1 hops rank k - 1 holds the complete part;
// on the copying lap it leaves that rank and overwrites each copy it reaches.
static void ring_lap(BufGen& g, int P, int first_offset, int kind) {
  for (int t = 0; t < P - 1; ++t) {
    g.begin();
    for (int k = 0; k < P; ++k) {
      const int at = ((k + first_offset + t) % P + P) % P;  // part k's position before this hop
      g.msg(kind, at, (at + 1) % P, k, k + 1);
    }
    g.end();
  }
}
static void gen_ring(int P, Exprs& ex, Logical& lg) {
  BufGen g(P, P, ex, lg);
  ring_lap(g, P, 0, K_REDUCE);   // part k starts at rank k
  ring_lap(g, P, -1, K_COPY);    // and leaves its owner, rank k - 1
}

// Non-power-of-two preparation / finalization (generalized-Allreduce paper,
// related work): excess rank P'+j hands its buffer to rank j and gets the
// result back.
static void fold_in(BufGen& g, int P, int Pp) {
  if (P == Pp) return;
  g.begin();
  for (int j = 0; j < P - Pp; ++j) g.msg(K_REDUCE, Pp + j, j, 0, g.C);
  g.end();
}
static void fold_out(BufGen& g, int P, int Pp) {
  if (P == Pp) return;
  g.begin();
  for (int j = 0; j < P - Pp; ++j) g.msg(K_COPY, j, Pp + j, 0, g.C);
  g.end();
}

// Recursive halving over ranks 0..P'-1 (P' parts, partner distance P'/2
// first): afterwards rank p holds the complete part p.
static void halving(BufGen& g, int Pp) {
  const int L = ceil_log2(Pp);
  for (int s = 0; s < L; ++s) {
    int d = Pp >> (s + 1);
    g.begin();
    for (int p = 0; p < Pp; ++p) {
      int base = p & ~(2 * d - 1);
      int give = base + ((p & d) ? 0 : d);
      g.msg(K_REDUCE, p, p ^ d, give, give + d);
    }
    g.end();
  }
}

// Recursive doubling all-gather: distances 1, 2, ..., each rank copying its
// current window of parts to p XOR d.
static void doubling(BufGen& g, int Pp) {
  const int L = ceil_log2(Pp);
  for (int s = L - 1; s >= 0; --s) {
    int d = Pp >> (s + 1);
    g.begin();
    for (int p = 0; p < Pp; ++p) {
      int base = p & ~(d - 1);
      g.msg(K_COPY, p, p ^ d, base, base + d);
    }
    g.end();
  }
}

// Recursive halving reduce-scatter + recursive doubling all-gather over P'
// parts, with fold-in / fold-out for the excess ranks.
static void gen_rh_rd(int P, Exprs& ex, Logical& lg) {
  int Pp = pow2_floor(P);
  BufGen g(P, Pp, ex, lg);
  fold_in(g, P, Pp);
  halving(g, Pp);
  doubling(g, Pp);
  fold_out(g, P, Pp);
}

// Reduce-scatter and all-gather halves (part q belongs to rank q; P parts).
// Ring: the two laps with part q's start moved by one, so that the combining
// lap of part q starts at rank q + 1 and ends at its owner q, and the copying
// lap starts from q.
static void gen_ring_rs(int P, Exprs& ex, Logical& lg) {
  BufGen g(P, P, ex, lg);
  ring_lap(g, P, 1, K_REDUCE);
}
static void gen_ring_ag(int P, Exprs& ex, Logical& lg) {
  BufGen g(P, P, ex, lg);
  ring_lap(g, P, 0, K_COPY);
}
// Direct: the one-root fold (rank order), then rank 0 hands part q to rank q;
// all-gather: every rank sends its part to every other rank in one step.
static void gen_direct_rs(int P, Exprs& ex, Logical& lg) {
  BufGen g(P, P, ex, lg);
  for (int s = 1; s < P; ++s) { g.begin(); g.msg(K_REDUCE, s, 0, 0, P); g.end(); }
  g.begin();
  for (int q = 1; q < P; ++q) g.msg(K_COPY, 0, q, q, q + 1);
  g.end();
}
static void gen_direct_ag(int P, Exprs& ex, Logical& lg) {
  BufGen g(P, P, ex, lg);
  g.begin();
  for (int q = 0; q < P; ++q)
    for (int d = 0; d < P; ++d)
      if (d != q) g.msg(K_COPY, q, d, q, q + 1);
  g.end();
}
static void gen_halving_rs(int P, Exprs& ex, Logical& lg) {
  BufGen g(P, P, ex, lg);
  halving(g, P);
}
static void gen_doubling_ag(int P, Exprs& ex, Logical& lg) {
  BufGen g(P, P, ex, lg);
  doubling(g, P);
}

// Recursive doubling: full-buffer exchange with partner p XOR d, d = P'/2 first.
static void gen_rd(int P, Exprs& ex, Logical& lg) {
  int Pp = pow2_floor(P);
  int L = ceil_log2(Pp);
  BufGen g(P, 1, ex, lg);
  fold_in(g, P, Pp);
  for (int s = 0; s < L; ++s) {
    int d = Pp >> (s + 1);
    g.begin();
    for (int p = 0; p < Pp; ++p) g.msg(K_REDUCE, p ^ d, p, 0, 1);
    g.end();
  }
  fold_out(g, P, Pp);
}

// Binomial-tree reduce ("Reduction Operator" page) + broadcast as its reverse.
static void gen_binomial(int P, Exprs& ex, Logical& lg) {
  int K = ceil_log2(P);
  BufGen g(P, 1, ex, lg);
  std::vector<char> active(P, 1);
  for (int k = 0; k < K; ++k) {
    int b = 1 << k;
    g.begin();
    for (int i = 0; i < P; ++i) {
      if (!active[i]) continue;
      if (i & b) active[i] = 0;
      else if (i + b < P) g.msg(K_REDUCE, i + b, i, 0, 1);
    }
    g.end();
  }
  for (int k = K - 1; k >= 0; --k) {
    int b = 1 << k;
    g.begin();
    for (int i = 0; i + b < P; i += 2 * b) g.msg(K_COPY, i, i + b, 0, 1);
    g.end();
  }
}

// Pipelined chain ("Reduction Operator" page, pipelined algorithm): m pieces;
// in reduce step t unit i passes piece t - (P - 1 - i) to i - 1, which
// combines it (P + m - 2 steps, the root holding the last piece at the end);
// then the broadcast down the chain, unit i passing piece t - i to i + 1.
static void gen_chain(int P, int m, Exprs& ex, Logical& lg) {
  BufGen g(P, m, ex, lg);
  for (int t = 0; t < P + m - 2; ++t) {
    g.begin();
    for (int i = 1; i < P; ++i) {
      int k = t - (P - 1 - i);
      if (k >= 0 && k < m) g.msg(K_REDUCE, i, i - 1, k, k + 1);
    }
    g.end();
  }
  for (int t = 0; t < P + m - 2; ++t) {
    g.begin();
    for (int i = 0; i + 1 < P; ++i) {
      int k = t - i;
      if (k >= 0 && k < m) g.msg(K_COPY, i, i + 1, k, k + 1);
    }
    g.end();
  }
}

// AHC (HCCL "AHC" page): Lc x G chunks; ring reduce-scatter inside each group,
// ring Allreduce per piece between its owners, one per group (the page's
// logical devices that share an ID), over G equal sub-pieces, ring all-gather
// inside each group.
static void gen_ahc(int P, const std::vector<int>& groups, Exprs& ex, Logical& lg) {
  int G = int(groups.size());
  int C = int(lcm_of(groups)) * G;
  BufGen g(P, C, ex, lg);
  std::vector<int> offs(G, 0), span(G);
  for (int a = 1; a < G; ++a) offs[a] = offs[a - 1] + groups[a - 1];
  for (int a = 0; a < G; ++a) span[a] = C / groups[a];
  int gmax = *std::max_element(groups.begin(), groups.end());
  for (int t = 0; t < gmax - 1; ++t) {
    g.begin();
    for (int a = 0; a < G; ++a) {
      int ga = groups[a];
      if (t >= ga - 1) continue;
      for (int l = 0; l < ga; ++l) {
        int k = ((l - t) % ga + ga) % ga;
        g.msg(K_REDUCE, offs[a] + l, offs[a] + (l + 1) % ga, k * span[a], (k + 1) * span[a]);
      }
    }
    g.end();
  }
  std::set<int> cuts;
  for (int a = 0; a < G; ++a)
    for (int k = 0; k <= groups[a]; ++k) cuts.insert(k * span[a]);
  std::vector<int> b(cuts.begin(), cuts.end());
  struct Piece { std::vector<int> owner; std::vector<int> sub; };
  std::vector<Piece> pieces;
  for (size_t q = 0; q + 1 < b.size(); ++q) {
    Piece pc;
    for (int a = 0; a < G; ++a) {
      int ka = b[q] / span[a];
      pc.owner.push_back(offs[a] + ((ka - 1) % groups[a] + groups[a]) % groups[a]);
    }
    int w = (b[q + 1] - b[q]) / G;
    for (int s = 0; s <= G; ++s) pc.sub.push_back(b[q] + s * w);
    pieces.push_back(pc);
  }
  for (int t = 0; t < G - 1; ++t) {
    g.begin();
    for (auto& pc : pieces)
      for (int s = 0; s < G; ++s) {
        int sp = ((s - t) % G + G) % G;
        g.msg(K_REDUCE, pc.owner[s], pc.owner[(s + 1) % G], pc.sub[sp], pc.sub[sp + 1]);
      }
    g.end();
  }
  for (int t = 0; t < G - 1; ++t) {
    g.begin();
    for (auto& pc : pieces)
      for (int s = 0; s < G; ++s) {
        int sp = ((s + 1 - t) % G + G) % G;
        g.msg(K_COPY, pc.owner[s], pc.owner[(s + 1) % G], pc.sub[sp], pc.sub[sp + 1]);
      }
    g.end();
  }
  for (int t = 0; t < gmax - 1; ++t) {
    g.begin();
    for (int a = 0; a < G; ++a) {
      int ga = groups[a];
      if (t >= ga - 1) continue;
      for (int l = 0; l < ga; ++l) {
        int k = ((l + 1 - t) % ga + ga) % ga;
        g.msg(K_COPY, offs[a] + l, offs[a] + (l + 1) % ga, k * span[a], (k + 1) * span[a]);
      }
    }
    g.end();
  }
}

// Generalized Allreduce (generalized-Allreduce paper, bandwidth-optimal,
// intermediate and latency-optimal sections). Placement j puts part i at rank
// t_j(i) = i + j mod P (cyclic group) or i XOR j (self-inverse group). The
// shifted schedules S_j, j < N_{L-r}, run together; an identical vector (same
// placement, same tree) is sent and combined once.
//
// steps S > ceil(log2 P) (the paper's conclusion: more steps, smaller pieces,
// up to the ring's 2(P - 1); not defined there): the same base step with a
// smaller h_i, the even share of the parts still to move, ceil((N_i - 1) /
// (S - i)), raised where needed so that N_{i+1} can still halve down to one
// vector in the remaining steps (N_i - 2^(S-i-1)). S = P - 1 moves one part
// per step. Cyclic group only.
static void levels(int P, int S, std::vector<int>& N, std::vector<int>& h) {
  const int L = ceil_log2(P);
  N.assign(1, P);
  h.clear();
  for (int i = 0; i < S; ++i) {
    int hi;
    if (S == L) {
      hi = N[i] / 2;
    } else {
      const int left = S - i;
      const int share = (N[i] - 1 + left - 1) / left;
      const int64_t reach = left - 1 >= 30 ? 0 : int64_t(N[i]) - (int64_t(1) << (left - 1));
      hi = int(std::max<int64_t>(share, reach));
    }
    h.push_back(hi);
    N.push_back(N[i] - hi);
  }
}

// The group T_P = Z_m1 x ... x Z_mt (generalized paper: any suitable group,
// Table 1): element k is the mixed-radix number with digits k mod m1,
// (k / m1) mod m2, ...; the operation adds digits modulo their radix. {P} is
// the cyclic group, {2, 2, ...} the self-inverse group of Table 1.b.
static std::vector<int> group_table(int P, const std::vector<int>& radices) {
  std::vector<int> t(size_t(P) * P);
  for (int a = 0; a < P; ++a)
    for (int b = 0; b < P; ++b) {
      int x = a, y = b, out = 0, w = 1;
      for (int m : radices) {
        out += ((x % m + y % m) % m) * w;
        x /= m;
        y /= m;
        w *= m;
      }
      t[size_t(a) * P + b] = out;
    }
  return t;
}

static void gen_generalized(int P, int r, const std::vector<int>& radices, Exprs& ex, Logical& lg,
                            int coll = C_ALLREDUCE, int steps = 0) {
  const int L = steps > 0 ? steps : ceil_log2(P);  // reduction steps
  std::vector<int> N, h;
  levels(P, L, N, h);
  const std::vector<int> op = group_table(P, radices);
  auto place = [&](int k, int j) { return op[size_t(k) * P + j]; };
  auto holder = [&](int i, int pl) { return op[size_t(i) * P + pl]; };
  lg.C = P;
  int J = N[L - r];
  // vals[j][k][atom]
  std::vector<std::vector<std::vector<int>>> vals(J, std::vector<std::vector<int>>(P, std::vector<int>(P)));
  for (int j = 0; j < J; ++j)
    for (int k = 0; k < P; ++k)
      for (int a = 0; a < P; ++a) vals[j][k][a] = holder(a, place(k, j));
  // (dst, atom, result) combined so far: an identical vector is combined once,
  // in this step or an earlier one (more steps can bring a shifted schedule
  // to a tree another one built before)
  std::unordered_set<uint64_t> seen;
  for (int i = 0; i < (coll == C_ALL_GATHER ? 0 : L); ++i) {
    lg.steps.emplace_back();
    auto& st = lg.steps.back();
    auto nv = vals;
    for (int j = 0; j < J; ++j)
      for (int k = N[i] - h[i]; k < N[i]; ++k) {
        int tgt = k - h[i];
        int pls = place(k, j), pld = place(tgt, j);
        for (int a = 0; a < P; ++a) {
          int sv = vals[j][k][a], ov = vals[j][tgt][a];
          int out = ex.combine(ov, sv);
          int src = holder(a, pls), dst = holder(a, pld);
          if (seen.insert((uint64_t(uint32_t(out)) << 16) | (uint64_t(dst) << 8) | uint64_t(a)).second)
            st.push_back({K_REDUCE, src, dst, a, sv, ov, out});
          nv[j][tgt][a] = out;
        }
      }
    vals.swap(nv);
  }
  if (coll == C_REDUCE_SCATTER) return;  // placement 0 holds part a at rank a
  std::vector<std::vector<int>> dist(P);
  for (int j = 0; j < J; ++j) dist[j] = vals[j][0];  // result j sits at placement j
  for (int i = L - r - 1; i >= 0; --i) {
    lg.steps.emplace_back();
    auto& st = lg.steps.back();
    for (int k = N[i] - h[i]; k < N[i]; ++k) {
      int from = k - h[i];
      dist[k] = dist[from];
      for (int a = 0; a < P; ++a) {
        int v = dist[from][a];
        st.push_back({K_COPY, holder(a, from), holder(a, k), a, v, -1, v});
      }
    }
  }
}

// ----------------------------------------------------------------------------
// spec validation
// ----------------------------------------------------------------------------
bool validate_spec(const Spec& s, std::string* err) {
  auto fail = [&](const std::string& m) { if (err) *err = m; return false; };
  if (s.P < 1 || s.P > kMaxRanks) return fail("P must be in [1, 256]");
  if (s.n < 0) return fail("n must be >= 0");
  if (s.batch < 1) return fail("batch must be >= 1");
  if (s.n > 0 && s.batch > (int64_t(1) << 40) / s.n) return fail("batch * n is too large");
  if (s.dtype < D_INT32 || s.dtype > D_BF16) return fail("unknown dtype");
  if (s.op < O_SUM || s.op > O_AVG) return fail("unknown op");
  if (s.op == O_AVG && s.dtype == D_INT32) return fail("avg is defined for fp32 and bf16 only");
  if (s.coll < C_ALLREDUCE || s.coll > C_ALL_GATHER) return fail("unknown collective");
  if (s.algo < 0 || s.algo >= A_NUM_ALGOS) return fail("unknown algorithm");
  int L = ceil_log2(s.P);
  if (s.steps != 0) {
    if (s.algo != A_GENERALIZED) return fail("steps applies to the generalized algorithm over the cyclic group");
    if (s.steps < L || s.steps > std::max(L, s.P - 1))
      return fail("steps must be in [ceil(log2 P), P - 1] (0: ceil(log2 P))");
    L = s.steps;
  }
  if (s.algo == A_GENERALIZED || s.algo == A_GENERALIZED_XOR) {
    if (s.knob < 0 || s.knob > L) return fail("knob r must be in [0, reduction steps]");
    if (s.algo == A_GENERALIZED_XOR && (s.P & (s.P - 1))) return fail("the XOR group needs P to be a power of two");
  }
  if (s.algo == A_CHAIN && (s.knob < 1 || s.knob > kMaxChainPieces))
    return fail("the chain's knob m (pieces) must be in [1, 4096]");
  if (s.coll != C_ALLREDUCE) {
    if (!half_supported(s.algo))
      return fail("reduce-scatter / all-gather support direct, ring, rh_rd, generalized and generalized_xor");
    if (s.algo == A_RH_RD && (s.P & (s.P - 1))) return fail("the halving / doubling half needs P to be a power of two");
    if ((s.algo == A_GENERALIZED || s.algo == A_GENERALIZED_XOR) && s.knob != 0)
      return fail("the generalized halves use knob r = 0");
  }
  if (s.algo == A_GENERALIZED && !s.groups.empty()) {
    int64_t prod = 1;
    for (int m : s.groups) {
      if (m < 2) return fail("group factors must be >= 2");
      prod *= m;
      if (prod > kMaxRanks) break;
    }
    if (prod != s.P) return fail("the group factors' product must be P");
  }
  if (s.algo != A_AHC && s.algo != A_GENERALIZED && !s.groups.empty())
    return fail("groups apply to AR_AHC (group sizes) and AR_GENERALIZED (group factors) only");
  if (s.algo == A_AHC) {
    if (s.groups.empty()) return fail("AHC needs group sizes");
    int sum = 0;
    for (int g : s.groups) {
      if (g < 1) return fail("AHC group sizes must be >= 1");
      sum += g;
    }
    if (sum != s.P) return fail("AHC group sizes must sum to P");
    int64_t C = lcm_of(s.groups) * int64_t(s.groups.size());
    if (C > 65536) return fail("AHC needs lcm(groups) * G <= 65536 chunks");
  }
  return true;
}

// ----------------------------------------------------------------------------
// realizer: logical ops -> slot table with snapshot semantics
// ----------------------------------------------------------------------------
static inline uint64_t ckey(int cell, int val) { return (uint64_t(uint32_t(cell)) << 32) | uint32_t(val); }

// What a rank's buffer must hold at the end, per part: a complete reduction
// (Allreduce everywhere; reduce-scatter at the part's owner), anything
// (reduce-scatter elsewhere), or the owner's own value (all-gather: the leaf).
constexpr int kNeedComplete = -2, kDontCare = -1;
static int target_of(int coll, int rank, int part) {
  if (coll == C_ALLREDUCE) return kNeedComplete;
  if (coll == C_REDUCE_SCATTER) return rank == part ? kNeedComplete : kDontCare;
  return part;
}

struct Realizer {
  const Spec& sp;
  Exprs& ex;
  const Logical& lg;
  int P, C;
  std::vector<std::vector<std::pair<int, int>>> cell;  // (slot, value)
  std::unordered_map<uint64_t, int> last_read;
  std::vector<int> final_val;
  int nslots = 1;
  std::string err;

  Realizer(const Spec& s, Exprs& e, const Logical& l) : sp(s), ex(e), lg(l), P(s.P), C(l.C) {}

  int slot_of(int c, int v) const {
    for (auto& sv : cell[c]) if (sv.second == v) return sv.first;
    return -1;
  }
  int value_at(int c, int slot) const {
    for (auto& sv : cell[c]) if (sv.first == slot) return sv.second;
    return -1;
  }
  void put(int c, int slot, int v) {
    for (auto& sv : cell[c]) if (sv.first == slot) { sv.second = v; return; }
    cell[c].push_back({slot, v});
  }

  bool run(std::vector<LOp>& flat, std::vector<int>& step_of, std::vector<int>& ssl,
           std::vector<int>& osl, std::vector<int>& dsl, std::vector<int>& pair) {
    cell.assign(size_t(P) * C, {});
    for (int p = 0; p < P; ++p)
      for (int a = 0; a < C; ++a) cell[size_t(p) * C + a].push_back({0, p});
    // liveness and finals
    std::vector<std::vector<int>> present(size_t(P) * C);
    for (int p = 0; p < P; ++p)
      for (int a = 0; a < C; ++a) present[size_t(p) * C + a].push_back(p);
    for (size_t s = 0; s < lg.steps.size(); ++s)
      for (auto& o : lg.steps[s]) {
        last_read[ckey(o.src * C + o.atom, o.src_val)] = int(s);
        if (o.kind == K_REDUCE) last_read[ckey(o.dst * C + o.atom, o.own_val)] = int(s);
        present[size_t(o.dst) * C + o.atom].push_back(o.out_val);
      }
    if (sp.coll != C_ALLREDUCE && C != P) { err = "a half needs one atom per part"; return false; }
    final_val.assign(size_t(P) * C, -1);
    for (size_t c = 0; c < present.size(); ++c) {
      const int tgt = target_of(sp.coll, int(c / C), int(c % C));
      if (tgt == kDontCare) continue;
      if (tgt >= 0) {  // an owner's own value, copied
        if (std::find(present[c].begin(), present[c].end(), tgt) == present[c].end()) {
          err = "a rank ends without an owner's part";
          return false;
        }
        final_val[c] = tgt;
        continue;
      }
      int fv = -1;
      for (int v : present[c]) {
        if (!ex.complete(v)) continue;
        if (fv >= 0 && fv != v) { err = "two different complete results at one cell"; return false; }
        fv = v;
      }
      if (fv < 0 && P > 1) { err = "a rank ends without the complete result"; return false; }
      final_val[c] = fv < 0 ? int(c / C) : fv;
    }
    const bool bf16 = sp.dtype == D_BF16;
    for (size_t s = 0; s < lg.steps.size(); ++s) {
      const auto& st = lg.steps[s];
      size_t base = flat.size();
      std::unordered_map<uint64_t, std::vector<int>> readers;
      std::map<std::tuple<int, int, int>, int> by_link;  // (src, dst, atom) -> op
      for (size_t i = 0; i < st.size(); ++i) {
        const LOp& o = st[i];
        readers[ckey(o.src * C + o.atom, o.src_val)].push_back(int(i));
        if (o.kind == K_REDUCE) readers[ckey(o.dst * C + o.atom, o.own_val)].push_back(int(i));
        if (o.kind == K_REDUCE) by_link[{o.src, o.dst, o.atom}] = int(i);
      }
      std::vector<int> partner(st.size(), -1);
      for (size_t i = 0; i < st.size(); ++i) {
        const LOp& o = st[i];
        if (o.kind != K_REDUCE) continue;
        auto it = by_link.find({o.dst, o.src, o.atom});
        if (it == by_link.end()) continue;
        const LOp& q = st[it->second];
        if (q.own_val == o.src_val && q.src_val == o.own_val) partner[i] = it->second;
      }
      std::unordered_set<uint64_t> written;
      std::vector<int> jointly(st.size(), 0);
      for (size_t i = 0; i < st.size(); ++i) {
        const LOp& o = st[i];
        int sc = o.src * C + o.atom, dc = o.dst * C + o.atom;
        int s_sl = slot_of(sc, o.src_val);
        int o_sl = o.kind == K_REDUCE ? slot_of(dc, o.own_val) : -1;
        if (s_sl < 0 || (o.kind == K_REDUCE && o_sl < 0)) { err = "operand not present (generator bug)"; return false; }
        if (slot_of(dc, o.out_val) >= 0) { err = "destination already holds the value"; return false; }
        bool used_pair = false;
        auto ok = [&](int sl) {
          used_pair = false;
          if (bf16 && sl == 0 && !ex.complete(o.out_val) && !ex.is_leaf(o.out_val)) return false;
          if (written.count(ckey(dc, sl))) return false;
          int v = value_at(dc, sl);
          if (v < 0) return true;
          if (v == final_val[dc]) return false;
          auto it = last_read.find(ckey(dc, v));
          int lr = it == last_read.end() ? -1 : it->second;
          if (lr > int(s)) return false;
          if (lr == int(s)) {
            for (int rd : readers[ckey(dc, v)]) {
              if (rd == int(i)) continue;
              if (rd == partner[i]) { used_pair = true; continue; }
              return false;
            }
          }
          return true;
        };
        int chosen = -1;
        std::vector<int> cand;
        if (o.out_val == final_val[dc]) cand.push_back(0);
        if (o_sl >= 0) cand.push_back(o_sl);
        for (int sl = 0; sl < 64; ++sl) cand.push_back(sl);
        bool pairx = false;
        for (int sl : cand) if (ok(sl)) { chosen = sl; pairx = used_pair; break; }
        if (chosen < 0) { err = "no free slot"; return false; }
        written.insert(ckey(dc, chosen));
        nslots = std::max(nslots, chosen + 1);
        if (pairx) { jointly[i] = 1; jointly[partner[i]] = 1; }
        flat.push_back(o);
        step_of.push_back(int(s));
        ssl.push_back(s_sl);
        osl.push_back(o_sl);
        dsl.push_back(chosen);
        pair.push_back(-1);
      }
      for (size_t i = 0; i < st.size(); ++i)
        if (jointly[i]) pair[base + i] = int(base) + partner[i];
      for (size_t i = 0; i < st.size(); ++i) put(st[i].dst * C + st[i].atom, dsl[base + i], st[i].out_val);
    }
    return true;
  }
};

// ----------------------------------------------------------------------------
// table checker (any table, including corrupted ones)
// ----------------------------------------------------------------------------
TableCheck check_table(int P, int64_t n, int dtype, const OpRec* ops, size_t count, int coll) {
  TableCheck tc;
  auto fail = [&](const std::string& m) { tc.ok = false; tc.message = m; return tc; };
  if (P < 1 || P > kMaxRanks) return fail("bad P");
  int nslots = 1;
  for (size_t i = 0; i < count; ++i) {
    const OpRec& o = ops[i];
    if (o.kind < K_REDUCE || o.kind > K_MOVE) return fail("bad kind at op " + std::to_string(i));
    if (o.src_rank < 0 || o.src_rank >= P || o.dst_rank < 0 || o.dst_rank >= P) return fail("bad rank at op " + std::to_string(i));
    if (o.src_slot < 0 || o.dst_slot < 0 || o.src_slot > 63 || o.dst_slot > 63) return fail("bad slot at op " + std::to_string(i));
    if (o.kind == K_REDUCE && (o.own_slot < 0 || o.own_slot > 63)) return fail("bad own slot at op " + std::to_string(i));
    if (o.offset < 0 || o.length < 0 || o.offset + o.length > n) return fail("range outside the buffer at op " + std::to_string(i));
    if ((o.kind == K_MOVE) != (o.src_rank == o.dst_rank)) return fail("only a MOVE stays on one rank (op " + std::to_string(i) + ")");
    if (i && o.step < ops[i - 1].step) return fail("ops not sorted by step");
    if (o.pair >= 0 && (size_t(o.pair) >= count || ops[o.pair].pair != int32_t(i) || ops[o.pair].step != o.step))
      return fail("inconsistent pair at op " + std::to_string(i));
    nslots = std::max({nslots, o.src_slot + 1, o.dst_slot + 1, o.own_slot + 1});
  }
  tc.nslots = nslots;
  // hazards per step
  size_t i0 = 0;
  while (i0 < count) {
    size_t i1 = i0;
    while (i1 < count && ops[i1].step == ops[i0].step) ++i1;
    struct Iv { int64_t lo, hi; int grp; bool w; };
    std::map<std::pair<int, int>, std::vector<Iv>> acc;
    std::map<int, std::set<int>> dests, srcs;
    for (size_t i = i0; i < i1; ++i) {
      const OpRec& o = ops[i];
      if (o.length == 0) continue;
      int grp = o.pair >= 0 ? std::min<int>(int(i), o.pair) : int(i);
      acc[{o.src_rank, o.src_slot}].push_back({o.offset, o.offset + o.length, grp, false});
      if (o.kind == K_REDUCE) acc[{o.dst_rank, o.own_slot}].push_back({o.offset, o.offset + o.length, grp, false});
      acc[{o.dst_rank, o.dst_slot}].push_back({o.offset, o.offset + o.length, grp, true});
      if (o.kind != K_MOVE) { dests[o.src_rank].insert(o.dst_rank); srcs[o.dst_rank].insert(o.src_rank); }
    }
    for (auto& kv : acc) {
      auto& v = kv.second;
      std::sort(v.begin(), v.end(), [](const Iv& a, const Iv& b) { return a.lo < b.lo; });
      for (size_t a = 0; a < v.size(); ++a)
        for (size_t b = a + 1; b < v.size() && v[b].lo < v[a].hi; ++b) {
          if (v[a].grp == v[b].grp) continue;
          if (v[a].w || v[b].w) {
            std::ostringstream m;
            m << "step " << ops[i0].step << ": " << (v[a].w && v[b].w ? "two writes" : "a write and a read")
              << " of rank " << kv.first.first << " slot " << kv.first.second << " overlap";
            return fail(m.str());
          }
        }
    }
    for (auto& kv : dests) if (kv.second.size() > 1) tc.single_port = false;
    for (auto& kv : srcs) if (kv.second.size() > 1) tc.single_port = false;
    i0 = i1;
  }
  // symbolic replay over elementary intervals (cut at part boundaries too:
  // a half's targets change from part to part)
  if (coll < C_ALLREDUCE || coll > C_ALL_GATHER) return fail("unknown collective");
  const int64_t part = (n + P - 1) / P;
  std::vector<int64_t> cuts = {0, n};
  for (size_t i = 0; i < count; ++i) { cuts.push_back(ops[i].offset); cuts.push_back(ops[i].offset + ops[i].length); }
  if (coll != C_ALLREDUCE)
    for (int q = 1; q < P; ++q) cuts.push_back(std::min<int64_t>(q * part, n));
  std::sort(cuts.begin(), cuts.end());
  cuts.erase(std::unique(cuts.begin(), cuts.end()), cuts.end());
  Exprs ex(P);
  for (size_t q = 0; q + 1 < cuts.size(); ++q) {
    int64_t lo = cuts[q], hi = cuts[q + 1];
    if (hi <= lo) continue;
    std::vector<int> val(size_t(P) * nslots, -1);
    std::vector<char> rnd(size_t(P) * nslots, 0);
    for (int p = 0; p < P; ++p) val[size_t(p) * nslots] = p;
    size_t j0 = 0;
    while (j0 < count) {
      size_t j1 = j0;
      while (j1 < count && ops[j1].step == ops[j0].step) ++j1;
      std::vector<std::tuple<size_t, int, char>> upd;
      for (size_t j = j0; j < j1; ++j) {
        const OpRec& o = ops[j];
        if (o.offset > lo || o.offset + o.length < hi) {
          if (o.offset < hi && o.offset + o.length > lo) return fail("op boundary inside an interval");
          continue;
        }
        size_t si = size_t(o.src_rank) * nslots + o.src_slot, di = size_t(o.dst_rank) * nslots + o.dst_slot;
        int sv = val[si];
        if (sv < 0) return fail("op " + std::to_string(j) + " reads an empty slot");
        int out;
        char r = rnd[si];
        if (o.kind == K_REDUCE) {
          size_t oi = size_t(o.dst_rank) * nslots + o.own_slot;
          int ov = val[oi];
          if (ov < 0) return fail("op " + std::to_string(j) + " reads an empty own slot");
          if (dtype == D_BF16 && (rnd[si] || rnd[oi])) return fail("a rounded bf16 value is combined again");
          out = ex.combine(ov, sv);
          r = 0;
        } else {
          out = sv;
        }
        if (dtype == D_BF16 && o.dst_slot == 0 && !ex.is_leaf(out)) {
          if (!ex.complete(out)) return fail("an incomplete bf16 partial is stored in the caller's buffer");
          r = 1;
        }
        upd.push_back({di, out, r});
      }
      for (auto& u : upd) { val[std::get<0>(u)] = std::get<1>(u); rnd[std::get<0>(u)] = std::get<2>(u); }
      j0 = j1;
    }
    const int owner = part > 0 ? int(lo / part) : 0;
    for (int p = 0; p < P; ++p) {
      int v = val[size_t(p) * nslots];
      const int tgt = target_of(coll, p, owner);
      if (P == 1 || tgt == kDontCare) continue;
      if (tgt >= 0 ? v != tgt : !ex.complete(v)) {
        std::ostringstream m;
        m << "rank " << p << (tgt >= 0 ? " does not hold the owner's part" : " does not hold the complete result")
          << " for elements [" << lo << ", " << hi << ")";
        return fail(m.str());
      }
    }
  }
  tc.ok = true;
  return tc;
}

// ----------------------------------------------------------------------------
// fused replay planner
// ----------------------------------------------------------------------------
static bool plan_fused(Schedule& s, std::string* err) {
  const int P = s.spec.P;
  const int S = s.nslots;
  s.prog.clear();
  s.ranges.clear();
  if (P == 1 || s.spec.n == 0) { s.fused_ok = true; return true; }
  std::vector<std::vector<int>> by_atom(s.C);
  // map element offsets back to atoms
  std::vector<int64_t> starts(s.C);
  for (int a = 0; a < s.C; ++a) starts[a] = s.atoms[a].first;
  for (size_t i = 0; i < s.ops.size(); ++i) {
    const OpRec& o = s.ops[i];
    if (o.length == 0) continue;
    // atoms tile [0, n) in order; find the first atom starting at the op's offset
    int a = int(std::lower_bound(starts.begin(), starts.end(), o.offset) - starts.begin());
    for (; a < s.C && s.atoms[a].first < o.offset + o.length; ++a) {
      if (s.atoms[a].second <= s.atoms[a].first) continue;
      if (s.atoms[a].first >= o.offset && s.atoms[a].second <= o.offset + o.length) by_atom[a].push_back(int(i));
    }
  }
  Exprs ex(P);
  std::unordered_map<int, int> need_memo;
  std::function<int(int)> need = [&](int id) -> int {
    if (ex.is_leaf(id)) return 1;
    auto it = need_memo.find(id);
    if (it != need_memo.end()) return it->second;
    int a = need(ex.left(id)), b = need(ex.right(id));
    int r = a == b ? a + 1 : std::max(a, b);
    need_memo[id] = r;
    return r;
  };
  std::vector<int32_t> last_words;
  for (int a = 0; a < s.C; ++a) {
    int64_t lo = s.atoms[a].first, hi = s.atoms[a].second;
    if (hi <= lo) continue;
    std::vector<int> val(size_t(P) * S, -1);
    std::vector<char> rnd(size_t(P) * S, 0);
    for (int p = 0; p < P; ++p) val[size_t(p) * S] = p;
    const auto& lst = by_atom[a];
    size_t j0 = 0;
    while (j0 < lst.size()) {
      size_t j1 = j0;
      while (j1 < lst.size() && s.ops[lst[j1]].step == s.ops[lst[j0]].step) ++j1;
      std::vector<std::tuple<size_t, int, char>> upd;
      for (size_t j = j0; j < j1; ++j) {
        const OpRec& o = s.ops[lst[j]];
        size_t si = size_t(o.src_rank) * S + o.src_slot, di = size_t(o.dst_rank) * S + o.dst_slot;
        int out = val[si];
        char r = rnd[si];
        if (o.kind == K_REDUCE) {
          size_t oi = size_t(o.dst_rank) * S + o.own_slot;
          if (rnd[si] || rnd[oi]) { *err = "a rounded value is combined again"; return false; }
          out = ex.combine(val[oi], val[si]);
          r = 0;
        }
        if (s.spec.dtype == D_BF16 && o.dst_slot == 0 && !ex.is_leaf(out)) r = 1;
        upd.push_back({di, out, r});
      }
      for (auto& u : upd) { val[std::get<0>(u)] = std::get<1>(u); rnd[std::get<0>(u)] = std::get<2>(u); }
      j0 = j1;
    }
    // distinct final trees and their output ranks
    std::vector<int> roots;
    std::vector<std::vector<int>> outs;
    for (int p = 0; p < P; ++p) {
      int v = val[size_t(p) * S];
      const int tgt = target_of(s.spec.coll, p, a);
      if (tgt == kDontCare) continue;
      if (tgt >= 0 ? v != tgt : !ex.complete(v)) { *err = "fused planner: incomplete result"; return false; }
      if (v == p) continue;  // the rank keeps its own value
      auto it = std::find(roots.begin(), roots.end(), v);
      if (it == roots.end()) { roots.push_back(v); outs.push_back({p}); }
      else outs[it - roots.begin()].push_back(p);
    }
    if (roots.empty()) continue;  // nothing to write in this atom
    std::vector<int32_t> words;
    words.push_back(int32_t(roots.size()));
    int range_need = 0;
    for (size_t t = 0; t < roots.size(); ++t) {
      // postfix, deeper-need child first (Sethi-Ullman order keeps the stack at need(root))
      std::vector<int> leaves, ncomb;
      std::vector<std::pair<int, int>> stack = {{roots[t], 0}};
      while (!stack.empty()) {
        auto [id, state] = stack.back();
        stack.pop_back();
        if (ex.is_leaf(id)) { leaves.push_back(id); ncomb.push_back(0); continue; }
        if (state == 0) {
          int l = ex.left(id), r = ex.right(id);
          int first = need(l) >= need(r) ? l : r, second = first == l ? r : l;
          stack.push_back({id, 1});
          stack.push_back({second, 0});
          stack.push_back({first, 0});
        } else {
          ncomb.back() += 1;
        }
      }
      int nd = need(roots[t]);
      range_need = std::max(range_need, nd);
      words.push_back(int32_t(leaves.size()));
      words.push_back(int32_t(outs[t].size()));
      for (int v : leaves) words.push_back(v);
      for (int v : ncomb) words.push_back(v);
      for (int v : outs[t]) words.push_back(v);
      s.max_leaves = std::max<int>(s.max_leaves, int(leaves.size()));
    }
    s.max_trees = std::max<int>(s.max_trees, int(roots.size()));
    s.max_need = std::max(s.max_need, range_need);
    if (!s.ranges.empty() && s.ranges.back().start + s.ranges.back().len == lo && words == last_words) {
      s.ranges.back().len += hi - lo;
    } else {
      FusedRange fr;
      fr.start = lo;
      fr.len = hi - lo;
      fr.prog = int32_t(s.prog.size());
      fr.ntrees = int32_t(roots.size());
      fr.need = range_need;
      s.prog.insert(s.prog.end(), words.begin(), words.end());
      s.ranges.push_back(fr);
      last_words = words;
    }
  }
  s.fused_ok = true;
  return true;
}

// ----------------------------------------------------------------------------
// DAG form of a range's program
// ----------------------------------------------------------------------------
std::vector<int32_t> DagProgram::words() const {
  std::vector<int32_t> w = {S, int32_t(leaves.size()), int32_t(level_start.size()) - 1, int32_t(instr.size()),
                            int32_t(outs.size())};
  w.insert(w.end(), leaves.begin(), leaves.end());
  w.insert(w.end(), level_start.begin(), level_start.end());
  for (uint32_t i : instr) w.push_back(int32_t(i));
  w.insert(w.end(), outs.begin(), outs.end());
  return w;
}

bool compile_dag(const int32_t* w, int P, DagProgram* out, std::string* err) {
  // nodes: leaves first (by first appearance), then combinations in creation order
  struct Node { int a, b, level; };
  std::vector<Node> nodes;
  std::vector<int> leaf_node(size_t(P), -1);
  std::unordered_map<uint64_t, int> ids;
  std::vector<std::pair<int, int>> roots;  // (node, output rank)
  out->leaves.clear();
  const int ntrees = w[0];
  const int32_t* t = w + 1;
  // leaf nodes get their ids in a first pass, so leaf k is node k and slot k
  for (int q = 0, off = 0; q < ntrees; ++q) {
    const int nl = t[off], no = t[off + 1];
    for (int k = 0; k < nl; ++k) {
      const int r = t[off + 2 + k];
      if (r < 0 || r >= P) { *err = "leaf rank out of range"; return false; }
      if (leaf_node[size_t(r)] < 0) {
        leaf_node[size_t(r)] = int(nodes.size());
        nodes.push_back({-1, -1, 0});
        out->leaves.push_back(r);
      }
    }
    off += 2 + 2 * nl + no;
  }
  const int nleaf = int(nodes.size());
  for (int q = 0; q < ntrees; ++q) {
    const int nl = t[0], no = t[1];
    const int32_t* leaf = t + 2;
    const int32_t* nc = leaf + nl;
    const int32_t* os = nc + nl;
    std::vector<int> st;
    for (int k = 0; k < nl; ++k) {
      st.push_back(leaf_node[size_t(leaf[k])]);
      for (int c = 0; c < nc[k]; ++c) {
        if (st.size() < 2) { *err = "malformed postfix program"; return false; }
        const int b = st.back();
        st.pop_back();
        const int a = st.back();
        st.pop_back();
        const uint64_t key = (uint64_t(uint32_t(std::min(a, b))) << 32) | uint32_t(std::max(a, b));
        auto it = ids.find(key);
        int id;
        if (it != ids.end()) {
          id = it->second;
        } else {
          id = int(nodes.size());
          nodes.push_back({a, b, 1 + std::max(nodes[size_t(a)].level, nodes[size_t(b)].level)});
          ids.emplace(key, id);
        }
        st.push_back(id);
      }
    }
    if (st.size() != 1) { *err = "malformed postfix program"; return false; }
    for (int j = 0; j < no; ++j) roots.push_back({st[0], os[j]});
    t = os + no;
  }
  // last level in which each node is read; outputs are read after every level
  int nlev = 0;
  for (const Node& nd : nodes) nlev = std::max(nlev, nd.level);
  std::vector<int> last(nodes.size(), 0);
  for (size_t i = size_t(nleaf); i < nodes.size(); ++i) {
    last[size_t(nodes[i].a)] = std::max(last[size_t(nodes[i].a)], nodes[i].level);
    last[size_t(nodes[i].b)] = std::max(last[size_t(nodes[i].b)], nodes[i].level);
  }
  for (auto& rt : roots) last[size_t(rt.first)] = nlev + 1;
  // by level, creation order within a level
  std::vector<std::vector<int>> by_level(size_t(nlev) + 1);
  for (size_t i = size_t(nleaf); i < nodes.size(); ++i) by_level[size_t(nodes[i].level)].push_back(int(i));
  // values whose last read is in level l (their slot is free from level l + 1),
  // and how many combinations of a level read each value
  std::vector<std::vector<int>> by_last(size_t(nlev) + 2);
  for (size_t i = 0; i < nodes.size(); ++i)
    if (last[i] <= nlev) by_last[size_t(last[i])].push_back(int(i));
  std::vector<int> readers(nodes.size(), 0);
  std::vector<char> taken(nodes.size(), 0);  // slot handed on to the combination that read it last
  std::vector<int> slot(nodes.size(), -1);
  std::set<int> pool;
  int S = nleaf;
  for (int i = 0; i < nleaf; ++i) slot[size_t(i)] = i;
  out->level_start.assign(1, 0);
  out->instr.clear();
  for (int l = 1; l <= nlev; ++l) {
    for (int id : by_last[size_t(l - 1)])
      if (!taken[size_t(id)]) pool.insert(slot[size_t(id)]);
    for (int id : by_level[size_t(l)]) {
      ++readers[size_t(nodes[size_t(id)].a)];
      ++readers[size_t(nodes[size_t(id)].b)];
    }
    for (int id : by_level[size_t(l)]) {
      const Node& nd = nodes[size_t(id)];
      int sl = -1;
      // an operand read for the last time, by this combination alone, passes its
      // slot on: the same lane reads both operands before it writes
      for (int op : {nd.a, nd.b}) {
        if (sl < 0 && last[size_t(op)] == l && readers[size_t(op)] == 1 && !taken[size_t(op)]) {
          taken[size_t(op)] = 1;
          sl = slot[size_t(op)];
        }
      }
      if (sl < 0) {
        if (!pool.empty()) {
          sl = *pool.begin();
          pool.erase(pool.begin());
        } else {
          sl = S++;
        }
      }
      slot[size_t(id)] = sl;
      out->instr.push_back(uint32_t(sl) | (uint32_t(slot[size_t(nd.a)]) << 10) | (uint32_t(slot[size_t(nd.b)]) << 20));
    }
    for (int id : by_level[size_t(l)]) {
      readers[size_t(nodes[size_t(id)].a)] = 0;
      readers[size_t(nodes[size_t(id)].b)] = 0;
    }
    out->level_start.push_back(int32_t(out->instr.size()));
  }
  if (S > kDagMaxSlots) { *err = "more than 1024 live values"; return false; }
  out->S = S;
  out->outs.clear();
  for (auto& rt : roots) out->outs.push_back(int32_t((slot[size_t(rt.first)] << 16) | rt.second));
  return true;
}

bool dag_renaming(const DagProgram& a, const DagProgram& b, int P, std::vector<int>* map) {
  if (a.S != b.S || a.leaves.size() != b.leaves.size() || a.level_start != b.level_start || a.instr != b.instr ||
      a.outs.size() != b.outs.size())
    return false;
  map->assign(size_t(P), -1);
  std::vector<int> inv(size_t(P), -1);
  auto bind = [&](int x, int y) {
    int& m = (*map)[size_t(x)];
    if (m < 0 && inv[size_t(y)] < 0) {
      m = y;
      inv[size_t(y)] = x;
      return true;
    }
    return m == y;
  };
  for (size_t k = 0; k < a.leaves.size(); ++k)
    if (!bind(a.leaves[k], b.leaves[k])) return false;
  // outputs are a set of (slot, rank): a's, renamed, must be b's in any order
  std::vector<std::pair<int, int>> oa, ob;
  for (size_t k = 0; k < a.outs.size(); ++k) {
    const int ra = a.outs[k] & 0xffff;
    if ((*map)[size_t(ra)] < 0) {  // a rank that is no leaf: pair it with b's output of the same slot
      int y = -1;
      for (size_t j = 0; j < b.outs.size() && y < 0; ++j)
        if ((b.outs[j] >> 16) == (a.outs[k] >> 16) && inv[size_t(b.outs[j] & 0xffff)] < 0) y = b.outs[j] & 0xffff;
      if (y < 0 || !bind(ra, y)) return false;
    }
    oa.push_back({a.outs[k] >> 16, (*map)[size_t(ra)]});
    ob.push_back({b.outs[k] >> 16, b.outs[k] & 0xffff});
  }
  std::sort(oa.begin(), oa.end());
  std::sort(ob.begin(), ob.end());
  if (oa != ob) return false;
  // complete the permutation with the ranks neither program names
  int free_y = 0;
  for (int x = 0; x < P; ++x) {
    if ((*map)[size_t(x)] >= 0) continue;
    if (inv[size_t(x)] < 0) {
      (*map)[size_t(x)] = x;
      inv[size_t(x)] = x;
      continue;
    }
    while (inv[size_t(free_y)] >= 0) ++free_y;
    (*map)[size_t(x)] = free_y;
    inv[size_t(free_y)] = x;
  }
  return true;
}

bool dag_plan(const Schedule& s, DagPlan* out, std::string* err, bool allow_shared) {
  const int P = s.spec.P;
  const size_t R = s.ranges.size();
  std::vector<DagProgram> progs(R);
  *out = DagPlan{};
  for (size_t r = 0; r < R; ++r) {
    if (!compile_dag(s.prog.data() + s.ranges[r].prog, P, &progs[r], err)) return false;
    out->S = std::max(out->S, progs[r].S);
    out->levels = std::max(out->levels, int(progs[r].level_start.size()) - 1);
    out->instr = std::max<int64_t>(out->instr, int64_t(progs[r].instr.size()));
  }
  out->offsets.assign(R, 0);
  if (R == 0) return true;
  // one program for every range when they differ only by a renaming of ranks
  out->shared = allow_shared;
  out->maps.assign(R * size_t(P), 0);
  std::vector<int> map;
  for (size_t r = 0; r < R && out->shared; ++r) {
    if (!dag_renaming(progs[0], progs[r], P, &map)) {
      out->shared = false;
      break;
    }
    for (int x = 0; x < P; ++x) out->maps[r * size_t(P) + size_t(x)] = uint8_t(map[size_t(x)]);
  }
  if (out->shared) {
    out->words = progs[0].words();
    return true;
  }
  out->maps.clear();
  for (size_t r = 0; r < R; ++r) {
    out->offsets[r] = int32_t(out->words.size());
    const std::vector<int32_t> w = progs[r].words();
    out->words.insert(out->words.end(), w.begin(), w.end());
  }
  return true;
}

// ----------------------------------------------------------------------------
// build
// ----------------------------------------------------------------------------
// Radices of the generalized algorithm's group: the caller's factors, else
// Z_P (cyclic) or Z_2^L (self-inverse).
static std::vector<int> radices_of(const Spec& s) {
  if (s.algo == A_GENERALIZED_XOR) return std::vector<int>(size_t(ceil_log2(s.P)), 2);
  if (!s.groups.empty()) return s.groups;
  return {s.P};
}

bool half_supported(int algo) {
  return algo == A_DIRECT || algo == A_RING || algo == A_RH_RD || algo == A_GENERALIZED || algo == A_GENERALIZED_XOR;
}

static bool generate(const Spec& spec, Exprs& ex, Logical& lg, std::string* err) {
  const int P = spec.P;
  if (P <= 1) return true;
  if (spec.coll != C_ALLREDUCE) {
    const bool rs = spec.coll == C_REDUCE_SCATTER;
    switch (spec.algo) {
      case A_DIRECT: rs ? gen_direct_rs(P, ex, lg) : gen_direct_ag(P, ex, lg); break;
      case A_RING: rs ? gen_ring_rs(P, ex, lg) : gen_ring_ag(P, ex, lg); break;
      case A_RH_RD: rs ? gen_halving_rs(P, ex, lg) : gen_doubling_ag(P, ex, lg); break;
      case A_GENERALIZED: gen_generalized(P, 0, radices_of(spec), ex, lg, spec.coll, spec.steps); break;
      case A_GENERALIZED_XOR: gen_generalized(P, 0, radices_of(spec), ex, lg, spec.coll); break;
      default: if (err) *err = "no reduce-scatter / all-gather half for this algorithm"; return false;
    }
    return true;
  }
  switch (spec.algo) {
    case A_DIRECT: gen_direct(P, ex, lg); break;
    case A_RING: gen_ring(P, ex, lg); break;
    case A_RH_RD: gen_rh_rd(P, ex, lg); break;
    case A_RD: gen_rd(P, ex, lg); break;
    case A_BINOMIAL: gen_binomial(P, ex, lg); break;
    case A_GENERALIZED: gen_generalized(P, spec.knob, radices_of(spec), ex, lg, C_ALLREDUCE, spec.steps); break;
    case A_GENERALIZED_XOR: gen_generalized(P, spec.knob, radices_of(spec), ex, lg); break;
    case A_AHC: gen_ahc(P, spec.groups, ex, lg); break;
    case A_CHAIN: gen_chain(P, spec.knob, ex, lg); break;
    default: if (err) *err = "unknown algorithm"; return false;
  }
  return true;
}

Schedule* build_schedule(const Spec& spec, std::string* err) {
  if (is_auto(spec)) {
    if (err) *err = "resolve AR_AUTO / AR_KNOB_AUTO before building";
    return nullptr;
  }
  if (!validate_spec(spec, err)) return nullptr;
  const int P = spec.P;
  Exprs ex(P);
  Logical lg;
  if (!generate(spec, ex, lg, err)) return nullptr;
  auto s = std::make_unique<Schedule>();
  s->spec = spec;
  s->nsteps = int(lg.steps.size());
  s->C = lg.C;
  s->atoms = partition(spec.n, lg.C);
  std::vector<LOp> flat;
  std::vector<int> step_of, ssl, osl, dsl, pair;
  Realizer rz(spec, ex, lg);
  if (P > 1 && !rz.run(flat, step_of, ssl, osl, dsl, pair)) {
    if (err) *err = "schedule realization failed: " + rz.err;
    return nullptr;
  }
  s->nslots = rz.nslots;
  // export: merge consecutive atoms of identical unpaired ops, drop empty ranges
  std::vector<int> rec_of(flat.size(), -1);
  for (size_t i = 0; i < flat.size(); ++i) {
    const LOp& o = flat[i];
    int64_t lo = s->atoms[o.atom].first, hi = s->atoms[o.atom].second;
    if (hi <= lo) continue;
    if (pair[i] < 0 && !s->ops.empty() && i > 0 && rec_of[i - 1] == int(s->ops.size()) - 1) {
      OpRec& last = s->ops.back();
      const LOp& q = flat[i - 1];
      const bool same_completion = s->completes.back() == uint8_t(o.kind == K_REDUCE && ex.complete(o.out_val));
      if (last.pair < 0 && pair[i - 1] < 0 && last.step == step_of[i] && q.kind == o.kind && q.src == o.src &&
          q.dst == o.dst && q.atom + 1 == o.atom && last.src_slot == ssl[i] && last.dst_slot == dsl[i] &&
          last.own_slot == osl[i] && last.offset + last.length == lo && same_completion) {
        last.length += hi - lo;
        rec_of[i] = int(s->ops.size()) - 1;
        continue;
      }
    }
    OpRec r{step_of[i], o.kind, o.src, ssl[i], o.dst, dsl[i], osl[i], -1, lo, hi - lo};
    rec_of[i] = int(s->ops.size());
    s->ops.push_back(r);
    s->completes.push_back(uint8_t(o.kind == K_REDUCE && ex.complete(o.out_val)));
  }
  for (size_t i = 0; i < flat.size(); ++i)
    if (pair[i] >= 0 && rec_of[i] >= 0) s->ops[rec_of[i]].pair = rec_of[pair[i]];
  // finalize moves: bring each final value into slot 0
  if (P > 1) {
    for (int p = 0; p < P; ++p) {
      for (int a = 0; a < s->C; ++a) {
        int c = p * s->C + a;
        int sl = rz.slot_of(c, rz.final_val[c]);
        int64_t lo = s->atoms[a].first, hi = s->atoms[a].second;
        if (sl <= 0 || hi <= lo) continue;
        if (!s->ops.empty()) {
          OpRec& last = s->ops.back();
          if (last.kind == K_MOVE && last.src_rank == p && last.src_slot == sl && last.offset + last.length == lo) {
            last.length += hi - lo;
            continue;
          }
        }
        s->ops.push_back({s->nsteps, K_MOVE, p, sl, p, 0, -1, -1, lo, hi - lo});
        s->completes.push_back(0);
        s->finalize_ops++;
      }
    }
  }
  s->steps_begin.assign(s->nsteps + 2, int32_t(s->ops.size()));
  for (int st = s->nsteps + 1; st >= 0; --st) {
    // first op with step >= st
    auto it = std::lower_bound(s->ops.begin(), s->ops.end(), st,
                               [](const OpRec& o, int v) { return o.step < v; });
    s->steps_begin[st] = int32_t(it - s->ops.begin());
  }
  TableCheck tc = check_table(P, spec.n, spec.dtype, s->ops.data(), s->ops.size(), spec.coll);
  if (!tc.ok) {
    if (err) *err = "internal: generated table fails its check: " + tc.message;
    return nullptr;
  }
  s->single_port = tc.single_port;
  std::string ferr;
  if (!plan_fused(*s, &ferr)) {
    s->fused_ok = false;
    s->fused_error = ferr;
  }
  return s.release();
}

// ----------------------------------------------------------------------------
// cost walk
// ----------------------------------------------------------------------------
void cost_steps(const Schedule& s, int64_t* sent, int64_t* recv, int64_t* reduced) {
  // A message is what crosses a link: ops of one step that read the same source
  // range of one rank for the same destination rank carry the same data (one
  // received vector combined into two different partials), so it is counted once.
  const int P = s.spec.P;
  std::fill(sent, sent + size_t(s.nsteps) * P, 0);
  std::fill(recv, recv + size_t(s.nsteps) * P, 0);
  std::fill(reduced, reduced + size_t(s.nsteps) * P, 0);
  std::set<std::tuple<int, int, int, int, int64_t, int64_t>> msgs;
  for (const OpRec& o : s.ops) {
    if (o.kind == K_MOVE || o.step >= s.nsteps) continue;
    if (msgs.insert({o.step, o.src_rank, o.src_slot, o.dst_rank, o.offset, o.length}).second) {
      sent[size_t(o.step) * P + o.src_rank] += o.length;
      recv[size_t(o.step) * P + o.dst_rank] += o.length;
    }
    if (o.kind == K_REDUCE) reduced[size_t(o.step) * P + o.dst_rank] += o.length;
  }
}

static double closed_form(const Schedule& s, double m, double alpha, double beta, double gamma) {
  const int P = s.spec.P;
  if (P <= 1) return 0.0;
  if (s.spec.coll != C_ALLREDUCE) return std::numeric_limits<double>::quiet_NaN();  // pages: Allreduce only
  const int L = ceil_log2(P);
  const double u = m / P;
  const int Pp = pow2_floor(P);
  const int Lp = ceil_log2(Pp);
  const double fold = P == Pp ? 0.0 : 2 * alpha + 2 * m * beta + m * gamma;
  switch (s.spec.algo) {
    case A_DIRECT:  // root receives and sends (P-1) m one message per step
      return 2 * (P - 1) * (alpha + m * beta) + (P - 1) * m * gamma;
    case A_RING:  // eqs. (15)-(16)
      return 2 * (P - 1) * alpha + 2 * (P - 1) * u * beta + (P - 1) * u * gamma;
    case A_RH_RD: {
      double up = m / Pp;
      return fold + 2 * Lp * alpha + 2 * (Pp - 1) * up * beta + (Pp - 1) * up * gamma;
    }
    case A_RD:
      return fold + Lp * (alpha + m * beta + m * gamma);
    case A_BINOMIAL:
      return 2 * L * (alpha + m * beta) + L * m * gamma;
    case A_GENERALIZED:
    case A_GENERALIZED_XOR: {
      int r = s.spec.knob;
      if (s.spec.steps > L) {  // more steps: every part still moves once each way (r = 0 only)
        if (r != 0) return std::numeric_limits<double>::quiet_NaN();
        return 2 * s.spec.steps * alpha + 2 * (P - 1) * u * beta + (P - 1) * u * gamma;
      }
      if (r >= L)  // latency-optimal: all vectors each step; worst-case combinations (2L-2) m
        return L * alpha + L * m * beta + (2 * L - 2) * m * gamma;
      double extra = double((1 << r) - 1);
      return (2 * L - r) * alpha + (2 * (P - 1) + extra * L) * u * beta + ((P - 1) + extra * (2 * L - 2)) * u * gamma;
    }
    case A_CHAIN: {  // "Reduction Operator" page: (T_start + (n/m) T_byte)(p + m - 2), then the broadcast
      const int k = s.spec.knob;
      const double piece = m / k;
      return (P + k - 2) * (alpha + piece * (beta + gamma)) + (P + k - 2) * (alpha + piece * beta);
    }
    default:
      return std::numeric_limits<double>::quiet_NaN();  // AHC: the page's formula is truncated
  }
}

CostOut cost_walk(const Schedule& s, double alpha, double beta, double gamma) {
  CostOut c{};
  const int P = s.spec.P;
  const double elt = elt_bytes(s.spec.dtype);
  const double batch = double(s.spec.batch);
  c.steps = s.nsteps;
  std::vector<int64_t> sent(size_t(s.nsteps) * P), recv(size_t(s.nsteps) * P), red(size_t(s.nsteps) * P);
  if (s.nsteps) cost_steps(s, sent.data(), recv.data(), red.data());
  std::vector<int64_t> rank_sent(P, 0), rank_red(P, 0);
  double t = 0;
  int64_t xb = 0, xg = 0;
  for (int st = 0; st < s.nsteps; ++st) {
    int64_t ms = 0, mr = 0, md = 0;
    for (int p = 0; p < P; ++p) {
      int64_t a = sent[size_t(st) * P + p], b = recv[size_t(st) * P + p], d = red[size_t(st) * P + p];
      ms = std::max(ms, a);
      mr = std::max(mr, b);
      md = std::max(md, d);
      c.sent_total += a;
      c.reduced_total += d;
      rank_sent[p] += a;
      rank_red[p] += d;
    }
    c.sent_busiest += ms;
    c.recv_busiest += mr;
    c.reduced_busiest += md;
    xb += std::max(ms, mr);
    xg += md;
  }
  t = alpha * double(s.nsteps) + beta * (double(xb) * elt * batch) + gamma * (double(xg) * elt * batch);
  c.max_rank_sent = P ? *std::max_element(rank_sent.begin(), rank_sent.end()) : 0;
  c.max_rank_reduced = P ? *std::max_element(rank_red.begin(), rank_red.end()) : 0;
  c.predicted_seconds = t;
  double m = double(s.spec.n) * batch * elt;
  c.closed_form_seconds = closed_form(s, m, alpha, beta, gamma);
  // bytes through HBM
  auto sz = [&](int slot) { return slot == 0 ? elt : double(acc_bytes(s.spec.dtype)); };
  double lit = 0;
  for (size_t i = 0; i < s.ops.size(); ++i) {
    const OpRec& o = s.ops[i];
    double len = double(o.length) * batch;
    if (o.kind == K_REDUCE) {
      if (o.pair >= 0) {
        if (size_t(o.pair) < i) continue;  // the partner's bytes are counted with it
        const OpRec& q = s.ops[o.pair];
        lit += len * (sz(o.src_slot) + sz(o.own_slot) + sz(o.dst_slot) + sz(q.dst_slot));
      } else {
        lit += len * (sz(o.src_slot) + sz(o.own_slot) + sz(o.dst_slot));
      }
    } else {
      lit += len * (sz(o.src_slot) + sz(o.dst_slot));
    }
  }
  c.literal_hbm_bytes = lit;
  double fz = 0;
  for (const FusedRange& r : s.ranges) {
    const int32_t* w = s.prog.data() + r.prog;
    int nt = *w++;
    for (int t2 = 0; t2 < nt; ++t2) {
      int nl = w[0], no = w[1];
      fz += double(r.len) * batch * elt * (nl + no);
      w += 2 + 2 * nl + no;
    }
  }
  c.fused_hbm_bytes = fz;
  // every input read once and every output written once: P n in and P n out
  // (Allreduce); P n in and n out (reduce-scatter); n in and (P - 1) n out
  // (all-gather: each part read at its owner, written to the others)
  const double pn = double(P) * double(s.spec.n) * batch * elt, n1 = double(s.spec.n) * batch * elt;
  c.essential_bytes = s.spec.coll == C_ALLREDUCE ? 2.0 * pn : s.spec.coll == C_REDUCE_SCATTER ? pn + n1 : pn;
  return c;
}

// ----------------------------------------------------------------------------
// cost-only step counts and model-driven selection
// ----------------------------------------------------------------------------
bool is_auto(const Spec& s) {
  return s.algo == kAutoAlgo ||
         ((s.algo == A_GENERALIZED || s.algo == A_GENERALIZED_XOR || s.algo == A_CHAIN) && s.knob == kAutoKnob);
}

// Piece counts to try for the pipelined chain: the floor and ceiling of the
// optimum of (P + m - 2)(2 alpha + (M / m)(2 beta + gamma)), the reduce and the
// broadcast of the "Reduction Operator" page's pipelined time with T_start =
// alpha and T_byte = beta + gamma (beta only for the broadcast): m* =
// sqrt(M (P - 2)(2 beta + gamma) / (2 alpha)), M the bytes of one rank.
std::vector<int> chain_pieces(const Spec& s, const CostModel& m) {
  const int cap = int(std::min<int64_t>(kMaxChainPieces, std::max<int64_t>(1, s.n)));
  const double M = double(s.n) * double(elt_bytes(s.dtype)) * double(s.batch);
  double x;
  if (s.P <= 2) x = 0.0;
  else if (m.alpha > 0) x = std::sqrt(M * double(s.P - 2) * (2 * m.beta + m.gamma) / (2 * m.alpha));
  else x = double(cap);
  std::vector<int> out;
  for (double v : {std::floor(x), std::ceil(x)}) {
    int k = v < 1 ? 1 : v > cap ? cap : int(v);
    if (out.empty() || out.back() != k) out.push_back(k);
  }
  return out;
}

bool step_counts(const Spec& spec, StepCounts* out, std::string* err) {
  if (!validate_spec(spec, err)) return false;
  const int P = spec.P;
  *out = StepCounts{};
  if (spec.n == 0 || P <= 1) return true;  // nothing moves: no steps
  Exprs ex(P);
  Logical lg;
  if (!generate(spec, ex, lg, err)) return false;
  const auto atoms = partition(spec.n, lg.C);
  const int S = int(lg.steps.size());
  out->nsteps = S;
  out->sent.assign(size_t(S) * P, 0);
  out->recv.assign(size_t(S) * P, 0);
  out->reduced.assign(size_t(S) * P, 0);
  std::unordered_set<uint64_t> msgs;
  for (int st = 0; st < S; ++st) {
    msgs.clear();
    int64_t* sent = out->sent.data() + size_t(st) * P;
    int64_t* recv = out->recv.data() + size_t(st) * P;
    int64_t* red = out->reduced.data() + size_t(st) * P;
    for (const LOp& o : lg.steps[st]) {
      int64_t len = atoms[o.atom].second - atoms[o.atom].first;
      if (len <= 0) continue;
      // value ids fit 31 bits, ranks 8, atoms 17 (AHC: lcm * G <= 65536)
      uint64_t key = (uint64_t(uint32_t(o.src_val)) << 33) | (uint64_t(o.src) << 25) |
                     (uint64_t(o.dst) << 17) | uint64_t(o.atom);
      if (msgs.insert(key).second) {
        sent[o.src] += len;
        recv[o.dst] += len;
      }
      if (o.kind == K_REDUCE) red[o.dst] += len;
    }
  }
  return true;
}

double model_seconds(const StepCounts& c, const Spec& spec, const CostModel& m) {
  const int P = spec.P;
  int64_t xb = 0, xg = 0;
  for (int st = 0; st < c.nsteps; ++st) {
    const int64_t* sent = c.sent.data() + size_t(st) * P;
    const int64_t* recv = c.recv.data() + size_t(st) * P;
    const int64_t* red = c.reduced.data() + size_t(st) * P;
    if (m.form == F_BUSIEST) {
      int64_t mb = 0, mg = 0;
      for (int p = 0; p < P; ++p) {
        mb = std::max(mb, std::max(sent[p], recv[p]));
        mg = std::max(mg, red[p]);
      }
      xb += mb;
      xg += mg;
    } else {
      for (int p = 0; p < P; ++p) {
        xb += sent[p];
        xg += red[p];
      }
    }
  }
  const double elt = elt_bytes(spec.dtype);
  const double batch = double(spec.batch);
  return m.alpha * double(c.nsteps) + m.beta * (double(xb) * elt * batch) + m.gamma * (double(xg) * elt * batch);
}

bool select_spec(const Spec& in, const CostModel& m, Spec* out, double* seconds, std::string* err) {
  auto fail = [&](const std::string& msg) { if (err) *err = msg; return false; };
  if (!is_auto(in)) {
    *out = in;
    if (seconds) {
      StepCounts c;
      if (!step_counts(in, &c, err)) return false;
      *seconds = model_seconds(c, in, m);
    }
    return true;
  }
  if (!(std::isfinite(m.alpha) && std::isfinite(m.beta) && std::isfinite(m.gamma)) || m.alpha < 0 ||
      m.beta < 0 || m.gamma < 0)
    return fail("the cost model needs finite, non-negative alpha, beta, gamma");
  if (in.P < 1 || in.P > kMaxRanks) return fail("P must be in [1, 256]");
  const int L = ceil_log2(in.P);
  const bool pow2 = (in.P & (in.P - 1)) == 0;
  std::vector<std::pair<int, int>> cand;  // (algo, knob), in the order ties are broken
  if (in.algo == kAutoAlgo && in.coll != C_ALLREDUCE) {
    cand.push_back({A_DIRECT, 0});
    cand.push_back({A_RING, 0});
    if (pow2) cand.push_back({A_RH_RD, 0});
    cand.push_back({A_GENERALIZED, 0});
    if (pow2) cand.push_back({A_GENERALIZED_XOR, 0});
  } else if (in.algo == kAutoAlgo) {
    for (int a : {A_DIRECT, A_RING, A_RH_RD, A_RD, A_BINOMIAL}) cand.push_back({a, 0});
    for (int r = 0; r <= L; ++r) cand.push_back({A_GENERALIZED, r});
    if (pow2)
      for (int r = 0; r <= L; ++r) cand.push_back({A_GENERALIZED_XOR, r});
    if (!in.groups.empty()) cand.push_back({A_AHC, 0});
    for (int k : chain_pieces(in, m)) cand.push_back({A_CHAIN, k});
  } else if (in.algo == A_CHAIN) {
    for (int k : chain_pieces(in, m)) cand.push_back({A_CHAIN, k});
  } else {
    const int S = in.steps > 0 ? in.steps : L;
    for (int r = 0; r <= (in.coll == C_ALLREDUCE ? S : 0); ++r) cand.push_back({in.algo, r});
  }
  bool have = false;
  double best_t = 0;
  int best_steps = 0;
  Spec best;
  for (auto [a, r] : cand) {
    Spec c = in;
    c.algo = a;
    c.knob = r;
    if (in.algo == kAutoAlgo && a != A_AHC) c.groups.clear();  // AR_AUTO's groups are AHC's
    StepCounts sc;
    if (!step_counts(c, &sc, err)) return false;
    double t = model_seconds(sc, c, m);
    if (!have || t < best_t || (t == best_t && sc.nsteps < best_steps)) {
      have = true;
      best_t = t;
      best_steps = sc.nsteps;
      best = c;
    }
  }
  *out = best;
  if (seconds) *seconds = best_t;
  return true;
}

}  // namespace ar

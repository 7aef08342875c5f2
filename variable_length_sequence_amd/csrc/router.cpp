// The NSP planner (NSP page, Section 4.1): the SP tree of Definition 1, the
// per-GPU cost model of Section 4.1.2 and Algorithm 1 of Section 4.1.3.
//
// A search state holds, per GPU, the forward and backward stage times and the
// sharded token load, plus which tree nodes already carry a sample (a node's
// all-to-all latency is paid once however many samples it packs).  Beam
// expansion scores every (state, node) child without building it: a child
// differs from its parent only on the node's ranks, so its critical load
// max_p C_p and token peak max_p T_p are one pass over the parent's arrays;
// only the w survivors are materialised.
#include "router.h"

#include <algorithm>
#include <cmath>

namespace vl {

namespace {

double throughput(const std::vector<double>& xs, const std::vector<double>& ys, double L) {
  if (L <= xs[0]) return ys[0];
  for (size_t a = 0; a + 1 < xs.size(); ++a) {
    if (L <= xs[a + 1]) {
      const double t = (L - xs[a]) / (xs[a + 1] - xs[a]);
      return ys[a] + t * (ys[a + 1] - ys[a]);
    }
  }
  return ys.back();
}

// Per-GPU forward and backward time of one sample of length L on a node of
// degree s, without the node's latency: all-to-all volume (alpha-beta model,
// BASP page, Section IV), attention compute at the measured throughput for
// documents of length L, and non-attention work on the GPU's L/s tokens.
void sample_cost(const CostParams& cm, double L, int32_t s, double& f, double& b) {
  const double pairs = L * (L + 1) / 2;
  const double tok = L / s;
  const double beta = 1.0 / (cm.a2a_gbs * 1e9);
  double comm[4] = {0.0, 0.0, 0.0, 0.0};
  if (s > 1) {
    const double frac = double(s - 1) / s;
    for (int i = 0; i < 4; ++i) comm[i] = frac * (tok * cm.bytes_per_token[i]) * beta;
  }
  const double comp_f = cm.fwd_flops_per_pair * pairs / s /
                        (throughput(cm.curve_len, cm.fwd_tflops, L) * 1e12);
  const double comp_b = cm.bwd_flops_per_pair * pairs / s /
                        (throughput(cm.curve_len, cm.bwd_tflops, L) * 1e12);
  const double dense_f = tok * cm.dense_fwd_flops_per_token / (cm.dense_tflops * 1e12);
  const double dense_b = tok * cm.dense_bwd_flops_per_token / (cm.dense_tflops * 1e12);
  f = (comm[0] + comm[1]) + comp_f + dense_f;
  b = (comm[2] + comm[3]) + comp_b + dense_b;
}

// Latency of a non-empty node of degree s: two all-to-alls per pass.
double node_latency(const CostParams& cm, int32_t s) {
  return s == 1 ? 0.0 : double(2 * (s - 1)) * cm.a2a_alpha_us * 1e-6;
}

struct State {
  std::vector<double> dfwd, dbwd, tok;
  std::vector<uint8_t> used;            // per node
  std::vector<int32_t> plan;            // per sample (-1: not yet placed)
  int32_t cap = 1 << 30;                // largest degree the monotone rule allows
  double grp_len = -1.0;                // length of the current equal-length group
  int32_t grp_min = 1 << 30;            // smallest degree used in that group
};

double max_cost(const State& S) {
  double m = -INFINITY;
  for (size_t p = 0; p < S.tok.size(); ++p) m = std::max(m, S.dfwd[p] + S.dbwd[p]);
  return m;
}

double max_tok(const State& S) {
  double m = -INFINITY;
  for (double t : S.tok) m = std::max(m, t);
  return m;
}

// The increments a sample adds on each of the node's GPUs.
void increments(const State& S, const CostParams& cm, double L, const TreeNode& u, int32_t ui,
                double& f, double& b) {
  sample_cost(cm, L, u.count, f, b);
  if (!S.used[ui]) {
    const double lat = node_latency(cm, u.count);
    f = lat + f;
    b = lat + b;
  }
}

void apply(State& S, const CostParams& cm, int32_t j, double L, const TreeNode& u, int32_t ui) {
  double f, b;
  increments(S, cm, L, u, ui, f, b);
  S.used[ui] = 1;
  for (int32_t p = u.first; p < u.first + u.count; ++p) {
    S.dfwd[p] += f;
    S.dbwd[p] += b;
    S.tok[p] += L / u.count;
  }
  S.plan[j] = ui;
  if (L != S.grp_len) {
    S.cap = std::min(S.cap, S.grp_min);
    S.grp_len = L;
    S.grp_min = u.count;
  } else {
    S.grp_min = std::min(S.grp_min, u.count);
  }
}

bool allowed(const State& S, double L, int32_t s, bool monotone) {
  if (!monotone) return true;
  const int32_t cap = (L == S.grp_len) ? S.cap : std::min(S.cap, S.grp_min);
  return s <= cap;
}

struct Child {
  int32_t parent, node;
  double max_c, max_t;
};

}  // namespace

bool sp_tree(int32_t n_gpus, int32_t sp_max, int32_t level_mask, std::vector<TreeNode>& nodes,
             std::string& err) {
  if (sp_max < 1 || (sp_max & (sp_max - 1))) return err = "sp_max must be a power of two", false;
  if (n_gpus < 1 || n_gpus % sp_max) return err = "sp_max must divide n_gpus", false;
  int32_t K = 0;
  while ((1 << K) < sp_max) ++K;
  const int32_t trees = n_gpus / sp_max;
  nodes.clear();
  for (int32_t d = 0; d <= K; ++d) {
    if (!((uint32_t(level_mask) >> d) & 1u)) continue;
    const int32_t w = 1 << (K - d);
    for (int32_t i = 0; i < (trees << d); ++i) nodes.push_back(TreeNode{d, i, i * w, w});
  }
  if (nodes.empty()) return err = "level_mask enables no tree level", false;
  return true;
}

bool nsp_route(const std::vector<double>& lengths, int32_t n_gpus, int32_t sp_max,
               const CostParams& cm, double token_budget, int32_t prefix, int32_t beam,
               bool monotone, int32_t level_mask, std::vector<TreeNode>& nodes, RouteResult& out,
               std::string& err) {
  if (!sp_tree(n_gpus, sp_max, level_mask, nodes, err)) return false;
  if (beam < 1) return err = "beam must be >= 1", false;
  const int32_t M = int32_t(lengths.size());
  std::vector<int32_t> order(M);
  for (int32_t j = 0; j < M; ++j) order[j] = j;
  std::stable_sort(order.begin(), order.end(),
                   [&](int32_t a, int32_t b) { return lengths[a] > lengths[b]; });
  const int32_t k = std::max(0, std::min(prefix, M));
  const int32_t n_nodes = int32_t(nodes.size());

  State zero;
  zero.dfwd.assign(n_gpus, 0.0);
  zero.dbwd.assign(n_gpus, 0.0);
  zero.tok.assign(n_gpus, 0.0);
  zero.used.assign(n_nodes, 0);
  zero.plan.assign(M, -1);
  std::vector<State> Q{zero};

  // long-prefix search
  std::vector<Child> kids;
  for (int32_t step = 0; step < k; ++step) {
    const int32_t j = order[step];
    const double L = lengths[j];
    kids.clear();
    for (int32_t q = 0; q < int32_t(Q.size()); ++q) {
      const State& S = Q[q];
      for (int32_t ui = 0; ui < n_nodes; ++ui) {
        const TreeNode& u = nodes[ui];
        if (!allowed(S, L, u.count, monotone)) continue;
        double f, b;
        increments(S, cm, L, u, ui, f, b);
        double mc = -INFINITY, mt = -INFINITY;
        for (int32_t p = 0; p < n_gpus; ++p) {
          if (p >= u.first && p < u.first + u.count) {
            mc = std::max(mc, (S.dfwd[p] + f) + (S.dbwd[p] + b));
            mt = std::max(mt, S.tok[p] + L / u.count);
          } else {
            mc = std::max(mc, S.dfwd[p] + S.dbwd[p]);
            mt = std::max(mt, S.tok[p]);
          }
        }
        kids.push_back(Child{q, ui, mc, mt});
      }
    }
    std::vector<Child> ok;
    for (const Child& c : kids)
      if (c.max_t <= token_budget) ok.push_back(c);
    if (!ok.empty()) {
      std::stable_sort(ok.begin(), ok.end(),
                       [](const Child& a, const Child& b) { return a.max_c < b.max_c; });
    } else {
      ok = kids;
      std::stable_sort(ok.begin(), ok.end(),
                       [](const Child& a, const Child& b) { return a.max_t < b.max_t; });
    }
    if (int32_t(ok.size()) > beam) ok.resize(beam);
    std::vector<State> next;
    next.reserve(ok.size());
    for (const Child& c : ok) {
      next.push_back(Q[c.parent]);
      apply(next.back(), cm, j, L, nodes[c.node], c.node);
    }
    Q.swap(next);
  }

  // greedy short-tail completion on the deepest enabled level
  const int32_t deepest = nodes.back().depth;
  std::vector<int32_t> units;
  for (int32_t ui = 0; ui < n_nodes; ++ui)
    if (nodes[ui].depth == deepest) units.push_back(ui);
  int32_t best_state = -1;
  double best_c = 0.0;
  for (int32_t q = 0; q < int32_t(Q.size()); ++q) {
    State& S = Q[q];
    for (int32_t step = k; step < M; ++step) {
      const int32_t j = order[step];
      const double L = lengths[j];
      int32_t pick = -1;
      double pick_load = 0.0;
      for (int32_t ui : units) {
        const TreeNode& u = nodes[ui];
        double mt = -INFINITY, load = -INFINITY;
        for (int32_t p = u.first; p < u.first + u.count; ++p) {
          mt = std::max(mt, S.tok[p] + L / u.count);
          load = std::max(load, S.dfwd[p] + S.dbwd[p]);
        }
        if (mt <= token_budget && (pick < 0 || load < pick_load)) {
          pick = ui;
          pick_load = load;
        }
      }
      if (pick < 0) {
        for (int32_t ui : units) {
          const TreeNode& u = nodes[ui];
          double tl = -INFINITY;
          for (int32_t p = u.first; p < u.first + u.count; ++p) tl = std::max(tl, S.tok[p]);
          if (pick < 0 || tl < pick_load) {
            pick = ui;
            pick_load = tl;
          }
        }
      }
      apply(S, cm, j, L, nodes[pick], pick);
    }
    const double c = max_cost(S);
    if (best_state < 0 || c < best_c) {
      best_state = q;
      best_c = c;
    }
  }
  const State& F = Q[best_state];
  out.node = F.plan;
  out.dfwd = F.dfwd;
  out.dbwd = F.dbwd;
  out.tok = F.tok;
  out.within_budget = max_tok(F) <= token_budget;
  return true;
}

void nsp_plan_cost(const std::vector<double>& lengths, const std::vector<TreeNode>& nodes,
                   const std::vector<int32_t>& node_of, int32_t n_gpus, const CostParams& cm,
                   std::vector<double>& dfwd, std::vector<double>& dbwd, std::vector<double>& tok) {
  State S;
  S.dfwd.assign(n_gpus, 0.0);
  S.dbwd.assign(n_gpus, 0.0);
  S.tok.assign(n_gpus, 0.0);
  S.used.assign(nodes.size(), 0);
  S.plan.assign(lengths.size(), -1);
  for (size_t j = 0; j < lengths.size(); ++j)
    apply(S, cm, int32_t(j), lengths[j], nodes[node_of[j]], node_of[j]);
  dfwd = S.dfwd;
  dbwd = S.dbwd;
  tok = S.tok;
}

}  // namespace vl

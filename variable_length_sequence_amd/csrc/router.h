// The NSP planner on the host: SP tree, per-GPU cost model and the
// prefix-search / greedy-tail routing heuristic (NSP page, Section 4.1).
#pragma once
#include <stdint.h>

#include <string>
#include <vector>

namespace vl {

struct CostParams {
  std::vector<double> curve_len, fwd_tflops, bwd_tflops;
  double fwd_flops_per_pair, bwd_flops_per_pair;
  double bytes_per_token[4];   // fwd prologue, fwd epilogue, bwd prologue, bwd epilogue
  double a2a_gbs, a2a_alpha_us;
  double dense_fwd_flops_per_token, dense_bwd_flops_per_token, dense_tflops;
};

struct TreeNode {
  int32_t depth, index;
  int32_t first, count;   // rank range [first, first + count)
};

struct RouteResult {
  std::vector<int32_t> node;            // per sample: index into the node list
  std::vector<double> dfwd, dbwd, tok;  // per GPU
  bool within_budget;
};

// Nodes of the enabled levels, by depth then index (n_gpus / sp_max trees).
bool sp_tree(int32_t n_gpus, int32_t sp_max, int32_t level_mask, std::vector<TreeNode>& nodes,
             std::string& err);

bool nsp_route(const std::vector<double>& lengths, int32_t n_gpus, int32_t sp_max,
               const CostParams& cm, double token_budget, int32_t prefix, int32_t beam,
               bool monotone, int32_t level_mask, std::vector<TreeNode>& nodes, RouteResult& out,
               std::string& err);

// Per-GPU stage times and token loads of a given plan (samples applied in
// index order); node_of[j] indexes `nodes`.
void nsp_plan_cost(const std::vector<double>& lengths, const std::vector<TreeNode>& nodes,
                   const std::vector<int32_t>& node_of, int32_t n_gpus, const CostParams& cm,
                   std::vector<double>& dfwd, std::vector<double>& dbwd, std::vector<double>& tok);

}  // namespace vl

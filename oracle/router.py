"""The NSP planner on the CPU: the SP tree, the per-GPU cost model and the
prefix-search / greedy-tail routing heuristic.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

NSP page, Section 4.1.1 (Definition 1, Figure 4): with spmax = 2^K the SP tree
is a complete binary tree of nodes (d, i), 0 <= d <= K; node (d, i) stands for
the aligned rank range R = [i 2^(K-d), (i+1) 2^(K-d)), an SP group of degree
2^(K-d).  A GPU takes part in the nodes on its leaf-to-root chain.

Section 4.1.2: a plan maps every sample to one node.  GPU p's token load is
the sum of L_j / |R(a(j))| over the samples routed to nodes containing p; its
attention time per pass is the sum, over the active nodes on its chain, of the
node's prologue (communication), compute and epilogue (communication) costs;
non-attention time follows from its token load and a dense throughput; the
per-GPU summary C_p adds the forward and backward stage times, and the
iteration proxy is max_p D_p^fwd + max_p D_p^bwd.

Section 4.1.3 (Algorithm 1): sort the samples longest first; search the first
k with a beam of width w (each state extended by every feasible node, states
over the token budget dropped, the w with the smallest max_p C_p kept); then
complete each surviving state greedily by placing the remaining samples,
longest first, on the least-loaded leaf unit that keeps the budget (else the
unit with the smallest token load); return the completed state with the
smallest max_p C_p.  Optionally a longer sample may not use a smaller SP
degree than a shorter one (the monotone-SP constraint).

Readings where the page is silent (the cost model's shape is the page's; its
terms are this library's):
  * compute: a sample of length L routed to a node of degree s costs each of
    the node's GPUs F(L) / s FLOPs at the measured per-GPU throughput for
    documents of length L (piecewise linear between measured lengths, clamped
    outside), F(L) = flops_per_pair * L (L + 1) / 2 (causal), per pass;
  * communication: each phase of a node of degree s > 1 is one all-to-all of
    the node's samples, costed by the alpha-beta model of the BASP page
    (Section IV, footnote: (s - 1)(alpha + m beta), m the per-peer message),
    i.e. alpha (s - 1) + ((s - 1) / s) (bytes per GPU) / bandwidth, with bytes
    per GPU = sum_j (L_j / s) * bytes per token of that phase;
  * non-attention: token load x dense FLOPs per token / dense throughput;
  * "effective leaf units" are the nodes of the deepest enabled tree level;
  * if no prefix extension keeps the token budget, the w extensions with the
    smallest max_p T_p are kept and the plan is reported over budget;
  * ties keep the first state in generation order (nodes enumerated by depth,
    then index; states in beam order).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from itertools import product
from typing import List, Sequence, Tuple

PHASES = ("fwd_prologue", "fwd_epilogue", "bwd_prologue", "bwd_epilogue")


@dataclass
class CostModel:
    curve_len: Sequence[float]          # document lengths of the measured curve (increasing)
    fwd_tflops: Sequence[float]         # measured per-GPU forward TFLOP/s at those lengths
    bwd_tflops: Sequence[float]         # measured per-GPU backward TFLOP/s
    fwd_flops_per_pair: float           # useful FLOPs per visible pair, all heads, forward
    bwd_flops_per_pair: float
    bytes_per_token: Tuple[float, float, float, float]   # per phase, in PHASES order
    a2a_gbs: float                      # per-GPU all-to-all bandwidth, GB/s
    a2a_alpha_us: float                 # per-peer latency, microseconds
    dense_fwd_flops_per_token: float = 0.0
    dense_bwd_flops_per_token: float = 0.0
    dense_tflops: float = 1.0


def throughput(curve_len, tflops, L: float) -> float:
    """Piecewise-linear interpolation of the measured curve, clamped at its ends."""
    if L <= curve_len[0]:
        return tflops[0]
    for a in range(len(curve_len) - 1):
        x0, x1 = curve_len[a], curve_len[a + 1]
        if L <= x1:
            t = (L - x0) / (x1 - x0)
            return tflops[a] + t * (tflops[a + 1] - tflops[a])
    return tflops[-1]


# ---------------------------------------------------------------- the SP tree
def tree_nodes(n_gpus: int, sp_max: int, level_mask: int = -1) -> List[Tuple[int, int]]:
    """Nodes (d, i) of the enabled levels, by depth then index; several trees
    side by side when n_gpus is a multiple of sp_max."""
    K = sp_max.bit_length() - 1
    if sp_max < 1 or (1 << K) != sp_max or n_gpus % sp_max:
        raise ValueError("sp_max must be a power of two dividing n_gpus")
    trees = n_gpus // sp_max
    return [(d, i) for d in range(K + 1) if (level_mask >> d) & 1
            for i in range(trees << d)]


def rank_range(node, sp_max: int) -> range:
    d, i = node
    K = sp_max.bit_length() - 1
    w = 1 << (K - d)
    return range(i * w, (i + 1) * w)


# ---------------------------------------------------------------- cost model
def sample_costs(cm: CostModel, L: float, s: int):
    """Per-GPU (fwd, bwd) time of one sample on a node of degree s, without
    the per-node latency terms, as (comm_f, comp_f, dense_f, comm_b, comp_b, dense_b)."""
    pairs = L * (L + 1) / 2
    tok = L / s
    beta = 1.0 / (cm.a2a_gbs * 1e9)
    if s > 1:
        frac = (s - 1) / s
        comm = [frac * (tok * b) * beta for b in cm.bytes_per_token]
    else:
        comm = [0.0, 0.0, 0.0, 0.0]
    comp_f = cm.fwd_flops_per_pair * pairs / s / (throughput(cm.curve_len, cm.fwd_tflops, L) * 1e12)
    comp_b = cm.bwd_flops_per_pair * pairs / s / (throughput(cm.curve_len, cm.bwd_tflops, L) * 1e12)
    dense_f = tok * cm.dense_fwd_flops_per_token / (cm.dense_tflops * 1e12)
    dense_b = tok * cm.dense_bwd_flops_per_token / (cm.dense_tflops * 1e12)
    return comm[0] + comm[1], comp_f, dense_f, comm[2] + comm[3], comp_b, dense_b


def node_latency(cm: CostModel, s: int) -> Tuple[float, float]:
    """(fwd, bwd) latency of a non-empty node: two all-to-alls per pass."""
    if s == 1:
        return 0.0, 0.0
    a = 2 * (s - 1) * cm.a2a_alpha_us * 1e-6
    return a, a


def plan_cost(lengths, plan, n_gpus: int, sp_max: int, cm: CostModel):
    """Evaluate a complete plan from scratch (no incremental state).

    Returns (C [P], tokens [P], Dfwd [P], Dbwd [P], load)."""
    dfwd = [0.0] * n_gpus
    dbwd = [0.0] * n_gpus
    tok = [0.0] * n_gpus
    used = {}
    for j, node in enumerate(plan):
        used.setdefault(node, []).append(j)
    for node, js in used.items():
        ranks = rank_range(node, sp_max)
        s = len(ranks)
        lf, lb = node_latency(cm, s)
        f = lf
        b = lb
        for j in js:
            cf, pf, df, cb, pb, db = sample_costs(cm, float(lengths[j]), s)
            f += cf + pf + df
            b += cb + pb + db
        for p in ranks:
            dfwd[p] += f
            dbwd[p] += b
            for j in js:
                tok[p] += lengths[j] / s
    C = [dfwd[p] + dbwd[p] for p in range(n_gpus)]
    return C, tok, dfwd, dbwd, max(dfwd) + max(dbwd)


# ---------------------------------------------------------------- Algorithm 1
@dataclass
class State:
    plan: dict = field(default_factory=dict)       # sample index -> node
    dfwd: list = None
    dbwd: list = None
    tok: list = None
    used: set = field(default_factory=set)
    cap: int = 1 << 30        # largest degree allowed by the monotone constraint
    grp_len: float = -1.0     # length of the samples of the current equal-length group
    grp_min: int = 1 << 30    # smallest degree used in that group

    def copy(self):
        return State(dict(self.plan), list(self.dfwd), list(self.dbwd), list(self.tok),
                     set(self.used), self.cap, self.grp_len, self.grp_min)

    def maxC(self):
        return max(self.dfwd[p] + self.dbwd[p] for p in range(len(self.tok)))

    def maxT(self):
        return max(self.tok)


def _extend(S: State, j: int, L: float, node, sp_max: int, cm: CostModel) -> State:
    ranks = rank_range(node, sp_max)
    s = len(ranks)
    T = S.copy()
    cf, pf, df, cb, pb, db = sample_costs(cm, L, s)
    f = cf + pf + df
    b = cb + pb + db
    if node not in T.used:
        lf, lb = node_latency(cm, s)
        f = lf + f
        b = lb + b
        T.used.add(node)
    for p in ranks:
        T.dfwd[p] += f
        T.dbwd[p] += b
        T.tok[p] += L / s
    T.plan[j] = node
    # monotone bookkeeping: samples arrive longest first
    if L != T.grp_len:
        T.cap = min(T.cap, T.grp_min)
        T.grp_len, T.grp_min = L, s
    else:
        T.grp_min = min(T.grp_min, s)
    return T


def _allowed(S: State, L: float, s: int, monotone: bool) -> bool:
    if not monotone:
        return True
    cap = S.cap if L == S.grp_len else min(S.cap, S.grp_min)
    return s <= cap


def route(lengths, n_gpus: int, sp_max: int, cm: CostModel, token_budget: float,
          prefix: int, beam: int, monotone: bool = False, level_mask: int = -1):
    """Algorithm 1.  Returns (plan as a list of nodes per sample, final state, within_budget)."""
    M = len(lengths)
    order = sorted(range(M), key=lambda j: (-lengths[j], j))
    head, tail = order[:prefix], order[prefix:]
    nodes = tree_nodes(n_gpus, sp_max, level_mask)
    if not nodes:
        raise ValueError("no tree level enabled")
    zero = State(dfwd=[0.0] * n_gpus, dbwd=[0.0] * n_gpus, tok=[0.0] * n_gpus)
    Q = [zero]
    for j in head:
        L = float(lengths[j])
        N = []
        for S in Q:
            for u in nodes:
                if _allowed(S, L, len(rank_range(u, sp_max)), monotone):
                    N.append(_extend(S, j, L, u, sp_max, cm))
        ok = [S for S in N if S.maxT() <= token_budget]
        if ok:
            Q = sorted(ok, key=lambda S: S.maxC())[:beam]
        else:
            Q = sorted(N, key=lambda S: S.maxT())[:beam]
    deepest = max(d for d, _ in nodes)
    units = [u for u in nodes if u[0] == deepest]
    done = []
    for S in Q:
        for j in tail:
            L = float(lengths[j])
            best, best_load = None, None
            for u in units:
                ranks = rank_range(u, sp_max)
                s = len(ranks)
                if max(S.tok[p] + L / s for p in ranks) <= token_budget:
                    load = max(S.dfwd[p] + S.dbwd[p] for p in ranks)
                    if best is None or load < best_load:
                        best, best_load = u, load
            if best is None:
                for u in units:
                    tl = max(S.tok[p] for p in rank_range(u, sp_max))
                    if best is None or tl < best_load:
                        best, best_load = u, tl
            S = _extend(S, j, L, best, sp_max, cm)
        done.append(S)
    final = min(done, key=lambda S: S.maxC())
    plan = [final.plan[j] for j in range(M)]
    return plan, final, final.maxT() <= token_budget


def brute_force(lengths, n_gpus: int, sp_max: int, cm: CostModel, token_budget: float,
                monotone: bool = False, level_mask: int = -1):
    """The smallest max_p C_p over every plan within the token budget (and the
    monotone constraint if asked), by enumeration; (value, plan) or (None, None)."""
    nodes = tree_nodes(n_gpus, sp_max, level_mask)
    best, best_plan = None, None
    for plan in product(nodes, repeat=len(lengths)):
        if monotone:
            deg = [len(rank_range(u, sp_max)) for u in plan]
            if any(lengths[a] > lengths[b] and deg[a] < deg[b]
                   for a in range(len(plan)) for b in range(len(plan))):
                continue
        C, tok, _, _, _ = plan_cost(lengths, plan, n_gpus, sp_max, cm)
        if max(tok) > token_budget:
            continue
        if best is None or max(C) < best:
            best, best_plan = max(C), list(plan)
    return best, best_plan

"""Pins of the oracle's NSP planner: the SP tree of Figure 4, the cost model
against hand-computed values, incremental state against from-scratch plan
evaluation, the beam search against brute force when it is exhaustive, and the
greedy tail against textbook longest-processing-time list scheduling."""
import heapq
import os

import numpy as np
import pytest

from oracle import router as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cm(**kw):
    base = dict(curve_len=[128.0, 1024.0, 8192.0, 65536.0], fwd_tflops=[250.0, 600.0, 900.0, 1050.0],
                bwd_tflops=[200.0, 500.0, 800.0, 950.0], fwd_flops_per_pair=4 * 128 * 32.0,
                bwd_flops_per_pair=10 * 128 * 32.0,
                bytes_per_token=(40 * 256.0, 32 * 256.0, 32 * 256.0, 40 * 256.0),
                a2a_gbs=80.0, a2a_alpha_us=15.0, dense_fwd_flops_per_token=2e8,
                dense_bwd_flops_per_token=4e8, dense_tflops=800.0)
    base.update(kw)
    return R.CostModel(**base)


def test_sp_tree_matches_figure4():
    rows, chain = [], None
    for ln in open(os.path.join(GOLDEN, "nsp_fig4_sp_tree.txt")):
        if ln.startswith("#") or not ln.strip():
            continue
        if ln.startswith("chain"):
            chain = [tuple(int(x) for x in part.split()) for part in ln.split(":")[1].split(",")]
        else:
            rows.append(tuple(int(x) for x in ln.split()))
    nodes = R.tree_nodes(8, 8)
    assert nodes == [(d, i) for d, i, _, _ in rows]
    for d, i, a, b in rows:
        assert list(R.rank_range((d, i), 8)) == list(range(a, b + 1))
    mine = [u for u in nodes if 5 in R.rank_range(u, 8)]
    assert mine == chain
    assert [len(R.rank_range(u, 8)) for u in mine] == [8, 4, 2, 1]


def test_tree_levels_and_forest():
    assert len(R.tree_nodes(16, 4)) == 4 * 7           # four trees of spmax 4
    two_level = R.tree_nodes(8, 8, level_mask=(1 << 0) | (1 << 3))
    assert {d for d, _ in two_level} == {0, 3} and len(two_level) == 9
    with pytest.raises(ValueError):
        R.tree_nodes(12, 8)
    with pytest.raises(ValueError):
        R.tree_nodes(12, 6)


def test_throughput_interpolation():
    xs, ys = [100.0, 200.0, 400.0], [10.0, 20.0, 60.0]
    assert R.throughput(xs, ys, 50) == 10.0 and R.throughput(xs, ys, 1000) == 60.0
    assert R.throughput(xs, ys, 150) == 15.0 and R.throughput(xs, ys, 300) == 40.0


def test_cost_of_one_sample_by_hand():
    # flat curve 1 TFLOP/s, 1e12 FLOPs per pair: a 3-token causal sample has
    # 6 pairs -> 6 s of forward compute, split over the node's GPUs
    cm = _cm(curve_len=[1.0], fwd_tflops=[1.0], bwd_tflops=[2.0], fwd_flops_per_pair=1e12,
             bwd_flops_per_pair=1e12, bytes_per_token=(1e9, 2e9, 3e9, 4e9), a2a_gbs=1.0,
             a2a_alpha_us=1e6, dense_fwd_flops_per_token=1e12, dense_bwd_flops_per_token=3e12,
             dense_tflops=1.0)
    # root of a 2-GPU tree: s = 2, 1.5 tokens per GPU
    C, tok, f, b, load = R.plan_cost([3], [(0, 0)], 2, 2, cm)
    # fwd: latency 2 * (s-1) * 1 s = 2; comm (1/2) * 1.5 * (1 + 2) = 2.25; compute 6/2 = 3;
    # dense 1.5 * 1 = 1.5
    assert f == [2 + 2.25 + 3 + 1.5] * 2
    # bwd: latency 2; comm (1/2) * 1.5 * (3 + 4) = 5.25; compute 6/2/2 = 1.5; dense 1.5 * 3 = 4.5
    assert b == [2 + 5.25 + 1.5 + 4.5] * 2
    assert tok == [1.5, 1.5] and load == f[0] + b[0] and C == [f[0] + b[0]] * 2
    # a leaf: no communication, all compute on its GPU, nothing on the other
    C, tok, f, b, _ = R.plan_cost([3], [(1, 1)], 2, 2, cm)
    assert f == [0.0, 6 + 3.0] and b == [0.0, 3 + 9.0] and tok == [0.0, 3.0]


def test_nested_nodes_add_along_the_chain():
    cm = _cm()
    L = [5000, 700]
    C, tok, _, _, _ = R.plan_cost(L, [(0, 0), (2, 1)], 4, 4, cm)
    C0, tok0, _, _, _ = R.plan_cost([5000], [(0, 0)], 4, 4, cm)
    C1, tok1, _, _, _ = R.plan_cost([700], [(2, 1)], 4, 4, cm)
    assert np.allclose(C, np.add(C0, C1), rtol=1e-14)
    assert tok == [1250.0, 1950.0, 1250.0, 1250.0]


def test_incremental_state_equals_plan_evaluation():
    rng = np.random.default_rng(3)
    cm = _cm()
    nodes = R.tree_nodes(8, 8)
    for _ in range(50):
        L = [int(x) for x in rng.integers(64, 20000, size=rng.integers(1, 9))]
        plan = [nodes[int(k)] for k in rng.integers(0, len(nodes), size=len(L))]
        S = R.State(dfwd=[0.0] * 8, dbwd=[0.0] * 8, tok=[0.0] * 8)
        for j in sorted(range(len(L)), key=lambda j: -L[j]):
            S = R._extend(S, j, float(L[j]), plan[j], 8, cm)
        C, tok, f, b, _ = R.plan_cost(L, plan, 8, 8, cm)
        assert np.allclose(S.dfwd, f, rtol=1e-13) and np.allclose(S.dbwd, b, rtol=1e-13)
        assert np.allclose(S.tok, tok, rtol=1e-13)
        assert abs(S.maxC() - max(C)) <= 1e-13 * max(C)


@pytest.mark.parametrize("monotone", [False, True])
@pytest.mark.parametrize("mask", [-1, 0b101])
def test_exhaustive_beam_equals_brute_force(monotone, mask):
    rng = np.random.default_rng(11 + monotone + mask)
    cm = _cm()
    for trial in range(6):
        M = int(rng.integers(1, 5))
        L = [int(x) for x in rng.integers(64, 30000, size=M)]
        budget = float(rng.choice([1e12, 0.55 * sum(L)]))
        best, _ = R.brute_force(L, 4, 4, cm, budget, monotone, mask)
        plan, S, ok = R.route(L, 4, 4, cm, budget, prefix=M, beam=10 ** 6, monotone=monotone,
                              level_mask=mask)
        if best is None:
            assert not ok
            continue
        assert ok
        C, tok, _, _, _ = R.plan_cost(L, plan, 4, 4, cm)
        assert abs(max(C) - best) <= 1e-12 * best
        assert max(tok) <= budget


def test_plans_respect_monotone_levels_and_budget():
    rng = np.random.default_rng(5)
    cm = _cm()
    for _ in range(20):
        L = [int(x) for x in rng.integers(64, 60000, size=12)]
        budget = 0.3 * sum(L)
        plan, S, ok = R.route(L, 8, 8, cm, budget, prefix=4, beam=8, monotone=True,
                              level_mask=0b1011)
        deg = [len(R.rank_range(u, 8)) for u in plan]
        assert all(u[0] in (0, 1, 3) for u in plan)
        for a in range(12):
            for b in range(12):
                if L[a] > L[b]:
                    assert deg[a] >= deg[b]
        _, tok, _, _, _ = R.plan_cost(L, plan, 8, 8, cm)
        assert ok == (max(tok) <= budget)


def test_greedy_tail_is_lpt_list_scheduling():
    # with no communication, constant throughput and an unlimited budget, the
    # tail places each sample (longest first) on the least-loaded GPU
    cm = _cm(curve_len=[1.0], fwd_tflops=[1.0], bwd_tflops=[1.0], bytes_per_token=(0, 0, 0, 0),
             a2a_alpha_us=0.0, dense_fwd_flops_per_token=0.0, dense_bwd_flops_per_token=0.0)
    rng = np.random.default_rng(2)
    for _ in range(10):
        L = [int(x) for x in rng.integers(1, 5000, size=30)]
        plan, S, _ = R.route(L, 8, 8, cm, 1e18, prefix=0, beam=1)
        heap = [(0.0, p) for p in range(8)]
        load = [0.0] * 8
        for j in sorted(range(30), key=lambda j: (-L[j], j)):
            c = (cm.fwd_flops_per_pair + cm.bwd_flops_per_pair) * L[j] * (L[j] + 1) / 2 / 1e12
            ld, p = heapq.heappop(heap)
            load[p] = ld + c
            heapq.heappush(heap, (load[p], p))
        assert abs(S.maxC() - max(load)) <= 1e-12 * max(load)


def test_over_budget_is_reported():
    cm = _cm()
    plan, S, ok = R.route([40000, 30000], 4, 4, cm, 1000.0, prefix=1, beam=4)
    assert not ok and len(plan) == 2


def test_beam_keeps_the_cheapest_states():
    # all-to-alls cost far more than the compute they save, so the best plan for
    # two equal samples on two GPUs puts one on each leaf; a beam of one must
    # find it by keeping the cheapest state (the root is generated first)
    cm = _cm(a2a_alpha_us=1e6)
    plan, S, ok = R.route([4096, 4096], 2, 2, cm, 1e12, prefix=2, beam=1)
    assert plan == [(1, 0), (1, 1)] and ok
    # and with free communication the root wins for a long sample
    cm = _cm(a2a_alpha_us=0.0, bytes_per_token=(0, 0, 0, 0))
    plan, _, _ = R.route([60000], 2, 2, cm, 1e12, prefix=1, beam=1)
    assert plan == [(0, 0)]

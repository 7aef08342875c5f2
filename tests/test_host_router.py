"""CPU tests of the library's NSP planner (nsp_route, nsp_plan_cost) against
the oracle's: identical plans and bitwise-identical per-GPU loads on random
long-tail batches across tree sizes, beams, prefixes, budgets, the monotone
rule and level masks; plan evaluation against the oracle's from-scratch
evaluation; the documented error codes."""
import ctypes

import numpy as np
import pytest

import variable_length_sequence_amd as vl
import workloads
from oracle import router as R

FIELDS = ("curve_len", "fwd_tflops", "bwd_tflops", "fwd_flops_per_pair", "bwd_flops_per_pair",
          "bytes_per_token", "a2a_gbs", "a2a_alpha_us", "dense_fwd_flops_per_token",
          "dense_bwd_flops_per_token", "dense_tflops")


def _models(rng):
    kw = dict(curve_len=[128.0, 512.0, 2048.0, 8192.0, 32768.0, 131072.0],
              fwd_tflops=list(np.sort(rng.uniform(100, 1200, 6))),
              bwd_tflops=list(np.sort(rng.uniform(80, 1000, 6))),
              fwd_flops_per_pair=4 * 128 * 32.0, bwd_flops_per_pair=10 * 128 * 32.0,
              bytes_per_token=tuple(float(x) for x in rng.uniform(1e3, 3e4, 4)),
              a2a_gbs=float(rng.uniform(50, 1000)), a2a_alpha_us=float(rng.uniform(0, 50)),
              dense_fwd_flops_per_token=float(rng.uniform(0, 1e9)),
              dense_bwd_flops_per_token=float(rng.uniform(0, 2e9)),
              dense_tflops=float(rng.uniform(300, 1500)))
    return R.CostModel(**kw), vl.CostModel(**kw)


def _batch(rng, n):
    x = 128 * (1 + rng.pareto(1.1, size=n))
    return [int(v) for v in np.clip(x, 64, 200000)]


CONFIGS = [  # n_gpus, sp_max, prefix, beam, monotone, level_mask, budget factor
    (4, 4, 3, 4, False, -1, 10.0),
    (8, 8, 4, 8, False, -1, 0.4),
    (8, 8, 6, 3, True, -1, 0.3),
    (16, 8, 5, 6, False, 0b1001, 0.25),
    (16, 16, 8, 16, True, 0b10111, 0.2),
    (32, 8, 2, 2, False, -1, 1.0),
    (64, 64, 8, 16, False, -1, 0.05),
    (8, 4, 0, 1, False, -1, 0.5),
    (8, 8, 20, 4, False, -1, 0.3),
    (4, 4, 5, 4, False, -1, 0.01),          # nothing fits: over budget
]


@pytest.mark.parametrize("cfg", CONFIGS)
def test_route_matches_oracle_bitwise(cfg):
    P, S, k, w, mono, mask, frac = cfg
    rng = np.random.default_rng(P * 131 + k * 7 + w)
    for trial in range(4):
        ocm, lcm = _models(rng)
        L = _batch(rng, int(rng.integers(1, 40)))
        budget = frac * sum(L) / P * 4
        plan, st, ok = R.route(L, P, S, ocm, budget, k, w, mono, mask)
        got = vl.nsp_route(L, P, S, lcm, budget, k, w, mono, mask)
        assert got["plan"] == plan
        assert np.array_equal(got["gpu_fwd"], np.array(st.dfwd))
        assert np.array_equal(got["gpu_bwd"], np.array(st.dbwd))
        assert np.array_equal(got["gpu_tokens"], np.array(st.tok))
        assert got["within_budget"] == ok


def test_route_pareto_batch_on_64_gpus():
    w = workloads.mixed_128k()
    rng = np.random.default_rng(0)
    ocm, lcm = _models(rng)
    budget = 1.2 * sum(w.lengths) / 64 * 8
    plan, st, ok = R.route(w.lengths, 64, 64, ocm, budget, 8, 16, True)
    got = vl.nsp_route(w.lengths, 64, 64, lcm, budget, 8, 16, True)
    assert got["plan"] == plan and np.array_equal(got["gpu_fwd"], np.array(st.dfwd))
    assert got["within_budget"] == ok


def test_plan_cost_matches_oracle():
    rng = np.random.default_rng(9)
    for _ in range(20):
        ocm, lcm = _models(rng)
        L = _batch(rng, int(rng.integers(1, 30)))
        nodes = R.tree_nodes(16, 8)
        plan = [nodes[int(i)] for i in rng.integers(0, len(nodes), len(L))]
        C, tok, f, b, load = R.plan_cost(L, plan, 16, 8, ocm)
        got = vl.nsp_plan_cost(L, plan, 16, 8, lcm)
        assert np.allclose(got["gpu_fwd"], f, rtol=1e-12, atol=0)
        assert np.allclose(got["gpu_bwd"], b, rtol=1e-12, atol=0)
        assert np.allclose(got["gpu_tokens"], tok, rtol=1e-12, atol=0)
        assert abs(got["load"] - load) <= 1e-12 * load


def test_route_empty_batch():
    _, lcm = _models(np.random.default_rng(1))
    got = vl.nsp_route([], 8, 8, lcm, 1e9)
    assert got["plan"] == [] and got["within_budget"] and not got["gpu_tokens"].any()


def test_router_rejects_bad_arguments():
    _, lcm = _models(np.random.default_rng(2))
    with pytest.raises(vl.VarlenError) as e:
        vl.nsp_route([10, 20], 12, 8, lcm, 1e9)
    assert e.value.code == -2
    with pytest.raises(vl.VarlenError) as e:
        vl.nsp_route([10, 20], 8, 6, lcm, 1e9)
    assert e.value.code == -2
    with pytest.raises(vl.VarlenError) as e:
        vl.nsp_route([10, 20], 8, 8, lcm, 1e9, level_mask=1 << 5)
    assert e.value.code == -2
    with pytest.raises(vl.VarlenError) as e:
        vl.nsp_route([10, -1], 8, 8, lcm, 1e9)
    assert e.value.code == -1
    with pytest.raises(vl.VarlenError) as e:
        vl.nsp_route([10, 20], 8, 8, lcm, 1e9, beam=0)
    assert e.value.code == -1
    bad = vl.CostModel(**{**lcm.__dict__, "curve_len": [128.0, 64.0] + list(lcm.curve_len[2:])})
    with pytest.raises(vl.VarlenError) as e:
        vl.nsp_route([10, 20], 8, 8, bad, 1e9)
    assert e.value.code == -1
    bad = vl.CostModel(**{**lcm.__dict__, "a2a_gbs": 0.0})
    with pytest.raises(vl.VarlenError) as e:
        vl.nsp_route([10, 20], 8, 8, bad, 1e9)
    assert e.value.code == -1
    with pytest.raises(vl.VarlenError) as e:
        vl.nsp_plan_cost([10], [(4, 0)], 8, 8, lcm)
    assert e.value.code == -2
    L = vl.lib()
    assert L.nsp_route(None, 2, 8, 8, None, 1e9, 1, 1, 0, -1, None, None, None, None, None,
                       None) == -1


def test_shipped_curve_routes_the_pareto_batch():
    # the measured MI355X curve shipped with the library drives a Ulysses cost
    # model; the library's plan equals the oracle's, and the planner's load
    # is far below packing every sample onto single GPUs (prefix 0)
    w = workloads.mixed_128k()
    lcm = vl.ulysses_cost_model(32, 4, 128, sp_max=64)
    ocm = R.CostModel(**{f: getattr(lcm, f) for f in FIELDS})
    P = 64
    budget = 2.0 * sum(w.lengths) / P
    got = vl.nsp_route(w.lengths, P, P, lcm, budget, 8, 16, True)
    plan, st, ok = R.route(w.lengths, P, P, ocm, budget, 8, 16, True)
    assert got["plan"] == plan and np.array_equal(got["gpu_fwd"], np.array(st.dfwd))
    leaves = vl.nsp_route(w.lengths, P, P, lcm, budget, 0, 1)
    assert got["load"] < 0.5 * leaves["load"]
    # the longest document is spread over more GPUs than the shortest
    deg = [P >> d for d, _ in got["plan"]]
    assert deg[int(np.argmax(w.lengths))] > deg[int(np.argmin(w.lengths))]


def test_ulysses_cost_model_terms_by_hand():
    curve = {"len": [128.0, 65536.0], "fwd_tflops": [100.0, 1000.0], "bwd_tflops": [80.0, 700.0]}
    # 32 q heads, 4 kv heads, d 128, bf16, 8-way groups: kv heads 4 < 8 are sent
    # to two ranks each, so the exchange carries 8 kv heads' worth per tensor
    cm = vl.ulysses_cost_model(32, 4, 128, sp_max=8, curve=curve, a2a_gbs=1000.0,
                               a2a_alpha_us=5.0)
    assert cm.fwd_flops_per_pair == 4 * 128 * 32 and cm.bwd_flops_per_pair == 10 * 128 * 32
    row = 128 * 2
    assert tuple(cm.bytes_per_token) == ((32 + 2 * 8) * row, 32 * row, 32 * row, (32 + 2 * 8) * row)
    # with at least as many kv heads as ranks nothing is replicated
    cm2 = vl.ulysses_cost_model(32, 8, 128, sp_max=8, curve=curve)
    assert cm2.bytes_per_token[0] == (32 + 2 * 8) * row
    cm3 = vl.ulysses_cost_model(32, 16, 64, sp_max=4, curve=curve)
    assert cm3.bytes_per_token[0] == (32 + 2 * 16) * 64 * 2


def test_shipped_curve_is_well_formed():
    import json
    c = json.load(open(vl.CURVE_PATH))
    L = c["len"]
    assert len(L) == len(c["fwd_tflops"]) == len(c["bwd_tflops"]) >= 2
    assert all(b > a for a, b in zip(L, L[1:]))
    assert all(x > 0 for x in c["fwd_tflops"] + c["bwd_tflops"])
    assert (c["heads_q"], c["heads_kv"], c["head_dim"]) == (32, 4, 128)

"""Pins of the oracle's router.

The pages show only the gate's call site ("MoE update", moe-forward
excerpt: it returns routing weights and expert indices); the router's steps are the plain reading written in the
oracle's header.  Pins: exhaustive subset search (a different algorithm for
the same selection), a special case that reduces to a plain top-k of the
logits, hand-worked examples whose answers follow from the definition, and the
invariants the layer's description fixes (weights sum to route_scale, at most
topk_groups groups per token, topk distinct experts).
"""
import itertools
import math

import numpy as np
import pytest

import oracle
import synth


def _tiny_inputs(seed, T=64, dims=synth.TINY, bias_sigma=0.1):
    rng = np.random.default_rng(seed)
    x = oracle.bf16_round(rng.standard_normal((T, dims.d_model)))
    gw = (rng.standard_normal((dims.n_experts, dims.d_model)) / math.sqrt(dims.d_model)).astype(np.float32)
    gb = (rng.standard_normal(dims.n_experts) * bias_sigma).astype(np.float32)
    return x, gw, gb


def _group_score_def(vals):
    return sum(sorted(vals)[-2:])


def _brute(b_row, dims):
    """Best group subset by total group score, then best expert subset by total biased score."""
    E, G, TG, K = dims.n_experts, dims.n_groups, dims.topk_groups, dims.topk
    epg = E // G
    gs = [_group_score_def(list(b_row[g * epg:(g + 1) * epg])) for g in range(G)]
    best_groups = max(itertools.combinations(range(G), TG), key=lambda c: sum(gs[g] for g in c))
    allowed = [e for g in best_groups for e in range(g * epg, (g + 1) * epg)]
    best = max(itertools.combinations(allowed, K), key=lambda c: sum(b_row[e] for e in c))
    return set(best), set(best_groups)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_routing_matches_subset_search(seed):
    dims = synth.TINY
    x, gw, gb = _tiny_inputs(seed)
    r = oracle.gate(x, gw, gb, dims)
    for t in range(x.shape[0]):
        experts, groups = _brute(r["b"][t], dims)
        assert set(r["idx"][t].tolist()) == experts
        assert set(r["groups"][t].tolist()) == groups


def test_routing_matches_subset_search_other_shape():
    dims = synth.Dims(d_model=256, n_experts=24, n_groups=6, topk_groups=3, topk=5, inter=128)
    x, gw, gb = _tiny_inputs(7, T=40, dims=dims, bias_sigma=0.3)
    r = oracle.gate(x, gw, gb, dims)
    for t in range(x.shape[0]):
        experts, _ = _brute(r["b"][t], dims)
        assert set(r["idx"][t].tolist()) == experts


def test_all_groups_no_bias_is_topk_of_logits():
    dims = synth.Dims(d_model=512, n_experts=16, n_groups=4, topk_groups=4, topk=4, inter=128)
    x, gw, _ = _tiny_inputs(3)
    r = oracle.gate(x, gw, np.zeros(16, np.float32), dims)
    z = x @ gw.astype(np.float64).T
    top = np.argsort(-z, axis=1)[:, :4]
    assert np.array_equal(r["idx"], top)


def test_weights_are_normalised_unbiased_sigmoid_scores():
    dims = synth.TINY
    x, gw, gb = _tiny_inputs(4, bias_sigma=0.5)
    r = oracle.gate(x, gw, gb, dims)
    for t in (0, 17, 63):
        z = [sum(float(x[t, j]) * float(gw[e, j]) for j in range(dims.d_model)) for e in r["idx"][t]]
        s = [1.0 / (1.0 + math.exp(-v)) for v in z]
        want = [2.5 * v / sum(s) for v in s]
        assert np.allclose(r["w"][t], want, rtol=1e-12, atol=0)


def test_invariants_tiny_workload():
    dims = synth.TINY
    x, gw, gb = _tiny_inputs(5)
    r = oracle.gate(x, gw, gb, dims)
    idx = r["idx"]
    assert np.allclose(r["w"].sum(1), dims.route_scale, rtol=0, atol=1e-12)
    assert np.all(r["w"] > 0)
    for t in range(idx.shape[0]):
        assert len(set(idx[t].tolist())) == dims.topk
        assert len(set((idx[t] // dims.experts_per_group).tolist())) <= dims.topk_groups
        # descending biased score
        bt = r["b"][t, idx[t]]
        assert np.all(np.diff(bt) <= 0)


def _worked(bias):
    # x = 0 makes every logit 0 and every score exactly 0.5, so b = 0.5 + bias
    dims = synth.Dims(d_model=128, n_experts=8, n_groups=4, topk_groups=2, topk=2, inter=128)
    x = np.zeros((1, 128))
    gw = np.ones((8, 128), np.float32)
    return dims, oracle.gate(x, gw, np.array(bias, np.float32), dims)


def test_worked_example_group_score_is_top2_sum_and_ties_go_low():
    # b per group: g0 (0.8, 0.5)=1.3, g1 (0.85, 0.2)=1.05, g2 (0.7, 0.7)=1.4, g3 (0.6, 0.55)=1.15
    # top-2 sums keep {g2, g0}; within them 0.8 (expert 0) then the 0.7 tie -> expert 4
    # (ranking groups by their best expert would keep {g1, g0} and pick experts 2, 0)
    dims, r = _worked([0.30, 0.00, 0.35, -0.30, 0.20, 0.20, 0.10, 0.05])
    assert r["idx"][0].tolist() == [0, 4]
    assert r["groups"][0].tolist() == [0, 2]
    assert np.allclose(r["w"][0], [1.25, 1.25])        # equal unbiased scores -> equal weights


def test_worked_example_excluded_groups_are_not_zero_filled():
    # all kept scores negative: g0 (-0.1, -0.2) is the best group with topk_groups = 1 below;
    # expert 2 (b = 0.3) sits in a weaker group and must not be picked
    dims = synth.Dims(d_model=128, n_experts=8, n_groups=4, topk_groups=1, topk=2, inter=128)
    x = np.zeros((1, 128))
    bias = np.array([-0.6, -0.7, -0.2, -1.4, -0.9, -0.9, -1.0, -1.0], np.float32)
    r = oracle.gate(x, np.ones((8, 128), np.float32), bias, dims)
    assert r["idx"][0].tolist() == [0, 1]


def test_near_tie_gaps():
    dims, r = _worked([0.30, 0.00, 0.35, -0.30, 0.20, 0.20, 0.10, 0.05])
    # kept experts' b sorted: 0.8, 0.7, 0.7, 0.5 -> K=2 gap 0; groups 1.4, 1.3 | 1.15 -> gap 0.15
    assert r["expert_gap"][0] == 0.0
    assert abs(r["group_gap"][0] - 0.15) < 1e-6

"""Pins for the router oracle: the pages' worked toy example, library
softmax / sigmoid, brute force over tiny inputs (full sorts and subset
enumeration, not k-round arg-max), closed-form special cases and the
DeepSeek-V3 decode-trace statistics."""

import itertools
import math

import numpy as np
import pytest
import scipy.special

from oracle import align as oalign
from oracle import formats as fm
from oracle import router as orouter


def _toy_inputs(golden, bias=None):
    g = golden("router_toy.json")
    E, H = g["E"], 64
    sc = {int(e): v for e, v in g["printed_scores"].items()}
    lg = np.full(E, 0.0)
    rng = np.random.default_rng(0)
    for e in range(E):
        lg[e] = math.log(sc[e] / (1 - sc[e])) if e in sc else rng.uniform(-2.0, g["other_expert_logit_max"])
    gate = np.zeros((E, H), dtype=np.float32)
    gate[:, 0] = lg
    x = np.zeros((1, H))
    x[0, 0] = 1.0
    return g, fm.f64_to_bf16_bits(x), gate


def test_toy_router_without_bias(golden):
    g, x, gate = _toy_inputs(golden)
    r = orouter.route(x, gate, None, k=2, scoring="sigmoid")
    assert r["ids"][0].tolist() == g["printed_no_bias"]["ids"]
    for e, s in g["printed_scores"].items():
        assert round(r["scores"][0, int(e)], 3) == s
    for j, e in enumerate(r["ids"][0]):
        assert round(r["weights"][0, j], 3) == g["printed_no_bias"]["weights"][str(e)]


def test_toy_router_with_bias(golden):
    g, x, gate = _toy_inputs(golden)
    b = np.full(g["E"], g["derived_biases"]["other"], dtype=np.float32)
    for e in ("0", "2", "5"):
        b[int(e)] = g["derived_biases"][e]
    r = orouter.route(x, gate, b, k=2, scoring="sigmoid")
    for e, key in g["printed_keys_with_bias"].items():
        assert round(r["keys"][0, int(e)], 3) == key
    assert r["ids"][0].tolist() == g["derived_with_bias"]["ids"]
    assert round(r["margin"][0], 3) == g["printed_gap_at_cut"]
    # the weights come from the unbiased scores 0.870 and 0.769
    for j, e in enumerate(r["ids"][0]):
        assert round(r["weights"][0, j], 3) == g["derived_with_bias"]["weights"][str(e)]
    # the same biases stored as bf16: 8.03 -> 8.0 and the choice flips
    bb = fm.bf16_bits_to_f64(fm.f64_to_bf16_bits(b)).astype(np.float32)
    assert bb[5] == g["printed_bf16_bias_flip"]["bias_5_bf16"]
    r2 = orouter.route(x, gate, bb, k=2, scoring="sigmoid")
    assert round(r2["keys"][0, 5], 3) == g["printed_bf16_bias_flip"]["key_5_after"]
    assert sorted(r2["ids"][0].tolist()) == g["printed_bf16_bias_flip"]["ids"]


def test_scores_match_scipy():
    rng = np.random.default_rng(3)
    lg = rng.normal(0, 3, size=(50, 37))
    assert np.allclose(orouter.scores(lg, "softmax"), scipy.special.softmax(lg, axis=1), rtol=1e-13, atol=0)
    assert np.allclose(orouter.scores(lg, "sigmoid"), scipy.special.expit(lg), rtol=1e-13, atol=0)
    assert np.allclose(orouter.scores(lg, "sqrtsoftplus"), np.sqrt(scipy.special.softplus(lg)), rtol=1e-13, atol=0)
    with pytest.raises(ValueError):
        orouter.scores(lg, "sqrt_softplus")


def test_sqrt_softplus_closed_forms():
    """sqrt(softplus): sqrt(ln 2) at 0; sqrt(l) + O(e^-l) for large l;
    exp(l / 2) (1 + O(e^l)) for very negative l; increasing, positive, and
    sqrt(log(1 + e^l)) by np.logaddexp on moderate l."""
    s = lambda v: orouter.scores(np.array([v], dtype=np.float64), "sqrtsoftplus")[0]
    assert s([0.0])[0] == pytest.approx(math.sqrt(math.log(2.0)), rel=1e-15)
    assert s([100.0])[0] == pytest.approx(10.0, rel=1e-15)
    assert s([800.0])[0] == pytest.approx(math.sqrt(800.0), rel=1e-15)  # no overflow
    assert s([-40.0])[0] == pytest.approx(math.exp(-20.0), rel=1e-12)
    assert s([-800.0])[0] == 0.0 or s([-800.0])[0] < 1e-170
    lg = np.linspace(-30, 30, 601)
    v = s(lg)
    assert np.all(np.diff(v) > 0) and np.all(v > 0)
    assert np.allclose(v, np.sqrt(np.logaddexp(0.0, lg)), rtol=1e-14, atol=0)


def test_logits_are_exact_products():
    rng = np.random.default_rng(4)
    x = fm.f64_to_bf16_bits(rng.normal(size=(5, 48)))
    gate = rng.normal(0, 0.02, size=(9, 48)).astype(np.float32)
    lg = orouter.logits(x, gate)
    xv = fm.bf16_bits_to_f64(x)
    for t in range(5):
        for e in range(9):
            ref = math.fsum(float(xv[t, h]) * float(gate[e, h]) for h in range(48))
            assert abs(lg[t, e] - ref) <= 1e-15 * max(1.0, abs(ref)) * 48


@pytest.mark.parametrize("E,k", [(3, 1), (5, 2), (8, 2), (10, 4), (10, 10)])
def test_topk_matches_full_sort_with_ties(E, k):
    rng = np.random.default_rng(E * 100 + k)
    keys = rng.integers(0, 4, size=(300, E)).astype(np.float64)  # many ties
    ids, margin = orouter.topk(keys, k)
    for t in range(keys.shape[0]):
        order = sorted(range(E), key=lambda e: (-keys[t, e], e))
        assert ids[t].tolist() == order[:k]
        expect = keys[t, order[k - 1]] - keys[t, order[k]] if k < E else math.inf
        assert margin[t] == expect


@pytest.mark.parametrize("E,n_group,topk_group,k", [(12, 4, 2, 3), (16, 4, 3, 5), (8, 2, 1, 2), (24, 8, 4, 8)])
def test_group_limit_matches_enumeration(E, n_group, topk_group, k):
    rng = np.random.default_rng(E + n_group * 7 + k)
    keys = rng.integers(0, 5, size=(200, E)).astype(np.float64)
    gsize = E // n_group
    allowed, gscore, kept = orouter.group_limit(keys, n_group, topk_group)
    ids, _ = orouter.topk(keys, k, allowed)
    for t in range(keys.shape[0]):
        gs = [max(keys[t, g * gsize + i] + keys[t, g * gsize + j]
                  for i, j in itertools.combinations(range(gsize), 2)) for g in range(n_group)]
        assert np.array_equal(gscore[t], gs)
        best = max(itertools.combinations(range(n_group), topk_group),
                   key=lambda s: (sum(gs[g] for g in s), [-g for g in s]))
        assert sorted(kept[t].tolist()) == list(best)
        cand = [e for e in range(E) if e // gsize in best]
        order = sorted(cand, key=lambda e: (-keys[t, e], e))
        assert ids[t].tolist() == order[:k]


def test_k_equals_E_softmax_renormalised_is_full_softmax():
    rng = np.random.default_rng(5)
    x = fm.f64_to_bf16_bits(rng.normal(size=(20, 32)))
    gate = rng.normal(0, 0.1, size=(6, 32)).astype(np.float32)
    r = orouter.route(x, gate, None, k=6, scoring="softmax")
    full = scipy.special.softmax(r["logits"], axis=1)
    w = np.zeros_like(full)
    np.put_along_axis(w, r["ids"], r["weights"], axis=1)
    assert np.allclose(w, full, rtol=1e-12, atol=0)


def test_top1_renormalised_weight_is_one_and_bias_changes_choice(golden):
    g = golden("combine_numpy.json")["bias_flip"]
    sc = np.array([g["scores"]])
    ids0, _ = orouter.topk(orouter.rank_keys(sc, None), 1)
    ids1, _ = orouter.topk(orouter.rank_keys(sc, np.array(g["bias"], dtype=np.float32)), 1)
    assert ids0[0, 0] == g["argmax_before"] and ids1[0, 0] == g["argmax_after"]
    assert orouter.weights(sc, ids1)[0, 0] == 1.0
    assert orouter.weights(sc, ids0)[0, 0] == 1.0


def test_weights_renormalise_then_scale():
    rng = np.random.default_rng(6)
    x = fm.f64_to_bf16_bits(rng.normal(size=(40, 64)))
    gate = rng.normal(0, 0.05, size=(16, 64)).astype(np.float32)
    bias = rng.normal(0, 0.1, size=16).astype(np.float32)
    r = orouter.route(x, gate, bias, k=4, scoring="sigmoid", n_group=4, topk_group=2, routed_scale=2.5)
    assert np.allclose(r["weights"].sum(axis=1), 2.5, rtol=1e-14)
    # weights come from the unbiased scores, in id order of the selection
    s = np.take_along_axis(r["scores"], r["ids"], axis=1)
    assert np.allclose(r["weights"], 2.5 * s / s.sum(axis=1, keepdims=True), rtol=1e-14)
    assert all(len(set(row)) == 4 for row in r["ids"].tolist())


def test_dsv3_decode_trace_statistics(golden):
    """[MoE] DeepSeek-V3 trace at T=64: about 222 of 256 experts touched and
    about 3,552 padded rows at BLOCK_M=16.  Synthetic random gates give
    near-uniform routing, so the touched count should sit near the closed form
    E(1-(1-k/E)^T) = 222.4; its spread under uniform routing is about 5."""
    from synth import get_config, make_x
    from synth.generate import _randn

    g = golden("moe_byte_model.json")["dsv3"]
    cfg = get_config("dsv3")
    gate = _randn((cfg.E, cfg.H), cfg.gate_std, "cpu", cfg.seed, cfg.name, "gate").numpy()
    bias = _randn((cfg.E,), cfg.bias_std, "cpu", cfg.seed, cfg.name, "bias").numpy()
    x = make_x(cfg, g["trace_T"])
    xb = x.view(__import__("torch").int16).numpy().view(np.uint16)
    r = orouter.route(xb, gate, bias, k=cfg.k, scoring="sigmoid", n_group=cfg.n_group,
                      topk_group=cfg.topk_group, routed_scale=cfg.routed_scale)
    touched = len(set(r["ids"].ravel().tolist()))
    closed = cfg.E * (1 - (1 - cfg.k / cfg.E) ** g["trace_T"])
    assert abs(closed - g["trace_touched_approx"]) < 1.0
    assert abs(touched - closed) < 0.08 * closed
    sid, bexp, total, bad = oalign.align(r["ids"].tolist(), cfg.E, g["trace_block_m"])
    assert len(sid) == g["trace_max_padded"] and len(bexp) == g["trace_expert_id_entries"]
    counts = np.bincount(r["ids"].ravel(), minlength=cfg.E)
    assert total == sum(-(-c // 16) * 16 for c in counts)
    assert abs(total - g["trace_padded_rows_approx"]) < 0.08 * g["trace_padded_rows_approx"]
    assert not bad

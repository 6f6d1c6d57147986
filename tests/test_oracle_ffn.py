"""Pins for the expert / combine / layer oracle: the [MoE] numpy combine
example, grouped == direct, the E = 1 reduction to a dense SwiGLU MLP
computed with torch's own silu and matmul, exact dequantisation checked
against torch's float8 cast, and error bounds of the activation quantiser."""

import numpy as np
import pytest
import torch

from oracle import ffn as offn
from oracle import formats as fm
from oracle import router as orouter
from synth import get_config, make_inputs, to_numpy
from synth.generate import quantize_fp8_block, quantize_mxfp4


def test_combine_example(golden):
    g = golden("combine_numpy.json")
    x = np.array(g["x"])
    scal = g["expert_scalars"]

    def expert_fn(e, rows):
        return rows @ (scal[e] * np.eye(2)).T

    yd, _ = offn.layer_direct(x, g["ids"], g["routing"], expert_fn)
    yg, _ = offn.layer_grouped(x, g["ids"], g["routing"], expert_fn, E=3)
    assert np.allclose(yd, g["derived_y"], rtol=0, atol=1e-14)
    assert np.allclose(yg, yd, rtol=0, atol=1e-14)


@pytest.mark.parametrize("fmt", ["bf16", "fp8", "mxfp4"])
def test_grouped_equals_direct(fmt):
    cfg = get_config("toy", wformat=fmt, E=6, k=3, H=256, F=128)
    inp = make_inputs(cfg, 24)
    W = offn.ExpertWeights(fmt, to_numpy(inp["w13"]), to_numpy(inp["w2"]),
                           to_numpy(inp["w13_scale"]), to_numpy(inp["w2_scale"]))
    r = orouter.route(to_numpy(inp["x"]), inp["gate"].numpy(), None, cfg.k, "softmax")
    x = fm.bf16_bits_to_f64(to_numpy(inp["x"]))
    fn = offn.make_expert_fn(W)
    yd, od = offn.layer_direct(x, r["ids"], r["weights"], fn)
    yg, og = offn.layer_grouped(x, r["ids"], r["weights"], fn, cfg.E)
    scale = np.abs(yd).max()
    assert np.abs(yd - yg).max() <= 1e-12 * scale
    assert np.abs(od - og).max() <= 1e-12 * np.abs(od).max()


def test_single_expert_is_dense_swiglu_mlp():
    """E = 1, k = 1 with renormalisation: the routed weight is 1 and the layer
    is the dense MLP w2 . (silu(w1 x) * (w3 x)) for every token."""
    cfg = get_config("toy", E=1, k=1, H=128, F=64)
    inp = make_inputs(cfg, 10)
    xb = to_numpy(inp["x"])
    r = orouter.route(xb, inp["gate"].numpy(), None, 1, "softmax")
    assert np.all(r["weights"] == 1.0)
    W = offn.ExpertWeights("bf16", to_numpy(inp["w13"]), to_numpy(inp["w2"]))
    y, _ = offn.layer(xb, r, W, E=1)
    xt = inp["x"].to(torch.float64)
    w13 = inp["w13"][0].to(torch.float64)
    w2 = inp["w2"][0].to(torch.float64)
    ref = torch.nn.functional.silu(xt @ w13[:64].T) * (xt @ w13[64:].T)
    ref = ref @ w2.T
    assert np.allclose(y, ref.numpy(), rtol=1e-12, atol=1e-14)


def test_fp8_block_dequant_matches_torch():
    g = torch.Generator().manual_seed(7)
    w = torch.randn((256, 384), generator=g) * 0.02
    codes, scale = quantize_fp8_block(w)
    ours = offn.dequant("fp8", codes.numpy(), scale.numpy())
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64)
    ref = ref * scale.to(torch.float64).repeat_interleave(128, 0).repeat_interleave(128, 1)
    assert np.array_equal(ours, ref.numpy())
    # and the stored values approximate the generating weights
    assert np.abs(ours - w.numpy()).max() <= 0.07 * np.abs(w.numpy()).max()


def test_mxfp4_dequant_hand_example():
    # one row of 32: codes 0..15 twice, scale code 126 (0.5)
    codes = np.array(list(range(16)) * 2, dtype=np.uint8)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)[None, :]
    vals = offn.dequant("mxfp4", packed, np.array([[126]], dtype=np.uint8))
    table = [0, .5, 1, 1.5, 2, 3, 4, 6]
    expect = np.array((table + [-v for v in table]) * 2) * 0.5
    assert np.array_equal(vals[0], expect)


def test_mxfp4_generator_roundtrip_is_nearest():
    g = torch.Generator().manual_seed(8)
    w = torch.randn((8, 64), generator=g)
    packed, e8 = quantize_mxfp4(w)
    vals = offn.dequant("mxfp4", packed.numpy(), e8.numpy())
    s = fm.e8m0_decode(e8.numpy()).repeat(32, axis=1)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    full = np.concatenate([-grid[::-1], grid])
    v = w.numpy() / s
    best = np.abs(np.clip(v, -6, 6)[..., None] - full).min(axis=-1)
    assert np.allclose(np.abs(vals / s - np.clip(v, -6, 6)), best, atol=1e-6)


@pytest.mark.parametrize("fmt,group", [("fp8", 128), ("mxfp4", 32)])
def test_activation_quantiser_error_bound(fmt, group):
    rng = np.random.default_rng(9)
    v = rng.normal(0, 1, size=(6, 256)).astype(np.float32).astype(np.float64)  # fp32 values, as the kernels hold
    v[2, :group] = 0.0  # an all-zero group
    q = offn.quantize_act(v, fmt)
    assert np.all(q[2, :group] == 0.0)
    for c0 in range(0, 256, group):
        blk, qb = v[:, c0:c0 + group], q[:, c0:c0 + group]
        amax = np.abs(blk).max(axis=1, keepdims=True)
        # e4m3 keeps 3 mantissa bits: |error| <= 2^-4 |v| in the normal
        # range, plus a subnormal floor of half of 2^-9 times the scale
        s = np.where(amax > 0, amax / 448.0, 1.0) if fmt == "fp8" else \
            np.array([[fm.pow2_at_least(a / 448.0) if a > 0 else 1.0] for a in amax[:, 0]])
        assert np.all(np.abs(qb - blk) <= 2.0 ** -4 * np.abs(blk) + 2.0 ** -10 * s + 1e-6 * np.abs(blk))
        assert np.all(np.abs(qb) <= 448.0 * s * (1 + 1e-6))


_E4M3_GRID = fm.e4m3_decode(np.arange(256, dtype=np.uint8))
_E4M3_GRID = _E4M3_GRID[np.isfinite(_E4M3_GRID)]


@pytest.mark.parametrize("fmt,group", [("fp8", 128), ("mxfp4", 32)])
def test_activation_quantiser_keeps_grid_values_with_pow2_group_scales(fmt, group):
    """Each group is e4m3 values times its own power of two, with one element
    at +-448 times it: the group's scale is exactly that power of two (amax /
    448, and the smallest power of two at least amax / 448, agree), so the
    quantiser returns every value unchanged.  A wrong group size, a scale
    from another group or a wrong scale rule changes some of them."""
    rng = np.random.default_rng(3)
    n, K = 5, 4 * group
    codes = rng.choice(_E4M3_GRID[np.abs(_E4M3_GRID) <= 256], size=(n, K))
    j = rng.integers(-6, 7, size=(n, K // group))
    codes[:, ::group] = np.where(rng.random((n, K // group)) < 0.5, -448.0, 448.0)
    v = codes * np.repeat(np.exp2(j.astype(np.float64)), group, axis=1)
    assert np.array_equal(offn.quantize_act(v, fmt), v)


@pytest.mark.parametrize("fmt,group", [("fp8", 128), ("mxfp4", 32)])
def test_activation_quantiser_scales_each_group_by_its_own_amax(fmt, group):
    """Neighbouring groups whose magnitudes differ by 10^6 (and an all-zero
    group): every group keeps its largest element to rounding (fp8: it maps to
    448 exactly; MX: to the e4m3 value nearest amax / s with s = the smallest
    power of two at least amax / 448) and the zero group stays zero.  A scale
    taken from the neighbouring group would flush the small group to zero or
    saturate the large one."""
    rng = np.random.default_rng(4)
    n, G = 4, 6
    v = rng.normal(0, 1, size=(n, G * group))
    mag = np.where(np.arange(G) % 2 == 0, 1e3, 1e-3)
    v = (v * np.repeat(mag, group)[None, :]).astype(np.float32)  # fp32 values, as the kernels hold
    v[1, 2 * group:3 * group] = 0.0
    q = offn.quantize_act(v, fmt)
    assert np.all(q[1, 2 * group:3 * group] == 0.0)
    for i in range(n):
        for g in range(G):
            blk, qb = v[i, g * group:(g + 1) * group], q[i, g * group:(g + 1) * group]
            amax = np.abs(blk).max()
            if amax == 0:
                continue
            m = np.argmax(np.abs(blk))
            # the scale and the scaled values in fp32
            q32 = amax / np.float32(448.0)
            s = float(q32) if fmt == "fp8" else fm.pow2_at_least(float(q32))
            scaled = (blk / np.float32(s)).astype(np.float64)
            assert 224.0 < scaled[m] * np.sign(blk[m]) <= 448.0 * (1 + 1e-6)
            # the group's largest element lands on (or next to) 448 x s
            assert abs(qb[m]) == pytest.approx(s * fm.e4m3_round(abs(scaled[m])), rel=1e-15)
            # every element is s times its nearest e4m3 value (brute force
            # over all 254 finite codes; ties have measure zero here)
            near = _E4M3_GRID[np.argmin(np.abs(_E4M3_GRID[None, :] - np.minimum(np.abs(scaled), 448.0)[:, None]),
                                        axis=1)] * np.sign(scaled)
            assert np.allclose(qb, s * near, rtol=1e-15, atol=0)


def test_mx_activation_scale_is_the_smallest_power_of_two_at_least_amax_over_448():
    """The MX activation scale ([MegaMoE] §3.5: a power of two at least
    amax / 448, the smallest one): amax exactly 448 * 2^j takes 2^j (the
    element maps to 448); a hair above takes 2^(j+1) (the element maps to
    224, the rest of the group halves its resolution); a hair below keeps
    2^j."""
    for j in (-3, 0, 5):
        for amax, scale in ((448.0 * 2.0 ** j, 2.0 ** j), (448.0 * 2.0 ** j * (1 + 2.0 ** -20), 2.0 ** (j + 1)),
                            (448.0 * 2.0 ** j * (1 - 2.0 ** -20), 2.0 ** j)):
            v = np.zeros((1, 32))
            v[0, 7] = amax
            v[0, 8] = 3.0 * 2.0 ** j  # 3 * 2^j / scale is on the e4m3 grid for both scales
            q = offn.quantize_act(v, "mxfp4")
            assert q[0, 7] == scale * fm.e4m3_round(amax / scale)
            assert q[0, 8] == 3.0 * 2.0 ** j
            assert fm.pow2_at_least(amax / 448.0) == scale
    assert np.array_equal(fm.pow2_at_least(np.array([0.75, 1.0, 1.5, 2.0 ** -130])),
                          np.array([1.0, 1.0, 2.0, 2.0 ** -130]))


def test_swiglu_clamp_worked_values_and_bounds():
    """[MegaMoE] §3.5: gate capped at L, up clipped to [-L, L] before SwiGLU.
    Hand values, L = inf as the plain SwiGLU, inputs inside the limit
    unchanged, and |act| <= max(silu(L), silu's minimum magnitude) * L."""
    import math
    silu = lambda v: v / (1.0 + math.exp(-v))
    assert offn.swiglu(5.0, -7.0, 3.0) == pytest.approx(silu(3.0) * -3.0, rel=1e-15)
    assert offn.swiglu(-2.0, 10.0, 3.0) == pytest.approx(silu(-2.0) * 3.0, rel=1e-15)  # no lower cap on the gate
    assert offn.swiglu(-40.0, -2.0, 3.0) == pytest.approx(silu(-40.0) * -2.0, rel=1e-15)
    rng = np.random.default_rng(11)
    g, u = rng.normal(0, 4, size=(2, 5000))
    assert np.array_equal(offn.swiglu(g, u), offn.silu(g) * u)
    assert np.array_equal(offn.swiglu(g, u, np.inf), offn.silu(g) * u)
    inside = (np.abs(g) < 2.5) & (np.abs(u) < 2.5)
    assert np.array_equal(offn.swiglu(g, u, 2.5)[inside], (offn.silu(g) * u)[inside])
    L = 2.5
    bound = max(silu(L), 0.2785) * L
    assert np.all(np.abs(offn.swiglu(g, u, L)) <= bound + 1e-12)
    assert np.any(np.abs(offn.swiglu(g, u, L)) > 0.9 * silu(L) * L)  # the cap is reached


def test_shared_expert_slot_is_routed_sum_plus_dense_expert():
    """The shared expert as slot k (id E, weight 1) gives the routed layer
    plus the shared expert's dense forward on every token."""
    cfg = get_config("toy", E=6, k=2, H=128, F=128)
    d = make_inputs(cfg, 9)
    from synth import make_weights
    W = make_weights(cfg, "cpu", n_shared=1)
    xb = to_numpy(d["x"])
    r = orouter.route(xb, to_numpy(W["gate"]), None, cfg.k, cfg.scoring)
    rs = orouter.with_shared_expert(r, cfg.E)
    assert rs["ids"].shape == (9, 3) and np.all(rs["ids"][:, 2] == cfg.E) and np.all(rs["weights"][:, 2] == 1.0)
    assert np.array_equal(rs["ids"][:, :2], r["ids"]) and np.array_equal(rs["weights"][:, :2], r["weights"])
    ew = offn.ExpertWeights("bf16", to_numpy(W["w13"]), to_numpy(W["w2"]))
    y_shared, _ = offn.layer(xb, rs, ew, cfg.E + 1)
    y_routed, _ = offn.layer(xb, r, ew, cfg.E + 1)
    W13, W2 = ew.expert(cfg.E)
    x = fm.bf16_bits_to_f64(xb)
    dense = x @ W13[:cfg.F].T, x @ W13[cfg.F:].T
    y_dense = (dense[0] / (1.0 + np.exp(-dense[0])) * dense[1]) @ W2.T
    assert np.allclose(y_shared, y_routed + y_dense, rtol=1e-12, atol=1e-15)

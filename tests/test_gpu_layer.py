"""GPU parity of moe_layer / moe_expert_ffn against the float64 oracle, on
every token: relative Frobenius error within the layer tolerance (2e-2 bf16, 5e-2 fp8 / MXFP4) and
every token's own error within three times it, at small sizes (several
tiles, ragged tails, every BLOCK_M) and at the full layer shapes in the
launch configuration the benchmark uses; for fp8 / MXFP4 also against the
oracle that quantises activations as the kernels do; plus HIP-graph capture
and determinism."""

import numpy as np
import pytest
import torch

from helpers import (EMULATE_TOL, LAYER_TOL, bf16_to_f64, check_output, check_routing, oracle_layer, oracle_route,
                     rel_fro, routing_for_layer, say)
from synth import get_config, make_weights, make_x

pytestmark = pytest.mark.gpu

_CACHE = {}


def weights_for(cfg):
    key = cfg
    if key not in _CACHE:
        _CACHE.clear()
        torch.cuda.empty_cache()
        _CACHE[key] = make_weights(cfg, "cuda")
    return _CACHE[key]


def run_layer(cfg, W, x, block_m=0, limit=np.inf):
    import mixture_experts_layer_04_amd as moe
    return moe.layer(x, W["gate"], W["bias"], W["w13"], W["w2"], cfg.k, cfg.scoring, cfg.n_group,
                     cfg.topk_group, cfg.renormalize, cfg.routed_scale, wformat=cfg.wformat,
                     w13_scale=W["w13_scale"], w2_scale=W["w2_scale"], block_m=block_m, return_routing=True,
                     swiglu_limit=limit)


def check_layer(cfg, T, block_m=0, limit=np.inf, dense=True, gate_bf16=False):
    """moe_layer against the oracle on every token.  ``dense``: against the
    dense-equivalent oracle (the headline tolerance); the quantised formats
    are also checked against the emulate-mode oracle.  ``gate_bf16``: the
    router takes the gate rows rounded to bf16 (both sides)."""
    say(f"layer {cfg.name} {cfg.wformat} E={cfg.E} H={cfg.H} F={cfg.F} k={cfg.k} T={T} block_m={block_m}"
        + (f" SwiGLU limit {limit}" if np.isfinite(limit) else "") + (" bf16 gate" if gate_bf16 else ""))
    W = weights_for(cfg)
    if gate_bf16:
        W = dict(W, gate=W["gate"].to(torch.bfloat16))
    x = make_x(cfg, T, "cuda")
    y, ids, w = run_layer(cfg, W, x, block_m, limit)
    torch.cuda.synchronize()
    r = oracle_route(cfg, x, W["gate"], W["bias"])
    check_routing(cfg, r, ids.cpu().numpy(), w.cpu().numpy())
    routing = routing_for_layer(cfg, r, ids.cpu().numpy())
    got = bf16_to_f64(y)
    err = None
    if dense:
        y_ref = oracle_layer(cfg, x, routing, W, limit=limit)
        err, _, _ = check_output(got, y_ref, LAYER_TOL[cfg.wformat], "dense-equivalent oracle")
    if cfg.wformat != "bf16":
        y_em = oracle_layer(cfg, x, routing, W, mode="emulate", limit=limit)
        e_em, _, _ = check_output(got, y_em, EMULATE_TOL, "emulate-mode oracle")
        err = e_em if err is None else err
    return x, W, y, ids, w, err


SMALL = [
    ("toy", {}, 16, 0),
    ("toy", dict(F=256), 100, 16),
    ("toy", dict(F=256), 100, 32),
    ("toy", dict(F=256), 300, 64),
    ("toy", dict(F=256), 300, 128),
    ("toy", dict(E=16, k=4, H=384, F=256, scoring="sigmoid", has_bias=True), 333, 0),
    ("toy", dict(E=16, k=4, H=256, F=128, scoring="sigmoid", has_bias=True, n_group=4, topk_group=2,
                 routed_scale=2.5), 64, 16),
    ("toy", dict(E=1, k=1, H=128, F=128), 19, 16),
    ("toy", dict(E=16, k=4, H=256, F=128, scoring="sqrtsoftplus", has_bias=True), 50, 16),
    # fp8 128x128 block scales (DeepSeek-V3 routing), several tiles and ragged tails
    ("dsv3", dict(E=16, H=512, F=512, k=4, n_group=4, topk_group=2), 37, 16),
    ("dsv3", dict(E=16, H=512, F=512, k=4, n_group=4, topk_group=2), 300, 32),
    ("dsv3", dict(E=16, H=1024, F=512, k=4, n_group=4, topk_group=2), 300, 64),
    ("dsv3", dict(E=8, H=512, F=1024, k=2, n_group=4, topk_group=2), 700, 128),
    # MXFP4 weights x fp8 activations (DeepSeek-V4 routing)
    ("dsv4", dict(E=16, H=512, F=512, k=4), 37, 16),
    ("dsv4", dict(E=16, H=512, F=512, k=4), 300, 32),
    ("dsv4", dict(E=16, H=1024, F=512, k=4), 300, 64),
    ("dsv4", dict(E=8, H=512, F=1024, k=2), 700, 128),
    # one GPU's share of DeepSeek-V4 over 8 GPUs: 32 experts at full dimensions
    ("dsv4", dict(E=32), 16, 0),
]


@pytest.mark.parametrize("name,over,T,bm", SMALL)
def test_layer_small_all_tokens(name, over, T, bm):
    cfg = get_config(name, **over)
    check_layer(cfg, T, bm)


CLAMPED = [("toy", dict(F=256), 100, 16, 0.25, True), ("toy", dict(F=256), 300, 64, 0.25, True),
           ("toy", dict(F=256), 300, 128, 0.25, True),
           # quantised formats at the same limit: judged against the oracle
           # that quantises the activations as the kernels do (a limit this
           # low leaves most SwiGLU values at a few levels, where one e4m3
           # rounding is a larger share of the dense-equivalent result)
           ("dsv3", dict(E=16, H=512, F=512, k=4, n_group=4, topk_group=2), 300, 32, 0.25, False),
           ("dsv3", dict(E=16, H=512, F=512, k=4, n_group=4, topk_group=2), 37, 16, 0.25, False),
           ("dsv4", dict(E=16, H=512, F=512, k=4), 37, 16, 0.25, False),
           ("dsv4", dict(E=8, H=512, F=1024, k=2), 700, 128, 0.25, False),
           ("dsv4", dict(E=16, H=512, F=512, k=4), 300, 32, 0.5, True)]


@pytest.mark.parametrize("name,over,T,bm,limit,dense", CLAMPED)
def test_layer_swiglu_clamp(name, over, T, bm, limit, dense):
    """The DeepSeek-V4 SwiGLU clamp ([MegaMoE] §3.5) with a limit that a
    large share of the gate and up values exceed (they are ~N(0, 0.3))."""
    cfg = get_config(name, **over)
    x, W, y, ids, w, err = check_layer(cfg, T, bm, limit=limit, dense=dense)
    # the clamp changes the layer by far more than the tolerance
    r = oracle_route(cfg, x, W["gate"], W["bias"])
    routing = routing_for_layer(cfg, r, ids.cpu().numpy())
    diff = rel_fro(oracle_layer(cfg, x, routing, W), oracle_layer(cfg, x, routing, W, limit=limit))
    say(f"  clamped vs unclamped oracle: {diff:.3e}")
    assert diff > 3 * LAYER_TOL[cfg.wformat]


FULL = [("qwen3", 1), ("qwen3", 64), ("qwen3", 1024), ("qwen3", 4096), ("glm", 1), ("glm", 8), ("glm", 512),
        ("dsv3", 1), ("dsv3", 256), ("dsv3", 2048), ("dsv4", 512), ("dsv4", 8192)]


@pytest.mark.parametrize("name,T", FULL)
def test_layer_full_size_all_tokens(name, T):
    """The configurations' own shapes, in the launch configuration bench.py
    times (block_m chosen by the library), every token compared."""
    cfg = get_config(name)
    check_layer(cfg, T, 0)


# the router on bf16 gate rows inside the layer: the one-launch decode
# router with its fused alignment (and x quantisation for MXFP4), and the
# prefill layout
BF16_GATE = [("toy", dict(E=16, k=4, H=384, F=256, scoring="sigmoid", has_bias=True), 333, 0),
             ("toy", dict(F=256), 3, 0), ("dsv4", dict(E=16, H=1024, F=512, k=4), 2, 0),
             ("dsv4", dict(E=16, H=1024, F=512, k=4), 300, 64), ("glm", {}, 8, 0)]


@pytest.mark.parametrize("name,over,T,bm", BF16_GATE)
def test_layer_bf16_gate(name, over, T, bm):
    cfg = get_config(name, **over)
    check_layer(cfg, T, bm, gate_bf16=True)


RENORM_OFF = [("toy", dict(F=256), 100, 16), ("qwen3", {}, 64, 0)]


@pytest.mark.parametrize("name,over,T,bm", RENORM_OFF)
def test_layer_softmax_without_renormalisation(name, over, T, bm):
    """Softmax top-k without renormalisation ([MoE] fused_topk listing, the
    renormalize flag): the weights are the chosen experts' softmax
    probabilities, which sum to less than one."""
    cfg = get_config(name, **dict(over, renormalize=False))
    x, W, y, ids, w, err = check_layer(cfg, T, bm)
    s = w.sum(dim=1).cpu().numpy()
    assert np.all(s < 1.0) and np.all(s > 0.0)


MATCH = [("toy", dict(F=256), 200, 32), ("toy", dict(F=256), 300, 128),
         ("dsv3", dict(E=16, H=512, F=512, k=4, n_group=4, topk_group=2), 37, 16),
         ("dsv3", dict(E=16, H=512, F=512, k=4, n_group=4, topk_group=2), 250, 32),
         ("dsv3", dict(E=16, H=512, F=512, k=4, n_group=4, topk_group=2), 300, 32),
         ("dsv4", dict(E=16, H=512, F=512, k=4), 37, 16), ("dsv4", dict(E=16, H=1024, F=512, k=4), 200, 64),
         ("dsv4", dict(E=16, H=1024, F=512, k=4), 400, 64)]


@pytest.mark.parametrize("name,over,T,bm", MATCH)
def test_expert_ffn_matches_layer(name, over, T, bm):
    """moe_layer gives the bits of moe_align + moe_expert_ffn on its routing.
    For the fp8 formats, where the router takes its one-launch decode layout
    (small T), it quantises x on the way and the FFN skips its quantisation
    kernel; elsewhere both quantise in the FFN."""
    import mixture_experts_layer_04_amd as moe
    cfg = get_config(name, **over)
    x, W, y, ids, w, _ = check_layer(cfg, T, bm)
    s, b, n = moe.align(ids, cfg.E, bm)
    y2 = moe.expert_ffn(x, W["w13"], W["w2"], ids, w, s, b, n, bm, wformat=cfg.wformat,
                        w13_scale=W["w13_scale"], w2_scale=W["w2_scale"])
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_layer_graph_capture_and_determinism():
    import mixture_experts_layer_04_amd as moe
    cfg = get_config("toy", F=256)
    W = weights_for(cfg)
    x = make_x(cfg, 150, "cuda")

    def call(out):
        return moe.layer(x, W["gate"], W["bias"], W["w13"], W["w2"], cfg.k, cfg.scoring, block_m=0, out=out)

    ref = call(None).clone()
    assert torch.equal(call(None), ref)  # deterministic
    y_static = torch.empty_like(ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(y_static)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(y_static)
    for i in range(3):
        y_static.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_static, ref), f"replay {i} differs"
        other = call(None)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(other, ref)


def test_layer_shapes_share_one_workspace():
    """Calls of different shapes (fused decode paths included) on one
    workspace give the bits of calls on fresh zeroed workspaces: every
    counter lives in the control block at the workspace's start and is left
    at zero."""
    import mixture_experts_layer_04_amd as moe
    shapes = [(dict(F=256), 100, 16), (dict(E=16, k=4, H=256, F=128, scoring="sigmoid", has_bias=True, n_group=4,
                                          topk_group=2, routed_scale=2.5), 64, 16),
              (dict(F=256), 3, 0), (dict(E=16, k=4, H=256, F=128), 17, 0), (dict(F=256), 100, 16),
              # paired bf16 tiles with their tile queues, at two shapes
              (dict(F=256), 300, 128), (dict(E=16, k=4, H=256, F=128), 700, 128), (dict(F=256), 300, 128)]
    shared = torch.zeros(1 << 26, dtype=torch.uint8, device="cuda")
    for over, T, bm in shapes:
        cfg = get_config("toy", **over)
        W = make_weights(cfg, "cuda")
        x = make_x(cfg, T, "cuda")
        kw = dict(wformat=cfg.wformat, w13_scale=W["w13_scale"], w2_scale=W["w2_scale"], block_m=bm)
        args = (x, W["gate"], W["bias"], W["w13"], W["w2"], cfg.k, cfg.scoring, cfg.n_group, cfg.topk_group,
                cfg.renormalize, cfg.routed_scale)
        need = moe.layer_workspace_size(T, cfg.H, cfg.E, cfg.F, cfg.k, bm, cfg.wformat)
        assert need <= shared.numel()
        y = moe.layer(*args, ws=shared, **kw)
        fresh = torch.zeros(need, dtype=torch.uint8, device="cuda")
        y_ref = moe.layer(*args, ws=fresh, **kw)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), (over, T, bm)
        assert int(shared[:65536].count_nonzero()) == 0, "control block not left at zero"


SHARED = [("toy", {}, 16, 0), ("toy", dict(F=256), 100, 16), ("toy", dict(F=256), 300, 64),
          ("toy", dict(F=256), 300, 128),
          ("dsv3", dict(E=16, H=512, F=512, k=4, n_group=4, topk_group=2), 300, 32),
          ("dsv4", dict(E=16, H=512, F=512, k=4), 37, 16), ("dsv4", dict(E=8, H=512, F=1024, k=2), 700, 128),
          ("dsv3", {}, 1, 0), ("dsv4", {}, 512, 0)]


@pytest.mark.parametrize("name,over,T,bm", SHARED)
def test_layer_shared_expert(name, over, T, bm):
    """The shared expert as an always-selected slot (id E, weight 1): the
    router writes slot k, the alignment and the grouped GEMMs treat it as
    expert E, and y adds its output (full DSV3 / DSV4 shapes included),
    every token compared."""
    import mixture_experts_layer_04_amd as moe
    cfg = get_config(name, **over)
    say(f"layer + shared expert {cfg.name} {cfg.wformat} E={cfg.E}+1 k={cfg.k}+1 T={T} block_m={bm}")
    _CACHE.clear()
    torch.cuda.empty_cache()
    W = make_weights(cfg, "cuda", n_shared=1)
    x = make_x(cfg, T, "cuda")
    y, ids, w = moe.layer(x, W["gate"], W["bias"], W["w13"], W["w2"], cfg.k, cfg.scoring, cfg.n_group,
                          cfg.topk_group, cfg.renormalize, cfg.routed_scale, wformat=cfg.wformat,
                          w13_scale=W["w13_scale"], w2_scale=W["w2_scale"], block_m=bm, return_routing=True,
                          n_shared=1)
    torch.cuda.synchronize()
    ids, w = ids.cpu().numpy(), w.cpu().numpy()
    assert ids.shape == (T, cfg.k + 1)
    assert np.all(ids[:, cfg.k] == cfg.E) and np.all(w[:, cfg.k] == 1.0)
    r = oracle_route(cfg, x, W["gate"], W["bias"])
    check_routing(cfg, r, ids[:, :cfg.k], w[:, :cfg.k])
    from oracle import router as orouter
    routing = orouter.with_shared_expert(routing_for_layer(cfg, r, ids[:, :cfg.k]), cfg.E)
    y_ref = oracle_layer(get_config(name, **dict(over, E=cfg.E + 1)), x, routing, W)
    check_output(bf16_to_f64(y), y_ref, LAYER_TOL[cfg.wformat], "dense-equivalent oracle")

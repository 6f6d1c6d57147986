"""GPU parity of moe_route_align (one launch for T <= 4): its ids and
weights equal moe_route's bit for bit, and its sorted_ids, block table and
padded length equal moe_align's on those ids and the oracle alignment's,
over one and several token tiles, group-limited routing, every BLOCK_M and
the prefill path (larger T)."""

import pytest
import torch

from helpers import oracle_align, say
from synth import get_config, make_router_weights, make_x

pytestmark = pytest.mark.gpu

CASES = [("toy", 16, 16), ("qwen3", 1, 16), ("qwen3", 17, 32), ("qwen3", 64, 16), ("glm", 1, 16), ("glm", 8, 64),
         ("dsv3", 1, 16), ("dsv3", 256, 128), ("dsv4", 3, 16), ("qwen3", 256, 64), ("glm", 300, 32),
         ("qwen3", 1, 1), ("glm", 33, 128)]


@pytest.mark.parametrize("name,T,bm", CASES)
def test_route_align_matches_route_then_align(name, T, bm):
    import mixture_experts_layer_04_amd as moe
    cfg = get_config(name)
    say(f"route+align {name} T={T} block_m={bm}")
    gate, bias = make_router_weights(cfg, "cuda")
    x = make_x(cfg, T, "cuda")
    args = (cfg.k, cfg.scoring, cfg.n_group, cfg.topk_group, cfg.renormalize, cfg.routed_scale)
    ids, w, s, b, n = moe.route_align(x, gate, bias, cfg.k, bm, *args[1:])
    ids_r, w_r = moe.route(x, gate, bias, *args)
    s_r, b_r, n_r = moe.align(ids_r, cfg.E, bm)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids_r)
    assert torch.equal(w.view(torch.int32), w_r.view(torch.int32))
    assert int(n.item()) == int(n_r.item())
    assert torch.equal(s, s_r) and torch.equal(b, b_r)
    so, bo, no, bad = oracle_align(ids, cfg.E, bm)
    assert not bad and int(n.item()) == no and s.cpu().tolist() == so and b.cpu().tolist() == bo


def test_route_align_repeated_calls_share_one_workspace():
    """The control-block counters return to zero: back-to-back calls of
    different shapes on one workspace give the same results as fresh ones."""
    import mixture_experts_layer_04_amd as moe
    ws = None
    for name, T, bm in (("qwen3", 40, 16), ("glm", 5, 32), ("qwen3", 40, 16), ("dsv3", 100, 64)):
        cfg = get_config(name)
        gate, bias = make_router_weights(cfg, "cuda")
        x = make_x(cfg, T, "cuda")
        need = moe.lib().moe_route_align_workspace_size(T, cfg.H, cfg.E, cfg.k, 0)
        if ws is None or ws.numel() < need:
            ws = torch.zeros(max(need, 1 << 22), dtype=torch.uint8, device="cuda")
        out = moe.route_align(x, gate, bias, cfg.k, bm, cfg.scoring, cfg.n_group, cfg.topk_group,
                              cfg.renormalize, cfg.routed_scale, ws=ws)
        ref = moe.route_align(x, gate, bias, cfg.k, bm, cfg.scoring, cfg.n_group, cfg.topk_group,
                              cfg.renormalize, cfg.routed_scale)
        for a, r in zip(out, ref):
            assert torch.equal(a, r)


@pytest.mark.parametrize("name,T,bm", [("dsv3", 1, 16), ("dsv3", 37, 32), ("dsv4", 300, 64), ("toy", 16, 16)])
def test_route_align_shared_expert_slot(name, T, bm):
    """n_shared = 1: slot k is (E, 1.0) for every token, the routed slots
    equal moe_route's, and the alignment equals moe_align over E + 1
    experts and k + 1 slots (and the oracle's)."""
    import mixture_experts_layer_04_amd as moe
    cfg = get_config(name)
    say(f"route+align + shared expert {name} T={T} block_m={bm}")
    gate, bias = make_router_weights(cfg, "cuda")
    x = make_x(cfg, T, "cuda")
    args = (cfg.scoring, cfg.n_group, cfg.topk_group, cfg.renormalize, cfg.routed_scale)
    ids, w, s, b, n = moe.route_align(x, gate, bias, cfg.k, bm, *args, n_shared=1)
    ids_r, w_r = moe.route(x, gate, bias, cfg.k, *args)
    torch.cuda.synchronize()
    assert ids.shape == (T, cfg.k + 1)
    assert torch.equal(ids[:, :cfg.k], ids_r) and torch.equal(w[:, :cfg.k].view(torch.int32), w_r.view(torch.int32))
    assert bool((ids[:, cfg.k] == cfg.E).all()) and bool((w[:, cfg.k] == 1.0).all())
    s_r, b_r, n_r = moe.align(ids.contiguous(), cfg.E + 1, bm)
    assert torch.equal(s, s_r) and torch.equal(b, b_r) and int(n.item()) == int(n_r.item())
    so, bo, no, bad = oracle_align(ids, cfg.E + 1, bm)
    assert not bad and s.cpu().tolist() == so and b.cpu().tolist() == bo and int(n.item()) == no

"""moe_layer_noalloc (the layer on the library's own scratch array, for
callers that cannot allocate) against moe_layer on a caller workspace,
through the C ABI: bit-identical outputs and routing, on two calls in a row
per case, the second with a smaller input; plus the host-side size check."""

import ctypes

import numpy as np
import pytest
import torch

from helpers import say
from synth import get_config, make_weights, make_x

MOE_E_INVAL, MOE_E_WORKSPACE = 1, 3

# (configuration, overrides, first T, second T): bf16 paired tiles / fused
# decode path, fp8 stream kernel + requantisation, MXFP4 tiled kernel, a
# group-limited router; the second call is always the smaller one
CASES = [
    ("toy", dict(F=256), 300, 17, 0),
    ("qwen3", {}, 64, 1, 0),
    ("dsv3", dict(E=16, H=512, F=512, k=4, n_group=4, topk_group=2), 300, 3, 0),
    ("dsv4", dict(E=16, H=512, F=512, k=4), 200, 37, 0),
    ("toy", dict(F=256), 700, 300, 128),
]


def _call(moe, noalloc, cfg, W, x, bm):
    kw = dict(wformat=cfg.wformat, w13_scale=W["w13_scale"], w2_scale=W["w2_scale"], block_m=bm,
              return_routing=True)
    args = (x, W["gate"], W["bias"], W["w13"], W["w2"], cfg.k, cfg.scoring, cfg.n_group, cfg.topk_group,
            cfg.renormalize, cfg.routed_scale)
    if noalloc:
        return moe.layer_noalloc(*args, **kw)
    need = moe.layer_workspace_size(x.shape[0], cfg.H, cfg.E, cfg.F, cfg.k, bm, cfg.wformat)
    ws = torch.zeros(need, dtype=torch.uint8, device=x.device)
    return moe.layer(*args, ws=ws, **kw)


@pytest.mark.gpu
@pytest.mark.parametrize("name,over,T1,T2,bm", CASES)
def test_layer_noalloc_matches_layer(name, over, T1, T2, bm):
    import mixture_experts_layer_04_amd as moe
    cfg = get_config(name, **over)
    W = make_weights(cfg, "cuda")
    for T in (T1, T2):
        say(f"noalloc {cfg.name} {cfg.wformat} E={cfg.E} H={cfg.H} F={cfg.F} k={cfg.k} T={T} block_m={bm}")
        x = make_x(cfg, T, "cuda")
        y, ids, w = _call(moe, True, cfg, W, x, bm)
        y_ref, ids_ref, w_ref = _call(moe, False, cfg, W, x, bm)
        torch.cuda.synchronize()
        assert torch.equal(ids, ids_ref)
        assert torch.equal(w.view(torch.int32), w_ref.view(torch.int32))
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
        assert bool(torch.isfinite(y.float()).all())


def test_layer_noalloc_rejects_oversized_shapes():
    """Host-side checks only (no GPU work is enqueued): a shape whose
    workspace exceeds the scratch array returns MOE_E_WORKSPACE, bad scalars
    MOE_E_INVAL, and an empty batch MOE_OK."""
    from mixture_experts_layer_04_amd import _lib
    L = _lib.lib()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: every call fails or returns before any launch

    def call(T, H, E, F, k, wformat=0, bm=0):
        sc = fake if wformat else None
        return L.moe_layer_noalloc(fake, fake, 1, None, wformat, fake, sc, fake, sc, T, H, E, F, k, 0, 1, 1, 0, 1,
                                   1.0, bm, float("inf"), fake, None, None, None)

    big = (8192, 4096, 256, 2048, 6)  # the 8192-token DeepSeek-V4-Flash-shaped prefill
    need = L.moe_layer_workspace_size(*big, 0, 0, 2)
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    assert call(*big, wformat=2) == MOE_E_WORKSPACE
    assert call(4096, 2048, 128, 768, 8) == MOE_E_WORKSPACE  # 208 MiB
    assert L.moe_layer_workspace_size(512, 4096, 288, 2304, 8, 0, 0, 0) <= _lib.NOALLOC_SCRATCH_BYTES
    assert call(16, 192, 8, 128, 2) == MOE_E_INVAL   # H not a multiple of 128
    assert call(-1, 256, 8, 128, 2) == MOE_E_INVAL
    assert call(0, 256, 8, 128, 2) == 0
    assert np.isfinite(need)

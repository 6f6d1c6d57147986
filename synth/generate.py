"""Seeded generation of layer inputs.

Recipe (per configuration; every tensor has its own random stream derived
from (master seed, tensor name[, T])):

* x     ~ N(0, x_std^2) drawn in float32, rounded to bf16 (RNE)   [T, H]
* gate  ~ N(0, gate_std^2) float32                                [E, H]
* bias  ~ N(0, bias_std^2) float32 (sigmoid configurations)       [E]
* w13   ~ N(0, w_std^2) float32 [E, 2F, H], w2 [E, H, F], stored as
  - bf16 (RNE),
  - fp8: e4m3 codes with one float32 scale amax/448 per 128x128 block,
  - mxfp4: e2m1 codes (round to nearest, ties to even, saturating at 6)
    packed two per byte along K (even element in the low nibble) with one
    e8m0 scale 2^(floor(log2 amax) - 2) per 32 values along K (the OCP MX
    rule; an all-zero group gets 2^0).

Weights do not depend on T, hidden states do.  Generation runs with torch on
the requested device (the random streams of CPU and GPU generators differ;
within one test both the HIP path and the oracle see the same tensors).
"""

import hashlib

import numpy as np
import torch

from .configs import LayerConfig

_E2M1_MID = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


def _seed_for(*parts):
    h = hashlib.sha256("/".join(str(p) for p in parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, *parts):
    g = torch.Generator(device=device)
    g.manual_seed(_seed_for(*parts))
    return g


def _randn(shape, std, device, *parts):
    g = _gen(device, *parts)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def quantize_fp8_block(w):
    """float32 [N, K] (N, K multiples of 128) -> (e4m3 codes uint8 [N, K],
    float32 scales [N/128, K/128]) with scale = amax/448 per block."""
    N, K = w.shape
    assert N % 128 == 0 and K % 128 == 0, "fp8 block weights need multiples of 128"
    blk = w.reshape(N // 128, 128, K // 128, 128)
    amax = blk.abs().amax(dim=(1, 3))
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (blk / scale[:, None, :, None]).clamp(-448.0, 448.0).reshape(N, K)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale.contiguous()


def quantize_mxfp4(w):
    """float32 [N, K] (K multiple of 32) -> (packed e2m1 uint8 [N, K/2],
    e8m0 uint8 [N, K/32])."""
    N, K = w.shape
    assert K % 32 == 0
    g = w.reshape(N, K // 32, 32)
    amax = g.abs().amax(dim=2)
    safe = torch.where(amax > 0, amax, torch.ones_like(amax))
    exp = torch.floor(torch.log2(safe)) - 2.0
    exp = torch.where(amax > 0, exp, torch.zeros_like(exp)).clamp(-127, 127)
    v = g / torch.exp2(exp)[:, :, None]
    a = v.abs().clamp(max=6.0)
    mids = torch.tensor(_E2M1_MID, device=w.device, dtype=torch.float32)
    code = (a[..., None] > mids).sum(dim=-1)
    tie_up = ((a[..., None] == mids) & (torch.arange(7, device=w.device) % 2 == 1)).sum(dim=-1)
    code = (code + tie_up).to(torch.uint8)
    code = code | ((v < 0) & (code > 0)).to(torch.uint8) << 3
    code = code.reshape(N, K)
    packed = code[:, 0::2] | (code[:, 1::2] << 4)
    e8 = (exp + 127).to(torch.uint8)
    return packed.contiguous(), e8.contiguous()


def _weights(cfg: LayerConfig, device, which, N, K, n_shared=0):
    """All experts of one weight tensor in its storage format (E routed
    experts, then n_shared more)."""
    E = cfg.E + n_shared
    if cfg.wformat == "bf16":
        out = torch.empty((E, N, K), dtype=torch.bfloat16, device=device)
        for e in range(E):
            out[e] = _randn((N, K), cfg.w_std, device, cfg.seed, cfg.name, which, e).to(torch.bfloat16)
        return out, None
    if cfg.wformat == "fp8":
        out = torch.empty((E, N, K), dtype=torch.uint8, device=device)
        sc = torch.empty((E, N // 128, K // 128), dtype=torch.float32, device=device)
        for e in range(E):
            out[e], sc[e] = quantize_fp8_block(_randn((N, K), cfg.w_std, device, cfg.seed, cfg.name, which, e))
        return out, sc
    if cfg.wformat == "mxfp4":
        out = torch.empty((E, N, K // 2), dtype=torch.uint8, device=device)
        sc = torch.empty((E, N, K // 32), dtype=torch.uint8, device=device)
        for e in range(E):
            out[e], sc[e] = quantize_mxfp4(_randn((N, K), cfg.w_std, device, cfg.seed, cfg.name, which, e))
        return out, sc
    raise ValueError(cfg.wformat)


def make_router_weights(cfg: LayerConfig, device="cpu"):
    """Gate [E, H] float32 and selection bias [E] float32 (or None)."""
    gate = _randn((cfg.E, cfg.H), cfg.gate_std, device, cfg.seed, cfg.name, "gate")
    bias = _randn((cfg.E,), cfg.bias_std, device, cfg.seed, cfg.name, "bias") if cfg.has_bias else None
    return gate, bias


def make_weights(cfg: LayerConfig, device="cpu", n_shared=0):
    """Router and expert weights of a configuration (independent of T).
    With n_shared = 1 the expert tensors hold one more expert (index E, the
    shared expert); the gate keeps its E rows."""
    gate, bias = make_router_weights(cfg, device)
    w13, w13_scale = _weights(cfg, device, "w13", 2 * cfg.F, cfg.H, n_shared)
    w2, w2_scale = _weights(cfg, device, "w2", cfg.H, cfg.F, n_shared)
    return {"gate": gate, "bias": bias, "w13": w13, "w13_scale": w13_scale,
            "w2": w2, "w2_scale": w2_scale}


def make_x(cfg: LayerConfig, T, device="cpu", salt=""):
    return _randn((T, cfg.H), cfg.x_std, device, cfg.seed, cfg.name, "x", T, salt).to(torch.bfloat16)


def make_inputs(cfg: LayerConfig, T, device="cpu", weights=None):
    """x plus all weights; pass ``weights`` to reuse them across T."""
    d = dict(weights) if weights is not None else make_weights(cfg, device)
    d["x"] = make_x(cfg, T, device)
    return d


def make_topk_ids(T, k, E, seed=0, kind="uniform", device="cpu"):
    """Routing ids [T, k] int32 for alignment tests, distinct per token.

    kind: "uniform" - k distinct experts uniformly at random;
          "skewed"  - distinct experts drawn with Zipf(1.2) weights;
          "hot"     - every token routes to experts 0..k-1 (one expert set)."""
    if kind == "hot":
        return torch.arange(k, dtype=torch.int32, device=device).repeat(T, 1)
    g = _gen("cpu", seed, "ids", T, k, E, kind)
    if kind == "uniform":
        ids = torch.rand((T, E), generator=g).argsort(dim=1)[:, :k]
    elif kind == "skewed":
        p = 1.0 / torch.arange(1, E + 1, dtype=torch.float64) ** 1.2
        ids = torch.multinomial(p.expand(T, E).contiguous(), k, replacement=False, generator=g)
    else:
        raise ValueError(kind)
    return ids.to(torch.int32).to(device)


def to_numpy(t):
    """A torch tensor -> numpy on the host, keeping the stored bits
    (bf16 -> uint16, fp8 / packed fp4 / e8m0 -> uint8)."""
    if t is None:
        return None
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cpu().numpy()
    return t.cpu().numpy()

"""Exact-arithmetic parity of moe_expert_ffn (bf16, fp8, MXFP4 weights).

The inputs are built so that every value the path produces is exactly
representable and every sum is exact in fp32, whatever the order:

* x holds small integers (-4..4), a column of 8, a column of 2, and 448 in
  every 32nd column (so each 1x128 and 1x32 activation group has amax 448 and
  the fp8 / MX activation scale is exactly 1);
* each gate row has 4 at the column of 8: g = 32 for every token, and
  silu(32) rounds to 32 in fp32;
* each up row has +-1 at three integer columns (|u| <= 12), except every 32nd
  SwiGLU column, whose up row (1.5 at the 8-column, 1 at the 2-column) gives
  u = 14, i.e. act = 448 = the e4m3 maximum, so the requantisation scales of
  the SwiGLU output are exactly 1 as well; every act = 32 u is on the e4m3
  grid;
* each w2 row has +-1 at two non-448 SwiGLU columns (|out| <= 768, a multiple
  of 32: exact in bf16);
* routing weights are 0.25 or 0.5 (k = 2): y is a multiple of 8 below 768.

The weight values are on the bf16, e4m3 and e2m1 grids with unit scales, so
the GPU result must equal the exact value (the float64 oracle rounded to the
nearest integer, all outputs being multiples of 8; a zero may come out as
-0) for every BLOCK_M and tile shape.  Together with the random-input parity tests
this pins the gather through sorted_ids, the gate / up row pairing, the
SwiGLU column, the GEMM2 scatter to the assignment slot and the slot-order
combine: a transposed operand, a wrong row or a shifted column changes the
exact result.

The power-of-two variant keeps these exact values but makes every scale a
different power of two: fp8 weight blocks 2^((block + e) mod 5 - 2), MX
e8m0 exponents that change from 32-group to 32-group, activation groups
whose amax is 448 * 2^j for j varying by group and token (x) or by SwiGLU
column group (the requantised act).  A scale applied to the wrong block,
group, row or token then changes the result.  The tile-queue cases are large
enough that the tiled kernels hand tiles out through their per-XCD queues.
"""

import numpy as np
import pytest
import torch

from helpers import say
from oracle import ffn as offn
from oracle import formats as fm
from synth import make_topk_ids, to_numpy

pytestmark = pytest.mark.gpu

_E2M1_CODE = {0.0: 0, 0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 6, 6.0: 7}


_E2M1_GRID = np.array(sorted(_E2M1_CODE))  # magnitudes in code order


def _encode_e2m1(w):
    """float32 [N, K] on the e2m1 grid -> packed uint8 [N, K/2] (element 2j in
    the low nibble of byte j)."""
    a = np.abs(w)
    codes = np.searchsorted(_E2M1_GRID, a).astype(np.uint8)
    assert np.array_equal(_E2M1_GRID[codes], a), "a value is not on the e2m1 grid"
    codes |= ((w < 0) & (a > 0)).astype(np.uint8) << 3
    return codes[:, 0::2] | (codes[:, 1::2] << 4)


def build(E, H, F, T, k, seed, kind="uniform"):
    rng = np.random.default_rng(seed)
    x = rng.integers(-4, 5, size=(T, H)).astype(np.float32)
    x[:, 1] = 8.0
    x[:, 2] = 2.0
    x[:, ::32] = 448.0
    free_h = np.array([h for h in range(H) if h % 32 != 0 and h not in (1, 2)])
    free_f = np.array([f for f in range(F) if f % 32 != 0])
    w13 = np.zeros((E, 2 * F, H), dtype=np.float32)
    w2 = np.zeros((E, H, F), dtype=np.float32)
    for e in range(E):
        w13[e, :F, 1] = 4.0
        for f in range(F):
            if f % 32 == 0:
                w13[e, F + f, 1] = 1.5
                w13[e, F + f, 2] = 1.0
            else:
                cols = rng.choice(free_h, 3, replace=False)
                w13[e, F + f, cols] = rng.choice([-1.0, 1.0], 3)
        for h in range(H):
            cols = rng.choice(free_f, 2, replace=False)
            w2[e, h, cols] = rng.choice([-1.0, 1.0], 2)
    ids = make_topk_ids(T, k, E, seed=seed, kind=kind)
    w = rng.choice([0.25, 0.5], size=(T, k)).astype(np.float32)
    return x, w13, w2, ids, w


def pow2_variant(x, w13, w2):
    """The same exact values with activation groups of different power-of-two
    amax: x[t, 32 i] = 448 * 2^j, j = (t + i) mod 5 - 2 (those columns meet
    no nonzero weight), and the up row of every 32nd SwiGLU column scaled by
    2^jf, jf = (f / 32 + e) mod 3, so that column's act is 448 * 2^jf, the
    largest of its group (the other act values are 32 u, |u| <= 12).  The
    fp8 scales of x (per 1 x 128: amax / 448) and of act, and the MX scales
    (per 32: the smallest power of two at least amax / 448), are then exact
    powers of two that differ from group to group and token to token; every
    quantised value stays exact and y is unchanged."""
    x, w13 = x.copy(), w13.copy()
    T, H = x.shape
    E, N13, _ = w13.shape
    F = N13 // 2
    j = (np.arange(T)[:, None] + np.arange(H // 32)[None, :]) % 5 - 2
    x[:, ::32] = 448.0 * np.exp2(j)
    for e in range(E):
        for f in range(0, F, 32):
            jf = (f // 32 + e) % 3
            w13[e, F + f, 1] = 1.5 * 2.0 ** jf
            w13[e, F + f, 2] = 2.0 ** jf
    return x, w13, w2


def _fp8_block_exponents(E, N, K):
    """2^s per 128 x 128 block, s = (block index + e) mod 5 - 2."""
    b = np.arange((N // 128) * (K // 128)).reshape(N // 128, K // 128)
    return np.stack([(b + e) % 5 - 2 for e in range(E)])


def _mx_group_exponents(w):
    """One e8m0 exponent per (expert, row, 32-group) for weights w [E, N, K]
    whose values are fixed: each group takes one of the exponents s in -3..4
    for which every value / 2^s is an e2m1 value (any s for an all-zero
    group), a different one from group to group."""
    E, N, K = w.shape
    g = np.abs(w).reshape(E, N, K // 32, 1, 32)
    cand = np.arange(-3, 5)
    scaled = g / np.exp2(cand.astype(np.float64))[:, None]
    ok = np.all((g == 0) | np.isin(scaled, _E2M1_GRID), axis=-1)  # [E, N, G, 8]
    count = ok.sum(axis=-1)
    assert np.all(count > 0)
    e_, n_, i_ = np.meshgrid(np.arange(E), np.arange(N), np.arange(K // 32), indexing="ij")
    pick = (7 * n_ + 3 * i_ + e_) % count  # index among the allowed exponents
    rank = np.cumsum(ok, axis=-1) - 1
    sel = ok & (rank == pick[..., None])
    return cand[np.argmax(sel, axis=-1)]


def to_device(fmt, x, w13, w2, pow2=False):
    """Stored tensors of each format: unit scales, or (``pow2``) scales that
    are distinct powers of two per fp8 128 x 128 block / MX 32-group, with the
    codes chosen so that code x scale is the same exact weight."""
    if pow2 and fmt == "fp8":
        E, N13, H = w13.shape
        F = w2.shape[2]
        s13 = np.exp2(_fp8_block_exponents(E, N13, H)).astype(np.float32)
        s2 = np.exp2(_fp8_block_exponents(E, H, F)).astype(np.float32)
        c13 = w13 / np.repeat(np.repeat(s13, 128, axis=1), 128, axis=2)
        c2 = w2 / np.repeat(np.repeat(s2, 128, axis=1), 128, axis=2)
        as_codes = lambda c: torch.from_numpy(c.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8)
        k13, k2 = as_codes(c13), as_codes(c2)
        # every code is exact: decoding gives back the value it encodes
        assert np.array_equal(fm.e4m3_decode(k13.numpy()), c13) and np.array_equal(fm.e4m3_decode(k2.numpy()), c2)
        xd = torch.from_numpy(x).to(torch.bfloat16).cuda()
        return xd, k13.cuda(), torch.from_numpy(s13).cuda(), k2.cuda(), torch.from_numpy(s2).cuda()
    if pow2 and fmt == "mxfp4":
        e13, e2 = _mx_group_exponents(w13), _mx_group_exponents(w2)
        c13 = w13 / np.repeat(np.exp2(e13.astype(np.float64)), 32, axis=2)
        c2 = w2 / np.repeat(np.exp2(e2.astype(np.float64)), 32, axis=2)
        p13 = np.stack([_encode_e2m1(c13[e]) for e in range(c13.shape[0])])
        p2 = np.stack([_encode_e2m1(c2[e]) for e in range(c2.shape[0])])
        xd = torch.from_numpy(x).to(torch.bfloat16).cuda()
        sc = lambda ex: torch.from_numpy((ex + 127).astype(np.uint8)).cuda()
        return xd, torch.from_numpy(p13).cuda(), sc(e13), torch.from_numpy(p2).cuda(), sc(e2)
    return _to_device_unit(fmt, x, w13, w2)


def _to_device_unit(fmt, x, w13, w2):
    """Stored tensors of each format (unit scales)."""
    xd = torch.from_numpy(x).to(torch.bfloat16).cuda()
    E, N13, H = w13.shape
    F = w2.shape[2]
    if fmt == "bf16":
        return xd, torch.from_numpy(w13).to(torch.bfloat16).cuda(), None, \
            torch.from_numpy(w2).to(torch.bfloat16).cuda(), None
    if fmt == "fp8":
        c13 = torch.from_numpy(w13).to(torch.float8_e4m3fn).view(torch.uint8).cuda()
        c2 = torch.from_numpy(w2).to(torch.float8_e4m3fn).view(torch.uint8).cuda()
        s13 = torch.ones((E, N13 // 128, H // 128), dtype=torch.float32, device="cuda")
        s2 = torch.ones((E, H // 128, F // 128), dtype=torch.float32, device="cuda")
        return xd, c13, s13, c2, s2
    p13 = np.stack([_encode_e2m1(w13[e]) for e in range(E)])
    p2 = np.stack([_encode_e2m1(w2[e]) for e in range(E)])
    s13 = torch.full((E, N13, H // 32), 127, dtype=torch.uint8, device="cuda")
    s2 = torch.full((E, H, F // 32), 127, dtype=torch.uint8, device="cuda")
    return xd, torch.from_numpy(p13).cuda(), s13, torch.from_numpy(p2).cuda(), s2


CASES = [("bf16", 256, 256, bm, T) for bm, T in ((16, 5), (16, 300), (32, 300), (64, 300), (128, 300))] + \
        [(f, 512, 512, bm, T) for f in ("fp8", "mxfp4") for bm, T in ((16, 3), (16, 200), (32, 200),
                                                                       (64, 200), (128, 200))]


# bf16 at BLOCK_M 64 and 128 (and 32 with enough rows per expert) runs the paired tiles (two blocks of one
# expert per tile): experts with an even and an odd number of blocks (uniform ids: 375
# and 500 rows per expert), uneven counts from skewed ids, one expert with
# one block (the hot expert set leaves the others empty), and a block table
# longer than one 1024-block chunk of the pair table, whose tiles the per-XCD
# queues hand out (every token compared).
PAIRED = [("bf16", 256, 256, 128, 1500, "uniform", None), ("bf16", 512, 384, 128, 2000, "uniform", None),
          ("bf16", 256, 512, 128, 3000, "skewed", None), ("bf16", 256, 256, 128, 100, "hot", None),
          ("bf16", 256, 128, 128, 70000, "uniform", None),
          # 64-row blocks paired too: an odd count (175 rows per expert) and uneven ones
          ("bf16", 512, 384, 64, 700, "uniform", None), ("bf16", 256, 256, 64, 1100, "skewed", None),
          # and 32-row blocks (paired once the experts average two rows or more
          # and there are more than 64 assignments): odd and uneven counts, and
          # more tiles than the XCDs' workgroups (per-XCD queues)
          ("bf16", 512, 384, 32, 700, "uniform", None), ("bf16", 256, 256, 32, 1100, "skewed", None),
          ("bf16", 256, 128, 32, 20000, "uniform", None)]


def _run_exact(fmt, H, F, bm, T, kind="uniform", sample=None, pow2=False):
    import mixture_experts_layer_04_amd as moe
    E, k = 8, 2
    say(f"exact probe {fmt} H={H} F={F} E={E} k={k} T={T} block_m={bm} ids={kind}"
        + (" power-of-two scales" if pow2 else ""))
    x, w13, w2, ids, w = build(E, H, F, T, k, seed=T + bm, kind=kind)
    if pow2:
        x, w13, w2 = pow2_variant(x, w13, w2)
    xd, c13, s13, c2, s2 = to_device(fmt, x, w13, w2, pow2)
    ids_d = ids.cuda()
    w_d = torch.from_numpy(w).cuda()
    s, b, n = moe.align(ids_d, E, bm)
    y = moe.expert_ffn(xd, c13, c2, ids_d, w_d, s, b, n, bm, wformat=fmt, w13_scale=s13, w2_scale=s2)
    torch.cuda.synchronize()
    weights = offn.ExpertWeights(fmt, to_numpy(c13), to_numpy(c2), to_numpy(s13), to_numpy(s2))
    tokens = None
    if sample is not None:
        tokens = np.sort(np.random.default_rng(T).choice(T, sample, replace=False))
        tokens[-1] = T - 1
    ref, _ = offn.layer(to_numpy(xd), {"ids": ids.numpy(), "weights": w}, weights, E, tokens=tokens)
    # every true output is a multiple of 8; the float64 oracle is off by
    # ~1e-11 because it takes silu(32) = 32 (1 - 1.3e-14), so its nearest
    # integer is the exact value
    exact = np.round(ref)
    assert np.max(np.abs(ref - exact)) < 1e-6 and np.all(exact % 8 == 0) and np.any(exact != 0)
    # exact equality of values (a zero may carry either sign)
    got = fm.bf16_bits_to_f64(to_numpy(y))
    if tokens is not None:
        got = got[tokens]
    bad = np.argwhere(got != exact)
    assert bad.size == 0, f"{len(bad)} of {got.size} outputs differ, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("fmt,H,F,bm,T", CASES)
def test_expert_ffn_exact(fmt, H, F, bm, T):
    _run_exact(fmt, H, F, bm, T)


@pytest.mark.parametrize("fmt,H,F,bm,T,kind,sample", PAIRED)
def test_expert_ffn_exact_paired_tiles(fmt, H, F, bm, T, kind, sample):
    _run_exact(fmt, H, F, bm, T, kind, sample)


# Every scale a power of two that differs from block to block (fp8 weights),
# from 32-group to 32-group (MX weights) and from activation group to group
# and token to token: a scale read from the wrong block, group, row or token
# changes the exact result.  Stream (16) and tiled (32 / 64 / 128) kernels.
POW2 = [(f, 512, 512, bm, T) for f in ("fp8", "mxfp4") for bm, T in ((16, 3), (16, 200), (32, 200), (64, 200),
                                                                     (128, 200))] + \
       [("fp8", 1024, 512, 128, 600), ("mxfp4", 512, 1024, 64, 600),
        # the paired MXFP4 kernels over 16 / 8 K steps (their copy rings and
        # the waits that end them run as at the full layer shapes)
        ("mxfp4", 2048, 1024, 128, 600), ("mxfp4", 2048, 1024, 64, 600)]


@pytest.mark.parametrize("fmt,H,F,bm,T", POW2)
def test_expert_ffn_exact_pow2_scales(fmt, H, F, bm, T):
    _run_exact(fmt, H, F, bm, T, pow2=True)


# Large enough that every XCD has more tiles than workgroups, so the tiled
# kernels take tiles from their per-XCD queues: every token compared.
QUEUE = [("fp8", 512, 512, 128, 40000), ("mxfp4", 512, 512, 128, 40000), ("mxfp4", 512, 512, 32, 12000),
         ("fp8", 512, 512, 64, 20000)]


@pytest.mark.parametrize("fmt,H,F,bm,T", QUEUE)
def test_expert_ffn_exact_tile_queue(fmt, H, F, bm, T):
    _run_exact(fmt, H, F, bm, T, pow2=True)

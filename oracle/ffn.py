"""Expert FFN, combine and full-layer oracle, in float64.

Test infrastructure only (see ``oracle/__init__``).

* An expert is gate, up and down projections stored as w13 [2F, H] (gate
  rows first, then up rows) and w2 [H, F] ([MoE] "Shapes, sourced": the
  fused w13_weight / w2_weight shapes; [MegaMoE] §3.5: the checkpoint keeps
  the gate columns before the up columns).
* Its output for one hidden state x is w2 . (silu(g) * u) with g = W1 x and
  u = W3 x, silu(g) = g / (1 + exp(-g)) ([Kernels] "The fused expert GEMM":
  SwiGLU silu(g) * u; [MegaMoE] §1.1: silu(gate) * up).  With a SwiGLU
  limit L, g is first capped at L and u clipped to [-L, L] ([MegaMoE] §3.5,
  the DeepSeek-V4 epilogue); L = inf is no clamp.
* The layer output of token t is sum_j w[t, j] * o[t, j], summed over the k
  slots in slot order ([Kernels] "Combine ...": a gather per token summing
  its k rows in a fixed order; [MegaMoE] §3.7: sum the slots in slot order).
  The grouped form (loop over experts, scatter back) is the other form of the
  [MoE] numpy check; the tests pin the two against each other.

Weight formats (dequantised exactly, never approximated):

* ``bf16``  - w13 / w2 as bf16 bits.
* ``fp8``   - e4m3 codes with one float32 scale per 128 x 128 block of the
  [N, K] matrix ([Kernels] "Combine, backward and low precision": 128 x 128
  weight blocks, 1 x 128 activation tiles).
* ``mxfp4`` - e2m1 codes packed two per byte along K plus one e8m0 scale per
  32 values along K ([MegaMoE] §1.1).

Activation modes:

* ``dense`` (headline parity reference): activations are not quantised.
* ``emulate``: x and the SwiGLU output are quantised as the quantised
  paths do: fp8 - e4m3 with a float scale amax/448 per 1 x 128 group;
  mxfp4 - e4m3 with a power-of-two scale pow2_at_least(amax/448) per 32
  ([MegaMoE] §3.5 requantisation); an all-zero group gets scale 1.  The
  scale and the scaled value are formed in fp32 (``quantize_act``), so the
  e4m3 codes of x are the kernels' own; the SwiGLU values the kernels
  quantise are their fp32 sums, which differ from this float64 value by
  rounding, so a value on a rounding tie may quantise one code apart.
  Pinned by the quantiser tests (grid values with power-of-two group
  scales come back unchanged; each group scales by its own amax; the MX
  scale at and around its power-of-two boundaries; nearest rounding by
  brute force).
"""

import numpy as np

from .formats import (E4M3_MAX, bf16_bits_to_f64, e2m1_decode, e4m3_decode,
                      e4m3_round, e8m0_decode, pow2_at_least, unpack_fp4)

WFORMATS = ("bf16", "fp8", "mxfp4")


# Value of every code, from the bit-field decoders (indexing a table is only
# faster than decoding each element; the values are the same).
_E4M3_TABLE = e4m3_decode(np.arange(256, dtype=np.uint8))
_E2M1_TABLE = e2m1_decode(np.arange(16))


def dequant(fmt, data, scale=None):
    """Exact float64 value of one stored [N, K] weight matrix: each code's
    value times the scale of the block (fp8: 128 x 128) or group (MX: 32
    along K) that holds it."""
    if fmt == "bf16":
        return bf16_bits_to_f64(data)
    if fmt == "fp8":
        q = _E4M3_TABLE[np.asarray(data, dtype=np.uint8)]
        s = np.asarray(scale, dtype=np.float32).astype(np.float64)
        n, k = q.shape
        if n % 128 == 0 and k % 128 == 0:  # every block whole: scale by broadcasting
            return (q.reshape(n // 128, 128, k // 128, 128) * s[:, None, :, None]).reshape(n, k)
        rows = np.repeat(s, 128, axis=0)[:n]
        return q * np.repeat(rows, 128, axis=1)[:, :k]
    if fmt == "mxfp4":
        q = _E2M1_TABLE[unpack_fp4(data, axis=-1)]
        s = e8m0_decode(scale)
        n, k = q.shape
        if k % 32 == 0:
            return (q.reshape(n, k // 32, 32) * s[:, :, None]).reshape(n, k)
        return q * np.repeat(s, 32, axis=1)[:, :k]
    raise ValueError(f"unknown weight format {fmt!r}")


class ExpertWeights:
    """Lazy per-expert access to stored weights.

    ``w13``, ``w2`` (and the scale tensors) may be anything indexable by an
    expert id that yields a numpy array for that expert (a numpy array of all
    experts works; tests wrap device tensors so that only the experts that
    are needed are copied)."""

    def __init__(self, fmt, w13, w2, w13_scale=None, w2_scale=None):
        if fmt not in WFORMATS:
            raise ValueError(f"unknown weight format {fmt!r}")
        self.fmt = fmt
        self.w13, self.w2 = w13, w2
        self.w13_scale, self.w2_scale = w13_scale, w2_scale

    def expert(self, e):
        s13 = None if self.w13_scale is None else np.asarray(self.w13_scale[e])
        s2 = None if self.w2_scale is None else np.asarray(self.w2_scale[e])
        W13 = dequant(self.fmt, np.asarray(self.w13[e]), s13)
        W2 = dequant(self.fmt, np.asarray(self.w2[e]), s2)
        return W13, W2


def silu(g):
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def quantize_act(v, fmt):
    """Emulate-mode activation quantisation of rows of ``v`` along its last
    axis (see module docstring), returning dequantised float64 values.

    Each group of 128 (fp8) or 32 (mxfp4) values of a row gets a scale s and
    each value becomes s * e4m3_round(value / s).  The pages fix the group
    sizes and the scale rule (amax / 448; for MX the smallest power of two at
    least amax / 448) but not the precision in which the scale and the
    scaled value are formed.  Reading: in fp32, the precision of the
    formats' scales: the values are taken as fp32, s = fp32(amax / 448)
    (MX: pow2_at_least of that fp32 quotient), value / s is an fp32
    division (correctly rounded), then rounded to the nearest e4m3 value
    with ties to even and saturation at 448.  An all-zero group gets s = 1.
    So the e4m3 code, an integer decided by floating point, is decided in
    the same precision on both sides."""
    v32 = np.asarray(v, dtype=np.float64).astype(np.float32)
    if fmt == "bf16":
        return np.asarray(v, dtype=np.float64)
    group = 128 if fmt == "fp8" else 32
    n, K = v32.shape
    pad = -K % group  # a short last group: zeros change neither amax nor the values
    g = np.pad(v32, ((0, 0), (0, pad))).reshape(n, (K + pad) // group, group)
    amax = np.abs(g).max(axis=2, keepdims=True)
    nz = amax > 0
    q = np.where(nz, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    if fmt == "fp8":
        s = q
    else:
        s = np.ones_like(q)
        s[nz] = pow2_at_least(q[nz].astype(np.float64)).astype(np.float32)
    scaled = (g / s).astype(np.float32)  # fp32 division, correctly rounded
    out = e4m3_round(scaled.astype(np.float64)) * s.astype(np.float64)
    return out.reshape(n, K + pad)[:, :K]


def swiglu(g, u, limit=np.inf):
    """silu(min(g, L)) * clip(u, -L, L) ([MegaMoE] §3.5); L = inf: silu(g) * u."""
    g = np.minimum(np.asarray(g, dtype=np.float64), limit)
    u = np.clip(np.asarray(u, dtype=np.float64), -limit, limit)
    return silu(g) * u


def expert_forward(X, W13, W2, act_fmt=None, limit=np.inf):
    """SwiGLU expert on the rows of X [n, H] -> [n, H].  With ``act_fmt``
    the SwiGLU output is quantised as in the emulate mode."""
    F = W13.shape[0] // 2
    g = X @ W13[:F].T
    u = X @ W13[F:].T
    a = swiglu(g, u, limit)
    if act_fmt is not None:
        a = quantize_act(a, act_fmt)
    return a @ W2.T


def combine_direct(outputs, w):
    """y[t] = sum_j w[t, j] * outputs[t, j] in slot order."""
    outputs = np.asarray(outputs, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    y = np.zeros((outputs.shape[0], outputs.shape[2]))
    for j in range(outputs.shape[1]):
        y += w[:, j, None] * outputs[:, j]
    return y


def layer_direct(x, ids, w, expert_fn):
    """Per token and slot: y[t] = sum_j w[t, j] * expert_fn(ids[t, j], x[t]).
    ``expert_fn(e, rows) -> outputs`` works on a [n, H] block of rows."""
    x = np.asarray(x, dtype=np.float64)
    T, k = np.asarray(ids).shape
    outs = np.zeros((T, k, x.shape[1]))
    for t in range(T):
        for j in range(k):
            outs[t, j] = expert_fn(int(ids[t][j]), x[t:t + 1])[0]
    return combine_direct(outs, w), outs


def layer_grouped(x, ids, w, expert_fn, E, workers=1):
    """Loop over experts, run each on the rows routed to it, scatter the
    weighted results back (the grouped form of the [MoE] numpy check).
    Also returns the per-assignment outputs [T, k, H].

    ``workers`` > 1 evaluates that many experts at a time on threads; each
    expert's rows and result are its own, so the result does not depend on
    it."""
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(ids)
    w = np.asarray(w, dtype=np.float64)
    T, k = ids.shape
    outs = np.zeros((T, k, x.shape[1]))
    work = []
    for e in range(E):
        toks, slots = np.nonzero(ids == e)
        if len(toks):
            work.append((e, toks, slots))

    def run(item):
        e, toks, slots = item
        outs[toks, slots] = expert_fn(e, x[toks])

    if workers > 1 and len(work) > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(run, work))
    else:
        for item in work:
            run(item)
    return combine_direct(outs, w), outs


def make_expert_fn(weights, mode="dense", limit=np.inf):
    """expert_fn for ``layer_*`` from an ExpertWeights.  An expert's
    dequantised matrices are made when it is called and dropped after, except
    that the last expert called is kept for a next call with the same id (the
    direct form calls one expert per slot); host memory stays at a few
    experts whatever E is."""
    last = {}
    act_fmt = None if mode == "dense" else weights.fmt

    def fn(e, rows):
        mats = last.get(e)
        if mats is None:
            mats = weights.expert(e)
            last.clear()
            last[e] = mats
        W13, W2 = mats
        if act_fmt is not None:
            rows = quantize_act(rows, act_fmt)
        return expert_forward(rows, W13, W2, act_fmt, limit)

    return fn


def layer(x_bits, route_out, weights, E, mode="dense", tokens=None, limit=np.inf, workers=1):
    """The full layer for the tokens in ``tokens`` (all by default), given a
    router result (``oracle.router.route``).  Returns (y [n, H] float64,
    per-assignment outputs [n, k, H]).  ``workers``: see layer_grouped."""
    x = bf16_bits_to_f64(x_bits)
    ids = route_out["ids"]
    w = route_out["weights"]
    if tokens is not None:
        x, ids, w = x[tokens], ids[tokens], w[tokens]
    if workers > 1:
        # one expert function per thread (its one-expert cache is its own)
        fns = {}

        def fn(e, rows):
            import threading
            key = threading.get_ident()
            if key not in fns:
                fns[key] = make_expert_fn(weights, mode, limit)
            return fns[key](e, rows)
    else:
        fn = make_expert_fn(weights, mode, limit)
    return layer_grouped(x, ids, w, fn, E, workers=workers)

"""Router oracle: gate logits -> scores -> rank keys -> (group limit) ->
k-round top-k -> weights, in float64.

Test infrastructure only (see ``oracle/__init__``).

The three router steps are those of [Router] §1.1 "Three Steps": one logit
per expert from the hidden state times the gate weight, a score per expert,
then the k best experts with their scores rescaled to sum to one.  The split
into a rank key (score + per-expert bias, used only for the choice) and a
weight (the unbiased score) is [Router] §1.3 "The Rank Key and the Weight"
(Fig. 3), and the same split appears in the grouped, bias-corrected routing
listing of [MoE] ("DeepSeek's actual routing is the grouped, bias-corrected
variant").

Readings where the pages leave a step open:

* ties in the rank key go to the lowest expert id ([Router] §5.3, Fig. 11;
  [Kernels] "Router: one fused kernel");
* ids are returned in round order (descending key, lowest id first);
* the renormalisation denominator is sum + 1e-20 ([Router] §4, the naive
  five-line router), and the routed scale multiplies after renormalising
  ([MoE], worked DeepSeek-V3 trace, step 2);
* the group score is the sum of the two largest rank keys of the group and
  groups are chosen with the same lowest-id tie rule ([MoE], grouped routing
  listing).
"""

import numpy as np

from .formats import bf16_bits_to_f64

SCORINGS = ("softmax", "sigmoid", "sqrtsoftplus")


def logits(x_bits, gate):
    """R1.  logits[t, e] = sum_h x[t, h] * gate[e, h] with x given as bf16
    bits [T, H] and the gate as float32 [E, H], both widened exactly.
    ([Router] §1.1 step one; §2.4 fp32 logits.)

    Pinned by the worked toy example (tests/golden/router_toy.json)."""
    x = bf16_bits_to_f64(x_bits)
    g = np.asarray(gate, dtype=np.float32).astype(np.float64)
    return x @ g.T


def scores(lg, scoring):
    """R2.  softmax over experts (max subtracted), an independent sigmoid
    per expert ([Router] §1.3; [MoE] fused_topk / grouped_topk listings), or
    the square root of a softplus per expert, the score DeepSeek-V4 uses in
    place of the sigmoid ([Router] §1.3, Fig. 3 discussion).  The softplus is
    written in its overflow-free form max(l, 0) + log1p(exp(-|l|)).

    Pinned against scipy.special.softmax / expit / softplus and closed forms
    (sqrt(ln 2) at 0, sqrt(l) for large l, exp(l / 2) for very negative l)."""
    lg = np.asarray(lg, dtype=np.float64)
    if scoring == "softmax":
        m = lg.max(axis=1, keepdims=True)
        e = np.exp(lg - m)
        return e / e.sum(axis=1, keepdims=True)
    if scoring == "sigmoid":
        with np.errstate(over="ignore"):
            return 1.0 / (1.0 + np.exp(-lg))
    if scoring == "sqrtsoftplus":
        return np.sqrt(np.maximum(lg, 0.0) + np.log1p(np.exp(-np.abs(lg))))
    raise ValueError(f"unsupported scoring function: {scoring!r}")


def rank_keys(sc, bias=None):
    """R3.  The rank key: the score plus the per-expert selection bias when
    the model has one, otherwise the score itself ([Router] §1.3)."""
    sc = np.asarray(sc, dtype=np.float64)
    if bias is None:
        return sc.copy()
    b = np.asarray(bias, dtype=np.float32).astype(np.float64)
    return sc + b[None, :]


def _rounds_argmax(values, count, allowed=None):
    """``count`` rounds of: take the largest remaining value (lowest index on
    ties), mark it used.  Returns indices [rows, count] in round order.

    This is the selection of [Router] §5.3 (Fig. 11) written out per row
    with numpy's argmax, which returns the first maximal index."""
    v = np.asarray(values, dtype=np.float64)
    rows = v.shape[0]
    avail = np.ones(v.shape, dtype=bool) if allowed is None else allowed.copy()
    out = np.empty((rows, count), dtype=np.int64)
    r = np.arange(rows)
    for j in range(count):
        masked = np.where(avail, v, -np.inf)
        # a row whose remaining candidates are all -inf would make argmax
        # pick an unavailable index; callers guarantee enough candidates
        if not np.all(avail.sum(axis=1) > 0):
            raise ValueError("not enough candidates for the requested count")
        best = masked.max(axis=1, keepdims=True)
        idx = np.argmax((masked == best) & avail, axis=1)
        out[:, j] = idx
        avail[r, idx] = False
    return out


def group_limit(keys, n_group, topk_group):
    """R4.  Group-limited routing: experts [g*E/n, (g+1)*E/n) form group g;
    a group's score is the sum of its two largest rank keys; the topk_group
    best groups stay (lowest group id on ties); the other experts are not
    allowed.  ([MoE] "Mixture of Experts", the grouped_topk listing and
    the second step of the DeepSeek-V3 trace, where the eight groups are
    ranked by the sum of their two best keys and four of them are kept.)

    Returns (allowed mask [T, E], group scores [T, n_group], kept groups
    [T, topk_group]).  Pinned by brute-force enumeration in the tests."""
    keys = np.asarray(keys, dtype=np.float64)
    T, E = keys.shape
    if n_group <= 1:
        return np.ones((T, E), dtype=bool), keys.max(axis=1, keepdims=True), np.zeros((T, 1), np.int64)
    if E % n_group:
        raise ValueError("n_group must divide E")
    gsize = E // n_group
    if gsize < 2:
        raise ValueError("a group needs at least two experts for its top-2 sum")
    grouped = keys.reshape(T, n_group, gsize)
    two_largest = np.sort(grouped, axis=2)[:, :, -2:]
    gscore = two_largest[:, :, 0] + two_largest[:, :, 1]
    kept = _rounds_argmax(gscore, topk_group)
    gmask = np.zeros((T, n_group), dtype=bool)
    gmask[np.arange(T)[:, None], kept] = True
    allowed = np.repeat(gmask, gsize, axis=1)
    return allowed, gscore, kept


def topk(keys, k, allowed=None):
    """R5.  k rounds of arg-max over the allowed experts with the lowest id
    winning ties; also the cut margin key_(k) - key_(k+1), the gap at the
    cut of [Router] §1.3 and §2.1 (+inf when no expert is left after k).

    Returns (ids [T, k] in round order, margin [T])."""
    keys = np.asarray(keys, dtype=np.float64)
    T, E = keys.shape
    if allowed is None:
        allowed = np.ones((T, E), dtype=bool)
    if np.any(allowed.sum(axis=1) < k):
        raise ValueError("k exceeds the number of allowed experts")
    ids = _rounds_argmax(keys, k, allowed)
    r = np.arange(T)
    kth = keys[r, ids[:, -1]]
    rest = allowed.copy()
    rest[r[:, None], ids] = False
    nxt = np.where(rest, keys, -np.inf).max(axis=1)
    margin = np.where(rest.any(axis=1), kth - nxt, np.inf)
    return ids, margin


def weights(sc, ids, renormalize=True, routed_scale=1.0):
    """R6.  The weight of a chosen expert is its (unbiased) score; with
    renormalisation it is divided by the sum over the k chosen plus 1e-20
    ([Router] §4, the naive router); then the routed scaling factor
    multiplies ([MoE] "Mixture of Experts", second step of the DeepSeek-V3
    trace: the weights are renormalised first and scaled after)."""
    sc = np.asarray(sc, dtype=np.float64)
    w = np.take_along_axis(sc, np.asarray(ids), axis=1)
    if renormalize:
        w = w / (w.sum(axis=1, keepdims=True) + 1e-20)
    return w * float(routed_scale)


def with_shared_expert(r, E):
    """The shared expert as an always-selected slot: ids and weights gain a
    slot k holding expert E with weight 1 for every token ([MoE], SGLang's
    fused shared expert: appended as expert id E, top-k becomes top-(k+1);
    [MegaMoE] §3.8: its output is added to the sum of the routed ones).
    Reading: the routed weights keep their renormalisation and scale, and
    the shared expert's output adds unscaled."""
    ids = np.asarray(r["ids"])
    w = np.asarray(r["weights"], dtype=np.float64)
    T = ids.shape[0]
    out = dict(r)
    out["ids"] = np.concatenate([ids, np.full((T, 1), E, dtype=ids.dtype)], axis=1)
    out["weights"] = np.concatenate([w, np.ones((T, 1))], axis=1)
    return out


def route(x_bits, gate, bias, k, scoring, n_group=1, topk_group=1,
          renormalize=True, routed_scale=1.0):
    """The whole router (R1-R6).  Returns a dict with logits, scores, keys,
    ids, weights, cut margin and group margin (inf without groups)."""
    lg = logits(x_bits, gate)
    sc = scores(lg, scoring)
    ky = rank_keys(sc, bias)
    allowed, gscore, _ = group_limit(ky, n_group, topk_group)
    ids, margin = topk(ky, k, allowed)
    w = weights(sc, ids, renormalize, routed_scale)
    if n_group > 1 and topk_group < n_group:
        gs = -np.sort(-gscore, axis=1)
        gmargin = gs[:, topk_group - 1] - gs[:, topk_group]
    else:
        gmargin = np.full(lg.shape[0], np.inf)
    return {"logits": lg, "scores": sc, "keys": ky, "ids": ids,
            "weights": w, "margin": margin, "group_margin": gmargin}

"""Shared helpers for the parity tests: oracle references on host copies of
the same seeded tensors the HIP path sees, and the acceptance checks."""

import os

import numpy as np
import torch

from oracle import align as oalign
from oracle import ffn as offn
from oracle import router as orouter
from synth import to_numpy

# Routing is compared id for id on tokens whose rank-key margin at the cut
# (and, with groups, the group-score margin) exceeds this.
MARGIN = 1e-5
# Layer tolerance (relative Frobenius error against the dense-equivalent
# oracle), per weight format.
LAYER_TOL = {"bf16": 2e-2, "fp8": 5e-2, "mxfp4": 5e-2}
# Every token's own relative error stays within this many times the layer
# tolerance (a lost or duplicated tile, which touches at most 128 tokens,
# cannot hide in the Frobenius norm of the whole output).
TOKEN_FACTOR = 3.0
# fp8 / MXFP4: relative Frobenius error against the oracle that quantises
# the activations as the kernels do (scales in float64, so a rare e4m3
# rounding flip of a value at a rounding boundary differs).
EMULATE_TOL = 1e-2
# Threads for the oracle's expert loop (the GPU host shares its CPUs).
ORACLE_WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))


def say(*a):
    print(*a, flush=True)


class LazyExperts:
    """Indexable by expert id; copies that expert's slice to the host on each
    access (nothing is kept, so host memory holds a few experts at a time)."""

    def __init__(self, t):
        self.t = t

    def __getitem__(self, e):
        return to_numpy(self.t[e])


def oracle_route(cfg, x, gate, bias):
    """The oracle router on the same inputs; a bf16 gate is handed over as
    its values (widened to float32, which is exact)."""
    if gate.dtype == torch.bfloat16:
        gate = gate.to(torch.float32)
    return orouter.route(to_numpy(x), to_numpy(gate), to_numpy(bias), cfg.k, cfg.scoring,
                         cfg.n_group, cfg.topk_group, cfg.renormalize, cfg.routed_scale)


def check_routing(cfg, r, ids_gpu, w_gpu, allow_frac=0.02):
    """Ids equal (in round order) and weights close on clear tokens; on
    near-tie tokens the GPU choice must be a valid alternative (k distinct
    allowed experts whose keys all reach the cut within the margin).  Returns
    (clear mask, number of near-tie tokens whose ids differ)."""
    ids_gpu = np.asarray(ids_gpu)
    w_gpu = np.asarray(w_gpu)
    clear = (r["margin"] > MARGIN) & (r["group_margin"] > MARGIN)
    assert np.array_equal(ids_gpu[clear], r["ids"][clear]), "routing ids differ on clear tokens"
    assert np.allclose(w_gpu[clear], r["weights"][clear], rtol=1e-5, atol=1e-6), "routing weights differ"
    differ = 0
    for t in np.nonzero(~clear)[0]:
        g = ids_gpu[t]
        if np.array_equal(g, r["ids"][t]):
            continue
        differ += 1
        assert len(set(g.tolist())) == cfg.k and np.all((g >= 0) & (g < cfg.E))
        cut = r["keys"][t, r["ids"][t, -1]]
        assert np.all(r["keys"][t, g] >= cut - 2 * MARGIN), f"token {t}: GPU choice is not a near tie"
    assert differ <= max(1, allow_frac * len(ids_gpu))
    return clear, differ


def routing_for_layer(cfg, r, ids_gpu):
    """The oracle's routing, with the GPU's ids (and oracle weights for them)
    on near-tie tokens where both choices are valid."""
    ids_gpu = np.asarray(ids_gpu).astype(np.int64)
    ids = r["ids"].copy()
    bad = np.any(ids != ids_gpu, axis=1)
    ids[bad] = ids_gpu[bad]
    w = orouter.weights(r["scores"], ids, cfg.renormalize, cfg.routed_scale)
    return {"ids": ids, "weights": w}


def oracle_layer(cfg, x, routing, weights_t, tokens=None, mode="dense", limit=np.inf):
    W = offn.ExpertWeights(cfg.wformat, LazyExperts(weights_t["w13"]), LazyExperts(weights_t["w2"]),
                           None if weights_t["w13_scale"] is None else LazyExperts(weights_t["w13_scale"]),
                           None if weights_t["w2_scale"] is None else LazyExperts(weights_t["w2_scale"]))
    y, _ = offn.layer(to_numpy(x), routing, W, cfg.E, mode=mode, tokens=tokens, limit=limit,
                      workers=ORACLE_WORKERS)
    return y


def rel_fro(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))


def token_errors(got, ref):
    """Relative error of every token (row): ||got_t - ref_t|| / ||ref_t||."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return np.linalg.norm(got - ref, axis=1) / np.maximum(np.linalg.norm(ref, axis=1), 1e-30)


def check_output(got, ref, tol, what="oracle"):
    """Relative Frobenius error within ``tol`` and every token's relative
    error within TOKEN_FACTOR * tol; returns (Frobenius error, worst token
    error, its index)."""
    err = rel_fro(got, ref)
    te = token_errors(got, ref)
    worst = int(np.argmax(te)) if len(te) else 0
    say(f"  vs {what}: rel. Frobenius {err:.3e} (tolerance {tol:.0e}), worst token {te[worst] if len(te) else 0:.3e} "
        f"(token {worst}, bound {TOKEN_FACTOR * tol:.0e})")
    assert np.all(np.isfinite(got))
    assert err <= tol, f"relative Frobenius error {err:.3e} against the {what} exceeds {tol:.0e}"
    assert np.all(te <= TOKEN_FACTOR * tol), \
        f"{int(np.sum(te > TOKEN_FACTOR * tol))} tokens exceed {TOKEN_FACTOR * tol:.0e} against the {what}, " \
        f"worst {te[worst]:.3e} at token {worst}"
    return err, float(te[worst]) if len(te) else 0.0, worst


def bf16_to_f64(t):
    return t.detach().to(torch.float64).cpu().numpy()


def oracle_align(ids_t, E, bm):
    return oalign.align(ids_t.cpu().tolist(), E, bm)

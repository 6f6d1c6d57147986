"""Python binding of libmoe: same names as the C ABI, torch tensors in and
out.  Argument marshalling only - every step runs in the HIP kernels.

Tensors must be CUDA (HIP) tensors, contiguous, with the dtypes of
include/moe.h: x bf16 [T, H]; gate float32 or bf16 [E, H] (the dtype sets
gate_is_fp32); bias float32 [E] or None;
w13 / w2 in the layout of the weight format (bf16, or uint8 codes plus
float32 (fp8) / uint8 e8m0 (mxfp4) scales).  Work goes onto the current
stream.  The workspace is a zero-initialised byte tensor cached per device
(or passed in); calls that overlap in time must not share one.
"""

import math

import torch

from ._lib import SCORING, STAGE, WFORMAT, check, lib

_WS = {}
# Workspaces the cache has outgrown.  They are never freed: a HIP graph
# captured with one keeps its address, and freeing it would let its replays
# write router partials and tile-queue counters into another tensor's memory.
_WS_RETIRED = []


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def workspace(device, nbytes):
    """A zero-filled workspace of at least ``nbytes`` on ``device`` (cached,
    grown on demand; the library leaves its counters at zero after each call,
    so the cached buffer stays valid; an outgrown one is kept alive, not
    freed, since a captured graph may still use it)."""
    device = torch.device(device)
    key = device.index if device.index is not None else torch.cuda.current_device()
    ws = _WS.get(key)
    if ws is None or ws.numel() < nbytes:
        if ws is not None:
            _WS_RETIRED.append(ws)
        ws = torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)
        _WS[key] = ws
    return ws


def _check_cuda(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("libmoe ops take GPU tensors")
            if not t.is_contiguous():
                raise ValueError("libmoe ops take contiguous tensors")


def _gate_is_fp32(gate):
    if gate.dtype == torch.float32:
        return 1
    if gate.dtype == torch.bfloat16:
        return 0
    raise ValueError(f"the gate is float32 or bfloat16, not {gate.dtype}")


def align_max_padded(T, k, E, block_m):
    return int(lib().moe_align_max_padded(T, k, E, block_m))


def align_max_blocks(T, k, E, block_m):
    return int(lib().moe_align_max_blocks(T, k, E, block_m))


def layer_block_m(T, k, E, F, wformat="bf16"):
    return int(lib().moe_layer_block_m(T, E, F, k, WFORMAT[wformat]))


def route(x, gate, bias, k, scoring="softmax", n_group=1, topk_group=1, renormalize=True,
          routed_scale=1.0, return_logits=False, ws=None):
    """moe_route -> (topk_ids int32 [T, k], topk_weights float32 [T, k][, logits])."""
    _check_cuda(x, gate, bias)
    T, H = x.shape
    E = gate.shape[0]
    ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    logits = torch.empty((T, E), dtype=torch.float32, device=x.device) if return_logits else None
    need = lib().moe_route_workspace_size(T, H, E)
    ws = workspace(x.device, need) if ws is None else ws
    check(lib().moe_route(_ptr(x), _ptr(gate), _gate_is_fp32(gate), _ptr(bias), T, H, E, k, n_group, topk_group,
                          SCORING[scoring], int(bool(renormalize)), float(routed_scale),
                          _ptr(ids), _ptr(w), _ptr(logits), _ptr(ws), ws.numel(), _stream(x.device)),
          "moe_route")
    return (ids, w, logits) if return_logits else (ids, w)


def route_align(x, gate, bias, k, block_m, scoring="softmax", n_group=1, topk_group=1, renormalize=True,
                routed_scale=1.0, ws=None, n_shared=0):
    """moe_route_align -> (topk_ids, topk_weights, sorted_ids, block_expert, num_post_padded [1]);
    with n_shared = 1 the ids / weights have k + 1 slots (slot k: the shared expert E, weight 1)."""
    _check_cuda(x, gate, bias)
    T, H = x.shape
    E = gate.shape[0]
    dev = x.device
    ka, Ea = k + n_shared, E + n_shared
    ids = torch.empty((T, ka), dtype=torch.int32, device=dev)
    w = torch.empty((T, ka), dtype=torch.float32, device=dev)
    sorted_ids = torch.empty(align_max_padded(T, ka, Ea, block_m), dtype=torch.int32, device=dev)
    block_expert = torch.empty(align_max_blocks(T, ka, Ea, block_m), dtype=torch.int32, device=dev)
    npp = torch.empty(1, dtype=torch.int32, device=dev)
    need = lib().moe_route_align_workspace_size(T, H, E, k, n_shared)
    ws = workspace(dev, need) if ws is None else ws
    check(lib().moe_route_align(_ptr(x), _ptr(gate), _gate_is_fp32(gate), _ptr(bias), T, H, E, k, n_shared,
                                n_group, topk_group, SCORING[scoring], int(bool(renormalize)), float(routed_scale),
                                block_m, _ptr(ids), _ptr(w), _ptr(sorted_ids), _ptr(block_expert), _ptr(npp),
                                _ptr(ws), ws.numel(), _stream(dev)), "moe_route_align")
    return ids, w, sorted_ids, block_expert, npp


def align(topk_ids, E, block_m, ws=None):
    """moe_align -> (sorted_ids, block_expert, num_post_padded [1]) on the device."""
    _check_cuda(topk_ids)
    T, k = topk_ids.shape
    dev = topk_ids.device
    sorted_ids = torch.empty(align_max_padded(T, k, E, block_m), dtype=torch.int32, device=dev)
    block_expert = torch.empty(align_max_blocks(T, k, E, block_m), dtype=torch.int32, device=dev)
    npp = torch.empty(1, dtype=torch.int32, device=dev)
    need = lib().moe_align_workspace_size(T, k, E)
    ws = workspace(dev, need) if ws is None else ws
    check(lib().moe_align(_ptr(topk_ids), T, k, E, block_m, _ptr(sorted_ids), _ptr(block_expert), _ptr(npp),
                          _ptr(ws), ws.numel(), _stream(dev)), "moe_align")
    return sorted_ids, block_expert, npp


def _dims(x, w13, w2, wformat):
    T, H = x.shape
    E = w13.shape[0]
    F = w13.shape[1] // 2
    return T, H, E, F


def expert_ffn(x, w13, w2, topk_ids, topk_weights, sorted_ids, block_expert, num_post_padded, block_m,
               wformat="bf16", w13_scale=None, w2_scale=None, ws=None, stages=None, out=None,
               swiglu_limit=math.inf):
    """moe_expert_ffn -> y bf16 [T, H].  ``stages`` (names from
    _lib.STAGE, or an int mask) selects moe_expert_ffn_stages instead."""
    _check_cuda(x, w13, w2, topk_ids, topk_weights, sorted_ids, block_expert, num_post_padded,
                w13_scale, w2_scale)
    T, H, E, F = _dims(x, w13, w2, wformat)
    k = topk_ids.shape[1]
    y = torch.empty((T, H), dtype=torch.bfloat16, device=x.device) if out is None else out
    wf = WFORMAT[wformat]
    need = lib().moe_expert_ffn_workspace_size(T, H, E, F, k, block_m, wf)
    ws = workspace(x.device, need) if ws is None else ws
    args = [_ptr(x), wf, _ptr(w13), _ptr(w13_scale), _ptr(w2), _ptr(w2_scale),
            _ptr(topk_ids), _ptr(topk_weights), _ptr(sorted_ids), _ptr(block_expert),
            _ptr(num_post_padded), T, H, E, F, k, block_m, float(swiglu_limit), _ptr(y), _ptr(ws), ws.numel()]
    if stages is None:
        check(lib().moe_expert_ffn(*args, _stream(x.device)), "moe_expert_ffn")
    else:
        mask = stages if isinstance(stages, int) else sum(STAGE[s] for s in stages)
        check(lib().moe_expert_ffn_stages(*args, mask, _stream(x.device)), "moe_expert_ffn_stages")
    return y


def layer_workspace_size(T, H, E, F, k, block_m=0, wformat="bf16", n_shared=0):
    return int(lib().moe_layer_workspace_size(T, H, E, F, k, n_shared, block_m, WFORMAT[wformat]))


def layer(x, gate, bias, w13, w2, k, scoring="softmax", n_group=1, topk_group=1, renormalize=True,
          routed_scale=1.0, wformat="bf16", w13_scale=None, w2_scale=None, block_m=0, return_routing=False,
          ws=None, out=None, swiglu_limit=math.inf, n_shared=0):
    """moe_layer -> y bf16 [T, H] (and topk ids / weights with return_routing).
    With n_shared = 1, w13 / w2 (and scales) hold the gate's E experts plus
    the shared expert last."""
    _check_cuda(x, gate, bias, w13, w2, w13_scale, w2_scale)
    T, H, Ew, F = _dims(x, w13, w2, wformat)
    E = gate.shape[0]
    if Ew != E + n_shared:
        raise ValueError(f"w13 holds {Ew} experts, the gate {E} and n_shared = {n_shared}")
    y = torch.empty((T, H), dtype=torch.bfloat16, device=x.device) if out is None else out
    ids = w = None
    if return_routing:
        ids = torch.empty((T, k + n_shared), dtype=torch.int32, device=x.device)
        w = torch.empty((T, k + n_shared), dtype=torch.float32, device=x.device)
    wf = WFORMAT[wformat]
    need = lib().moe_layer_workspace_size(T, H, E, F, k, n_shared, block_m, wf)
    ws = workspace(x.device, need) if ws is None else ws
    check(lib().moe_layer(_ptr(x), _ptr(gate), _gate_is_fp32(gate), _ptr(bias), wf, _ptr(w13), _ptr(w13_scale),
                          _ptr(w2), _ptr(w2_scale), T, H, E, F, k, n_shared, n_group, topk_group, SCORING[scoring],
                          int(bool(renormalize)), float(routed_scale), block_m, float(swiglu_limit), _ptr(y),
                          _ptr(ids), _ptr(w),
                          _ptr(ws), ws.numel(), _stream(x.device)), "moe_layer")
    return (y, ids, w) if return_routing else y


def layer_noalloc(x, gate, bias, w13, w2, k, scoring="softmax", n_group=1, topk_group=1, renormalize=True,
                  routed_scale=1.0, wformat="bf16", w13_scale=None, w2_scale=None, block_m=0,
                  return_routing=False, out=None, swiglu_limit=math.inf, n_shared=0):
    """moe_layer_noalloc: moe_layer on the library's own scratch array (no
    workspace; the outputs are still the caller's tensors, allocated here
    unless ``out`` is given)."""
    _check_cuda(x, gate, bias, w13, w2, w13_scale, w2_scale, out)
    T, H, Ew, F = _dims(x, w13, w2, wformat)
    E = gate.shape[0]
    if Ew != E + n_shared:
        raise ValueError(f"w13 holds {Ew} experts, the gate {E} and n_shared = {n_shared}")
    y = torch.empty((T, H), dtype=torch.bfloat16, device=x.device) if out is None else out
    ids = w = None
    if return_routing:
        ids = torch.empty((T, k + n_shared), dtype=torch.int32, device=x.device)
        w = torch.empty((T, k + n_shared), dtype=torch.float32, device=x.device)
    check(lib().moe_layer_noalloc(_ptr(x), _ptr(gate), _gate_is_fp32(gate), _ptr(bias), WFORMAT[wformat],
                                  _ptr(w13), _ptr(w13_scale), _ptr(w2), _ptr(w2_scale), T, H, E, F, k, n_shared,
                                  n_group, topk_group, SCORING[scoring], int(bool(renormalize)),
                                  float(routed_scale), block_m, float(swiglu_limit), _ptr(y), _ptr(ids), _ptr(w),
                                  _stream(x.device)),
          "moe_layer_noalloc")
    return (y, ids, w) if return_routing else y


def debug_error(ws):
    """Synchronises and returns (and clears) the sticky alignment error bits."""
    return int(lib().moe_debug_error(_ptr(ws), _stream(ws.device)))


def probe_empty(device="cuda"):
    check(lib().moe_probe_empty(_stream(torch.device(device))), "moe_probe_empty")


def probe_mfma(kind, accs, grid, iters, sink=None, device="cuda"):
    """Enqueues the matrix-core issue-rate probe (kind: 0 bf16 16x16x32,
    1 bf16 32x32x16, 2 e4m3 x e4m3, 3 e4m3 x e2m1, 4 e2m1 x e2m1)."""
    dev = torch.device(device)
    if sink is None:
        sink = torch.empty(int(lib().moe_probe_mfma_sink_len(grid)), dtype=torch.float32, device=dev)
    check(lib().moe_probe_mfma(kind, accs, grid, iters, _ptr(sink), _stream(dev)), "moe_probe_mfma")
    return sink


def probe_read(t, sink=None):
    """Reads every byte of ``t`` once (the bare weight-read kernel)."""
    nbytes = t.numel() * t.element_size()
    if sink is None:
        sink = torch.empty(int(lib().moe_probe_read_sink_len(nbytes)), dtype=torch.float32, device=t.device)
    check(lib().moe_probe_read(_ptr(t), nbytes, _ptr(sink), _stream(t.device)), "moe_probe_read")
    return sink

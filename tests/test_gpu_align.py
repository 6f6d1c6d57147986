"""GPU parity of moe_align: bit-exact sorted_ids, block table and padded
length against the oracle for identical topk_ids, including the [MoE]
docstring example, counts of 0 / 1 / BLOCK_M / BLOCK_M+1, the empty batch,
skewed and single-expert-set routings, E = 1024 and invalid ids."""

import pytest
import torch

from helpers import oracle_align, say
from synth import make_topk_ids

pytestmark = pytest.mark.gpu


def _check(ids, E, bm):
    import mixture_experts_layer_04_amd as moe
    s, b, n = moe.align(ids, E, bm)
    so, bo, no, _ = oracle_align(ids, E, bm)
    assert int(n.item()) == no
    assert s.cpu().tolist() == so
    assert b.cpu().tolist() == bo


def test_align_docstring_example(golden):
    g = golden("align_docstring.json")
    ids = torch.tensor([[e - 1 for e in row] for row in g["topk_ids_one_based"]], dtype=torch.int32).cuda()
    import mixture_experts_layer_04_amd as moe
    s, b, n = moe.align(ids, g["num_experts"], g["block_size"])
    m = len(g["printed_sorted_token_ids"])
    assert int(n.item()) == m
    assert s.cpu().tolist()[:m] == g["printed_sorted_token_ids"]
    assert b.cpu().tolist()[: m // g["block_size"]] == g["derived_block_expert_zero_based"]
    _check(ids, g["num_experts"], g["block_size"])


CASES = [
    (1, 8, 128, 16, "uniform"), (64, 8, 128, 16, "uniform"), (4096, 8, 128, 64, "uniform"),
    (4096, 8, 128, 128, "skewed"), (512, 8, 288, 16, "uniform"), (8192, 6, 256, 128, "uniform"),
    (2048, 8, 256, 64, "skewed"), (37, 3, 1024, 32, "uniform"), (333, 8, 600, 16, "skewed"),
    (100, 4, 16, 16, "hot"), (5000, 2, 8, 128, "uniform"), (16, 2, 8, 16, "uniform"),
    (1, 1, 1, 16, "uniform"), (77, 6, 256, 1, "uniform"),
    # the one-wave path (at most 64 assignments) and just past it
    (8, 8, 128, 16, "uniform"), (8, 8, 64, 16, "hot"), (64, 1, 1024, 32, "uniform"), (7, 2, 16, 1, "skewed"),
    (32, 2, 8, 128, "hot"), (13, 5, 1024, 16, "uniform"), (65, 1, 4, 16, "uniform"),
    # around the switch to the multi-workgroup path (12288 assignments)
    (12287, 1, 64, 16, "uniform"), (6144, 2, 64, 16, "skewed"), (1536, 8, 1024, 16, "uniform"),
    (65536, 8, 256, 128, "uniform"), (13000, 1, 1, 64, "uniform"),
]


@pytest.mark.parametrize("T,k,E,bm,kind", CASES)
def test_align_parity(T, k, E, bm, kind):
    say(f"align T={T} k={k} E={E} bm={bm} {kind}")
    ids = make_topk_ids(T, k, E, seed=T + E, kind=kind, device="cuda")
    _check(ids, E, bm)


def test_align_boundary_counts():
    bm, E = 16, 6
    flat = [1] + [2] * bm + [3] * (bm + 1) + [5] * 3  # expert 0 and 4 empty
    ids = torch.tensor(flat, dtype=torch.int32).view(-1, 1).cuda()
    _check(ids, E, bm)


def test_align_empty():
    ids = torch.empty((0, 8), dtype=torch.int32, device="cuda")
    _check(ids, 128, 16)


def test_align_invalid_ids_are_skipped_and_flagged():
    import mixture_experts_layer_04_amd as moe
    ws = torch.zeros(65536, dtype=torch.uint8, device="cuda")
    ids = torch.tensor([[0, -1], [5, 1], [2, 3]], dtype=torch.int32).cuda()
    s, b, n = moe.align(ids, 4, 16, ws=ws)
    so, bo, no, bad = oracle_align(ids, 4, 16)
    assert bad and s.cpu().tolist() == so and int(n.item()) == no
    assert moe.debug_error(ws) == 1
    assert moe.debug_error(ws) == 0  # cleared
    ids = torch.tensor([[0, -1]], dtype=torch.int32).cuda()
    moe.align(ids, 4, 16, ws=ws)
    assert moe.debug_error(ws) == 0  # -1 alone is not an error


def test_align_invalid_ids_multi_workgroup():
    import mixture_experts_layer_04_amd as moe
    T, k, E, bm = 4096, 4, 64, 32
    ids = make_topk_ids(T, k, E, seed=7, device="cuda")
    ids[5, 1] = -1
    ids[100, 0] = E + 3
    ids[4000, 3] = -7
    ws = torch.zeros(moe.lib().moe_align_workspace_size(T, k, E), dtype=torch.uint8, device="cuda")
    s, b, n = moe.align(ids, E, bm, ws=ws)
    so, bo, no, bad = oracle_align(ids, E, bm)
    assert bad and s.cpu().tolist() == so and b.cpu().tolist() == bo and int(n.item()) == no
    assert moe.debug_error(ws) == 1
    ids[100, 0] = 0
    ids[4000, 3] = 1
    s, b, n = moe.align(ids, E, bm, ws=ws)  # the counter left at zero: a second call works
    so, bo, no, _ = oracle_align(ids, E, bm)
    assert s.cpu().tolist() == so and b.cpu().tolist() == bo and int(n.item()) == no
    assert moe.debug_error(ws) == 0

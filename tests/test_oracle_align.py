"""Pins for the alignment oracle: the docstring example of [MoE] bit for
bit, the BLOCK_M = 1 special case against numpy's stable argsort, the
padded-length identity of [Kernels], and the structural invariants."""

import numpy as np
import pytest

from oracle import align as oalign
from synth import make_topk_ids


def check_invariants(ids, E, bm, sid, bexp, total):
    flat = np.asarray(ids).reshape(-1)
    A = flat.size
    valid = (flat >= 0) & (flat < E)
    counts = np.bincount(flat[valid], minlength=E)
    assert total == int(sum(-(-c // bm) * bm for c in counts))
    assert total % bm == 0
    assert len(sid) == A + E * (bm - 1)
    assert len(bexp) == -(-len(sid) // bm)
    real = [a for a in sid if a != A]
    assert sorted(real) == np.nonzero(valid)[0].tolist()  # a permutation of the valid a
    assert all(a == A for a in sid[total:])
    for b in range(total // bm):
        e = bexp[b]
        rows = [a for a in sid[b * bm:(b + 1) * bm] if a != A]
        assert all(flat[a] == e for a in rows)  # one expert per block
        assert rows == sorted(rows)  # stable within the block
    assert all(e == -1 for e in bexp[total // bm:])
    # experts appear in ascending order, each with ceil(count/bm) blocks
    used = bexp[: total // bm]
    assert used == sorted(used)
    for e in range(E):
        assert used.count(e) == -(-counts[e] // bm)


def test_docstring_example_bit_exact(golden):
    g = golden("align_docstring.json")
    ids = [[e - 1 for e in row] for row in g["topk_ids_one_based"]]
    flat_one_based = [e for row in g["topk_ids_one_based"] for e in row]
    assert flat_one_based == g["printed_flat_one_based"]
    sid, bexp, total, bad = oalign.align(ids, g["num_experts"], g["block_size"])
    n = len(g["printed_sorted_token_ids"])
    assert total == n == g["derived_num_tokens_post_padded"]
    assert sid[:n] == g["printed_sorted_token_ids"]
    assert sid[n:] == [g["printed_sentinel"]] * (len(sid) - n)
    assert bexp[: n // g["block_size"]] == g["derived_block_expert_zero_based"]
    assert all(e == -1 for e in bexp[n // g["block_size"]:])
    assert not bad


@pytest.mark.parametrize("kind", ["uniform", "skewed", "hot"])
@pytest.mark.parametrize("T,k,E", [(1, 1, 4), (7, 2, 8), (64, 8, 128), (333, 6, 40)])
def test_block1_is_stable_argsort(kind, T, k, E):
    ids = make_topk_ids(T, k, E, seed=11, kind=kind).numpy()
    sid, bexp, total, _ = oalign.align(ids.tolist(), E, 1)
    flat = ids.reshape(-1)
    assert total == flat.size
    assert sid[:total] == np.argsort(flat, kind="stable").tolist()
    assert bexp[:total] == flat[np.argsort(flat, kind="stable")].tolist()


@pytest.mark.parametrize("bm", [4, 16, 32, 64, 128])
@pytest.mark.parametrize("kind", ["uniform", "skewed", "hot"])
def test_invariants(bm, kind):
    T, k, E = 97, 6, 24
    ids = make_topk_ids(T, k, E, seed=bm, kind=kind).numpy()
    sid, bexp, total, bad = oalign.align(ids.tolist(), E, bm)
    check_invariants(ids, E, bm, sid, bexp, total)
    assert not bad


def test_counts_zero_one_block_and_block_plus_one():
    bm, E = 16, 5
    # expert 0: 0 rows, 1: 1 row, 2: exactly bm rows, 3: bm + 1 rows, 4: 2
    flat = [1] + [2] * bm + [3] * (bm + 1) + [4] * 2
    ids = [[e] for e in flat]
    sid, bexp, total, _ = oalign.align(ids, E, bm)
    assert total == 0 + bm + bm + 2 * bm + bm
    assert bexp[: total // bm] == [1, 2, 3, 3, 4]
    check_invariants(ids, E, bm, sid, bexp, total)


def test_empty_and_invalid_ids():
    sid, bexp, total, bad = oalign.align([], 8, 16)
    assert total == 0 and sid == [0] * (8 * 15) and all(e == -1 for e in bexp)
    ids = [[0, -1], [5, 1]]  # -1 is skipped silently, 5 is out of range for E=4
    sid, bexp, total, bad = oalign.align(ids, 4, 2)
    assert bad
    assert total == 4 and sid[:4] == [0, 4, 3, 4]
    sid, bexp, total, bad = oalign.align([[0, -1]], 4, 2)
    assert not bad and total == 2


def test_padded_length_identity_and_worst_case(golden):
    g = golden("moe_byte_model.json")["dsv3"]
    A = g["trace_T"] * g["k"]
    assert oalign.max_padded(A, g["E"], g["trace_block_m"]) == g["trace_max_padded"]
    assert oalign.max_blocks(A, g["E"], g["trace_block_m"]) == g["trace_expert_id_entries"]
    for kind in ("uniform", "skewed", "hot"):
        ids = make_topk_ids(64, 8, 256, seed=3, kind=kind).numpy()
        sid, bexp, total, _ = oalign.align(ids.tolist(), 256, 16)
        counts = np.bincount(ids.reshape(-1), minlength=256)
        assert total == int((np.ceil(counts / 16) * 16).sum()) <= A + 256 * 15

"""Block-alignment oracle, in plain Python.

Test infrastructure only (see ``oracle/__init__``).

What is computed follows [MoE] "vLLM's Triton path: align, then index"
(the worked docstring example and the description of the kernel: per-expert
counts, each count rounded up to a whole block, an exclusive scan into
offsets, the block-to-expert table with -1 after the padded length) and
[Kernels] "Alignment: making ragged routing tileable" (flat assignment id
a = t*k + j, padding rows marked by the sentinel T*k, worst-case sizing
T*k + E*(BLOCK_M-1) so the padded length can stay on the device).

Readings where the pages leave a step open:

* within one expert the assignments keep ascending a (a stable order, which
  is what the docstring example shows);
* every slot of ``sorted_ids`` that holds no assignment, up to the worst-case
  length, holds the sentinel T*k; ``block_expert`` is -1 from the padded
  length up to its worst-case length;
* an id of -1 is skipped (not an assignment of any local expert); any other
  id outside [0, E) is skipped too and reported in ``bad_ids``.

Pinned by the docstring example (tests/golden/align_docstring.json), by the
special case BLOCK_M = 1 (a stable argsort) and by the invariants.
"""


def max_padded(num_assignments, E, block_m):
    """Worst-case padded length T*k + E*(BLOCK_M-1) ([Kernels] Alignment)."""
    return num_assignments + E * (block_m - 1)


def max_blocks(num_assignments, E, block_m):
    return -(-max_padded(num_assignments, E, block_m) // block_m)


def align(topk_ids, E, block_m):
    """Returns (sorted_ids list, block_expert list, num_post_padded, bad_ids).

    ``topk_ids`` is any nested sequence / array of shape [T, k]."""
    flat = [int(v) for row in topk_ids for v in row]
    A = len(flat)
    per_expert = [[] for _ in range(E)]
    bad_ids = False
    for a, e in enumerate(flat):  # ascending a keeps the order stable
        if 0 <= e < E:
            per_expert[e].append(a)
        elif e != -1:
            bad_ids = True
    n_slots = max_padded(A, E, block_m)
    n_blocks = max_blocks(A, E, block_m)
    sorted_ids = [A] * n_slots
    block_expert = [-1] * n_blocks
    start = 0
    for e in range(E):
        members = per_expert[e]
        padded = -(-len(members) // block_m) * block_m
        for r, a in enumerate(members):
            sorted_ids[start + r] = a
        for b in range(start // block_m, (start + padded) // block_m):
            block_expert[b] = e
        start += padded
    return sorted_ids, block_expert, start, bad_ids

"""The copy waits of the paired MXFP4 GEMM kernels (host check).

Each of the kernel's two copy streams (activation rows, weight rows) issues
L copy instructions per K step, D steps ahead of the step that reads them, and
every wave also copies one scale group (four steps' worth of e8m0 scales)
right after the copies of every fourth step.  Before step s a wave waits
until at most n of its copies are in flight, n being the number it issued
after the last copy of step s (copies complete in issue order).  The kernel
computes n in closed form (``copies_after`` in ffn_gemm.hip, restated below);
this test replays the issue order instruction by instruction and counts.  A
count one too high lets the barrier pass while a copy of step s is still
landing in LDS.

GEMM1's weight waves also issue their epilogue stores between the next
tile's copies ahead of step 0 and that tile's first step (vector memory
operations complete in issue order, stores included); the kernel adds their
count to the waits of the steps whose copies went out before them.
"""

import pytest

SCG = 4  # steps per scale group


def copies_after(L, D, s, nk, ng):
    """The kernel's closed form."""
    n = L * (min(s + D - 1, nk - 1) - s)
    for i in range(D):
        u = s - D + i
        if u >= 0 and u % SCG == 0 and u // SCG + 1 < ng:
            n += 1
    return n


def kernel_wait(L, D, s, nk, ng, stores):
    """The kernel's count with `stores` stores after the copies ahead of step 0."""
    return copies_after(L, D, s, nk, ng) + (stores if s < D else 0)


def replay(L, D, nk, stores=0):
    """Issue order of one tile: scale group 0, the copies of steps 0..D-1,
    `stores` stores, then at each step s the copies of step s + D (if it
    exists) and, when s is a multiple of SCG, scale group s / SCG + 1 (if it
    exists)."""
    ng = nk // SCG
    seq = [("scale", 0)] + [("copy", st) for st in range(min(D, nk)) for _ in range(L)]
    seq += [("store", i) for i in range(stores)]
    after = []
    for s in range(nk):
        last = max(i for i, item in enumerate(seq) if item == ("copy", s))
        after.append(len(seq) - 1 - last)
        if s + D < nk:
            seq += [("copy", s + D)] * L
        if s % SCG == 0 and s // SCG + 1 < ng:
            seq.append(("scale", s // SCG + 1))
    return after, ng


@pytest.mark.parametrize("L", [4, 8])
@pytest.mark.parametrize("D", [1, 2, 3, 4])
@pytest.mark.parametrize("nk", [4, 8, 16, 32, 64])
def test_copies_after_matches_issue_order(L, D, nk):
    after, ng = replay(L, D, nk)
    for s in range(nk):
        assert copies_after(L, D, s, nk, ng) == after[s], f"step {s}"


@pytest.mark.parametrize("L", [4, 8])
@pytest.mark.parametrize("D", [1, 2, 3])
@pytest.mark.parametrize("nk", [4, 8, 32])
@pytest.mark.parametrize("stores", [0, 2, 4, 8])
def test_waits_with_epilogue_stores(L, D, nk, stores):
    after, ng = replay(L, D, nk, stores)
    for s in range(nk):
        assert kernel_wait(L, D, s, nk, ng, stores) == after[s], f"step {s}"
        # a lower count of stores only waits longer
        assert kernel_wait(L, D, s, nk, ng, 0) <= after[s]


def test_scale_group_lands_before_its_first_step():
    """With D < SCG a scale group is issued before the copies of its first
    step, so the wait ahead of that step covers it (D = SCG would not)."""
    for D in range(1, SCG):
        for nk in (8, 16, 32):
            ng = nk // SCG
            seq = [("scale", 0)] + [("copy", st) for st in range(D) for _ in range(4)]
            for s in range(nk):
                if s + D < nk:
                    seq += [("copy", s + D)] * 4
                if s % SCG == 0 and s // SCG + 1 < ng:
                    seq.append(("scale", s // SCG + 1))
            for G in range(ng):
                first_copy = min(i for i, it in enumerate(seq) if it == ("copy", G * SCG))
                assert seq.index(("scale", G)) < first_copy

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


def replay(L, D, nk):
    """Issue order of one tile: scale group 0, the copies of steps 0..D-1,
    then at each step s the copies of step s + D (if it exists) and, when s
    is a multiple of SCG, scale group s / SCG + 1 (if it exists)."""
    ng = nk // SCG
    seq = [("scale", 0)] + [("copy", st) for st in range(min(D, nk)) for _ in range(L)]
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

"""The counted waits of the LDS-staged backward kernels (csrc/rmsn_bwd_lds.h),
checked on a model of a wavefront's vector-memory counter.

A wavefront's vector memory operations complete in issue order, so waiting
until at most K of them are outstanding means every operation older than the
newest K has completed. Each kernel waits, at iteration j, with
K = (ST - 1) * L + min(j, ST) * Q, where ST is the number of LDS stages, L the
copies that fill one stage (per lane) and Q the dx stores of one iteration.
The model replays each kernel's issue order (prologue, then per iteration:
wait, read stage j % ST, refill it with block j + ST, store dx) and checks
that the wait is exact: the stage read at iteration j has completed, and
exactly K operations are newer than its last copy (no wait is looser, and
none waits for copies of later stages). Extra operations the compiler may
add (spill stores, reloads) only make each wait stricter.
"""

import pytest


def _replay(prologue, ST, L, Q, walk):
    """Issue order of one wavefront as a list of ("copy", block) / ("store", j) /
    ("other", i); returns, per iteration, the number of operations newer than
    the last copy of the block read there, and the wait threshold used."""
    ops = list(prologue)
    out = []
    for j in range(walk):
        K = (ST - 1) * L + min(j, ST) * Q
        last = max(i for i, op in enumerate(ops) if op == ("copy", j))
        out.append((len(ops) - 1 - last, K))
        ops += [("copy", j + ST)] * L
        ops += [("store", j)] * Q
    return out


def _bwd_lds_prologue(ST, L, kvecs):
    # the weights are copied into the last stage's slots first, then stages
    # 0 .. ST-2; after a wait of (ST - 1) * L the weights are read and stage
    # ST - 1 is issued
    ops = [("other", q) for q in range(kvecs)]
    for s in range(ST - 1):
        ops += [("copy", s)] * L
    newer = len(ops) - kvecs  # operations newer than the last weight copy
    assert newer == (ST - 1) * L, "the prologue's wait for the weights"
    ops += [("copy", ST - 1)] * L
    return ops


# (inputs per stage: x, dy and dh with the residual add; stages built) of bwd_lds
LDS_BUILT = [(2, st) for st in (2, 3, 4, 6, 8)] + [(3, st) for st in (2, 3, 4, 6)]


@pytest.mark.parametrize("nin,ST", LDS_BUILT)
@pytest.mark.parametrize("kvecs", [1, 2])  # weight vectors per lane: 16-bit or fp32 weights
def test_bwd_lds_waits_are_exact(nin, ST, kvecs):
    L, Q = nin + 1, 1  # the inputs and rstd; one dx store per iteration
    for walk in range(1, 3 * ST + 3):
        for newer, K in _replay(_bwd_lds_prologue(ST, L, kvecs), ST, L, Q, walk):
            assert newer == K


# (vectors per lane, stages) of bwd_wide_lds
WIDE_LDS_BUILT = [(2, 1), (2, 2), (3, 1), (4, 1), (4, 2), (6, 1)]


@pytest.mark.parametrize("vpt,ST", WIDE_LDS_BUILT)
def test_bwd_wide_lds_waits_are_exact(vpt, ST):
    L, Q = 2 * vpt + 1, vpt  # x and dy vectors and rstd; vpt dx stores per row
    prologue = []
    for s in range(ST):  # the kept weights are waited for before the prologue
        prologue += [("copy", s)] * L
    for walk in range(1, 3 * ST + 3):
        for newer, K in _replay(prologue, ST, L, Q, walk):
            assert newer == K


def test_model_catches_a_loose_wait():
    """A threshold one larger than the formula leaves the stage's last copy
    possibly in flight: the model must see newer < K + 1."""
    ST, L, Q = 2, 3, 1
    for newer, K in _replay(_bwd_lds_prologue(ST, L, 1), ST, L, Q, 5):
        assert newer < K + 1

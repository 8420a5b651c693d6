"""The split-row backward's exchange (csrc/rmsn_bwd_split.h), checked on a
model under random interleavings.

Each of K members of a group walks the same rows. For its i-th row a member
writes the word (tag i + 1, its part) into word i % 2 of its own slot, then
reads every partner's word i % 2 until the tag reads i + 1, and only then
moves to row i + 1. The model runs the K members as interleaved steps under a
seeded random scheduler (one member advances one step at a time, polls that
do not match simply fail and are retried later) and checks that every part a
member takes is the partner's part for that same row, and that the walk never
deadlocks: two words per slot suffice because a member reaches row i + 2 only
after every partner published row i + 1, which each did after reading row i.
A variant with one word per slot is shown to fail, so the check has teeth.
"""

import random

import pytest


def _run(K, rows, seed, words=2):
    rng = random.Random(seed)
    slots = [[(0, None)] * words for _ in range(K)]  # (tag, value); zeroed by the fill kernel
    # per member: row index, phase ("publish" or "read"), next partner to read, parts taken
    st = [{"i": 0, "phase": "publish", "p": 0, "got": []} for _ in range(K)]
    taken = {}
    steps = 0
    while any(s["i"] < rows for s in st):
        live = [k for k in range(K) if st[k]["i"] < rows]
        # deadlock: no live member can make progress
        def can_move(k):
            s = st[k]
            if s["phase"] == "publish":
                return True
            p = s["p"]
            return slots[p][s["i"] % words][0] == s["i"] + 1
        movable = [k for k in live if can_move(k)]
        if not movable:
            return None, steps
        k = rng.choice(movable)
        s = st[k]
        if s["phase"] == "publish":
            slots[k][s["i"] % words] = (s["i"] + 1, (k, s["i"]))
            s["phase"], s["p"], s["got"] = "read", 0, []
        else:
            tag, val = slots[s["p"]][s["i"] % words]
            s["got"].append(val)
            s["p"] += 1
            if s["p"] == K:
                taken[(k, s["i"])] = s["got"]
                s["i"] += 1
                s["phase"] = "publish"
        steps += 1
    return taken, steps


@pytest.mark.parametrize("K", [2, 3, 4, 16])
def test_every_part_taken_is_the_partners_part_for_that_row(K):
    for seed in range(200):
        rows = 1 + seed % 7
        taken, _ = _run(K, rows, seed)
        assert taken is not None, f"deadlock K={K} rows={rows} seed={seed}"
        for (k, i), got in taken.items():
            assert got == [(p, i) for p in range(K)], (K, rows, seed, k, i, got)


def test_one_word_per_slot_fails():
    """With one word per slot a fast member overwrites its part for row i with
    row i + 1's before a slow partner has read it; the slow partner then waits
    for a tag that never comes back."""
    failures = 0
    for seed in range(200):
        taken, _ = _run(3, 6, seed, words=1)
        if taken is None:
            failures += 1
    assert failures > 0

"""The split-row backward's exchange (csrc/rmsn_bwd_split.h), checked on a
model under random interleavings.

Each of K members of a group walks the same rows. For its i-th row a member
writes the word (tag i + 1, its part) into word i % 2 of its own slot, then
reads every partner's word i % 2 until the tag reads i + 1, and only then
moves to row i + 1. The kernel polls all partners at once (one lane each), so
the model lets a member take its partners' words in any order, whichever is
ready first (and, as a second case, strictly in member order). It runs the K
members as interleaved steps under a seeded random scheduler (one member
advances one step at a time; polls that do not match simply fail and are
retried later) and checks that every part a member takes is the partner's
part for that same row, and that the walk never deadlocks: two words per
slot suffice because a member reaches row i + 2 only after every partner
published row i + 1, which each did after reading row i. A variant with one
word per slot is shown to fail, so the check has teeth.
"""

import random

import pytest


def _run(K, rows, seed, words=2, order="any"):
    rng = random.Random(seed)
    slots = [[(0, None)] * words for _ in range(K)]  # (tag, value); zeroed by the fill kernel
    # per member: row index, phase ("publish" or "read"), partners not yet read, parts taken
    st = [{"i": 0, "phase": "publish", "left": [], "got": {}} for _ in range(K)]
    taken = {}
    steps = 0

    def ready(k):
        """The partners member k may take now: any unread one whose tag is this row's
        (order "any"), or only the next one in member order (order "member")."""
        s = st[k]
        cand = s["left"] if order == "any" else s["left"][:1]
        return [p for p in cand if slots[p][s["i"] % words][0] == s["i"] + 1]

    while any(s["i"] < rows for s in st):
        live = [k for k in range(K) if st[k]["i"] < rows]
        movable = [k for k in live if st[k]["phase"] == "publish" or ready(k)]
        if not movable:  # deadlock: no live member can make progress
            return None, steps
        k = rng.choice(movable)
        s = st[k]
        if s["phase"] == "publish":
            slots[k][s["i"] % words] = (s["i"] + 1, (k, s["i"]))
            s["phase"], s["left"], s["got"] = "read", list(range(K)), {}
        else:
            p = rng.choice(ready(k))
            s["got"][p] = slots[p][s["i"] % words][1]
            s["left"].remove(p)
            if not s["left"]:
                taken[(k, s["i"])] = [s["got"][q] for q in range(K)]  # added in member order
                s["i"] += 1
                s["phase"] = "publish"
        steps += 1
    return taken, steps


@pytest.mark.parametrize("order", ["any", "member"])
@pytest.mark.parametrize("K", [2, 3, 4, 16])
def test_every_part_taken_is_the_partners_part_for_that_row(K, order):
    for seed in range(200):
        rows = 1 + seed % 7
        taken, _ = _run(K, rows, seed, order=order)
        assert taken is not None, f"deadlock K={K} rows={rows} seed={seed}"
        for (k, i), got in taken.items():
            assert got == [(p, i) for p in range(K)], (K, rows, seed, k, i, got)


def test_one_word_per_slot_fails():
    """With one word per slot a fast member overwrites its part for row i with
    row i + 1's before a slow partner has read it; the slow partner then waits
    for a tag that never comes back."""
    for order in ("any", "member"):
        failures = 0
        for seed in range(200):
            taken, _ = _run(3, 6, seed, words=1, order=order)
            if taken is None:
                failures += 1
        assert failures > 0, order

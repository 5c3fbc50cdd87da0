"""A model of the in-launch merge's synchronization, checked over every interleaving.

The main kernel's work-groups of one merge group (segments 0 .. S-1 of a
sequence and head group) synchronize through one 32-bit word (arrivals in bits
0-7, a generation above them) and a 64-bit mask of shares handed to the last
arrival (csrc/segment_merge.h, merge_in_launch). Each step below is one atomic
operation of a work-group's thread 0, taken in a single global order: the
kernel issues each of its second atomics only once its first is performed, so
the pairs that the argument rests on (set the bit, then read the word; move the
generation, then take the mask) are ordered as in this model.

A waiting work-group may give up after any poll (the bounded wait): the search
takes both branches at every poll. Over all interleavings and choices it checks
that every share is merged at least once, only after every work-group has
written its partials, and that the call leaves the arrivals and the mask at
zero and the generation one higher, ready for the next call.

The search is exhaustive for S = 2, 3 and 4 (163290 states at 4; two calls in a row at
S = 2); it runs on the CPU in about a second.
"""

import pytest

GEN = 1 << 8
COUNT = GEN - 1
MAX_POLLS = 2   # polls before a waiter may still choose to wait once more


def initial(S, word=0, handed=0):
    # per work-group: (pc, g0, polls); pc names the next step
    return (word, handed, tuple(("arrive", 0, 0) for _ in range(S)), frozenset(), 0)


def steps(state, S):
    """All successor states (one atomic step of one work-group)."""
    word, handed, wgs, merged, written = state
    out = []
    for k, (pc, g0, polls) in enumerate(wgs):
        def put(new_pc, new_g0=g0, new_polls=polls, w=word, h=handed, m=merged, wr=written):
            lst = list(wgs)
            lst[k] = (new_pc, new_g0, new_polls)
            out.append((w, h, tuple(lst), m, wr))

        def merge(shares, m=None):
            # a merge reads every segment's partials: all must be written
            assert written == (1 << S) - 1, "merge before every partial was written"
            return (merged if m is None else m) | frozenset(shares)

        if pc == "arrive":
            # partials written (stores complete), then the arrival is counted
            old = word
            wr = written | (1 << k)
            if (old & COUNT) == S - 1:
                put("bump", old >> 8, w=old + 1, wr=wr)
            else:
                put("poll", old >> 8, w=old + 1, wr=wr)
        elif pc == "bump":
            # the last arrival: count S + (256 - S) carries into the generation
            put("merge_last", w=word + (GEN - S))
        elif pc == "merge_last":
            put("take_mask", m=merge({k}))
        elif pc == "take_mask":
            # exchange(handed, 0), then merge every handed-over share
            rescued = {s for s in range(S) if handed >> s & 1}
            put("done", h=0, m=merge(rescued))
        elif pc == "poll":
            if (word >> 8) != g0:
                put("merge_own")
            else:
                if polls < MAX_POLLS:
                    put("poll", new_polls=polls + 1)   # still waiting
                put("give_up")                         # the time limit passed
        elif pc == "give_up":
            put("recheck", h=handed | (1 << k))        # fetch_or(handed, bit)
        elif pc == "recheck":
            if (word >> 8) != g0:                      # fetch_add(word, 0)
                put("clear_bit")
            else:
                put("done")                            # the last arrival will see the bit
        elif pc == "clear_bit":
            put("merge_own", h=handed & ~(1 << k))     # fetch_and(handed, ~bit)
        elif pc == "merge_own":
            put("done", m=merge({k}))
    return out


def explore(S, start):
    """Every final state reachable from start (all work-groups done)."""
    finals, seen, stack = set(), set(), [start]
    while stack:
        st = stack.pop()
        if st in seen:
            continue
        seen.add(st)
        nxt = steps(st, S)
        if not nxt:
            assert all(pc == "done" for pc, _, _ in st[2]), f"stuck: {st}"
            finals.add(st)
        stack.extend(nxt)
    return finals, len(seen)


@pytest.mark.parametrize("S", [2, 3, 4])
def test_every_share_merged_and_state_restored(S):
    start_word = 5 * GEN   # an arbitrary earlier generation, arrivals zero
    finals, n = explore(S, initial(S, word=start_word))
    assert n > 10 and finals
    for word, handed, wgs, merged, written in finals:
        assert merged == frozenset(range(S)), merged
        assert written == (1 << S) - 1
        assert word == start_word + GEN, (word, start_word)   # count 0, generation + 1
        assert handed == 0


def test_two_calls_in_a_row():
    """The second call starts from every state the first can leave."""
    S = 2
    finals, _ = explore(S, initial(S))
    for word, handed, _, _, _ in finals:
        finals2, _ = explore(S, initial(S, word=word, handed=handed))
        for word2, handed2, _, merged2, _ in finals2:
            assert merged2 == frozenset(range(S))
            assert word2 == 2 * GEN and handed2 == 0


def test_a_planted_mistake_is_caught():
    """Without the re-read after setting the bit, a share can be left unmerged:
    the check above would fail. Planted in the model, on the CPU."""
    S = 2
    original = steps

    def broken(state, S_):
        out = []
        for st in original(state, S_):
            lst = list(st[2])
            # a waiter that gives up exits right after setting its bit
            lst = [("done", g0, p) if pc == "recheck" else (pc, g0, p) for pc, g0, p in lst]
            out.append((st[0], st[1], tuple(lst), st[3], st[4]))
        return out

    finals, seen, stack = set(), set(), [initial(S)]
    while stack:
        st = stack.pop()
        if st in seen:
            continue
        seen.add(st)
        nxt = broken(st, S)
        if not nxt:
            finals.add(st)
        stack.extend(nxt)
    assert any(merged != frozenset(range(S)) for _, _, _, merged, _ in finals)

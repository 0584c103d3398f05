"""The FP8 row rendezvous's counting protocol, checked on the CPU by exploring every interleaving.

The GEMM kernels merge each row's absmax across the column tiles of a row block with a
rendezvous in the workspace: every tile publishes its slots, reads the block's release flag,
arrives at its group's counter (the group's last arrival resets that counter and, with the
two-level merge, folds the group's slots into the group slot), the last group to arrive at the
block counter resets it and raises the flag to the next generation, and every tile waits until
the flag differs from what it read, then reads the slots.

This test restates those steps as a small state machine per tile, with each load, store and
atomic as one indivisible step performed in program order (the order the kernels enforce with
their waits; the memory-ordering argument itself is not what is checked here), and explores
every reachable state for a few row-block shapes, over two consecutive calls on one workspace.
It checks that
  * no state is stuck with tiles still waiting (no deadlock, no lost release),
  * no tile reads before every slot it reads was written (tile slots, or group slots),
  * after a call the counters are back at zero and the flag has moved by exactly one, so the
    next call starts from a valid state,
  * a flag raised by the block cannot be seen before the tile has arrived (a tile reads the
    flag before arriving, and the raise needs every arrival).
"""
import pytest

# per-tile program counters
PUBLISH, READ_FLAG, ARRIVE_GROUP, RESET_GROUP, FOLD, ARRIVE_BLOCK, RESET_BLOCK, RAISE, WAIT, READ, DONE = range(11)


def explore(need, group, two_level, flag0=7, read_flag_first=True):
    """All reachable states of one call; returns the terminal shared states and the state count.
    read_flag_first=False moves the flag read after the group arrival (the order the kernels
    must not use)."""
    groups = (need + group - 1) // group
    in_group = [min(group, need - g * group) for g in range(groups)]
    gof = [t // group for t in range(need)]

    # state: (tiles, rec, gc, flag, slots, gslots); tile = (pc, gen, last, old_block)
    start = (tuple((PUBLISH, None, False, None) for _ in range(need)), 0, (0,) * groups, flag0,
             (False,) * need, (False,) * groups)
    seen, stack, terminal = {start}, [start], set()
    while stack:
        tiles, rec, gc, flag, slots, gslots = st = stack.pop()
        moves = []
        for t, (pc, gen, last, old_block) in enumerate(tiles):
            g = gof[t]

            def put(**kw):
                nt = list(tiles)
                nt[t] = kw.pop("tile")
                vals = dict(rec=rec, gc=gc, flag=flag, slots=slots, gslots=gslots)
                vals.update(kw)
                moves.append((tuple(nt), vals["rec"], vals["gc"], vals["flag"], vals["slots"], vals["gslots"]))

            if pc == PUBLISH:
                s = list(slots)
                s[t] = True
                put(tile=(READ_FLAG if read_flag_first else ARRIVE_GROUP, gen, last, old_block), slots=tuple(s))
            elif pc == READ_FLAG:
                if read_flag_first:
                    put(tile=(ARRIVE_GROUP, flag, last, old_block))
                else:  # after the arrival: on to what the arrival decided
                    put(tile=((FOLD if two_level else ARRIVE_BLOCK) if last else WAIT, flag, last, old_block))
            elif pc == ARRIVE_GROUP:
                c = list(gc)
                old = c[g]
                c[g] += 1
                put(tile=(RESET_GROUP, gen, old == in_group[g] - 1, old_block), gc=tuple(c))
            elif pc == RESET_GROUP:
                after = (FOLD if two_level else ARRIVE_BLOCK) if last else WAIT
                if not read_flag_first:
                    after = READ_FLAG
                if last:
                    c = list(gc)
                    c[g] = 0
                    put(tile=(after, gen, last, old_block), gc=tuple(c))
                else:
                    put(tile=(after, gen, last, old_block))
            elif pc == FOLD:
                # the group's last arrival reads every slot of its group
                members = [u for u in range(need) if gof[u] == g]
                assert all(slots[u] for u in members), ("fold before the group published", st)
                gs = list(gslots)
                gs[g] = True
                put(tile=(ARRIVE_BLOCK, gen, last, old_block), gslots=tuple(gs))
            elif pc == ARRIVE_BLOCK:
                put(tile=(RESET_BLOCK if rec == groups - 1 else WAIT, gen, last, rec), rec=rec + 1)
            elif pc == RESET_BLOCK:
                put(tile=(RAISE, gen, last, old_block), rec=0)
            elif pc == RAISE:
                put(tile=(WAIT, gen, last, old_block), flag=gen + 1)
            elif pc == WAIT:
                if flag != gen:  # enabled only once the flag has moved
                    put(tile=(READ, gen, last, old_block))
            elif pc == READ:
                if two_level:
                    assert all(gslots), ("group slots read before every group folded", st)
                assert all(slots), ("slots read before every tile published", st)
                assert flag == gen + 1, ("a tile saw a flag other than the next generation", st)
                put(tile=(DONE, gen, last, old_block))
        if not moves:
            assert all(pc == DONE for pc, *_ in tiles), ("stuck: tiles wait for a release that never comes", st)
            terminal.add((rec, gc, flag))
        for m in moves:
            if m not in seen:
                seen.add(m)
                stack.append(m)
    return terminal, len(seen)


@pytest.mark.parametrize("need,group,two_level", [
    (1, 2, False), (2, 2, False), (3, 2, False), (4, 2, False),   # decode-like: slots read directly
    (1, 2, True), (3, 2, True), (4, 2, True), (5, 2, True), (4, 3, True),  # group slots, uneven groups
])
def test_rendezvous_counting(need, group, two_level):
    flag0 = 7
    terminal, states = explore(need, group, two_level, flag0)
    groups = (need + group - 1) // group
    assert states > need  # the search really interleaved the tiles
    # every interleaving ends with the counters reset and the flag one generation further
    assert terminal == {(0, (0,) * groups, flag0 + 1)}, terminal
    # so the next call on the same workspace starts where the first one did, one generation on
    terminal2, _ = explore(need, group, two_level, flag0 + 1)
    assert terminal2 == {(0, (0,) * groups, flag0 + 2)}


def test_reading_the_flag_after_arriving_can_deadlock():
    """Why a tile reads the flag before it arrives: read after, the last arrival's raise may be
    what it reads, and it then waits for a generation that never comes. The same exploration with
    the two steps swapped finds such a stuck state (and the one-tile block, which has no other
    arrival to race with, still completes)."""
    for two_level in (False, True):
        with pytest.raises(AssertionError, match="stuck"):
            explore(2, 2, two_level, read_flag_first=False)
    terminal, _ = explore(1, 2, False, read_flag_first=False)
    assert terminal == {(0, (0,), 8)}

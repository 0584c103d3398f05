"""Tile tickets for the FP8 row rendezvous, checked on the CPU by exploring every schedule.

When a quantised call has more tiles than the device holds at once, each workgroup draws a
ticket when it starts (an atomic increment of a workspace counter; the workgroup that draws the
last ticket resets the counter for the next call), processes the tile that ticket names in
row-block-major order, and waits at the rendezvous until every column tile of its row block has
arrived. The host refuses such a call unless the device can hold one row block's tiles at once.

This test restates that as a state machine: `resident` workgroup slots, workgroups dispatched in
order whenever a slot is free, each drawing, arriving and waiting as one step each, and explores
every order in which the running workgroups take their steps. It checks that every schedule
finishes (no state where every running workgroup waits for a tile no running workgroup holds)
and leaves the counter at zero, whenever `resident` is at least the tiles per row block, and
that with fewer slots a stuck schedule exists, which is why the host check is there.
"""
import pytest

DRAW, ARRIVE, WAIT = range(3)


def explore(blocks, per_block, resident):
    total = blocks * per_block
    # state: (counter, dispatched, running (sorted tuple of (phase, ticket)), arrivals per block)
    start = (0, 0, (), (0,) * blocks)
    seen, stack, finals = {start}, [start], set()
    while stack:
        counter, dispatched, running, arr = st = stack.pop()
        moves = []
        if dispatched < total and len(running) < resident:
            moves.append((counter, dispatched + 1, tuple(sorted(running + ((DRAW, -1),))), arr))
        for i, (phase, ticket) in enumerate(running):
            rest = running[:i] + running[i + 1:]
            if phase == DRAW:
                t = counter
                nc = 0 if t == total - 1 else counter + 1
                moves.append((nc, dispatched, tuple(sorted(rest + ((ARRIVE, t),))), arr))
            elif phase == ARRIVE:
                a = list(arr)
                a[ticket // per_block] += 1
                moves.append((counter, dispatched, tuple(sorted(rest + ((WAIT, ticket),))), tuple(a)))
            elif phase == WAIT and arr[ticket // per_block] == per_block:
                moves.append((counter, dispatched, tuple(sorted(rest)), arr))  # done: the slot frees
        if not moves:
            assert dispatched == total and not running, ("stuck", st)
            finals.add((counter, arr))
        for m in moves:
            if m not in seen:
                seen.add(m)
                stack.append(m)
    return finals


@pytest.mark.parametrize("blocks,per_block,resident", [(3, 2, 2), (3, 2, 3), (2, 3, 3), (3, 3, 4), (4, 2, 3)])
def test_every_schedule_finishes(blocks, per_block, resident):
    finals = explore(blocks, per_block, resident)
    # every tile arrived, and the counter is back at zero for the next call
    assert finals == {(0, (per_block,) * blocks)}


@pytest.mark.parametrize("blocks,per_block,resident", [(2, 3, 2), (3, 2, 1)])
def test_fewer_slots_than_a_row_block_can_stick(blocks, per_block, resident):
    with pytest.raises(AssertionError, match="stuck"):
        explore(blocks, per_block, resident)

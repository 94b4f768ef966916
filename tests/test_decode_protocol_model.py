"""CPU model of the decode kernel's cross-workgroup protocol (the split-K tile
counters, the router-completion counter and the row-group claims of the
fused top-16, with the call parity that lets consecutive calls share one
workspace without a finish counter).

Each workgroup is a Python generator that yields before every access to the
shared counters; a seeded scheduler interleaves the workgroups of one launch
in random orders (every interleaving of atomic steps is a legal execution
under sequentially consistent atomics). Consecutive launches run one after
the other, as launches on one stream do, with row counts changing from call
to call. Checked: every row group of a call is selected exactly once, only
after every router tile of that call is combined; the per-tile counters are
back at zero after every call; the pair the next call will use is cleared
and the parity flips once per call.

The model mirrors the kernel's steps (decode_route_kernel, router_unit,
latent_unit, first_claim and the claim loop), with the whole route's tile
counts and the packed launch's K splits.
"""
import random

import pytest

ROW_GROUP = 4
RT_TILES, LAT_TILES = 28, 56


class Workspace:
    def __init__(self):
        self.tile = {("rt", t): 0 for t in range(RT_TILES)}
        self.tile.update({("lat", t): 0 for t in range(LAT_TILES)})
        self.par = 0
        self.pair = [[0, 0], [0, 0]]        # per parity: {router tiles combined, groups claimed}


class Call:
    def __init__(self, rows, splits_l, splits_r):
        self.rows = rows
        self.splits_l, self.splits_r = splits_l, splits_r
        self.rt_combined = 0                # tiles whose logits are stored (ground truth)
        self.selected = []                  # row groups in the order they were selected
        self.bad = []


def row_phase(ws, call, par, first_row, claimer):
    """The claim loop: select group r, then (if rows remain past it) claim
    the next group; stop when a claim lands past the last row."""
    r = first_row
    while r >= 0:
        more = r + ROW_GROUP < call.rows
        if call.rt_combined != RT_TILES:
            call.bad.append(("selected before the logits were complete", r, claimer))
        call.selected.append(r)
        yield
        nxt = -1
        if more:
            c = ROW_GROUP + ws.pair[par][1]
            ws.pair[par][1] += ROW_GROUP   # one atomic add
            yield
            if c < call.rows:
                nxt = c
        r = nxt


def router_unit(ws, call, b):
    par = ws.par & 1                        # thread 0 reads the parity at the start
    yield
    tile = b % RT_TILES
    prev = ws.tile[("rt", tile)]            # publish the partial: counter add
    ws.tile[("rt", tile)] += 1
    yield
    if prev != call.splits_r - 1:
        return
    call.rt_combined += 1                   # the tile's logits are stored
    ws.tile[("rt", tile)] = 0
    yield
    prev = ws.pair[par][0]                  # router completion counter
    ws.pair[par][0] += 1
    yield
    if prev != RT_TILES - 1:
        return
    yield from row_phase(ws, call, par, 0, ("router", b))
    other = ws.pair[par ^ 1]                # the previous call's pair: clear it,
    other[0] = 0
    yield
    other[1] = 0
    yield
    ws.par = par ^ 1                        # then flip the parity
    yield


def latent_unit(ws, call, b):
    par = ws.par & 1
    yield
    tile = b % LAT_TILES
    prev = ws.tile[("lat", tile)]
    ws.tile[("lat", tile)] += 1
    yield
    if prev != call.splits_l - 1:
        return
    ws.tile[("lat", tile)] = 0
    yield
    # first claim: one coherent load of the pair, a claim only if the router
    # is complete and a group is left
    done, claimed = ws.pair[par]
    yield
    r = -1
    if done == RT_TILES and ROW_GROUP + claimed < call.rows:
        c = ROW_GROUP + ws.pair[par][1]
        ws.pair[par][1] += ROW_GROUP
        yield
        if c < call.rows:
            r = c
    if r >= 0:
        yield from row_phase(ws, call, par, r, ("latent", b))


def run_call(ws, rng, rows, splits_l=4, splits_r=8):
    call = Call(rows, splits_l, splits_r)
    par0 = ws.par
    wgs = [router_unit(ws, call, b) for b in range(RT_TILES * splits_r)]
    wgs += [latent_unit(ws, call, b) for b in range(LAT_TILES * splits_l)]
    # dispatch: workgroups start in index order but run at any relative pace;
    # a not-yet-started workgroup may start at any point
    live = []
    pending = list(wgs)
    while pending or live:
        if pending and (not live or rng.random() < 0.3):
            live.append(pending.pop(0))
            continue
        g = live[rng.randrange(len(live))]
        try:
            next(g)
        except StopIteration:
            live.remove(g)
    assert not call.bad, call.bad[:3]
    groups = list(range(0, rows, ROW_GROUP))
    assert sorted(call.selected) == groups, (rows, call.selected)
    assert all(v == 0 for v in ws.tile.values())
    assert ws.par == par0 ^ 1
    assert ws.pair[ws.par] == [0, 0]
    return call


@pytest.mark.parametrize("seed", range(6))
def test_protocol_over_consecutive_calls(seed):
    rng = random.Random(seed)
    ws = Workspace()
    for _ in range(12):
        rows = rng.randint(1, 20)
        splits_l = rng.choice([4, 8])
        run_call(ws, rng, rows, splits_l=splits_l, splits_r=8)


def test_every_width_in_sequence():
    rng = random.Random(99)
    ws = Workspace()
    for rows in list(range(1, 21)) + list(range(20, 0, -1)):
        run_call(ws, rng, rows)


def test_model_catches_a_missing_clear():
    """The model is sharp enough to see a planted slip: without clearing the
    other pair, the second call's claims start from the stale count and a row
    group goes unselected, or the pair is not idle."""
    rng = random.Random(5)
    ws = Workspace()
    run_call(ws, rng, 20)
    ws.pair[ws.par] = [RT_TILES, 16]        # as if the clear had been skipped
    with pytest.raises(AssertionError):
        run_call(ws, rng, 20)

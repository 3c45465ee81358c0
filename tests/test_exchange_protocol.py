"""CPU model of the fused amax's grid exchange (host logic, no GPU).

The single-pass quantizer finds the tensor amax by an exchange through a
caller-owned workspace: every workgroup reads the generation word, posts
(generation, its maximum) in its arrival slot, workgroup 0 collects the
arrivals and posts (generation, amax) in every release slot; every wait is
bounded, and a workgroup whose wait expires computes the amax directly.

This model replays that protocol step by step under chosen interleavings of
workgroup starts, for two rules of when the generation word advances:

- "on_collect": workgroup 0 stores the generation once it has released the
  amax, whether or not its wait expired;
- "last_reader": every workgroup counts itself after posting its arrival
  (so after reading the generation) and the one that completes the count
  stores the generation; this is the rule the kernel implements.

With "on_collect", a workgroup of call N that starts after workgroup 0 gave
up reads call N+1's generation and posts its stale maximum under it; call
N+1's workgroup 0 can then take that for a fresh arrival. "last_reader"
never lets a workgroup read a generation other than its own call's.
"""
import itertools
import random

import pytest


class Workspace:
    def __init__(self, slots=64):
        self.gen = 0
        self.count = 0
        self.arrive = [(0, 0)] * slots
        self.release = [(0, 0)] * slots


def run_call(ws, maxima, order, rule, late=(), wg0_gives_up=False, poll_before_late=True):
    """One call on `ws`. `maxima[i]` is workgroup i's maximum. `order` is the
    order in which workgroups start (workgroup 0 first, as it is dispatched
    first). Workgroups in `late` start only after workgroup 0 has finished its
    collection (they were not resident). With `wg0_gives_up`, workgroup 0's
    wait expires before any late workgroup arrives. Returns the amax every
    workgroup ends with."""
    grid = len(maxima)
    true_max = max(maxima)
    gen = {}
    rank = {}
    result = {}

    def start(i):
        gen[i] = ws.gen + 1  # read at the start of the kernel
        ws.arrive[i] = (gen[i], maxima[i])  # the post carries the value read
        if rule == "last_reader":
            rank[i] = ws.count
            ws.count += 1

    def finish(i):
        if rule == "last_reader" and rank[i] == grid - 1:
            ws.count = 0
            ws.gen = gen[i]

    early = [i for i in order if i not in late]
    assert early[0] == 0
    for i in early:
        start(i)
    # workgroup 0 collects: an arrival counts when its slot carries gen[0]
    got = [ws.arrive[i] for i in range(grid)]
    complete = all(g == gen[0] for g, _ in got)
    if complete and not wg0_gives_up:
        amax = max(v for _, v in got)
    else:
        amax = true_max  # wait expired: the direct amax
    for i in range(grid):
        ws.release[i] = (gen[0], amax)
    if rule == "on_collect":
        ws.gen = gen[0]
    result[0] = amax
    for i in early[1:]:
        g, v = ws.release[i]
        result[i] = v if g == gen[i] else true_max
    for i in late:
        start(i)
        g, v = ws.release[i]
        result[i] = v if g == gen[i] else true_max  # else its own wait expires
    for i in order:
        finish(i)
    return result


def call_outputs(ws, maxima, order, rule, **kw):
    res = run_call(ws, maxima, order, rule, **kw)
    return set(res.values())


@pytest.mark.parametrize("rule,stale", [("on_collect", True), ("last_reader", False)])
def test_late_workgroup_after_expired_wait(rule, stale):
    """Call 1 (a large maximum in workgroup 3, which starts late, after
    workgroup 0's wait expired), then call 2 on a tensor with small maxima.
    Under "on_collect" workgroup 3 of call 1 posts under call 2's
    generation and call 2 returns call 1's maximum."""
    ws = Workspace()
    grid = 4
    out1 = call_outputs(ws, [1, 2, 3, 1000], [0, 1, 2, 3], rule, late=(3,), wg0_gives_up=True)
    assert out1 == {1000}  # call 1 itself is always right
    # call 2: workgroup 0 polls before workgroup 3 has posted again; model
    # that by letting workgroup 3 start late once more (without an expiry)
    out2 = call_outputs(ws, [5, 6, 7, 8], [0, 1, 2, 3], rule, late=(3,))
    if stale:
        assert 1000 in out2  # the previous tensor's maximum leaks into call 2
    else:
        assert out2 == {8}
    assert ws.count == 0
    _ = grid


def test_last_reader_every_interleaving():
    """Every start order and every choice of late workgroups, over three
    consecutive calls with different maxima and expired or met waits: each
    call's every workgroup ends with that call's own amax, the generation
    advances by one per call and the count is back at zero."""
    grid = 4
    for perm in itertools.permutations(range(1, grid)):
        order = [0, *perm]
        for nlate in range(grid):
            for late in itertools.combinations(perm, nlate):
                ws = Workspace()
                for call, gives_up in enumerate((True, False, True)):
                    maxima = [10 * call + k + 1 for k in range(grid)]
                    maxima[perm[0]] += 1000 * (3 - call)  # each call's amax is distinct
                    res = run_call(ws, maxima, order, "last_reader", late=late, wg0_gives_up=gives_up)
                    assert set(res.values()) == {max(maxima)}
                    assert ws.gen == call + 1 and ws.count == 0


def test_last_reader_random_grids_and_sizes():
    """Random grid sizes from call to call (a smaller grid leaves higher
    slots untouched) with random late sets."""
    rng = random.Random(5)
    ws = Workspace()
    for call in range(200):
        grid = rng.randint(1, 12)
        maxima = [rng.randint(0, 10 ** 6) for _ in range(grid)]
        order = [0, *rng.sample(range(1, grid), grid - 1)]
        late = tuple(i for i in order[1:] if rng.random() < 0.3)
        res = run_call(ws, maxima, order, "last_reader", late=late, wg0_gives_up=rng.random() < 0.3)
        assert set(res.values()) == {max(maxima)}
        assert ws.gen == call + 1 and ws.count == 0

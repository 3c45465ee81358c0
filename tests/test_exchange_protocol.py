"""CPU model of the fused amax's grid exchange (host logic, no GPU).

The single-pass quantizer finds the tensor amax by an exchange through a
caller-owned workspace: every workgroup reads the generation word, posts
(generation, its maximum) in its arrival slot, workgroup 0 collects the
arrivals and posts (generation, amax) in every release slot; every wait is
bounded, and a workgroup whose wait expires computes the amax directly.

This model replays that protocol step by step under chosen interleavings of
workgroup starts, for three rules of when the generation word advances:

- "on_collect": workgroup 0 stores the generation once it has released the
  amax, whether or not its wait expired;
- "last_reader": every workgroup counts itself after posting its arrival
  (so after reading the generation) and the one that completes the count
  stores the generation;
- "count_on_expiry": the rule the kernel implements. When workgroup 0 has
  collected every arrival (each one carries the generation its workgroup
  read, so all have read it), it stores the generation as before. When its
  wait expired, it flags its release posts, and every workgroup of the call
  (workgroup 0, those that see a flagged release, those whose own wait
  expired) counts itself under a tag of the call's generation; the one that
  completes the count for that tag stores the generation. A workgroup whose
  own wait expired in a call where workgroup 0 did collect everything also
  counts, but under that call's tag, which no later call shares.

With "on_collect", a workgroup of call N that starts after workgroup 0 gave
up reads call N+1's generation and posts its stale maximum under it; call
N+1's workgroup 0 can then take that for a fresh arrival. The other two
rules never let a workgroup read a generation other than its own call's;
"count_on_expiry" needs no atomic operation when no wait expires.
"""
import itertools
import random

import pytest


FLAG = 1 << 31  # the sign bit of the released amax (an amax has none)


class Workspace:
    def __init__(self, slots=64):
        self.gen = 0
        self.count = 0
        self.tagged = (0, 0)  # count_on_expiry: (generation tag, count)
        self.arrive = [(0, 0)] * slots
        self.release = [(0, 0)] * slots


def run_call(ws, maxima, order, rule, late=(), wg0_gives_up=False, own_expiry=()):
    """One call on `ws`. `maxima[i]` is workgroup i's maximum. `order` is the
    order in which workgroups start (workgroup 0 first, as it is dispatched
    first). Workgroups in `late` start only after workgroup 0 has finished its
    collection (they were not resident). With `wg0_gives_up`, workgroup 0's
    wait expires before any late workgroup arrives. Workgroups in
    `own_expiry` give up waiting for their release before workgroup 0 posts
    it. Returns the amax every workgroup ends with."""
    grid = len(maxima)
    true_max = max(maxima)
    gen = {}
    rank = {}
    result = {}

    def count_expired(i):
        tag, n = ws.tagged
        n = n + 1 if tag == gen[i] else 1
        ws.tagged = (gen[i], n)
        if n == grid:
            ws.gen = gen[i]

    def start(i):
        gen[i] = ws.gen + 1  # read at the start of the kernel
        ws.arrive[i] = (gen[i], maxima[i])  # the post carries the value read
        if rule == "last_reader":
            rank[i] = ws.count
            ws.count += 1

    def take_release(i):
        if i in own_expiry:
            if rule == "count_on_expiry":
                count_expired(i)
            return true_max  # the direct amax
        g, v = ws.release[i]
        if g != gen[i]:
            if rule == "count_on_expiry":
                count_expired(i)
            return true_max  # its own wait expires
        if rule == "count_on_expiry" and v & FLAG:
            count_expired(i)
        return v & ~FLAG

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
    complete = all(g == gen[0] for g, _ in got) and not wg0_gives_up
    amax = max(v for _, v in got) if complete else true_max  # else the direct amax
    flag = FLAG if (rule == "count_on_expiry" and not complete) else 0
    for i in range(grid):
        ws.release[i] = (gen[0], amax | flag)
    if rule == "on_collect" or (rule == "count_on_expiry" and complete):
        ws.gen = gen[0]
    if rule == "count_on_expiry" and not complete:
        count_expired(0)
    result[0] = amax
    for i in early[1:]:
        result[i] = take_release(i)
    for i in late:
        start(i)
        result[i] = take_release(i)
    for i in order:
        finish(i)
    return result


def call_outputs(ws, maxima, order, rule, **kw):
    res = run_call(ws, maxima, order, rule, **kw)
    return set(res.values())


@pytest.mark.parametrize("rule,stale", [("on_collect", True), ("last_reader", False),
                                       ("count_on_expiry", False)])
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


@pytest.mark.parametrize("rule", ["last_reader", "count_on_expiry"])
def test_every_interleaving(rule):
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
                    res = run_call(ws, maxima, order, rule, late=late, wg0_gives_up=gives_up)
                    assert set(res.values()) == {max(maxima)}
                    assert ws.gen == call + 1 and ws.count == 0


def test_count_on_expiry_own_expiries():
    """Workgroups whose own wait expires, with workgroup 0 collecting
    everything (their counts stay under that call's tag and never complete)
    or not; every call still advances the generation exactly once."""
    grid = 4
    for gives_up in (False, True):
        for nexp in range(1, grid):
            for own in itertools.combinations(range(1, grid), nexp):
                ws = Workspace()
                for call in range(3):
                    maxima = [7 * call + k for k in range(grid)]
                    res = run_call(ws, maxima, list(range(grid)), "count_on_expiry", wg0_gives_up=gives_up,
                                   own_expiry=own)
                    assert set(res.values()) == {max(maxima)}
                    assert ws.gen == call + 1


@pytest.mark.parametrize("rule", ["last_reader", "count_on_expiry"])
def test_random_grids_and_sizes(rule):
    """Random grid sizes from call to call (a smaller grid leaves higher
    slots untouched) with random late sets."""
    rng = random.Random(5)
    ws = Workspace()
    for call in range(200):
        grid = rng.randint(1, 12)
        maxima = [rng.randint(0, 10 ** 6) for _ in range(grid)]
        order = [0, *rng.sample(range(1, grid), grid - 1)]
        late = tuple(i for i in order[1:] if rng.random() < 0.3)
        own = tuple(i for i in range(1, grid) if rng.random() < 0.1)
        res = run_call(ws, maxima, order, rule, late=late, wg0_gives_up=rng.random() < 0.3,
                       own_expiry=own if rule == "count_on_expiry" else ())
        assert set(res.values()) == {max(maxima)}
        assert ws.gen == call + 1 and ws.count == 0

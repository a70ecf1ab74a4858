"""CPU model of the batch-1 work-queue protocol of k_moe_layer (layer.hip):
where each workgroup claims units (at launch, in the router peel, at the top
of the unit loop, and one unit early inside runs of routed FC1 and FC2
units) and where it counts itself out on the exit counter (during its last
FC2 or combine unit once the claimed next index is past the end of the
queue, else after the loop).  Workgroups advance one protocol step at a time
in a random interleaving.  Checked: every unit of the queue is claimed
exactly once; no workgroup claims after it has counted itself out; every
workgroup counts out once; and the last count comes after the last claim,
so the queue reset it triggers cannot be undone by a later claim."""
import random

import pytest

# batch-1 unit counts at the K3 shape (router, routing, shared FC1, routed
# FC1, shared FC2, routed FC2, combine) and a small shape
K3 = dict(n_rt=224, n_ro=1, n_s1=384, n_f1=16 * 96, n_s2=224, n_f2=16 * 56, n_cb=28)
SMALL = dict(n_rt=8, n_ro=1, n_s1=4, n_f1=3 * 4, n_s2=2, n_f2=3 * 2, n_cb=2)


class Queue:
    def __init__(self, c, grid):
        self.c = c
        self.b_f1 = c["n_rt"] + c["n_ro"] + c["n_s1"]
        self.b_s2 = self.b_f1 + c["n_f1"]
        self.b_f2 = self.b_s2 + c["n_s2"]
        self.total = self.b_f2 + c["n_f2"] + c["n_cb"]
        self.grid = grid
        self.n_static = min(grid, self.b_f1)
        self.nq = 2 if grid >= 16 else 1
        self.heads = [0, 0]
        self.claimed = []
        self.events = []  # ("claim", w, unit) / ("count", w)

    def q(self, w):
        return (w >> 3) & 1 if self.nq > 1 else 0

    def claim(self, w):
        c = self.heads[self.q(w)]
        self.heads[self.q(w)] += 1
        unit = self.n_static + self.q(w) + self.nq * c
        self.claimed.append(unit)
        self.events.append(("claim", w, unit))
        return unit

    def kind(self, u):
        if u < self.c["n_rt"]:
            return "router"
        if u < self.b_f1:
            return "front"
        if u < self.b_s2:
            return "fc1"
        if u < self.b_f2:
            return "sh2"
        if u < self.b_f2 + self.c["n_f2"]:
            return "fc2"
        if u < self.total:
            return "combine"
        return "end"


def workgroup(Q, w):
    """One workgroup's protocol steps (a generator: each yield lets others run)."""
    exited = False

    def count_out_early(nxt):
        nonlocal exited
        if not exited and nxt >= Q.total:
            Q.events.append(("count", w))
            exited = True

    u = w if w < Q.n_static else -1
    if u < 0:
        u = Q.claim(w)
        yield
    if 0 <= u < Q.c["n_rt"]:  # the router peel
        nxt = Q.claim(w)
        yield
        u = nxt
    while True:
        if u >= Q.total:
            break
        nxt = Q.claim(w)  # top of the unit loop
        yield
        k = Q.kind(u)
        if k in ("fc1", "fc2"):  # a run: the unit before claims the one after next
            while True:
                if k == "fc2":
                    count_out_early(nxt)  # at the post, during the unit
                nxt2 = None
                if Q.kind(nxt) == k:
                    nxt2 = Q.claim(w)
                yield
                u = nxt
                if Q.kind(u) != k:
                    break
                nxt = nxt2
            continue
        if k == "combine":
            count_out_early(nxt)  # after the combine's polls
        yield
        u = nxt
    if not exited:
        Q.events.append(("count", w))


def run(c, grid, seed):
    Q = Queue(c, grid)
    gens = [workgroup(Q, w) for w in range(grid)]
    rng = random.Random(seed)
    live = list(range(grid))
    while live:
        i = rng.randrange(len(live))
        try:
            next(gens[live[i]])
        except StopIteration:
            live.pop(i)
    return Q


@pytest.mark.parametrize("shape,grid", [(SMALL, 1), (SMALL, 3), (SMALL, 16), (SMALL, 17), (SMALL, 40),
                                        (K3, 16), (K3, 100), (K3, 512)])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_batch1_queue_protocol(shape, grid, seed):
    Q = run(shape, grid, seed)
    real = sorted(u for u in Q.claimed if u < Q.total)
    assert real == list(range(Q.n_static, Q.total))  # every queue unit claimed exactly once
    counts = [i for i, e in enumerate(Q.events) if e[0] == "count"]
    assert len(counts) == grid and len({Q.events[i][1] for i in counts}) == grid
    last_claim = max(i for i, e in enumerate(Q.events) if e[0] == "claim")
    assert counts[-1] > last_claim  # the reset follows every claim
    counted = set()
    for e in Q.events:
        if e[0] == "count":
            counted.add(e[1])
        else:
            assert e[1] not in counted, "a workgroup claimed after counting itself out"
    # each workgroup's claims past the end: exactly one
    past = {}
    for e in Q.events:
        if e[0] == "claim" and e[2] >= Q.total:
            past[e[1]] = past.get(e[1], 0) + 1
    assert all(past.get(w, 0) == 1 for w in range(grid))

"""A step-by-step model of the persistent GEMM's tile claims (test infrastructure), used to check
that the protocol finishes every tile when some locality groups have no resident workgroup.

What it models, as the kernel does it:
- The tile list: expert waves, each with a Linear-1 run and a Linear-2 run over its m-blocks,
  in the Expert-Wave order or the interleaved order with lead D; runs are cut into units, and
  Linear-1 units and Linear-2 units are each dealt round-robin to the groups in list order,
  so each group's list is its units in list order.
- A workgroup takes records from its own group's list (fetch-and-add on the cursor), then
  from the other groups' lists in turn once its own is used up.
- Linear-1 completions are held in batches of two (lead >= 2) and released before the
  workgroup takes a Linear-2 tile, when its own list runs out, and at exit; a Linear-2 tile
  waits until its m-block has all its Linear-1 releases.
- Deferral (the kernel's kDeferTicks): a Linear-2 tile that has waited `defer_after` steps is
  set aside; the workgroup then takes only runnable records (the first unclaimed record of a
  group list, if it is a Linear-1 tile or a ready Linear-2 tile; compare-and-swap), releases
  each completion at once, and takes the deferred tile back when it is ready. A resumed tile
  is never deferred again. `defer_after=None` is the protocol without deferral.
"""
from __future__ import annotations

import random
from dataclasses import dataclass, field


@dataclass
class Tile:
    idx: int    # position in the whole list
    l2: bool
    mb: int


def build_lists(mblocks_per_wave, n1, n2, unit, order, lead, groups):
    """Returns (whole list, per-group lists, Linear-1 tiles per m-block)."""
    nw = len(mblocks_per_wave)
    first = [sum(mblocks_per_wave[:w]) for w in range(nw)]
    runs1, runs2 = [], []
    for w in range(nw):
        mbs = range(first[w], first[w] + mblocks_per_wave[w])
        r1 = [(False, m) for m in mbs for _ in range(n1)]
        r2 = [(True, m) for m in mbs for _ in range(n2)]
        runs1.append([r1[i:i + unit] for i in range(0, len(r1), unit)])
        runs2.append([r2[i:i + unit] for i in range(0, len(r2), unit)])
    units = []
    if order == "expert_wave":
        for w in range(nw):
            units += runs1[w] + runs2[w]
    else:
        for w in range(min(lead, nw)):
            units += runs1[w]
        for w in range(nw):
            a = runs1[w + lead] if w + lead < nw else []
            b = runs2[w]
            merged, ai = [], 0
            for bi, u in enumerate(b):
                merged.append(u)
                # Linear-1 unit v goes right after Linear-2 unit ceil((v + 1) b / a)
                while ai < len(a) and -(-(ai + 1) * len(b) // len(a)) <= bi + 1:
                    merged.append(a[ai])
                    ai += 1
            merged += a[ai:]
            units += merged
    tiles, per_group = [], [[] for _ in range(groups)]
    c1 = c2 = 0
    for u in units:
        l2 = u[0][0]
        g = (c2 if l2 else c1) % groups
        if l2:
            c2 += 1
        else:
            c1 += 1
        for (is2, m) in u:
            t = Tile(len(tiles), is2, m)
            tiles.append(t)
            per_group[g].append(t)
    return tiles, per_group, n1


@dataclass
class WG:
    group: int
    state: str = "claim"     # claim, run, wait, done
    tile: Tile | None = None
    left: int = 0
    waited: int = 0
    scan: int = 0            # groups whose lists it has used up
    pend: list = field(default_factory=list)
    deferred: Tile | None = None
    resumed: bool = False


def simulate(per_group, need, wgs_per_group, batch=2, defer_after=None, t1=5, t2=3, seed=0,
             max_steps=200000):
    """Runs the model; returns (finished, steps, starts: tile idx -> step, done: tile idx -> step)."""
    rng = random.Random(seed)
    G = len(per_group)
    cursor = [0] * G
    ready = {}
    wgs = [WG(g) for g in range(G) for _ in range(wgs_per_group[g])]
    total = sum(len(l) for l in per_group)
    finished, starts = {}, {}

    def release(w):
        for m in w.pend:
            ready[m] = ready.get(m, 0) + 1
        w.pend.clear()

    def is_ready(t):
        return ready.get(t.mb, 0) >= need

    def start(w, t, step):
        assert t.idx not in starts, "a tile ran twice"
        if t.l2:
            assert is_ready(t), "a Linear-2 tile started before its rows were ready"
        starts[t.idx] = step
        w.state, w.tile = "run", t
        w.left = max(1, (t2 if t.l2 else t1) + rng.randint(-1, 1))

    def help_claim(w):
        for h in range(G):
            g = (w.group + h) % G
            lst = per_group[g]
            if cursor[g] < len(lst):
                t = lst[cursor[g]]
                if not t.l2 or is_ready(t):
                    cursor[g] += 1  # the compare-and-swap succeeds (one actor at a time)
                    return t
        return None

    step = 0
    while len(finished) < total and step < max_steps:
        step += 1
        order = list(range(len(wgs)))
        rng.shuffle(order)
        for i in order:
            w = wgs[i]
            if w.state == "done":
                continue
            if w.state == "run":
                w.left -= 1
                if w.left == 0:
                    t = w.tile
                    finished[t.idx] = step
                    if not t.l2:
                        w.pend.append(t.mb)
                        if len(w.pend) >= batch or w.deferred is not None:
                            release(w)
                    w.state, w.tile = "claim", None
                continue
            if w.state == "wait":
                t = w.tile
                if is_ready(t):
                    start(w, t, step)
                    continue
                w.waited += 1
                if (defer_after is not None and w.deferred is None and not w.resumed
                        and w.waited > defer_after):
                    w.deferred, w.state, w.tile = t, "claim", None
                continue
            # claim
            if w.deferred is not None:
                if is_ready(w.deferred):
                    t, w.deferred = w.deferred, None
                    w.resumed = True
                    start(w, t, step)
                    continue
                t = help_claim(w)
                if t is not None:
                    w.resumed = False
                    start(w, t, step)
                continue
            t = None
            while w.scan < G:
                g = (w.group + w.scan) % G
                pos = cursor[g]
                cursor[g] += 1  # fetch-and-add
                if pos < len(per_group[g]):
                    t = per_group[g][pos]
                    break
                w.scan += 1
                if w.pend:
                    release(w)  # the flush when its own list runs out
            if t is None:
                release(w)
                w.state = "done"
                continue
            w.resumed = False
            if t.l2:
                release(w)
                w.state, w.tile, w.waited = "wait", t, 0
                if is_ready(t):
                    start(w, t, step)
            else:
                start(w, t, step)
    return len(finished) == total, step, starts, finished

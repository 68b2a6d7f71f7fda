"""The persistent GEMM's claim protocol on a model (tests/progress_model.py): with a locality
group, or all but one, without resident workgroups, deferring Linear-2 tiles that wait too long
and taking runnable records lets the resident workgroups finish every tile, in both orders and
at every lead; without the deferral the same runs stall. Every run also checks that no tile
runs twice and that no Linear-2 tile starts before its m-block's Linear-1 releases."""
import random

import pytest

from tests.progress_model import build_lists, simulate

GROUPS = 8


def configs():
    rng = random.Random(7)
    out = []
    for order, lead in [("expert_wave", 0), ("interleaved", 1), ("interleaved", 2), ("interleaved", 8)]:
        for k in range(3):
            mbw = [rng.randint(4, 10) for _ in range(8)]
            out.append((order, lead, mbw, k))
    return out


CONFIGS = configs()


def run(order, lead, mbw, wgs, defer_after, seed, batch=None):
    _, per_group, need = build_lists(mbw, n1=6, n2=4, unit=8, order=order, lead=lead, groups=GROUPS)
    if batch is None:
        batch = 2 if (order == "interleaved" and lead >= 2) else 1
    return simulate(per_group, need, wgs, batch=batch, defer_after=defer_after, seed=seed, max_steps=20000)


@pytest.mark.parametrize("order,lead,mbw,seed", CONFIGS)
def test_every_group_resident_finishes_with_and_without_deferral(order, lead, mbw, seed):
    for defer_after in (None, 30):
        ok, steps, _, _ = run(order, lead, mbw, [3] * GROUPS, defer_after, seed)
        assert ok, (order, lead, defer_after)


@pytest.mark.parametrize("order,lead,mbw,seed", CONFIGS)
@pytest.mark.parametrize("absent", [(0,), (3, 5), tuple(range(1, GROUPS))])
def test_absent_groups_finish_with_deferral(order, lead, mbw, seed, absent):
    wgs = [0 if g in absent else 3 for g in range(GROUPS)]
    ok, steps, starts, done = run(order, lead, mbw, wgs, 30, seed)
    assert ok, (order, lead, absent)


def test_without_deferral_an_absent_group_stalls_the_list():
    # in the Expert-Wave order and at leads 1 and 2, every resident workgroup ends up waiting on
    # a Linear-2 tile whose Linear-1 tiles sit unclaimed in group 0's list (with every
    # Linear-1 tile first, lead 8, enough of them run out of work and take that list over)
    for order, lead, mbw, seed in CONFIGS:
        if order == "interleaved" and lead >= 8:
            continue
        ok, _, _, _ = run(order, lead, mbw, [0] + [3] * (GROUPS - 1), None, seed)
        assert not ok, (order, lead)
        ok, _, _, _ = run(order, lead, mbw, [0] + [3] * (GROUPS - 1), 30, seed)
        assert ok, (order, lead)


def test_deferral_costs_little_with_every_group_resident():
    # with every group resident a long wait is rare (the groups progress alike); where one
    # happens, the workgroup runs other runnable tiles meanwhile, so the run is not longer
    for order, lead, mbw, seed in CONFIGS:
        a = run(order, lead, mbw, [3] * GROUPS, None, seed)
        b = run(order, lead, mbw, [3] * GROUPS, 30, seed)
        assert a[0] and b[0] and b[1] <= 1.1 * a[1], (order, lead, a[1], b[1])


def test_a_single_workgroup_finishes_everything():
    for order, lead, mbw, seed in CONFIGS[:4]:
        wgs = [0] * GROUPS
        wgs[5] = 1
        ok, _, _, _ = run(order, lead, mbw, wgs, 10, seed)
        assert ok

"""A host-side model of the work-claiming protocol of the persistent kernels
(mixed_hist_kernel, gumbel_mixed_kernel, pair_hist_kernel and the streamed
pair kernel): workgroups take select-unit groups, then dense pairs, from
workspace counters with fetch-and-add, and stop at the first claim past the
end; the finisher clears the counters for the next call.

The model runs the claim loops of every workgroup under random
interleavings, one atomic at a time, and checks that
  * every loop ends, within (items + workgroups) claims per counter,
    whatever the interleaving;
  * every group and every pair is taken exactly once;
  * the counters end at items + workgroups (each workgroup's last claim
    overshoots by one), so a counter that the finisher clears starts the
    next call at zero;
  * two calls in a row on the same counters, the second smaller, take every
    item again only when the counters were cleared in between; without the
    clear the second call takes nothing (wrong results, never a hang).
No claim loop waits on another workgroup, so none can hang: the only shared
state is a counter that only grows."""
import random

import pytest


class Counters:
    def __init__(self):
        self.c = {"groups": 0, "pairs": 0}

    def fetch_add(self, name):
        v = self.c[name]
        self.c[name] = v + 1
        return v


def workgroup(ctr, ngroups, npairs, taken_groups, taken_pairs, spread_units=None):
    """One workgroup's claim loops as a generator: each yield is one atomic.
    spread_units: the no-dense-pair mode, where single units are claimed."""
    if spread_units is not None:
        while True:
            u = ctr.fetch_add("groups")
            yield
            if u >= spread_units:
                return
            taken_groups.append(u)
    while True:
        g = ctr.fetch_add("groups")
        yield
        if g >= ngroups:
            break
        taken_groups.append(g)
    while True:
        t = ctr.fetch_add("pairs")
        yield
        if t >= npairs:
            return
        taken_pairs.append(t)


def run_call(ctr, nwg, ngroups, npairs, rng, spread=False):
    taken_g, taken_p = [], []
    gens = [workgroup(ctr, ngroups, npairs, taken_g, taken_p, spread_units=ngroups if spread else None)
            for _ in range(nwg)]
    live = list(range(nwg))
    steps = 0
    bound = 2 * (ngroups + npairs + 2 * nwg) + 10
    while live:
        i = rng.choice(live)
        try:
            next(gens[i])
        except StopIteration:
            live.remove(i)
        steps += 1
        assert steps <= bound, "a claim loop did not end"
    return taken_g, taken_p


@pytest.mark.parametrize("seed", range(20))
@pytest.mark.parametrize("nwg,ngroups,npairs", [(256, 272, 539), (8, 3, 0), (4, 0, 5), (256, 240, 0), (16, 1, 1)])
def test_claims_end_and_take_every_item_once(seed, nwg, ngroups, npairs):
    rng = random.Random(seed * 1009 + nwg)
    ctr = Counters()
    spread = npairs == 0
    g, p = run_call(ctr, nwg, ngroups, npairs, rng, spread=spread)
    assert sorted(g) == list(range(ngroups))
    assert sorted(p) == list(range(npairs))
    per_wg_overshoot = 1
    assert ctr.c["groups"] == ngroups + nwg * per_wg_overshoot
    if not spread:
        assert ctr.c["pairs"] == npairs + nwg * per_wg_overshoot


def test_headline_unit_count_two_calls():
    # 3840 single units (the headline's select units) over 3840 wavefronts'
    # worth of claimers, then a smaller call on the same counters after the
    # finisher's clear.
    rng = random.Random(7)
    ctr = Counters()
    g, _ = run_call(ctr, 1024, 3840, 0, rng, spread=True)
    assert sorted(g) == list(range(3840))
    ctr.c = {"groups": 0, "pairs": 0}   # the finisher's clear
    g, p = run_call(ctr, 256, 120, 77, rng)
    assert sorted(g) == list(range(120)) and sorted(p) == list(range(77))


def test_missing_clear_skips_work_but_ends():
    # Without the clear the second call's claims all start past its end: every
    # loop still ends at once, and nothing is taken (the outputs would be
    # wrong, which the GPU tests' second calls would show).
    rng = random.Random(11)
    ctr = Counters()
    run_call(ctr, 64, 50, 40, rng)
    g, p = run_call(ctr, 64, 30, 20, rng)
    assert g == [] and p == []

"""Host checks of the workload definitions (no GPU)."""

import json

from muon_newton_schulz_amd import workloads as W


def test_frozen_ragged_shapes_are_the_seeded_draw():
    # the committed JSON is what the seeded recipe draws; every ragged run
    # reads the JSON
    frozen = W.frozen_ragged_shapes()
    assert frozen == W.ragged_shapes()
    assert W.workload("ragged_500").shapes == frozen
    data = json.load(open(W.RAGGED_500_JSON))
    assert data["count"] == len(frozen) == 500
    assert data["params"] == sum(r * c for r, c in frozen)


def test_ragged_draw_properties():
    shapes = W.frozen_ragged_shapes()
    for i, (r, c) in enumerate(shapes):
        assert 512 <= min(r, c) and max(r, c) <= 8192
        kind = i % 3
        if kind == 0:
            assert r == c
        elif kind == 1:
            assert r >= c
        else:
            assert r <= c
        if i % 10 != 0:
            assert r % 64 == 0 and c % 64 == 0
    # every tenth matrix leaves the 64 grid (unless clamped at 8192 on both sides)
    off = [i for i, (r, c) in enumerate(shapes) if r % 64 or c % 64]
    assert all(i % 10 == 0 for i in off) and len(off) >= 45
    # the flat buffer reaches past 2^32 elements: offsets there are exercised
    wl = W.workload("ragged_500")
    assert wl.offsets()[-1] > 2 ** 32

"""Pins of the oracle's route map: a stable, token-major counting sort by expert.

Per-expert counts, prefix offsets and routed blocks: 'integrate EXL3 Trellis into the fused
W4A16 API' (sparkinfer PR #90), review of route_pack.py; route map materialised once:
'serve canonical Fruit QSRT atoms' (b12x PR #129), Hot path; stable token-major packing:
'Share trellis preparation across native and EXL3 containers' (b12x PR #433), review of
route_pack.py."""
import numpy as np
import pytest

import oracle_np as O


@pytest.mark.parametrize("R,E,block_m,p_bad", [(8, 8, 8, 0.0), (128, 96, 16, 0.0), (16384, 96, 64, 0.0),
                                               (5120, 128, 32, 0.0), (512, 256, 48, 0.05), (0, 4, 8, 0.0)])
def test_route_map_vs_numpy_stable_argsort(R, E, block_m, p_bad):
    rng = np.random.default_rng(R + E)
    ids = rng.integers(0, E, size=R).astype(np.int64)
    bad = rng.random(R) < p_bad
    ids[bad] = np.where(rng.random(bad.sum()) < 0.5, -1, E + 3)
    m = O.route_map(ids, E, block_m)
    valid = (ids >= 0) & (ids < E)
    assert m["invalid"] == int((~valid).sum())
    assert np.array_equal(m["counts"], np.bincount(ids[valid], minlength=E))
    assert m["offsets"][0] == 0 and np.array_equal(np.diff(m["offsets"]), m["counts"])
    order = np.argsort(np.where(valid, ids, E + 10), kind="stable")[: valid.sum()]
    assert np.array_equal(m["sorted_routes"], order)
    slot = np.full(R, -1)
    slot[order] = np.arange(order.size)
    assert np.array_equal(m["route_slot"], slot)
    # tiles: expert-major, block_m rows each, remainder last
    exp_tiles = []
    for e in range(E):
        for r0 in range(0, int(m["counts"][e]), block_m):
            exp_tiles.append((e, int(m["offsets"][e]) + r0, min(block_m, int(m["counts"][e]) - r0)))
    got = list(zip(m["tile_expert"].tolist(), m["tile_row0"].tolist(), m["tile_rows"].tolist()))
    assert got == exp_tiles


def test_route_map_hand_case():
    ids = np.array([[2, 0], [0, 1], [2, 1]], np.int64)    # routes 0..5 -> experts 2,0,0,1,2,1
    m = O.route_map(ids, 3, 8)
    assert list(m["counts"]) == [2, 2, 2]
    assert list(m["offsets"]) == [0, 2, 4, 6]
    assert list(m["sorted_routes"]) == [1, 2, 3, 5, 0, 4]
    assert list(m["route_slot"]) == [4, 0, 1, 2, 5, 3]
    assert m["num_tiles"] == 3

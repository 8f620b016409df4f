"""The stream-K split plan, checked on the CPU through the library's own
host-side copies of the functions its kernels use (split_lo, split_owner,
split_piece, split_tile_owners, piece_slot, cta_order).

A split launch shares the T*S (tile, stage) iterations of a GEMM out to G
workgroups in contiguous ranges; a tile cut by a range boundary is summed
from pieces that publish partial tiles into numbered slots, the last piece
to arrive adding them in piece order. A wrong owner, slot or piece count
would read another tile's partial sums or wait for a piece that never
comes, so the invariants are checked over many (T, S, G), including every
plan the cost models choose for the layer shapes used here.
"""

import itertools

import numpy as np
import pytest

from ternary_weight_quantization_amd import binding as B


def _check_plan(T, S, G):
    p = B.bitnet_debug_split_pieces(T, S, G)
    W = T * S
    # contiguous, equal-as-possible ranges: lo(v) = floor(v W / G)
    lo = [v * W // G for v in range(G + 1)]
    assert all(lo[v + 1] > lo[v] for v in range(G)), "a workgroup with an empty range"
    # every (tile, stage) covered exactly once, by the workgroup whose range holds it
    cover = np.zeros((T, S), dtype=np.int64)
    for v, t, s0, s1 in zip(p["v"], p["t"], p["s0"], p["s1"]):
        assert 0 <= t < T and 0 <= s0 < s1 <= S
        cover[t, s0:s1] += 1
        assert lo[v] <= t * S + s0 and t * S + s1 <= lo[v + 1]
    assert np.all(cover == 1)
    # each workgroup's pieces tile its range in order
    for v in range(G):
        sel = np.nonzero(p["v"] == v)[0]
        its = [(int(p["t"][i]) * S + int(p["s0"][i]), int(p["t"][i]) * S + int(p["s1"][i])) for i in sel]
        assert its[0][0] == lo[v] and its[-1][1] == lo[v + 1]
        assert all(a[1] == b[0] for a, b in zip(its, its[1:]))
    # per tile: pieces from consecutive workgroups va .. va + n - 1 in stage
    # order, the count and first owner the kernel derives agree with them
    split_slots = []
    for t in range(T):
        sel = np.nonzero(p["t"] == t)[0]
        vs = [int(p["v"][i]) for i in sel]
        assert vs == list(range(vs[0], vs[0] + len(vs)))
        assert all(int(p["va"][i]) == vs[0] and int(p["n"][i]) == len(vs) for i in sel)
        assert [int(p["s0"][i]) for i in sel][0] == 0 and [int(p["s1"][i]) for i in sel][-1] == S
        if len(vs) == 1:
            assert int(p["s0"][sel[0]]) == 0 and int(p["s1"][sel[0]]) == S  # whole: no partials
        else:
            split_slots += [int(p["slot"][i]) for i in sel]
    # the pieces of split tiles own distinct slots inside the reserved count
    nslots = B.bitnet_debug_partial_slots(T, G)
    assert nslots == min(2 * G, G + T - 1)
    assert len(split_slots) == len(set(split_slots))
    assert all(0 <= s < nslots for s in split_slots)
    return p


# (the launchers never plan more workgroups than iterations)
@pytest.mark.parametrize("T,S,G", [c for c in itertools.product([1, 2, 3, 7, 16, 80, 160], [1, 2, 5, 20, 54, 108],
                                                                [2, 3, 8, 17, 120, 136, 256]) if c[2] <= c[0] * c[1]])
def test_split_plan_invariants(T, S, G):
    _check_plan(T, S, G)


def test_split_plan_layer_shapes():
    """Plans at the layer shapes, as the cost models choose them or as the
    split knob forces them: the forward at 4096x6912->2560 (160 tiles of 54
    stages on 256 workgroups) and at 4096x2560->6912 (432 x 20), dX at
    4096x2560->6912 on its pair share (160 tiles of 108 stages on 120), the
    8-layer stack's down-projection forward (80 tiles of 54 stages on 256)
    and a ragged 270 x 64 over 136."""
    for T, S, G in ((160, 54, 256), (160, 108, 120), (80, 54, 256), (270, 64, 136), (432, 20, 256)):
        p = _check_plan(T, S, G)
        assert len(p["v"]) <= G + T - 1


def test_split_plan_random():
    rng = np.random.default_rng(7)
    for _ in range(300):
        T = int(rng.integers(1, 600))
        S = int(rng.integers(1, 130))
        G = int(rng.integers(2, 257))
        if G <= T * S:
            _check_plan(T, S, G)


def test_cta_order_is_xcd_contiguous_permutation():
    """Workgroup b runs on XCD b % 8; the virtual indices form a permutation
    in which each XCD owns one contiguous range, in XCD order."""
    for G in list(range(1, 40)) + [120, 136, 255, 256]:
        v = B.bitnet_debug_cta_order(G)
        assert sorted(v.tolist()) == list(range(G))
        starts = []
        for x in range(8):
            mine = sorted(int(v[b]) for b in range(x, G, 8))
            if mine:
                assert mine == list(range(mine[0], mine[0] + len(mine)))
                starts.append(mine[0])
        assert starts == sorted(starts)

"""Pins of the oracle's clustering-free raster blocks (VMoBA 1D-2D-3D block
partition; CPU only): a hand-derived labelling, the block shapes and sizes,
and the three partitions as special cases."""

import numpy as np

import oracle


def test_raster_worked_example():
    """Hand-derived: a 2 x 3 x 4 grid in 1 x 2 x 3 blocks has 2 x 2 x 2 = 8
    blocks; frame 0 rows 0-1 split at w = 3 into blocks 0 | 1, row 2 (an edge
    block of one row) into 2 | 3; frame 1 the same plus 4."""
    labels, C = oracle.raster_blocks(2, 3, 4, 1, 2, 3)
    assert C == 8
    want = [0, 0, 0, 1, 0, 0, 0, 1, 2, 2, 2, 3,
            4, 4, 4, 5, 4, 4, 4, 5, 6, 6, 6, 7]
    assert labels.tolist() == want


def test_raster_blocks_are_boxes(rng):
    for _ in range(10):
        F, H, W = (int(x) for x in rng.integers(1, 9, size=3))
        bt, bh, bw = int(rng.integers(1, F + 1)), int(rng.integers(1, H + 1)), int(rng.integers(1, W + 1))
        labels, C = oracle.raster_blocks(F, H, W, bt, bh, bw)
        assert C == -(-F // bt) * -(-H // bh) * -(-W // bw)
        assert sorted(set(labels.tolist())) == list(range(C))
        t, h, w = np.unravel_index(np.arange(F * H * W), (F, H, W))
        for c in range(C):
            m = labels == c
            # a block is the box of its extent: every (t, h, w) inside it
            box = (np.ptp(t[m]) + 1) * (np.ptp(h[m]) + 1) * (np.ptp(w[m]) + 1)
            assert box == m.sum() and np.ptp(t[m]) < bt and np.ptp(h[m]) < bh and np.ptp(w[m]) < bw
        # blocks numbered in raster order of their first token
        firsts = [int(np.nonzero(labels == c)[0][0]) for c in range(C)]
        bc = [(t[f] // bt, h[f] // bh, w[f] // bw) for f in firsts]
        assert bc == sorted(bc)


def test_raster_partitions_1d_2d_3d():
    F, H, W = 4, 6, 8
    one, C1 = oracle.raster_blocks(F, H, W, 2, H, W)        # 1D: chunks of frames
    assert C1 == 2 and np.array_equal(one, np.repeat([0, 1], 2 * H * W))
    two, C2 = oracle.raster_blocks(F, H, W, F, 3, 4)        # 2D: spatial tiles through all frames
    assert C2 == 4 and np.all(np.bincount(two) == F * 3 * 4)
    assert np.array_equal(two[:H * W], two[H * W:2 * H * W])  # every frame tiled alike
    three, C3 = oracle.raster_blocks(F, H, W, 2, 3, 4)      # 3D: cubes
    assert C3 == 8 and np.all(np.bincount(three) == 24)
    whole, C0 = oracle.raster_blocks(F, H, W, F, H, W)
    assert C0 == 1 and not whole.any()

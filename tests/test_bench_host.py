"""The bench's host-side accounting on hand-built walks (CPU only): the
realised acceptance counts a child tried after its earlier siblings'
rejection as one more test, and the acceptance by sibling rank divides each
rank's acceptances by the times it was tried."""

import types

import numpy as np

import bench


def _w():
    # root 0 with children 1, 2, 3; node 1 with child 4; V = 10
    parent = np.array([[-1, 0, 0, 0, 1]], np.int32)
    return types.SimpleNamespace(parent=parent, B=1, N=5, V=10, Hkv=1, D=8)


def test_realised_and_rank_acceptance_by_hand():
    w = _w()
    # offset 0: child 1 accepted, then child 4 accepted (a leaf): 2 tests, 2 accepted
    # offset 1: children 1, 2 rejected, 3 accepted: 3 tests, 1 accepted
    # offset 2: all three children rejected: 3 tests, 0 accepted
    paths = np.full((3, 1, 5), -1, np.int32)
    paths[0, 0, :3] = [0, 1, 4]
    paths[1, 0, :2] = [0, 3]
    paths[2, 0, :1] = [0]
    naccs = np.array([[2], [1], [0]], np.int32)
    st = bench.acceptance_stats(w, paths, naccs)
    assert st["realised_acceptance"] == round(3 / 8, 4)
    assert st["mean_emitted_per_step"] == round((3 + 2 + 1) / 3, 3)
    rates, tried = bench.rank_acceptance(w, paths, naccs, K=3)
    # rank 1 tried 4 times (root x3, node 1 x1), accepted twice; rank 2 tried
    # twice, never accepted; rank 3 tried twice, accepted once
    assert list(tried) == [4, 2, 2]
    assert rates == [0.5, 0.0, 0.5]

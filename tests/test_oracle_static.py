"""Pins of the oracle's static block mask (local boxes + anchor slabs).

The rule follows the Sol-Attn article (bjdmk.com.cn), section 3.2: a pair is
kept when both tokens share a local window or when either is an anchor; the
oracle applies it to block coordinates.  The pins below do not restate that
predicate: they check counts that factor over the grid dimensions, the
equivalence-class structure of the local part, the anchor counts, symmetry,
and, on a one-dimensional grid of one-token blocks, the article's token-level
rule through an inclusion-exclusion count worked out per window.
"""
import itertools
import math

import numpy as np
import pytest

import oracle


def _grid_blocks(grid, block):
    return [math.ceil(g / b) for g, b in zip(grid, block)]


def _kept(grid, block, local, anchor_t):
    mask, counts = oracle.static_mask(grid, block, local, anchor_t)
    N = oracle.num_blocks(grid, block)
    keep = oracle.mask_to_bool(mask[0, 0], N)
    return keep, counts[0, 0]


CASES = [((8, 16, 16), (4, 8, 8)), ((31, 22, 40), (4, 8, 8)), ((9, 17, 23), (4, 8, 8)), ((12, 16, 24), (2, 2, 2)),
         ((5, 9, 7), (4, 8, 8))]


@pytest.mark.parametrize("grid,block", CASES)
def test_identity_and_dense(grid, block):
    keep, _ = _kept(grid, block, (1, 1, 1), 0)
    assert np.array_equal(keep, np.eye(keep.shape[0], dtype=bool))
    n = _grid_blocks(grid, block)
    keep, counts = _kept(grid, block, tuple(n), 0)
    assert keep.all() and (counts == keep.shape[0]).all()


@pytest.mark.parametrize("grid,block", CASES)
@pytest.mark.parametrize("local", [(1, 1, 2), (2, 1, 1), (2, 2, 2), (3, 2, 5), (1, 3, 1)])
def test_local_boxes_factor_over_dimensions(grid, block, local):
    keep, counts = _kept(grid, block, local, 0)
    n = _grid_blocks(grid, block)
    # box sizes along each dimension: full boxes of l, a ragged last one
    sizes = [[min(l, nd - s) for s in range(0, nd, l)] for nd, l in zip(n, local)]
    # kept pairs = sum over boxes of volume^2, which factors over the dimensions
    assert keep.sum() == math.prod(sum(x * x for x in sz) for sz in sizes)
    assert counts.sum() == keep.sum()
    # an equivalence relation whose classes are the boxes
    assert keep.diagonal().all() and np.array_equal(keep, keep.T)
    k = keep.astype(np.int64)
    assert np.array_equal((k @ k) > 0, keep)
    assert len({r.tobytes() for r in keep}) == math.prod(len(sz) for sz in sizes)


@pytest.mark.parametrize("grid,block", CASES)
@pytest.mark.parametrize("anchor_t", [1, 2, 3])
def test_anchor_slabs(grid, block, anchor_t):
    keep, counts = _kept(grid, block, (1, 1, 1), anchor_t)
    nT, nH, nW = _grid_blocks(grid, block)
    N = nT * nH * nW
    n_anchor = math.ceil(nT / anchor_t) * nH * nW
    anchor_rows = (counts == N)
    assert anchor_rows.sum() == n_anchor
    assert (counts[~anchor_rows] == 1 + n_anchor).all()
    assert np.array_equal(keep, keep.T)


@pytest.mark.parametrize("T,window,stride", [(10, 4, 4), (16, 4, 3), (23, 5, 7), (64, 8, 16), (7, 7, 2), (9, 1, 1)])
def test_one_dimensional_token_rule(T, window, stride):
    """Grid (T, 1, 1) in one-token blocks: the article's token mask, counted per window."""
    keep, _ = _kept((T, 1, 1), (1, 1, 1), (window, 1, 1), stride)
    anchors = [q for q in range(T) if q % stride == 0]
    A = len(anchors)
    total = 0
    for s in range(0, T, window):
        w = min(window, T - s)
        a_in = sum(1 for q in anchors if s <= q < s + w)
        total += w * w - (2 * a_in * w - a_in * a_in)  # same-window pairs with no anchor in them
    total += 2 * A * T - A * A                          # pairs with an anchor on either side
    assert keep.sum() == total
    for q, k in itertools.product(range(T), repeat=2):  # and every anchor row / column is full
        if q % stride == 0 or k % stride == 0:
            assert keep[q, k]


def test_batch_heads_broadcast():
    mask, counts = oracle.static_mask((9, 17, 23), (4, 8, 8), (2, 1, 2), 2, B=2, heads=3)
    assert mask.shape[:2] == (2, 3) and counts.shape == (2, 3, 27)
    assert (mask == mask[0, 0]).all() and (counts == counts[0, 0]).all()

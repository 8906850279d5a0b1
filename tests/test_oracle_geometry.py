"""Pins for the oracle's 3D block organisation (CPU only).

Pinned to: the VSA guide's printed routing example (section 3), the Sol-Attn
article's 393,216-token count (section 2.1), closed forms of the block
product, and a brute-force token enumeration written here.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_vsa_printed_example():
    ex = _load("vsa_routing_example.json")
    grid, block = tuple(ex["dit_seq_shape"]), tuple(ex["block_size"])
    assert math.prod(grid) == ex["seq_len"]
    assert math.prod(block) == ex["tokens_per_block"]
    n = oracle.num_blocks(grid, block)
    assert n == ex["num_blocks"]
    assert [math.ceil(g / b) for g, b in zip(grid, block)] == ex["num_blocks_factors"]
    # keep ratio of the printed top-k, rounded as printed (one decimal, percent)
    assert round(100.0 * ex["topk"] / n, 1) == ex["keep_ratio_percent"]


def test_long_video_token_count():
    ex = _load("long_video_tokens.json")
    assert math.prod(ex["grid"]) == ex["tokens"]
    assert oracle.num_blocks(tuple(ex["grid"]), tuple(ex["h3_block_size"])) == 24 * 16 * 16


@pytest.mark.parametrize("grid,block,n", [
    ((21, 45, 80), (4, 8, 8), 6 * 6 * 10),
    ((8, 16, 16), (4, 8, 8), 8),          # 2048 tokens / 256 per block
    ((5, 9, 7), (4, 8, 8), 4),
    ((1, 1, 1), (4, 8, 8), 1),
    ((4, 8, 8), (4, 8, 8), 1),
    ((96, 64, 64), (4, 4, 4), 6144),
])
def test_num_blocks_closed_form(grid, block, n):
    assert oracle.num_blocks(grid, block) == n


def test_invalid_geometry():
    assert oracle.num_blocks((0, 8, 8), (4, 8, 8)) == -1
    assert oracle.num_blocks((8, 8, 8), (4, 0, 8)) == -1


def _brute_blocks(grid, block):
    """Enumerate tokens and assign each to its block by integer division."""
    T, H, W = grid
    bt, bh, bw = block
    nH, nW = -(-H // bh), -(-W // bw)
    t, y, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    blk = ((t // bt) * nH + (y // bh)) * nW + (x // bw)
    return blk.reshape(-1)


@pytest.mark.parametrize("grid,block,hist", [
    ((31, 22, 40), (4, 8, 8), {256: 70, 192: 45, 144: 5}),
    ((21, 45, 80), (4, 8, 8), {256: 250, 160: 50, 64: 50, 40: 10}),
    ((8, 16, 16), (4, 8, 8), {256: 8}),
    ((5, 9, 7), (4, 8, 8), {224: 1, 28: 1, 56: 1, 7: 1}),
])
def test_block_table_and_token_map(grid, block, hist):
    tab = oracle.block_table(grid, block)
    counts = tab[:, 6]
    got = {int(c): int(n) for c, n in zip(*np.unique(counts, return_counts=True))}
    assert got == hist
    L = math.prod(grid)
    assert counts.sum() == L
    tb = oracle.token_block(grid, block)
    assert (tb >= 0).all()
    assert np.array_equal(tb, _brute_blocks(grid, block))
    assert np.array_equal(np.bincount(tb, minlength=len(tab)), counts)
    # every block's box lies inside the grid and its count is its volume
    T, H, W = grid
    assert (tab[:, 0] + tab[:, 3] <= T).all() and (tab[:, 1] + tab[:, 4] <= H).all()
    assert (tab[:, 2] + tab[:, 5] <= W).all()
    assert np.array_equal(tab[:, 3] * tab[:, 4] * tab[:, 5], counts)


def test_long_video_blocks_uniform():
    tab = oracle.block_table((96, 64, 64), (4, 4, 4))
    assert (tab[:, 6] == 64).all() and len(tab) == 6144

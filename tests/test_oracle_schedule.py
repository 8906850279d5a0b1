"""Pins of the oracle's work items and LPT queues (the one-GPU share of the
FVAttn abstract's runtime load balancing).

Checked against things other than the rule's own text: item costs against a
count over the token-level block map (and, for one-block items, against the
C oracle's real-pair count); the items partition the block grid; a
hand-worked head of four one-token blocks (cost ties go to the lower item);
the closed form for at most one head per queue; Graham's bound for any list
schedule; and, on three queues, the LPT bound 4/3 - 1/9 against the optimum
found by brute force."""
import itertools

import numpy as np
import pytest

import oracle


def _random_mask(rng, B, heads, N, density):
    keep = rng.random((B * heads, N, N)) < density
    keep[:, np.arange(N), np.arange(N)] = True  # every row keeps its own block
    words = (N + 31) // 32
    padded = np.zeros((B * heads, N, words * 32), dtype=np.uint64)
    padded[..., :N] = keep
    m = (padded.reshape(B * heads, N, words, 32) << np.arange(32, dtype=np.uint64)).sum(-1).astype(np.uint32)
    return m.reshape(B, heads, N, words)


@pytest.mark.parametrize("grid,block,group", [((9, 17, 23), (4, 8, 8), (1, 1, 1)),
                                               ((10, 9, 13), (4, 4, 4), (2, 1, 2)),
                                               ((5, 12, 19), (2, 8, 8), (1, 1, 2)),
                                               ((7, 6, 5), (2, 2, 2), (2, 1, 2))])
def test_costs_from_token_map(grid, block, group):
    rng = np.random.default_rng(3)
    B, heads = 2, 3
    N = oracle.num_blocks(grid, block)
    mask = _random_mask(rng, B, heads, N, 0.3)
    cost, order, qoff = oracle.lpt_schedule(grid, block, mask, B, heads, group=group)
    items = oracle.work_items(grid, block, group)
    # the items partition the blocks
    flat = sorted(n for it in items for n in it)
    assert flat == list(range(N))
    nT, nH, nW = (-(-d // b) for d, b in zip(grid, block))
    assert len(items) == -(-nT // group[0]) * -(-nH // group[1]) * -(-nW // group[2])
    # cost = query tokens of the members x key tokens of the union, counted on the token map
    tb = oracle.token_block(grid, block)
    keep = oracle.mask_to_bool(mask, N).reshape(B * heads, N, N)
    G = len(items)
    for h in range(B * heads):
        for g, members in enumerate(items):
            inq = np.isin(tb, members)
            union = keep[h, members].any(0)
            assert cost[h * G + g] == int(inq.sum()) * int(union[tb].sum())
    if group == (1, 1, 1):
        assert int(cost.sum()) == oracle.real_pairs(grid, block, mask)
    # order is a permutation; queues cover it
    assert sorted(order.tolist()) == list(range(B * heads * G))
    assert qoff[0] == 0 and qoff[-1] == B * heads * G and (np.diff(qoff) >= 0).all()


def test_hand_worked_head():
    # four one-token blocks in a row; block i keeps {0}, {0,1,2}, {0,1}, {0,1,2}
    grid, block = (1, 1, 4), (1, 1, 1)
    rows = [[0], [0, 1, 2], [0, 1], [0, 1, 2]]
    mask = np.zeros((1, 1, 4, 1), dtype=np.uint32)
    for i, js in enumerate(rows):
        for j in js:
            mask[0, 0, i, 0] |= np.uint32(1 << j)
    cost, order, qoff = oracle.lpt_schedule(grid, block, mask, 1, 1, group=(1, 1, 1))
    assert cost.tolist() == [1, 3, 2, 3]
    assert order.tolist() == [1, 3, 2, 0]  # equal costs 3: item 1 before item 3
    assert qoff.tolist() == [0] + [4] * 8
    cost, order, qoff = oracle.lpt_schedule(grid, block, mask, 1, 1, group=(1, 1, 1), naive=True)
    assert order.tolist() == [0, 1, 2, 3] and qoff.tolist() == [0] + [4] * 8
    # one item of all four blocks: 4 query tokens x 3 key tokens (blocks 0, 1, 2)
    cost, order, qoff = oracle.lpt_schedule(grid, block, mask, 1, 1, group=(1, 1, 4))
    assert cost.tolist() == [12]


def _head_loads(cost, order, qoff, G, queues):
    loads = []
    for x in range(queues):
        ids = order[qoff[x]:qoff[x + 1]]
        loads.append(int(cost[ids].sum()))
        heads = sorted(set((ids // G).tolist()))
        for h in heads:  # a head's items stay together on one queue
            assert ((order[qoff[x]:qoff[x + 1]] // G) == h).sum() == G
    return loads


def test_one_head_per_queue_closed_form():
    rng = np.random.default_rng(11)
    grid, block = (8, 16, 16), (4, 8, 8)
    N = oracle.num_blocks(grid, block)
    heads = 6
    mask = _random_mask(rng, 1, heads, N, 0.5)
    cost, order, qoff = oracle.lpt_schedule(grid, block, mask, 1, heads)
    G = N
    hc = cost.reshape(heads, G).sum(1)
    rank = sorted(range(heads), key=lambda h: (-hc[h], h))
    # r-th heaviest head alone on queue r; queues past the heads are empty
    assert qoff.tolist() == [min(x, heads) * G for x in range(9)]
    for r, h in enumerate(rank):
        assert set((order[qoff[r]:qoff[r + 1]] // G).tolist()) == {h}


@pytest.mark.parametrize("heads,queues,seed", [(9, 3, 0), (8, 3, 1), (7, 3, 2), (20, 8, 3)])
def test_lpt_bounds(heads, queues, seed):
    rng = np.random.default_rng(seed)
    grid, block = (4, 16, 24), (4, 8, 8)
    N = oracle.num_blocks(grid, block)
    # heads of very different densities
    mask = np.concatenate([_random_mask(rng, 1, 1, N, d) for d in rng.uniform(0.05, 0.9, heads)], axis=1)
    cost, order, qoff = oracle.lpt_schedule(grid, block, mask, 1, heads, queues=queues)
    G = N
    loads = _head_loads(cost, order, qoff, G, queues)
    hc = cost.reshape(heads, G).sum(1)
    assert sum(loads) == int(hc.sum())
    # Graham: any list schedule ends by total/m + (1 - 1/m) * largest job
    assert max(loads) <= hc.sum() / queues + (1 - 1 / queues) * hc.max() + 1e-9
    if queues ** heads <= 3 ** 9:
        best = min(max(np.bincount(np.array(a), weights=hc, minlength=queues))
                   for a in itertools.product(range(queues), repeat=heads))
        assert max(loads) <= (4 / 3 - 1 / (3 * queues)) * best + 1e-9

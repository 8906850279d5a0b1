"""The attention plan's work items and queues, read back through the C ABI
(fva_attn_schedule), bit-exact against the oracle's LPT schedule (MI355X).

Seeded random masks (every row keeps its own block, many equal costs so the
tie rules are exercised) on one-block items with ragged edges, 2x1x2 groups
of 64-token blocks, 1x1x2 groups of 128-token blocks, more heads than
queues, B = 2, the naive order and heads placed by the caller."""
import zlib

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
import adaptive_block_sparse_tile_amd as fva  # noqa: E402

pytestmark = pytest.mark.gpu


def _random_mask(rng, B, heads, N, density):
    keep = rng.random((B * heads, N, N)) < density
    keep[:, np.arange(N), np.arange(N)] = True
    words = (N + 31) // 32
    padded = np.zeros((B * heads, N, words * 32), dtype=np.uint64)
    padded[..., :N] = keep
    m = (padded.reshape(B * heads, N, words, 32) << np.arange(32, dtype=np.uint64)).sum(-1).astype(np.uint32)
    return m.reshape(B, heads, N, words)


CASES = [
    # name, B, heads, D, grid, block, density
    ("wan14b_shape", 1, 40, 128, (31, 22, 40), (4, 8, 8), 0.5),
    ("ragged_b2", 2, 5, 64, (9, 17, 23), (4, 8, 8), 0.3),
    ("grouped64", 1, 10, 128, (16, 30, 36), (4, 4, 4), 0.15),
    ("grouped128", 1, 12, 64, (6, 16, 40), (2, 8, 8), 0.4),
    ("grouped64_ragged", 2, 3, 64, (7, 6, 5), (2, 2, 2), 0.5),
]


def _plan(B, heads, D, grid, block, mask, sched="lpt", head_xcd=None):
    L = grid[0] * grid[1] * grid[2]
    kv = torch.zeros((B, L, heads, D), dtype=torch.bfloat16, device="cuda")
    mask_d = torch.from_numpy(mask.view(np.int32)).cuda()
    ws = fva.attn_plan(kv, kv, grid, block, mask_d, sched=sched, head_xcd=head_xcd)
    order, qoff, cost = fva.attn_schedule((B, L, heads, D), grid, block, ws)
    torch.cuda.synchronize()
    return (order.cpu().numpy().astype(np.int64), qoff.cpu().numpy().astype(np.int64),
            cost.cpu().numpy().view(np.uint32).astype(np.int64))


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_schedule_matches_oracle(case):
    name, B, heads, D, grid, block, density = case
    print("\n[%s] B=%d heads=%d D=%d grid=%s block=%s" % (name, B, heads, D, grid, block), flush=True)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    N = oracle.num_blocks(grid, block)
    mask = _random_mask(rng, B, heads, N, density)
    L = grid[0] * grid[1] * grid[2]
    n_items = fva.attn_items((B, L, heads, D), grid, block)
    cost_o, order_o, qoff_o = oracle.lpt_schedule(grid, block, mask, B, heads)
    assert n_items == cost_o.size
    order, qoff, cost = _plan(B, heads, D, grid, block, mask)
    assert np.array_equal(cost, cost_o)
    assert np.array_equal(qoff, qoff_o)
    assert np.array_equal(order, order_o)
    # naive: item order on queue 0
    order, qoff, cost = _plan(B, heads, D, grid, block, mask, sched="naive")
    c2, o2, q2 = oracle.lpt_schedule(grid, block, mask, B, heads, naive=True)
    assert np.array_equal(cost, c2) and np.array_equal(order, o2) and np.array_equal(qoff, q2)


def test_schedule_heads_placed_by_caller():
    B, heads, D, grid, block = 1, 12, 128, (9, 17, 23), (4, 8, 8)
    rng = np.random.default_rng(7)
    N = oracle.num_blocks(grid, block)
    mask = _random_mask(rng, B, heads, N, 0.4)
    hx = rng.integers(0, 8, size=B * heads).astype(np.int32)
    hx[:3] = 5  # several heads on one queue, some queues empty
    order, qoff, cost = _plan(B, heads, D, grid, block, mask, sched="xcd",
                              head_xcd=torch.from_numpy(hx).cuda())
    c2, o2, q2 = oracle.lpt_schedule(grid, block, mask, B, heads, head_xcd=hx)
    assert np.array_equal(cost, c2) and np.array_equal(order, o2) and np.array_equal(qoff, q2)

"""Pins of the oracle's slack-aware sparse augmentation (one-GPU form).

Costs are the attention kernel's time model: a query block of c_i tokens
takes ceil(ceil(c_i/32)/2) steps per 64-key chunk on its busiest SIMD, a key
block of c_j tokens is ceil(c_j/64) chunks (written out here as a table).

Checked against things other than the rule's own text: an independent stable
argsort for each row's candidate order; the partition of head costs over the
XCDs; that nothing is added to the critical XCD and no XCD passes the
makespan; that every XCD either exhausts its offers or is left with less slack
than the largest possible offer; superset of the routed mask; special cases
with no slack (equal heads, dense rows, zero rounds)."""
import numpy as np
import pytest

import fvgen
import oracle


def _routed(wl, q=None, k=None):
    if q is None:
        q, k, _ = fvgen.generate_qkv(wl)
    S = oracle.scores(oracle.pool(q, wl.grid, wl.block), oracle.pool(k, wl.grid, wl.block))
    mask, cnt, flags, st = oracle.route(q, k, wl.grid, wl.block, wl.top_p, wl.k_floor)
    return S, mask


def _wl(name, heads, grid, block, top_p, k_floor, D=64):
    taus = tuple(np.linspace(0.4, 5.0, heads))
    return fvgen.Workload(name, 61, heads, D, grid, block, 8, "list", taus, top_p, k_floor)


CASES = [_wl("h12", 12, (9, 17, 23), (4, 8, 8), 0.8, 2), _wl("h11_small", 11, (6, 8, 8), (2, 4, 4), 0.7, 3),
         fvgen.WORKLOADS["wan14b"]]


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_invariants(wl):
    S, mask = _routed(wl)
    rounds = 4
    mo, co, hx, load, added, flags = oracle.sasa(S, mask, wl.grid, wl.block, rounds)
    B, H, N, _ = S.shape
    keep = oracle.mask_to_bool(mask, N).reshape(B * H, N, N)
    out = oracle.mask_to_bool(mo, N).reshape(B * H, N, N)
    assert (out >= keep).all()
    assert np.array_equal(co.reshape(-1, N), out.sum(-1))
    c = oracle.block_table(wl.grid, wl.block)[:, 6].astype(np.int64)
    # the kernel's time per (query block, key block): steps per chunk on the busiest SIMD times key chunks
    cost = np.array([[(((ci + 31) // 32 + 1) // 2) * ((cj + 63) // 64) for cj in c] for ci in c], dtype=np.int64)
    # head costs partition over the XCDs
    head_cost = (keep * cost[None]).sum((1, 2))
    for x in range(8):
        assert load[x] == head_cost[hx == x].sum()
    M = load.max()
    assert added[np.argmax(load)] == 0
    assert ((load + added) <= M).all()
    # the added cost is what the new bits cost, per XCD
    new = out & ~keep
    per_head = (new * cost[None]).sum((1, 2))
    for x in range(8):
        assert added[x] == per_head[hx == x].sum()
    # per row: the added blocks are the first ones of the dropped order (stable argsort of -score)
    for h in range(B * H):
        for i in range(N):
            a = int(new[h, i].sum())
            if a == 0:
                continue
            key = np.where(keep[h, i], np.inf, -S.reshape(B * H, N, N)[h, i])
            order = np.argsort(key, kind="stable")
            assert set(order[:a].tolist()) == set(np.nonzero(new[h, i])[0].tolist())
            assert a <= rounds
    # every XCD either ran out of offers or kept less slack than the largest offer
    biggest = int(cost.max())
    for x in range(8):
        rows_x = [h for h in range(B * H) if hx[h] == x]
        dropped = sum(int(min(rounds, (~keep[h]).sum(-1)[i])) for h in rows_x for i in range(N))
        taken = int(sum(new[h].sum() for h in rows_x))
        if taken < dropped:
            assert M - (load[x] + added[x]) < biggest


def test_no_slack_equal_heads():
    wl = _wl("eq", 1, (9, 17, 23), (4, 8, 8), 0.8, 2)
    q, k, _ = fvgen.generate_qkv(wl)
    q8, k8 = np.repeat(q, 8, axis=2), np.repeat(k, 8, axis=2)
    wl8 = _wl("eq8", 8, (9, 17, 23), (4, 8, 8), 0.8, 2)
    S, mask = _routed(wl8, q8, k8)
    mo, co, hx, load, added, flags = oracle.sasa(S, mask, wl8.grid, wl8.block, 4)
    assert sorted(hx.tolist()) == list(range(8))
    assert (load == load[0]).all() and (added == 0).all() and np.array_equal(mo, mask)


def test_dense_rows_and_zero_rounds():
    wl = _wl("dense", 5, (9, 17, 23), (4, 8, 8), 1.0, 1)
    S, mask = _routed(wl)
    mo, _, _, _, added, _ = oracle.sasa(S, mask, wl.grid, wl.block, 4)
    assert np.array_equal(mo, mask) and (added == 0).all()
    wl = CASES[0]
    S, mask = _routed(wl)
    mo, _, _, _, added, _ = oracle.sasa(S, mask, wl.grid, wl.block, 0)
    assert np.array_equal(mo, mask) and (added == 0).all()


def test_time_model_rates():
    """Steps per chunk on the busiest SIMD for the kernel's wavefront layout
    (8 wavefronts, two per SIMD; tiles of 32 rows; blocks of at most 6 tiles
    split key halves): full 256-token blocks 4, the Wan layer's ragged 192- and
    144-token blocks 3 each (the pair count would charge 144 only 0.5625 of a
    full block), 128 tokens 2, 64 tokens 1; a 144-token key block is 3 chunks,
    as many as a 192-token one."""
    assert oracle.sasa_row_rate([256, 224, 192, 160, 144, 128, 96, 64, 40, 32]).tolist() == \
        [4, 4, 3, 3, 3, 2, 2, 1, 1, 1]
    assert oracle.sasa_key_chunks([256, 192, 144, 64, 40]).tolist() == [4, 3, 3, 1, 1]


W8 = [1000, 1040, 960, 1000, 1090, 920, 1010, 980]


@pytest.mark.parametrize("wl", CASES[:2], ids=lambda w: w.name)
def test_weighted_xcds(wl):
    """XCDs of unequal speed w_x: every head went to the XCD where it finished
    first at the time (replayed here), nothing is added to the critical XCD
    (largest load/w), no XCD passes the critical time ((load + added) / w <=
    load_m / w_m), and an XCD that did not run out of offers has less weighted
    slack left than the largest offer; equal weights give the unweighted result."""
    S, mask = _routed(wl)
    rounds = 4
    B, H, N, _ = S.shape
    mo, co, hx, load, added, flags = oracle.sasa(S, mask, wl.grid, wl.block, rounds, xcd_weight=W8)
    keep = oracle.mask_to_bool(mask, N).reshape(B * H, N, N)
    c = oracle.block_table(wl.grid, wl.block)[:, 6].astype(np.int64)
    cost = np.array([[(((ci + 31) // 32 + 1) // 2) * ((cj + 63) // 64) for cj in c] for ci in c], dtype=np.int64)
    head_cost = (keep * cost[None]).sum((1, 2))
    ld = [0] * 8
    for h in sorted(range(B * H), key=lambda h: (-int(head_cost[h]), h)):
        finish = [(ld[x] + int(head_cost[h])) / W8[x] for x in range(8)]
        best = min(range(8), key=lambda x: (finish[x], x))
        assert hx[h] == best
        ld[best] += int(head_cost[h])
    assert ld == load.tolist()
    m = max(range(8), key=lambda x: (load[x] / W8[x], -x))
    assert added[m] == 0
    for x in range(8):
        assert (load[x] + added[x]) * W8[m] <= load[m] * W8[x]
    out = oracle.mask_to_bool(mo, N).reshape(B * H, N, N)
    new = out & ~keep
    biggest = int(cost.max())
    for x in range(8):
        rows_x = [h for h in range(B * H) if hx[h] == x]
        dropped = sum(int(min(rounds, (~keep[h]).sum(-1)[i])) for h in rows_x for i in range(N))
        taken = int(sum(new[h].sum() for h in rows_x))
        if taken < dropped:
            assert load[m] * W8[x] // W8[m] - (load[x] + added[x]) < biggest
    # a different placement than the unweighted one, and equal weights reproduce it
    plain = oracle.sasa(S, mask, wl.grid, wl.block, rounds)
    same = oracle.sasa(S, mask, wl.grid, wl.block, rounds, xcd_weight=[7] * 8)
    for a, b in zip(plain, same):
        assert np.array_equal(a, b)

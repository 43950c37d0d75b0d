"""CPU tests of how a bf16 forward step splits the key ranges of its query blocks (the host
planner behind ra_fwd_step_plan, and the item -> (block, part) mapping the kernel runs).

What must hold for correctness: every query block is covered exactly once, whole or as its two
halves.  What makes it fast: items go out in nonincreasing work, and the split is taken only
where the grid leaves compute units idle (at most one item per unit), never to rebalance a
grid that fills the chip.  Tile counts are recomputed here from the oracle's token
positions, not from the library's key-limit formula."""
import ctypes

import numpy as np
import pytest
import torch

import ring_attention_long_amd as ra
from oracle import shard_tokens
from ring_attention_long_amd import _lib

FIXED = 3    # the planner's per-workgroup cost, in key tiles


def tiles_of_blocks(L, N, q_shard, kv_shard, layout, causal, rows):
    """Key tiles (64 keys) the workgroup of each query block walks, from global positions."""
    toks = shard_tokens(layout, N, L)
    pos_q, pos_k = toks[q_shard], toks[kv_shard]
    out = []
    for r0 in range(0, L, rows):
        last = min(r0 + rows, L) - 1
        n_keys = int(np.sum(pos_k <= pos_q[last])) if causal else L
        out.append(-(-n_keys // 64))
    return out


def check_plan(L, h, n_kv, N, q_shard, kv_shard, layout, causal, n_cu, b=1):
    items, rows = ra.fwd_step_plan(b=b, L=L, h=h, n_kv=n_kv, N=N, q_shard=q_shard, kv_shard=kv_shard,
                                   causal=causal, layout=layout, n_cu=n_cu)
    n_qb = -(-L // rows)
    seen = {}
    for blk, part in items:
        assert 0 <= blk < n_qb
        seen.setdefault(blk, []).append(part)
    assert sorted(seen) == list(range(n_qb)), "every block covered"
    for blk, parts in seen.items():
        assert sorted(parts) in ([-1], [0, 1]), f"block {blk}: {parts}"
    G = h // n_kv
    inner = n_kv * b * (G // (4 if G % 4 == 0 else 2 if G % 2 == 0 else 1))
    assert len(items) <= max(n_qb, n_cu // inner), "more items than units"
    if n_qb >= n_cu // inner:
        assert all(part < 0 for _, part in items), "a grid that fills the chip is not split"
    tiles = tiles_of_blocks(L, N, q_shard, kv_shard, layout, causal, rows)
    cost = [tiles[blk] + FIXED if part < 0 else (tiles[blk] + 1) // 2 + FIXED for blk, part in items]
    assert all(a >= c for a, c in zip(cost, cost[1:])), f"not heaviest first: {cost}"
    return items, rows, tiles


CASES = [(L, layout, causal, qs, ks)
         for L in (64, 200, 1000, 2048, 4096)
         for layout, causal in (("contiguous", False), ("contiguous", True), ("striped", True), ("zigzag", True))
         for qs, ks in ((0, 0), (3, 1), (1, 3))]


@pytest.mark.parametrize("L,layout,causal,qs,ks", CASES)
@pytest.mark.parametrize("h,n_kv", [(32, 8), (8, 4), (4, 4)])
def test_plan_covers_every_block_once_heaviest_first(L, layout, causal, qs, ks, h, n_kv):
    for n_cu in (256, 80):
        check_plan(L, h, n_kv, 4, qs, ks, layout, causal, n_cu)


def test_plan_splits_only_where_units_sit_idle():
    # striped causal, L = 1024: 16 query blocks of 64 rows (block i sees i + 1 key tiles) for
    # each of 8 KV heads, 32 units per head on 256: the heavy half is split, the longest item
    # shrinks, at most one item per unit
    items, rows, tiles = check_plan(1024, 32, 8, 8, 0, 0, "striped", True, 256)
    assert rows == 64 and tiles == list(range(1, 17))
    split = {blk for blk, part in items if part >= 0}
    assert split and max(split) == 15 and len(items) <= 32
    longest = max(t + FIXED if b not in split else (t + 1) // 2 + FIXED for b, t in enumerate(tiles))
    assert 10 * longest <= 9 * (16 + FIXED)
    # few blocks all of one length: every block split, one item per unit
    items, _, _ = check_plan(1024, 32, 8, 8, 0, 0, "contiguous", False, 256)
    assert all(part >= 0 for _, part in items) and len(items) == 32
    # fewer KV heads leave more units per block list: L = 2048 splits with 2 KV heads
    items, _, _ = check_plan(2048, 8, 2, 8, 0, 0, "striped", True, 256)
    assert any(part >= 0 for _, part in items) and len(items) <= 128
    # a grid that fills the chip already is not split, however uneven its blocks
    for L, layout, causal in ((2048, "striped", True), (2048, "contiguous", False), (4096, "striped", True)):
        items, _, _ = check_plan(L, 32, 8, 8, 0, 0, layout, causal, 256)
        assert all(part < 0 for _, part in items), (L, layout)
    # beyond the second accumulator's range (L > 4096) a step runs every block whole
    items, rows = ra.fwd_step_plan(b=1, L=8192, h=32, n_kv=8, N=8, q_shard=0, kv_shard=0, causal=True,
                                   layout="striped", n_cu=256)
    assert len(items) == 128 and [blk for blk, _ in items] == list(range(127, -1, -1))


def test_plan_errors_and_workspace_sizes():
    lib = _lib.lib()
    p = ra.make_problem(b=1, L=256, h=2, n_kv=1, d=64, N=4, causal=True, layout="striped", dtype=torch.float32)
    n = ctypes.c_int32(0)
    rows = ctypes.c_int32(0)
    assert lib.ra_fwd_step_plan(ctypes.byref(p), 0, 0, 256, None, None, 0, ctypes.byref(n),
                                ctypes.byref(rows)) == _lib.RA_ERR_UNSUPPORTED
    p = ra.make_problem(b=1, L=256, h=8, n_kv=2, d=128, N=4, causal=True, layout="striped", dtype=torch.bfloat16)
    assert lib.ra_fwd_step_plan(ctypes.byref(p), 0, 0, 0, None, None, 0, ctypes.byref(n),
                                ctypes.byref(rows)) == _lib.RA_ERR_INVALID_ARG
    assert lib.ra_fwd_step_plan(ctypes.byref(p), 4, 0, 256, None, None, 0, ctypes.byref(n),
                                ctypes.byref(rows)) == _lib.RA_ERR_INVALID_ARG
    # max_items = 0: only the count
    assert lib.ra_fwd_step_plan(ctypes.byref(p), 0, 0, 256, None, None, 0, ctypes.byref(n), ctypes.byref(rows)) == 0
    assert n.value >= 4 and rows.value == 64

    def al(x):
        return -(-x // 256) * 256

    def ws(**cfg):   # one launch per ring step: the pass that may split blocks
        q = ra.make_problem(**cfg, causal=True, layout="striped", dtype=torch.bfloat16, steps_per_launch=1)
        return lib.ra_ring_fwd_workspace(ctypes.byref(q))

    for b, L, h, n_kv in ((1, 2048, 32, 8), (2, 330, 8, 2), (1, 4096, 4, 4), (1, 4097, 4, 4), (1, 8192, 32, 8)):
        base = 4 * al(b * L * n_kv * 128 * 2) + al(b * L * h * 128 * 4)
        second = al(b * L * h * 128 * 4) + al(b * h * L * 4) if L <= 4096 else 0
        assert ws(b=b, L=L, h=h, n_kv=n_kv, d=128, N=4) == base + second, (b, L, h, n_kv)

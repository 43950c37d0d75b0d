"""Forward passes of short shards with the second accumulator: heavy query blocks run their key
range as two workgroups merging into two accumulators that the pass folds together (bf16,
L <= 4096, no packed documents, one launch per ring step).  Each case first checks, with the
device's compute-unit count, that the plan really splits blocks in its steps; then the pass
must match the oracle, and so must the same pass without the second accumulator (every block
whole), with the two close to each other (they differ only in the order of the fp32 sums)."""
import numpy as np
import pytest
import torch

import ring_attention_long_amd as ra
from gpu_helpers import announce, check_bf16, f64, full_size_rows, make_inputs, oracle_ring, oracle_ring_rows, to_gpu
from oracle import ring_order

pytestmark = pytest.mark.gpu


def _al(x):
    return -(-x // 256) * 256


def base_workspace(cfg):
    """ra_ring_fwd's workspace without the second accumulator (KV double buffer, fp32 acc)."""
    b, L, h, n_kv, d = (cfg[x] for x in ("b", "L", "h", "n_kv", "d"))
    return 4 * _al(b * L * n_kv * d * 2) + _al(b * L * h * d * 4)


def step_plans(cfg, shard, layout, causal):
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    return [ra.fwd_step_plan(b=cfg["b"], L=cfg["L"], h=cfg["h"], n_kv=cfg["n_kv"], N=cfg["N"], q_shard=shard,
                             kv_shard=src, causal=causal, layout=layout, n_cu=n_cu)[0]
            for src in ring_order(cfg["N"], shard)]


def split_blocks(items):
    return {blk for blk, part in items if part >= 0}


def both_passes(inp, cfg, shard, layout, causal):
    q, k_all, v_all = (to_gpu(inp[x], "bf16") for x in ("q", "k_all", "v_all"))
    o1, l1 = ra.ring_fwd(q, k_all, v_all, q_shard=shard, causal=causal, layout=layout, steps_per_launch=1)
    ws = torch.empty(base_workspace(cfg), device="cuda", dtype=torch.uint8)
    o2, l2 = ra.ring_fwd(q, k_all, v_all, q_shard=shard, causal=causal, layout=layout, workspace=ws,
                         steps_per_launch=1)
    torch.cuda.synchronize()
    return (o1, l1), (o2, l2)


CASES = [
    # query heads per KV head 4 (64-row blocks), ragged L, two batch rows
    (dict(b=2, L=1000, h=8, n_kv=2, d=128, N=4), "striped", True, 3),
    # 2 (128-row blocks)
    (dict(b=1, L=1024, h=8, n_kv=4, d=128, N=4), "zigzag", True, 2),
    # 1 (256-row blocks), odd ring size
    (dict(b=1, L=1536, h=4, n_kv=4, d=128, N=3), "contiguous", True, 2),
    (dict(b=1, L=640, h=8, n_kv=2, d=128, N=4), "contiguous", False, 1),
    # three batch rows, one query head per KV head
    (dict(b=3, L=640, h=4, n_kv=4, d=128, N=3), "striped", True, 1),
    # two batch rows, 2 query heads per KV head, ragged zigzag shard
    (dict(b=2, L=500, h=8, n_kv=4, d=128, N=4), "zigzag", True, 0),
]


@pytest.mark.parametrize("cfg,layout,causal,shard", CASES)
def test_split_pass_matches_oracle_and_unsplit_pass(cfg, layout, causal, shard):
    plans = step_plans(cfg, shard, layout, causal)
    assert any(split_blocks(p) for p in plans), "the plan splits no block: the case tests nothing"
    announce("split pass", cfg, layout, "causal", causal, "shard", shard,
             "split blocks per step", [len(split_blocks(p)) for p in plans])
    inp = make_inputs(**cfg, q_shard=shard, seed=1200 + shard, dtype="bf16")
    (o1, l1), (o2, l2) = both_passes(inp, cfg, shard, layout, causal)
    O, LSE = oracle_ring(inp, N=cfg["N"], shard=shard, layout=layout, causal=causal)
    check_bf16(o1, l1, O, LSE, "with the second accumulator")
    check_bf16(o2, l2, O, LSE, "without")
    d_o = np.abs(f64(o1) - f64(o2)).max()
    fin = np.isfinite(f64(l2))
    d_l = np.abs(f64(l1)[fin] - f64(l2)[fin]).max()
    announce(f"split vs unsplit: max |dO| {d_o:.3e}, max |dLSE| {d_l:.3e}")
    assert d_o <= 2e-2 and d_l <= 1e-4


def test_block_split_after_the_first_step():
    """Contiguous causal, last shard: the first step (its own shard, triangular) splits only
    its heavy blocks, the later full steps split every block, so the light blocks' second
    accumulator rows are first written by a merge into rows the first step marked empty."""
    cfg = dict(b=1, L=1024, h=32, n_kv=8, d=128, N=4)
    shard = 3
    plans = step_plans(cfg, shard, "contiguous", True)
    first, later = split_blocks(plans[0]), set.union(*(split_blocks(p) for p in plans[1:]))
    announce("split after the first step", cfg, "first", sorted(first), "later", sorted(later))
    assert later - first, "no block is split later than the first step"
    inp = make_inputs(**cfg, q_shard=shard, seed=1210, dtype="bf16")
    (o1, l1), (o2, l2) = both_passes(inp, cfg, shard, "contiguous", True)
    O, LSE = oracle_ring(inp, N=cfg["N"], shard=shard, layout="contiguous", causal=True)
    check_bf16(o1, l1, O, LSE, "split later")
    check_bf16(o2, l2, O, LSE, "unsplit")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("L,h,n_kv,shard", [(1024, 32, 8, 0), (1024, 32, 8, 5), (2048, 8, 2, 3)])
def test_split_striped_causal_sweep_shapes(L, h, n_kv, shard):
    """Short striped causal shards (N = 8) with every step split, on ~300 sampled rows (every
    64-row block class, both halves' boundary rows): the small-L sweep's shape (h = 32,
    n_kv = 8) and, at L = 2048, a grid that splits only with fewer KV heads."""
    cfg = dict(b=1, L=L, h=h, n_kv=n_kv, d=128, N=8)
    plans = step_plans(cfg, shard, "striped", True)
    assert all(split_blocks(p) for p in plans)
    inp = make_inputs(**cfg, q_shard=shard, seed=1220 + shard, dtype="bf16")
    rows = full_size_rows(L, 1230 + shard)
    announce("split sweep shape", cfg, "shard", shard, "rows", rows.size)
    (o1, l1), _ = both_passes(inp, cfg, shard, "striped", True)
    O, LSE = oracle_ring_rows(inp, N=8, shard=shard, layout="striped", causal=True, rows=rows)
    ri = torch.from_numpy(rows).to(o1.device)
    check_bf16(o1[:, ri], l1[:, :, ri], O, LSE, f"L={L} h={h} shard {shard}")

"""The allocation-free forward pass (ra_ring_fwd_noalloc) against ra_ring_fwd given a workspace
of the array's size: the same kernels on the same inputs (batched steps, the second accumulator,
exactly when they fit in the array), so outputs must be
bit-identical, on calls in a row (each no larger, so it runs over what the one before left in
the shared scratch array), in bf16 and fp32; a problem whose workspace exceeds the array is
refused without writing anything."""
import ctypes

import numpy as np
import pytest
import torch

import ring_attention_long_amd as ra
from gpu_helpers import announce, check_bf16, make_inputs, oracle_ring, to_gpu
from ring_attention_long_amd import _lib

pytestmark = pytest.mark.gpu


def _inputs(cfg, dtype, seed, shard):
    inp = make_inputs(**cfg, q_shard=shard, seed=seed, dtype=dtype)
    return inp, [to_gpu(inp[x], dtype) for x in ("q", "k_all", "v_all")]


def test_noalloc_matches_ring_fwd_two_calls():
    cases = [  # (config, steps per launch, dtype, layout, shard): each call no larger than the one before
        # all remote steps in one launch: 14 K/V slots, the accumulator and the second one, 60 MiB
        # (the launches split their query blocks)
        (dict(b=1, L=1024, h=32, n_kv=8, d=128, N=8), 0, "bf16", "striped", 5),
        # all remote steps in one launch: 6 K/V slots and the accumulator, 56 MiB; the second
        # accumulator (32 MiB more) does not fit
        (dict(b=1, L=2048, h=32, n_kv=8, d=128, N=4), 0, "bf16", "striped", 1),
        # one launch per step: 48 MiB without the second accumulator, 80 MiB with it: unsplit
        (dict(b=1, L=2048, h=32, n_kv=8, d=128, N=4), 1, "bf16", "striped", 1),
        # 48 MiB with the second accumulator: the split path
        (dict(b=1, L=2048, h=16, n_kv=8, d=128, N=4), 1, "bf16", "striped", 2),
        (dict(b=2, L=330, h=8, n_kv=2, d=128, N=3), 0, "bf16", "zigzag", 2),
        (dict(b=1, L=256, h=2, n_kv=1, d=64, N=4), 0, "f32", "contiguous", 3),
    ]
    scratch = _lib.RA_NOALLOC_SCRATCH_BYTES
    ws = torch.empty(scratch, device="cuda", dtype=torch.uint8)
    for n, (cfg, spl, dtype, layout, shard) in enumerate(cases):
        p = ra.make_problem(**cfg, causal=True, layout=layout, steps_per_launch=spl,
                            dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
        need = _lib.lib().ra_ring_fwd_workspace(ctypes.byref(p))
        assert need > 0
        second = (cfg["b"] * cfg["L"] * cfg["h"] * cfg["d"] * 4 + 255) // 256 * 256 + \
            (cfg["b"] * cfg["h"] * cfg["L"] * 4 + 255) // 256 * 256
        if n in (1, 2):
            assert need - second <= scratch < need     # the second accumulator does not fit
        elif n in (0, 3):
            assert need <= scratch
        announce("ring_fwd_noalloc call", n, cfg, "steps per launch", spl, dtype, layout, "shard", shard,
                 "workspace", need)
        inp, (q, k_all, v_all) = _inputs(cfg, dtype, 900 + n, shard)
        o_ref, lse_ref = ra.ring_fwd(q, k_all, v_all, q_shard=shard, causal=True, layout=layout, workspace=ws,
                                     steps_per_launch=spl)
        o, lse = ra.ring_fwd_noalloc(q, k_all, v_all, q_shard=shard, causal=True, layout=layout,
                                     steps_per_launch=spl)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
        if dtype == "bf16":
            O, LSE = oracle_ring(inp, N=cfg["N"], shard=shard, layout=layout, causal=True)
            check_bf16(o, lse, O, LSE, f"noalloc call {n}")


def test_noalloc_repeated_on_one_stream_and_without_side_stream():
    """Back-to-back calls on one stream reuse the array and events; all equal ra_ring_fwd."""
    cfg = dict(b=1, L=512, h=8, n_kv=2, d=128, N=5)
    inp, (q, k_all, v_all) = _inputs(cfg, "bf16", 910, 4)
    o_ref, lse_ref = ra.ring_fwd(q, k_all, v_all, q_shard=4, causal=True, layout="striped")
    announce("ring_fwd_noalloc x4 back to back")
    outs = [ra.ring_fwd_noalloc(q, k_all, v_all, q_shard=4, causal=True, layout="striped",
                                copy_stream=None if i % 2 else "auto") for i in range(4)]
    torch.cuda.synchronize()
    for o, lse in outs:
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)


def test_noalloc_refuses_oversized_problem():
    cfg = dict(b=1, L=8192, h=32, n_kv=8, d=128, N=2)          # ~134 MB of workspace
    p = ra.make_problem(**cfg, causal=True, layout="striped", dtype=torch.bfloat16)
    assert _lib.lib().ra_ring_fwd_workspace(ctypes.byref(p)) > _lib.RA_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(1, 8192, 32, 128, device="cuda", dtype=torch.bfloat16)
    kv = torch.zeros(2, 1, 8192, 8, 128, device="cuda", dtype=torch.bfloat16)
    o = torch.full_like(q, 7.0)
    lse = torch.full((1, 32, 8192), 7.0, device="cuda")
    announce("ring_fwd_noalloc oversized")
    with pytest.raises(ra.RaError) as ei:
        ra.ring_fwd_noalloc(q, kv, kv, q_shard=0, causal=True, layout="striped", out=o, lse_out=lse)
    assert ei.value.status == _lib.RA_ERR_WORKSPACE and "scratch" in ei.value.detail
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())

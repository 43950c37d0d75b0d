"""Ordering of the staging buffers (page 1, "Practical Implementation Patterns": the
incoming block must have arrived before a step reads it, and a buffer is refilled only after
the step that read it).  The copy stream is held back by a bounded spin before each pass, the
whole workspace starts as NaN, and with RA_POISON_STAGING=1 every staging buffer is refilled
with NaN on the copy stream as soon as its step (or the launch running it) has finished.  A
step that read a buffer before its copy landed, or after it was consumed, would see NaN; the
results must instead be bit-identical to a plain pass.  The forward (one launch per step with
its double buffer, and batched steps with a slot per remote shard), the backward and the
key/value-stationary backward are checked, and the test confirms afterwards that the poison
really ran."""
import ctypes

import numpy as np
import pytest
import torch

import ring_attention_long_amd as ra
from gpu_helpers import announce, make_inputs, to_gpu
from ring_attention_long_amd import _lib

pytestmark = pytest.mark.gpu

SPIN_CYCLES = 20_000_000          # a bounded spin of roughly 10 ms on the copy stream


def _held_back_stream():
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        torch.cuda._sleep(SPIN_CYCLES)
    return s


def _nan_workspace(nbytes):
    return torch.full((nbytes,), 255, dtype=torch.uint8, device="cuda")


def _all_ones(t):
    return bool((t == 255).all())


CFG = dict(b=1, L=256, h=8, n_kv=2, d=128, N=6)
SHARD = 2


def _staging_regions(ws, shard_bytes, n=4):
    A = (shard_bytes + 255) // 256 * 256
    return [ws[i * A: i * A + shard_bytes] for i in range(n)]


@pytest.mark.parametrize("spl", [1, 2, 0])
def test_forward_order_under_delay_and_poison(monkeypatch, spl):
    inp = make_inputs(**CFG, q_shard=SHARD, seed=1201, dtype="bf16")
    q, k_all, v_all = (to_gpu(inp[x], "bf16") for x in ("q", "k_all", "v_all"))
    announce("ordering: forward, plain pass, steps per launch", spl)
    o_ref, lse_ref = ra.ring_fwd(q, k_all, v_all, q_shard=SHARD, causal=True, layout="striped",
                                 steps_per_launch=spl)
    torch.cuda.synchronize()
    p = ra.make_problem(**CFG, causal=True, layout="striped", dtype=torch.bfloat16, steps_per_launch=spl)
    ws = _nan_workspace(_lib.lib().ra_ring_fwd_workspace(ctypes.byref(p)))
    monkeypatch.setenv("RA_POISON_STAGING", "1")
    announce("ordering: forward, copy stream held back, NaN workspace, poison after each launch")
    o, lse = ra.ring_fwd(q, k_all, v_all, q_shard=SHARD, causal=True, layout="striped",
                         copy_stream=_held_back_stream(), workspace=ws, steps_per_launch=spl)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    shard_bytes = CFG["b"] * CFG["L"] * CFG["n_kv"] * CFG["d"] * 2
    # K0, V0, K1, V1 of the double buffer, or the K and V slots of the N - 1 remote shards
    n_regions = 4 if spl == 1 else 2 * (CFG["N"] - 1)
    assert all(_all_ones(r) for r in _staging_regions(ws, shard_bytes, n_regions)), "staging buffers were not poisoned"


def test_backward_order_under_delay_and_poison(monkeypatch):
    inp = make_inputs(**CFG, q_shard=SHARD, seed=1202, dtype="bf16", with_dout=True)
    q, k_all, v_all, dout = (to_gpu(inp[x], "bf16") for x in ("q", "k_all", "v_all", "dout"))
    o, lse = ra.ring_fwd(q, k_all, v_all, q_shard=SHARD, causal=True, layout="zigzag")
    announce("ordering: backward, plain pass")
    ref = ra.ring_bwd(q, k_all, v_all, o, dout, lse, q_shard=SHARD, causal=True, layout="zigzag")
    torch.cuda.synchronize()
    p = ra.make_problem(**CFG, causal=True, layout="zigzag", dtype=torch.bfloat16)
    ws = _nan_workspace(_lib.lib().ra_ring_bwd_workspace(ctypes.byref(p)))
    monkeypatch.setenv("RA_POISON_STAGING", "1")
    announce("ordering: backward, copy stream held back, NaN workspace, poison after each step")
    got = ra.ring_bwd(q, k_all, v_all, o, dout, lse, q_shard=SHARD, causal=True, layout="zigzag",
                      copy_stream=_held_back_stream(), workspace=ws)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(got, ref))
    shard_bytes = CFG["b"] * CFG["L"] * CFG["n_kv"] * CFG["d"] * 2
    assert all(_all_ones(r) for r in _staging_regions(ws, shard_bytes)), "staging buffers were not poisoned"


def test_kv_stationary_order_under_delay_and_poison(monkeypatch):
    import synth
    N, b, L, h, n_kv, d = CFG["N"], CFG["b"], CFG["L"], CFG["h"], CFG["n_kv"], CFG["d"]
    q = np.stack([synth.normal((b, L, h, d), seed=1203, name="q", shard=j) for j in range(N)])
    do = np.stack([synth.normal((b, L, h, d), seed=1203, name="do", shard=j) for j in range(N)])
    k = np.stack([synth.normal((b, L, n_kv, d), seed=1203, name="k", shard=j) for j in range(N)])
    v = np.stack([synth.normal((b, L, n_kv, d), seed=1203, name="v", shard=j) for j in range(N)])
    qg, dog, kg, vg = (to_gpu(x, "bf16") for x in (q, do, k, v))
    lse_all, delta_all = [], []
    for i in range(N):
        oi, li = ra.ring_fwd(qg[i].contiguous(), kg, vg, q_shard=i, causal=True, layout="striped")
        lse_all.append(li)
        delta_all.append(ra.bwd_preprocess(oi, dog[i].contiguous()))
    lse_all, delta_all = torch.stack(lse_all), torch.stack(delta_all)
    args = (kg[3].contiguous(), vg[3].contiguous(), qg, dog, lse_all, delta_all)
    announce("ordering: key/value-stationary backward, plain pass")
    ref = ra.ring_bwd_kv_stationary(*args, kv_shard=3, causal=True, layout="striped")
    torch.cuda.synchronize()
    p = ra.make_problem(**CFG, causal=True, layout="striped", dtype=torch.bfloat16)
    ws = _nan_workspace(_lib.lib().ra_ring_bwd_kv_stationary_workspace(ctypes.byref(p)))
    monkeypatch.setenv("RA_POISON_STAGING", "1")
    announce("ordering: key/value-stationary backward, copy stream held back, NaN workspace, poison")
    got = ra.ring_bwd_kv_stationary(*args, kv_shard=3, causal=True, layout="striped",
                                    copy_stream=_held_back_stream(), workspace=ws)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(got, ref))
    assert _all_ones(ws), "staging buffers were not poisoned"

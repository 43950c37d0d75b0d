"""GPU parity of the key/value-stationary backward schedule (page 1, "The Backward Pass and
Gradient Exchange": output gradients circulate while keys and values stay) against the fp64
oracle.  Every device runs its pass; each shard's dQ is the sum of all devices'
contributions, each device's dK and dV are complete.  The forward's O and LSE and the
preprocess's D come from the library itself, as on a real ring."""
import numpy as np
import pytest
import torch

import ring_attention_long_amd as ra
import synth
from gpu_helpers import (BWD_FULL, BWD_FULL_KV_HEAD, announce, bwd_full_cols, bwd_full_inputs, bwd_full_key_grads,
                         f64, full_size_rows, gather_cols, to_gpu)
from oracle import shard_grads
from test_gpu_bwd import check_grad, oracle_dq_rows

pytestmark = pytest.mark.gpu


def all_shards(*, b, L, h, n_kv, d, N, seed):
    q = np.stack([synth.normal((b, L, h, d), seed=seed, name="q", shard=j) for j in range(N)])
    do = np.stack([synth.normal((b, L, h, d), seed=seed, name="do", shard=j) for j in range(N)])
    k = np.stack([synth.normal((b, L, n_kv, d), seed=seed, name="k", shard=j) for j in range(N)])
    v = np.stack([synth.normal((b, L, n_kv, d), seed=seed, name="v", shard=j) for j in range(N)])
    return q, do, k, v


def forward_all(qg, kg, vg, dog, *, causal, layout):
    """What every home device holds before the backward: O, LSE and D of its query shard."""
    N = qg.shape[0]
    lse_all, delta_all = [], []
    for i in range(N):
        o, lse = ra.ring_fwd(qg[i].contiguous(), kg, vg, q_shard=i, causal=causal, layout=layout)
        lse_all.append(lse)
        delta_all.append(ra.bwd_preprocess(o, dog[i].contiguous()))
    return torch.stack(lse_all), torch.stack(delta_all)


def stationary_all(qg, kg, vg, dog, lse_all, delta_all, *, causal, layout):
    N = qg.shape[0]
    dq = torch.zeros(qg.shape, device="cuda", dtype=torch.float32)
    dk, dv = [], []
    for j in range(N):
        dq_j, dk_j, dv_j = ra.ring_bwd_kv_stationary(kg[j].contiguous(), vg[j].contiguous(), qg, dog, lse_all,
                                                     delta_all, kv_shard=j, causal=causal, layout=layout)
        dq += dq_j
        dk.append(dk_j)
        dv.append(dv_j)
    torch.cuda.synchronize()
    return dq, torch.stack(dk), torch.stack(dv)


@pytest.mark.parametrize("layout,causal", [("contiguous", False), ("contiguous", True),
                                           ("striped", True), ("zigzag", True)])
def test_kv_stationary_matches_oracle(layout, causal):
    cfg = dict(b=1, L=200, h=8, n_kv=2, d=128, N=3)
    announce("kv-stationary backward", layout, "causal", causal, cfg)
    q, do, k, v = all_shards(**cfg, seed=301)
    qg, dog, kg, vg = (to_gpu(x, "bf16") for x in (q, do, k, v))
    lse_all, delta_all = forward_all(qg, kg, vg, dog, causal=causal, layout=layout)
    dq, dk, dv = stationary_all(qg, kg, vg, dog, lse_all, delta_all, causal=causal, layout=layout)
    x = [a.astype(np.float64) for a in (q, do, k, v)]
    rdk = np.zeros(k.shape)
    rdv = np.zeros(v.shape)
    for i in range(3):
        rq, rk, rv = shard_grads(x[0][i], x[2], x[3], x[1][i], N=3, shard=i, layout=layout, causal=causal)
        check_grad(dq[i], rq, f"dq shard {i} {layout} {causal}")
        rdk += rk
        rdv += rv
    for j in range(3):
        check_grad(dk[j], rdk[j], f"dk shard {j} {layout} {causal}")
        check_grad(dv[j], rdv[j], f"dv shard {j} {layout} {causal}")


@pytest.mark.timeout(900)
def test_kv_stationary_full_size():
    """S = 65536 (N = 8, L = 8192, h = 32, n_kv = 8, d = 128, bf16), striped causal, every
    device's stationary pass: dK, dV of 144 keys spread over all 8 KV shards (KV head 2) and
    the summed dQ of ~300 sampled rows of two shards against the oracle, element by element."""
    N, L = BWD_FULL["N"], BWD_FULL["L"]
    announce("kv-stationary full size: inputs")
    q, do, k, v = bwd_full_inputs()
    qg, dog, kg, vg = (to_gpu(x, "bf16") for x in (q, do, k, v))
    announce("kv-stationary full size: forward of every shard")
    lse_all, delta_all = forward_all(qg, kg, vg, dog, causal=True, layout="striped")
    announce("kv-stationary full size: stationary pass of every device")
    dq, dk, dv = stationary_all(qg, kg, vg, dog, lse_all, delta_all, causal=True, layout="striped")
    cols = bwd_full_cols()
    announce(f"kv-stationary full size: oracle dK, dV of {len(cols)} keys from every query shard")
    rdk, rdv = bwd_full_key_grads(list(range(N)))
    check_grad(gather_cols(dk, cols, BWD_FULL_KV_HEAD), rdk, "full size dk sampled keys")
    check_grad(gather_cols(dv, cols, BWD_FULL_KV_HEAD), rdv, "full size dv sampled keys")
    x = [a.astype(np.float64) for a in (q, do, k, v)]
    for i in (0, 5):
        rows = full_size_rows(L, 6006 + i)
        announce(f"kv-stationary full size: oracle dQ of {rows.size} rows of shard {i}")
        ref = oracle_dq_rows(x[0][i], x[2], x[3], x[1][i], rows, N=N, shard=i, layout="striped", causal=True)
        check_grad(dq[i][:, torch.from_numpy(rows).cuda()], ref, f"full size dq shard {i} sampled rows")


def test_kv_stationary_batch_and_single_shard():
    """b = 2 with N = 1 (no staging at all) against the oracle."""
    cfg = dict(b=2, L=150, h=4, n_kv=2, d=128, N=1)
    announce("kv-stationary b=2 N=1")
    q, do, k, v = all_shards(**cfg, seed=303)
    qg, dog, kg, vg = (to_gpu(x, "bf16") for x in (q, do, k, v))
    lse_all, delta_all = forward_all(qg, kg, vg, dog, causal=True, layout="contiguous")
    dq, dk, dv = stationary_all(qg, kg, vg, dog, lse_all, delta_all, causal=True, layout="contiguous")
    x = [a.astype(np.float64) for a in (q, do, k, v)]
    rq, rk, rv = shard_grads(x[0][0], x[2], x[3], x[1][0], N=1, shard=0, layout="contiguous", causal=True)
    check_grad(dq[0], rq, "b=2 N=1 dq")
    check_grad(dk[0], rk[0], "b=2 N=1 dk")
    check_grad(dv[0], rv[0], "b=2 N=1 dv")


def test_kv_stationary_staging_stream_does_not_change_results():
    """Staging on the side stream or on the compute stream gives bit-identical gradients."""
    cfg = dict(b=1, L=128, h=8, n_kv=2, d=128, N=4)
    q, do, k, v = all_shards(**cfg, seed=304)
    qg, dog, kg, vg = (to_gpu(x, "bf16") for x in (q, do, k, v))
    lse_all, delta_all = forward_all(qg, kg, vg, dog, causal=True, layout="striped")
    args = (kg[2].contiguous(), vg[2].contiguous(), qg, dog, lse_all, delta_all)
    announce("kv-stationary: side stream vs compute stream")
    a = ra.ring_bwd_kv_stationary(*args, kv_shard=2, causal=True, layout="striped")
    b = ra.ring_bwd_kv_stationary(*args, kv_shard=2, causal=True, layout="striped", copy_stream=None)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))

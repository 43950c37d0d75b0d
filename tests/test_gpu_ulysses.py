"""GPU parity of the all-to-all sequence-parallel path (page 3, sections 4.2 and 7) against the
fp64 oracle.  Each device's share covers h/N query heads of the whole sequence; filling the
output one head group at a time must give, for every shard, exactly what the oracle's
attention of that shard's queries to the whole sequence gives (the quantity a ring device
also computes)."""
import numpy as np
import pytest
import torch

import ring_attention_long_amd as ra
import synth
from gpu_helpers import announce, check_bf16, check_f32, f64, full_size_rows, oracle_ring_rows, to_gpu
from oracle import LAYOUTS, shard_attention

pytestmark = pytest.mark.gpu


def all_shards(*, b, L, h, n_kv, d, N, seed, dtype):
    q = np.stack([synth.normal((b, L, h, d), seed=seed, name="q", shard=j, dtype=dtype) for j in range(N)])
    k = np.stack([synth.normal((b, L, n_kv, d), seed=seed, name="k", shard=j, dtype=dtype) for j in range(N)])
    v = np.stack([synth.normal((b, L, n_kv, d), seed=seed, name="v", shard=j, dtype=dtype) for j in range(N)])
    return q, k, v


def run_all_groups(q, k, v, *, N, causal, layout):
    out = lse = None
    for g in range(N):
        out, lse = ra.ulysses_fwd(q, k, v, head_group=g, causal=causal, layout=layout, out=out, lse_out=lse)
    torch.cuda.synchronize()
    return out, lse


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("causal", [True, False])
def test_ulysses_bf16_every_shard(layout, causal):
    cfg = dict(b=2, L=100, h=8, n_kv=4, d=128, N=4)          # S = 400: six full key tiles and a ragged one
    announce("ulysses bf16", layout, "causal", causal, cfg)
    q, k, v = all_shards(**cfg, seed=201, dtype="bf16")
    out, lse = run_all_groups(to_gpu(q, "bf16"), to_gpu(k, "bf16"), to_gpu(v, "bf16"), N=4, causal=causal,
                              layout=layout)
    x = {n: a.astype(np.float64) for n, a in (("q", q), ("k", k), ("v", v))}
    for j in range(4):
        O, LSE = shard_attention(x["q"][j], x["k"], x["v"], N=4, shard=j, layout=layout, causal=causal)
        check_bf16(out[j], lse[j], O, LSE, f"ulysses {layout} {causal} shard {j}")


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("causal", [True, False])
def test_ulysses_f32_every_shard(layout, causal):
    cfg = dict(b=1, L=50, h=4, n_kv=2, d=64, N=2)            # S = 100, GQA 2
    announce("ulysses f32", layout, "causal", causal, cfg)
    q, k, v = all_shards(**cfg, seed=202, dtype="f32")
    out, lse = run_all_groups(to_gpu(q, "f32"), to_gpu(k, "f32"), to_gpu(v, "f32"), N=2, causal=causal,
                              layout=layout)
    for j in range(2):
        O, LSE = shard_attention(q[j].astype(np.float64), k.astype(np.float64), v.astype(np.float64), N=2,
                                 shard=j, layout=layout, causal=causal)
        check_f32(out[j], lse[j], O, LSE, f"ulysses f32 {layout} {causal} shard {j}")


def test_ulysses_writes_only_its_head_group():
    cfg = dict(b=1, L=64, h=8, n_kv=4, d=128, N=4)
    q, k, v = all_shards(**cfg, seed=203, dtype="bf16")
    qg, kg, vg = to_gpu(q, "bf16"), to_gpu(k, "bf16"), to_gpu(v, "bf16")
    out = torch.full((4, 1, 64, 8, 128), 7.0, device="cuda", dtype=torch.bfloat16)
    lse = torch.full((4, 1, 8, 64), 7.0, device="cuda", dtype=torch.float32)
    announce("ulysses head group 2 only")
    ra.ulysses_fwd(qg, kg, vg, head_group=2, causal=True, layout="striped", out=out, lse_out=lse)
    torch.cuda.synchronize()
    o, l = f64(out), f64(lse)
    others = [hq for hq in range(8) if hq not in (4, 5)]
    assert np.all(o[:, :, :, others] == 7.0) and np.all(l[:, :, others] == 7.0)
    assert not np.any(o[:, :, :, 4:6] == 7.0)
    # the written heads agree with the oracle
    x = [a.astype(np.float64) for a in (q, k, v)]
    O, LSE = shard_attention(x[0][1], x[1], x[2], N=4, shard=1, layout="striped", causal=True)
    check_bf16(out[1][:, :, 4:6], lse[1][:, 4:6], O[:, :, 4:6], LSE[:, 4:6], "ulysses group 2, shard 1")


def test_ulysses_matches_ring_fwd():
    """Both spreadings of the same attention agree with each other on every shard (each is
    also checked against the oracle above)."""
    cfg = dict(b=1, L=128, h=8, n_kv=2, d=128, N=2)
    q, k, v = all_shards(**cfg, seed=204, dtype="bf16")
    qg, kg, vg = to_gpu(q, "bf16"), to_gpu(k, "bf16"), to_gpu(v, "bf16")
    announce("ulysses vs ring, zigzag causal")
    out, lse = run_all_groups(qg, kg, vg, N=2, causal=True, layout="zigzag")
    for j in range(2):
        o_r, l_r = ra.ring_fwd(qg[j].contiguous(), kg, vg, q_shard=j, causal=True, layout="zigzag")
        torch.cuda.synchronize()
        d_o = (out[j].float() - o_r.float()).abs().max().item()
        d_l = (lse[j] - l_r).abs().max().item()
        announce(f"shard {j}: max |O diff| {d_o:.3e}, max |LSE diff| {d_l:.3e}")
        assert d_o <= 2e-2 and d_l <= 1e-3


@pytest.mark.timeout(600)
def test_ulysses_full_size_sampled():
    """S = 262144 (N = 8 shards of 32768, h = 32, n_kv = 8, d = 128, bf16), striped causal,
    head group 5, in the launch configuration of the benchmark; sampled rows of two shards
    against the oracle."""
    N, L, h, n_kv, d = 8, 32768, 32, 8, 128
    announce("ulysses full size: generating inputs")
    q, k, v = all_shards(b=1, L=L, h=h, n_kv=n_kv, d=d, N=N, seed=205, dtype="bf16")
    qg, kg, vg = to_gpu(q, "bf16"), to_gpu(k, "bf16"), to_gpu(v, "bf16")
    announce("ulysses full size: running head group 5")
    out, lse = ra.ulysses_fwd(qg, kg, vg, head_group=5, causal=True, layout="striped")
    torch.cuda.synchronize()
    heads = slice(20, 24)
    for j in (0, 7):
        rows = full_size_rows(L, 205 + j)
        announce(f"ulysses full size: oracle, shard {j}, {rows.size} rows")
        inp = {"q": q[j][:, :, heads], "k_all": k[:, :, :, 5:6], "v_all": v[:, :, :, 5:6]}
        O, LSE = oracle_ring_rows(inp, N=N, shard=j, layout="striped", causal=True, rows=rows)
        idx = torch.from_numpy(rows).cuda()
        check_bf16(out[j][:, idx][:, :, heads], lse[j][:, heads][:, :, idx], O, LSE,
                   f"ulysses full size shard {j} {rows.size} rows")


def _dout_all(*, b, L, h, d, N, seed):
    return np.stack([synth.normal((b, L, h, d), seed=seed, name="do", shard=j) for j in range(N)])


@pytest.mark.parametrize("layout,causal", [("contiguous", False), ("contiguous", True), ("striped", True),
                                           ("zigzag", True)])
def test_ulysses_bwd_every_shard(layout, causal):
    """Every head group's backward fills dQ of every shard and dK, dV of every KV shard; each
    must equal the exact gradients (the forward's O and LSE come from the same scheme)."""
    from test_gpu_bwd import check_grad
    from oracle import shard_grads
    cfg = dict(b=1, L=100, h=8, n_kv=4, d=128, N=4)
    announce("ulysses bwd", layout, "causal", causal, cfg)
    q, k, v = all_shards(**cfg, seed=211, dtype="bf16")
    do = _dout_all(b=1, L=100, h=8, d=128, N=4, seed=211)
    qg, kg, vg, dog = (to_gpu(x, "bf16") for x in (q, k, v, do))
    o, lse = run_all_groups(qg, kg, vg, N=4, causal=causal, layout=layout)
    out = None
    for g in range(4):
        out = ra.ulysses_bwd(qg, kg, vg, o, dog, lse, head_group=g, causal=causal, layout=layout, out=out)
    torch.cuda.synchronize()
    dq, dk, dv = out
    x = [a.astype(np.float64) for a in (q, k, v, do)]
    rdk, rdv = np.zeros(k.shape), np.zeros(v.shape)
    for i in range(4):
        rq, rk, rv = shard_grads(x[0][i], x[1], x[2], x[3][i], N=4, shard=i, layout=layout, causal=causal)
        check_grad(dq[i], rq, f"ulysses dq shard {i} {layout} {causal}")
        rdk += rk
        rdv += rv
    for j in range(4):
        check_grad(dk[j], rdk[j], f"ulysses dk shard {j} {layout} {causal}")
        check_grad(dv[j], rdv[j], f"ulysses dv shard {j} {layout} {causal}")


@pytest.mark.timeout(900)
def test_ulysses_bwd_full_size():
    """S = 65536 (N = 8, L = 8192, h = 32, n_kv = 8, d = 128, bf16), striped causal, head group
    2 (query heads 8..11, KV head 2): dK, dV of 144 keys spread over all 8 KV shards and dQ of
    ~300 sampled rows of three shards against the oracle, element by element."""
    from test_gpu_bwd import check_grad, oracle_dq_rows
    from gpu_helpers import (BWD_FULL, BWD_FULL_KV_HEAD, bwd_full_cols, bwd_full_inputs, bwd_full_key_grads,
                             full_size_rows, gather_cols)
    N, L, grp = BWD_FULL["N"], BWD_FULL["L"], BWD_FULL_KV_HEAD
    hs = slice(4 * grp, 4 * grp + 4)
    announce("ulysses bwd full size: inputs")
    q, do, k, v = bwd_full_inputs()
    qg, kg, vg, dog = (to_gpu(x, "bf16") for x in (q, k, v, do))
    announce("ulysses bwd full size: forward and backward of head group 2")
    o, lse = ra.ulysses_fwd(qg, kg, vg, head_group=grp, causal=True, layout="striped")
    dq, dk, dv = ra.ulysses_bwd(qg, kg, vg, o, dog, lse, head_group=grp, causal=True, layout="striped")
    torch.cuda.synchronize()
    cols = bwd_full_cols()
    announce(f"ulysses bwd full size: oracle dK, dV of {len(cols)} keys from every query shard")
    rdk, rdv = bwd_full_key_grads(list(range(N)))
    check_grad(gather_cols(dk, cols, grp), rdk, "full size dk sampled keys")
    check_grad(gather_cols(dv, cols, grp), rdv, "full size dv sampled keys")
    x = [a.astype(np.float64) for a in (q, k, v, do)]
    for i in (0, 3, 7):
        rows = full_size_rows(L, 7007 + i)
        announce(f"ulysses bwd full size: oracle dQ of {rows.size} rows of shard {i}")
        ref = oracle_dq_rows(x[0][i][:, :, hs], x[1][:, :, :, grp:grp + 1], x[2][:, :, :, grp:grp + 1],
                             x[3][i][:, :, hs], rows, N=N, shard=i, layout="striped", causal=True)
        check_grad(dq[i][:, torch.from_numpy(rows).cuda()][:, :, hs], ref, f"full size dq rows shard {i}")


@pytest.mark.parametrize("cfg", [dict(b=1, L=130, h=4, n_kv=2, d=128, N=1),     # no exchange at all
                                 dict(b=2, L=64, h=4, n_kv=4, d=128, N=4)])     # one query and one KV head each
def test_ulysses_edge_shapes(cfg):
    N = cfg["N"]
    announce("ulysses edge", cfg)
    q, k, v = all_shards(**cfg, seed=221, dtype="bf16")
    out, lse = run_all_groups(to_gpu(q, "bf16"), to_gpu(k, "bf16"), to_gpu(v, "bf16"), N=N, causal=True,
                              layout="zigzag")
    x = [a.astype(np.float64) for a in (q, k, v)]
    for j in range(N):
        O, LSE = shard_attention(x[0][j], x[1], x[2], N=N, shard=j, layout="zigzag", causal=True)
        check_bf16(out[j], lse[j], O, LSE, f"ulysses edge shard {j}")

"""GPU parity of the two-dimensional arrangement (page 3, sections 7 and 8: heads and sequence
cut together; a device holds S/N_s tokens of h/N_h heads during attention) against the fp64
oracle.  One call per (head group, ring rank) fills the outputs of every device; each device's
rows must equal the oracle's attention of its queries, at the global positions usp_tokens
gives them, over every key of the sequence."""
import numpy as np
import pytest
import torch

import ring_attention_long_amd as ra
import synth
from gpu_helpers import announce, check_bf16, check_f32, full_size_rows, run_threads, to_gpu
from oracle import LAYOUTS, attention_over_shards, usp_tokens

pytestmark = pytest.mark.gpu


def all_devices(*, b, L, h, n_kv, d, N, seed, dtype):
    q = np.stack([synth.normal((b, L, h, d), seed=seed, name="q", shard=j, dtype=dtype) for j in range(N)])
    k = np.stack([synth.normal((b, L, n_kv, d), seed=seed, name="k", shard=j, dtype=dtype) for j in range(N)])
    v = np.stack([synth.normal((b, L, n_kv, d), seed=seed, name="v", shard=j, dtype=dtype) for j in range(N)])
    return q, k, v


def run_every_share(qg, kg, vg, *, N_h, causal, layout):
    N = qg.shape[0]
    out = lse = None
    for r in range(N // N_h):
        for g in range(N_h):
            out, lse = ra.usp_fwd(qg, kg, vg, n_head_groups=N_h, head_group=g, ring_rank=r, causal=causal,
                                  layout=layout, out=out, lse_out=lse)
    torch.cuda.synchronize()
    return out, lse


def oracle_device(q, k, v, *, j, N_h, N_s, layout, causal, rows=None):
    """Device j's queries against every key of the sequence, by global position."""
    L = q.shape[2]
    toks = usp_tokens(layout, N_h, N_s, L)
    k_cat = np.concatenate([k[i] for i in range(N_h * N_s)], axis=1)
    v_cat = np.concatenate([v[i] for i in range(N_h * N_s)], axis=1)
    return attention_over_shards(q[j], k_cat, v_cat, toks[j], np.concatenate(toks), causal=causal, rows=rows)


@pytest.mark.parametrize("layout,causal", [("contiguous", False), ("contiguous", True), ("striped", True),
                                           ("zigzag", True)])
@pytest.mark.parametrize("N_h,N_s", [(2, 2), (2, 3), (4, 1), (1, 4)])
def test_usp_bf16_every_device(layout, causal, N_h, N_s):
    cfg = dict(b=2, L=100, h=8, n_kv=4, d=128, N=N_h * N_s)     # ring shards of 100 N_h tokens, ragged tiles
    announce("usp bf16", layout, "causal", causal, "N_h", N_h, "N_s", N_s, cfg)
    q, k, v = all_devices(**cfg, seed=401, dtype="bf16")
    out, lse = run_every_share(to_gpu(q, "bf16"), to_gpu(k, "bf16"), to_gpu(v, "bf16"), N_h=N_h, causal=causal,
                               layout=layout)
    x = [a.astype(np.float64) for a in (q, k, v)]
    for j in range(cfg["N"]):
        O, LSE = oracle_device(*x, j=j, N_h=N_h, N_s=N_s, layout=layout, causal=causal)
        check_bf16(out[j], lse[j], O, LSE, f"usp {layout} {causal} {N_h}x{N_s} device {j}")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_usp_f32_every_device(layout):
    cfg = dict(b=1, L=40, h=4, n_kv=2, d=64, N=4)
    announce("usp f32", layout, cfg)
    q, k, v = all_devices(**cfg, seed=402, dtype="f32")
    out, lse = run_every_share(to_gpu(q, "f32"), to_gpu(k, "f32"), to_gpu(v, "f32"), N_h=2, causal=True,
                               layout=layout)
    x = [a.astype(np.float64) for a in (q, k, v)]
    for j in range(4):
        O, LSE = oracle_device(*x, j=j, N_h=2, N_s=2, layout=layout, causal=True)
        check_f32(out[j], lse[j], O, LSE, f"usp f32 {layout} device {j}")


def test_usp_limits_equal_the_ring_and_the_all_to_all_path():
    """N_h = 1 is the ring (ra_ring_fwd of every shard, one launch per ring step as the
    two-dimensional share runs its ring) and N_s = 1 the all-to-all path (ra_ulysses_fwd of
    every head group), bit for bit: the same kernels on the same problems."""
    cfg = dict(b=1, L=192, h=8, n_kv=4, d=128, N=4)
    q, k, v = all_devices(**cfg, seed=403, dtype="bf16")
    qg, kg, vg = to_gpu(q, "bf16"), to_gpu(k, "bf16"), to_gpu(v, "bf16")
    announce("usp limits: N_h = 1 vs ring, N_s = 1 vs all-to-all")
    out, lse = run_every_share(qg, kg, vg, N_h=1, causal=True, layout="zigzag")
    for j in range(4):
        o_r, l_r = ra.ring_fwd(qg[j].contiguous(), kg, vg, q_shard=j, causal=True, layout="zigzag",
                               steps_per_launch=1)
        torch.cuda.synchronize()
        assert torch.equal(out[j], o_r) and torch.equal(lse[j], l_r)
    out, lse = run_every_share(qg, kg, vg, N_h=4, causal=True, layout="striped")
    uo = ul = None
    for g in range(4):
        uo, ul = ra.ulysses_fwd(qg, kg, vg, head_group=g, causal=True, layout="contiguous", out=uo, lse_out=ul)
    torch.cuda.synchronize()
    assert torch.equal(out, uo) and torch.equal(lse, ul)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("N_h,N_s", [(2, 4), (4, 2)])
def test_usp_full_size_sampled(N_h, N_s):
    """S = 262144 (N = 8 devices of L = 32768, h = 32, n_kv = 8, d = 128, bf16), striped causal
    over the ring shards: device (1, N_s - 1)'s share, ~300 sampled rows of each of its ring
    shard's devices (its head group's heads) against the oracle."""
    N, L, h, n_kv, d = 8, 32768, 32, 8, 128
    announce(f"usp full size {N_h}x{N_s}: inputs")
    q, k, v = all_devices(b=1, L=L, h=h, n_kv=n_kv, d=d, N=N, seed=404, dtype="bf16")
    qg, kg, vg = to_gpu(q, "bf16"), to_gpu(k, "bf16"), to_gpu(v, "bf16")
    g, r = 1, N_s - 1
    announce(f"usp full size {N_h}x{N_s}: share of head group {g}, ring rank {r}")
    out, lse = ra.usp_fwd(qg, kg, vg, n_head_groups=N_h, head_group=g, ring_rank=r, causal=True, layout="striped")
    torch.cuda.synchronize()
    Hg, Kg = h // N_h, n_kv // N_h
    hs, ks = slice(g * Hg, (g + 1) * Hg), slice(g * Kg, (g + 1) * Kg)
    toks = usp_tokens("striped", N_h, N_s, L)
    pos_k = np.concatenate(toks)
    k_cat = np.concatenate([k[i][:, :, ks] for i in range(N)], axis=1).astype(np.float64)
    v_cat = np.concatenate([v[i][:, :, ks] for i in range(N)], axis=1).astype(np.float64)
    k_cat = np.ascontiguousarray(k_cat.transpose(0, 2, 1, 3)).transpose(0, 2, 1, 3)
    v_cat = np.ascontiguousarray(v_cat.transpose(0, 2, 1, 3)).transpose(0, 2, 1, 3)
    for j in range(r * N_h, (r + 1) * N_h):
        rows = full_size_rows(L, 404 + j)
        announce(f"usp full size {N_h}x{N_s}: oracle, device {j}, {rows.size} rows")
        qj = q[j][:, :, hs].astype(np.float64)
        G = Hg // Kg
        chunks = np.array_split(rows, max(1, rows.size // 160))
        jobs = [(hq, c) for hq in range(Hg) for c in chunks]
        res = run_threads(lambda job: attention_over_shards(
            qj[:, :, job[0]:job[0] + 1], k_cat[:, :, job[0] // G:job[0] // G + 1],
            v_cat[:, :, job[0] // G:job[0] // G + 1], toks[j], pos_k, causal=True, rows=job[1]), jobs)
        O = np.zeros((1, rows.size, Hg, d))
        LSE = np.zeros((1, Hg, rows.size))
        for (hq, c), (o_, l_) in zip(jobs, res):
            r0 = int(np.searchsorted(rows, c[0]))
            O[:, r0:r0 + c.size, hq] = o_[:, :, 0]
            LSE[:, hq, r0:r0 + c.size] = l_[:, 0]
        idx = torch.from_numpy(rows).cuda()
        check_bf16(out[j][:, idx][:, :, hs], lse[j][:, hs][:, :, idx], O, LSE,
                   f"usp full size {N_h}x{N_s} device {j}")

"""Shared helpers of the GPU parity tests: seeded inputs on the device, the oracle on the
same values, and the tolerance checks."""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch
from threadpoolctl import threadpool_limits

import synth
from oracle import attention_over_shards, key_grads, shard_attention, shard_tokens, step_attention

# Tolerances: fp32 path norm-wise relative 1e-5; bf16 inputs with fp32 accumulation
# max abs 2e-2 and mean abs 2e-3 on the output, LSE abs 1e-3.
F32_REL = 1e-5
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
LSE_ABS = 1e-3


def announce(*parts):
    print("[gpu-case]", *parts, flush=True)
    sys.stdout.flush()


def torch_dtype(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def make_inputs(*, b, L, h, n_kv, d, N, q_shard, seed, dtype, with_dout=False):
    return synth.shard_inputs(b=b, L=L, h=h, n_kv=n_kv, d=d, N=N, q_shard=q_shard, seed=seed,
                              dtype=dtype, with_dout=with_dout)


def to_gpu(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=torch_dtype(dtype))


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def check_f32(o, lse, O_ref, LSE_ref, what=""):
    """Norm-wise relative error: max |o - ref| / max |ref| <= 1e-5 for O and for LSE
    (rows with LSE = -inf must match exactly).  The element-wise relative error
    |o - ref| / (|ref| + 1e-3) and the largest absolute error are reported beside it."""
    o, lse = f64(o), f64(lse)
    fin = np.isfinite(LSE_ref)
    assert np.array_equal(np.isfinite(lse), fin), f"{what}: -inf rows differ"
    eo = np.max(np.abs(o - O_ref)) / max(np.max(np.abs(O_ref)), 1e-30)
    el = np.max(np.abs(lse[fin] - LSE_ref[fin])) / max(np.max(np.abs(LSE_ref[fin])), 1e-30) if fin.any() else 0.0
    ew = np.max(np.abs(o - O_ref) / (np.abs(O_ref) + 1e-3))
    announce(f"{what} f32 rel err O={eo:.3e} LSE={el:.3e}; element-wise O={ew:.3e}, "
             f"max abs O={np.max(np.abs(o - O_ref)):.3e}")
    assert eo <= F32_REL, f"{what}: O rel err {eo}"
    assert el <= F32_REL, f"{what}: LSE rel err {el}"
    assert np.all(o[~np.broadcast_to(np.transpose(fin, (0, 2, 1))[..., None], o.shape)] == 0)


def check_bf16(o, lse, O_ref, LSE_ref, what=""):
    o, lse = f64(o), f64(lse)
    fin = np.isfinite(LSE_ref)
    assert np.array_equal(np.isfinite(lse), fin), f"{what}: -inf rows differ"
    err = np.abs(o - O_ref)
    el = np.max(np.abs(lse[fin] - LSE_ref[fin])) if fin.any() else 0.0
    announce(f"{what} bf16 max abs {err.max():.3e} mean abs {err.mean():.3e} LSE abs {el:.3e}")
    assert err.max() <= BF16_MAX_ABS, f"{what}: max abs err {err.max()}"
    assert err.mean() <= BF16_MEAN_ABS, f"{what}: mean abs err {err.mean()}"
    assert el <= LSE_ABS, f"{what}: LSE abs err {el}"


def oracle_ring(inp, *, N, shard, layout, causal, rows=None):
    q = inp["q"].astype(np.float64)
    return shard_attention(q, inp["k_all"].astype(np.float64), inp["v_all"].astype(np.float64),
                           N=N, shard=shard, layout=layout, causal=causal, rows=rows)


def oracle_step(inp, *, N, q_shard, kv_shard, layout, causal):
    return step_attention(inp["q"].astype(np.float64), inp["k_all"][kv_shard].astype(np.float64),
                          inp["v_all"][kv_shard].astype(np.float64), N=N, q_shard=q_shard,
                          kv_shard=kv_shard, layout=layout, causal=causal)


def prefix_means_global(v_all, layout, N):
    """For Q = 0 (uniform weights): mean over keys at global positions <= P for every P,
    in fp64 from the per-shard values.  Returns ([b, S, n_kv, d] prefix means, positions)."""
    L = v_all.shape[2]
    toks = shard_tokens(layout, N, L)
    S = N * L
    g = np.zeros((v_all.shape[1], S) + v_all.shape[3:])
    for j in range(N):
        g[:, toks[j]] = v_all[j]
    cs = np.cumsum(g, axis=1)
    cnt = np.arange(1, S + 1, dtype=np.float64)
    return cs / cnt[None, :, None, None], toks


# ------------------------------------------------------------------ oracle on many rows
def oracle_threads():
    """Worker threads for the oracle: the host's cores (at most 16, the share of one GPU)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def run_threads(fn, jobs):
    """fn over jobs on oracle_threads() threads, BLAS single-threaded inside each (numpy
    releases the GIL in its array work, so the threads run in parallel)."""
    with threadpool_limits(1):
        with ThreadPoolExecutor(oracle_threads()) as ex:
            return list(ex.map(fn, jobs))


def full_size_rows(L, seed, n_random=160):
    """Query rows compared at full size (>= 256): the first and last 32 (the lightest and
    heaviest causal work), rows at every position class of a 64-row tile and of its 32-row
    halves (0, 1, 31, 32, 62, 63) in twelve tiles spread over the shard, sixteen rows around
    the half-shard boundary (zigzag's chunk edge), and seeded random rows."""
    rows = set(range(min(32, L))) | set(range(max(0, L - 32), L))
    for t in np.linspace(0, max(0, L // 64 - 1), 12).astype(int):
        rows |= {64 * int(t) + c for c in (0, 1, 31, 32, 62, 63)}
    rows |= set(range(max(0, L // 2 - 8), min(L, L // 2 + 8)))
    rows |= set(np.random.default_rng(seed).integers(0, L, n_random).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < L), dtype=np.int64)


def _heads_contiguous(x):
    """[b, S, n, d] array whose [bi, :, g, :] slices are contiguous (one copy up front)."""
    return np.ascontiguousarray(np.transpose(x, (0, 2, 1, 3))).transpose(0, 2, 1, 3)


def oracle_ring_rows(inp, *, N, shard, layout, causal, rows, q=None, docs=None):
    """shard_attention for the given query rows, spread over threads: the shards' keys and
    values are concatenated once and shared by every thread.  `docs`: packed-document
    bounds (one packing for the whole batch)."""
    q = (inp["q"] if q is None else q).astype(np.float64)
    L = q.shape[1]
    toks = shard_tokens(layout, N, L)
    k_cat = _heads_contiguous(np.concatenate([inp["k_all"][j] for j in range(N)], axis=1).astype(np.float64))
    v_cat = _heads_contiguous(np.concatenate([inp["v_all"][j] for j in range(N)], axis=1).astype(np.float64))
    pos_k = np.concatenate(toks)
    rows = np.asarray(rows, dtype=np.int64)
    h, G = q.shape[2], q.shape[2] // k_cat.shape[2]
    # one job = one query head and a tall block of rows (each job streams its KV head once)
    chunks = np.array_split(rows, max(1, rows.size // 160))
    jobs = [(hq, rr) for hq in range(h) for rr in chunks]

    def one(job):
        hq, rr = job
        g = hq // G
        return attention_over_shards(q[:, :, hq:hq + 1], k_cat[:, :, g:g + 1], v_cat[:, :, g:g + 1],
                                     toks[shard], pos_k, causal=causal, rows=rr, docs=docs)
    res = run_threads(one, jobs)
    O = np.zeros((q.shape[0], rows.size, h, q.shape[3]))
    LSE = np.zeros((q.shape[0], h, rows.size))
    at = {id(c): (int(np.searchsorted(rows, c[0])) if c.size else 0) for c in chunks}
    for (hq, rr), (o, l) in zip(jobs, res):
        r0 = at[id(rr)]
        O[:, r0:r0 + rr.size, hq] = o[:, :, 0]
        LSE[:, hq, r0:r0 + rr.size] = l[:, 0]
    return O, LSE


# ------------------------------------------------------------------ full-size backward
# Every full-size backward test (the rotating ring, the key/value-stationary schedule and the
# all-to-all path) uses the same inputs, S = 65536 striped causal with h = 32, n_kv = 8,
# d = 128, so that the oracle's key gradients, which need every row's softmax over the whole
# sequence, are computed once per query shard and shared.
BWD_FULL = dict(b=1, L=8192, h=32, n_kv=8, d=128, N=8)
BWD_FULL_SEED = 1005
BWD_FULL_KV_HEAD = 2                       # head group 2 of the all-to-all path (N = 8)


def bwd_full_inputs():
    """q, dout [N, b, L, h, d], k, v [N, b, L, n_kv, d] (float32 holding bf16 values): the same
    streams as synth.shard_inputs, so shard i's slice is its make_inputs(q_shard=i)."""
    c, s = BWD_FULL, BWD_FULL_SEED
    q = np.stack([synth.normal((c["b"], c["L"], c["h"], c["d"]), seed=s, name="q", shard=j) for j in range(c["N"])])
    do = np.stack([synth.normal((c["b"], c["L"], c["h"], c["d"]), seed=s, name="do", shard=j) for j in range(c["N"])])
    k = np.stack([synth.normal((c["b"], c["L"], c["n_kv"], c["d"]), seed=s, name="k", shard=j) for j in range(c["N"])])
    v = np.stack([synth.normal((c["b"], c["L"], c["n_kv"], c["d"]), seed=s, name="v", shard=j) for j in range(c["N"])])
    return q, do, k, v


def bwd_full_cols():
    """Keys whose dK, dV are compared, as (KV shard, local index): in every shard the first
    and last keys, both sides of 32-, 64- and 128-key tile edges and of the half-shard, and
    seeded random keys."""
    L, N = BWD_FULL["L"], BWD_FULL["N"]
    rng = np.random.default_rng(4242)
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, L // 2 - 1, L // 2, L - 2, L - 1]
    return [(j, int(u)) for j in range(N) for u in sorted(set(fixed) | set(rng.integers(0, L, 6).tolist()))]


_KEY_GRADS_CACHE = {}


def bwd_full_key_grads(shards):
    """The oracle's dK, dV [b, C, d] of bwd_full_cols() for KV head BWD_FULL_KV_HEAD from each
    query shard in `shards` (each computed once per session, rows spread over threads)."""
    todo = [i for i in shards if i not in _KEY_GRADS_CACHE]
    if todo:
        q, do, k, v = (x.astype(np.float64) for x in bwd_full_inputs())
        cols = bwd_full_cols()
        L = BWD_FULL["L"]
        parts = np.array_split(np.arange(L), 2 * oracle_threads())
        jobs = [(i, rr) for i in todo for rr in parts]
        res = run_threads(lambda job: key_grads(q[job[0]:job[0] + 1], do[job[0]:job[0] + 1], k, v, N=BWD_FULL["N"],
                                                query_shards=[job[0]], kv_head=BWD_FULL_KV_HEAD, cols=cols,
                                                layout="striped", causal=True, rows=job[1]), jobs)
        for i in todo:
            mine = [r for (j, _), r in zip(jobs, res) if j == i]
            _KEY_GRADS_CACHE[i] = (sum(r[0] for r in mine), sum(r[1] for r in mine))
    return (sum(_KEY_GRADS_CACHE[i][0] for i in shards), sum(_KEY_GRADS_CACHE[i][1] for i in shards))


def gather_cols(t, cols, kv_head):
    """t [N, b, L, n_kv, d] (device tensor) -> [b, C, d] float64 of the listed keys."""
    j = torch.as_tensor([c[0] for c in cols], device=t.device)
    u = torch.as_tensor([c[1] for c in cols], device=t.device)
    return f64(t[j, :, u, kv_head].permute(1, 0, 2))

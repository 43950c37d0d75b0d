"""Shared helpers of the GPU parity tests: seeded inputs on the device, the oracle on the
same values, and the tolerance checks."""
import sys

import numpy as np
import torch

import synth
from oracle import shard_attention, shard_tokens, step_attention

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
    (rows with LSE = -inf must match exactly)."""
    o, lse = f64(o), f64(lse)
    fin = np.isfinite(LSE_ref)
    assert np.array_equal(np.isfinite(lse), fin), f"{what}: -inf rows differ"
    eo = np.max(np.abs(o - O_ref)) / max(np.max(np.abs(O_ref)), 1e-30)
    el = np.max(np.abs(lse[fin] - LSE_ref[fin])) / max(np.max(np.abs(LSE_ref[fin])), 1e-30) if fin.any() else 0.0
    announce(f"{what} f32 rel err O={eo:.3e} LSE={el:.3e}")
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

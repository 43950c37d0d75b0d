"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws iid standard-normal numbers and rounds them to the storage dtype.  It
holds none of the attention method's arithmetic (no positions, masks, softmax or
merging), so both the HIP path and the oracle may consume what it produces.

Every tensor is drawn from its own numpy PCG64 stream keyed by (seed, tensor name, shard),
so a single shard's tensor can be generated without drawing the others.  bf16 values are
produced by round-to-nearest-even of the fp32 draw and returned as float32 arrays holding
bf16-exact values: converting them to torch.bfloat16 (GPU side) or float64 (oracle side)
is exact.
"""
from __future__ import annotations

import numpy as np

_TENSOR_IDS = {"q": 1, "k": 2, "v": 3, "do": 4}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def normal(shape, *, seed: int, name: str, shard: int = 0, dtype: str = "bf16",
           scale: float = 1.0) -> np.ndarray:
    """iid N(0, 1) (times `scale`) of `shape`, rounded to `dtype` ('bf16' or 'f32')."""
    rng = np.random.default_rng([int(seed), _TENSOR_IDS[name], int(shard)])
    x = rng.standard_normal(size=tuple(shape), dtype=np.float32)
    if scale != 1.0:
        x = (x * np.float32(scale)).astype(np.float32)
    if dtype == "bf16":
        return round_to_bf16(x)
    if dtype == "f32":
        return x
    raise ValueError(f"unknown dtype {dtype!r}")


def shard_inputs(*, b, L, h, n_kv, d, N, q_shard, seed, dtype="bf16", with_dout=False):
    """Inputs of one device's ring pass.

    Returns dict with q [b, L, h, d] (shard q_shard's queries), k_all and v_all
    [N, b, L, n_kv, d] (every shard's keys and values in that shard's local order) and,
    if asked, dout [b, L, h, d].  All float32 numpy arrays holding `dtype`-exact values.
    """
    out = {
        "q": normal((b, L, h, d), seed=seed, name="q", shard=q_shard, dtype=dtype),
        "k_all": np.stack([normal((b, L, n_kv, d), seed=seed, name="k", shard=j, dtype=dtype)
                           for j in range(N)]),
        "v_all": np.stack([normal((b, L, n_kv, d), seed=seed, name="v", shard=j, dtype=dtype)
                           for j in range(N)]),
    }
    if with_dout:
        out["dout"] = normal((b, L, h, d), seed=seed, name="do", shard=q_shard, dtype=dtype)
    return out


def document_bounds(S: int, *, seed: int, mean_len: float, min_len: int = 1,
                    max_len: int | None = None) -> np.ndarray:
    """Packed-window document boundaries [0, b_1, ..., S] (int64): lengths drawn from a
    seeded lognormal with the given mean (sigma 1, a heavy-tailed mix of short and long
    documents), clipped to [min_len, max_len], the last document cut at the window end."""
    rng = np.random.default_rng([seed, 7])
    hi = S if max_len is None else max_len
    sigma = 1.0
    mu = np.log(max(mean_len, 1.0)) - sigma * sigma / 2
    bounds = [0]
    while bounds[-1] < S:
        n = int(np.clip(round(rng.lognormal(mu, sigma)), min_len, hi))
        bounds.append(min(S, bounds[-1] + n))
    return np.asarray(bounds, dtype=np.int64)

"""Seeded random configurations of the ring forward (bf16 and fp32) and backward (bf16),
each compared with the oracle element by element.  They pair up what the targeted tests
keep apart: ragged L in every layout, GQA groups of 1 to 6 query heads, rings of 2 to 12
shards, packed documents, each choice of ring steps per launch, batch rows.  The draws come
from fixed seeds, so every run checks the same cases; each case is printed before it runs."""
import numpy as np
import pytest
import torch

import ring_attention_long_amd as ra
import synth
from gpu_helpers import announce, check_bf16, check_f32, f64, make_inputs, oracle_ring, oracle_ring_rows, to_gpu
from oracle import shard_grads

pytestmark = pytest.mark.gpu

HEADS = [(8, 2), (4, 4), (6, 2), (12, 4), (3, 1), (6, 1)]
LAYOUTS = ["contiguous", "striped", "zigzag"]


def _draw(n, seed, *, docs_prob, max_L):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        h, n_kv = HEADS[rng.integers(len(HEADS))]
        layout = LAYOUTS[rng.integers(len(LAYOUTS))]
        L = int(rng.integers(33, max_L))
        L += L % 2 if layout == "zigzag" else 0
        N = int(rng.integers(2, 13))
        docs = bool(rng.random() < docs_prob)
        out.append(dict(b=1 if docs else int(rng.integers(1, 3)), L=L, h=h, n_kv=n_kv, N=N, layout=layout,
                        causal=bool(rng.random() < 0.75), shard=int(rng.integers(N)),
                        spl=int(rng.choice([0, 1, 2, 3])), docs=docs,
                        mean_doc=int(rng.integers(24, 3 * L)), seed=int(rng.integers(1 << 30))))
    return out


FWD = _draw(64, 2024, docs_prob=0.3, max_L=420)
BWD = _draw(24, 2025, docs_prob=0.3, max_L=260)


def _docs(c):
    """(GPU row bounds for the library, global document bounds for the oracle), or Nones."""
    if not c["docs"]:
        return None, None
    bounds = synth.document_bounds(c["N"] * c["L"], seed=c["seed"], mean_len=c["mean_doc"]).astype(np.int32)
    db, de = ra.document_ranges(bounds, N=c["N"], L=c["L"], shard=c["shard"], layout=c["layout"])
    return (torch.from_numpy(db[None]).cuda(), torch.from_numpy(de[None]).cuda()), bounds


def _inputs(c, dtype, d=128, with_dout=False):
    return make_inputs(b=c["b"], L=c["L"], h=c["h"], n_kv=c["n_kv"], d=d, N=c["N"], q_shard=c["shard"],
                       seed=c["seed"], dtype=dtype, with_dout=with_dout)


@pytest.mark.parametrize("i", range(len(FWD)))
def test_random_forward_bf16(i):
    c = FWD[i]
    announce("random bf16 forward", i, c)
    inp = _inputs(c, "bf16")
    q, k_all, v_all = (to_gpu(inp[x], "bf16") for x in ("q", "k_all", "v_all"))
    docs, bounds = _docs(c)
    o, lse = ra.ring_fwd(q, k_all, v_all, q_shard=c["shard"], causal=c["causal"], layout=c["layout"], docs=docs,
                         steps_per_launch=c["spl"])
    torch.cuda.synchronize()
    if bounds is None:
        O, LSE = oracle_ring(inp, N=c["N"], shard=c["shard"], layout=c["layout"], causal=c["causal"])
    else:
        O, LSE = oracle_ring_rows(inp, N=c["N"], shard=c["shard"], layout=c["layout"], causal=c["causal"],
                                  rows=np.arange(c["L"]), docs=bounds)
    check_bf16(o, lse, O, LSE, f"random bf16 forward {i}")


@pytest.mark.parametrize("i", range(16))
def test_random_forward_f32(i):
    c = dict(FWD[i], docs=False)
    d = 64 if i % 2 else 128
    announce("random fp32 forward", i, c, "d", d)
    inp = _inputs(c, "f32", d=d)
    q, k_all, v_all = (to_gpu(inp[x], "f32") for x in ("q", "k_all", "v_all"))
    o, lse = ra.ring_fwd(q, k_all, v_all, q_shard=c["shard"], causal=c["causal"], layout=c["layout"])
    torch.cuda.synchronize()
    O, LSE = oracle_ring(inp, N=c["N"], shard=c["shard"], layout=c["layout"], causal=c["causal"])
    check_f32(o, lse, O, LSE, f"random fp32 forward {i}")


def _check_grad(got, ref, what):
    """The backward tolerance of the targeted tests: max abs error <= 2e-2 * max(1, rms(ref)),
    mean abs error <= 2e-3 * max(1, rms(ref))."""
    got = f64(got)
    scale = max(1.0, float(np.sqrt(np.mean(ref ** 2))))
    err = np.abs(got - ref)
    announce(f"{what}: max abs {err.max():.3e} mean abs {err.mean():.3e} (rms ref {scale:.3f})")
    assert err.max() <= 2e-2 * scale, what
    assert err.mean() <= 2e-3 * scale, what


@pytest.mark.parametrize("i", range(len(BWD)))
def test_random_backward(i):
    c = BWD[i]
    announce("random backward", i, c)
    inp = _inputs(c, "bf16", with_dout=True)
    q, k_all, v_all, dout = (to_gpu(inp[x], "bf16") for x in ("q", "k_all", "v_all", "dout"))
    docs, bounds = _docs(c)
    kw = dict(q_shard=c["shard"], causal=c["causal"], layout=c["layout"], docs=docs)
    o, lse = ra.ring_fwd(q, k_all, v_all, steps_per_launch=c["spl"], **kw)
    dq, dk, dv = ra.ring_bwd(q, k_all, v_all, o, dout, lse, **kw)
    torch.cuda.synchronize()
    x = {k_: inp[k_].astype(np.float64) for k_ in ("q", "k_all", "v_all", "dout")}
    rdq, rdk, rdv = shard_grads(x["q"], x["k_all"], x["v_all"], x["dout"], N=c["N"], shard=c["shard"],
                                layout=c["layout"], causal=c["causal"], docs=bounds)
    for got, ref, name in ((dq, rdq, "dq"), (dk, rdk, "dk"), (dv, rdv, "dv")):
        _check_grad(got, ref, f"random backward {i} {name}")

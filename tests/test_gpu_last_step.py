"""The last live step of a bf16 forward pass writes the output itself: its epilogue casts the
merged rows to bf16 (and copies over, cast, the rows the step leaves alone) instead of
writing the fp32 accumulator for a separate finalize pass.  The cases below run without the
second accumulator (base workspace), so every pass ends this way, and reach each of the
epilogue's paths:

* contiguous causal shard 0: one live step, so the first step (partial epilogue) is the last;
* contiguous causal shards 1 and 2 of 4: the last live step is not the last ring step;
* striped and zigzag shard 0: the last step's KV shard comes after the query shard, so row 0
  (and with zigzag a whole chunk of workgroups) sees no key in it;
* ragged L: rows past the shard end in the last query block;
* packed documents: many workgroups of the last step have no key tile at all.

Every element is compared with the oracle."""
import numpy as np
import pytest
import torch

import ring_attention_long_amd as ra
import synth
from gpu_helpers import announce, check_bf16, make_inputs, oracle_ring, oracle_ring_rows, to_gpu

pytestmark = pytest.mark.gpu


def _al(x):
    return -(-x // 256) * 256


def base_workspace(b, L, h, n_kv, d):
    """ra_ring_fwd's workspace without the second accumulator (KV double buffer, fp32 acc)."""
    return torch.empty(4 * _al(b * L * n_kv * d * 2) + _al(b * L * h * d * 4), device="cuda", dtype=torch.uint8)


@pytest.mark.parametrize("layout,causal", [("contiguous", False), ("contiguous", True),
                                           ("striped", True), ("zigzag", True)])
def test_last_step_writes_output_every_shard(layout, causal):
    cfg = dict(b=2, L=330, h=8, n_kv=2, d=128, N=4)
    for shard in range(cfg["N"]):
        announce("last-step output", layout, "causal", causal, "shard", shard, cfg)
        inp = make_inputs(**cfg, q_shard=shard, seed=1300 + shard, dtype="bf16")
        q, k_all, v_all = (to_gpu(inp[x], "bf16") for x in ("q", "k_all", "v_all"))
        o, lse = ra.ring_fwd(q, k_all, v_all, q_shard=shard, causal=causal, layout=layout,
                             workspace=base_workspace(cfg["b"], cfg["L"], cfg["h"], cfg["n_kv"], cfg["d"]))
        torch.cuda.synchronize()
        O, LSE = oracle_ring(inp, N=cfg["N"], shard=shard, layout=layout, causal=causal)
        check_bf16(o, lse, O, LSE, f"{layout} causal={causal} shard {shard}")


def test_last_step_writes_output_long_tiles_single_step():
    """96-key tiles (L >= 16384), contiguous causal shard 0 of 2: the only live step writes
    the output from its partial epilogue."""
    cfg = dict(b=1, L=16448, h=4, n_kv=4, d=128, N=2)
    announce("last-step output, one live step", cfg)
    inp = make_inputs(**cfg, q_shard=0, seed=1310, dtype="bf16")
    q, k_all, v_all = (to_gpu(inp[x], "bf16") for x in ("q", "k_all", "v_all"))
    o, lse = ra.ring_fwd(q, k_all, v_all, q_shard=0, causal=True, layout="contiguous")
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, 200), np.arange(cfg["L"] - 200, cfg["L"]),
                                     np.random.default_rng(1311).integers(0, cfg["L"], 200)]))
    O, LSE = oracle_ring_rows(inp, N=2, shard=0, layout="contiguous", causal=True, rows=rows)
    ri = torch.from_numpy(rows).to(o.device)
    check_bf16(o[:, ri], lse[:, :, ri], O, LSE, "long tiles, one live step")


@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
def test_last_step_writes_output_packed_documents(layout):
    cfg = dict(b=1, L=640, h=8, n_kv=2, d=128, N=4)
    bounds = synth.document_bounds(cfg["N"] * cfg["L"], seed=1320, mean_len=300).astype(np.int32)
    for shard in (0, 3):
        announce("last-step output, packed", layout, "shard", shard, cfg)
        inp = make_inputs(**cfg, q_shard=shard, seed=1321 + shard, dtype="bf16")
        q, k_all, v_all = (to_gpu(inp[x], "bf16") for x in ("q", "k_all", "v_all"))
        db, de = ra.document_ranges(bounds, N=cfg["N"], L=cfg["L"], shard=shard, layout=layout)
        docs = (torch.from_numpy(db[None]).cuda(), torch.from_numpy(de[None]).cuda())
        o, lse = ra.ring_fwd(q, k_all, v_all, q_shard=shard, causal=True, layout=layout, docs=docs)
        torch.cuda.synchronize()
        O, LSE = oracle_ring_rows(inp, N=cfg["N"], shard=shard, layout=layout, causal=True,
                                  rows=np.arange(cfg["L"]), docs=bounds)
        check_bf16(o, lse, O, LSE, f"packed {layout} shard {shard}")

"""GPU parity with packed documents (page 3, section 5: documents packed end to end into one
window, a block-diagonal mask stopping attention across documents) against the fp64
oracle.  The kernels get per-row document bounds built by ra.document_ranges (itself
checked against the oracle on the CPU); the oracle gets the global document bounds."""
import numpy as np
import pytest
import torch

import ring_attention_long_amd as ra
import synth
from gpu_helpers import (announce, check_bf16, check_f32, f64, full_size_rows, make_inputs, oracle_ring_rows,
                         run_threads, to_gpu)
from oracle import LAYOUTS, key_grads, shard_attention, shard_dq_rows, shard_grads, shard_tokens, step_attention

pytestmark = pytest.mark.gpu

# S = 600 (N = 3, L = 200): one-token documents, documents inside one tile, documents
# crossing shards, a one-token document at the end
HAND = np.array([0, 1, 2, 66, 67, 130, 300, 301, 450, 599, 600], dtype=np.int32)


def gpu_docs(bounds_per_batch, *, N, L, shard, layout):
    rng = [ra.document_ranges(bd, N=N, L=L, shard=shard, layout=layout) for bd in bounds_per_batch]
    begin = torch.from_numpy(np.stack([r[0] for r in rng])).cuda()
    end = torch.from_numpy(np.stack([r[1] for r in rng])).cuda()
    return begin, end


def oracle_ring_docs(inp, bounds_per_batch, *, N, shard, layout, causal, rows=None):
    outs = [shard_attention(inp["q"][bi:bi + 1].astype(np.float64),
                            inp["k_all"][:, bi:bi + 1].astype(np.float64),
                            inp["v_all"][:, bi:bi + 1].astype(np.float64), N=N, shard=shard,
                            layout=layout, causal=causal, rows=rows, docs=bd)
            for bi, bd in enumerate(bounds_per_batch)]
    return np.concatenate([o[0] for o in outs]), np.concatenate([o[1] for o in outs])


def check_grad(got, ref, what):
    got = f64(got) if isinstance(got, torch.Tensor) else got
    scale = max(1.0, float(np.sqrt(np.mean(ref ** 2))))
    err = np.abs(got - ref)
    announce(f"{what}: max abs {err.max():.3e} mean abs {err.mean():.3e} (rms ref {scale:.3f})")
    assert err.max() <= 2e-2 * scale, what
    assert err.mean() <= 2e-3 * scale, what


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("causal", [True, False])
def test_ring_fwd_packed_small(layout, causal):
    cfg = dict(b=2, L=200, h=8, n_kv=2, d=128, N=3)
    bounds = [HAND, synth.document_bounds(600, seed=11, mean_len=40).astype(np.int32)]
    for shard in (0, 2):
        announce("packed ring_fwd", layout, "causal", causal, "shard", shard, cfg)
        inp = make_inputs(**cfg, q_shard=shard, seed=61 + shard, dtype="bf16")
        docs = gpu_docs(bounds, N=3, L=200, shard=shard, layout=layout)
        o, lse = ra.ring_fwd(to_gpu(inp["q"], "bf16"), to_gpu(inp["k_all"], "bf16"),
                             to_gpu(inp["v_all"], "bf16"), q_shard=shard, causal=causal,
                             layout=layout, docs=docs)
        torch.cuda.synchronize()
        O, LSE = oracle_ring_docs(inp, bounds, N=3, shard=shard, layout=layout, causal=causal)
        check_bf16(o, lse, O, LSE, f"packed ring {layout} {causal} shard {shard}")


@pytest.mark.parametrize("layout,causal", [("striped", True), ("zigzag", False), ("contiguous", True)])
def test_step_fwd_packed_every_pair(layout, causal):
    cfg = dict(b=1, L=200, h=4, n_kv=1, d=128, N=3)
    for qs in range(3):
        inp = make_inputs(**cfg, q_shard=qs, seed=71 + qs, dtype="bf16")
        q = to_gpu(inp["q"], "bf16")
        docs = gpu_docs([HAND], N=3, L=200, shard=qs, layout=layout)
        for kv in range(3):
            announce("packed step_fwd", layout, causal, "q", qs, "kv", kv)
            o, lse = ra.step_fwd(q, to_gpu(inp["k_all"][kv], "bf16"), to_gpu(inp["v_all"][kv], "bf16"),
                                 N=3, q_shard=qs, kv_shard=kv, causal=causal, layout=layout, docs=docs)
            torch.cuda.synchronize()
            O, LSE = step_attention(inp["q"].astype(np.float64), inp["k_all"][kv].astype(np.float64),
                                    inp["v_all"][kv].astype(np.float64), N=3, q_shard=qs,
                                    kv_shard=kv, layout=layout, causal=causal, docs=HAND)
            check_bf16(o, lse, O, LSE, f"packed step {layout} q{qs} kv{kv}")


@pytest.mark.parametrize("layout", ["contiguous", "striped"])
def test_ring_fwd_packed_f32(layout):
    cfg = dict(b=1, L=64, h=2, n_kv=1, d=64, N=4)
    bounds = [synth.document_bounds(256, seed=13, mean_len=20).astype(np.int32)]
    for shard in range(4):
        announce("packed ring_fwd f32", layout, "shard", shard)
        inp = make_inputs(**cfg, q_shard=shard, seed=81, dtype="f32")
        docs = gpu_docs(bounds, N=4, L=64, shard=shard, layout=layout)
        o, lse = ra.ring_fwd(to_gpu(inp["q"], "f32"), to_gpu(inp["k_all"], "f32"),
                             to_gpu(inp["v_all"], "f32"), q_shard=shard, causal=True,
                             layout=layout, docs=docs)
        torch.cuda.synchronize()
        O, LSE = oracle_ring_docs(inp, bounds, N=4, shard=shard, layout=layout, causal=True)
        check_f32(o, lse, O, LSE, f"packed f32 {layout} shard {shard}")


def test_one_document_matches_no_packing_exactly():
    """One document over the whole window: the same kernels and tiles as no packing.  The
    unpacked pass gets a workspace without the second accumulator, which packed passes never
    keep, so that both run every query block whole (with one launch per step, and with the
    remote steps batched into one launch)."""
    cfg = dict(b=1, L=256, h=8, n_kv=2, d=128, N=4)
    inp = make_inputs(**cfg, q_shard=1, seed=91, dtype="bf16")
    q, k, v = (to_gpu(inp[x], "bf16") for x in ("q", "k_all", "v_all"))
    docs = gpu_docs([np.array([0, 1024], dtype=np.int32)], N=4, L=256, shard=1, layout="striped")
    pad = lambda x: (x + 255) // 256 * 256  # noqa: E731
    shard, acc = pad(256 * 2 * 128 * 2), pad(256 * 8 * 128 * 4)
    for spl, nbytes in ((1, 4 * shard + acc), (0, 2 * 3 * shard + acc)):
        announce("packed single document == unpacked, steps per launch", spl)
        ws = torch.empty(nbytes, device="cuda", dtype=torch.uint8)
        o1, l1 = ra.ring_fwd(q, k, v, q_shard=1, causal=True, layout="striped", steps_per_launch=spl,
                             workspace=ws)
        o2, l2 = ra.ring_fwd(q, k, v, q_shard=1, causal=True, layout="striped", docs=docs, steps_per_launch=spl)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("causal", [True, False])
def test_ring_bwd_packed_small(layout, causal):
    cfg = dict(b=1, L=200, h=8, n_kv=2, d=128, N=3)
    bounds = synth.document_bounds(600, seed=17, mean_len=40).astype(np.int32)
    for shard in (0, 2):
        announce("packed ring_bwd", layout, "causal", causal, "shard", shard)
        inp = make_inputs(**cfg, q_shard=shard, seed=101 + shard, dtype="bf16", with_dout=True)
        q, k_all, v_all, dout = (to_gpu(inp[x], "bf16") for x in ("q", "k_all", "v_all", "dout"))
        docs = gpu_docs([bounds], N=3, L=200, shard=shard, layout=layout)
        o, lse = ra.ring_fwd(q, k_all, v_all, q_shard=shard, causal=causal, layout=layout, docs=docs)
        dq, dk, dv = ra.ring_bwd(q, k_all, v_all, o, dout, lse, q_shard=shard, causal=causal,
                                 layout=layout, docs=docs)
        torch.cuda.synchronize()
        x = {k_: inp[k_].astype(np.float64) for k_ in ("q", "k_all", "v_all", "dout")}
        rdq, rdk, rdv = shard_grads(x["q"], x["k_all"], x["v_all"], x["dout"], N=3, shard=shard,
                                    layout=layout, causal=causal, docs=bounds)
        check_grad(dq, rdq, f"packed dq {layout} {causal} shard {shard}")
        check_grad(dk, rdk, f"packed dk {layout} {causal} shard {shard}")
        check_grad(dv, rdv, f"packed dv {layout} {causal} shard {shard}")


def _boundary_rows(bounds, layout, N, L, shard, extra):
    """Local rows at document starts and ends (and a few others), for sampled checks."""
    pos = shard_tokens(layout, N, L)[shard]
    edges = np.concatenate([bounds[1:-1], bounds[1:-1] - 1])
    rows = np.nonzero(np.isin(pos, edges))[0]
    rows = np.unique(np.concatenate([rows[:: max(1, rows.size // 12)], extra]))
    return rows[(rows >= 0) & (rows < L)]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("shard", [0, 5])
def test_packed_fwd_full_size(shard):
    """S = 262144, N = 8, h = 32, n_kv = 8, bf16, striped causal, documents of mean length 4096."""
    N, L = 8, 32768
    cfg = dict(b=1, L=L, h=32, n_kv=8, d=128, N=N)
    bounds = synth.document_bounds(N * L, seed=1006, mean_len=4096).astype(np.int32)
    announce("packed full size fwd, shard", shard, "documents", bounds.size - 1)
    inp = make_inputs(**cfg, q_shard=shard, seed=1006, dtype="bf16")
    docs = gpu_docs([bounds], N=N, L=L, shard=shard, layout="striped")
    o, lse = ra.ring_fwd(to_gpu(inp["q"], "bf16"), to_gpu(inp["k_all"], "bf16"),
                         to_gpu(inp["v_all"], "bf16"), q_shard=shard, causal=True,
                         layout="striped", docs=docs)
    torch.cuda.synchronize()
    rows = _boundary_rows(bounds, "striped", N, L, shard, full_size_rows(L, 1006 + shard))
    announce(f"oracle on {rows.size} rows")
    O, LSE = oracle_ring_rows(inp, N=N, shard=shard, layout="striped", causal=True, rows=rows, docs=bounds)
    idx = torch.as_tensor(rows, device="cuda")
    check_bf16(o[:, idx], lse[:, :, idx], O, LSE, f"packed full size shard {shard} {rows.size} rows")


@pytest.mark.timeout(900)
def test_packed_bwd_full_size():
    """S = 65536, N = 8, h = 32, n_kv = 8, bf16, striped causal, documents of mean length 2048,
    query shard 3: dQ of sampled rows (every document edge class and ~300 more) and dK, dV of
    keys at document edges and spread over all 8 KV shards (KV head 2) against the oracle,
    element by element; and the sum identities of dK and dV."""
    from test_gpu_bwd import check_grad, oracle_dq_rows
    from gpu_helpers import bwd_full_cols, gather_cols
    N, L, h, n_kv, shard, g = 8, 8192, 32, 8, 3, 2
    cfg = dict(b=1, L=L, h=h, n_kv=n_kv, d=128, N=N)
    bounds = synth.document_bounds(N * L, seed=1007, mean_len=2048).astype(np.int32)
    announce("packed full size bwd, documents", bounds.size - 1)
    inp = make_inputs(**cfg, q_shard=shard, seed=1007, dtype="bf16", with_dout=True)
    q, k_all, v_all, dout = (to_gpu(inp[x], "bf16") for x in ("q", "k_all", "v_all", "dout"))
    docs = gpu_docs([bounds], N=N, L=L, shard=shard, layout="striped")
    o, lse = ra.ring_fwd(q, k_all, v_all, q_shard=shard, causal=True, layout="striped", docs=docs)
    dq, dk, dv = ra.ring_bwd(q, k_all, v_all, o, dout, lse, q_shard=shard, causal=True,
                             layout="striped", docs=docs)
    torch.cuda.synchronize()
    x = {k_: inp[k_].astype(np.float64) for k_ in ("q", "k_all", "v_all", "dout")}
    rows = _boundary_rows(bounds, "striped", N, L, shard, full_size_rows(L, 1107))
    announce(f"oracle dQ of {rows.size} rows")
    rdq = oracle_dq_rows_docs(x, rows, N=N, shard=shard, bounds=bounds)
    check_grad(dq[:, torch.as_tensor(rows, device="cuda")], rdq, "packed full size dq rows")
    toks = shard_tokens("striped", N, L)
    edge_pos = np.concatenate([bounds[1:-1], bounds[1:-1] - 1])
    edge_cols = [(j, int(u)) for j in range(N) for u in np.nonzero(np.isin(toks[j], edge_pos))[0][::7]]
    cols = sorted(set(bwd_full_cols()) | set(edge_cols))
    announce(f"oracle dK, dV of {len(cols)} keys (KV head {g})")
    parts = np.array_split(np.arange(L), 32)
    res = run_threads(lambda rr: key_grads(x["q"][None], x["dout"][None], x["k_all"], x["v_all"], N=N,
                                           query_shards=[shard], kv_head=g, cols=cols, layout="striped",
                                           causal=True, docs=bounds, rows=rr), parts)
    rdk, rdv = sum(r[0] for r in res), sum(r[1] for r in res)
    check_grad(gather_cols(dk, cols, g), rdk, "packed full size dk sampled keys")
    check_grad(gather_cols(dv, cols, g), rdv, "packed full size dv sampled keys")
    dk_sum = f64(dk.sum(dim=(0, 2)))
    dv_sum = f64(dv.sum(dim=(0, 2)))
    do_sum = x["dout"].sum(axis=1).reshape(1, n_kv, h // n_kv, 128).sum(axis=2)
    announce(f"sum dK max abs {np.abs(dk_sum).max():.3e}; sum dV err {np.abs(dv_sum - do_sum).max():.3e}")
    assert np.abs(dk_sum).max() <= 2e-2 * np.sqrt(L)
    assert np.abs(dv_sum - do_sum).max() <= 2e-2 * np.sqrt(L)


def oracle_dq_rows_docs(x, rows, *, N, shard, bounds):
    """shard_dq_rows with packed documents, one KV group per thread."""
    h, n_kv = x["q"].shape[2], x["k_all"].shape[3]
    G = h // n_kv

    def one(g):
        hs = slice(g * G, (g + 1) * G)
        return shard_dq_rows(x["q"][:, :, hs], x["k_all"][:, :, :, g:g + 1], x["v_all"][:, :, :, g:g + 1],
                             x["dout"][:, :, hs], rows, N=N, shard=shard, layout="striped", causal=True, docs=bounds)
    return np.concatenate(run_threads(one, list(range(n_kv))), axis=2)


@pytest.mark.parametrize("causal", [True, False])
def test_every_token_its_own_document(causal):
    """One token per document: each row sees only itself, so O = its own V row (exactly) and
    LSE = scale q.k of its own key (closed form, no oracle call)."""
    N, L, h, n_kv, d, shard = 4, 256, 8, 2, 128, 1
    bounds = np.arange(N * L + 1, dtype=np.int32)
    for layout in LAYOUTS:
        announce("one token per document", layout, "causal", causal)
        inp = make_inputs(b=1, L=L, h=h, n_kv=n_kv, d=d, N=N, q_shard=shard, seed=111, dtype="bf16")
        docs = gpu_docs([bounds], N=N, L=L, shard=shard, layout=layout)
        o, lse = ra.ring_fwd(to_gpu(inp["q"], "bf16"), to_gpu(inp["k_all"], "bf16"),
                             to_gpu(inp["v_all"], "bf16"), q_shard=shard, causal=causal,
                             layout=layout, docs=docs)
        torch.cuda.synchronize()
        toks = shard_tokens(layout, N, L)
        owner = np.empty(N * L, dtype=np.int64)
        local = np.empty(N * L, dtype=np.int64)
        for j in range(N):
            owner[toks[j]] = j
            local[toks[j]] = np.arange(L)
        P = toks[shard]
        grp = h // n_kv
        v_self = np.stack([inp["v_all"][owner[p], 0, local[p]] for p in P])      # [L, n_kv, d]
        k_self = np.stack([inp["k_all"][owner[p], 0, local[p]] for p in P])
        want_o = np.repeat(v_self, grp, axis=1).astype(np.float64)               # [L, h, d]
        s_self = np.einsum("thd,thd->ht", inp["q"][0].astype(np.float64),
                           np.repeat(k_self, grp, axis=1).astype(np.float64)) / np.sqrt(d)
        assert np.array_equal(f64(o)[0], want_o)
        assert np.abs(f64(lse)[0] - s_self).max() <= 1e-3

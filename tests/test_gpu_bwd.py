"""GPU parity of the backward (ra_ring_bwd / ra_step_bwd) against the fp64 oracle.

The GPU backward consumes the GPU forward's own O and LSE; the oracle computes the exact
gradients from the same seeded q, k, v, dO.  Tolerance per gradient tensor (the pages give
none): max abs error <= 2e-2 * max(1, rms(ref)) and mean abs error <= 2e-3 * max(1, rms(ref)).
"""
import numpy as np
import pytest
import torch

import ring_attention_long_amd as ra
from gpu_helpers import (BWD_FULL, BWD_FULL_KV_HEAD, BWD_FULL_SEED, announce, bwd_full_cols,
                         bwd_full_key_grads, f64, full_size_rows, gather_cols, make_inputs, run_threads,
                         to_gpu)
from oracle import LAYOUTS, key_grads, ring_order, shard_dq_rows, shard_grads, shard_tokens

pytestmark = pytest.mark.gpu


def check_grad(got, ref, what):
    got = f64(got) if isinstance(got, torch.Tensor) else got
    scale = max(1.0, float(np.sqrt(np.mean(ref ** 2))))
    err = np.abs(got - ref)
    announce(f"{what}: max abs {err.max():.3e} mean abs {err.mean():.3e} (rms ref {scale:.3f})")
    assert err.max() <= 2e-2 * scale, what
    assert err.mean() <= 2e-3 * scale, what


def _run(cfg, layout, causal, shard, seed, copy_stream="auto", minimum_workspace=False):
    N = cfg["N"]
    inp = make_inputs(**cfg, q_shard=shard, seed=seed, dtype="bf16", with_dout=True)
    q, k_all, v_all = (to_gpu(inp[x], "bf16") for x in ("q", "k_all", "v_all"))
    dout = to_gpu(inp["dout"], "bf16")
    o, lse = ra.ring_fwd(q, k_all, v_all, q_shard=shard, causal=causal, layout=layout)
    ws = None
    if minimum_workspace:   # every key block of the dK/dV kernel whole, as in ra_step_bwd
        n = ra.ring_bwd_workspace_bytes(q, k_all, causal=causal, layout=layout, minimum=True)
        ws = torch.empty(n, device="cuda", dtype=torch.uint8)
    dq, dk, dv = ra.ring_bwd(q, k_all, v_all, o, dout, lse, q_shard=shard, causal=causal,
                             layout=layout, copy_stream=copy_stream, workspace=ws)
    torch.cuda.synchronize()
    return inp, (q, k_all, v_all, dout, o, lse), (dq, dk, dv)


@pytest.mark.parametrize("layout,causal", [("contiguous", False), ("contiguous", True),
                                           ("striped", True), ("zigzag", True)])
@pytest.mark.parametrize("h,n_kv", [(8, 2), (4, 4), (6, 2)])
def test_ring_bwd_small(layout, causal, h, n_kv):
    cfg = dict(b=1, L=200, h=h, n_kv=n_kv, d=128, N=3)
    for shard in (0, 2):
        announce("ring_bwd", layout, "causal", causal, "shard", shard, cfg)
        inp, _, (dq, dk, dv) = _run(cfg, layout, causal, shard, seed=81 + shard)
        x = {k_: inp[k_].astype(np.float64) for k_ in ("q", "k_all", "v_all", "dout")}
        rdq, rdk, rdv = shard_grads(x["q"], x["k_all"], x["v_all"], x["dout"], N=3, shard=shard,
                                    layout=layout, causal=causal)
        check_grad(dq, rdq, f"dq {layout} {causal} shard {shard}")
        check_grad(dk, rdk, f"dk {layout} {causal} shard {shard}")
        check_grad(dv, rdv, f"dv {layout} {causal} shard {shard}")


def test_ring_bwd_batch_and_tiny_shards():
    for cfg, layout in ((dict(b=2, L=70, h=4, n_kv=1, d=128, N=2), "striped"),
                        (dict(b=1, L=2, h=4, n_kv=2, d=128, N=3), "zigzag")):
        for shard in range(cfg["N"]):
            announce("ring_bwd edge", layout, cfg, "shard", shard)
            inp, _, (dq, dk, dv) = _run(cfg, layout, True, shard, seed=91)
            x = {k_: inp[k_].astype(np.float64) for k_ in ("q", "k_all", "v_all", "dout")}
            rdq, rdk, rdv = shard_grads(x["q"], x["k_all"], x["v_all"], x["dout"], N=cfg["N"],
                                        shard=shard, layout=layout, causal=True)
            check_grad(dq, rdq, "dq edge")
            check_grad(dk, rdk, "dk edge")
            check_grad(dv, rdv, "dv edge")


@pytest.mark.parametrize("layout", ["striped", "contiguous"])
def test_ring_bwd_large_logits(layout):
    """Q x 4 (exact in bf16): logits up to ~15 and |LSE| / scale ~ 150, where the dK/dV
    kernel's bf16 (hi, lo) pair of -LSE / scale carries the most absolute error.  dQ and dV
    pass the usual gates.  dK's largest error grows with the logit scale in bf16 (dS rounded
    to bf16 meets larger Q): max abs 6.4e-2 at x4 and 0.16 at x8 on these inputs, the same
    to three digits with the statistics read per row from LDS instead of folded into the
    products, above the generic max gate; dK is held to the mean gate.  The normalisation of
    P, which a wrong LSE would break, is checked by sum over keys of dV = sum over the
    group's rows of dO (the dK identity's residual, bf16 noise of dS times Q, grows with
    the scale of Q and is checked at unit scale in the full-size test)."""
    cfg = dict(b=1, L=160, h=8, n_kv=2, d=128, N=4)
    N, L, h, n_kv = 4, 160, 8, 2
    shard = 2
    inp = make_inputs(**cfg, q_shard=shard, seed=97, dtype="bf16", with_dout=True)
    inp["q"] = inp["q"] * 4.0
    q, k_all, v_all, dout = (to_gpu(inp[x], "bf16") for x in ("q", "k_all", "v_all", "dout"))
    announce("ring_bwd large logits", layout, cfg)
    o, lse = ra.ring_fwd(q, k_all, v_all, q_shard=shard, causal=True, layout=layout)
    dq, dk, dv = ra.ring_bwd(q, k_all, v_all, o, dout, lse, q_shard=shard, causal=True, layout=layout)
    torch.cuda.synchronize()
    x = {k_: inp[k_].astype(np.float64) for k_ in ("q", "k_all", "v_all", "dout")}
    rdq, rdk, rdv = shard_grads(x["q"], x["k_all"], x["v_all"], x["dout"], N=N, shard=shard,
                                layout=layout, causal=True)
    check_grad(dq, rdq, f"dq large logits {layout}")
    check_grad(dv, rdv, f"dv large logits {layout}")
    err = np.abs(f64(dk) - rdk)
    scale = max(1.0, float(np.sqrt(np.mean(rdk ** 2))))
    announce(f"dk large logits {layout}: max abs {err.max():.3e} mean abs {err.mean():.3e} (rms ref {scale:.3f})")
    assert err.mean() <= 2e-3 * scale
    dv_sum = f64(dv.sum(dim=(0, 2)))                       # [b, n_kv, d], over every key seen
    do_sum = x["dout"].sum(axis=1).reshape(1, n_kv, h // n_kv, 128).sum(axis=2)
    announce(f"sum dV err {np.abs(dv_sum - do_sum).max():.3e}")
    assert np.abs(dv_sum - do_sum).max() <= 2e-2 * np.sqrt(L)


def test_step_bwd_sums_to_ring_bwd():
    """ra_step_bwd over the ring order, with ra_bwd_preprocess, equals ra_ring_bwd given the
    minimum workspace (the same kernels: every key block of the dK/dV kernel whole)."""
    cfg = dict(b=1, L=160, h=8, n_kv=2, d=128, N=4)
    shard = 1
    inp, (q, k_all, v_all, dout, o, lse), (dq, dk, dv) = _run(cfg, "striped", True, shard, seed=95,
                                                              minimum_workspace=True)
    delta = ra.bwd_preprocess(o, dout)
    dq2 = torch.zeros_like(dq)
    dk2 = torch.zeros_like(dk)
    dv2 = torch.zeros_like(dv)
    for src in ring_order(4, shard):
        ra.step_bwd(q, k_all[src], v_all[src], dout, lse, delta, N=4, q_shard=shard, kv_shard=src,
                    causal=True, layout="striped", dq_acc=dq2, dk_acc=dk2[src], dv_acc=dv2[src])
    torch.cuda.synchronize()
    announce("step_bwd vs ring_bwd")
    for a_, b_ in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert torch.allclose(a_, b_, rtol=1e-5, atol=1e-5)


def test_bwd_preprocess_is_rowsum_of_products():
    g = torch.Generator().manual_seed(3)
    o = torch.randn(2, 37, 3, 128, generator=g).to(torch.bfloat16)
    do = torch.randn(2, 37, 3, 128, generator=g).to(torch.bfloat16)
    want = (o.double() * do.double()).sum(-1).permute(0, 2, 1).numpy()
    announce("bwd_preprocess")
    got = ra.bwd_preprocess(o.cuda(), do.cuda())
    torch.cuda.synchronize()
    np.testing.assert_allclose(f64(got), want, rtol=1e-5, atol=1e-4)


# ------------------------------------------------------------------ full size (config 5)
def oracle_dq_rows(q, k_all, v_all, dout, rows, *, N, shard, layout, causal):
    """shard_dq_rows (float64 inputs) with one KV group per thread."""
    h, n_kv = q.shape[2], k_all.shape[3]
    G = h // n_kv

    def one(g):
        hs = slice(g * G, (g + 1) * G)
        return shard_dq_rows(q[:, :, hs], k_all[:, :, :, g:g + 1], v_all[:, :, :, g:g + 1], dout[:, :, hs], rows,
                             N=N, shard=shard, layout=layout, causal=causal)
    return np.concatenate(run_threads(one, list(range(n_kv))), axis=2)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("shard", [0, 7])
def test_config5_full_size(shard):
    """S = 65536, N = 8 (L = 8192), h = 32, n_kv = 8, d = 128, bf16, causal striped: dQ of
    ~300 sampled rows (every head) and dK, dV of 144 keys spread over all 8 KV shards (KV
    head 2) against the oracle, element by element; plus the Q = 0 closed form for dV of
    every key."""
    cfg = dict(BWD_FULL)
    N, L, h, n_kv = 8, 8192, 32, 8
    announce("config5 ring_bwd full size, shard", shard)
    inp, (q, k_all, v_all, dout, o, lse), (dq, dk, dv) = _run(cfg, "striped", True, shard, seed=BWD_FULL_SEED)
    x = {k_: inp[k_].astype(np.float64) for k_ in ("q", "k_all", "v_all", "dout")}
    # (1) dQ of sampled rows
    rows = full_size_rows(L, 5005 + shard)
    announce(f"oracle dQ on {rows.size} rows")
    rdq = oracle_dq_rows(x["q"], x["k_all"], x["v_all"], x["dout"], rows, N=N, shard=shard, layout="striped",
                         causal=True)
    check_grad(dq[:, torch.as_tensor(rows, device="cuda")], rdq, f"config5 dq {rows.size} sampled rows")
    # (2) dK, dV of sampled keys of every KV shard
    cols = bwd_full_cols()
    announce(f"oracle dK, dV of {len(cols)} keys (KV head {BWD_FULL_KV_HEAD}) from shard {shard}'s rows")
    rdk, rdv = bwd_full_key_grads([shard])
    check_grad(gather_cols(dk, cols, BWD_FULL_KV_HEAD), rdk, "config5 dk sampled keys")
    check_grad(gather_cols(dv, cols, BWD_FULL_KV_HEAD), rdv, "config5 dv sampled keys")
    # (3) identities over all keys: sum dK = 0 per KV head (key-shift invariance); sum dV =
    #     sum of dO over the group's query rows (softmax rows sum to one)
    dk_sum = f64(dk.sum(dim=(0, 2)))                       # [b, n_kv, d]
    dv_sum = f64(dv.sum(dim=(0, 2)))
    do_sum = x["dout"].sum(axis=1).reshape(1, n_kv, h // n_kv, 128).sum(axis=2)
    announce(f"sum dK max abs {np.abs(dk_sum).max():.3e}; sum dV err {np.abs(dv_sum - do_sum).max():.3e}")
    assert np.abs(dk_sum).max() <= 2e-2 * np.sqrt(L)
    assert np.abs(dv_sum - do_sum).max() <= 2e-2 * np.sqrt(L)
    # (4) Q = 0: uniform weights 1/n_r; dK = 0 exactly and dV_c = sum over rows r that see
    #     key c of dO_r / n_r (summed over the group's heads), every key of every shard
    q0 = torch.zeros_like(q)
    o0, lse0 = ra.ring_fwd(q0, k_all, v_all, q_shard=shard, causal=True, layout="striped")
    dq0, dk0, dv0 = ra.ring_bwd(q0, k_all, v_all, o0, dout, lse0, q_shard=shard, causal=True,
                                layout="striped")
    torch.cuda.synchronize()
    assert float(dk0.abs().max()) == 0.0
    toks = shard_tokens("striped", N, L)
    pos_q = toks[shard]                                    # increasing
    w = x["dout"][0] / (pos_q + 1.0)[:, None, None]        # [L, h, d]
    wg = w.reshape(L, n_kv, h // n_kv, 128).sum(axis=2)   # [L, n_kv, d]
    suffix = np.cumsum(wg[::-1], axis=0)[::-1]             # suffix[r] = sum over rows >= r
    want = np.zeros((N, L, n_kv, 128))
    for j in range(N):
        first = np.searchsorted(pos_q, toks[j], side="left")   # first row with pos >= key pos
        valid = first < L
        want[j][valid] = suffix[first[valid]]
    check_grad(dv0[:, 0], want, "config5 dV closed form (Q = 0)")


def test_ring_bwd_timed_matches_untimed():
    """The timed pass gives bit-identical gradients; every live step has an interval inside the
    pass, skipped steps report -1, and each staged copy ends before its step begins."""
    cfg = dict(b=1, L=192, h=8, n_kv=2, d=128, N=4)
    inp = make_inputs(**cfg, q_shard=1, seed=97, dtype="bf16", with_dout=True)
    q, k_all, v_all, dout = (to_gpu(inp[x], "bf16") for x in ("q", "k_all", "v_all", "dout"))
    o, lse = ra.ring_fwd(q, k_all, v_all, q_shard=1, causal=True, layout="contiguous")
    announce("ring_bwd timed vs untimed, contiguous causal shard 1")
    a = ra.ring_bwd(q, k_all, v_all, o, dout, lse, q_shard=1, causal=True, layout="contiguous")
    *b, tm = ra.ring_bwd(q, k_all, v_all, o, dout, lse, q_shard=1, causal=True, layout="contiguous", timed=True)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    live = [k for k in range(4) if tm["step_begin_ms"][k] >= 0]
    assert live == [0, 1]          # contiguous causal: shard 1 sees shards 1 and 0 only
    for k in live:
        assert 0 <= tm["step_begin_ms"][k] < tm["step_end_ms"][k] <= tm["total_ms"]
        if k >= 1:
            assert tm["copy_end_ms"][k] <= tm["step_begin_ms"][k] + 1e-3


def test_ring_bwd_overwrites_every_output_element():
    """ra_ring_bwd writes dq and every shard's dk, dv whatever they held: outputs filled with
    NaN come back equal to a pass into fresh buffers.  Cases: contiguous causal (dead steps,
    whose shards are filled with zeros; shard 0 has one live step), striped and zigzag causal
    (workgroups whose keys no query of the step sees store zeros), a ragged L, GQA 3."""
    cfg = dict(b=2, L=150, h=6, n_kv=2, d=128, N=4)
    for layout in ("contiguous", "striped", "zigzag"):
        for shard in (0, 3):
            announce("ring_bwd outputs overwritten", layout, "shard", shard)
            inp = make_inputs(**cfg, q_shard=shard, seed=171 + shard, dtype="bf16", with_dout=True)
            q, k_all, v_all, dout = (to_gpu(inp[x], "bf16") for x in ("q", "k_all", "v_all", "dout"))
            o, lse = ra.ring_fwd(q, k_all, v_all, q_shard=shard, causal=True, layout=layout)
            ref = ra.ring_bwd(q, k_all, v_all, o, dout, lse, q_shard=shard, causal=True, layout=layout)
            nan = tuple(torch.full_like(t, float("nan")) for t in ref)
            got = ra.ring_bwd(q, k_all, v_all, o, dout, lse, q_shard=shard, causal=True, layout=layout, out=nan)
            torch.cuda.synchronize()
            for a, b in zip(ref, got):
                assert torch.equal(a, b)


@pytest.mark.parametrize("cfg,layout,causal", [
    (dict(b=1, L=2048, h=32, n_kv=8, d=128, N=8), "striped", True),     # 16 key blocks x 8 KV heads
    (dict(b=2, L=700, h=6, n_kv=2, d=128, N=3), "zigzag", True),        # GQA 3, ragged, two batch rows
    (dict(b=1, L=520, h=8, n_kv=4, d=128, N=4), "contiguous", False),
    (dict(b=1, L=384, h=4, n_kv=4, d=128, N=4), "contiguous", True),
])
def test_ring_bwd_split_key_blocks(cfg, layout, causal):
    """Short shards whose key blocks leave compute units idle: with the second dK, dV buffers in
    the workspace the dK/dV kernel runs the query tiles of the heaviest key blocks as two
    workgroups and adds the halves after the kernel.  Against the oracle (sampled rows and keys
    at L = 2048, everything below); against the pass with the minimum workspace (whole key
    blocks: dQ bit-identical, dK and dV close and not identical, which shows the split ran);
    and with the workspace filled with NaN beforehand (bit-identical)."""
    N, L = cfg["N"], cfg["L"]
    shard = N - 1
    announce("ring_bwd split key blocks", layout, causal, cfg)
    inp = make_inputs(**cfg, q_shard=shard, seed=2300, dtype="bf16", with_dout=True)
    q, k_all, v_all, dout = (to_gpu(inp[x], "bf16") for x in ("q", "k_all", "v_all", "dout"))
    o, lse = ra.ring_fwd(q, k_all, v_all, q_shard=shard, causal=causal, layout=layout)
    full = ra.ring_bwd_workspace_bytes(q, k_all, causal=causal, layout=layout)
    small = ra.ring_bwd_workspace_bytes(q, k_all, causal=causal, layout=layout, minimum=True)
    assert full > small > 0
    outs = {}
    for name, nbytes, nan in (("split", full, False), ("nan", full, True), ("whole", small, False)):
        ws = torch.zeros(nbytes, device="cuda", dtype=torch.uint8)
        if nan:
            ws.view(-1)[: nbytes // 4 * 4].view(torch.float32).fill_(float("nan"))
        outs[name] = ra.ring_bwd(q, k_all, v_all, o, dout, lse, q_shard=shard, causal=causal, layout=layout,
                                 workspace=ws)
    torch.cuda.synchronize()
    dq, dk, dv = outs["split"]
    assert all(torch.equal(a_, b_) for a_, b_ in zip(outs["split"], outs["nan"]))
    assert torch.equal(dq, outs["whole"][0])
    for a_, b_, what in ((dk, outs["whole"][1], "dk"), (dv, outs["whole"][2], "dv")):
        d = float((a_ - b_).abs().max())
        announce(f"{what} split vs whole: max |diff| {d:.3e}")
        assert d <= 1e-3 * max(1.0, float(b_.abs().max()))
    assert not (torch.equal(dk, outs["whole"][1]) and torch.equal(dv, outs["whole"][2])), "no key block split"
    x = {k_: inp[k_].astype(np.float64) for k_ in ("q", "k_all", "v_all", "dout")}
    if L <= 1024:
        rdq, rdk, rdv = shard_grads(x["q"], x["k_all"], x["v_all"], x["dout"], N=N, shard=shard,
                                    layout=layout, causal=causal)
        check_grad(dq, rdq, "split dq")
        check_grad(dk, rdk, "split dk")
        check_grad(dv, rdv, "split dv")
    else:
        rows = full_size_rows(L, 2301)
        rdq = oracle_dq_rows(x["q"], x["k_all"], x["v_all"], x["dout"], rows, N=N, shard=shard, layout=layout,
                             causal=causal)
        check_grad(dq[:, torch.as_tensor(rows, device="cuda")], rdq, "split dq sampled rows")
        cols = [(j, c) for j in range(N) for c in (0, 1, 63, 64, 127, 128, 129, L // 2, L - 1)]
        rdk, rdv = key_grads(x["q"][None], x["dout"][None], x["k_all"], x["v_all"], N=N, query_shards=[shard],
                             kv_head=3, cols=cols, layout=layout, causal=causal)
        check_grad(gather_cols(dk, cols, 3), rdk, "split dk sampled keys")
        check_grad(gather_cols(dv, cols, 3), rdv, "split dv sampled keys")

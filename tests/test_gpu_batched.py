"""Forward passes with ring steps batched into launches (ra_problem.steps_per_launch >= 2, and
the library's choice 0: all remote steps in one launch for short steps or packed documents,
up to 4 per launch for long steps):
after step 0 each workgroup walks several KV shards in ring order with its online-softmax
state (m, l, O) on chip and merges once (page 1, "Blockwise Attention and Online Softmax
Formulations": the state carried from one block to the next), and every remote shard is
staged into a slot of its own.  Every case
is compared with the oracle element by element (sampled rows for the long-tile case); the
batched pass is also compared with the one-launch-per-step pass (close: they differ in the
order of fp32 sums and in where the merges happen) and the timed pass with the untimed one
(bit-identical).  Cases reach: groups of 2 and 3 steps and the rest of the ring in one
launch; contiguous causal shards whose later groups hold no live step (their copies still
run); ragged L; several batch rows; 4, 1 and 3 query heads per KV head; packed documents
(workgroups without any key in a whole batch); large logits (rescaling across shard
boundaries); 96-key tiles; short shards whose launches split query blocks over two
workgroups through the second accumulator (fewer and more work items than compute units)."""
import numpy as np
import pytest
import torch

import ring_attention_long_amd as ra
import synth
from gpu_helpers import (announce, check_bf16, f64, full_size_rows, make_inputs, oracle_ring, oracle_ring_rows,
                         to_gpu)

pytestmark = pytest.mark.gpu


def _tensors(inp):
    return [to_gpu(inp[x], "bf16") for x in ("q", "k_all", "v_all")]


def _close(a, b, what):
    d = np.abs(f64(a) - f64(b)).max()
    announce(f"{what}: max |diff| {d:.3e}")
    return d


@pytest.mark.parametrize("layout,causal", [("contiguous", False), ("contiguous", True),
                                           ("striped", True), ("zigzag", True)])
@pytest.mark.parametrize("spl", [2, 3, 0])
def test_batched_every_shard_matches_oracle(layout, causal, spl):
    cfg = dict(b=2, L=330, h=8, n_kv=2, d=128, N=5)
    for shard in range(cfg["N"]):
        announce("batched pass", layout, "causal", causal, "steps per launch", spl, "shard", shard, cfg)
        inp = make_inputs(**cfg, q_shard=shard, seed=1400 + shard, dtype="bf16")
        q, k_all, v_all = _tensors(inp)
        o, lse = ra.ring_fwd(q, k_all, v_all, q_shard=shard, causal=causal, layout=layout, steps_per_launch=spl)
        o1, l1 = ra.ring_fwd(q, k_all, v_all, q_shard=shard, causal=causal, layout=layout, steps_per_launch=1)
        torch.cuda.synchronize()
        O, LSE = oracle_ring(inp, N=cfg["N"], shard=shard, layout=layout, causal=causal)
        check_bf16(o, lse, O, LSE, f"batched {layout} {causal} spl {spl} shard {shard}")
        assert _close(o, o1, "batched vs one launch per step") <= 2e-2
        fin = torch.isfinite(l1)
        assert torch.equal(torch.isfinite(lse), fin)
        assert float((lse[fin] - l1[fin]).abs().max()) <= 1e-4


@pytest.mark.parametrize("h,n_kv", [(4, 1), (4, 4), (6, 2)])
def test_batched_head_groupings(h, n_kv):
    cfg = dict(b=3, L=200, h=h, n_kv=n_kv, d=128, N=4)
    for layout in ("striped", "zigzag"):
        announce("batched pass, heads", h, n_kv, layout)
        inp = make_inputs(**cfg, q_shard=1, seed=1410 + h, dtype="bf16")
        q, k_all, v_all = _tensors(inp)
        o, lse = ra.ring_fwd(q, k_all, v_all, q_shard=1, causal=True, layout=layout)
        torch.cuda.synchronize()
        O, LSE = oracle_ring(inp, N=cfg["N"], shard=1, layout=layout, causal=True)
        check_bf16(o, lse, O, LSE, f"batched h{h} kv{n_kv} {layout}")


def test_batched_default_equals_explicit_and_timed():
    """Short steps (b h L^2 <= 2^33): the library's choice is all remote steps in one launch;
    the timed pass runs the same launches and reports them by their first step."""
    cfg = dict(b=1, L=512, h=8, n_kv=2, d=128, N=6)
    inp = make_inputs(**cfg, q_shard=4, seed=1420, dtype="bf16")
    q, k_all, v_all = _tensors(inp)
    o0, l0 = ra.ring_fwd(q, k_all, v_all, q_shard=4, causal=True, layout="striped")
    o5, l5 = ra.ring_fwd(q, k_all, v_all, q_shard=4, causal=True, layout="striped", steps_per_launch=5)
    ot, lt, tm = ra.ring_fwd_timed(q, k_all, v_all, q_shard=4, causal=True, layout="striped")
    o2, l2, tm2 = ra.ring_fwd_timed(q, k_all, v_all, q_shard=4, causal=True, layout="striped", steps_per_launch=2)
    torch.cuda.synchronize()
    announce("timed launches", tm["launch_steps"], tm2["launch_steps"])
    assert torch.equal(o0, o5) and torch.equal(l0, l5)
    assert torch.equal(o0, ot) and torch.equal(l0, lt)
    assert tm["launch_steps"] == [1, 5, 0, 0, 0, 0]
    assert tm2["launch_steps"] == [1, 2, 0, 2, 0, 1]
    for t, starts in ((tm, [0, 1]), (tm2, [0, 1, 3, 5])):
        for k in range(cfg["N"]):
            timed = t["step_begin_ms"][k] >= 0
            assert timed == (k in starts)
            if timed:
                assert t["step_end_ms"][k] > t["step_begin_ms"][k]
            if k >= 1:
                assert t["copy_end_ms"][k] >= t["copy_begin_ms"][k] >= 0
        # each launch starts after the copies of its shards
        for s in starts[1:]:
            n = t["launch_steps"][s]
            assert t["step_begin_ms"][s] >= max(t["copy_end_ms"][s:s + n]) - 1e-3
    O, LSE = oracle_ring(inp, N=cfg["N"], shard=4, layout="striped", causal=True)
    check_bf16(o0, l0, O, LSE, "library's choice, all remote steps in one launch")
    check_bf16(o2, l2, O, LSE, "timed, 2 steps per launch")


def test_batched_default_long_steps_four_per_launch():
    """Long steps (b h L^2 > 2^33: L = 16448, h = 32): the library's choice is four steps per
    launch (step 0, ring steps 1..4, then 5), the same launches as steps_per_launch = 4."""
    L, h, n_kv, d, N = 16448, 32, 8, 128, 6
    g = torch.Generator(device="cuda").manual_seed(1425)
    mk = lambda *s: torch.randn(*s, device="cuda", generator=g).to(torch.bfloat16)
    q, k_all, v_all = mk(1, L, h, d), mk(N, 1, L, n_kv, d), mk(N, 1, L, n_kv, d)
    announce("long steps, library's choice", dict(L=L, h=h, n_kv=n_kv, N=N))
    o0, l0, tm = ra.ring_fwd_timed(q, k_all, v_all, q_shard=2, causal=True, layout="zigzag")
    o4, l4 = ra.ring_fwd(q, k_all, v_all, q_shard=2, causal=True, layout="zigzag", steps_per_launch=4)
    torch.cuda.synchronize()
    assert tm["launch_steps"] == [1, 4, 0, 0, 0, 1]
    assert torch.equal(o0, o4) and torch.equal(l0, l4)


@pytest.mark.parametrize("N", [16, 32])
def test_batched_large_ring_one_launch(N):
    """Rings larger than the measured N = 8: short steps put all N - 1 remote shards in one
    launch (each workgroup walks up to 31 KV shards with its state on chip)."""
    cfg = dict(b=1, L=96, h=4, n_kv=2, d=128, N=N)
    for layout, causal, shard in (("striped", True, N - 1), ("zigzag", True, N // 2), ("contiguous", False, 3),
                                  ("contiguous", True, N - 2)):
        announce("large ring", N, layout, causal, "shard", shard)
        inp = make_inputs(**cfg, q_shard=shard, seed=1470 + N + shard, dtype="bf16")
        q, k_all, v_all = _tensors(inp)
        o, lse, tm = ra.ring_fwd_timed(q, k_all, v_all, q_shard=shard, causal=causal, layout=layout)
        torch.cuda.synchronize()
        live = [x for x in tm["launch_steps"] if x > 0]
        assert tm["launch_steps"][0] == 1 and len(live) <= 2 and sum(tm["launch_steps"]) <= N
        O, LSE = oracle_ring(inp, N=N, shard=shard, layout=layout, causal=causal)
        check_bf16(o, lse, O, LSE, f"N={N} {layout} causal={causal} shard {shard}")


def test_batched_contiguous_dead_groups():
    """Contiguous causal, shard 1 of 6 with 2 steps per launch: the group (1, 2) holds the one
    live remote step, the groups (3, 4) and (5) none, so the group (1, 2) writes the output
    while the copies of the later shards still run."""
    cfg = dict(b=1, L=300, h=8, n_kv=2, d=128, N=6)
    inp = make_inputs(**cfg, q_shard=1, seed=1430, dtype="bf16")
    q, k_all, v_all = _tensors(inp)
    o, lse, tm = ra.ring_fwd_timed(q, k_all, v_all, q_shard=1, causal=True, layout="contiguous", steps_per_launch=2)
    torch.cuda.synchronize()
    assert tm["launch_steps"] == [1, 2, 0, 0, 0, 0]
    O, LSE = oracle_ring(inp, N=cfg["N"], shard=1, layout="contiguous", causal=True)
    check_bf16(o, lse, O, LSE, "contiguous shard 1, later groups dead")


@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
def test_batched_packed_documents(layout):
    cfg = dict(b=1, L=640, h=8, n_kv=2, d=128, N=4)
    bounds = synth.document_bounds(cfg["N"] * cfg["L"], seed=1440, mean_len=200).astype(np.int32)
    for shard in (0, 3):
        for spl in (0, 2):
            announce("batched packed", layout, "shard", shard, "steps per launch", spl)
            inp = make_inputs(**cfg, q_shard=shard, seed=1441 + shard, dtype="bf16")
            q, k_all, v_all = _tensors(inp)
            db, de = ra.document_ranges(bounds, N=cfg["N"], L=cfg["L"], shard=shard, layout=layout)
            docs = (torch.from_numpy(db[None]).cuda(), torch.from_numpy(de[None]).cuda())
            o, lse = ra.ring_fwd(q, k_all, v_all, q_shard=shard, causal=True, layout=layout, docs=docs,
                                 steps_per_launch=spl)
            torch.cuda.synchronize()
            O, LSE = oracle_ring_rows(inp, N=cfg["N"], shard=shard, layout=layout, causal=True,
                                      rows=np.arange(cfg["L"]), docs=bounds)
            check_bf16(o, lse, O, LSE, f"batched packed {layout} shard {shard} spl {spl}")


def test_batched_packed_default_takes_every_remote_step():
    """With packed documents the library's choice is all remote steps in one launch."""
    cfg = dict(b=1, L=256, h=8, n_kv=2, d=128, N=6)
    bounds = synth.document_bounds(cfg["N"] * cfg["L"], seed=1445, mean_len=150).astype(np.int32)
    inp = make_inputs(**cfg, q_shard=2, seed=1446, dtype="bf16")
    q, k_all, v_all = _tensors(inp)
    db, de = ra.document_ranges(bounds, N=cfg["N"], L=cfg["L"], shard=2, layout="zigzag")
    docs = (torch.from_numpy(db[None]).cuda(), torch.from_numpy(de[None]).cuda())
    o, lse, tm = ra.ring_fwd_timed(q, k_all, v_all, q_shard=2, causal=True, layout="zigzag", docs=docs)
    torch.cuda.synchronize()
    announce("packed default launches", tm["launch_steps"])
    assert tm["launch_steps"] == [1, 5, 0, 0, 0, 0]
    O, LSE = oracle_ring_rows(inp, N=cfg["N"], shard=2, layout="zigzag", causal=True, rows=np.arange(cfg["L"]),
                              docs=bounds)
    check_bf16(o, lse, O, LSE, "packed, all remote steps in one launch")


def test_batched_large_logits():
    """Q x 8: row maxima jump between shards, so the lazy rescale runs across shard boundaries
    inside a launch."""
    cfg = dict(b=1, L=256, h=8, n_kv=2, d=128, N=5)
    inp = make_inputs(**cfg, q_shard=2, seed=1450, dtype="bf16")
    inp["q"] = (inp["q"].astype(np.float32) * 8).astype(inp["q"].dtype)
    q, k_all, v_all = _tensors(inp)
    for layout, causal in (("striped", True), ("contiguous", False)):
        announce("batched large logits", layout, causal)
        o, lse = ra.ring_fwd(q, k_all, v_all, q_shard=2, causal=causal, layout=layout)
        torch.cuda.synchronize()
        O, LSE = oracle_ring(inp, N=cfg["N"], shard=2, layout=layout, causal=causal)
        check_bf16(o, lse, O, LSE, f"batched x8 {layout}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("layout,causal", [("striped", True), ("contiguous", False)])
def test_batched_long_tiles_ragged_sampled(layout, causal):
    """96-key tiles (L >= 16384), a ragged shard, three shards: step 0 and one launch of two."""
    cfg = dict(b=1, L=16448, h=8, n_kv=2, d=128, N=3)
    inp = make_inputs(**cfg, q_shard=1, seed=1460, dtype="bf16")
    q, k_all, v_all = _tensors(inp)
    o, lse, tm = ra.ring_fwd_timed(q, k_all, v_all, q_shard=1, causal=causal, layout=layout)
    torch.cuda.synchronize()
    assert tm["launch_steps"] == [1, 2, 0]
    rows = full_size_rows(cfg["L"], 1461)
    announce("batched long tiles", layout, causal, "rows", rows.size)
    O, LSE = oracle_ring_rows(inp, N=3, shard=1, layout=layout, causal=causal, rows=rows)
    ri = torch.from_numpy(rows).to(o.device)
    check_bf16(o[:, ri], lse[:, :, ri], O, LSE, f"batched long tiles {layout}")


def _second_acc_bytes(cfg):
    pad = lambda x: (x + 255) // 256 * 256  # noqa: E731
    b, L, h, d = cfg["b"], cfg["L"], cfg["h"], cfg["d"]
    return pad(b * L * h * d * 4) + pad(b * h * L * 4)


@pytest.mark.parametrize("layout,causal", [("striped", True), ("contiguous", False), ("zigzag", True),
                                           ("contiguous", True)])
def test_batched_split_short_shards(layout, causal):
    """Short shards whose launches leave compute units idle (2 KV heads x ceil(L / 64) query
    blocks, far fewer workgroups than units): with the second accumulator in the workspace,
    step 0 and the batched launch split the key ranges of query blocks over two workgroups
    (in a batched launch, every KV shard's range of a block in two halves), the second half
    merging into the second accumulator, and the pass ends by folding it into the output.
    Against the oracle; against the same pass without the second accumulator in the workspace
    (every block whole: close, and the LSE differs in its last bits, which shows the split
    ran); and with the workspace filled with NaN beforehand (bit-identical)."""
    cfg = dict(b=1, L=250, h=8, n_kv=2, d=128, N=6)
    for shard in (0, 2, 5):
        announce("batched split", layout, "causal", causal, "shard", shard, cfg)
        inp = make_inputs(**cfg, q_shard=shard, seed=1600 + shard, dtype="bf16")
        q, k_all, v_all = _tensors(inp)
        full = ra.ring_workspace_bytes(q, k_all, causal=causal, layout=layout)
        outs = {}
        for name, nbytes, fill in (("zero", full, 0), ("nan", full, None), ("whole", full - _second_acc_bytes(cfg), 0)):
            ws = torch.zeros(nbytes, device="cuda", dtype=torch.uint8)
            if fill is None:
                ws.view(-1)[: nbytes // 4 * 4].view(torch.float32).fill_(float("nan"))
            outs[name] = ra.ring_fwd(q, k_all, v_all, q_shard=shard, causal=causal, layout=layout, workspace=ws)
        torch.cuda.synchronize()
        O, LSE = oracle_ring(inp, N=cfg["N"], shard=shard, layout=layout, causal=causal)
        o, lse = outs["zero"]
        check_bf16(o, lse, O, LSE, f"batched split {layout} {causal} shard {shard}")
        check_bf16(*outs["whole"], O, LSE, f"batched whole blocks {layout} {causal} shard {shard}")
        assert torch.equal(o, outs["nan"][0]) and torch.equal(lse, outs["nan"][1])
        assert _close(o, outs["whole"][0], "split vs whole blocks") <= 2e-2
        assert float((lse - outs["whole"][1]).abs().max()) <= 1e-4
        assert not torch.equal(lse, outs["whole"][1]), "the second accumulator was not used"


@pytest.mark.parametrize("layout,causal", [("striped", True), ("zigzag", True)])
def test_batched_split_more_items_than_units(layout, causal):
    """h = 32, n_kv = 8, L = 2048, N = 8: a batched launch has as many query blocks (32 per KV
    head) as compute units per KV head, and with a causal mask the heaviest blocks do twice
    the mean work over the seven shards.  The plan (list schedule over the units, in launch
    order) then splits blocks although the items outnumber the units.  Sampled rows against
    the oracle (every 64-row tile class, both ends, the half-shard edge), the whole-block pass
    close with an LSE that differs in its last bits (the split ran), and a NaN-filled
    workspace bit-identical."""
    cfg = dict(b=1, L=2048, h=32, n_kv=8, d=128, N=8)
    shard = 3
    announce("batched split, more items than units", layout, cfg)
    inp = make_inputs(**cfg, q_shard=shard, seed=1700, dtype="bf16")
    q, k_all, v_all = _tensors(inp)
    full = ra.ring_workspace_bytes(q, k_all, causal=causal, layout=layout)
    outs = {}
    for name, nbytes, nan in (("split", full, False), ("nan", full, True), ("whole", full - _second_acc_bytes(cfg), False)):
        ws = torch.zeros(nbytes, device="cuda", dtype=torch.uint8)
        if nan:
            ws.view(-1)[: nbytes // 4 * 4].view(torch.float32).fill_(float("nan"))
        outs[name] = ra.ring_fwd(q, k_all, v_all, q_shard=shard, causal=causal, layout=layout, workspace=ws)
    torch.cuda.synchronize()
    o, lse = outs["split"]
    assert torch.equal(o, outs["nan"][0]) and torch.equal(lse, outs["nan"][1])
    assert _close(o, outs["whole"][0], "split vs whole blocks") <= 2e-2
    assert float((lse - outs["whole"][1]).abs().max()) <= 1e-4
    assert not torch.equal(lse, outs["whole"][1]), "the second accumulator was not used"
    rows = full_size_rows(cfg["L"], 1701)
    O, LSE = oracle_ring_rows(inp, N=cfg["N"], shard=shard, layout=layout, causal=causal, rows=rows)
    idx = torch.as_tensor(rows, device="cuda")
    check_bf16(o[:, idx], lse[:, :, idx], O, LSE, f"batched split {layout}, {rows.size} sampled rows")

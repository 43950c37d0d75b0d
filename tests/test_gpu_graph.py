"""Ring passes captured in a HIP graph and replayed.  The passes record no memsets (buffers that
must start at a value are filled by kernels), the side stream's staging joins the compute stream
through events (graph edges under capture), and the batched pass that splits query blocks ends
with the fold of its second accumulator.  Each graph is replayed several times with eager passes
and synchronisations in between, and every replay must equal the eager result bit for bit."""
import pytest
import torch

import ring_attention_long_amd as ra
from gpu_helpers import announce, make_inputs, to_gpu

pytestmark = pytest.mark.gpu


def _replays_equal(run, outs, what):
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()                       # warm-up on a side stream, as capture wants
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for i in range(3):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        announce(f"{what}: replay {i}")
        assert all(torch.equal(a, b) for a, b in zip(outs, ref)), f"{what}: replay {i} differs"
        run()                                        # eager work between replays
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(outs, ref)), f"{what}: eager pass after replay {i}"


@pytest.mark.parametrize("cfg,spl,layout,causal", [
    # batched, query blocks split over idle units, fold at the end
    (dict(b=1, L=1024, h=32, n_kv=8, d=128, N=8), 0, "striped", True),
    # batched, more items than units
    (dict(b=1, L=2048, h=32, n_kv=8, d=128, N=8), 0, "zigzag", True),
    # one launch per step with the split
    (dict(b=1, L=640, h=8, n_kv=2, d=128, N=4), 1, "contiguous", False),
    # batched without a split (blocks fill the units evenly), the last launch writes the output
    (dict(b=1, L=2048, h=32, n_kv=8, d=128, N=4), 0, "contiguous", False),
])
def test_ring_fwd_graph_replays(cfg, spl, layout, causal):
    shard = 1
    inp = make_inputs(**cfg, q_shard=shard, seed=2100, dtype="bf16")
    q, k_all, v_all = (to_gpu(inp[x], "bf16") for x in ("q", "k_all", "v_all"))
    ws = torch.empty(ra.ring_workspace_bytes(q, k_all, causal=causal, layout=layout, steps_per_launch=spl),
                     device="cuda", dtype=torch.uint8)
    o = torch.empty_like(q)
    lse = torch.empty((cfg["b"], cfg["h"], cfg["L"]), device="cuda", dtype=torch.float32)

    def run():
        ra.ring_fwd(q, k_all, v_all, q_shard=shard, causal=causal, layout=layout, workspace=ws, out=o, lse_out=lse,
                    steps_per_launch=spl)
    _replays_equal(run, [o, lse], f"ring_fwd graph {layout} causal {causal} spl {spl} L {cfg['L']}")


def test_ring_fwd_noalloc_graph_replays():
    cfg = dict(b=1, L=1024, h=32, n_kv=8, d=128, N=8)
    inp = make_inputs(**cfg, q_shard=5, seed=2101, dtype="bf16")
    q, k_all, v_all = (to_gpu(inp[x], "bf16") for x in ("q", "k_all", "v_all"))
    o = torch.empty_like(q)
    lse = torch.empty((1, 32, 1024), device="cuda", dtype=torch.float32)

    def run():
        ra.ring_fwd_noalloc(q, k_all, v_all, q_shard=5, causal=True, layout="striped", out=o, lse_out=lse)
    _replays_equal(run, [o, lse], "ring_fwd_noalloc graph")


def test_ring_bwd_graph_replays():
    cfg = dict(b=1, L=512, h=8, n_kv=2, d=128, N=4)
    inp = make_inputs(**cfg, q_shard=2, seed=2102, dtype="bf16", with_dout=True)
    q, k_all, v_all, dout = (to_gpu(inp[x], "bf16") for x in ("q", "k_all", "v_all", "dout"))
    o, lse = ra.ring_fwd(q, k_all, v_all, q_shard=2, causal=True, layout="contiguous")
    ws = torch.empty(ra.ring_bwd_workspace_bytes(q, k_all, causal=True, layout="contiguous"), device="cuda",
                     dtype=torch.uint8)
    outs = [torch.empty((1, 512, 8, 128), device="cuda", dtype=torch.float32),
            torch.empty((4, 1, 512, 2, 128), device="cuda", dtype=torch.float32),
            torch.empty((4, 1, 512, 2, 128), device="cuda", dtype=torch.float32)]

    def run():   # contiguous causal shard 2: steps 0..2 live, step 3 dead (its shard's dK, dV filled)
        ra.ring_bwd(q, k_all, v_all, o, dout, lse, q_shard=2, causal=True, layout="contiguous", workspace=ws,
                    out=tuple(outs))
    _replays_equal(run, outs, "ring_bwd graph")

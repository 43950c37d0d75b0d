"""Pins of the oracle's sequence partition, ring schedule and work counts against the
pages' worked examples and closed forms."""
import numpy as np
import pytest

from oracle import LAYOUTS, allowed_pairs, ring_order, shard_tokens


def test_page3_eight_token_example(golden):
    g = golden("layout_example.json")
    for layout in ("contiguous", "striped"):
        got = [list(map(int, t)) for t in shard_tokens(layout, g["N"], g["L"])]
        assert got == g[layout], layout


def test_page1_zigzag_chunk_assignment(golden):
    g = golden("zigzag_example.json")
    N = g["N"]
    toks = shard_tokens("zigzag", N, 2)          # chunk size 1 -> tokens are chunk ids
    for p, chunks in g["chunks_per_device"].items():
        assert list(map(int, toks[int(p)])) == chunks
    # equal work: N/2 full-block equivalents per device (L large, diagonal ~ half block)
    L = 400
    for p in range(N):
        eq = allowed_pairs("zigzag", N, L, p) / (L * L)      # in L x L block units
        assert eq == pytest.approx(g["block_equivalents_per_device"], abs=1e-2)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("N,L", [(1, 4), (3, 4), (4, 6), (8, 8)])
def test_partition_is_a_bijection_in_increasing_local_order(layout, N, L):
    toks = shard_tokens(layout, N, L)
    allp = np.sort(np.concatenate(toks))
    np.testing.assert_array_equal(allp, np.arange(N * L))
    for t in toks:
        assert t.size == L and np.all(np.diff(t) > 0)


def test_ring_schedule_matches_page4_block_index():
    """Page 4, 'The Ring Communication Protocol': at iteration idx device i holds the block
    of device (i - idx) mod N; step 0 is the device's own block."""
    for N in (1, 2, 5, 8):
        for i in range(N):
            assert ring_order(N, i) == [(i - idx) % N for idx in range(N)]


def test_pair_counts_closed_forms():
    """Contiguous shard i: i L^2 + L(L+1)/2 (W_i proportional to i+1);
    striped shard p: N L (L-1)/2 + L (p+1); zigzag: N L^2 / 2 + L/2 for every p;
    all shards together: S (S+1) / 2."""
    for N, L in [(2, 4), (4, 6), (8, 16)]:
        S = N * L
        tot = {lay: 0 for lay in LAYOUTS}
        for p in range(N):
            c = allowed_pairs("contiguous", N, L, p)
            s = allowed_pairs("striped", N, L, p)
            z = allowed_pairs("zigzag", N, L, p)
            assert c == p * L * L + L * (L + 1) // 2
            assert s == N * L * (L - 1) // 2 + L * (p + 1)
            assert 2 * z == N * L * L + L
            tot["contiguous"] += c
            tot["striped"] += s
            tot["zigzag"] += z
        for lay in LAYOUTS:
            assert tot[lay] == S * (S + 1) // 2
        assert allowed_pairs("striped", N, L, 0, causal=False) == L * S


def test_contiguous_live_steps_expose_imbalance():
    """With N = 8 contiguous shards, shard 0 has 1 live ring step and shard 7 has 8."""
    N, L = 8, 16
    for i in range(N):
        live = sum(allowed_pairs("contiguous", N, L, i, src) > 0 for src in range(N))
        assert live == i + 1


def test_zigzag_chunk_pairs_live_per_step():
    """Off the diagonal step exactly 2 of the 4 (L/2)-chunk pairs are live; on the diagonal
    step (src = i) 3 are, two of them the half-masked diagonal chunks."""
    N, L = 4, 8
    C = L // 2
    for i in range(N):
        for src in range(N):
            live = 0
            for a in range(2):
                for c in range(2):
                    qi = shard_tokens("zigzag", N, L)[i][a * C:(a + 1) * C]
                    ks = shard_tokens("zigzag", N, L)[src][c * C:(c + 1) * C]
                    live += int(ks.min() <= qi.max())
            assert live == (3 if src == i else 2)


def test_page3_causal_utilisation_table(golden):
    """Utilisation of contiguous causal sharding = mean work / max work.
    Counting live blocks (diagonal as a whole block) gives (N+1)/2N; counting pairs
    (diagonal as a half block, large L) gives N/(2N-1)."""
    g = golden("causal_utilisation.json")
    tol = g["printed_precision_percent"]
    for N_s, pct in g["whole_diagonal_percent"].items():
        N, L = int(N_s), 4
        W = [sum(allowed_pairs("contiguous", N, L, i, src) > 0 for src in range(N))
             for i in range(N)]
        assert 100 * np.mean(W) / max(W) == pytest.approx(pct, abs=tol)
    for N_s, pct in g["half_diagonal_percent"].items():
        N, L = int(N_s), 512
        W = [allowed_pairs("contiguous", N, L, i) for i in range(N)]
        assert 100 * np.mean(W) / max(W) == pytest.approx(pct, abs=tol)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_usp_tokens_reduce_to_the_ring_and_all_to_all_layouts(layout):
    """The two-dimensional arrangement: N_h = 1 is the ring's sharding, N_s = 1 the all-to-all
    path's contiguous one; every split is a bijection onto [0, S) whose N_h pieces of a ring
    shard concatenate to that ring shard."""
    from oracle import usp_tokens
    L = 6
    for N in (1, 2, 4, 6):
        assert all(np.array_equal(a, b) for a, b in zip(usp_tokens(layout, 1, N, L), shard_tokens(layout, N, L)))
        flat = usp_tokens(layout, N, 1, L)
        assert all(np.array_equal(t, np.arange(g * L, (g + 1) * L)) for g, t in enumerate(flat))
    for N_h, N_s in ((2, 2), (2, 3), (3, 2), (4, 2)):
        toks = usp_tokens(layout, N_h, N_s, L)
        S = N_h * N_s * L
        assert np.array_equal(np.sort(np.concatenate(toks)), np.arange(S))
        ring = shard_tokens(layout, N_s, N_h * L)
        for r in range(N_s):
            assert np.array_equal(np.concatenate(toks[r * N_h:(r + 1) * N_h]), ring[r])


def test_usp_tokens_small_example():
    """8 tokens, 2 head groups x 2 sequence shards, striped: the ring shards are the even and
    the odd positions; each is split in two halves."""
    from oracle import usp_tokens
    toks = usp_tokens("striped", 2, 2, 2)
    assert [t.tolist() for t in toks] == [[0, 2], [4, 6], [1, 3], [5, 7]]

"""Pins of the fp64 oracle's forward (O, LSE), step and merge functions against facts fixed
by the pages and by the mathematics: closed forms, invariants, brute force on tiny inputs.

Each test is chosen so that a plausible slip in the oracle (a dropped scale, a transposed
operand, an exclusive causal boundary, a wrong GQA grouping, a missing rescale, a merge
that ignores the LSE) makes at least one of them fail.
"""
import itertools
import math

import numpy as np
import pytest

from oracle import (LAYOUTS, attend, brute_force_row, merge, online_blocks, ring_order,
                    shard_attention, shard_tokens, step_attention)

RNG = np.random.default_rng(12345)


def rand(*shape):
    return RNG.standard_normal(shape)


def global_order(x_all, layout, N):
    """Reassemble per-shard [N, b, L, ...] data into global token order [b, S, ...]."""
    toks = shard_tokens(layout, N, x_all.shape[2])
    S = N * x_all.shape[2]
    out = np.zeros((x_all.shape[1], S) + x_all.shape[3:])
    for j in range(N):
        out[:, toks[j]] = x_all[j]
    return out


# ----------------------------------------------------------------------------- closed forms
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("causal", [False, True])
def test_identical_keys_give_prefix_mean(layout, causal):
    """All keys equal -> every allowed key has the same logit, so O is the plain mean of the
    allowed values and LSE = scale * q.k + ln(#allowed)."""
    N, b, L, h, n_kv, d = 4, 1, 6, 2, 1, 8
    k0 = rand(d)
    k_all = np.broadcast_to(k0, (N, b, L, n_kv, d)).copy()
    v_all = rand(N, b, L, n_kv, d)
    v_glob = global_order(v_all, layout, N)                       # [b, S, n_kv, d]
    toks = shard_tokens(layout, N, L)
    for shard in range(N):
        q = rand(b, L, h, d)
        O, LSE = shard_attention(q, k_all, v_all, N=N, shard=shard, layout=layout, causal=causal)
        for t in range(L):
            P = toks[shard][t]
            n = P + 1 if causal else N * L
            mean_v = v_glob[0, :n, 0].mean(axis=0)
            for hq in range(h):
                np.testing.assert_allclose(O[0, t, hq], mean_v, rtol=1e-12, atol=1e-12)
                s = q[0, t, hq] @ k0 / math.sqrt(d)
                assert LSE[0, hq, t] == pytest.approx(s + math.log(n), abs=1e-12)


def test_single_key_returns_its_value():
    d = 5
    q, k, v = rand(1, 1, 1, d), rand(1, 1, 1, 1, d), rand(1, 1, 1, 1, d)
    O, LSE = shard_attention(q, k, v, N=1, shard=0, causal=True)
    np.testing.assert_allclose(O[0, 0, 0], v[0, 0, 0, 0], rtol=0, atol=1e-15)
    assert LSE[0, 0, 0] == pytest.approx(float(q[0, 0, 0] @ k[0, 0, 0, 0]) / math.sqrt(d), abs=1e-14)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_causal_first_token_sees_only_itself(layout):
    """Global position 0 may attend only to itself (inclusive mask): O = V_0 exactly."""
    N, b, L, h, n_kv, d = 4, 1, 4, 2, 2, 6
    q, k_all, v_all = rand(b, L, h, d), rand(N, b, L, n_kv, d), rand(N, b, L, n_kv, d)
    toks = shard_tokens(layout, N, L)
    owner = [j for j in range(N) if 0 in toks[j]][0]
    t0 = int(np.where(toks[owner] == 0)[0][0])
    O, LSE = shard_attention(q, k_all, v_all, N=N, shard=owner, layout=layout, causal=True)
    for hq in range(h):
        g = hq // (h // n_kv)
        np.testing.assert_allclose(O[0, t0, hq], v_all[owner, 0, t0, g], rtol=0, atol=1e-14)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_give_uniform_weights(layout, causal):
    """Q = 0 -> all logits 0 -> uniform weights: O = mean of allowed values, LSE = ln(n)."""
    N, b, L, h, n_kv, d = 3, 2, 4, 4, 2, 3
    q = np.zeros((b, L, h, d))
    k_all, v_all = rand(N, b, L, n_kv, d), rand(N, b, L, n_kv, d)
    v_glob = global_order(v_all, layout, N)
    csum = np.cumsum(v_glob, axis=1)                                # prefix sums over positions
    toks = shard_tokens(layout, N, L)
    for shard in range(N):
        O, LSE = shard_attention(q, k_all, v_all, N=N, shard=shard, layout=layout, causal=causal)
        for t in range(L):
            n = toks[shard][t] + 1 if causal else N * L
            for hq in range(h):
                g = hq // (h // n_kv)
                np.testing.assert_allclose(O[:, t, hq], csum[:, n - 1, g] / n, rtol=1e-12, atol=1e-12)
                np.testing.assert_allclose(LSE[:, hq, t], math.log(n), rtol=0, atol=1e-12)


def test_two_keys_with_known_weight_ratio():
    """q.k2 * (1/sqrt d) - q.k1 * (1/sqrt d) = ln 3 -> weights 1/4 and 3/4, LSE = ln 4.
    Pins the 1/sqrt(d) scale (d = 4 -> scale 1/2) and the exponential."""
    d = 4
    q = np.array([2 * math.log(3.0), 0, 0, 0])
    keys = np.array([[0.0, 0, 0, 0], [1.0, 0, 0, 0]])
    vals = np.array([[1.0, 0.0], [0.0, 1.0]])
    O, LSE = attend(q[None], np.array([5]), keys, vals, np.array([0, 1]), causal=False,
                    scale=1 / math.sqrt(d))
    np.testing.assert_allclose(O[0], [0.25, 0.75], rtol=0, atol=1e-15)
    assert LSE[0] == pytest.approx(math.log(4.0), abs=1e-15)
    # the same query through the shard-level entry, keys as two shards of one token each
    O2, LSE2 = shard_attention(q.reshape(1, 1, 1, 4), keys.reshape(2, 1, 1, 1, 4),
                               np.array([[1.0, 0, 0, 0], [0, 1.0, 0, 0]]).reshape(2, 1, 1, 1, 4),
                               N=2, shard=0, causal=False)
    np.testing.assert_allclose(O2[0, 0, 0, :2], [0.25, 0.75], rtol=0, atol=1e-15)


def test_causal_boundary_is_inclusive_and_directional():
    """Key at the query's own position is allowed, the next one is not."""
    d = 2
    q = np.array([[0.0, 0.0]])
    keys = np.zeros((3, d))
    vals = np.array([[1.0], [10.0], [100.0]])
    O, LSE = attend(q, np.array([1]), keys, vals, np.array([0, 1, 2]), causal=True, scale=1.0)
    assert O[0, 0] == pytest.approx(5.5)          # mean of positions 0 and 1 only
    assert LSE[0] == pytest.approx(math.log(2.0))


# ----------------------------------------------------------------------------- brute force
@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("causal", [False, True])
def test_matches_pure_python_brute_force(layout, causal):
    N, b, L, h, n_kv, d = 3, 1, 4, 4, 2, 3
    q, k_all, v_all = rand(b, L, h, d), rand(N, b, L, n_kv, d), rand(N, b, L, n_kv, d)
    scale = 0.7
    toks = shard_tokens(layout, N, L)
    for shard in range(N):
        O, LSE = shard_attention(q, k_all, v_all, N=N, shard=shard, layout=layout,
                                 causal=causal, scale=scale)
        for t in range(L):
            for hq in range(h):
                g = hq // (h // n_kv)
                keys, vals, allowed = [], [], []
                for j in range(N):
                    for u in range(L):
                        keys.append(list(k_all[j, 0, u, g]))
                        vals.append(list(v_all[j, 0, u, g]))
                        allowed.append((not causal) or toks[j][u] <= toks[shard][t])
                o_bf, lse_bf = brute_force_row(list(q[0, t, hq]), keys, vals, allowed, scale)
                np.testing.assert_allclose(O[0, t, hq], o_bf, rtol=1e-12, atol=1e-13)
                assert LSE[0, hq, t] == pytest.approx(lse_bf, abs=1e-12)


# ----------------------------------------------------------------------------- invariants
def test_noncausal_invariant_to_kv_shard_order():
    N, b, L, h, n_kv, d = 4, 1, 5, 2, 1, 4
    q, k_all, v_all = rand(b, L, h, d), rand(N, b, L, n_kv, d), rand(N, b, L, n_kv, d)
    O, LSE = shard_attention(q, k_all, v_all, N=N, shard=1, causal=False)
    for perm in [(3, 2, 1, 0), (1, 3, 0, 2)]:
        Op, LSEp = shard_attention(q, k_all[list(perm)], v_all[list(perm)], N=N, shard=1,
                                   causal=False)
        np.testing.assert_allclose(Op, O, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(LSEp, LSE, rtol=1e-12, atol=1e-13)


def test_value_affine_equivariance():
    N, b, L, h, n_kv, d = 2, 1, 4, 2, 1, 3
    q, k_all, v_all = rand(b, L, h, d), rand(N, b, L, n_kv, d), rand(N, b, L, n_kv, d)
    a, c = 2.5, rand(d)
    O, _ = shard_attention(q, k_all, v_all, N=N, shard=1, layout="striped", causal=True)
    O2, _ = shard_attention(q, k_all, a * v_all + c, N=N, shard=1, layout="striped", causal=True)
    np.testing.assert_allclose(O2, a * O + c, rtol=1e-12, atol=1e-12)


def test_key_shift_invariance():
    """K += u for every key leaves O unchanged and shifts LSE by scale * q.u."""
    N, b, L, h, n_kv, d = 2, 1, 4, 2, 1, 3
    q, k_all, v_all = rand(b, L, h, d), rand(N, b, L, n_kv, d), rand(N, b, L, n_kv, d)
    u = rand(d)
    O, LSE = shard_attention(q, k_all, v_all, N=N, shard=0, layout="zigzag", causal=True)
    O2, LSE2 = shard_attention(q, k_all + u, v_all, N=N, shard=0, layout="zigzag", causal=True)
    np.testing.assert_allclose(O2, O, rtol=1e-11, atol=1e-12)
    shift = np.einsum("bthd,d->bht", q, u) / math.sqrt(d)
    np.testing.assert_allclose(LSE2, LSE + shift, rtol=1e-12, atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv_heads():
    N, b, L, h, n_kv, d = 2, 1, 3, 4, 2, 3
    q, k_all, v_all = rand(b, L, h, d), rand(N, b, L, n_kv, d), rand(N, b, L, n_kv, d)
    O, LSE = shard_attention(q, k_all, v_all, N=N, shard=1, layout="striped", causal=True)
    rep = [0, 0, 1, 1]
    O2, LSE2 = shard_attention(q, k_all[:, :, :, rep], v_all[:, :, :, rep], N=N, shard=1,
                               layout="striped", causal=True)
    np.testing.assert_allclose(O2, O, rtol=0, atol=0)
    np.testing.assert_allclose(LSE2, LSE, rtol=0, atol=0)


def test_gqa_groups_are_consecutive_heads():
    """Values constant per KV head: query head hq must read KV head hq // (h // n_kv)."""
    N, b, L, h, n_kv, d = 2, 1, 3, 8, 2, 2
    q, k_all = rand(b, L, h, d), rand(N, b, L, n_kv, d)
    v_all = np.zeros((N, b, L, n_kv, d))
    for g in range(n_kv):
        v_all[:, :, :, g, :] = g + 1.0
    O, _ = shard_attention(q, k_all, v_all, N=N, shard=0, causal=False)
    for hq in range(h):
        np.testing.assert_allclose(O[0, :, hq], hq // (h // n_kv) + 1.0, rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------- online softmax
def test_online_recurrence_equals_full_softmax_for_every_split_and_order():
    """The pages' recurrence over any split of the keys into blocks, visited in any order,
    gives the plain softmax result (brute force over all splits of C = 7 keys)."""
    C, R, d = 7, 3, 4
    q, keys, vals = rand(R, d), rand(C, d), rand(C, 2)
    pos_q, pos_k = np.array([2, 4, 6]), np.arange(C)
    for causal in (False, True):
        O_ref, LSE_ref = attend(q, pos_q, keys, vals, pos_k, causal=causal, scale=0.5)
        for cuts in itertools.product([0, 1], repeat=C - 1):
            edges = [0] + [i + 1 for i, c in enumerate(cuts) if c] + [C]
            blocks = [(keys[a:z], vals[a:z], pos_k[a:z]) for a, z in zip(edges, edges[1:])]
            orders = list(itertools.permutations(range(len(blocks))))[:6]
            for order in orders:
                O, LSE = online_blocks(q, pos_q, [blocks[i] for i in order], causal=causal,
                                       scale=0.5)
                np.testing.assert_allclose(O, O_ref, rtol=1e-12, atol=1e-13)
                np.testing.assert_allclose(LSE, LSE_ref, rtol=1e-12, atol=1e-13)


def test_online_recurrence_without_rescale_would_differ():
    """Guard that the test above bites: dropping the exp(m_old - m_new) factor changes the
    result whenever the running max grows."""
    q = np.array([[1.0]])
    keys = np.array([[0.0], [5.0]])
    vals = np.array([[1.0], [2.0]])
    blocks = [(keys[:1], vals[:1], np.array([0])), (keys[1:], vals[1:], np.array([1]))]
    O, _ = online_blocks(q, np.array([1]), blocks, causal=False, scale=1.0)
    O_ref, _ = attend(q, np.array([1]), keys, vals, np.array([0, 1]), causal=False, scale=1.0)
    np.testing.assert_allclose(O, O_ref, rtol=1e-14)
    # unscaled accumulation: weights exp(0-0) for block 1 and exp(5-5) for block 2 -> 0.5/0.5
    assert abs(O_ref[0, 0] - 1.5) > 0.4


# ----------------------------------------------------------------------------- merge
def _rand_partial(b=1, R=3, h=2, d=4):
    return rand(b, R, h, d), rand(b, h, R)


def test_merge_worked_example():
    """l_a = e^0 = 1, l_b = e^{ln 3} = 3  ->  O = (O_a + 3 O_b) / 4, LSE = ln 4."""
    oa, ob = np.ones((1, 1, 1, 2)), np.array([[[[0.0, 4.0]]]])
    O, LSE = merge(oa, np.array([[[0.0]]]), ob, np.array([[[math.log(3.0)]]]))
    np.testing.assert_allclose(O[0, 0, 0], [0.25, 3.25], rtol=1e-15)
    assert LSE[0, 0, 0] == pytest.approx(math.log(4.0), abs=1e-15)


def test_merge_is_commutative_associative_with_identity():
    a, b_, c = _rand_partial(), _rand_partial(), _rand_partial()
    ident = (np.zeros_like(a[0]), np.full_like(a[1], -np.inf))
    ab = merge(*a, *b_)
    ba = merge(*b_, *a)
    np.testing.assert_allclose(ab[0], ba[0], rtol=1e-14)
    np.testing.assert_allclose(ab[1], ba[1], rtol=1e-14)
    l1 = merge(*merge(*a, *b_), *c)
    l2 = merge(*a, *merge(*b_, *c))
    np.testing.assert_allclose(l1[0], l2[0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l1[1], l2[1], rtol=1e-13)
    ai = merge(*a, *ident)
    np.testing.assert_array_equal(ai[0], a[0])
    np.testing.assert_array_equal(ai[1], a[1])
    ee = merge(*ident, *ident)
    assert np.all(ee[0] == 0) and np.all(np.isneginf(ee[1]))


def test_merge_survives_huge_lse():
    """Large logits (the overflow hazard of an unrescaled sum) merge without inf/nan."""
    oa, ob = np.ones((1, 1, 1, 1)), np.zeros((1, 1, 1, 1))
    O, LSE = merge(oa, np.array([[[1000.0]]]), ob, np.array([[[1000.0]]]))
    assert O[0, 0, 0, 0] == pytest.approx(0.5) and LSE[0, 0, 0] == pytest.approx(1000 + math.log(2))


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("causal", [False, True])
def test_ring_of_step_merges_equals_whole_sequence(layout, causal):
    """Merging the per-step partials in ring order gives the whole-sequence result."""
    N, b, L, h, n_kv, d = 4, 1, 4, 4, 2, 3
    q, k_all, v_all = rand(b, L, h, d), rand(N, b, L, n_kv, d), rand(N, b, L, n_kv, d)
    for shard in range(N):
        O_ref, LSE_ref = shard_attention(q, k_all, v_all, N=N, shard=shard, layout=layout,
                                         causal=causal)
        acc = (np.zeros_like(O_ref), np.full_like(LSE_ref, -np.inf))
        for src in ring_order(N, shard):
            part = step_attention(q, k_all[src], v_all[src], N=N, q_shard=shard,
                                  kv_shard=src, layout=layout, causal=causal)
            acc = merge(*acc, *part)
        np.testing.assert_allclose(acc[0], O_ref, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(acc[1], LSE_ref, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------- empty rows
def test_contiguous_future_shard_is_fully_masked():
    N, b, L, h, n_kv, d = 4, 1, 3, 2, 1, 2
    q, k, v = rand(b, L, h, d), rand(b, L, n_kv, d), rand(b, L, n_kv, d)
    O, LSE = step_attention(q, k, v, N=N, q_shard=1, kv_shard=2, layout="contiguous", causal=True)
    assert np.all(O == 0) and np.all(np.isneginf(LSE))


def test_striped_later_shard_masks_only_first_row():
    """Striped: shard i's row 0 is global position i; shard src > i holds positions
    src, src+N, ... so row 0 sees none of them, row t sees t of them."""
    N, b, L, h, n_kv, d = 4, 1, 5, 1, 1, 2
    q, k, v = np.zeros((b, L, h, d)), rand(b, L, n_kv, d), rand(b, L, n_kv, d)
    O, LSE = step_attention(q, k, v, N=N, q_shard=1, kv_shard=3, layout="striped", causal=True)
    assert np.isneginf(LSE[0, 0, 0]) and np.all(O[0, 0] == 0)
    for t in range(1, L):
        assert LSE[0, 0, t] == pytest.approx(math.log(t))

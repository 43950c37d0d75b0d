"""Pins of the oracle's packed-document mask (page 3, section 5: documents packed end to end
in one window, a block-diagonal mask stopping attention across documents).  None of these
retypes the mask: each compares against an independent route (attending each document on
its own, other layouts, brute force with Python loops, closed-form pair counts)."""
import math

import numpy as np
import pytest

import synth
from oracle import (LAYOUTS, allowed_pairs, brute_force_row, document_of, shard_attention,
                    shard_grads, shard_tokens)


def _global_inputs(S, h, n_kv, d, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((1, S, h, d)), rng.standard_normal((1, S, n_kv, d)),
            rng.standard_normal((1, S, n_kv, d)), rng.standard_normal((1, S, h, d)))


def _sharded(x_global, layout, N, L, kv=True):
    toks = shard_tokens(layout, N, L)
    return np.stack([x_global[:, t] for t in toks]) if kv else [x_global[:, t] for t in toks]


DOCS = np.array([0, 7, 8, 19, 33, 40])      # lengths 7, 1, 11, 14, 7


@pytest.mark.parametrize("causal", [True, False])
def test_packed_window_equals_each_document_alone(causal):
    S, h, n_kv, d = 40, 4, 2, 8
    q, k, v, _ = _global_inputs(S, h, n_kv, d, 1)
    O, LSE = shard_attention(q, k[None], v[None], N=1, shard=0, causal=causal, docs=DOCS)
    for a, b in zip(DOCS[:-1], DOCS[1:]):
        o, lse = shard_attention(q[:, a:b], k[None, :, a:b], v[None, :, a:b], N=1, shard=0,
                                 causal=causal)
        np.testing.assert_allclose(O[:, a:b], o, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(LSE[:, :, a:b], lse, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_packed_result_by_global_position_is_layout_independent(causal):
    N, L, h, n_kv, d = 4, 10, 2, 1, 8
    S = N * L
    q, k, v, _ = _global_inputs(S, h, n_kv, d, 2)
    ref = None
    for layout in LAYOUTS:
        toks = shard_tokens(layout, N, L)
        k_all, v_all = _sharded(k, layout, N, L), _sharded(v, layout, N, L)
        O = np.zeros((1, S, h, d))
        LSE = np.zeros((1, h, S))
        for p in range(N):
            o, lse = shard_attention(q[:, toks[p]], k_all, v_all, N=N, shard=p, layout=layout,
                                     causal=causal, docs=DOCS)
            O[:, toks[p]] = o
            LSE[:, :, toks[p]] = lse
        if ref is None:
            ref = (O, LSE)
        else:
            np.testing.assert_allclose(O, ref[0], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(LSE, ref[1], rtol=1e-12, atol=1e-12)


def test_one_document_is_no_packing():
    N, L, h, n_kv, d = 3, 6, 2, 2, 4
    q, k, v, _ = _global_inputs(N * L, h, n_kv, d, 3)
    for layout in LAYOUTS:
        k_all, v_all = _sharded(k, layout, N, L), _sharded(v, layout, N, L)
        qs = _sharded(q, layout, N, L, kv=False)
        for p in range(N):
            a = shard_attention(qs[p], k_all, v_all, N=N, shard=p, layout=layout, causal=True)
            b = shard_attention(qs[p], k_all, v_all, N=N, shard=p, layout=layout, causal=True,
                                docs=np.array([0, N * L]))
            np.testing.assert_array_equal(a[0], b[0])
            np.testing.assert_array_equal(a[1], b[1])


def test_one_token_per_document_attends_to_itself():
    S, h, d = 12, 2, 4
    q, k, v, _ = _global_inputs(S, h, h, d, 4)
    O, LSE = shard_attention(q, k[None], v[None], N=1, shard=0, causal=False,
                             docs=np.arange(S + 1))
    np.testing.assert_allclose(O[0], v[0], rtol=1e-12, atol=1e-12)
    s_self = np.einsum("thd,thd->ht", q[0], k[0]) / math.sqrt(d)
    np.testing.assert_allclose(LSE[0], s_self, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_packed_pair_counts_closed_form(layout):
    N, L = 4, 10
    n = np.diff(DOCS)
    causal_total = sum(allowed_pairs(layout, N, L, p, None, True, docs=DOCS) for p in range(N))
    full_total = sum(allowed_pairs(layout, N, L, p, None, False, docs=DOCS) for p in range(N))
    assert causal_total == int((n * (n + 1) // 2).sum())
    assert full_total == int((n * n).sum())
    # per KV shard the counts add up to the whole-sequence count
    for p in range(N):
        assert sum(allowed_pairs(layout, N, L, p, j, True, docs=DOCS) for j in range(N)) == \
            allowed_pairs(layout, N, L, p, None, True, docs=DOCS)


def test_packed_rows_match_pure_python_brute_force():
    N, L, h, n_kv, d = 2, 8, 1, 1, 4
    S = N * L
    docs = np.array([0, 3, 11, 16])
    q, k, v, _ = _global_inputs(S, h, n_kv, d, 5)
    layout = "striped"
    toks = shard_tokens(layout, N, L)
    k_all, v_all = _sharded(k, layout, N, L), _sharded(v, layout, N, L)
    pos_k = np.concatenate(toks)
    keys = np.concatenate([k_all[j][0, :, 0] for j in range(N)])
    vals = np.concatenate([v_all[j][0, :, 0] for j in range(N)])
    for p in range(N):
        O, LSE = shard_attention(q[:, toks[p]], k_all, v_all, N=N, shard=p, layout=layout,
                                 causal=True, docs=docs)
        for r, P in enumerate(toks[p]):
            start = max(x for x in docs[:-1].tolist() if x <= P)   # the query's document start
            allowed = [bool(start <= int(c) <= int(P)) for c in pos_k]
            o, lse = brute_force_row(q[0, P, 0].tolist(), keys.tolist(), vals.tolist(), allowed,
                                     1 / math.sqrt(d))
            np.testing.assert_allclose(O[0, r, 0], o, rtol=1e-10, atol=1e-12)
            assert abs(LSE[0, 0, r] - lse) < 1e-10


@pytest.mark.parametrize("causal", [True, False])
def test_packed_gradients_equal_each_document_alone(causal):
    S, h, n_kv, d = 40, 4, 2, 8
    q, k, v, do = _global_inputs(S, h, n_kv, d, 6)
    dq, dk, dv = shard_grads(q, k[None], v[None], do, N=1, shard=0, causal=causal, docs=DOCS)
    for a, b in zip(DOCS[:-1], DOCS[1:]):
        gq, gk, gv = shard_grads(q[:, a:b], k[None, :, a:b], v[None, :, a:b], do[:, a:b], N=1,
                                 shard=0, causal=causal)
        np.testing.assert_allclose(dq[:, a:b], gq, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dk[0, :, a:b], gk[0], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dv[0, :, a:b], gv[0], rtol=1e-10, atol=1e-12)


def test_document_of_and_bounds_generator():
    b = synth.document_bounds(1000, seed=3, mean_len=50)
    assert b[0] == 0 and b[-1] == 1000 and np.all(np.diff(b) >= 1)
    np.testing.assert_array_equal(document_of([0, 6, 7, 8, 39], DOCS), [0, 0, 1, 2, 4])
    b2 = synth.document_bounds(1000, seed=3, mean_len=50)
    np.testing.assert_array_equal(b, b2)

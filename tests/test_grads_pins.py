"""Pins of the oracle's backward (shard_grads) by central finite differences of the oracle's
own forward (itself pinned in test_oracle_pins.py) and by exact identities."""
import numpy as np
import pytest

from oracle import shard_attention, shard_grads, shard_tokens

RNG = np.random.default_rng(777)


def _loss(q, k_all, v_all, dout, **kw):
    O, _ = shard_attention(q, k_all, v_all, **kw)
    return float(np.sum(O * dout))


@pytest.mark.parametrize("layout,causal", [("contiguous", False), ("striped", True),
                                           ("zigzag", True), ("contiguous", True)])
def test_gradients_match_central_differences(layout, causal):
    N, b, L, h, n_kv, d = 2, 1, 4, 4, 2, 3
    q = RNG.standard_normal((b, L, h, d))
    k_all = RNG.standard_normal((N, b, L, n_kv, d))
    v_all = RNG.standard_normal((N, b, L, n_kv, d))
    dout = RNG.standard_normal((b, L, h, d))
    kw = dict(N=N, shard=1, layout=layout, causal=causal)
    dq, dk, dv = shard_grads(q, k_all, v_all, dout, **kw)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k_all, dk), ("v", v_all, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            orig = x[idx]
            x[idx] = orig + eps
            fp = _loss(q, k_all, v_all, dout, **kw)
            x[idx] = orig - eps
            fm = _loss(q, k_all, v_all, dout, **kw)
            x[idx] = orig
            num[idx] = (fp - fm) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8, err_msg=name)


def test_gradient_identities():
    """Key-shift invariance -> sum of dK over all keys is 0 (per KV head); softmax rows sum to
    one -> sum of dV over all keys equals the sum of dO over the group's query rows."""
    N, b, L, h, n_kv, d = 3, 1, 5, 4, 2, 4
    q = RNG.standard_normal((b, L, h, d))
    k_all = RNG.standard_normal((N, b, L, n_kv, d))
    v_all = RNG.standard_normal((N, b, L, n_kv, d))
    dout = RNG.standard_normal((b, L, h, d))
    for layout, causal in (("striped", True), ("contiguous", False)):
        dq, dk, dv = shard_grads(q, k_all, v_all, dout, N=N, shard=2, layout=layout, causal=causal)
        np.testing.assert_allclose(dk.sum(axis=(0, 2)), 0.0, atol=1e-12)
        grp = h // n_kv
        for g in range(n_kv):
            np.testing.assert_allclose(dv.sum(axis=(0, 2))[:, g],
                                       dout[:, :, g * grp:(g + 1) * grp].sum(axis=(1, 2)),
                                       rtol=1e-12, atol=1e-12)


def test_first_token_query_gradient_is_zero():
    """Global position 0 attends only to itself: P = 1, so dS = 0 and dQ_0 = 0."""
    N, b, L, h, n_kv, d = 4, 1, 4, 2, 1, 3
    q = RNG.standard_normal((b, L, h, d))
    k_all = RNG.standard_normal((N, b, L, n_kv, d))
    v_all = RNG.standard_normal((N, b, L, n_kv, d))
    dout = RNG.standard_normal((b, L, h, d))
    for layout in ("contiguous", "striped", "zigzag"):
        toks = shard_tokens(layout, N, L)
        owner = [j for j in range(N) if 0 in toks[j]][0]
        dq, _, _ = shard_grads(q, k_all, v_all, dout, N=N, shard=owner, layout=layout, causal=True)
        t0 = int(np.where(toks[owner] == 0)[0][0])
        np.testing.assert_allclose(dq[0, t0], 0.0, atol=1e-14)


def test_zero_queries_value_gradient_is_prefix_weighted():
    """Q = 0 -> uniform weights 1/n_r over allowed keys: dV_c = sum over rows r that may see
    c of dO_r / n_r, with n_r = (global position of r) + 1 under the causal mask."""
    N, b, L, h, n_kv, d = 2, 1, 3, 1, 1, 2
    q = np.zeros((b, L, h, d))
    k_all = RNG.standard_normal((N, b, L, n_kv, d))
    v_all = RNG.standard_normal((N, b, L, n_kv, d))
    dout = RNG.standard_normal((b, L, h, d))
    toks = shard_tokens("striped", N, L)
    _, _, dv = shard_grads(q, k_all, v_all, dout, N=N, shard=1, layout="striped", causal=True)
    for j in range(N):
        for u in range(L):
            pk = toks[j][u]
            want = sum(dout[0, r, 0] / (toks[1][r] + 1) for r in range(L) if pk <= toks[1][r])
            np.testing.assert_allclose(dv[j, 0, u, 0], want, rtol=1e-12, atol=1e-14)


def test_dq_rows_match_finite_differences():
    """shard_dq_rows (a subset of rows) against central differences of the forward."""
    from oracle import shard_dq_rows
    N, b, L, h, n_kv, d = 2, 1, 4, 2, 1, 3
    q = RNG.standard_normal((b, L, h, d))
    k_all = RNG.standard_normal((N, b, L, n_kv, d))
    v_all = RNG.standard_normal((N, b, L, n_kv, d))
    dout = RNG.standard_normal((b, L, h, d))
    kw = dict(N=N, shard=0, layout="striped", causal=True)
    rows = [1, 3]
    got = shard_dq_rows(q, k_all, v_all, dout, rows, **kw)
    eps = 1e-6
    for ri, r in enumerate(rows):
        for hq in range(h):
            for e in range(d):
                orig = q[0, r, hq, e]
                q[0, r, hq, e] = orig + eps
                fp = _loss(q, k_all, v_all, dout, **kw)
                q[0, r, hq, e] = orig - eps
                fm = _loss(q, k_all, v_all, dout, **kw)
                q[0, r, hq, e] = orig
                assert got[0, ri, hq, e] == pytest.approx((fp - fm) / (2 * eps), rel=1e-6, abs=1e-8)


def _key_loss(q_sh, do_sh, k_all, v_all, shards, **kw):
    """sum over the listed query shards of sum(dO_i * O_i)."""
    return sum(float(np.sum(shard_attention(q_sh[n], k_all, v_all, shard=i, **kw)[0] * do_sh[n]))
               for n, i in enumerate(shards))


@pytest.mark.parametrize("layout,causal", [("striped", True), ("zigzag", True), ("contiguous", False)])
def test_key_grads_match_central_differences(layout, causal):
    """key_grads (selected keys, summed over two query shards and the GQA group) against
    central differences of the forward with respect to those keys' K and V entries."""
    from oracle import key_grads
    N, b, L, h, n_kv, d = 3, 1, 4, 4, 2, 3
    shards = [0, 2]
    q_sh = RNG.standard_normal((2, b, L, h, d))
    do_sh = RNG.standard_normal((2, b, L, h, d))
    k_all = RNG.standard_normal((N, b, L, n_kv, d))
    v_all = RNG.standard_normal((N, b, L, n_kv, d))
    cols = [(0, 0), (1, 3), (2, 1)]
    g = 1
    kw = dict(N=N, layout=layout, causal=causal)
    dk, dv = key_grads(q_sh, do_sh, k_all, v_all, query_shards=shards, kv_head=g, cols=cols,
                       row_block=3, **kw)
    eps = 1e-6
    for ci, (j, u) in enumerate(cols):
        for x, got in ((k_all, dk), (v_all, dv)):
            for e in range(d):
                orig = x[j, 0, u, g, e]
                x[j, 0, u, g, e] = orig + eps
                fp = _key_loss(q_sh, do_sh, k_all, v_all, shards, **kw)
                x[j, 0, u, g, e] = orig - eps
                fm = _key_loss(q_sh, do_sh, k_all, v_all, shards, **kw)
                x[j, 0, u, g, e] = orig
                assert got[0, ci, e] == pytest.approx((fp - fm) / (2 * eps), rel=1e-6, abs=1e-8)


@pytest.mark.parametrize("layout,causal,docs", [("striped", True, None), ("contiguous", True, None),
                                                ("zigzag", True, [0, 5, 6, 13, 24]),
                                                ("contiguous", False, None)])
def test_key_grads_equal_summed_shard_grads(layout, causal, docs):
    """Every key of every shard, over all query shards, b = 2, with small row blocks (so the
    per-block key trimming is exercised) and split row sets added together: equals the sum
    of shard_grads' per-KV-shard dK, dV over the query shards."""
    from oracle import key_grads
    N, b, L, h, n_kv, d = 3, 2, 8, 6, 2, 4
    q_sh = RNG.standard_normal((N, b, L, h, d))
    do_sh = RNG.standard_normal((N, b, L, h, d))
    k_all = RNG.standard_normal((N, b, L, n_kv, d))
    v_all = RNG.standard_normal((N, b, L, n_kv, d))
    kw = dict(N=N, layout=layout, causal=causal, docs=docs)
    want_k = np.zeros_like(k_all)
    want_v = np.zeros_like(v_all)
    for i in range(N):
        _, rk, rv = shard_grads(q_sh[i], k_all, v_all, do_sh[i], shard=i, **kw)
        want_k += rk
        want_v += rv
    cols = [(j, u) for j in range(N) for u in range(L)]
    for g in range(n_kv):
        parts = [key_grads(q_sh, do_sh, k_all, v_all, query_shards=list(range(N)), kv_head=g,
                           cols=cols, rows=rr, row_block=2, **kw)
                 for rr in (np.arange(0, 3), np.arange(3, L))]
        dk = parts[0][0] + parts[1][0]
        dv = parts[0][1] + parts[1][1]
        for ci, (j, u) in enumerate(cols):
            np.testing.assert_allclose(dk[:, ci], want_k[j, :, u, g], rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(dv[:, ci], want_v[j, :, u, g], rtol=1e-10, atol=1e-12)

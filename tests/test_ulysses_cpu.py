"""CPU checks of the all-to-all sequence-parallel path (page 3, sections 4.2 and 7): its byte
and work model against the page's printed figures, and the C-ABI's validation of it.  No
kernel is launched."""
import ctypes

import pytest

from ring_attention_long_amd import _lib, accounting
from test_abi_cpu import FAKE, _no_hip_device, _prob


def test_alltoall_bytes_match_page3(golden):
    """Page 3, section 4.2: with GQA (h = 32, n_kv = 8) one device receives ~0.587 GB in the
    two exchanges against the ring's 0.94 GB (ratio ~0.63); with MHA (n_kv = h) the
    exchanges come to 0.94 GB."""
    g = golden("alltoall_accounting.json")
    S, N, b, h, n_kv, d, p = g["S"], g["N"], g["b"], g["h"], g["n_kv"], g["d"], g["bytes_per_element"]
    u = accounting.ulysses_bytes_per_device(b, S, N, h, n_kv, d, p)
    r = accounting.ring_kv_bytes_per_pass(b, S, N, n_kv, d, p)
    assert u / 1e9 == pytest.approx(g["ulysses_gb_gqa"], abs=0.0005)
    assert r / 1e9 == pytest.approx(g["ring_gb_gqa"], abs=0.005)
    # exactly (2h + 2 n_kv) / (2 N n_kv) = 0.625; the page rounds 0.587 / 0.94 = 0.6245 to 0.63
    assert u / r == pytest.approx(g["ulysses_over_ring_gqa"], abs=0.01)
    assert accounting.ulysses_bytes_per_device(b, S, N, h, h, d, p) / 1e9 == pytest.approx(g["ulysses_gb_mha"], abs=0.005)
    # the ring's bytes scale with n_kv, the exchanges' with h + n_kv
    assert accounting.ring_kv_bytes_per_pass(b, S, N, h, d, p) == 4 * r


def test_alltoall_work_equals_ring_work_per_device():
    """Page 3, section 7: a device's attention after the exchange, 4 b S^2 (h/N) d, equals a
    ring device's N steps of 4 b L S h d (L = S/N)."""
    for (b, S, N, h, d) in ((1, 262144, 8, 32, 128), (2, 4096, 4, 8, 64)):
        L = S // N
        ring = N * 4 * b * L * L * h * d
        assert accounting.ulysses_flops_noncausal(b, S, N, h, d) == ring


def test_ulysses_workspace_size():
    """Gathered Q (h/N heads) and K, V (n_kv/N heads) of the whole sequence in the input
    dtype, an fp32 output and the fp32 LSE, each padded to 256 bytes."""
    lib = _lib.lib()
    pad = lambda x: (x + 255) // 256 * 256  # noqa: E731
    for dtype, es in ((1, 2), (0, 4)):
        p = _prob(b=2, L=100, h=8, n_kv=4, N=4, dtype=dtype, layout=1)
        S = 400
        want = (pad(2 * S * 2 * 128 * es) + 2 * pad(2 * S * 1 * 128 * es) + pad(2 * S * 2 * 128 * 4)
                + pad(2 * 2 * S * 4))
        if dtype == 1:     # the second accumulator (bf16, whole sequence <= 4096 tokens)
            want += pad(2 * S * 2 * 128 * 4) + pad(2 * 2 * S * 4)
        assert lib.ra_ulysses_fwd_workspace(ctypes.byref(p)) == want


@pytest.mark.parametrize("kw,status", [
    (dict(h=6, n_kv=2, N=4), _lib.RA_ERR_INVALID_ARG),      # h not a multiple of N
    (dict(h=8, n_kv=2, N=4), _lib.RA_ERR_INVALID_ARG),      # n_kv not a multiple of N
    (dict(d=96), _lib.RA_ERR_UNSUPPORTED),
    (dict(layout=2, L=127), _lib.RA_ERR_INVALID_ARG),
])
def test_ulysses_rejects_bad_problems(kw, status):
    lib = _lib.lib()
    base = dict(h=8, n_kv=4, N=4)
    base.update(kw)
    p = _prob(**base)
    assert lib.ra_ulysses_fwd_workspace(ctypes.byref(p)) == 0
    st = lib.ra_ulysses_fwd(ctypes.byref(p), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert st == status
    assert lib.ra_last_error()


def test_ulysses_rejects_bad_arguments():
    lib = _lib.lib()
    p = _prob(h=8, n_kv=4, N=4)
    need = lib.ra_ulysses_fwd_workspace(ctypes.byref(p))
    assert need > 0
    call = lambda g, q=FAKE, ws=need, lse=FAKE: lib.ra_ulysses_fwd(  # noqa: E731
        ctypes.byref(p), g, q, FAKE, FAKE, FAKE, lse, FAKE, ws, None)
    assert call(4) == _lib.RA_ERR_INVALID_ARG and b"head_group" in lib.ra_last_error()
    assert call(-1) == _lib.RA_ERR_INVALID_ARG
    assert call(0, q=None) == _lib.RA_ERR_INVALID_ARG and b"q_all is NULL" in lib.ra_last_error()
    assert call(0, q=ctypes.c_void_p(0x10008)) == _lib.RA_ERR_INVALID_ARG
    second = 512 * 2 * 128 * 4 + 2 * 512 * 4     # the optional second accumulator (S = 512, 2 heads)
    assert call(0, ws=need - second - 1) == _lib.RA_ERR_WORKSPACE
    tm = _lib.RaUlyssesTiming()
    assert lib.ra_ulysses_fwd_timed(ctypes.byref(p), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, None,
                                    None) == _lib.RA_ERR_INVALID_ARG
    assert lib.ra_ulysses_fwd_timed(ctypes.byref(p), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - second - 1, None,
                                    ctypes.byref(tm)) == _lib.RA_ERR_WORKSPACE
    # packed documents are not part of this path
    pd = _prob(h=8, n_kv=4, N=4)
    pd.doc_begin = pd.doc_end = FAKE.value
    assert lib.ra_ulysses_fwd_workspace(ctypes.byref(pd)) == 0
    assert lib.ra_ulysses_fwd(ctypes.byref(pd), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need, None) == \
        _lib.RA_ERR_UNSUPPORTED
    if _no_hip_device():                      # valid arguments reach the first launch
        assert call(3) == _lib.RA_ERR_HIP
        assert b"device" in lib.ra_last_error().lower()


def test_ulysses_bwd_workspace_and_validation():
    """The backward's workspace: Q, O, dO (h/N heads) and K, V (n_kv/N heads) of the whole
    sequence in bf16, LSE and D, and the fp32 dQ, dK, dV, each padded to 256 bytes."""
    lib = _lib.lib()
    pad = lambda x: (x + 255) // 256 * 256  # noqa: E731
    p = _prob(b=1, L=100, h=8, n_kv=4, N=4)
    S = 400
    want = (3 * pad(S * 2 * 128 * 2) + 2 * pad(S * 1 * 128 * 2) + 2 * pad(2 * S * 4) + pad(S * 2 * 128 * 4)
            + 2 * pad(S * 1 * 128 * 4))
    need = lib.ra_ulysses_bwd_workspace(ctypes.byref(p))
    assert need == want
    call = lambda g, prob=p, ws=need, q=FAKE: lib.ra_ulysses_bwd(  # noqa: E731
        ctypes.byref(prob), g, q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None)
    assert call(4) == _lib.RA_ERR_INVALID_ARG
    assert call(0, q=None) == _lib.RA_ERR_INVALID_ARG
    assert call(0, ws=need - 1) == _lib.RA_ERR_WORKSPACE
    bad = _prob(b=1, L=100, h=6, n_kv=2, N=4)
    assert lib.ra_ulysses_bwd_workspace(ctypes.byref(bad)) == 0 and call(0, prob=bad) == _lib.RA_ERR_INVALID_ARG
    f32 = _prob(b=1, L=100, h=8, n_kv=4, N=4, dtype=0)
    assert lib.ra_ulysses_bwd_workspace(ctypes.byref(f32)) == 0 and call(0, prob=f32) == _lib.RA_ERR_UNSUPPORTED
    if _no_hip_device():
        assert call(1) == _lib.RA_ERR_HIP


def test_usp_bytes_between_ring_and_all_to_all(golden):
    """Page 3, section 8's table: the two-dimensional arrangement receives between the ring's
    (N-1)/N 2 S n_kv d p and the all-to-all's (N-1)/N (S/N)(2h + 2 n_kv) d p, by the split;
    its limits are those two figures (0.94 and 0.587 GB at the page's shapes)."""
    g = golden("alltoall_accounting.json")
    S, b, N, h, n_kv, d, p = (g[k] for k in ("S", "b", "N", "h", "n_kv", "d", "bytes_per_element"))
    ring = accounting.usp_bytes_per_device(b, S, 1, N, h, n_kv, d, p)
    a2a = accounting.usp_bytes_per_device(b, S, N, 1, h, n_kv, d, p)
    assert ring == pytest.approx(accounting.ring_kv_bytes_per_pass(b, S, N, n_kv, d, p))
    assert a2a == pytest.approx(accounting.ulysses_bytes_per_device(b, S, N, h, n_kv, d, p))
    assert round(ring / 1e9, 2) == g["ring_gb_gqa"] and round(a2a / 1e9, 3) == g["ulysses_gb_gqa"]
    for N_h, N_s in ((2, 4), (4, 2)):
        mid = accounting.usp_bytes_per_device(b, S, N_h, N_s, h, n_kv, d, p)
        assert a2a < mid < ring
    # more head groups move more of the traffic into the (cheaper here) all-to-all
    assert accounting.usp_bytes_per_device(b, S, 4, 2, h, n_kv, d, p) < \
        accounting.usp_bytes_per_device(b, S, 2, 4, h, n_kv, d, p)


def test_usp_workspace_and_validation():
    """The two-dimensional path: workspace = the ring shard's gathered Q, K and V of every ring
    shard (head group), an fp32 output, the LSE and the ring's two staging buffers; both
    dimensions must divide; bad ranks, pointers and workspaces are refused before any launch."""
    lib = _lib.lib()
    pad = lambda x: (x + 255) // 256 * 256  # noqa: E731
    p = _prob(L=100, h=8, n_kv=4, N=4, layout=2)                 # N_h = 2, N_s = 2: ring shards of 200 tokens
    Lr, Hg, Kg, Ns = 200, 4, 2, 2
    want = pad(Lr * Hg * 128 * 2) + 2 * pad(Ns * Lr * Kg * 128 * 2) + pad(Lr * Hg * 128 * 4) + pad(Hg * Lr * 4) \
        + 4 * pad(Lr * Kg * 128 * 2) + pad(Lr * Hg * 128 * 4) + pad(Hg * Lr * 4)   # last two: second accumulator
    assert lib.ra_usp_fwd_workspace(ctypes.byref(p), 2) == want
    few_kv = _prob(L=100, h=8, n_kv=2, N=4)
    for pp, n_hg, why in ((p, 3, b"divide"), (p, 8, b"divide"), (p, 0, b"divide"), (few_kv, 4, b"multiples")):
        assert lib.ra_usp_fwd_workspace(ctypes.byref(pp), n_hg) == 0
        assert lib.ra_usp_fwd(ctypes.byref(pp), n_hg, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None,
                              None) == _lib.RA_ERR_INVALID_ARG
        assert why in lib.ra_last_error()
    odd = _prob(L=3, h=8, n_kv=4, N=4, layout=2)                  # zigzag ring shard of 3 tokens (N_h = 1)
    assert lib.ra_usp_fwd_workspace(ctypes.byref(odd), 1) == 0
    assert lib.ra_usp_fwd_workspace(ctypes.byref(odd), 2) > 0      # 6 tokens per ring shard: even
    call = lambda g, r, q=FAKE, ws=want: lib.ra_usp_fwd(  # noqa: E731
        ctypes.byref(p), 2, g, r, q, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None, None)
    assert call(2, 0) == _lib.RA_ERR_INVALID_ARG and b"head_group" in lib.ra_last_error()
    assert call(0, 2) == _lib.RA_ERR_INVALID_ARG and b"ring_rank" in lib.ra_last_error()
    assert call(0, 0, q=None) == _lib.RA_ERR_INVALID_ARG and b"q_all is NULL" in lib.ra_last_error()
    assert call(0, 0, ws=want - pad(Lr * Hg * 128 * 4) - pad(Hg * Lr * 4) - 1) == _lib.RA_ERR_WORKSPACE
    assert lib.ra_usp_fwd_timed(ctypes.byref(p), 2, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, want, None, None,
                                None) == _lib.RA_ERR_INVALID_ARG
    pd = _prob(L=100, h=8, n_kv=4, N=4)
    pd.doc_begin = pd.doc_end = FAKE.value
    assert lib.ra_usp_fwd(ctypes.byref(pd), 2, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, want, None, None) == \
        _lib.RA_ERR_UNSUPPORTED

"""CPU checks of the two backward schedules: the byte model of each step (page 4, "The Backward
Pass: Symmetric Ring Operation"; page 1, "The Backward Pass and Gradient Exchange") and the
C-ABI's validation of the key/value-stationary pass.  No kernel is launched."""
import ctypes

import pytest

from ring_attention_long_amd import _lib, accounting
from test_abi_cpu import FAKE, _no_hip_device, _prob


def test_rotating_step_moves_twice_the_forward_bytes_with_gradients_in_the_input_dtype():
    """Page 4: a backward step moves K, V and dK, dV, twice the forward's data; with fp32
    accumulators (as here) three times."""
    b, L, n_kv, d = 1, 32768, 8, 128
    fwd = accounting.kv_bytes_per_step(b, L, n_kv, d, 2)
    assert accounting.bwd_bytes_per_step_kv_rotating(b, L, n_kv, d, 2, acc_bytes=2) == 2 * fwd
    assert accounting.bwd_bytes_per_step_kv_rotating(b, L, n_kv, d, 2) == 3 * fwd


def test_stationary_schedule_bytes():
    """Per step the stationary schedule moves Q, dO (h heads), LSE, D and the fp32 dQ: for MHA
    that is less than the rotating schedule's K, V, dK, dV, for GQA (h = 4 n_kv) more."""
    b, L, d = 1, 8192, 128
    rot_mha = accounting.bwd_bytes_per_step_kv_rotating(b, L, 32, d, 2)
    sta_mha = accounting.bwd_bytes_per_step_kv_stationary(b, L, 32, d, 2)
    assert sta_mha < rot_mha
    assert sta_mha == b * L * 32 * d * 8 + 8 * b * 32 * L
    rot_gqa = accounting.bwd_bytes_per_step_kv_rotating(b, L, 8, d, 2)
    sta_gqa = accounting.bwd_bytes_per_step_kv_stationary(b, L, 32, d, 2)
    assert sta_gqa / rot_gqa == pytest.approx((32 * (8 * d + 8)) / (8 * 12 * d), rel=1e-12)
    assert sta_gqa > 2.6 * rot_gqa


def test_kv_stationary_workspace_and_validation():
    lib = _lib.lib()
    p = _prob(L=200, h=8, n_kv=2, N=3)
    pad = lambda x: (x + 255) // 256 * 256  # noqa: E731
    need = lib.ra_ring_bwd_kv_stationary_workspace(ctypes.byref(p))
    assert need == 2 * (2 * pad(200 * 8 * 128 * 2) + 2 * pad(8 * 200 * 4))
    call = lambda ks, ws=need, q=FAKE, prob=p: lib.ra_ring_bwd_kv_stationary(  # noqa: E731
        ctypes.byref(prob), ks, FAKE, FAKE, q, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None, None)
    assert call(3) == _lib.RA_ERR_INVALID_ARG and b"kv_shard" in lib.ra_last_error()
    assert call(0, q=None) == _lib.RA_ERR_INVALID_ARG and b"q_all is NULL" in lib.ra_last_error()
    assert call(0, ws=need - 1) == _lib.RA_ERR_WORKSPACE
    f32 = _prob(L=200, h=8, n_kv=2, N=3, dtype=0)
    assert lib.ra_ring_bwd_kv_stationary_workspace(ctypes.byref(f32)) == 0
    assert call(0, prob=f32) == _lib.RA_ERR_UNSUPPORTED
    docs = _prob(L=200, h=8, n_kv=2, N=3)
    docs.doc_begin = docs.doc_end = FAKE.value
    assert lib.ra_ring_bwd_kv_stationary_workspace(ctypes.byref(docs)) == 0
    assert call(0, prob=docs) == _lib.RA_ERR_UNSUPPORTED
    if _no_hip_device():                      # valid arguments reach the first launch
        assert call(1) == _lib.RA_ERR_HIP

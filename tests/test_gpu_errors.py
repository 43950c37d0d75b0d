"""On any error the library enqueues nothing and writes nothing: outputs filled with a
sentinel keep it when an entry point rejects its arguments on a GPU (the errors are all
found by validation, before any launch)."""
import ctypes

import pytest
import torch

import ring_attention_long_amd as ra
from ring_attention_long_amd import _lib
from gpu_helpers import announce

pytestmark = pytest.mark.gpu

SENTINEL = 7.0


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _filled(shape, dtype=torch.float32):
    return torch.full(shape, SENTINEL, device="cuda", dtype=dtype)


def _unchanged(*ts):
    torch.cuda.synchronize()
    return all(bool(torch.all(t == SENTINEL)) for t in ts)


def test_rejected_calls_write_nothing():
    lib = _lib.lib()
    b, L, h, n_kv, d, N = 1, 128, 8, 4, 128, 4
    q = torch.randn((b, L, h, d), device="cuda", dtype=torch.bfloat16)
    k_all = torch.randn((N, b, L, n_kv, d), device="cuda", dtype=torch.bfloat16)
    v_all = torch.randn_like(k_all)
    p = ra.make_problem(b=b, L=L, h=h, n_kv=n_kv, d=d, N=N, causal=True, layout="striped")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    announce("errors: ra_step_fwd with q_shard = N")
    o, lse = _filled((b, L, h, d)), _filled((b, h, L))
    assert lib.ra_step_fwd(ctypes.byref(p), N, 0, _p(q), _p(k_all[0]), _p(v_all[0]), _p(o), _p(lse), s) == \
        _lib.RA_ERR_INVALID_ARG
    assert _unchanged(o, lse)

    announce("errors: ra_ring_fwd with a workspace one byte short")
    p1 = _lib.RaProblem.from_buffer_copy(p)
    p1.steps_per_launch = 1
    need = lib.ra_ring_fwd_workspace(ctypes.byref(p1))
    # one launch per step (what the library falls back to when the slots of batched steps do
    # not fit) without the optional second accumulator of short shards (fp32 [b][L][h][d], LSE)
    need_min = need - (b * L * h * d * 4 + b * h * L * 4)
    ws = torch.empty(need, device="cuda", dtype=torch.uint8)
    o16 = _filled((b, L, h, d), torch.bfloat16)
    assert lib.ra_ring_fwd(ctypes.byref(p1), 0, _p(q), _p(k_all), _p(v_all), _p(o16), _p(lse), _p(ws),
                           need_min - 1, s, None) == _lib.RA_ERR_WORKSPACE
    assert _unchanged(o16, lse)
    ws = torch.empty(need, device="cuda", dtype=torch.uint8)
    o16 = _filled((b, L, h, d), torch.bfloat16)
    assert lib.ra_ring_fwd(ctypes.byref(p), 0, _p(q), _p(k_all), _p(v_all), _p(o16), _p(lse), _p(ws), need_min - 1,
                           s, None) == _lib.RA_ERR_WORKSPACE
    assert _unchanged(o16, lse)

    announce("errors: ra_step_bwd with kv_shard = -1")
    dq, dk, dv = _filled((b, L, h, d)), _filled((b, L, n_kv, d)), _filled((b, L, n_kv, d))
    dl = _filled((b, h, L))
    assert lib.ra_step_bwd(ctypes.byref(p), 0, -1, _p(q), _p(k_all[0]), _p(v_all[0]), _p(q), _p(lse), _p(dl),
                           _p(dq), _p(dk), _p(dv), s) == _lib.RA_ERR_INVALID_ARG
    assert _unchanged(dq, dk, dv)

    announce("errors: ra_ulysses_fwd with head_group = N")
    q_all = torch.randn((N, b, L, h, d), device="cuda", dtype=torch.bfloat16)
    o_all, lse_all = _filled((N, b, L, h, d), torch.bfloat16), _filled((N, b, h, L))
    uws = torch.empty(lib.ra_ulysses_fwd_workspace(ctypes.byref(p)), device="cuda", dtype=torch.uint8)
    assert lib.ra_ulysses_fwd(ctypes.byref(p), N, _p(q_all), _p(k_all), _p(v_all), _p(o_all), _p(lse_all),
                              _p(uws), uws.numel(), s) == _lib.RA_ERR_INVALID_ARG
    assert _unchanged(o_all, lse_all)

    announce("errors: ra_ring_bwd_kv_stationary with a workspace one byte short")
    need = lib.ra_ring_bwd_kv_stationary_workspace(ctypes.byref(p))
    sws = torch.empty(need, device="cuda", dtype=torch.uint8)
    dq_all = _filled((N, b, L, h, d))
    lse_all2, dl_all = _filled((N, b, h, L)), _filled((N, b, h, L))
    assert lib.ra_ring_bwd_kv_stationary(ctypes.byref(p), 0, _p(k_all[0]), _p(v_all[0]), _p(q_all), _p(q_all),
                                         _p(lse_all2), _p(dl_all), _p(dq_all), _p(dk), _p(dv), _p(sws), need - 1,
                                         s, None) == _lib.RA_ERR_WORKSPACE
    assert _unchanged(dq_all, dk, dv)


def test_binding_refuses_host_and_strided_buffers():
    """The binding hands the library only contiguous GPU tensors of one device: a workspace in
    host memory or a strided output is refused before any call (the kernels would fault on
    such addresses), and a workspace of another element type is sized in bytes."""
    b, L, h, n_kv, d, N = 1, 128, 8, 4, 128, 4
    q = torch.randn((b, L, h, d), device="cuda", dtype=torch.bfloat16)
    k_all = torch.randn((N, b, L, n_kv, d), device="cuda", dtype=torch.bfloat16)
    v_all = torch.randn_like(k_all)
    kw = dict(q_shard=1, causal=True, layout="striped")
    need = ra.ring_workspace_bytes(q, k_all, causal=True, layout="striped")
    announce("binding: host workspace, strided output, fp32 workspace")
    o_host_ws = _filled((b, L, h, d), torch.bfloat16)
    with pytest.raises(ValueError):
        ra.ring_fwd(q, k_all, v_all, **kw, workspace=torch.empty(need, dtype=torch.uint8), out=o_host_ws)
    assert _unchanged(o_host_ws)
    o_strided = _filled((b, h, L, d), torch.bfloat16).transpose(1, 2)
    with pytest.raises(ValueError):
        ra.ring_fwd(q, k_all, v_all, **kw, out=o_strided)
    assert _unchanged(o_strided)
    o_ref, l_ref = ra.ring_fwd(q, k_all, v_all, **kw)
    ws32 = torch.empty((need + 3) // 4, device="cuda", dtype=torch.float32)
    o32, l32 = ra.ring_fwd(q, k_all, v_all, **kw, workspace=ws32)
    torch.cuda.synchronize()
    assert torch.equal(o_ref, o32) and torch.equal(l_ref, l32)

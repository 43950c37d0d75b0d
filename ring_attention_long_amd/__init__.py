"""ring_attention_long_amd — one device's share of Ring Attention on MI355X (gfx950).

A thin torch-facing binding over libra.so (include/ra.h).  Every step of the computation
runs in the library's HIP kernels; this module only checks tensor shapes, allocates the
outputs with torch and passes device pointers and HIP streams through ctypes.

Entry points (same names as the C-ABI, without the ``ra_`` prefix):
    step_fwd      one ring step: queries of one shard against one KV shard -> (O, LSE) partial
    merge_lse     in-place merge of a partial into a running (O, LSE)
    finalize      fp32 accumulator -> output dtype
    ring_fwd      the whole forward ring pass of one device (double-buffered KV staging on a
                  side stream)
    ring_fwd_timed  ring_fwd plus per-step kernel and copy timings
    bwd_preprocess  delta = rowsum(dO * O)
    step_bwd      one backward ring step (accumulates dQ, dK, dV)
    ring_bwd      the whole backward ring pass of one device
    ring_bwd_kv_stationary  the other gradient schedule: keys and values stay, the query
                  shards (Q, dO, LSE, D) pass by and dQ contributions travel with them
    allowed_pairs   host-side count of allowed (query, key) pairs (useful-FLOP accounting)
    ulysses_fwd   one device's share of all-to-all sequence parallelism: whole-sequence
                  attention for a group of h/N heads, exchanged in and out by copy kernels
    ulysses_fwd_timed  ulysses_fwd plus the time of its gather, attention and scatter
    ulysses_bwd   the backward of that share (gradients of the group's heads, sent back)

Tensor layouts (page 1, "Practical Implementation Patterns": batch, sequence, heads, dim):
    q, o [b, L, h, d];  k, v [b, L, n_kv, d];  k_all, v_all [N, b, L, n_kv, d];
    lse [b, h, L] fp32 (natural log, scaled-logit units).
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import RA_BF16, RA_F32, RA_LAYOUT, RaError, RaProblem, RaRingTiming, RaUlyssesTiming, check

__all__ = ["step_fwd", "merge_lse", "finalize", "ring_fwd", "ring_fwd_timed", "ring_fwd_noalloc", "allowed_pairs",
           "bwd_preprocess", "step_bwd", "ring_bwd", "ring_bwd_workspace_bytes",
           "ring_bwd_kv_stationary", "ulysses_fwd", "ulysses_fwd_timed", "ulysses_workspace_bytes",
           "ulysses_bwd", "usp_fwd", "usp_workspace_bytes", "make_problem", "RaError", "library_path"]

_DTYPES = {torch.float32: RA_F32, torch.bfloat16: RA_BF16}
_copy_streams: dict[int, torch.cuda.Stream] = {}


def library_path() -> str:
    return _lib.LIB_PATH


def make_problem(*, b, L, h, n_kv, d, N, causal=False, layout="contiguous",
                 dtype=torch.bfloat16, scale=None, docs=None, steps_per_launch=0) -> RaProblem:
    """The C-ABI problem descriptor.  docs: None, or (doc_begin, doc_end), int32 GPU tensors
    [b, L] holding each query row's packed-document bounds (see document_ranges).
    steps_per_launch: ring steps per launch of a bf16 forward pass (0: the library's choice,
    1: one launch per step; see ra_problem in include/ra.h)."""
    if layout not in RA_LAYOUT:
        raise ValueError(f"layout must be one of {sorted(RA_LAYOUT)}")
    if dtype not in _DTYPES:
        raise ValueError(f"dtype must be float32 or bfloat16, got {dtype}")
    db = de = None
    if docs is not None:
        begin, end = docs
        _need(begin, "doc_begin", (b, L), torch.int32)
        _need(end, "doc_end", (b, L), torch.int32)
        db, de = begin.data_ptr(), end.data_ptr()
    return RaProblem(b, L, h, n_kv, d, N, int(bool(causal)), RA_LAYOUT[layout], _DTYPES[dtype],
                     0.0 if scale is None else float(scale), db, de, int(steps_per_launch))


def document_ranges(bounds, *, N, L, shard, layout="contiguous"):
    """Host-side: per-row packed-document bounds of shard `shard` (numpy int32 arrays [L],
    begin and end), from the documents' global start positions bounds = [0, ..., N * L]."""
    import numpy as np
    bounds = np.ascontiguousarray(bounds, dtype=np.int32)
    begin = np.empty(L, dtype=np.int32)
    end = np.empty(L, dtype=np.int32)
    p = make_problem(b=1, L=L, h=1, n_kv=1, d=128, N=N, layout=layout)
    check(_lib.lib().ra_document_ranges(ctypes.byref(p), shard, bounds.ctypes.data,
                                        bounds.size - 1, begin.ctypes.data, end.ctypes.data),
          "ra_document_ranges")
    return begin, end


def allowed_pairs_packed(doc_begin, doc_end, *, N, q_shard, kv_shard=-1, causal=True,
                         layout="contiguous") -> int:
    """Host-only pair count with packed documents; doc_begin, doc_end numpy int32 [b, L]."""
    import numpy as np
    db = np.ascontiguousarray(doc_begin, dtype=np.int32)
    de = np.ascontiguousarray(doc_end, dtype=np.int32)
    b, L = db.shape
    p = make_problem(b=b, L=L, h=1, n_kv=1, d=128, N=N, causal=causal, layout=layout)
    n = int(_lib.lib().ra_allowed_pairs_packed(ctypes.byref(p), q_shard, kv_shard, db.ctypes.data,
                                               de.ctypes.data))
    if n < 0:
        raise ValueError("invalid arguments to allowed_pairs_packed")
    return n


def _ptr(t: torch.Tensor) -> ctypes.c_void_p:
    """Address of a tensor handed to the library, which reads and writes it from its kernels:
    only a contiguous GPU tensor qualifies (a host or strided one would fault the GPU)."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError("the library takes GPU tensors only")
    if not t.is_contiguous():
        raise ValueError("the library takes contiguous tensors only")
    return ctypes.c_void_p(t.data_ptr())


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _one_device(*ts) -> torch.device:
    """The one GPU all given tensors (None skipped) live on."""
    devs = {t.device for t in ts if t is not None}
    if len(devs) != 1:
        raise ValueError(f"tensors on several devices: {sorted(str(x) for x in devs)}")
    dev = devs.pop()
    if dev.type != "cuda":
        raise ValueError(f"tensors must be on a GPU, not {dev}")
    return dev


def _stream(s, device=None) -> ctypes.c_void_p:
    if s is None:
        s = torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _copy_stream_arg(copy_stream, device):
    cs = copy_stream_for(device) if copy_stream == "auto" else copy_stream
    return ctypes.c_void_p(cs.cuda_stream) if cs is not None else None


def _run(device, name, *args) -> None:
    """Call library entry point `name` with `device` current (the pass's events and the
    default stream belong to it) and raise RaError on a status other than RA_OK."""
    with torch.cuda.device(device):
        check(getattr(_lib.lib(), name)(*args), name)


def _need(t: torch.Tensor, name: str, shape, dtype) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _shapes_from_q(q, kv):
    b, L, h, d = q.shape
    n_kv = kv.shape[-2]
    return b, L, h, n_kv, d


def step_fwd(q, k, v, *, N, q_shard, kv_shard, causal=False, layout="contiguous", scale=None,
             stream=None, docs=None):
    """One ring step: shard q_shard's queries q [b, L, h, d] against the keys/values of shard
    kv_shard (k, v [b, L, n_kv, d]).  Returns the normalised partial (o_part [b, L, h, d]
    fp32, lse_part [b, h, L] fp32); rows with no allowed key get (0, -inf)."""
    b, L, h, n_kv, d = _shapes_from_q(q, k)
    _need(q, "q", (b, L, h, d), q.dtype)
    _need(k, "k", (b, L, n_kv, d), q.dtype)
    _need(v, "v", (b, L, n_kv, d), q.dtype)
    p = make_problem(b=b, L=L, h=h, n_kv=n_kv, d=d, N=N, causal=causal, layout=layout,
                     dtype=q.dtype, scale=scale, docs=docs)
    o = torch.empty((b, L, h, d), device=q.device, dtype=torch.float32)
    lse = torch.empty((b, h, L), device=q.device, dtype=torch.float32)
    dev = _one_device(q, k, v, *(docs or ()))
    _run(dev, "ra_step_fwd", ctypes.byref(p), q_shard, kv_shard, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
         _stream(stream, dev))
    return o, lse


def merge_lse(o_acc, lse_acc, o_part, lse_part, *, stream=None):
    """In place: (o_acc, lse_acc) <- merge of (o_acc, lse_acc) and (o_part, lse_part).
    All fp32; o [b, L, h, d], lse [b, h, L]."""
    b, L, h, d = o_acc.shape
    for t, n, shp in ((o_acc, "o_acc", (b, L, h, d)), (o_part, "o_part", (b, L, h, d)),
                      (lse_acc, "lse_acc", (b, h, L)), (lse_part, "lse_part", (b, h, L))):
        _need(t, n, shp, torch.float32)
    p = make_problem(b=b, L=L, h=h, n_kv=h, d=d, N=1, dtype=torch.float32)
    dev = _one_device(o_acc, lse_acc, o_part, lse_part)
    _run(dev, "ra_merge_lse", ctypes.byref(p), _ptr(o_acc), _ptr(lse_acc), _ptr(o_part), _ptr(lse_part),
         _stream(stream, dev))
    return o_acc, lse_acc


def finalize(o_acc, dtype=torch.bfloat16, *, stream=None):
    """fp32 accumulator [b, L, h, d] -> new tensor of `dtype` (bf16: round to nearest even)."""
    b, L, h, d = o_acc.shape
    _need(o_acc, "o_acc", (b, L, h, d), torch.float32)
    p = make_problem(b=b, L=L, h=h, n_kv=h, d=d, N=1, dtype=dtype)
    o = torch.empty((b, L, h, d), device=o_acc.device, dtype=dtype)
    dev = _one_device(o_acc)
    _run(dev, "ra_finalize", ctypes.byref(p), _ptr(o_acc), _ptr(o), _stream(stream, dev))
    return o


def copy_stream_for(device) -> torch.cuda.Stream:
    """The side stream (default priority) used for KV staging on `device`."""
    idx = torch.device(device).index
    if idx is None:
        idx = torch.cuda.current_device()
    if idx not in _copy_streams:
        _copy_streams[idx] = torch.cuda.Stream(device=idx)
    return _copy_streams[idx]


def ring_workspace_bytes(q, k_all, *, causal=False, layout="contiguous", scale=None, steps_per_launch=0) -> int:
    N, b, L, n_kv, d = k_all.shape
    p = make_problem(b=b, L=L, h=q.shape[2], n_kv=n_kv, d=d, N=N, causal=causal, layout=layout,
                     dtype=q.dtype, scale=scale, steps_per_launch=steps_per_launch)
    return int(_lib.lib().ra_ring_fwd_workspace(ctypes.byref(p)))


def fwd_step_plan(*, b, L, h, n_kv, d=128, N, q_shard, kv_shard, causal=False, layout="contiguous", n_cu=256):
    """Work items of one bf16 forward ring step with the second accumulator (ra_fwd_step_plan):
    returns ([(block, part), ...] in launch order, rows per block); part -1 = whole block."""
    p = make_problem(b=b, L=L, h=h, n_kv=n_kv, d=d, N=N, causal=causal, layout=layout, dtype=torch.bfloat16)
    cap = 256
    block = (ctypes.c_int32 * cap)()
    part = (ctypes.c_int32 * cap)()
    n = ctypes.c_int32(0)
    rows = ctypes.c_int32(0)
    check(_lib.lib().ra_fwd_step_plan(ctypes.byref(p), q_shard, kv_shard, n_cu, block, part, cap, ctypes.byref(n),
                                      ctypes.byref(rows)), "ra_fwd_step_plan")
    return [(block[i], part[i]) for i in range(min(n.value, cap))], rows.value


def _ring_args(q, k_all, v_all, causal, layout, scale, workspace, out, lse_out, docs=None, steps_per_launch=0):
    N, b, L, n_kv, d = k_all.shape
    h = q.shape[2]
    _need(q, "q", (b, L, h, d), q.dtype)
    _need(k_all, "k_all", (N, b, L, n_kv, d), q.dtype)
    _need(v_all, "v_all", (N, b, L, n_kv, d), q.dtype)
    p = make_problem(b=b, L=L, h=h, n_kv=n_kv, d=d, N=N, causal=causal, layout=layout,
                     dtype=q.dtype, scale=scale, docs=docs, steps_per_launch=steps_per_launch)
    need = int(_lib.lib().ra_ring_fwd_workspace(ctypes.byref(p)))
    if need == 0:
        raise RaError(int(_lib.RA_ERR_INVALID_ARG), "ra_ring_fwd_workspace")
    if workspace is None:
        workspace = torch.empty(need, device=q.device, dtype=torch.uint8)
    o = out if out is not None else torch.empty((b, L, h, d), device=q.device, dtype=q.dtype)
    lse = lse_out if lse_out is not None else torch.empty((b, h, L), device=q.device,
                                                          dtype=torch.float32)
    _need(o, "o", (b, L, h, d), q.dtype)
    _need(lse, "lse", (b, h, L), torch.float32)
    dev = _one_device(q, k_all, v_all, o, lse, workspace, *(docs or ()))
    return p, workspace, o, lse, dev


def ring_fwd(q, k_all, v_all, *, q_shard, causal=False, layout="contiguous", scale=None,
             stream=None, copy_stream="auto", workspace=None, out=None, lse_out=None, docs=None,
             steps_per_launch=0):
    """Forward ring pass of device q_shard: q [b, L, h, d] against all N KV shards
    k_all, v_all [N, b, L, n_kv, d] in ring order.  Returns (o [b, L, h, d] in q's dtype,
    lse [b, h, L] fp32).  copy_stream="auto" stages KV on a side stream; None stages on
    the compute stream."""
    p, ws, o, lse, dev = _ring_args(q, k_all, v_all, causal, layout, scale, workspace, out, lse_out,
                                     docs, steps_per_launch)
    _run(dev, "ra_ring_fwd", ctypes.byref(p), q_shard, _ptr(q), _ptr(k_all), _ptr(v_all), _ptr(o), _ptr(lse),
         _ptr(ws), _nbytes(ws), _stream(stream, dev), _copy_stream_arg(copy_stream, dev))
    return o, lse


def ring_fwd_timed(q, k_all, v_all, *, q_shard, causal=False, layout="contiguous", scale=None,
                   stream=None, copy_stream="auto", workspace=None, out=None, lse_out=None, steps_per_launch=0,
                   docs=None):
    """ring_fwd plus timings (ms from entry): returns (o, lse, dict).  Synchronises."""
    p, ws, o, lse, dev = _ring_args(q, k_all, v_all, causal, layout, scale, workspace, out, lse_out,
                                     docs, steps_per_launch)
    tm = RaRingTiming()
    _run(dev, "ra_ring_fwd_timed", ctypes.byref(p), q_shard, _ptr(q), _ptr(k_all), _ptr(v_all), _ptr(o),
         _ptr(lse), _ptr(ws), _nbytes(ws), _stream(stream, dev), _copy_stream_arg(copy_stream, dev),
         ctypes.byref(tm))
    n = tm.n_steps
    timing = {
        "step_begin_ms": list(tm.step_begin_ms[:n]), "step_end_ms": list(tm.step_end_ms[:n]),
        "copy_begin_ms": list(tm.copy_begin_ms[:n]), "copy_end_ms": list(tm.copy_end_ms[:n]),
        "total_ms": tm.total_ms, "launch_steps": list(tm.launch_steps[:n]),
    }
    return o, lse, timing


def ring_fwd_noalloc(q, k_all, v_all, *, q_shard, causal=False, layout="contiguous", scale=None,
                     stream=None, copy_stream="auto", out=None, lse_out=None, docs=None, steps_per_launch=0):
    """ring_fwd through ra_ring_fwd_noalloc: no workspace (the library's fixed scratch array of
    the current device holds it).  Outputs are allocated here unless given."""
    N, b, L, n_kv, d = k_all.shape
    h = q.shape[2]
    _need(q, "q", (b, L, h, d), q.dtype)
    _need(k_all, "k_all", (N, b, L, n_kv, d), q.dtype)
    _need(v_all, "v_all", (N, b, L, n_kv, d), q.dtype)
    p = make_problem(b=b, L=L, h=h, n_kv=n_kv, d=d, N=N, causal=causal, layout=layout,
                     dtype=q.dtype, scale=scale, docs=docs, steps_per_launch=steps_per_launch)
    o = out if out is not None else torch.empty((b, L, h, d), device=q.device, dtype=q.dtype)
    lse = lse_out if lse_out is not None else torch.empty((b, h, L), device=q.device, dtype=torch.float32)
    _need(o, "o", (b, L, h, d), q.dtype)
    _need(lse, "lse", (b, h, L), torch.float32)
    dev = _one_device(q, k_all, v_all, o, lse, *(docs or ()))
    _run(dev, "ra_ring_fwd_noalloc", ctypes.byref(p), q_shard, _ptr(q), _ptr(k_all), _ptr(v_all), _ptr(o),
         _ptr(lse), _stream(stream, dev), _copy_stream_arg(copy_stream, dev))
    return o, lse


def ulysses_workspace_bytes(q_all, k_all, *, causal=False, layout="contiguous", scale=None) -> int:
    """Workspace of ulysses_fwd for q_all [N, b, L, h, d], k_all [N, b, L, n_kv, d] (0 if the
    problem is not valid for the all-to-all path)."""
    N, b, L, h, d = q_all.shape
    p = make_problem(b=b, L=L, h=h, n_kv=k_all.shape[3], d=d, N=N, causal=causal, layout=layout,
                     dtype=q_all.dtype, scale=scale)
    return int(_lib.lib().ra_ulysses_fwd_workspace(ctypes.byref(p)))


def _ulysses_args(q_all, k_all, v_all, causal, layout, scale, workspace, out, lse_out):
    N, b, L, h, d = q_all.shape
    n_kv = k_all.shape[3]
    _need(q_all, "q_all", (N, b, L, h, d), q_all.dtype)
    _need(k_all, "k_all", (N, b, L, n_kv, d), q_all.dtype)
    _need(v_all, "v_all", (N, b, L, n_kv, d), q_all.dtype)
    p = make_problem(b=b, L=L, h=h, n_kv=n_kv, d=d, N=N, causal=causal, layout=layout,
                     dtype=q_all.dtype, scale=scale)
    need = int(_lib.lib().ra_ulysses_fwd_workspace(ctypes.byref(p)))
    if need == 0:
        raise RaError(int(_lib.RA_ERR_INVALID_ARG), "ra_ulysses_fwd_workspace")
    if workspace is None:
        workspace = torch.empty(need, device=q_all.device, dtype=torch.uint8)
    o = out if out is not None else torch.zeros((N, b, L, h, d), device=q_all.device, dtype=q_all.dtype)
    lse = lse_out if lse_out is not None else torch.full((N, b, h, L), float("-inf"),
                                                         device=q_all.device, dtype=torch.float32)
    _need(o, "o_all", (N, b, L, h, d), q_all.dtype)
    _need(lse, "lse_all", (N, b, h, L), torch.float32)
    dev = _one_device(q_all, k_all, v_all, o, lse, workspace)
    return p, workspace, o, lse, dev


def ulysses_fwd(q_all, k_all, v_all, *, head_group, causal=False, layout="contiguous", scale=None,
                stream=None, workspace=None, out=None, lse_out=None):
    """Device head_group's share of all-to-all sequence parallelism: q_all [N, b, L, h, d],
    k_all, v_all [N, b, L, n_kv, d] (every shard, each in its own layout order).  Writes query
    heads [head_group h/N, (head_group+1) h/N) of every shard into out [N, b, L, h, d]
    (q's dtype) and lse_out [N, b, h, L] fp32 (allocated if None: zeros and -inf elsewhere)
    and returns them; call it for every head group to fill them."""
    p, ws, o, lse, dev = _ulysses_args(q_all, k_all, v_all, causal, layout, scale, workspace, out, lse_out)
    _run(dev, "ra_ulysses_fwd", ctypes.byref(p), head_group, _ptr(q_all), _ptr(k_all), _ptr(v_all), _ptr(o),
         _ptr(lse), _ptr(ws), _nbytes(ws), _stream(stream, dev))
    return o, lse


def ulysses_fwd_timed(q_all, k_all, v_all, *, head_group, causal=False, layout="contiguous",
                      scale=None, stream=None, workspace=None, out=None, lse_out=None):
    """ulysses_fwd plus the time of its parts: returns (o, lse, dict with gather_ms,
    attend_ms, scatter_ms, total_ms).  Synchronises."""
    p, ws, o, lse, dev = _ulysses_args(q_all, k_all, v_all, causal, layout, scale, workspace, out, lse_out)
    tm = RaUlyssesTiming()
    _run(dev, "ra_ulysses_fwd_timed", ctypes.byref(p), head_group, _ptr(q_all), _ptr(k_all), _ptr(v_all),
         _ptr(o), _ptr(lse), _ptr(ws), _nbytes(ws), _stream(stream, dev), ctypes.byref(tm))
    return o, lse, {"gather_ms": tm.gather_ms, "attend_ms": tm.attend_ms,
                    "scatter_ms": tm.scatter_ms, "total_ms": tm.total_ms}


def ulysses_bwd(q_all, k_all, v_all, o_all, dout_all, lse_all, *, head_group, causal=False,
                layout="contiguous", scale=None, stream=None, workspace=None, out=None):
    """Backward of device head_group's share of the all-to-all scheme.  q_all, o_all, dout_all
    [N, b, L, h, d] (bf16), k_all, v_all [N, b, L, n_kv, d], lse_all [N, b, h, L] fp32.  Writes
    the group's heads of (dq_all [N, b, L, h, d], dk_all, dv_all [N, b, L, n_kv, d]) fp32
    (allocated as zeros if out is None) and returns them; call it for every head group to
    fill them."""
    N, b, L, h, d = q_all.shape
    n_kv = k_all.shape[3]
    for t, n, shp in ((q_all, "q_all", (N, b, L, h, d)), (o_all, "o_all", (N, b, L, h, d)),
                      (dout_all, "dout_all", (N, b, L, h, d)), (k_all, "k_all", (N, b, L, n_kv, d)),
                      (v_all, "v_all", (N, b, L, n_kv, d))):
        _need(t, n, shp, q_all.dtype)
    _need(lse_all, "lse_all", (N, b, h, L), torch.float32)
    p = make_problem(b=b, L=L, h=h, n_kv=n_kv, d=d, N=N, causal=causal, layout=layout,
                     dtype=q_all.dtype, scale=scale)
    need = int(_lib.lib().ra_ulysses_bwd_workspace(ctypes.byref(p)))
    if need == 0:
        raise RaError(int(_lib.RA_ERR_UNSUPPORTED), "ra_ulysses_bwd_workspace")
    if workspace is None:
        workspace = torch.empty(need, device=q_all.device, dtype=torch.uint8)
    if out is None:
        out = (torch.zeros((N, b, L, h, d), device=q_all.device, dtype=torch.float32),
               torch.zeros((N, b, L, n_kv, d), device=q_all.device, dtype=torch.float32),
               torch.zeros((N, b, L, n_kv, d), device=q_all.device, dtype=torch.float32))
    dq, dk, dv = out
    _need(dq, "dq_all", (N, b, L, h, d), torch.float32)
    _need(dk, "dk_all", (N, b, L, n_kv, d), torch.float32)
    _need(dv, "dv_all", (N, b, L, n_kv, d), torch.float32)
    dev = _one_device(q_all, k_all, v_all, o_all, dout_all, lse_all, dq, dk, dv, workspace)
    _run(dev, "ra_ulysses_bwd", ctypes.byref(p), head_group, _ptr(q_all), _ptr(k_all), _ptr(v_all), _ptr(o_all),
         _ptr(dout_all), _ptr(lse_all), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), _nbytes(workspace),
         _stream(stream, dev))
    return dq, dk, dv


def usp_workspace_bytes(q_all, k_all, *, n_head_groups, causal=False, layout="contiguous", scale=None) -> int:
    N, b, L, h, d = q_all.shape
    p = make_problem(b=b, L=L, h=h, n_kv=k_all.shape[3], d=d, N=N, causal=causal, layout=layout,
                     dtype=q_all.dtype, scale=scale)
    return int(_lib.lib().ra_usp_fwd_workspace(ctypes.byref(p), n_head_groups))


def usp_fwd(q_all, k_all, v_all, *, n_head_groups, head_group, ring_rank, causal=False, layout="contiguous",
            scale=None, stream=None, copy_stream="auto", workspace=None, out=None, lse_out=None, timed=False):
    """Device (head_group, ring_rank)'s share of the two-dimensional arrangement (n_head_groups
    head groups x N / n_head_groups ring shards): q_all [N, b, L, h, d], k_all, v_all
    [N, b, L, n_kv, d], device r * n_head_groups + g holding piece g of ring shard r.  Writes
    the head group's heads of the ring shard's devices into out [N, b, L, h, d] and lse_out
    [N, b, h, L] (allocated if None: zeros and -inf elsewhere) and returns them (and, with
    timed=True, the parts' times in ms; that call synchronises)."""
    N, b, L, h, d = q_all.shape
    n_kv = k_all.shape[3]
    _need(q_all, "q_all", (N, b, L, h, d), q_all.dtype)
    _need(k_all, "k_all", (N, b, L, n_kv, d), q_all.dtype)
    _need(v_all, "v_all", (N, b, L, n_kv, d), q_all.dtype)
    p = make_problem(b=b, L=L, h=h, n_kv=n_kv, d=d, N=N, causal=causal, layout=layout, dtype=q_all.dtype,
                     scale=scale)
    need = int(_lib.lib().ra_usp_fwd_workspace(ctypes.byref(p), n_head_groups))
    if need == 0:
        raise RaError(int(_lib.RA_ERR_INVALID_ARG), "ra_usp_fwd_workspace")
    if workspace is None:
        workspace = torch.empty(need, device=q_all.device, dtype=torch.uint8)
    o = out if out is not None else torch.zeros((N, b, L, h, d), device=q_all.device, dtype=q_all.dtype)
    lse = lse_out if lse_out is not None else torch.full((N, b, h, L), float("-inf"), device=q_all.device,
                                                         dtype=torch.float32)
    _need(o, "o_all", (N, b, L, h, d), q_all.dtype)
    _need(lse, "lse_all", (N, b, h, L), torch.float32)
    dev = _one_device(q_all, k_all, v_all, o, lse, workspace)
    args = (ctypes.byref(p), n_head_groups, head_group, ring_rank, _ptr(q_all), _ptr(k_all), _ptr(v_all), _ptr(o),
            _ptr(lse), _ptr(workspace), _nbytes(workspace), _stream(stream, dev),
            _copy_stream_arg(copy_stream, dev))
    if not timed:
        _run(dev, "ra_usp_fwd", *args)
        return o, lse
    tm = _lib.RaUspTiming()
    _run(dev, "ra_usp_fwd_timed", *args, ctypes.byref(tm))
    return o, lse, {k: getattr(tm, k) for k, _ in _lib.RaUspTiming._fields_}


def bwd_preprocess(o, dout, *, stream=None):
    """delta [b, h, L] fp32 = rowsum(dout * o) for o, dout [b, L, h, d] bf16."""
    b, L, h, d = o.shape
    _need(o, "o", (b, L, h, d), o.dtype)
    _need(dout, "dout", (b, L, h, d), o.dtype)
    p = make_problem(b=b, L=L, h=h, n_kv=h, d=d, N=1, dtype=o.dtype)
    delta = torch.empty((b, h, L), device=o.device, dtype=torch.float32)
    dev = _one_device(o, dout)
    _run(dev, "ra_bwd_preprocess", ctypes.byref(p), _ptr(o), _ptr(dout), _ptr(delta), _stream(stream, dev))
    return delta


def step_bwd(q, k, v, dout, lse, delta, *, N, q_shard, kv_shard, causal=False,
             layout="contiguous", scale=None, dq_acc=None, dk_acc=None, dv_acc=None,
             stream=None, docs=None):
    """One backward ring step: adds this (query shard, KV shard) pair's contributions to
    dq_acc [b, L, h, d] and dk_acc, dv_acc [b, L, n_kv, d] (fp32; zeros when not given).
    Returns (dq_acc, dk_acc, dv_acc)."""
    b, L, h, n_kv, d = _shapes_from_q(q, k)
    for t, n, shp in ((q, "q", (b, L, h, d)), (k, "k", (b, L, n_kv, d)), (v, "v", (b, L, n_kv, d)),
                      (dout, "dout", (b, L, h, d))):
        _need(t, n, shp, q.dtype)
    _need(lse, "lse", (b, h, L), torch.float32)
    _need(delta, "delta", (b, h, L), torch.float32)
    z = lambda shp: torch.zeros(shp, device=q.device, dtype=torch.float32)  # noqa: E731
    dq_acc = z((b, L, h, d)) if dq_acc is None else dq_acc
    dk_acc = z((b, L, n_kv, d)) if dk_acc is None else dk_acc
    dv_acc = z((b, L, n_kv, d)) if dv_acc is None else dv_acc
    _need(dq_acc, "dq_acc", (b, L, h, d), torch.float32)
    _need(dk_acc, "dk_acc", (b, L, n_kv, d), torch.float32)
    _need(dv_acc, "dv_acc", (b, L, n_kv, d), torch.float32)
    p = make_problem(b=b, L=L, h=h, n_kv=n_kv, d=d, N=N, causal=causal, layout=layout,
                     dtype=q.dtype, scale=scale, docs=docs)
    dev = _one_device(q, k, v, dout, lse, delta, dq_acc, dk_acc, dv_acc, *(docs or ()))
    _run(dev, "ra_step_bwd", ctypes.byref(p), q_shard, kv_shard, _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse),
         _ptr(delta), _ptr(dq_acc), _ptr(dk_acc), _ptr(dv_acc), _stream(stream, dev))
    return dq_acc, dk_acc, dv_acc


def ring_bwd_workspace_bytes(q, k_all, *, causal=False, layout="contiguous", scale=None,
                             minimum=False) -> int:
    """Workspace of ring_bwd for q [b, L, h, d], k_all [N, b, L, n_kv, d] (0 if invalid): the
    size the library asks for, or with minimum=True the smallest it accepts (every key block of
    the dK/dV kernel then runs whole)."""
    N, b, L, n_kv, d = k_all.shape
    p = make_problem(b=b, L=L, h=q.shape[2], n_kv=n_kv, d=d, N=N, causal=causal, layout=layout,
                     dtype=q.dtype, scale=scale)
    fn = _lib.lib().ra_ring_bwd_workspace_min if minimum else _lib.lib().ra_ring_bwd_workspace
    return int(fn(ctypes.byref(p)))


def ring_bwd(q, k_all, v_all, o, dout, lse, *, q_shard, causal=False, layout="contiguous",
             scale=None, stream=None, copy_stream="auto", workspace=None, out=None, docs=None,
             timed=False):
    """Backward ring pass of device q_shard.  q, o, dout [b, L, h, d] (bf16), lse [b, h, L]
    from the forward, k_all, v_all [N, b, L, n_kv, d].  Returns fp32 (dq [b, L, h, d],
    dk_all [N, b, L, n_kv, d], dv_all [N, b, L, n_kv, d]), written into `out` when given;
    timed=True adds per-step timings (as ring_fwd_timed) and synchronises."""
    N, b, L, n_kv, d = k_all.shape
    h = q.shape[2]
    _need(q, "q", (b, L, h, d), q.dtype)
    _need(k_all, "k_all", (N, b, L, n_kv, d), q.dtype)
    _need(v_all, "v_all", (N, b, L, n_kv, d), q.dtype)
    _need(o, "o", (b, L, h, d), q.dtype)
    _need(dout, "dout", (b, L, h, d), q.dtype)
    _need(lse, "lse", (b, h, L), torch.float32)
    p = make_problem(b=b, L=L, h=h, n_kv=n_kv, d=d, N=N, causal=causal, layout=layout,
                     dtype=q.dtype, scale=scale, docs=docs)
    need = int(_lib.lib().ra_ring_bwd_workspace_min(ctypes.byref(p)))
    if need == 0:
        raise RaError(int(_lib.RA_ERR_UNSUPPORTED), "ra_ring_bwd_workspace")
    if workspace is None:
        workspace = torch.empty(int(_lib.lib().ra_ring_bwd_workspace(ctypes.byref(p))), device=q.device,
                                dtype=torch.uint8)
    if out is None:
        dq = torch.empty((b, L, h, d), device=q.device, dtype=torch.float32)
        dk = torch.empty((N, b, L, n_kv, d), device=q.device, dtype=torch.float32)
        dv = torch.empty((N, b, L, n_kv, d), device=q.device, dtype=torch.float32)
    else:
        dq, dk, dv = out
        _need(dq, "dq", (b, L, h, d), torch.float32)
        _need(dk, "dk_all", (N, b, L, n_kv, d), torch.float32)
        _need(dv, "dv_all", (N, b, L, n_kv, d), torch.float32)
    _need(workspace, "workspace", (workspace.numel(),), torch.uint8)
    if workspace.numel() < need:
        raise RaError(int(_lib.RA_ERR_WORKSPACE), "ra_ring_bwd")
    dev = _one_device(q, k_all, v_all, o, dout, lse, dq, dk, dv, workspace, *(docs or ()))
    args = (ctypes.byref(p), q_shard, _ptr(q), _ptr(k_all), _ptr(v_all), _ptr(o), _ptr(dout), _ptr(lse),
            _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), _nbytes(workspace), _stream(stream, dev),
            _copy_stream_arg(copy_stream, dev))
    if not timed:
        _run(dev, "ra_ring_bwd", *args)
        return dq, dk, dv
    tm = RaRingTiming()
    _run(dev, "ra_ring_bwd_timed", *args, ctypes.byref(tm))
    n = tm.n_steps
    return dq, dk, dv, {"step_begin_ms": list(tm.step_begin_ms[:n]), "step_end_ms": list(tm.step_end_ms[:n]),
                        "copy_begin_ms": list(tm.copy_begin_ms[:n]), "copy_end_ms": list(tm.copy_end_ms[:n]),
                        "total_ms": tm.total_ms, "launch_steps": list(tm.launch_steps[:n])}


def ring_bwd_kv_stationary(k, v, q_all, dout_all, lse_all, delta_all, *, kv_shard, causal=False,
                           layout="contiguous", scale=None, stream=None, copy_stream="auto",
                           workspace=None, out=None):
    """Backward ring pass with keys and values stationary, device kv_shard's share: k, v
    [b, L, n_kv, d] (bf16) stay, every query shard passes by with q_all, dout_all
    [N, b, L, h, d], lse_all and delta_all [N, b, h, L] (fp32, D from bwd_preprocess on each
    shard's home).  Returns fp32 (dq_all [N, b, L, h, d]: this device's contributions to
    every shard's dQ, dk, dv [b, L, n_kv, d]: its KV shard's gradients), into `out` if given."""
    N, b, L, h, d = q_all.shape
    n_kv = k.shape[2]
    _need(k, "k", (b, L, n_kv, d), q_all.dtype)
    _need(v, "v", (b, L, n_kv, d), q_all.dtype)
    _need(q_all, "q_all", (N, b, L, h, d), q_all.dtype)
    _need(dout_all, "dout_all", (N, b, L, h, d), q_all.dtype)
    _need(lse_all, "lse_all", (N, b, h, L), torch.float32)
    _need(delta_all, "delta_all", (N, b, h, L), torch.float32)
    p = make_problem(b=b, L=L, h=h, n_kv=n_kv, d=d, N=N, causal=causal, layout=layout,
                     dtype=q_all.dtype, scale=scale)
    need = int(_lib.lib().ra_ring_bwd_kv_stationary_workspace(ctypes.byref(p)))
    if need == 0:
        raise RaError(int(_lib.RA_ERR_UNSUPPORTED), "ra_ring_bwd_kv_stationary_workspace")
    if workspace is None:
        workspace = torch.empty(need, device=q_all.device, dtype=torch.uint8)
    if out is None:
        dq = torch.empty((N, b, L, h, d), device=q_all.device, dtype=torch.float32)
        dk = torch.empty((b, L, n_kv, d), device=q_all.device, dtype=torch.float32)
        dv = torch.empty((b, L, n_kv, d), device=q_all.device, dtype=torch.float32)
    else:
        dq, dk, dv = out
        _need(dq, "dq_all", (N, b, L, h, d), torch.float32)
        _need(dk, "dk", (b, L, n_kv, d), torch.float32)
        _need(dv, "dv", (b, L, n_kv, d), torch.float32)
    _need(workspace, "workspace", (workspace.numel(),), torch.uint8)
    if workspace.numel() < need:
        raise RaError(int(_lib.RA_ERR_WORKSPACE), "ra_ring_bwd_kv_stationary")
    dev = _one_device(k, v, q_all, dout_all, lse_all, delta_all, dq, dk, dv, workspace)
    _run(dev, "ra_ring_bwd_kv_stationary", ctypes.byref(p), kv_shard, _ptr(k), _ptr(v), _ptr(q_all),
         _ptr(dout_all), _ptr(lse_all), _ptr(delta_all), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
         _nbytes(workspace), _stream(stream, dev), _copy_stream_arg(copy_stream, dev))
    return dq, dk, dv


def allowed_pairs(*, b=1, L, N, q_shard, kv_shard=-1, causal=True, layout="contiguous") -> int:
    """Allowed (query, key) pairs of shard q_shard against kv_shard (-1: all shards), summed
    over the batch.  Host-only; forward useful FLOPs = 4 * d * h * pairs."""
    p = make_problem(b=b, L=L, h=1, n_kv=1, d=128, N=N, causal=causal, layout=layout,
                     dtype=torch.bfloat16)
    n = int(_lib.lib().ra_allowed_pairs(ctypes.byref(p), q_shard, kv_shard))
    if n < 0:
        raise ValueError("invalid arguments to allowed_pairs")
    return n

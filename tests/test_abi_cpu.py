"""CPU-only checks of the C-ABI library: it loads, exports every entry point include/ra.h
declares, rejects bad arguments before touching the GPU, and its host-side accounting
agrees with the oracle.  No kernel is launched here."""
import ctypes
import os
import re

import numpy as np
import pytest

from conftest import ROOT
from oracle import LAYOUTS, allowed_pairs as oracle_pairs

ra = pytest.importorskip("ring_attention_long_amd")
from ring_attention_long_amd import _lib  # noqa: E402
from ring_attention_long_amd import accounting  # noqa: E402

HEADER = os.path.join(ROOT, "include", "ra.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ra_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = _lib.lib()
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), f"{n} declared in ra.h but not exported"
    bound = {s[0] for s in _lib.SIGNATURES}
    assert set(names) == bound, "python binding and header disagree"


def _prob(**kw):
    base = dict(b=1, L=128, h=4, n_kv=2, d=128, N=4, causal=1, layout=0, dtype=1, scale=0.0, steps_per_launch=0)
    base.update(kw)
    p = _lib.RaProblem(*[base[k] for k in ("b", "L", "h", "n_kv", "d", "N", "causal",
                                           "layout", "dtype")], base["scale"])
    p.steps_per_launch = base["steps_per_launch"]
    return p


FAKE = ctypes.c_void_p(0x10000)       # aligned, never dereferenced: validation fails first


@pytest.mark.parametrize("kw,status", [
    (dict(h=3, n_kv=2), _lib.RA_ERR_INVALID_ARG),
    (dict(L=0), _lib.RA_ERR_INVALID_ARG),
    (dict(N=0), _lib.RA_ERR_INVALID_ARG),
    (dict(layout=7), _lib.RA_ERR_INVALID_ARG),
    (dict(dtype=5), _lib.RA_ERR_INVALID_ARG),
    (dict(causal=2), _lib.RA_ERR_INVALID_ARG),
    (dict(layout=2, L=127), _lib.RA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), _lib.RA_ERR_INVALID_ARG),
    (dict(d=96), _lib.RA_ERR_UNSUPPORTED),
    (dict(dtype=0, d=32), _lib.RA_ERR_UNSUPPORTED),
])
def test_step_fwd_rejects_bad_problems(kw, status):
    lib = _lib.lib()
    p = _prob(**kw)
    st = lib.ra_step_fwd(ctypes.byref(p), 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert st == status
    assert lib.ra_last_error()


def test_step_fwd_rejects_bad_shards_and_pointers():
    lib = _lib.lib()
    p = _prob()
    assert lib.ra_step_fwd(ctypes.byref(p), 4, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None) == _lib.RA_ERR_INVALID_ARG
    assert lib.ra_step_fwd(ctypes.byref(p), 0, -1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == _lib.RA_ERR_INVALID_ARG
    assert lib.ra_step_fwd(ctypes.byref(p), 0, 0, None, FAKE, FAKE, FAKE, FAKE, None) == _lib.RA_ERR_INVALID_ARG
    assert b"q is NULL" in lib.ra_last_error()
    mis = ctypes.c_void_p(0x10008)
    assert lib.ra_step_fwd(ctypes.byref(p), 0, 0, FAKE, mis, FAKE, FAKE, FAKE, None) == _lib.RA_ERR_INVALID_ARG
    assert b"aligned" in lib.ra_last_error()
    assert lib.ra_step_fwd(None, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None) == _lib.RA_ERR_INVALID_ARG


def test_bf16_kv_slice_limit():
    """K/V rows are staged through 32-bit buffer offsets below 2^31: a (batch, KV head) slice of
    2 GiB or more is refused before anything is enqueued, and the largest that fits is not."""
    lib = _lib.lib()
    big = _prob(L=1 << 20, n_kv=8, h=8, N=1)          # 2^20 * 8 * 128 * 2 = 2 GiB
    assert lib.ra_step_fwd(ctypes.byref(big), 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None) == _lib.RA_ERR_UNSUPPORTED
    assert b"2 GiB" in lib.ra_last_error()
    if _no_hip_device():                                # valid arguments reach the launch
        fits = _prob(L=(1 << 20) - 64, n_kv=8, h=8, N=1)
        assert lib.ra_step_fwd(ctypes.byref(fits), 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None) == _lib.RA_ERR_HIP


def test_ring_fwd_rejects_small_workspace():
    lib = _lib.lib()
    p = _prob(steps_per_launch=1)
    need = lib.ra_ring_fwd_workspace(ctypes.byref(p))
    # one launch per step, a short bf16 shard: the workspace ends with the optional second
    # accumulator (fp32 [b][L][h][d] and LSE [b][h][L]); less than the rest is refused
    second = 128 * 4 * 128 * 4 + 4 * 128 * 4
    st = lib.ra_ring_fwd(ctypes.byref(p), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - second - 1, None, None)
    assert st == _lib.RA_ERR_WORKSPACE
    tm = _lib.RaRingTiming()
    st = lib.ra_ring_fwd_timed(ctypes.byref(p), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - second - 1,
                               None, None, ctypes.byref(tm))
    assert st == _lib.RA_ERR_WORKSPACE
    assert lib.ra_ring_fwd_timed(ctypes.byref(p), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need,
                                 None, None, None) == _lib.RA_ERR_INVALID_ARG
    # batched steps asked for explicitly: the slots of every remote shard are required (the
    # workspace asked for ends with the same optional second accumulator)
    pb = _prob(steps_per_launch=2)
    bneed_f = lib.ra_ring_fwd_workspace(ctypes.byref(pb))
    assert bneed_f - second > need - second
    assert lib.ra_ring_fwd(ctypes.byref(pb), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, bneed_f - second - 1, None,
                           None) == _lib.RA_ERR_WORKSPACE
    assert b"steps per launch" in lib.ra_last_error()
    # the library's choice (0) takes one launch per step when the slots do not fit, so the
    # one-step minimum still holds
    p0 = _prob()
    assert lib.ra_ring_fwd_workspace(ctypes.byref(p0)) == bneed_f
    assert lib.ra_ring_fwd(ctypes.byref(p0), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - second - 1, None,
                           None) == _lib.RA_ERR_WORKSPACE
    bneed = lib.ra_ring_bwd_workspace_min(ctypes.byref(p))
    assert lib.ra_ring_bwd_timed(ctypes.byref(p), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 bneed, None, None, None) == _lib.RA_ERR_INVALID_ARG
    assert lib.ra_ring_bwd_timed(ctypes.byref(p), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                 bneed - 1, None, None, ctypes.byref(tm)) == _lib.RA_ERR_WORKSPACE
    assert lib.ra_ring_fwd(ctypes.byref(_prob(steps_per_launch=-2)), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                           bneed_f, None, None) == _lib.RA_ERR_INVALID_ARG


def test_binding_pointer_and_device_checks():
    """The binding's last gate before a library call: only GPU tensors become pointers, and
    the tensors of one call must share one GPU."""
    import torch

    import ring_attention_long_amd as ra
    with pytest.raises(ValueError):
        ra._ptr(torch.zeros(4))
    with pytest.raises(ValueError):
        ra._one_device(torch.zeros(1), None)
    assert ra._nbytes(torch.zeros(3, dtype=torch.float32)) == 12


def test_ring_fwd_rejects_ring_above_limit():
    """N above the driver's limit (128) is refused before anything else, on the one-launch-
    per-step and the batched path alike (both keep per-step events in fixed arrays)."""
    lib = _lib.lib()
    tm = _lib.RaRingTiming()
    for spl in (0, 1, 4):
        for dtype in (0, 1):
            p = _prob(N=129, dtype=dtype, steps_per_launch=spl)
            ws = lib.ra_ring_fwd_workspace(ctypes.byref(p))
            assert lib.ra_ring_fwd(ctypes.byref(p), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None,
                                   None) == _lib.RA_ERR_UNSUPPORTED, (spl, dtype)
            assert b"ring size" in lib.ra_last_error()
            assert lib.ra_ring_fwd_timed(ctypes.byref(p), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None, None,
                                         ctypes.byref(tm)) in (_lib.RA_ERR_UNSUPPORTED, _lib.RA_ERR_INVALID_ARG)
    p = _prob(N=128, steps_per_launch=4)
    assert lib.ra_ring_fwd(ctypes.byref(p), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None,
                           None) == _lib.RA_ERR_WORKSPACE


def _no_hip_device():
    """True when the HIP runtime sees no device at all (this container), so a call with
    valid arguments fails at its first HIP call and never touches memory."""
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        return False
    n = ctypes.c_int(-1)
    err = hip.hipGetDeviceCount(ctypes.byref(n))
    return err != 0 or n.value == 0


@pytest.mark.skipif(not _no_hip_device(), reason="needs a host without a GPU: the arguments are dummies")
def test_hip_failure_is_reported_as_ra_err_hip():
    """A HIP failure after validation comes back as RA_ERR_HIP with HIP's own text, from every
    entry point that launches work (here forced by the absence of a device)."""
    lib = _lib.lib()
    p = _prob()
    ws = lib.ra_ring_fwd_workspace(ctypes.byref(p))
    calls = {
        "ra_step_fwd": lambda: lib.ra_step_fwd(ctypes.byref(p), 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None),
        "ra_merge_lse": lambda: lib.ra_merge_lse(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, None),
        "ra_ring_fwd": lambda: lib.ra_ring_fwd(ctypes.byref(p), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws,
                                               None, None),
        "ra_step_bwd": lambda: lib.ra_step_bwd(ctypes.byref(p), 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                               FAKE, FAKE, FAKE, FAKE, None),
        "ra_ring_bwd": lambda: lib.ra_ring_bwd(ctypes.byref(p), 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                               FAKE, FAKE, FAKE, lib.ra_ring_bwd_workspace(ctypes.byref(p)),
                                               None, None),
    }
    for name, call in calls.items():
        assert call() == _lib.RA_ERR_HIP, name
        detail = lib.ra_last_error()
        assert detail and b"device" in detail.lower(), (name, detail)
    assert b"HIP" in lib.ra_status_string(_lib.RA_ERR_HIP).upper()


def test_workspace_size_is_two_kv_buffers_plus_fp32_accumulator():
    """Page 4, memory analysis: a device holds its own and one incoming KV block.  With one
    launch per ring step: the two staging buffers (K and V each) plus the fp32 output
    accumulator of bf16 problems, and for short bf16 shards (L <= 4096) the second
    accumulator with its LSE.  With bf16 steps batched into launches (the default for N >= 3):
    a slot for every remote shard's K and V, the fp32 accumulator and, for short shards, the
    same second accumulator."""
    lib = _lib.lib()
    pad = lambda x: (x + 255) // 256 * 256  # noqa: E731
    for dtype, esz in ((1, 2), (0, 4)):
        for L in (1000, 5000):
            for spl in (0, 1, 2):
                p = _prob(dtype=dtype, L=L, b=2, steps_per_launch=spl)
                shard = 2 * L * 2 * 128 * esz
                acc = pad(2 * L * 4 * 128 * 4) if dtype == 1 else 0
                if dtype == 1 and spl != 1:      # batched: N - 1 = 3 remote shards
                    want = 2 * 3 * pad(shard) + acc
                else:
                    want = 4 * pad(shard) + acc
                if dtype == 1 and L <= 4096:
                    want += pad(2 * L * 4 * 128 * 4) + pad(2 * 4 * L * 4)
                assert lib.ra_ring_fwd_workspace(ctypes.byref(p)) == want, (dtype, L, spl)
    # N <= 2: nothing to batch
    p = _prob(N=2, L=1000)
    assert lib.ra_ring_fwd_workspace(ctypes.byref(p)) == 4 * pad(1000 * 2 * 128 * 2) + pad(1000 * 4 * 128 * 4) * 2 + pad(4 * 1000 * 4)
    assert lib.ra_ring_fwd_workspace(ctypes.byref(_prob(h=3))) == 0
    assert lib.ra_ring_fwd_workspace(ctypes.byref(_prob(steps_per_launch=-1))) == 0


def test_status_strings():
    lib = _lib.lib()
    for s in (0, -1, -2, -3, -4, 17):
        assert lib.ra_status_string(s)


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("N,L", [(1, 6), (4, 6), (8, 10), (3, 64)])
def test_allowed_pairs_match_oracle(layout, N, L):
    for causal in (False, True):
        for q_shard in range(N):
            for kv in [-1] + list(range(N)):
                want = oracle_pairs(layout, N, L, q_shard, None if kv < 0 else kv, causal=causal)
                got = ra.allowed_pairs(b=1, L=L, N=N, q_shard=q_shard, kv_shard=kv,
                                       causal=causal, layout=layout)
                assert got == want
    assert ra.allowed_pairs(b=3, L=L, N=N, q_shard=0, causal=False, layout=layout) == 3 * L * L * N


def test_page3_step_accounting(golden):
    """Page 3, sections 2, 4 and 4.1 at S = 262144, N = 8, h = 32, n_kv = 8, d = 128, bf16:
    17.6 TFLOP per non-causal step, 134 MB of KV per step, 140.7 TFLOP per device per layer,
    0.94 GB received per layer, I_step = 131072 and I ~ 149797 FLOP/byte."""
    g = golden("step_accounting.json")
    S, N, b, h, n_kv, d, p = g["S"], g["N"], g["b"], g["h"], g["n_kv"], g["d"], g["bytes_per_element"]
    L = S // N
    assert accounting.step_flops_noncausal(b, L, h, d) / 1e12 == pytest.approx(g["step_tflop"], abs=0.05)
    assert accounting.kv_bytes_per_step(b, L, n_kv, d, p) / 1e6 == pytest.approx(g["step_kv_megabytes"], abs=0.5)
    assert N * accounting.step_flops_noncausal(b, L, h, d) / 1e12 == pytest.approx(g["device_layer_tflop"], abs=0.05)
    assert (N - 1) * accounting.kv_bytes_per_step(b, L, n_kv, d, p) / 1e9 == pytest.approx(g["received_gb_per_layer"], abs=0.005)
    assert accounting.step_intensity(h, n_kv, S, N) == g["I_step"]
    assert accounting.layer_intensity(h, n_kv, S, N) == pytest.approx(g["I_layer"], abs=1)
    # the A100 example: 17.6 TFLOP at 312 TFLOP/s -> 56.4 ms; 134 MB at 300 GB/s -> 0.447 ms
    ms = accounting.step_flops_noncausal(b, L, h, d) / (g["a100_peak_tflops"] * 1e12) * 1e3
    assert ms == pytest.approx(g["a100_step_ms_at_peak"], abs=0.05)
    tx = accounting.kv_bytes_per_step(b, L, n_kv, d, p) / (g["nvlink_gbps_unidirectional"] * 1e9) * 1e3
    assert tx == pytest.approx(g["nvlink_step_transfer_ms"], abs=0.001)
    assert g["a100_peak_tflops"] * 1e12 / (g["nvlink_gbps_unidirectional"] * 1e9) == g["beta_a100_nvlink"]
    # useful FLOPs from pair counts reproduce the non-causal step figure
    pairs = ra.allowed_pairs(b=b, L=L, N=N, q_shard=0, kv_shard=0, causal=False)
    assert accounting.flops_from_pairs(pairs, h, d) == accounting.step_flops_noncausal(b, L, h, d)


def test_kv_limit_host_matches_oracle_prefix_property():
    """Host accounting counts, per query row, the prefix of keys allowed; the oracle counts
    pairs from explicit positions.  Agreement per (query shard, KV shard) above pins the
    per-row limit used by the kernels for masking and tile skipping."""
    N, L = 4, 8
    for layout in LAYOUTS:
        tot = sum(ra.allowed_pairs(L=L, N=N, q_shard=i, causal=True, layout=layout) for i in range(N))
        S = N * L
        assert tot == S * (S + 1) // 2


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=0), _lib.RA_ERR_UNSUPPORTED),          # fp32 backward has no kernel
    (dict(d=64, dtype=0), _lib.RA_ERR_UNSUPPORTED),
    (dict(d=96), _lib.RA_ERR_UNSUPPORTED),
    (dict(h=3, n_kv=2), _lib.RA_ERR_INVALID_ARG),
    (dict(L=0), _lib.RA_ERR_INVALID_ARG),
    (dict(b=1, L=1 << 20, h=8192), _lib.RA_ERR_UNSUPPORTED),   # slice above 2 GiB
])
def test_backward_entry_points_reject_bad_problems(kw, status):
    lib = _lib.lib()
    p = _prob(**kw)
    assert lib.ra_bwd_preprocess(ctypes.byref(p), FAKE, FAKE, FAKE, None) == status
    assert lib.ra_step_bwd(ctypes.byref(p), 0, 0, *([FAKE] * 9), None) == status
    assert lib.ra_ring_bwd_workspace(ctypes.byref(p)) == 0
    assert lib.ra_ring_bwd(ctypes.byref(p), 0, *([FAKE] * 10), 1 << 40, None, None) == status


def test_backward_rejects_bad_shards_pointers_and_workspace():
    lib = _lib.lib()
    p = _prob()
    assert lib.ra_step_bwd(ctypes.byref(p), 4, 0, *([FAKE] * 9), None) == _lib.RA_ERR_INVALID_ARG
    assert lib.ra_step_bwd(ctypes.byref(p), 0, -1, *([FAKE] * 9), None) == _lib.RA_ERR_INVALID_ARG
    mis = ctypes.c_void_p(0x10008)
    args = [FAKE] * 9
    args[7] = mis                                        # dk_acc misaligned
    assert lib.ra_step_bwd(ctypes.byref(p), 0, 0, *args, None) == _lib.RA_ERR_INVALID_ARG
    assert lib.ra_bwd_preprocess(ctypes.byref(p), FAKE, None, FAKE, None) == _lib.RA_ERR_INVALID_ARG
    need = lib.ra_ring_bwd_workspace_min(ctypes.byref(p))
    st = lib.ra_ring_bwd(ctypes.byref(p), 0, *([FAKE] * 10), need - 1, None, None)
    assert st == _lib.RA_ERR_WORKSPACE
    assert lib.ra_ring_bwd(ctypes.byref(p), -1, *([FAKE] * 10), need, None, None) == _lib.RA_ERR_INVALID_ARG


def test_backward_workspace_is_two_kv_buffers_plus_delta():
    """Minimum: double-buffered K and V staging (as in the forward) plus D = rowsum(dO * O).
    Asked for: for shards of L <= 4096, then second dK and dV buffers (fp32 [b][L][n_kv][d]
    each) for key blocks whose query tiles run as two workgroups."""
    lib = _lib.lib()
    pad = lambda x: (x + 255) // 256 * 256  # noqa: E731
    for L, second in ((1000, True), (4096, True), (4097, False)):
        p = _prob(L=L, b=2)
        want = 4 * pad(2 * L * 2 * 128 * 2) + pad(2 * 4 * L * 4)
        assert lib.ra_ring_bwd_workspace_min(ctypes.byref(p)) == want
        extra = 2 * pad(2 * L * 2 * 128 * 4) if second else 0
        assert lib.ra_ring_bwd_workspace(ctypes.byref(p)) == want + extra, L
    assert lib.ra_ring_bwd_workspace_min(ctypes.byref(_prob(d=64))) == 0


# ------------------------------------------------------------------ packed documents (host side)
DOC_BOUNDS = np.array([0, 7, 8, 19, 33, 40], dtype=np.int32)


@pytest.mark.parametrize("layout", LAYOUTS)
def test_document_ranges_match_oracle(layout):
    from oracle import document_of, shard_tokens
    N, L = 4, 10
    for shard in range(N):
        begin, end = ra.document_ranges(DOC_BOUNDS, N=N, L=L, shard=shard, layout=layout)
        doc = document_of(shard_tokens(layout, N, L)[shard], DOC_BOUNDS)
        np.testing.assert_array_equal(begin, DOC_BOUNDS[doc])
        np.testing.assert_array_equal(end, DOC_BOUNDS[doc + 1])


@pytest.mark.parametrize("layout", LAYOUTS)
@pytest.mark.parametrize("causal", [True, False])
def test_allowed_pairs_packed_match_oracle(layout, causal):
    N, L = 4, 10
    for shard in range(N):
        begin, end = ra.document_ranges(DOC_BOUNDS, N=N, L=L, shard=shard, layout=layout)
        for kv in [-1] + list(range(N)):
            got = ra.allowed_pairs_packed(begin[None], end[None], N=N, q_shard=shard, kv_shard=kv,
                                          causal=causal, layout=layout)
            want = oracle_pairs(layout, N, L, shard, None if kv < 0 else kv, causal,
                                docs=DOC_BOUNDS)
            assert got == want, (shard, kv)


def test_document_inputs_are_validated():
    lib = _lib.lib()
    p = _prob()
    p.doc_begin = FAKE.value            # doc_end missing
    assert lib.ra_step_fwd(ctypes.byref(p), 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None) == _lib.RA_ERR_INVALID_ARG
    p.doc_end = 0x10002                 # misaligned
    assert lib.ra_step_fwd(ctypes.byref(p), 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, None) == _lib.RA_ERR_INVALID_ARG
    assert lib.ra_step_bwd(ctypes.byref(p), 0, 0, *([FAKE] * 9), None) == _lib.RA_ERR_INVALID_ARG
    with pytest.raises(ra.RaError):     # bounds must run from 0 to S, strictly increasing
        ra.document_ranges(np.array([0, 5, 5, 40], dtype=np.int32), N=4, L=10, shard=0)
    with pytest.raises(ra.RaError):
        ra.document_ranges(np.array([0, 39], dtype=np.int32), N=4, L=10, shard=0)


def test_noalloc_scratch_limit_and_validation():
    """ra_ring_fwd_noalloc: the scratch size in the header is the binding's; a problem whose
    workspace exceeds it, a bad shard and a null pointer are refused before any HIP call."""
    text = open(os.path.join(ROOT, "include", "ra.h")).read()
    m = re.search(r"#define RA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.RA_NOALLOC_SCRATCH_BYTES
    lib = _lib.lib()
    big = _prob(L=8192, h=32, n_kv=8, d=128, N=2, dtype=_lib.RA_BF16)
    assert lib.ra_ring_fwd_workspace(ctypes.byref(big)) > _lib.RA_NOALLOC_SCRATCH_BYTES
    assert lib.ra_ring_fwd_noalloc(ctypes.byref(big), 0, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == \
        _lib.RA_ERR_WORKSPACE
    assert b"scratch" in lib.ra_last_error()
    p = _prob()
    assert lib.ra_ring_fwd_noalloc(ctypes.byref(p), p.N, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) == \
        _lib.RA_ERR_INVALID_ARG
    assert lib.ra_ring_fwd_noalloc(ctypes.byref(p), 0, FAKE, None, FAKE, FAKE, FAKE, None, None) == \
        _lib.RA_ERR_INVALID_ARG
    assert b"k_all is NULL" in lib.ra_last_error()

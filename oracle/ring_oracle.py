"""Plain fp64 CPU oracle for one device's share of Ring Attention.

TEST INFRASTRUCTURE ONLY. The only code allowed to import, call or run anything in
this module is: the test suite under ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``.  The product (``ring_attention_long_amd``)
never imports it and has no CPU fallback through it.

What it computes
----------------
Ring Attention reaches exactly the plain softmax-attention result (page 1, "Blockwise
Attention and Online Softmax Formulations": the recurrence yields the identical result as
full-sequence softmax attention; page 4, "The Permutation Invariance Property"). So the
oracle *is* the plain definition of scaled dot-product attention (page 1, "The Memory and
Communication Bottlenecks in Long Sequences", the SDPA equation), evaluated over every key
of the whole sequence at once, with an explicit boolean causal mask built from global token
positions (page 1, "Causal Masking Dynamics"; page 3, section 3: the mask is applied by each
token's original position).  It never tiles over keys and never uses the online softmax,
except in ``online_blocks``, which is the pages' recurrence written out on purpose so the
tests can check that recurrence against the plain definition.

Readings taken where the pages are silent or garbled:
  * LSE = m + ln(l): natural log of the softmax denominator, in units of the *scaled* logit.
  * scale = 1/sqrt(d) with d the per-head dimension.
  * causal is inclusive: a token attends to itself (page 1, "j <= i").
  * GQA groups are consecutive: query head hq reads KV head hq // (h // n_kv).
  * a query row with no allowed key gives O = 0 and LSE = -inf (no NaN); merging such a
    partial is the identity.
  * zigzag: 2N chunks of L/2 tokens; shard p holds chunk p followed by chunk 2N-1-p.
  * packed documents: a key is allowed only in the query's own document, on top of the
    causal rule; documents are given by their global start positions.

Pins (tests/test_oracle_pins.py, tests/test_layout_pins.py, tests/test_grads_pins.py):
every public function below has at least one pin that does not retype its own formula:
closed forms (identical keys, single key, Q = 0 prefix means, a two-key softmax with a
known weight ratio), the pages' worked layout example, invariants (KV order, V-affine,
key shift, GQA == repeated-head MHA), brute force in pure Python on tiny inputs, central
finite differences for the gradients, and the pages' closed-form pair counts.

All arrays are numpy float64.  Shapes follow the pages' (batch, seq, heads, head_dim)
layout (page 1, "Practical Implementation Patterns"):
  q        [b, L, h, d]        one shard's queries
  k_all    [N, b, L, n_kv, d]  every shard's keys, each in its own local (layout) order
  v_all    [N, b, L, n_kv, d]
  O        [b, R, h, d]        R = number of query rows asked for
  LSE      [b, h, R]
"""

from __future__ import annotations

import math

import numpy as np

LAYOUTS = ("contiguous", "striped", "zigzag")


# --------------------------------------------------------------------------------------
# Sequence partition (page 1, "Causal Masking Dynamics: Striped Attention and Zig-Zag
# Topologies"; page 3, section 6)
# --------------------------------------------------------------------------------------
def shard_tokens(layout: str, N: int, L: int) -> list[np.ndarray]:
    """Global token positions held by each of the N shards, in each shard's local order.

    Built by *assigning* tokens exactly as the pages describe, not by a per-index formula:
      contiguous: the sequence cut into N consecutive pieces of L tokens (device 0 holds
                  [0, L-1], device 1 holds [L, 2L-1], ...).
      striped:    token t goes to device t mod N (page 1, "1. Striped Attention"); each
                  device keeps its tokens in increasing order.
      zigzag:     the sequence cut into 2N chunks; device p holds chunks p and 2N-1-p
                  (page 1, "2. Zig-Zag Ring Attention"), chunk p first.
    """
    if layout not in LAYOUTS:
        raise ValueError(f"unknown layout {layout!r}")
    S = N * L
    seq = np.arange(S, dtype=np.int64)
    if layout == "contiguous":
        return [seq[p * L:(p + 1) * L].copy() for p in range(N)]
    if layout == "striped":
        buckets: list[list[int]] = [[] for _ in range(N)]
        for t in range(S):
            buckets[t % N].append(t)
        return [np.asarray(b_, dtype=np.int64) for b_ in buckets]
    if L % 2:
        raise ValueError("zigzag needs an even shard length")
    chunks = np.split(seq, 2 * N)
    return [np.concatenate([chunks[p], chunks[2 * N - 1 - p]]) for p in range(N)]


def usp_tokens(layout: str, N_h: int, N_s: int, L: int) -> list[np.ndarray]:
    """Global positions held by each of the N = N_h * N_s devices of the two-dimensional
    (head x sequence) arrangement, before its first exchange (page 3, section 7: heads and
    sequence are cut at the same time; section 8's table: during attention a device holds
    S/N_s tokens of h/N_h heads).  The sequence is cut into N_s ring shards of N_h * L tokens
    under `layout`, exactly as shard_tokens(layout, N_s, N_h * L); ring shard r is then split
    into N_h consecutive pieces of L tokens, and device r * N_h + g holds piece g (all
    heads).  Returns one array of L positions per device, in the device's local order."""
    ring = shard_tokens(layout, N_s, N_h * L)
    return [ring[j // N_h][(j % N_h) * L:(j % N_h + 1) * L].copy() for j in range(N_h * N_s)]


def ring_order(N: int, shard: int) -> list[int]:
    """KV shard held at ring step k = 0..N-1 by device `shard`.

    Page 4, "The Ring Communication Protocol": each device sends to (i+1) mod N and receives
    from (i-1) mod N, so at iteration idx it holds the block of device (i - idx) mod N.
    Written as an explicit simulation of the hand-offs rather than that formula.
    """
    held = list(range(N))                   # held[p] = origin of the block device p holds
    order = []
    for _ in range(N):
        order.append(held[shard])
        held = [held[(p - 1) % N] for p in range(N)]   # every device receives from p-1
    return order


# --------------------------------------------------------------------------------------
# Plain attention over an explicit key set
# --------------------------------------------------------------------------------------
def _default_scale(d: int, scale: float | None) -> float:
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


# --------------------------------------------------------------------------------------
# Packed documents (page 3, section 5: several documents packed end to end into one window,
# with a block-diagonal mask that stops attention across documents).  `docs` lists the
# documents' global start positions followed by the window length: [0, b_1, ..., S].
# --------------------------------------------------------------------------------------
def document_of(pos, docs) -> np.ndarray:
    """Index of the document holding each global position."""
    return np.searchsorted(np.asarray(docs), np.asarray(pos), side="right") - 1


def allowed_mask(pos_q, pos_k, *, causal: bool, docs=None) -> np.ndarray:
    """[R, C] boolean: may query at pos_q[r] attend key at pos_k[c]?  Causal keeps keys at
    or before the query (inclusive); packed documents keep keys of the query's document."""
    pos_q = np.asarray(pos_q)
    pos_k = np.asarray(pos_k)
    if causal:
        m = pos_k[None, :] <= pos_q[:, None]
    else:
        m = np.ones((pos_q.size, pos_k.size), dtype=bool)
    if docs is not None:
        m &= document_of(pos_q, docs)[:, None] == document_of(pos_k, docs)[None, :]
    return m


def attend(q_rows, pos_q, keys, vals, pos_k, *, causal: bool, scale: float, docs=None):
    """softmax(q K^T * scale) V over an explicit key set, for one head.

    q_rows [R, d], keys [C, d], vals [C, dv], pos_q [R], pos_k [C]  ->  (O [R, dv], LSE [R]).
    A key is allowed for a query iff allowed_mask says so (causal: pos_k <= pos_q,
    inclusive; packed: same document).  Rows with no allowed key return O = 0, LSE = -inf.
    """
    s = (q_rows @ keys.T) * scale                                   # [R, C]
    allowed = allowed_mask(pos_q, pos_k, causal=causal, docs=docs)
    s = np.where(allowed, s, -np.inf)
    any_allowed = allowed.any(axis=1)
    m = np.where(any_allowed, s.max(axis=1, initial=-np.inf), 0.0)
    e = np.where(allowed, np.exp(s - m[:, None]), 0.0)
    den = e.sum(axis=1)
    lse = np.where(any_allowed, m + np.log(np.where(any_allowed, den, 1.0)), -np.inf)
    w = np.where(any_allowed[:, None], e / np.where(any_allowed, den, 1.0)[:, None], 0.0)
    return w @ vals, lse


def _gqa_group(h: int, n_kv: int) -> int:
    if h % n_kv:
        raise ValueError("h must be a multiple of n_kv")
    return h // n_kv


def attention_over_shards(q, k_sel, v_sel, pos_q, pos_k, *, causal, scale=None, rows=None,
                          docs=None):
    """Attention of q [b, L, h, d] against an explicit concatenated key set.

    k_sel, v_sel [b, C, n_kv, d] with global positions pos_k [C]; pos_q [L].
    Returns (O [b, R, h, d], LSE [b, h, R]) for the query rows `rows` (default: all).
    """
    b, L, h, d = q.shape
    n_kv = k_sel.shape[2]
    group = _gqa_group(h, n_kv)
    sc = _default_scale(d, scale)
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    O = np.zeros((b, rows.size, h, v_sel.shape[3]))
    LSE = np.zeros((b, h, rows.size))
    for bi in range(b):
        for hq in range(h):
            g = hq // group
            O[bi, :, hq, :], LSE[bi, hq, :] = attend(
                q[bi, rows, hq, :], pos_q[rows], k_sel[bi, :, g, :], v_sel[bi, :, g, :],
                pos_k, causal=causal, scale=sc, docs=docs)
    return O, LSE


def shard_attention(q, k_all, v_all, *, N, shard, layout="contiguous", causal=False,
                    scale=None, rows=None, docs=None):
    """What device `shard` must output after the whole ring pass: its queries attended to
    every key of the sequence (all N shards at once), with the causal mask by global
    position.  This is the quantity Ring Attention computes exactly."""
    Nk, b, L, n_kv, d = k_all.shape
    if Nk != N:
        raise ValueError("k_all must hold N shards")
    toks = shard_tokens(layout, N, L)
    k_cat = np.concatenate([k_all[j] for j in range(N)], axis=1)   # [b, N*L, n_kv, d]
    v_cat = np.concatenate([v_all[j] for j in range(N)], axis=1)
    pos_k = np.concatenate(toks)
    return attention_over_shards(q, k_cat, v_cat, toks[shard], pos_k, causal=causal,
                                 scale=scale, rows=rows, docs=docs)


def step_attention(q, k, v, *, N, q_shard, kv_shard, layout="contiguous", causal=False,
                   scale=None, rows=None, docs=None):
    """One ring step: device q_shard's queries against the single KV shard kv_shard
    (k, v [b, L, n_kv, d]).  Rows with no allowed key in this shard give (0, -inf)."""
    L = q.shape[1]
    toks = shard_tokens(layout, N, L)
    return attention_over_shards(q, k, v, toks[q_shard], toks[kv_shard], causal=causal,
                                 scale=scale, rows=rows, docs=docs)


# --------------------------------------------------------------------------------------
# Merging partial results (page 2, "FlashAttention Integration": the two partial outputs
# are rescaled to the new maximum and added; page 3, section 3: the running state must be
# carried as a whole, passing O alone is wrong)
# --------------------------------------------------------------------------------------
def merge(o_a, lse_a, o_b, lse_b):
    """Combine two normalised partials (O, LSE) over disjoint key sets.

    O_x [b, R, h, d], LSE_x [b, h, R].  The denominators are l_x = exp(LSE_x); the merged
    denominator is l_a + l_b and each partial is weighted by l_x / (l_a + l_b), computed
    around M = max(LSE_a, LSE_b) so nothing overflows.  (-inf, -inf) merges to (0, -inf).
    """
    M = np.maximum(lse_a, lse_b)
    finite = np.isfinite(M)
    Ms = np.where(finite, M, 0.0)
    wa = np.where(finite, np.exp(lse_a - Ms), 0.0)
    wb = np.where(finite, np.exp(lse_b - Ms), 0.0)
    tot = wa + wb
    lse = np.where(finite, Ms + np.log(np.where(finite, tot, 1.0)), -np.inf)
    fa = np.where(finite, wa / np.where(finite, tot, 1.0), 0.0)   # [b, h, R]
    fb = np.where(finite, wb / np.where(finite, tot, 1.0), 0.0)
    fa = np.transpose(fa, (0, 2, 1))[..., None]                    # [b, R, h, 1]
    fb = np.transpose(fb, (0, 2, 1))[..., None]
    return fa * o_a + fb * o_b, lse


# --------------------------------------------------------------------------------------
# The pages' online-softmax recurrence, written out (page 1, "Blockwise Attention and
# Online Softmax Formulations"; page 4, "Incremental Blockwise Attention")
# --------------------------------------------------------------------------------------
def online_blocks(q_rows, pos_q, blocks, *, causal, scale):
    """Run the running-max / running-sum / unnormalised-output recurrence over `blocks`
    = [(keys [C, d], vals [C, dv], pos_k [C]), ...] in the given order, for one head.

    State per row: m (running max of logits), l (running sum of exp(logit - m)),
    O (unnormalised weighted sum of values).  Initial state m = -inf, l = 0, O = 0.
    For each block: m_new = max(m, rowmax S); P = exp(S - m_new); l = exp(m - m_new) l +
    rowsum P; O = exp(m - m_new) O + P V.  Output O / l and LSE = m + ln l.
    A row that has seen no allowed key yet keeps its initial state (the factor
    exp(m - m_new) is taken as 1 while both are -inf).
    """
    R = q_rows.shape[0]
    dv = blocks[0][1].shape[1]
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    O = np.zeros((R, dv))
    for keys, vals, pos_k in blocks:
        S = (q_rows @ keys.T) * scale
        if causal:
            S = np.where(pos_k[None, :] <= pos_q[:, None], S, -np.inf)
        m_new = np.maximum(m, S.max(axis=1, initial=-np.inf))
        seen = np.isfinite(m_new)
        alpha = np.where(seen, np.exp(np.where(seen, m - np.where(seen, m_new, 0.0), 0.0)), 1.0)
        P = np.where(seen[:, None], np.exp(S - np.where(seen, m_new, 0.0)[:, None]), 0.0)
        l = alpha * l + P.sum(axis=1)
        O = alpha[:, None] * O + P @ vals
        m = m_new
    seen = l > 0
    out = np.where(seen[:, None], O / np.where(seen, l, 1.0)[:, None], 0.0)
    lse = np.where(seen, m + np.log(np.where(seen, l, 1.0)), -np.inf)
    return out, lse


# --------------------------------------------------------------------------------------
# Backward for one device's share (page 1, "The Backward Pass and Gradient Exchange";
# page 4, "The Backward Pass: Symmetric Ring Operation").  The pages only name the flows
# (P is recomputed from the saved statistics; dQ stays local; dK, dV travel with K, V);
# the gradients themselves are the textbook softmax-attention gradients, no autograd.
# --------------------------------------------------------------------------------------
def shard_grads(q, k_all, v_all, dout, *, N, shard, layout="contiguous", causal=False,
                scale=None, docs=None):
    """Gradients of sum(dout * O_shard) with respect to the shard's Q and every shard's
    K, V, where O_shard is shard_attention(...) of device `shard`.

    With P = exp(s - LSE) (0 where masked):
        dV_c  = sum_r P[r,c] dO_r
        dP    = dO V^T
        D_r   = dO_r . O_r
        dS    = P * (dP - D)
        dQ_r  = scale * sum_c dS[r,c] K_c
        dK_c  = scale * sum_r dS[r,c] Q_r
    dK, dV are summed over the query heads of each KV group and returned per KV shard:
    dq [b, L, h, d], dk, dv [N, b, L, n_kv, d].
    """
    Nk, b, L, n_kv, d = k_all.shape
    h = q.shape[2]
    group = _gqa_group(h, n_kv)
    sc = _default_scale(d, scale)
    toks = shard_tokens(layout, N, L)
    pos_q = toks[shard]
    pos_k = np.concatenate(toks)
    k_cat = np.concatenate([k_all[j] for j in range(N)], axis=1)
    v_cat = np.concatenate([v_all[j] for j in range(N)], axis=1)
    dq = np.zeros_like(q)
    dk_cat = np.zeros_like(k_cat)
    dv_cat = np.zeros_like(v_cat)
    for bi in range(b):
        for hq in range(h):
            g = hq // group
            Qh, Kh, Vh, dOh = q[bi, :, hq], k_cat[bi, :, g], v_cat[bi, :, g], dout[bi, :, hq]
            s = (Qh @ Kh.T) * sc
            allowed = allowed_mask(pos_q, pos_k, causal=causal, docs=docs)
            s = np.where(allowed, s, -np.inf)
            m = s.max(axis=1, initial=-np.inf)
            m = np.where(np.isfinite(m), m, 0.0)
            e = np.where(allowed, np.exp(s - m[:, None]), 0.0)
            den = e.sum(axis=1)
            P = np.where(den[:, None] > 0, e / np.where(den > 0, den, 1.0)[:, None], 0.0)
            Oh = P @ Vh
            dV = P.T @ dOh
            dP = dOh @ Vh.T
            D = np.sum(dOh * Oh, axis=1)
            dS = P * (dP - D[:, None])
            dq[bi, :, hq] = sc * (dS @ Kh)
            dk_cat[bi, :, g] += sc * (dS.T @ Qh)
            dv_cat[bi, :, g] += dV
    dk = np.stack(np.split(dk_cat, N, axis=1))
    dv = np.stack(np.split(dv_cat, N, axis=1))
    return dq, dk, dv


def shard_dq_rows(q, k_all, v_all, dout, rows, *, N, shard, layout="contiguous", causal=False,
                  scale=None, docs=None):
    """dQ of selected query rows only (same definition as shard_grads, evaluated for the
    given rows; a row's dQ needs only its own P, O and D).  Returns dq [b, R, h, d]."""
    Nk, b, L, n_kv, d = k_all.shape
    h = q.shape[2]
    group = _gqa_group(h, n_kv)
    sc = _default_scale(d, scale)
    toks = shard_tokens(layout, N, L)
    rows = np.asarray(rows, dtype=np.int64)
    pos_q = toks[shard][rows]
    pos_k = np.concatenate(toks)
    k_cat = np.concatenate([k_all[j] for j in range(N)], axis=1)
    v_cat = np.concatenate([v_all[j] for j in range(N)], axis=1)
    dq = np.zeros((b, rows.size, h, d))
    for bi in range(b):
        for hq in range(h):
            g = hq // group
            Qh, Kh, Vh, dOh = q[bi, rows, hq], k_cat[bi, :, g], v_cat[bi, :, g], dout[bi, rows, hq]
            s = (Qh @ Kh.T) * sc
            allowed = allowed_mask(pos_q, pos_k, causal=causal, docs=docs)
            s = np.where(allowed, s, -np.inf)
            m = s.max(axis=1, initial=-np.inf)
            m = np.where(np.isfinite(m), m, 0.0)
            e = np.where(allowed, np.exp(s - m[:, None]), 0.0)
            den = e.sum(axis=1)
            P = np.where(den[:, None] > 0, e / np.where(den > 0, den, 1.0)[:, None], 0.0)
            Oh = P @ Vh
            dP = dOh @ Vh.T
            D = np.sum(dOh * Oh, axis=1)
            dS = P * (dP - D[:, None])
            dq[bi, :, hq] = sc * (dS @ Kh)
    return dq


def key_grads(q_shards, dout_shards, k_all, v_all, *, N, query_shards, kv_head, cols,
              layout="contiguous", causal=False, scale=None, docs=None, rows=None, row_block=128):
    """dK and dV of selected keys of one KV head (same definition as shard_grads), summed
    over the KV group's query heads and over the rows `rows` (default: every row) of each
    of the listed query shards.

    q_shards, dout_shards [Q, b, L, h, d] hold the queries and output gradients of the
    query shards named by `query_shards` (length Q, same order); k_all, v_all
    [N, b, L, n_kv, d] every shard's keys and values; `cols` lists keys as (kv shard,
    local index) pairs.  Returns dk, dv [b, C, d] for those C keys.  Both are sums over
    rows, so disjoint row sets may be evaluated separately and added.

    A key's gradients need P and D of every row that may attend to it, and those need the
    row's softmax over the whole sequence: so each row is evaluated against every key
    (s, the mask, P = softmax over the allowed keys, O = P V, D = dO . O), and only the
    selected keys' columns of P and dS = P * (dP - D) are kept:
        dV_c = sum_r P[r,c] dO_r,   dK_c = scale * sum_r dS[r,c] Q_r.
    Rows are taken `row_block` at a time (each row's quantities depend on that row alone);
    keys that no row of the block may attend carry weight zero and are left out.
    """
    Nk, b, L, n_kv, d = k_all.shape
    h = q_shards.shape[3]
    group = _gqa_group(h, n_kv)
    sc = _default_scale(d, scale)
    toks = shard_tokens(layout, N, L)
    pos_k = np.concatenate(toks)                            # key j*L + u is (shard j, local u)
    sel = np.asarray([j * L + u for j, u in cols], dtype=np.int64)
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    dk = np.zeros((b, sel.size, d))
    dv = np.zeros((b, sel.size, d))
    g = kv_head
    for qi, i in enumerate(query_shards):
        for r0 in range(0, rows.size, row_block):
            rr = rows[r0:r0 + row_block]
            allowed = allowed_mask(toks[i][rr], pos_k, causal=causal, docs=docs)   # [R, S]
            keep = np.flatnonzero(allowed.any(axis=0) | np.isin(np.arange(pos_k.size), sel))
            allowed = allowed[:, keep]
            where_sel = np.searchsorted(keep, sel)                  # selected keys among `keep`
            for bi in range(b):
                Kh, Vh = k_all[keep // L, bi, keep % L, g], v_all[keep // L, bi, keep % L, g]
                for hq in range(g * group, (g + 1) * group):
                    Qr, dOr = q_shards[qi, bi, rr, hq], dout_shards[qi, bi, rr, hq]
                    s = np.where(allowed, (Qr @ Kh.T) * sc, -np.inf)
                    m = s.max(axis=1, initial=-np.inf)
                    m = np.where(np.isfinite(m), m, 0.0)
                    e = np.where(allowed, np.exp(s - m[:, None]), 0.0)
                    den = e.sum(axis=1)
                    P = np.where(den[:, None] > 0, e / np.where(den > 0, den, 1.0)[:, None], 0.0)
                    D = np.sum(dOr * (P @ Vh), axis=1)
                    Pc = P[:, where_sel]
                    dS = Pc * (dOr @ Vh[where_sel].T - D[:, None])
                    dk[bi] += sc * (dS.T @ Qr)
                    dv[bi] += Pc.T @ dOr
    return dk, dv


# --------------------------------------------------------------------------------------
# Work accounting by direct count (page 3, section 6: work is the number of allowed
# query-key pairs; page 3, section 2: total FLOPs 4 b S^2 h d non-causal)
# --------------------------------------------------------------------------------------
def allowed_pairs(layout: str, N: int, L: int, q_shard: int, kv_shard: int | None = None,
                  causal: bool = True, docs=None) -> int:
    """Number of (query, key) pairs device q_shard may attend to, against one KV shard or
    (kv_shard=None) the whole sequence.  Counted from the explicit positions."""
    toks = shard_tokens(layout, N, L)
    pos_q = toks[q_shard]
    pos_k = np.sort(np.concatenate(toks) if kv_shard is None else toks[kv_shard])
    if docs is not None:
        return int(allowed_mask(pos_q, pos_k, causal=causal, docs=docs).sum())
    if not causal:
        return int(pos_q.size * pos_k.size)
    return int(np.searchsorted(pos_k, pos_q, side="right").sum())


# --------------------------------------------------------------------------------------
# Brute force for tiny inputs: pure Python loops, math.exp, no numpy arithmetic
# --------------------------------------------------------------------------------------
def brute_force_row(q_row, keys, vals, allowed, scale):
    """One query row, one head: returns (O list, LSE float); ([0..], -inf) if none allowed."""
    logits = []
    for c, kc in enumerate(keys):
        if allowed[c]:
            logits.append((c, scale * sum(float(a) * float(b_) for a, b_ in zip(q_row, kc))))
    dv = len(vals[0])
    if not logits:
        return [0.0] * dv, -math.inf
    mx = max(x for _, x in logits)
    z = sum(math.exp(x - mx) for _, x in logits)
    out = [0.0] * dv
    for c, x in logits:
        w = math.exp(x - mx) / z
        for e in range(dv):
            out[e] += w * float(vals[c][e])
    return out, mx + math.log(z)

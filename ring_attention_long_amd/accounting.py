"""Work and traffic accounting for the ring pass (host-side arithmetic only).

Formulas follow page 3 (section 2, invariants; section 4, arithmetic intensity; section 4.1,
the per-step example) and page 1 ("Overlapping Arithmetic and Communication Ratios"):
  * one non-causal step of L queries against L keys: 4 b L^2 h d FLOPs (two GEMMs,
    2 FLOPs per multiply-add);
  * with a causal mask only allowed pairs count: 4 h d FLOPs per allowed (query, key) pair;
  * KV bytes received per step: 2 b L n_kv d p (K and V, p bytes per element);
  * step intensity I_step = (h / n_kv) * L and whole-layer intensity
    I = (h / n_kv) * S / (N - 1) FLOPs per received byte;
  * all-to-all sequence parallelism (page 3, sections 4.2 and 7): per device and layer the
    two exchanges move (N-1)/N of its S/N slice of Q and O (h heads) and K and V (n_kv
    heads), and the attention work is 4 b S^2 (h/N) d, the same as a ring device's;
  * the two-dimensional arrangement (page 3, sections 7 and 8) receives "between the two,
    by the split": the all-to-all among N_h devices on S/N_s tokens plus a ring over N_s.
"""
from __future__ import annotations

MI355X_BF16_DENSE_TFLOPS = 2516.6    # 256 CU x 2.4 GHz x 4096 FLOP/clk/CU, dense
MI355X_HBM_GBPS = 8000.0


def step_flops_noncausal(b: int, L: int, h: int, d: int) -> int:
    return 4 * b * L * L * h * d


def flops_from_pairs(pairs: int, h: int, d: int) -> int:
    """Useful forward FLOPs for `pairs` allowed (query, key) pairs per query head
    (pairs already summed over the batch)."""
    return 4 * h * d * pairs


def kv_bytes_per_step(b: int, L: int, n_kv: int, d: int, elem_bytes: int) -> int:
    return 2 * b * L * n_kv * d * elem_bytes


def step_intensity(h: int, n_kv: int, S: int, N: int) -> float:
    return (h / n_kv) * (S / N)


def layer_intensity(h: int, n_kv: int, S: int, N: int) -> float:
    return (h / n_kv) * S / (N - 1)


def merge_bytes(b: int, L: int, h: int, d: int) -> int:
    """HBM bytes of one standalone merge: read O_acc, O_part, write O_acc (fp32) plus the
    same three passes over the LSE rows."""
    return 3 * 4 * b * L * h * d + 3 * 4 * b * h * L


def ring_kv_bytes_per_pass(b: int, S: int, N: int, n_kv: int, d: int, elem_bytes: int) -> int:
    """KV bytes one device receives over a forward ring pass: N-1 shards (its own is local)."""
    return (N - 1) * kv_bytes_per_step(b, S // N, n_kv, d, elem_bytes)


def ulysses_bytes_per_device(b: int, S: int, N: int, h: int, n_kv: int, d: int, elem_bytes: int) -> float:
    """Bytes one device receives in the two all-to-all exchanges of one layer: (N-1)/N of an
    S/N slice of Q and O (h heads each) and of K and V (n_kv heads each)."""
    return (N - 1) / N * b * (S / N) * (2 * h + 2 * n_kv) * d * elem_bytes


def usp_bytes_per_device(b: int, S: int, N_h: int, N_s: int, h: int, n_kv: int, d: int,
                         elem_bytes: int) -> float:
    """Bytes one device of the two-dimensional arrangement (N_h head groups x N_s sequence
    shards; page 3, sections 7 and 8) receives per layer: the two all-to-all exchanges among
    the N_h devices that share a ring shard of S/N_s tokens, plus the ring over the N_s
    devices of its head group, which passes the K and V of n_kv/N_h heads.  N_h = 1 gives
    the ring's figure and N_s = 1 the all-to-all's; other splits lie between the two."""
    a2a = ulysses_bytes_per_device(b, S // N_s, N_h, h, n_kv, d, elem_bytes)
    ring = (N_s - 1) / N_s * 2 * b * S * (n_kv / N_h) * d * elem_bytes
    return a2a + ring


def ulysses_flops_noncausal(b: int, S: int, N: int, h: int, d: int) -> int:
    """Attention work of one device after the exchange: whole sequence, h/N heads."""
    return 4 * b * S * S * (h // N) * d


def bwd_bytes_per_step_kv_rotating(b: int, L: int, n_kv: int, d: int, elem_bytes: int,
                                   acc_bytes: int = 4) -> int:
    """Backward ring step with K, V and their gradient accumulators rotating (page 4, "The
    Backward Pass: Symmetric Ring Operation": (k, v, dk, dv) move together)."""
    return b * L * n_kv * d * (2 * elem_bytes + 2 * acc_bytes)


def bwd_bytes_per_step_kv_stationary(b: int, L: int, h: int, d: int, elem_bytes: int,
                                     acc_bytes: int = 4) -> int:
    """Backward ring step with K, V stationary (page 1, "The Backward Pass and Gradient
    Exchange"): a query shard's Q and dO, its LSE and D (fp32) and its dQ accumulator move."""
    return b * L * h * d * (2 * elem_bytes + acc_bytes) + 2 * 4 * b * h * L

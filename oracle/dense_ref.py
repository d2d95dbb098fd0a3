"""Dense attention on contiguous K/V: the brute-force cross-check of the paged
oracle.

TEST INFRASTRUCTURE ONLY - see ``oracle/__init__.py``.

Standard attention works on a contiguous KV cache (Dissecting vLLM,
"PagedAttention: Virtual Memory for KV Cache"); this is that formulation,
written as whole-matrix numpy on the per-sequence K/V *before* they are laid
into blocks. It never sees a block table, so agreement with
``paged_ref.decode_ref`` pins the table walk, and agreement of both with the
closed forms in the tests pins the arithmetic.

    O = softmax(scale * Q K^T + M) V

with K, V repeated along the head axis so query head h uses KV head h // G,
and M = -inf above the bottom-right causal diagonal when ``causal`` is set
(query row i of L_q sees keys 0 .. n - L_q + i), 0 elsewhere.
"""

import numpy as np

from .numerics import to_f64


def dense_attention_ref(q, k, v, scale, causal=False):
    """q: [L_q, H_q, d]; k, v: [n, H_kv, d] contiguous; returns [L_q, H_q, d] f64."""
    q = to_f64(q)
    k = to_f64(k)
    v = to_f64(v)
    q_len, num_q_heads, _ = q.shape
    n, num_kv_heads, _ = k.shape
    if n == 0:
        return np.zeros_like(q)
    group = num_q_heads // num_kv_heads
    k_rep = np.repeat(k, group, axis=1)          # [n, H_q, d]
    v_rep = np.repeat(v, group, axis=1)
    logits = scale * np.einsum("qhd,nhd->hqn", q, k_rep)   # [H_q, L_q, n]
    if causal:
        rows = np.arange(q_len)[:, None]
        cols = np.arange(n)[None, :]
        allowed = cols <= (n - q_len + rows)
        logits = np.where(allowed[None, :, :], logits, -np.inf)
    logits = logits - logits.max(axis=-1, keepdims=True)
    weights = np.exp(logits)
    weights = weights / weights.sum(axis=-1, keepdims=True)
    return np.einsum("hqn,nhd->qhd", weights, v_rep)

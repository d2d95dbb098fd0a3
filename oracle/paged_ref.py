"""Paged-attention oracle: scatter, decode and prefill chunk, walked through a
block table in float64.

TEST INFRASTRUCTURE ONLY - see ``oracle/__init__.py``.

What the pages fix, and which passage each step follows:

* The KV cache is cut into fixed-size physical blocks of 16 or 32 tokens and a
  per-sequence block table maps logical token positions to physical blocks
  (How vLLM gets real throughput on H100s, "PagedAttention borrows from
  operating systems"; vLLM architecture, memory and benchmarks deep dive,
  "PagedAttention: a 1960s idea for modern GPUs").
* The attention kernel walks that table at run time and gathers K/V from the
  scattered blocks (Dissecting vLLM, "PagedAttention: Virtual Memory for KV
  Cache"). Paging changes where K and V live, not what attention computes, so
  the result is plain scaled-dot-product softmax attention over the logical
  sequence; the oracle evaluates exactly that, in logical order.
* Decode attends one new query per sequence over all tokens before it and the
  token itself (High-Throughput LLM Inference & Training, the "token 501"
  passage); grouped-query attention shares each KV head among a group of query
  heads (all three blog rewrites: 4 KV heads, head dim 256).
* Prefill is dense, and a chunk of a long prompt is processed against the cache
  interleaved with decode tokens (vLLM architecture... deep dive, "Hardware-level
  optimizations"); a chunk row sees every cached key up to its own position.

Readings where the pages are silent:

* cache layout ``[num_blocks, num_kv_heads, block_size, head_dim]``, K and V in
  separate tensors; slot = physical_block * block_size + offset; slot < 0 skips.
* query head ``h`` reads KV head ``h // (num_q_heads // num_kv_heads)``.
* ``context_lens`` counts the new token, whose K/V were written first.
* a sequence with context 0 yields a zero output row.
* block-table entries past ``ceil(n / block_size)`` and slots past ``n`` in the
  last block are never read (they may hold anything, NaN included).

The softmax here is the two-pass definition (max, then exponentials and their
sum); it shares no algorithm with the device's online softmax.
"""

import numpy as np

from .numerics import to_f64


def reshape_and_cache_ref(key, value, key_cache, value_cache, slot_mapping):
    """Return copies of the caches with token ``t``'s K/V written to slot
    ``slot_mapping[t]``.

    key, value:              [T, H_kv, d]  stored element type
    key_cache, value_cache:  [NB, H_kv, bs, d], same element type
    slot_mapping:            [T] integers; slot = block * bs + offset; < 0 skips

    A pure copy: every written element carries the source's exact bits and
    every other element keeps its prior bits. (Blocks are filled as tokens
    arrive: How vLLM gets real throughput on H100s, "PagedAttention borrows
    from operating systems".)
    """
    key = np.asarray(key)
    value = np.asarray(value)
    kc = np.array(key_cache, copy=True)
    vc = np.array(value_cache, copy=True)
    if key.dtype != kc.dtype or value.dtype != vc.dtype:
        raise TypeError("cache and source element types differ")
    block_size = kc.shape[2]
    slots = np.asarray(slot_mapping).astype(np.int64)
    for t in range(key.shape[0]):
        slot = int(slots[t])
        if slot < 0:
            continue
        block, offset = divmod(slot, block_size)
        for h in range(key.shape[1]):
            kc[block, h, offset, :] = key[t, h, :]
            vc[block, h, offset, :] = value[t, h, :]
    return kc, vc


def _gather_sequence(cache, block_table_row, n, kv_head):
    """Logical rows 0..n-1 of one KV head, looked up through the block table:
    position j lives in physical block table[j // bs], row j % bs."""
    block_size = cache.shape[2]
    positions = np.arange(n)
    phys = np.asarray(block_table_row)[positions // block_size].astype(np.int64)
    return to_f64(cache[phys, kv_head, positions % block_size, :])


def _softmax_weighted_sum(scores, values):
    """Two-pass softmax of ``scores`` (length n) applied to ``values`` [n, d]."""
    m = np.max(scores)
    p = np.exp(scores - m)
    return (p @ values) / np.sum(p)


def decode_ref(query, key_cache, value_cache, block_tables, context_lens, scale):
    """Decode attention for one query per sequence, float64 output.

    query:        [S, H_q, d]          stored element type
    key_cache:    [NB, H_kv, bs, d]
    value_cache:  [NB, H_kv, bs, d]
    block_tables: [S, max_blocks]      physical block ids
    context_lens: [S]                  tokens attended, including the new one
    scale:        softmax scale (1/sqrt(d) in every workload here)

    out[b, h] = sum_j softmax_j(scale * q[b,h] . k_j) v_j over j < n_b, with
    k_j, v_j the rows of KV head h // G at logical position j.
    """
    q_all = to_f64(query)
    num_seqs, num_q_heads, head_dim = q_all.shape
    num_kv_heads = key_cache.shape[1]
    if num_q_heads % num_kv_heads:
        raise ValueError("query heads must be a multiple of KV heads")
    group = num_q_heads // num_kv_heads
    out = np.zeros((num_seqs, num_q_heads, head_dim), dtype=np.float64)
    for b in range(num_seqs):
        n = int(context_lens[b])
        if n == 0:
            continue
        for kv in range(num_kv_heads):
            keys = _gather_sequence(key_cache, block_tables[b], n, kv)
            vals = _gather_sequence(value_cache, block_tables[b], n, kv)
            for h in range(kv * group, (kv + 1) * group):
                scores = scale * (keys @ q_all[b, h])
                out[b, h] = _softmax_weighted_sum(scores, vals)
    return out


def prefill_chunk_ref(query, key_cache, value_cache, block_tables, context_lens,
                      cu_q_lens, scale):
    """Causal chunk attention against the paged cache, float64 output.

    query:      [total_q, H_q, d]; rows cu_q_lens[b] .. cu_q_lens[b+1]-1 belong
                to sequence b, whose chunk K/V are already in the cache.
    context_lens[b] = n counts the cached prefix plus the chunk; with L_q chunk
    rows, row i sits at absolute position n - L_q + i and sees keys 0 .. that
    position (the chunk's last row is aligned with the last cached token).
    """
    q_all = to_f64(query)
    total_q, num_q_heads, head_dim = q_all.shape
    num_kv_heads = key_cache.shape[1]
    group = num_q_heads // num_kv_heads
    out = np.zeros((total_q, num_q_heads, head_dim), dtype=np.float64)
    cu = np.asarray(cu_q_lens).astype(np.int64)
    for b in range(len(cu) - 1):
        n = int(context_lens[b])
        q_len = int(cu[b + 1] - cu[b])
        if q_len == 0:
            continue
        if q_len > n:
            raise ValueError("chunk longer than the context that holds it")
        for kv in range(num_kv_heads):
            keys = _gather_sequence(key_cache, block_tables[b], n, kv)
            vals = _gather_sequence(value_cache, block_tables[b], n, kv)
            for i in range(q_len):
                visible = n - q_len + i + 1
                for h in range(kv * group, (kv + 1) * group):
                    scores = scale * (keys[:visible] @ q_all[cu[b] + i, h])
                    out[cu[b] + i, h] = _softmax_weighted_sum(scores, vals[:visible])
    return out


def attention_partial_ref(query_row, keys, values, scale):
    """One partial result of attention over a subset of a row's keys, the
    quantity a context split produces: with s_j = scale * q . k_j,
    m = max_j s_j, l = sum_j exp(s_j - m), o = sum_j exp(s_j - m) v_j / l.
    An empty subset gives (o = 0, m = -inf, l = 0).

    query_row: [d] float64; keys, values: [n, d] float64. Returns (o, m, l)."""
    if keys.shape[0] == 0:
        return np.zeros(values.shape[1]), -np.inf, 0.0
    s = scale * (keys @ query_row)
    m = np.max(s)
    p = np.exp(s - m)
    return (p @ values) / np.sum(p), m, float(np.sum(p))


def merge_partials_ref(partials):
    """Attention over the union of disjoint key subsets from their partials
    (o_i, m_i, l_i): with M = max_i m_i and w_i = l_i exp(m_i - M),
    out = sum_i w_i o_i / sum_i w_i. Empty partials (l_i = 0) contribute
    nothing; if every partial is empty the result is 0 (an empty context)."""
    live = [(o, m, l) for o, m, l in partials if l > 0]
    if not live:
        return np.zeros_like(partials[0][0])
    big_m = max(m for _, m, _ in live)
    w = [l * np.exp(m - big_m) for _, m, l in live]
    return sum(wi * o for wi, (o, _, _) in zip(w, live)) / sum(w)


def decode_shared_prefix_ref(query, key_cache, value_cache, block_tables, context_lens,
                             cu_groups, prefix_lens, scale):
    """Decode for sequences grouped by a shared prompt, evaluated the way the
    sharing allows: group g is sequences cu_groups[g] .. cu_groups[g+1] - 1,
    whose first P_g = prefix_lens[g] positions hold the same K/V (forked
    rollouts of one prompt point at the prompt's physical blocks: How vLLM
    gets real throughput on H100s, "PagedAttention borrows from operating
    systems"; Dissecting vLLM, "PagedAttention: Virtual Memory for KV
    Cache"). For a member b with n_b tokens, one partial covers positions
    0 .. min(P_g, n_b) - 1, read through the group's FIRST member's table, and
    one covers P_g .. n_b - 1 through b's own table; the two are merged with
    merge_partials_ref. Sequences in no group are attended as in decode_ref.
    When the prefix really is shared this equals decode_ref up to rounding
    order (the merge is exact); it is the definition the grouped device path
    follows, checked against decode_ref by the pins."""
    q_all = to_f64(query)
    num_seqs, num_q_heads, head_dim = q_all.shape
    num_kv_heads = key_cache.shape[1]
    group = num_q_heads // num_kv_heads
    out = np.zeros((num_seqs, num_q_heads, head_dim), dtype=np.float64)
    cu = np.asarray(cu_groups).astype(np.int64)
    owner = {}  # sequence -> (first member, prefix length)
    for g in range(len(cu) - 1):
        for b in range(int(cu[g]), int(cu[g + 1])):
            owner[b] = (int(cu[g]), int(prefix_lens[g]))
    for b in range(num_seqs):
        n = int(context_lens[b])
        first, p_len = owner.get(b, (b, 0))
        shared = min(p_len, n)
        for kv in range(num_kv_heads):
            k_pre = _gather_sequence(key_cache, block_tables[first], shared, kv)
            v_pre = _gather_sequence(value_cache, block_tables[first], shared, kv)
            k_all = _gather_sequence(key_cache, block_tables[b], n, kv)
            v_all = _gather_sequence(value_cache, block_tables[b], n, kv)
            k_tail, v_tail = k_all[shared:], v_all[shared:]
            for h in range(kv * group, (kv + 1) * group):
                parts = [attention_partial_ref(q_all[b, h], k_pre, v_pre, scale),
                         attention_partial_ref(q_all[b, h], k_tail, v_tail, scale)]
                out[b, h] = merge_partials_ref(parts)
    return out

"""KV-cache footprint and slot accounting (closed forms from the pages).

TEST INFRASTRUCTURE ONLY - see ``oracle/__init__.py``.

* Footprint: the cache stores K and V (the factor 2) for every full-attention
  layer, KV head, head-dim element and token, each at the stored precision:
  M = 2 * L * H_kv * d_head * T * b (High-Throughput LLM Inference &
  Training, KV-footprint paragraph; per layer, L = 1, in vLLM architecture,
  memory and benchmarks deep dive, "Why the KV cache eats your VRAM").
* Contiguous reservation gives every request room for the maximum length;
  paged allocation gives a request ceil(n / bs) blocks of bs slots, so only the
  last block can hold unused slots (same two pages: Figures 1 and 2, and
  "PagedAttention: a 1960s idea for modern GPUs").
"""


def kv_bytes(num_layers, num_kv_heads, head_dim, num_tokens, bytes_per_elem):
    """Bytes of K plus V for one sequence: 2 * L * H_kv * d * T * b."""
    return 2 * num_layers * num_kv_heads * head_dim * num_tokens * bytes_per_elem


def blocks_needed(n, block_size):
    """Blocks a sequence of n tokens occupies: ceil(n / block_size)."""
    if n < 0 or block_size <= 0:
        raise ValueError("need n >= 0 and block_size > 0")
    return -(-n // block_size)


def paged_slots(lengths, block_size):
    """Token slots reserved by paged allocation: sum of bs * ceil(n / bs)."""
    return sum(block_size * blocks_needed(n, block_size) for n in lengths)


def contiguous_slots(lengths, max_len):
    """Token slots reserved when every request gets room for ``max_len``."""
    if any(n > max_len for n in lengths):
        raise ValueError("a request exceeds the reserved maximum")
    return len(lengths) * max_len


def internal_fragmentation(lengths, block_size):
    """Unused fraction of the slots that paged allocation reserves."""
    reserved = paged_slots(lengths, block_size)
    if reserved == 0:
        return 0.0
    return (reserved - sum(lengths)) / reserved

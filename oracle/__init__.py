"""Plain CPU oracle for paged attention.

TEST INFRASTRUCTURE ONLY. This package exists to prove the HIP library right;
it is never part of the product path. Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it. It imports nothing from ``paged_kv_cache_215_amd`` (the HIP path)
and the HIP path imports nothing from here: the two share no code, headers,
helpers or constants.

Everything is plain numpy in float64, written from the definitions on the
source pages, with no blocking, fusion or reordering beyond what those
definitions state:

* ``paged_ref.reshape_and_cache_ref`` - cache-write scatter through a slot map.
* ``paged_ref.decode_ref``            - one-query-per-sequence attention walked
                                        through a block table, two-pass softmax.
* ``paged_ref.prefill_chunk_ref``     - causal query chunk against the cache.
* ``paged_ref.attention_partial_ref`` / ``merge_partials_ref`` - the partial
                                        result of one context split and the
                                        log-sum-exp merge of partials.
* ``paged_ref.decode_shared_prefix_ref`` - decode of copy-on-write groups as a
                                        shared-prefix partial (first member's
                                        table) merged with each tail.
* ``dense_ref.dense_attention_ref``   - the same attention as a matrix formula
                                        on contiguous K/V (no block table).
* ``accounting``                      - KV footprint closed form and slot
                                        accounting for paged vs contiguous
                                        allocation.
* ``block_manager``                   - block pool with on-demand allocation,
                                        reference-counted sharing, copy-on-write
                                        at divergence, and the block copy.
* ``scheduler``                       - iteration-level batching: eject, resume,
                                        admit, chunked prefill, decode, and
                                        preemption by swapping to host blocks.
* ``fp8``                             - E4M3 code values, the saturating
                                        round-to-nearest-even quantizer with
                                        per-head scales, FP8 scatter, decode and
                                        chunked prefill on the dequantized cache.

Pins (checked by ``tests/test_oracle*.py`` with ``-m "not gpu"``): dense
brute force, closed forms (n = 1, uniform keys, two-token softmax, GQA head
mapping), invariance under block permutation, copy-on-write sharing, NaN
poison in unused slots and block size, and the pages' printed numbers for
the KV footprint and the Figure 1/2 allocation example.
"""

from . import accounting, dense_ref, numerics, paged_ref  # noqa: F401
from .accounting import (  # noqa: F401
    contiguous_slots,
    internal_fragmentation,
    kv_bytes,
    paged_slots,
)
from . import block_manager, fp8, scheduler  # noqa: F401
from .dense_ref import dense_attention_ref  # noqa: F401
from .numerics import bf16_bits_to_f64, to_f64  # noqa: F401
from .paged_ref import (  # noqa: F401
    attention_partial_ref,
    decode_ref,
    decode_shared_prefix_ref,
    merge_partials_ref,
    prefill_chunk_ref,
    reshape_and_cache_ref,
)

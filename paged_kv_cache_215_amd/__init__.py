"""Paged attention for AMD Instinct MI355X (gfx950).

A KV cache cut into fixed-size physical blocks of 16 or 32 tokens, mapped per
sequence by a block table, with three operations implemented as hand-written
HIP kernels behind the C ABI in ``include/pa.h``:

* ``pa_reshape_and_cache`` - scatter new K/V rows into their block slots;
* ``pa_decode``            - one-query-per-sequence attention (GQA) over the
                             paged context, split over the context with a
                             separate merge kernel;
* ``pa_prefill_chunk``     - a causal query chunk against the paged cache on
                             the matrix cores;
* ``pa_decode_shared``     - decode of a batch with copy-on-write groups: each
                             group's shared prompt blocks read once for all
                             its members (a matrix-core pass), each member's
                             tail by the decode kernels, merged by
                             log-sum-exp; ``find_shared_prefixes`` finds the
                             groups from the block tables;
* ``pa_decode_noalloc``    - ``pa_decode`` on a static scratch inside the
                             library, for callers that cannot allocate;
* ``pa_reshape_and_cache_fp8`` / ``pa_decode_fp8`` / ``pa_prefill_chunk_fp8``
                           - the same scatter, decode and prefill chunk over
                             an FP8 (E4M3) cache with one scale per KV head
                             for K and for V;
* ``BlockManager`` / ``pa_copy_blocks`` - the host block manager (on-demand
                             blocks, reference-counted sharing, copy-on-write)
                             and the device block copy it asks for;
* ``pa_swap_out`` / ``pa_swap_in`` - batched block moves between the device
                             cache and a pinned host pool (preemption);
* ``Scheduler``            - the iteration-level batching scheduler (C++);
* ``engine.Engine``        - the C++ step driver of ``include/pa_engine.h``:
                             runs the scheduler's plans on the GPU (BF16 or
                             FP8 caches), with decode-only iterations
                             replayed from a HIP graph.

The Python functions below only marshal torch tensors to that ABI.
"""

from ._lib import (  # noqa: F401
    LIB_PATH,
    PA_DTYPE_BF16,
    PA_DTYPE_F32,
    PA_DTYPE_FP8_E4M3,
    SIGNATURES,
    BlockManager,
    Scheduler,
    PaError,
    lib,
    decode_workspace,
    pa_copy_blocks,
    pa_swap_in,
    pa_swap_out,
    pa_decode,
    pa_decode_fp8,
    pa_decode_noalloc,
    pa_decode_shared,
    pa_decode_shared_workspace_size,
    decode_shared_workspace,
    find_shared_prefixes,
    pa_decode_workspace_init,
    pa_decode_workspace_size,
    pa_prefill_chunk,
    pa_prefill_chunk_fp8,
    pa_prefill_chunk_workspace_size,
    pa_reshape_and_cache,
    pa_reshape_and_cache_fp8,
)

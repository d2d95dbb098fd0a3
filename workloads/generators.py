"""Seeded generators for the paged-attention workloads.

Structure (context lengths, block tables, pool size, slot mapping) comes from
``numpy.random.default_rng(seed)``; values come from a seeded torch generator
on the target device: N(0, 1) drawn in float32 and rounded to the stored type
(round-to-nearest-even for BF16). Every slot that no sequence owns - the tail
of a sequence's last block and every block nobody holds - is filled with NaN,
so a reader of unowned memory shows up in the result.

Workload recipes (shapes from the pages' GQA example of 4 KV heads and head
dimension 256; sharing from their GRPO rollouts; lengths from their
continuous-batching example of 50/120/240/1024 generated tokens):

  c1_tiny          1 seq, 1 layer, 1 KV / 4 query heads, d 64, bs 16, n = 100,
                   fp32, pool of 32 blocks, table = first 7 of a permutation.
  c2_layer_decode  32 seqs, 4 KV / 16 query heads, d 256, bs 16, BF16,
                   n ~ U{512..8192}, pool = ceil(1.1 * blocks), shuffled.
  c3_full_step     64 seqs x 16 layers, n = 8192, bs 32, BF16; exactly 16384
                   blocks per layer, permuted; the new token (position 8191) is
                   written through the slot mapping before it is attended.
  c4_grpo_cow      8 prompts x 16 rollouts; each prompt's 4096 tokens sit in
                   blocks shared by its rollouts, private tails ~ U{0..1024}.
  c5_mixed_step    255 decode seqs, n = min(Geom(1/1500), 6000) + one of
                   {50, 120, 240, 1024}, new token written first; plus one
                   512-row prefill chunk on a 3584-token paged prefix.
"""

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

BF16 = torch.bfloat16
F32 = torch.float32


@dataclass
class PagedLayout:
    """Block-table structure of a batch (host side, numpy)."""

    block_size: int
    num_blocks: int                 # physical pool size
    context_lens: np.ndarray        # int32 [S]
    block_tables: np.ndarray        # int32 [S, max_blocks]; -1 past each sequence's blocks
    used_slots: np.ndarray          # int32 [num_blocks]; slots some sequence owns (0..bs)


def _ceil_div(a, b):
    return -(-a // b)


def draw_layout(rng, context_lens, block_size, *, pool_slack=0.1, exact_pool=False,
                shared_prefix=None, pool_blocks=None):
    """Assign physical blocks to sequences from a shuffled pool.

    shared_prefix = (group_size, prefix_len): consecutive groups of
    ``group_size`` sequences share the blocks of their first ``prefix_len``
    tokens (prefix_len a multiple of block_size); the remaining tokens of each
    sequence go to private blocks. The pool holds ``pool_blocks`` blocks if
    given, else exactly the blocks needed (``exact_pool``), else that count
    times 1 + ``pool_slack``, rounded up. Blocks are drawn without replacement
    in the order of ``rng.permutation(pool)``.
    """
    lens = np.asarray(context_lens, dtype=np.int64)
    num_seqs = len(lens)
    if shared_prefix is not None:
        group_size, prefix_len = shared_prefix
        if prefix_len % block_size:
            raise ValueError("shared prefix must end on a block boundary")
        if num_seqs % group_size:
            raise ValueError("sequence count must be a multiple of the group size")
        if np.any(lens < prefix_len):
            raise ValueError("every sharing sequence must hold the whole prefix")
        prefix_blocks = prefix_len // block_size
        num_groups = num_seqs // group_size
        private = [_ceil_div(int(n) - prefix_len, block_size) for n in lens]
        total = num_groups * prefix_blocks + sum(private)
    else:
        prefix_blocks = 0
        private = [_ceil_div(int(n), block_size) for n in lens]
        total = sum(private)

    if pool_blocks is not None:
        if pool_blocks < total:
            raise ValueError("pool smaller than the blocks the batch needs")
        pool = int(pool_blocks)
    else:
        pool = total if exact_pool else int(np.ceil((1.0 + pool_slack) * total))
    pool = max(pool, 1)
    order = rng.permutation(pool).astype(np.int64)
    cursor = 0

    def take(count):
        nonlocal cursor
        got = order[cursor:cursor + count]
        cursor += count
        return got

    blocks_per_seq = [prefix_blocks + p for p in private]
    max_blocks = max(1, max(blocks_per_seq) if blocks_per_seq else 1)
    tables = np.full((num_seqs, max_blocks), -1, dtype=np.int32)
    used = np.zeros(pool, dtype=np.int32)
    if shared_prefix is not None:
        group_size = shared_prefix[0]
        for grp in range(num_seqs // group_size):
            shared = take(prefix_blocks)
            used[shared] = block_size
            for b in range(grp * group_size, (grp + 1) * group_size):
                tables[b, :prefix_blocks] = shared
    for b in range(num_seqs):
        own = take(private[b])
        tables[b, prefix_blocks:prefix_blocks + private[b]] = own
        used[own] = block_size
        if private[b]:
            tail = int(lens[b]) % block_size
            if tail:
                used[own[-1]] = tail
    return PagedLayout(block_size, pool, lens.astype(np.int32), tables, used)


@dataclass
class PrefillPart:
    """Chunked-prefill queries appended after the decode sequences."""

    query: torch.Tensor             # [total_q, H_q, d]
    block_tables: torch.Tensor      # int32 [S_p, max_blocks]
    context_lens: torch.Tensor      # int32 [S_p], prefix + chunk
    cu_q_lens: torch.Tensor         # int32 [S_p + 1]
    max_q_len: int
    q_lens: List[int]
    prefix_lens: List[int]


@dataclass
class DecodeCase:
    name: str
    dtype: torch.dtype
    num_layers: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    scale: float
    layout: PagedLayout             # every sequence: decode ones first, then prefill ones
    num_decode_seqs: int
    block_tables: torch.Tensor      # int32 [S_dec, max_blocks] (device)
    context_lens: torch.Tensor      # int32 [S_dec] (device)
    max_context_len: int
    key_caches: List[torch.Tensor]  # per layer [NB, H_kv, bs, d]
    value_caches: List[torch.Tensor]
    queries: List[torch.Tensor]     # per layer [S_dec, H_q, d]
    slot_mapping: Optional[torch.Tensor] = None       # int64 [T]
    new_keys: List[torch.Tensor] = field(default_factory=list)    # per layer [T, H_kv, d]
    new_values: List[torch.Tensor] = field(default_factory=list)
    prefill: Optional[PrefillPart] = None
    kv_fp8: bool = False            # caches hold E4M3 codes (uint8)
    k_scales: List[torch.Tensor] = field(default_factory=list)   # per layer float32 [H_kv]
    v_scales: List[torch.Tensor] = field(default_factory=list)

    @property
    def num_seqs(self):
        return self.num_decode_seqs


def _fill_randn(t, gen, chunk=1 << 26):
    """Fill ``t`` with N(0,1) drawn in float32 and rounded to t's dtype."""
    flat = t.view(-1)
    for start in range(0, flat.numel(), chunk):
        stop = min(start + chunk, flat.numel())
        draw = torch.randn(stop - start, generator=gen, device=t.device, dtype=F32)
        flat[start:stop].copy_(draw)
    return t


def _randn(shape, dtype, device, gen):
    return _fill_randn(torch.empty(shape, dtype=dtype, device=device), gen)


def _poison_unowned(cache, used_slots):
    """NaN into every slot that no sequence owns."""
    block_size = cache.shape[2]
    used = torch.as_tensor(used_slots, device=cache.device).to(torch.int64)
    slot_idx = torch.arange(block_size, device=cache.device)
    unowned = slot_idx[None, :] >= used[:, None]           # [NB, bs]
    cache.masked_fill_(unowned[:, None, :, None], float("nan"))


# E4M3 code of NaN (S.1111.111), the poison of unowned slots in an FP8 cache.
FP8_NAN_CODE = 0x7F


def _fp8_codes(shape, device, gen):
    """E4M3 codes whose values spread like N(0, 64^2): normal draws scaled by
    64, clipped to the format's +-448 and cast with torch's own E4M3 cast.
    The per-head scales are separate inputs, so the caches dequantize to
    roughly N(0, (64 s)^2)."""
    x = torch.randn(shape, generator=gen, device=device, dtype=F32).mul_(64.0).clamp_(-448.0, 448.0)
    return x.to(torch.float8_e4m3fn).view(torch.uint8)


def _fp8_scales(num_kv_heads, device, gen):
    """Per-head float32 scales drawn around 1/64 (uniform in [0.5, 2] / 64)."""
    u = torch.rand(num_kv_heads, generator=gen, device=device, dtype=F32)
    return (0.5 + 1.5 * u) / 64.0


def _poison_unowned_codes(cache, used_slots):
    block_size = cache.shape[2]
    used = torch.as_tensor(used_slots, device=cache.device).to(torch.int64)
    slot_idx = torch.arange(block_size, device=cache.device)
    unowned = slot_idx[None, :] >= used[:, None]
    cache.masked_fill_(unowned[:, None, :, None], FP8_NAN_CODE)


def make_case(*, name, seed, context_lens, num_q_heads, num_kv_heads, head_dim,
              block_size, dtype=BF16, device="cpu", num_layers=1, pool_slack=0.1,
              exact_pool=False, shared_prefix=None, pool_blocks=None,
              write_new_token=False, prefill_chunks=(), poison=True, gen_device=None,
              structure_only=False, kv_fp8=False):
    """Build a decode (+ optional prefill-chunk) case.

    context_lens: decode sequences' lengths, new token included.
    prefill_chunks: (prefix_len, q_len) per extra sequence; its context is
        prefix_len + q_len and its chunk tokens are written through the slot
        mapping before the chunk is attended.
    write_new_token: each decode sequence's last position is written through
        the slot mapping (the new token), so a step is "write, then attend".
    gen_device: where values are drawn (defaults to ``device``); c1_tiny draws
        on the host and moves the result.
    structure_only: draw lengths, tables and slots but no value tensors.
    kv_fp8: the caches hold E4M3 codes (uint8) with per-layer, per-head
        float32 scales in ``k_scales`` / ``v_scales``; queries and new K/V rows
        keep ``dtype``; unowned slots hold the NaN code.
    """
    rng = np.random.default_rng(seed)
    gen_device = torch.device(gen_device or device)
    device = torch.device(device)
    dec_lens = [int(n) for n in context_lens]
    pre = [(int(p), int(q)) for p, q in prefill_chunks]
    all_lens = dec_lens + [p + q for p, q in pre]
    layout = draw_layout(rng, all_lens, block_size, pool_slack=pool_slack,
                         exact_pool=exact_pool, shared_prefix=shared_prefix,
                         pool_blocks=pool_blocks)
    num_dec = len(dec_lens)

    # Slot mapping: decode new tokens first, then every chunk token.
    slots = []
    if write_new_token:
        for b, n in enumerate(dec_lens):
            if n > 0:
                pos = n - 1
                slots.append(int(layout.block_tables[b, pos // block_size]) * block_size
                             + pos % block_size)
    for i, (p, q) in enumerate(pre):
        b = num_dec + i
        for pos in range(p, p + q):
            slots.append(int(layout.block_tables[b, pos // block_size]) * block_size
                         + pos % block_size)
    num_new = len(slots)

    gen = torch.Generator(device=gen_device)
    gen.manual_seed(int(seed))
    kv_shape = (layout.num_blocks, num_kv_heads, block_size, head_dim)
    key_caches, value_caches, queries, new_keys, new_values = [], [], [], [], []
    k_scales, v_scales = [], []
    for _ in range(0 if structure_only else num_layers):
        if kv_fp8:
            kc = _fp8_codes(kv_shape, gen_device, gen)
            vc = _fp8_codes(kv_shape, gen_device, gen)
            if poison:
                _poison_unowned_codes(kc, layout.used_slots)
                _poison_unowned_codes(vc, layout.used_slots)
            k_scales.append(_fp8_scales(num_kv_heads, gen_device, gen).to(device))
            v_scales.append(_fp8_scales(num_kv_heads, gen_device, gen).to(device))
        else:
            kc = _randn(kv_shape, dtype, gen_device, gen)
            vc = _randn(kv_shape, dtype, gen_device, gen)
            if poison:
                _poison_unowned(kc, layout.used_slots)
                _poison_unowned(vc, layout.used_slots)
        key_caches.append(kc.to(device))
        value_caches.append(vc.to(device))
        queries.append(_randn((num_dec, num_q_heads, head_dim), dtype, gen_device, gen).to(device))
        if num_new:
            new_keys.append(_randn((num_new, num_kv_heads, head_dim), dtype, gen_device, gen).to(device))
            new_values.append(_randn((num_new, num_kv_heads, head_dim), dtype, gen_device, gen).to(device))
    prefill = None
    if pre and not structure_only:
        q_lens = [q for _, q in pre]
        total_q = sum(q_lens)
        cu = np.zeros(len(pre) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(q_lens)
        prefill = PrefillPart(
            query=_randn((total_q, num_q_heads, head_dim), dtype, gen_device, gen).to(device),
            block_tables=torch.as_tensor(layout.block_tables[num_dec:]).to(device),
            context_lens=torch.as_tensor(layout.context_lens[num_dec:]).to(device),
            cu_q_lens=torch.as_tensor(cu).to(device),
            max_q_len=max(q_lens),
            q_lens=q_lens,
            prefix_lens=[p for p, _ in pre],
        )
    return DecodeCase(
        name=name, dtype=dtype, num_layers=num_layers, num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
        scale=1.0 / float(np.sqrt(head_dim)), layout=layout, num_decode_seqs=num_dec,
        block_tables=torch.as_tensor(layout.block_tables[:num_dec]).contiguous().to(device),
        context_lens=torch.as_tensor(layout.context_lens[:num_dec]).contiguous().to(device),
        max_context_len=max(dec_lens) if dec_lens else 0,
        key_caches=key_caches, value_caches=value_caches, queries=queries,
        slot_mapping=(torch.as_tensor(np.asarray(slots, dtype=np.int64)).to(device)
                      if num_new else None),
        new_keys=new_keys, new_values=new_values, prefill=prefill,
        kv_fp8=kv_fp8, k_scales=k_scales, v_scales=v_scales,
    )


# --------------------------------------------------------------------------
# The five named workloads.

def _c1(device, **kw):
    # Table = first 7 entries of a permutation of a 32-block pool.
    case = make_case(name="c1_tiny", seed=1, context_lens=[100], num_q_heads=4,
                     num_kv_heads=1, head_dim=64, block_size=16, dtype=F32,
                     device=device, gen_device="cpu", pool_blocks=32, **kw)
    assert case.layout.num_blocks == 32
    return case


def _c2(device, **kw):
    rng = np.random.default_rng(2)
    lens = rng.integers(512, 8192, size=32, endpoint=True)
    return make_case(name="c2_layer_decode", seed=2, context_lens=lens, num_q_heads=16,
                     num_kv_heads=4, head_dim=256, block_size=16, device=device, **kw)


def _c3(device, num_layers=16, **kw):
    return make_case(name="c3_full_step", seed=3, context_lens=[8192] * 64, num_q_heads=16,
                     num_kv_heads=4, head_dim=256, block_size=32, device=device,
                     num_layers=num_layers, exact_pool=True, write_new_token=True, **kw)


def _c4(device, **kw):
    rng = np.random.default_rng(4)
    tails = rng.integers(0, 1024, size=128, endpoint=True)
    return make_case(name="c4_grpo_cow", seed=4, context_lens=4096 + tails, num_q_heads=16,
                     num_kv_heads=4, head_dim=256, block_size=16, device=device,
                     shared_prefix=(16, 4096), **kw)


def _c5(device, **kw):
    rng = np.random.default_rng(5)
    prompt = np.minimum(rng.geometric(1.0 / 1500.0, size=255), 6000)
    generated = rng.choice(np.array([50, 120, 240, 1024]), size=255)
    return make_case(name="c5_mixed_step", seed=5, context_lens=prompt + generated,
                     num_q_heads=16, num_kv_heads=4, head_dim=256, block_size=16,
                     device=device, write_new_token=True, prefill_chunks=[(3584, 512)], **kw)


CONFIGS = {
    "c1_tiny": _c1,
    "c2_layer_decode": _c2,
    "c3_full_step": _c3,
    "c4_grpo_cow": _c4,
    "c5_mixed_step": _c5,
}


def make_config_case(name, device="cpu", **kw):
    return CONFIGS[name](device, **kw)


def to_numpy_bits(t):
    """Tensor -> numpy on the host; BF16 comes back as its uint16 bit patterns."""
    t = t.detach()
    if t.dtype == BF16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()

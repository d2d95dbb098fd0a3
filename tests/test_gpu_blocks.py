"""GPU parity of the block copy (pa_copy_blocks) and of a copy-on-write
rollout step driven by the native block manager: fork a prompt whose last
block is partial into 8 rollouts, run the copies, write each rollout's new
token, decode. The oracle replays the same step with its own block manager,
scatter, block copy and decode, starting from the same initial pool."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_215_amd as pa
from gpu_helpers import ATOL, max_abs_err, say
from oracle.block_manager import BlockManagerRef, copy_blocks_ref, move_blocks_ref
from workloads import to_numpy_bits

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _pool(nb, hkv, bs, d, dtype, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    if dtype == torch.uint8:
        kc = torch.randint(0, 256, (nb, hkv, bs, d), generator=g, dtype=torch.uint8)
        vc = torch.randint(0, 256, (nb, hkv, bs, d), generator=g, dtype=torch.uint8)
    else:
        kc = torch.randn((nb, hkv, bs, d), generator=g).to(dtype)
        vc = torch.randn((nb, hkv, bs, d), generator=g).to(dtype)
    return kc.to(DEV), vc.to(DEV)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.uint8])
@pytest.mark.parametrize("block_size", [16, 32])
@pytest.mark.parametrize("head_dim", [64, 256])
def test_copy_blocks_bit_exact(dtype, block_size, head_dim):
    nb, hkv = 200, 4
    kc, vc = _pool(nb, hkv, block_size, head_dim, dtype, seed=head_dim + block_size)
    rng = np.random.default_rng(block_size)
    perm = rng.permutation(nb)
    pairs = np.stack([perm[:60], perm[60:120]], axis=1).astype(np.int64)   # independent
    pairs = np.concatenate([pairs, [[5, nb + 3], [-1, 7], [nb, 2]]])       # skipped
    kb, vb = to_numpy_bits(kc), to_numpy_bits(vc)
    valid = [(int(s), int(d)) for s, d in pairs if 0 <= s < nb and 0 <= d < nb]
    want_k, want_v = copy_blocks_ref(kb, vb, valid)
    say(f"[copy] {dtype} bs{block_size} d{head_dim}: {len(valid)} pairs")
    pa.pa_copy_blocks(kc, vc, torch.from_numpy(pairs).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(to_numpy_bits(kc).view(np.uint8), want_k.view(np.uint8))
    assert np.array_equal(to_numpy_bits(vc).view(np.uint8), want_v.view(np.uint8))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32, torch.uint8])
@pytest.mark.parametrize("block_size", [16, 32])
def test_swap_round_trip_every_element_type(dtype, block_size):
    # device -> pinned host pool -> other device blocks, bit for bit; pairs
    # outside either pool are skipped
    nb, nh, hkv, d = 96, 40, 4, 128
    kc, vc = _pool(nb, hkv, block_size, d, dtype, seed=block_size + 1)
    hk = torch.zeros((nh,) + tuple(kc.shape[1:]), dtype=dtype).pin_memory()
    hv = torch.zeros((nh,) + tuple(kc.shape[1:]), dtype=dtype).pin_memory()
    rng = np.random.default_rng(block_size)
    src = rng.permutation(nb)[:30]
    dst = rng.permutation(nh)[:30]
    out_pairs = np.stack([src, dst], axis=1).astype(np.int64)
    out_pairs = np.concatenate([out_pairs, [[nb, 1], [2, nh], [-3, 0]]])
    kb, vb = to_numpy_bits(kc), to_numpy_bits(vc)
    valid_out = [(int(a), int(b)) for a, b in out_pairs if 0 <= a < nb and 0 <= b < nh]
    want_hk, want_hv = move_blocks_ref(kb, vb, to_numpy_bits(hk), to_numpy_bits(hv), valid_out)
    say(f"[swap] {dtype} bs{block_size}: {len(valid_out)} blocks out")
    pa.pa_swap_out(kc, vc, hk, hv, torch.from_numpy(out_pairs).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(to_numpy_bits(hk).view(np.uint8), want_hk.view(np.uint8))
    assert np.array_equal(to_numpy_bits(hv).view(np.uint8), want_hv.view(np.uint8))
    back = rng.permutation(nb)[:30]
    in_pairs = np.stack([dst, back], axis=1).astype(np.int64)
    in_pairs = np.concatenate([in_pairs, [[nh, 0], [0, nb]]])
    valid_in = [(int(a), int(b)) for a, b in in_pairs if 0 <= a < nh and 0 <= b < nb]
    want_k, want_v = move_blocks_ref(want_hk, want_hv, kb, vb, valid_in)
    pa.pa_swap_in(kc, vc, hk, hv, torch.from_numpy(in_pairs).pin_memory())
    torch.cuda.synchronize()
    assert np.array_equal(to_numpy_bits(kc).view(np.uint8), want_k.view(np.uint8))
    assert np.array_equal(to_numpy_bits(vc).view(np.uint8), want_v.view(np.uint8))


def test_copy_blocks_many_pairs_several_launches():
    # more pairs than one launch's grid.y holds
    nb, hkv, bs, d = 140_000, 1, 16, 64
    kc = torch.zeros((nb, hkv, bs, d), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    ids = torch.arange(nb, device=DEV, dtype=torch.float32)
    kc.copy_(ids[:, None, None, None].expand_as(kc))
    vc.copy_((-ids)[:, None, None, None].expand_as(vc))
    src = torch.arange(0, 70_000, device=DEV, dtype=torch.int64)
    pairs = torch.stack([src, src + 70_000], dim=1).contiguous()
    pa.pa_copy_blocks(kc, vc, pairs)
    torch.cuda.synchronize()
    assert torch.equal(kc[70_000:], kc[:70_000]) and torch.equal(vc[70_000:], vc[:70_000])


def test_rollout_step_copy_on_write():
    hq, hkv, d, bs = 16, 4, 256, 16
    prompt, rollouts, steps = 4100, 8, 3
    nb, cap = 400, 300
    scale = 1.0 / np.sqrt(d)
    kc, vc = _pool(nb, hkv, bs, d, torch.bfloat16, seed=3)
    k0, v0 = to_numpy_bits(kc), to_numpy_bits(vc)        # the oracle's starting pool
    g = torch.Generator(device=DEV)
    g.manual_seed(11)
    pk = torch.randn((prompt, hkv, d), generator=g, device=DEV).to(torch.bfloat16)
    pv = torch.randn((prompt, hkv, d), generator=g, device=DEV).to(torch.bfloat16)

    bm = pa.BlockManager(nb, bs, cap)
    ref = BlockManagerRef(nb, bs, cap)
    ok, oc = bm.add(0), ref.add(0)
    st, slots = bm.append(0, prompt)
    _, rslots = ref.append(0, prompt)
    assert st == 0 and slots.tolist() == rslots
    pa.pa_reshape_and_cache(pk, pv, kc, vc, torch.from_numpy(slots).to(DEV))
    ok_, ov_ = oracle.reshape_and_cache_ref(to_numpy_bits(pk), to_numpy_bits(pv), k0, v0, rslots)
    for r in range(1, rollouts + 1):
        assert bm.fork(0, r) == 0 and ref.fork(0, r) == "ok"
    bm.free(0)
    ref.free(0)
    seqs = list(range(1, rollouts + 1))
    copies_seen = 0
    for step in range(steps):
        new_slots, ref_slots = [], []
        for r in seqs:
            st, s = bm.append(r, 1)
            rst, rs = ref.append(r, 1)
            assert st == 0 and s.tolist() == rs
            new_slots.extend(s.tolist())
            ref_slots.extend(rs)
        # copies first (run by run), then the new tokens
        ref_pairs = ref.take_copies()
        got_pairs = []
        while True:
            run = bm.take_copies()
            if len(run) == 0:
                break
            got_pairs.extend(map(tuple, run.tolist()))
            pa.pa_copy_blocks(kc, vc, torch.from_numpy(run).to(DEV))
        assert got_pairs == ref_pairs
        copies_seen += len(got_pairs)
        ok_, ov_ = copy_blocks_ref(ok_, ov_, ref_pairs)
        nk = torch.randn((rollouts, hkv, d), generator=g, device=DEV).to(torch.bfloat16)
        nv = torch.randn((rollouts, hkv, d), generator=g, device=DEV).to(torch.bfloat16)
        pa.pa_reshape_and_cache(nk, nv, kc, vc, torch.tensor(new_slots, device=DEV))
        ok_, ov_ = oracle.reshape_and_cache_ref(to_numpy_bits(nk), to_numpy_bits(nv), ok_, ov_,
                                                ref_slots)
        tables, lens = bm.tables(seqs)
        q = torch.randn((rollouts, hq, d), generator=g, device=DEV).to(torch.bfloat16)
        out = pa.pa_decode(q, kc, vc, torch.from_numpy(tables).to(DEV),
                           torch.from_numpy(lens).to(DEV), scale, int(lens.max()))
        torch.cuda.synchronize()
        rt = np.array([ref.table(r) + [-1] * (cap - len(ref.table(r))) for r in seqs],
                      dtype=np.int32)
        want = oracle.decode_ref(to_numpy_bits(q), ok_, ov_, rt,
                                 np.array([ref.length(r) for r in seqs]), scale)
        err = max_abs_err(out.cpu().numpy(), want)
        say(f"[rollout cow] step {step}: {len(got_pairs)} copies, max-abs err {err:.3e}")
        assert err <= ATOL
        # the cache the device holds equals the oracle's, byte for byte
        assert np.array_equal(to_numpy_bits(kc), ok_) and np.array_equal(to_numpy_bits(vc), ov_)
    assert copies_seen == rollouts - 1     # only the shared partial prompt block is copied
    bm.close()

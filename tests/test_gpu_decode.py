"""GPU parity of pa_decode (through the C ABI) against the fp64 CPU oracle:
max-abs error <= 1e-3 on float32 outputs, plus bit-level invariants."""

import math

import numpy as np
import pytest
import torch

import paged_kv_cache_215_amd as pa
from gpu_helpers import (ATOL, gpu_decode, max_abs_err, oracle_decode, oracle_decode_after_write,
                         say)
from workloads import make_case, make_config_case

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _check(case, layer=0, seqs=None, tag=""):
    say(f"[decode] {case.name} layer={layer} {tag}")
    out = gpu_decode(case, layer)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    if seqs is not None:
        got = got[list(seqs)]
    want = oracle_decode(case, layer, seqs)
    assert np.all(np.isfinite(got)), "non-finite output"
    err = max_abs_err(got, want)
    say(f"    max-abs err {err:.3e}")
    assert err <= ATOL, f"{case.name}: max-abs error {err}"
    return out


def test_c1_tiny_fp32():
    case = make_config_case("c1_tiny", device=DEV)
    _check(case)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("head_dim", [64, 128, 256])
@pytest.mark.parametrize("group", [1, 2, 4, 8])
@pytest.mark.parametrize("block_size", [16, 32])
def test_shapes_ragged(dtype, head_dim, group, block_size):
    # lengths around tile (16), block and partition (>= 64 tokens) edges
    lens = [1, 15, 16, 17, block_size - 1, block_size + 1, 63, 64, 65, 200, 1000, 2500]
    case = make_case(name=f"ragged_d{head_dim}_g{group}_bs{block_size}", seed=head_dim + group,
                     context_lens=lens, num_q_heads=2 * group, num_kv_heads=2,
                     head_dim=head_dim, block_size=block_size, dtype=dtype, device=DEV)
    _check(case, tag=str(dtype))


def test_zero_and_single_token_contexts():
    lens = [0, 1, 0, 5, 0]
    case = make_case(name="zeros", seed=7, context_lens=lens, num_q_heads=16, num_kv_heads=4,
                     head_dim=256, block_size=16, device=DEV)
    out = _check(case)
    o = out.cpu().numpy()
    assert np.all(o[0] == 0) and np.all(o[2] == 0) and np.all(o[4] == 0)
    # n = 1: the output is that token's value row exactly (weights are 1)
    v0 = case.value_caches[0][int(case.layout.block_tables[1, 0]), :, 0, :].float().cpu().numpy()
    for h in range(16):
        np.testing.assert_array_equal(o[1, h], v0[h // 4])


def test_c2_layer_decode_full():
    _check(make_config_case("c2_layer_decode", device=DEV))


def test_c4_grpo_cow_full():
    _check(make_config_case("c4_grpo_cow", device=DEV))


def test_c5_mixed_decode_part_full():
    case = make_config_case("c5_mixed_step", device=DEV)
    # write, then attend: the new tokens go in first; the oracle applies its
    # own write to a copy of the caches taken before the device's
    kb, vb = case.key_caches[0].clone(), case.value_caches[0].clone()
    pa.pa_reshape_and_cache(case.new_keys[0], case.new_values[0], case.key_caches[0],
                            case.value_caches[0], case.slot_mapping)
    say(f"[decode] {case.name} (write, then attend)")
    got = gpu_decode(case).cpu().numpy()
    want = oracle_decode_after_write(case, kb, vb)
    err = max_abs_err(got, want)
    say(f"    max-abs err {err:.3e}")
    assert np.all(np.isfinite(got)) and err <= ATOL


def test_c3_full_step_full_layers():
    # The full 16-layer, 64 x 8192-token step in the launch configuration the
    # benchmark times. Every sequence of layers 0, 5, 10 and 15 is checked
    # against the oracle (in chunks of 16 sequences, to bound host memory).
    case = make_config_case("c3_full_step", device=DEV)
    layers = [0, 5, 10, 15]
    # copies of the checked layers before the device writes the new tokens
    before = {layer: (case.key_caches[layer].clone(), case.value_caches[layer].clone())
              for layer in layers}
    outs = []
    for layer in range(case.num_layers):
        pa.pa_reshape_and_cache(case.new_keys[layer], case.new_values[layer],
                                case.key_caches[layer], case.value_caches[layer],
                                case.slot_mapping)
        outs.append(gpu_decode(case, layer))
    torch.cuda.synchronize()
    S = case.num_decode_seqs
    for layer in layers:
        got_all = outs[layer].cpu().numpy()
        assert np.all(np.isfinite(got_all))
        worst = 0.0
        for s0 in range(0, S, 16):
            seqs = list(range(s0, min(S, s0 + 16)))
            want = oracle_decode_after_write(case, *before[layer], layer=layer, seqs=seqs)
            worst = max(worst, max_abs_err(got_all[seqs], want))
        say(f"[decode] c3 layer {layer}, all {S} sequences: max-abs err {worst:.3e}")
        assert worst <= ATOL
        del before[layer]


def test_block_permutation_bit_identical():
    lens = [300, 77, 1024, 16]
    case = make_case(name="perm", seed=11, context_lens=lens, num_q_heads=16, num_kv_heads=4,
                     head_dim=256, block_size=16, device=DEV)
    base = gpu_decode(case)
    nb = case.layout.num_blocks
    perm = torch.as_tensor(np.random.default_rng(3).permutation(nb), device=DEV)
    kc2 = torch.empty_like(case.key_caches[0])
    vc2 = torch.empty_like(case.value_caches[0])
    kc2[perm] = case.key_caches[0]
    vc2[perm] = case.value_caches[0]
    bt = case.block_tables.long()
    bt2 = torch.where(bt >= 0, perm[bt.clamp(min=0)], bt).to(torch.int32).contiguous()
    moved = pa.pa_decode(case.queries[0], kc2, vc2, bt2, case.context_lens, case.scale,
                         case.max_context_len)
    torch.cuda.synchronize()
    assert torch.equal(base, moved)


def test_run_to_run_bit_identical():
    case = make_config_case("c2_layer_decode", device=DEV)
    a = gpu_decode(case)
    b = gpu_decode(case)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_copy_on_write_shared_vs_private_bit_identical():
    # Two rollouts sharing a 512-token prompt's blocks vs. holding private
    # copies of those blocks: identical outputs.
    case = make_case(name="cow", seed=12, context_lens=[512 + 40, 512 + 300], num_q_heads=16,
                     num_kv_heads=4, head_dim=256, block_size=16, device=DEV,
                     shared_prefix=(2, 512), pool_slack=1.0)
    shared = gpu_decode(case)
    bt = case.block_tables.clone()
    kc = case.key_caches[0].clone()
    vc = case.value_caches[0].clone()
    # give sequence 1 private copies of the 32 prompt blocks
    free = [i for i in range(case.layout.num_blocks)
            if case.layout.used_slots[i] == 0][:32]
    assert len(free) == 32, "pool slack too small for the private copies"
    src = bt[1, :32].long()
    dst = torch.as_tensor(free, device=DEV)
    kc[dst] = kc[src]
    vc[dst] = vc[src]
    bt[1, :32] = dst.to(torch.int32)
    private = pa.pa_decode(case.queries[0], kc, vc, bt, case.context_lens, case.scale,
                           case.max_context_len)
    torch.cuda.synchronize()
    assert torch.equal(shared, private)


def test_out_of_range_table_entry_never_faults():
    # An invalid table entry must not be dereferenced; the other rows stay exact.
    lens = [100, 100]
    case = make_case(name="badentry", seed=13, context_lens=lens, num_q_heads=4, num_kv_heads=1,
                     head_dim=64, block_size=16, device=DEV)
    bt = case.block_tables.clone()
    bt[0, 2] = 10 ** 8
    out = pa.pa_decode(case.queries[0], case.key_caches[0], case.value_caches[0], bt,
                       case.context_lens, case.scale, case.max_context_len)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = oracle_decode(case, 0, [1])
    assert max_abs_err(got[1:2], want) <= ATOL


def test_workspace_size_matches_partition_geometry():
    # every launch shape in this file fits the advertised workspace
    need = pa.pa_decode_workspace_size(64, 16, 4, 256, 32, 8192)
    assert need > 0 and need % 16 == 0


def test_workspace_reused_across_batches():
    # One zero-filled workspace, sized for the largest call, serves a ragged
    # batch, a uniform batch and a ragged batch again in stream order (the
    # work-queue counter is left at zero by every call).
    cases = [
        make_case(name="reuse_a", seed=21, context_lens=[700, 33, 5000, 1], num_q_heads=16,
                  num_kv_heads=4, head_dim=256, block_size=16, device=DEV),
        make_case(name="reuse_b", seed=22, context_lens=[4096] * 8, num_q_heads=16,
                  num_kv_heads=4, head_dim=256, block_size=16, device=DEV),
        make_case(name="reuse_c", seed=23, context_lens=[64, 8000, 300], num_q_heads=16,
                  num_kv_heads=4, head_dim=256, block_size=16, device=DEV),
    ]
    ws = pa.decode_workspace(8, 16, 4, 256, 16, 8192, torch.device(DEV))
    for case in cases:
        out = pa.pa_decode(case.queries[0], case.key_caches[0], case.value_caches[0],
                           case.block_tables, case.context_lens, case.scale, 8192, workspace=ws)
        torch.cuda.synchronize()
        err = max_abs_err(out.cpu().numpy(), oracle_decode(case))
        say(f"[decode] {case.name} with a shared workspace: max-abs err {err:.3e}")
        assert err <= ATOL


def test_large_batch_spans_several_launches():
    # more than 4096 sequences: the library splits the batch into launches
    lens = np.random.default_rng(24).integers(1, 80, size=4500)
    case = make_case(name="big_batch", seed=24, context_lens=lens, num_q_heads=2,
                     num_kv_heads=1, head_dim=64, block_size=16, device=DEV)
    out = gpu_decode(case)
    torch.cuda.synchronize()
    seqs = [0, 1, 4095, 4096, 4097, 4499]
    err = max_abs_err(out.cpu().numpy()[seqs], oracle_decode(case, 0, seqs))
    say(f"[decode] 4500 sequences: sampled max-abs err {err:.3e}")
    assert err <= ATOL


@pytest.mark.parametrize("group", [4, 8])
def test_ragged_batch_every_sequence(group):
    # 1500 ragged sequences (empty ones included): each wave of the plan ranks
    # several 64-sequence chunks when it orders the last partitions, longest
    # first, for the ticket counter; every output row is checked, so a unit
    # handed out twice or never shows up
    lens = np.random.default_rng(25).integers(0, 700, size=1500)
    case = make_case(name=f"ragged_1500_g{group}", seed=25 + group, context_lens=lens,
                     num_q_heads=2 * group, num_kv_heads=2, head_dim=64, block_size=16, device=DEV)
    _check(case)


@pytest.mark.parametrize("kv_fp8", [False, True])
def test_very_long_contexts(kv_fp8):
    # contexts far past one partition's staged block table (up to 128K
    # tokens) next to short ones; every sequence against the oracle
    lens = [131072, 100003, 1, 65553]
    case = make_case(name="long_ctx", seed=31, context_lens=lens, num_q_heads=16, num_kv_heads=4,
                     head_dim=256, block_size=32, device=DEV, kv_fp8=kv_fp8)
    if kv_fp8:
        out = pa.pa_decode_fp8(case.queries[0], case.key_caches[0], case.value_caches[0],
                               case.k_scales[0], case.v_scales[0], case.block_tables,
                               case.context_lens, case.scale, case.max_context_len)
    else:
        out = gpu_decode(case)
    torch.cuda.synchronize()
    err = max_abs_err(out.cpu().numpy(), oracle_decode(case))
    say(f"[decode] contexts {lens} (fp8={kv_fp8}): max-abs err {err:.3e}")
    assert np.all(np.isfinite(out.cpu().numpy())) and err <= ATOL


@pytest.mark.parametrize("seed", range(6))
def test_ragged_partition_sizes_sweep(seed):
    # Ragged batches whose per-CU share of the tokens lands on many different
    # multiples of 128 (the plan's partition size for ragged lengths), with
    # sequences shorter than, equal to and several times that size, at both
    # block sizes and several head shapes: every sequence against the oracle.
    rng = np.random.default_rng(1000 + seed)
    num_seqs = int(rng.choice([12, 24, 40, 64]))
    group = int(rng.choice([1, 2, 4, 8]))
    num_kv = int(rng.choice([2, 4]))
    head_dim = int(rng.choice([64, 128]))
    block_size = int(rng.choice([16, 32]))
    lens = rng.integers(1, 9000, size=num_seqs)
    lens[: num_seqs // 4] = rng.integers(1, 300, size=num_seqs // 4)  # short ones too
    case = make_case(name=f"plan_sweep_{seed}", seed=seed, context_lens=lens,
                     num_q_heads=group * num_kv, num_kv_heads=num_kv, head_dim=head_dim,
                     block_size=block_size, device=DEV)
    share = int(lens.sum()) * num_kv / 256
    _check(case, tag=f"S={num_seqs} G={group} Hkv={num_kv} d={head_dim} bs={block_size} "
                     f"share~{share:.0f} tokens/CU")

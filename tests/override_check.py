"""Parity of the library under the launch-shape overrides read from the
environment (heads per wave, waves per workgroup, context splits, XCD
remapping for prefill; waves per workgroup and units per CU for decode).
The overrides are read once per process, so test_gpu_overrides.py runs this
script in a child process per setting. Prints one line per case and exits 1
on the first case above the tolerance."""

import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(HERE))

import numpy as np  # noqa: E402
import torch  # noqa: E402

import oracle  # noqa: E402
import paged_kv_cache_215_amd as pa  # noqa: E402
from gpu_helpers import ATOL, gpu_decode, gpu_prefill, max_abs_err, oracle_decode  # noqa: E402
from workloads import make_case, to_numpy_bits  # noqa: E402

DEV = "cuda"


def prefill_case(head_dim, group, prefix, rows, seed):
    case = make_case(name=f"ov_pf_d{head_dim}_g{group}_{prefix}_{rows}", seed=seed,
                     context_lens=[], num_q_heads=2 * group, num_kv_heads=2, head_dim=head_dim,
                     block_size=16, device=DEV, prefill_chunks=[(prefix, rows)])
    key_before = case.key_caches[0].clone()
    value_before = case.value_caches[0].clone()
    pa.pa_reshape_and_cache(case.new_keys[0], case.new_values[0], case.key_caches[0],
                            case.value_caches[0], case.slot_mapping)
    out = gpu_prefill(case)
    torch.cuda.synchronize()
    p = case.prefill
    lay = case.layout
    kc, vc = oracle.reshape_and_cache_ref(
        to_numpy_bits(case.new_keys[0]), to_numpy_bits(case.new_values[0]),
        to_numpy_bits(key_before), to_numpy_bits(value_before), case.slot_mapping.cpu().numpy())
    want = oracle.prefill_chunk_ref(to_numpy_bits(p.query), kc, vc, lay.block_tables,
                                    lay.context_lens, p.cu_q_lens.cpu().numpy(), case.scale)
    return case.name, max_abs_err(out.cpu().numpy(), want)


def decode_case(head_dim, group, lens, seed):
    case = make_case(name=f"ov_dec_d{head_dim}_g{group}", seed=seed, context_lens=lens,
                     num_q_heads=4 * group, num_kv_heads=4, head_dim=head_dim, block_size=16,
                     device=DEV)
    out = gpu_decode(case)
    torch.cuda.synchronize()
    return case.name, max_abs_err(out.cpu().numpy(), oracle_decode(case))


def main():
    setting = " ".join(f"{k}={v}" for k, v in sorted(os.environ.items()) if k.startswith("PA_"))
    print(f"[overrides] {setting or '(none)'}", flush=True)
    cases = []
    for d in (64, 128, 256):
        for g in (1, 2, 4, 8):
            cases.append(lambda d=d, g=g: prefill_case(d, g, 45, 37, d + g))
    cases.append(lambda: prefill_case(256, 4, 700, 130, 5))
    for d in (128, 256):
        for g in (4, 8):
            cases.append(lambda d=d, g=g: decode_case(d, g, [1, 17, 300, 1030, 2049, 4100],
                                                      d * g))
    # equal lengths, one unit per CU: the plan's equal-length branch
    cases.append(lambda: decode_case(256, 4, [1024] * 64, 11))
    worst = 0.0
    for run in cases:
        name, err = run()
        print(f"    {name}: max-abs err {err:.3e}", flush=True)
        worst = max(worst, err)
        if not np.isfinite(err) or err > ATOL:
            print(f"[overrides] FAILED {name}", flush=True)
            return 1
    print(f"[overrides] ok, worst {worst:.3e}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())

"""Host-side parts of bench.py (CPU): the algorithmic-byte accounting that the
roofline divides by, the one-GPU guard, and the source hash that ties the
committed HBM counters to the kernel they were taken on."""

import json
import os
import subprocess
import sys

import numpy as np

import bench
from workloads import make_config_case

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c3_algorithmic_bytes_closed_form():
    # 64 sequences x 8192 tokens, 4 KV heads of d 256 in BF16 (K and V), the
    # BF16 query and float32 output of 16 heads, one int32 table entry per
    # block of 32 tokens
    c = make_config_case("c3_full_step", structure_only=True)
    got = bench.decode_bytes(c.layout, 64, 16, 4, 256, 2)
    kv = 2 * 64 * 8192 * 4 * 256 * 2
    q, out, table = 64 * 16 * 256 * 2, 64 * 16 * 256 * 4, 64 * (8192 // 32) * 4
    assert got == kv + q + out + table == 2_149_122_048


def test_fp8_bytes_count_one_byte_per_element_and_the_scales():
    c = make_config_case("c3_full_step", structure_only=True)
    bf16 = bench.decode_bytes(c.layout, 64, 16, 4, 256, 2)
    fp8 = bench.decode_bytes(c.layout, 64, 16, 4, 256, 2, kv_bytes=1)
    kv_bf16 = 2 * 64 * 8192 * 4 * 256 * 2
    assert fp8 == bf16 - kv_bf16 // 2 + 2 * 4 * 4


def test_shared_prompt_blocks_count_once():
    # 8 prompts of 4096 tokens, each shared by 16 rollouts whose private tails
    # have their own blocks: unique K/V rows = 8 * 4096 + sum of the tails
    c = make_config_case("c4_grpo_cow", structure_only=True)
    lens = c.layout.context_lens.astype(np.int64)
    per_token = 2 * 4 * 256 * 2
    fixed = bench.decode_bytes(c.layout, 128, 16, 4, 256, 2) - int(lens.sum()) * per_token
    unique = bench.decode_bytes(c.layout, 128, 16, 4, 256, 2, unique_blocks=True)
    assert unique - fixed == (8 * 4096 + int((lens - 4096).sum())) * per_token
    assert unique < bench.decode_bytes(c.layout, 128, 16, 4, 256, 2)


def test_more_than_one_gpu_is_refused():
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                          capture_output=True, text=True, timeout=120)
    assert proc.returncode == 2
    assert "one GPU" in proc.stderr
    assert proc.stdout == ""


def test_source_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    src = tmp_path / "k.hip"
    src.write_text("int f(int x) { return x + 1; }  // add one\n")
    h0 = bench.source_hash(["k.hip"])
    src.write_text("/* a block\n comment */\nint f(int x) {\n  return x + 1;  // one more\n}\n")
    assert bench.source_hash(["k.hip"]) == h0
    src.write_text("int f(int x) { return x + 2; }\n")
    assert bench.source_hash(["k.hip"]) != h0


def test_kernel_names_match_the_committed_kernel_traces():
    # the kernel bench.py names in its roofline entry is the one the committed
    # rocprofv3 summaries of the same workloads list first
    for fp8, trace in ((False, "decode_c3_kernel_trace.md"), (True, "decode_fp8_c3_kernel_trace.md")):
        name = bench.decode_kernel_name(fp8, 16 // 4, 256)
        text = open(os.path.join(ROOT, "profiles", trace)).read()
        first = [ln for ln in text.splitlines() if ln.startswith("| `pa::")][0]
        assert f"pa::{name}<" in first, (trace, first)


def test_prefill_counter_summary(tmp_path):
    # matrix-unit busy = busy cycles / (SIMDs x kernel cycles), with the kernel
    # length taken as one XCD's share of GRBM_GUI_ACTIVE
    pmc = tmp_path / "pmc_prefill_c5" / "run"
    pmc.mkdir(parents=True)
    name = "void pa::prefill_kernel<256, 4, 1, 8, 64>(pa::PrefillArgs)"
    cycles = 100000
    busy = bench.SIMDS * cycles // 4                        # a quarter of the SIMD cycles
    values = {"SQ_INSTS_MFMA": busy // 16, "SQ_VALU_MFMA_BUSY_CYCLES": busy,
              "SQ_WAVE_CYCLES": 1000, "SQ_WAIT_ANY": 300, "SQ_ACTIVE_INST_VALU": 200,
              "GRBM_GUI_ACTIVE": cycles * bench.XCDS}
    rows = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value"]
    for d in (1, 2):                                          # two dispatches, same values
        rows += [f'{d},"{name}",{c},{v}' for c, v in values.items()]
        rows.append(f'{d},"void pa::decode_merge_kernel<256>(pa::DecodeArgs)",SQ_INSTS_MFMA,7')
    (pmc / "p_counter_collection.csv").write_text("\n".join(rows) + "\n")
    out = tmp_path / "profiles"
    out.mkdir()
    bench._summarize_prefill_counters(str(tmp_path / "pmc_prefill_c5"), str(tmp_path / "kt_none"),
                                      str(out))
    text = (out / "prefill_c5_counters.md").read_text()
    assert "Matrix-unit busy: 25.0 %" in text
    assert "16.0 busy cycles per matrix instruction" in text
    assert "Waves waiting: 30.0 %" in text and "VALU issue: 20.0 %" in text
    assert f"Kernel length: {cycles:,} cycles" in text


def test_committed_counter_summaries_are_consistent():
    # every HBM counter summary under profiles/ was taken with a command the
    # bench still defines, on the workload whose algorithmic bytes the bench
    # computes today, and reads no more than a quarter above them
    for key, stem in bench.COUNTER_SETS.items():
        with open(os.path.join(ROOT, "profiles", stem + ".json")) as f:
            c = json.load(f)
        assert c["algorithmic_bytes_per_call"] == bench._algorithmic_decode_bytes(*key), stem
        for tag, cmd in c["commands"].items():
            assert bench.PROFILE_COMMANDS[tag] == cmd, (stem, tag)
        ratio = c["hbm_bytes_per_call"] / c["algorithmic_bytes_per_call"]
        assert 0.95 <= ratio <= 1.25, (stem, ratio)

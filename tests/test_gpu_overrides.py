"""GPU parity under each launch-shape override (environment settings read once
per process, so each setting runs tests/override_check.py in a child process
of its own, one at a time)."""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))

SETTINGS = [
    {"PA_PREFILL_HPW": "2"},
    {"PA_PREFILL_HPW": "4"},
    {"PA_PREFILL_WAVES": "4", "PA_PREFILL_HPW": "2"},
    {"PA_PREFILL_WAVES": "8"},
    {"PA_PREFILL_KEYTILE": "32"},
    {"PA_PREFILL_WAVES": "8", "PA_PREFILL_HPW": "2", "PA_PREFILL_KEYTILE": "64"},
    {"PA_PREFILL_TARGET_WGS": "64", "PA_PREFILL_XCD": "0"},
    {"PA_PREFILL_TARGET_WGS": "4096"},
    {"PA_DECODE_WAVES": "4"},
    {"PA_DECODE_UNITS_PER_CU": "1"},
    {"PA_DECODE_UNITS_PER_CU": "8"},
]


@pytest.mark.parametrize("setting", SETTINGS, ids=lambda s: ",".join(f"{k}={v}" for k, v in s.items()))
def test_override(setting):
    env = {k: v for k, v in os.environ.items() if not k.startswith("PA_")}
    env.update(setting)
    proc = subprocess.run([sys.executable, os.path.join(HERE, "override_check.py")], env=env,
                          capture_output=True, text=True, timeout=240)
    print(proc.stdout, flush=True)
    assert proc.returncode == 0, proc.stdout[-2000:] + proc.stderr[-2000:]

"""The debug build with device-side metadata checks (libpa_kv_checked.so, PA_DEVICE_CHECKS=1).

Its cases run in a process of their own that loads that library (tests/device_checks_cases.py):
clean calls over every kernel path leave no flag and match the oracle; a block id past
num_blocks, a row length past max_seq_len, a prefill row with more queries than tokens and an
append slot past the pool each set their flag.  Every bad case stays inside the buffers even
for a kernel without the check, so no case can fault the GPU.
"""
import json
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CHECKED = os.path.join(os.path.dirname(HERE), "paged_kv_attention_13_amd", "libpa_kv_checked.so")


@pytest.mark.gpu
def test_checked_build_flags_bad_metadata():
    print("\n[case] device checks: clean paths, bad block id / length / query count / slot", flush=True)
    assert os.path.exists(CHECKED), "build it: python -m paged_kv_attention_13_amd.build --checked"
    env = dict(os.environ, PA_LIB_PATH=CHECKED)
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "device_checks_cases.py")], env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    res = json.loads([ln for ln in r.stdout.splitlines() if ln.startswith("{")][-1])
    assert res["checks"] == 1 and res["lib"] == "libpa_kv_checked.so"
    assert res["clean_flags"] == 0, res
    for path, e in res["clean_err"].items():
        assert e < 3e-2, (path, e)
    assert res["block_id"] == 1, res          # PA_CHECK_BLOCK_ID
    assert res["seq_len"] == 2, res           # PA_CHECK_SEQ_LEN
    assert res["q_len"] == 4, res             # PA_CHECK_Q_LEN
    assert res["slot"] == 8, res              # PA_CHECK_SLOT

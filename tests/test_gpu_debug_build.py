"""The parity suites again (the full-size workloads included), against libkvq_debug.so:
the same kernels compiled with KVQ_DEBUG, where every block index, CSR row range, outlier
entry, append slot and split range a kernel derives is checked on the device (a failed
check sets a flag word; nothing traps), and every entry point waits for its launches and
returns KVQ_ERR_HIP if a check failed.  The suites run in a child process that loads the debug library through
KVQ_LIBRARY; the graph tests are left out because a debug entry point synchronises the
device, which graph capture forbids."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEBUG_LIB = os.path.join(ROOT, "decode_attention_10_amd", "libkvq_debug.so")
SUITES = ["tests/test_gpu_uniform.py", "tests/test_gpu_nuq.py", "tests/test_gpu_workloads.py",
          "tests/test_zz_no_alloc.py"]


@pytest.mark.gpu
def test_parity_suites_pass_with_device_bounds_checks():
    if not os.path.exists(DEBUG_LIB):
        pytest.fail(f"{DEBUG_LIB} is missing: build it with `python decode_attention_10_amd/build.py`")
    env = dict(os.environ, KVQ_LIBRARY=DEBUG_LIB)
    check = ("import sys, pytest, decode_attention_10_amd as K; "
             f"assert K.LIB_PATH == {DEBUG_LIB!r}, K.LIB_PATH; "
             f"rc = pytest.main(['-x', '-q', '-m', 'gpu', '-p', 'no:cacheprovider', *{SUITES!r}]); "
             "maps = open('/proc/self/maps').read(); "
             "assert 'libkvq_debug.so' in maps and '/libkvq.so' not in maps; "
             "sys.exit(int(rc))")
    r = subprocess.run([sys.executable, "-u", "-c", check], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=1500)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-3000:]
    assert " passed" in r.stdout and "failed" not in r.stdout, r.stdout[-2000:]

"""The C ABI's host-side validation built with AddressSanitizer and UndefinedBehavior-
Sanitizer (host code only; no GPU): a C++ driver makes the bad calls of test_abi.py and
more, and each must return its error status with a message, with no sanitizer report.
The sanitizers instrument the host code only (each -fsanitize= follows -Xarch_host), and
no call reaches the GPU, so this runs on a machine without one."""
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

WANT = {
    "layout_bits3": 2, "layout_cap100": 1, "layout_cap_over": 1, "layout_batch0": 1,
    "layout_resid100": 1, "layout_sink": 1, "layout_null": 1, "layout_csr_over": 1,
    "qk_null": 1, "qk_align": 4, "qk_off16": 1, "qk_cap": 3, "qk_stride": 1, "qv_n48": 1,
    "append_full": 3, "append_resid": 1,
    "dec_hq4": 1, "dec_hq15": 2, "dec_rope": 2, "dec_scale": 1, "dec_qalign": 4, "dec_out": 1,
    "noalloc_hq4": 1, "noalloc_theta": 1, "nuq_csr_int32": 3,
}


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc is not installed")
def test_host_validation_under_asan_and_ubsan(tmp_path):
    csrc = os.path.join(ROOT, "decode_attention_10_amd", "csrc")
    srcs = sorted(glob.glob(os.path.join(csrc, "*.hip")))
    flags = ["--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all",
             "-I", os.path.join(ROOT, "include"), "-I", csrc, "-Wno-unused-command-line-argument"]
    from concurrent.futures import ThreadPoolExecutor

    def compile_one(s):
        o = str(tmp_path / (os.path.basename(s) + ".o"))
        lang = ["-x", "hip"] if s.endswith(".hip") else ["-x", "c++"]
        r = subprocess.run([HIPCC, *flags, *lang, "-c", s, "-o", o], capture_output=True,
                           text=True, timeout=600)
        assert r.returncode == 0, r.stderr[-3000:]
        return o

    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(compile_one,
                           srcs + [os.path.join(ROOT, "tests", "sanitize", "abi_checks.cpp")]))
    exe = str(tmp_path / "abi_checks")
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address",
                        "-Xarch_host", "-fsanitize=undefined", *objs, "-o", exe],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-3000:]
    syms = subprocess.run(["nm", exe], capture_output=True, text=True).stdout
    assert "__asan_init" in syms and "__ubsan_handle" in syms     # both runtimes linked in
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=99",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=98",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "Sanitizer" not in r.stderr, r.stderr[-4000:]
    got = {}
    for line in r.stdout.splitlines():
        name, val = line.split(" ", 1)
        got.setdefault(name, []).append(val)
    for name, status in WANT.items():
        assert got.get(name, [None])[0] == str(status), (name, got.get(name))
        assert "no-message" not in got.get(name, []), name
    assert got["append_state"] == ["128 128"]                   # an error changed nothing
    assert got["csr_needed"] == [str(128 * ((((1 << 28) * 700) + 9999) // 10000))]
    assert got["ws_bad"] == ["0"]

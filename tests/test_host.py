"""Host-side checks: the product path stays apart from the oracle, the binding fails loudly
without its library, and the bench's byte accounting matches the workloads' shapes."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "decode_attention_10_amd")


def test_product_sources_never_import_the_oracle():
    import re
    pat = re.compile(r"^\s*(import\s+oracle|from\s+oracle|#\s*include\s*[<\"][^>\"]*oracle)",
                     re.M)
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert not pat.search(text), f"{f} imports or includes the oracle"


def test_importing_the_binding_loads_no_oracle():
    code = ("import sys; sys.path.insert(0, %r); import decode_attention_10_amd; "
            "print(any(m == 'oracle' or m.startswith('oracle.') for m in sys.modules))" % ROOT)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "False"


def test_binding_without_library_raises(tmp_path):
    pkg = tmp_path / "decode_attention_10_amd"
    pkg.mkdir()
    (pkg / "__init__.py").write_text(open(os.path.join(PKG, "__init__.py")).read())
    code = ("import sys; sys.path.insert(0, %r)\n"
            "try:\n    import decode_attention_10_amd\nexcept ImportError as e:\n"
            "    print('raised', 'missing' in str(e))\n" % str(tmp_path))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=120)
    assert r.stdout.strip() == "raised True", r.stdout + r.stderr


def test_build_entry_compiles_a_tree_without_built_libraries(tmp_path):
    """build() must compile from sources alone: the package refuses to import without its
    library, so the build script may not be reached through the package import."""
    import shutil
    for d in ("include", "kvq_synth"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    shutil.copytree(PKG, tmp_path / "decode_attention_10_amd",
                    ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    shutil.copy(os.path.join(ROOT, "__graft_entry__.py"), tmp_path)
    assert not (tmp_path / "decode_attention_10_amd" / "libkvq.so").exists()
    code = "import sys; sys.path.insert(0, %r); import __graft_entry__ as g; g.build()" % (
        str(tmp_path))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       timeout=900, cwd=str(tmp_path))
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    assert (tmp_path / "decode_attention_10_amd" / "libkvq.so").exists()
    assert (tmp_path / "kvq_synth" / "libkvq_synth.so").exists()


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_match_the_configs():
    """Bytes per decode from the shapes (codes, metadata, fp16 window, q, out; for KVQuant
    the CSR too): 0.115 / 117.6 / 681.7 / 101.2 MB and 3.662 GB for the five configs."""
    sys.path.insert(0, ROOT)
    import bench
    import kvq_synth as S
    W = S.WORKLOADS
    got = {n: bench.decode_bytes(W[n], W[n].n_packed, W[n].n_resid)
           for n in ("tiny", "llama2_7b", "llama2_13b_k4v2", "llama3_8b_gqa")}
    got["kvquant_1m"] = bench.nuq_decode_bytes(W["kvquant_1m"], W["kvquant_1m"].n_packed)
    want = {"tiny": (0.115, 1e6, 3), "llama2_7b": (117.6, 1e6, 1),
            "llama2_13b_k4v2": (681.7, 1e6, 1), "llama3_8b_gqa": (101.2, 1e6, 1),
            "kvquant_1m": (3.662, 1e9, 3)}
    for n, (value, unit, digits) in want.items():
        assert round(got[n] / unit, digits) == value, n
    # per-unit figure used for the roofline: 459,520 B per (batch, kv head) of llama2_7b
    assert got["llama2_7b"] == 256 * 459520          # q and out shares included per unit


def test_bench_cpu_baseline_legs_run_the_oracle():
    """The bench's oracle legs: worker processes from a fork server, 1 and 2 workers on the
    tiny workload, each reporting decode and quantize rates in GB/s and its core count."""
    import multiprocessing as mp
    sys.path.insert(0, ROOT)
    import bench
    ctx = mp.get_context("forkserver")
    for workers in (1, 2):
        r = bench.finish_cpu_leg(bench.start_cpu_leg(ctx, "tiny", workers, 0.5), "tiny",
                                 timeout_s=240)
        assert r["cores"] == workers and r["unit_runs"] >= workers
        assert r["decode_gbs"] > 0 and r["quantize_gbs"] > 0
        assert "tiny" in r["sample"]

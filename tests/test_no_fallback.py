"""The product path has no fallback: with the native library missing, the
binding raises on first use instead of computing anything another way, and
the bench refuses to run. Runs in subprocesses on the CPU (no GPU call)."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(code, env_extra):
    env = dict(os.environ, **env_extra)
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=120)


def test_binding_raises_without_library():
    r = _run("from transformer_attention_06_amd import native\n"
             "try:\n    native.lib()\nexcept OSError as e:\n    print('raised:', e)\nelse:\n    print('loaded')",
             {"NCATTN_LIB": os.path.join(ROOT, "no_such_dir", "libncattn.so")})
    assert r.returncode == 0, r.stderr
    assert "raised:" in r.stdout and "not found" in r.stdout


def test_entry_point_raises_without_library():
    # an entry point called with placeholder arguments fails at the library
    # load, before it could compute anything
    r = _run("from transformer_attention_06_amd import native\n"
             "try:\n    native.nc_attn_decode_workspace_bytes(1, 1, 1, 1, 64, 16)\n"
             "except OSError:\n    print('raised')",
             {"NCATTN_LIB": os.path.join(ROOT, "no_such_dir", "libncattn.so")})
    assert r.returncode == 0, r.stderr
    assert "raised" in r.stdout


def test_bench_refuses_without_gpu():
    import pytest
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    r = subprocess.run([sys.executable, "bench.py", "--steps", "1", "--warmup", "0"], cwd=ROOT, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert r.stdout.strip() == ""  # no result line

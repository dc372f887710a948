"""Host-side checks of the package's ground rules (no GPU needed).

* bench.py measures one GPU and refuses a multi-GPU request with a message;
* nothing in the product package reaches the CPU oracle (only the tests, the
  smoke check and the benchmark's CPU baseline may);
* the product path has no CPU fallback: a missing HIP library, or host
  tensors, raise instead of computing anything;
* the build/smoke entry points exist.
"""

import ast
import os
import subprocess
import sys

import pytest
import torch

import hadamard_rotated_int8_amd as cr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "hadamard_rotated_int8_amd")


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert not r.stdout.strip()  # no JSON line


def _imported_modules(path):
    tree = ast.parse(open(path).read(), filename=path)
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            yield from (a.name for a in node.names)
        elif isinstance(node, ast.ImportFrom):
            yield node.module or ""


def test_product_package_never_reaches_the_oracle():
    seen = 0
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            path = os.path.join(dirpath, f)
            if f.endswith(".py"):
                seen += 1
                mods = list(_imported_modules(path))
                assert not any(m == "oracle" or m.startswith("oracle.") for m in mods), path
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                assert "convrot_oracle" not in open(path).read(), path
    assert seen >= 3


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(cr, "LIB_PATH", str(tmp_path / "libconvrot.so"))
    monkeypatch.setattr(cr, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        cr.lib()


def test_host_tensors_are_refused():
    x = torch.zeros(4, 16, dtype=torch.float32)
    with pytest.raises(Exception):
        cr.pack_activations(x, 16)
    with pytest.raises(Exception):
        cr.quantize_weights(torch.zeros(8, 16), 16)


def test_entry_points_exist():
    sys.path.insert(0, ROOT)
    import __graft_entry__ as entry

    assert callable(entry.build) and callable(entry.smoke)

"""The source digest that ties profiler counters to the kernels they were
taken on does not depend on where the repository is checked out."""
import os
import shutil
import subprocess
import sys


def test_source_digest_is_location_independent(tmp_path):
    from sparse_causal_attention_amd import build

    here = build.source_digest()
    root = os.path.dirname(os.path.dirname(os.path.abspath(build.__file__)))
    dst = tmp_path / "elsewhere"
    shutil.copytree(os.path.join(root, "sparse_causal_attention_amd"), dst / "sparse_causal_attention_amd",
                    ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    shutil.copytree(os.path.join(root, "include"), dst / "include")
    out = subprocess.run([sys.executable, "-c", "from sparse_causal_attention_amd import build; "
                          "print(build.source_digest())"], cwd=dst, capture_output=True, text=True, check=True)
    assert out.stdout.strip() == here

"""CPU checks of the build from a clean checkout.

The files a commit would hold (tracked plus untracked, not ignored) are copied to a fresh
directory, where no libattn.so exists.  There the package must import, every compute call
must fail with ImportError (there is no non-HIP path), and __graft_entry__.build() must
compile libattn.so for gfx950 with every symbol include/attn.h declares.
"""
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def checkout_files():
    try:
        out = subprocess.run(["git", "ls-files", "--cached", "--others", "--exclude-standard"],
                             cwd=ROOT, capture_output=True, text=True, check=True).stdout
    except (OSError, subprocess.CalledProcessError):
        pytest.skip("git is not available to list the checkout")
    return [f for f in out.splitlines() if f and os.path.isfile(os.path.join(ROOT, f))]


@pytest.fixture(scope="module")
def clean_tree(tmp_path_factory):
    dst = tmp_path_factory.mktemp("clean_checkout")
    for f in checkout_files():
        os.makedirs(os.path.join(dst, os.path.dirname(f)), exist_ok=True)
        shutil.copy2(os.path.join(ROOT, f), os.path.join(dst, f))
    assert not os.path.exists(os.path.join(dst, "exact_attention_08_amd", "libattn.so"))
    return str(dst)


def run_py(tree, code, timeout=120):
    return subprocess.run([sys.executable, "-c", code], cwd=tree, capture_output=True,
                          text=True, timeout=timeout)


def test_package_imports_without_the_library_and_compute_calls_fail(clean_tree):
    p = run_py(clean_tree, "import exact_attention_08_amd.build as b; print(b.LIB)")
    assert p.returncode == 0, p.stderr
    code = ("import exact_attention_08_amd as a\n"
            "try:\n"
            "    a.lib()\n"
            "except ImportError as e:\n"
            "    print('IMPORT_ERROR', e)\n")
    p = run_py(clean_tree, code)
    assert p.returncode == 0, p.stderr
    assert "IMPORT_ERROR" in p.stdout and "not built" in p.stdout


def test_graft_build_compiles_the_library_from_a_clean_checkout(clean_tree):
    p = run_py(clean_tree, "import __graft_entry__ as g; g.build()", timeout=900)
    assert p.returncode == 0, p.stdout[-2000:] + p.stderr[-2000:]
    lib = os.path.join(clean_tree, "exact_attention_08_amd", "libattn.so")
    assert os.path.exists(lib)
    out = subprocess.run(["nm", "-D", "--defined-only", lib], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)$", out, re.M))
    header = open(os.path.join(clean_tree, "include", "attn.h")).read()
    declared = set(re.findall(r"^(?:int|size_t)\s+(attn_\w+)\s*\(", header, re.M))
    assert declared and declared <= exported

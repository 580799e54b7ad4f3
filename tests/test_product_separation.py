"""The product path stands on its own: the package and its kernel sources never reference the CPU reference
(oracle/), and without the HIP library every call fails loudly instead of falling back to the CPU."""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_package_never_references_the_reference():
    pkg = os.path.join(ROOT, "rank_shared_kv_amd")
    hits = []
    for dirpath, _, files in os.walk(pkg):
        for name in files:
            if name.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                path = os.path.join(dirpath, name)
                with open(path, encoding="utf-8") as f:
                    for i, line in enumerate(f, 1):
                        if re.search(r"\boracle\b", line):
                            hits.append(f"{os.path.relpath(path, ROOT)}:{i}: {line.strip()}")
    assert not hits, "the product mentions the reference:\n" + "\n".join(hits)


def test_missing_library_fails_loudly():
    code = ("import rank_shared_kv_amd as lk\n"
            "try:\n"
            "    lk.lrkv_decode_workspace_bytes(lk.make_dims(1, 4, 16, 4, 64, 0), 64)\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n"
            "else:\n"
            "    print('no error')\n")
    env = dict(os.environ, LRKV_LIBRARY=os.path.join(ROOT, "no_such_dir", "liblrkv.so"))
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    assert res.stdout.startswith("raised:") and "missing" in res.stdout, res.stdout

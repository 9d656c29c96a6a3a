"""The build entry point works on a tree where libdllm.so does not exist yet
(a fresh checkout): the build script is reached without importing the
package, whose import requires the library."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.timeout(120)
def test_builder_loads_without_built_library(tmp_path):
    pkg = tmp_path / "diffusion_lm_gemm_amd"
    pkg.mkdir()
    for f in ("__init__.py", "build.py"):
        shutil.copy(os.path.join(ROOT, "diffusion_lm_gemm_amd", f), pkg / f)
    shutil.copy(os.path.join(ROOT, "__graft_entry__.py"), tmp_path / "__graft_entry__.py")
    code = (
        "import sys, __graft_entry__ as g\n"
        "b = g._load_builder()\n"
        "assert callable(b.build) and b.LIB.startswith(sys.argv[1])\n"
        "assert 'diffusion_lm_gemm_amd' not in sys.modules\n"
        "try:\n"
        "    import diffusion_lm_gemm_amd\n"
        "except ImportError as e:\n"
        "    assert 'not built' in str(e)\n"
        "else:\n"
        "    raise AssertionError('the package imported without its library')\n"
        "print('ok')\n"
    )
    r = subprocess.run([sys.executable, "-c", code, str(tmp_path)], cwd=tmp_path, capture_output=True, text=True,
                       timeout=100)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "ok"

"""The build entry point must work on a fresh checkout: loading the build
scripts may not import the binding package, whose import fails until the
library it loads has been built."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_build_scripts_load_without_the_package():
    code = (
        "import sys, os\n"
        "import __graft_entry__ as g\n"
        "lib = g._load_by_path('_b', os.path.join(g.ROOT, 'diffusion_transformer_relu_amd', 'build.py'))\n"
        "orc = g._load_by_path('_o', os.path.join(g.ROOT, 'oracle', 'build.py'))\n"
        "assert callable(lib.build) and callable(orc.build)\n"
        "assert 'diffusion_transformer_relu_amd' not in sys.modules\n"
        "print('ok')\n")
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert res.returncode == 0 and res.stdout.strip() == "ok", res.stderr

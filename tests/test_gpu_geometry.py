"""Launch-geometry invariance: block indices and SR draws are functions of tile
coordinates, so other grid sizes, tile orders and encode mappings must give bit-identical outputs.

The calls of tests/geometry_calls.py run here with the default launch settings and in a child process
with the NVFP4Q_* settings of geometry_calls.CHILD_ENV (read once per process by the library).
"""
import os
import subprocess
import sys

import numpy as np
import pytest

from tests import geometry_calls

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_outputs_do_not_depend_on_launch_geometry(gpu_lib, tmp_path):
    here = geometry_calls.run_all(gpu_lib)
    out = tmp_path / "child.npz"
    env = dict(os.environ, **geometry_calls.CHILD_ENV)
    print("child launch settings:", geometry_calls.CHILD_ENV, flush=True)
    subprocess.run([sys.executable, os.path.join(ROOT, "tests", "geometry_calls.py"), str(out)], env=env,
                   check=True, timeout=110)
    child = np.load(out)
    assert sorted(child.files) == sorted(here)
    for k, v in here.items():
        c = child[k]
        assert c.shape == v.shape, k
        bad = np.flatnonzero(c.reshape(-1) != v.reshape(-1))
        assert bad.size == 0, f"{k}: {bad.size} of {v.size} differ under other launch settings"

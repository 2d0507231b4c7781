"""Every kernel with a launch capped far below its chunk count, so that the
striding loops run (at real sizes a launch has one workgroup per chunk up to
2^30): the library is told the cap through LAYERADAM_MAX_GRID, which it reads
once per process, so each cap runs tests/grid_stride_child.py in a child
process."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("grid", [1, 7, 300])
def test_striding_loops_with_a_capped_grid(grid):
    print(f"case grid cap {grid}", flush=True)
    env = dict(os.environ, LAYERADAM_MAX_GRID=str(grid))
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "grid_stride_child.py")],
                       env=env, capture_output=True, text=True, timeout=240)
    print(r.stdout[-3000:], r.stderr[-3000:], flush=True)
    assert r.returncode == 0 and "grid stride ok" in r.stdout

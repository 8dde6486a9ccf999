"""The forward under the library's environment switches matches the fp64
oracle: GQA_ATTN_PACK=0 (no query-head packing) and GQA_FWD_PERSISTENT=0
(one workgroup per row tile for variable-length batches). The library reads
each switch once per process, so the cases run in a child process
(tests/env_switch_child.py)."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("mode,var", [("unpacked", "GQA_ATTN_PACK"), ("one_tile", "GQA_FWD_PERSISTENT")])
def test_forward_under_switch(mode, var):
    env = dict(os.environ)
    env[var] = "0"
    res = subprocess.run([sys.executable, "-u", os.path.join(HERE, "env_switch_child.py"), mode], env=env,
                         capture_output=True, text=True, timeout=240)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert f"{mode} ok" in res.stdout

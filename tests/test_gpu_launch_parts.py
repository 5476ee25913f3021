"""Shares, groups and quantizations split into several launches agree with
the oracle bit for bit. The split normally starts past 2^34 elements per
share; a child process lowers the bound to 4096 elements
(QRS_MAX_LAUNCH_ELEMS) and runs every entry point at small sizes
(tests/launch_parts_cases.py): ragged last launches, one-row launches of a
row-strided share, all shares of a group advancing together, and the
prepared launch."""

import os
import subprocess
import sys

import pytest

from gpu_util import log

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def test_every_entry_point_split_into_small_launches(gpu):
    env = dict(os.environ, QRS_MAX_LAUNCH_ELEMS="4096")
    log("[parts] child process with QRS_MAX_LAUNCH_ELEMS=4096")
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "launch_parts_cases.py")], env=env,
                       capture_output=True, text=True, timeout=300)
    log(r.stderr[-3000:])
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "all cases match the oracle" in r.stdout

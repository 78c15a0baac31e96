"""The C ABI from plain C: tests/host/c_client.c (built by the package's
build step, no Python or torch inside) calibrates, appends and decodes on
every path through libloki.so and checks ids, cross-path agreement, the
k = S equality with the dense baseline and the argument checks."""

import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "tests", "host", "c_client")


def test_plain_c_client_runs_every_path():
    if not os.path.exists(CLIENT):
        pytest.fail("tests/host/c_client is not built: run __graft_entry__.build()")
    r = subprocess.run([CLIENT], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "ok"

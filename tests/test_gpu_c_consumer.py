"""The C ABI from a plain C program (tests/c/ra_c_consumer.c), run on the GPU as a child
process: a causal zigzag share with Q = 0, every row checked against the closed form
(lse = ln of the allowed-key count, out = the mean of those V rows), and an invalid call
that must return RA_ERR_ARG with a message."""

import subprocess

import pytest

from tests.c_consumer import build
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def test_plain_c_consumer_runs(tmp_path):
    exe = build(str(tmp_path / "ra_c_consumer"))
    say("plain C consumer")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    say(r.stdout.strip())
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok")

"""The C ABI used from plain C, without Python or torch: tests/host/c_round.c
(built by __graft_entry__.build()) allocates with hipMalloc, runs a round
through moe_ep_dispatch and one through moe_ep_dispatch_noalloc, and checks
placement, the invalid fill and a combine whose exact result is each
token's destination mask (expert rows 2^d; NaN in rows never sent)."""

from __future__ import annotations

import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "host", "c_round")


def test_c_round():
    assert os.path.exists(BIN), f"{BIN} is missing: run __graft_entry__.build()"
    print("[c_abi] c_round", flush=True)
    p = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    assert p.returncode == 0, p.stdout + p.stderr
    assert "c_round ok" in p.stdout

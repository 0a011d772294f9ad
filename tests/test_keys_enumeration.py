"""The key-major work-item enumeration (csrc/attn_bwd_keys.h, shared by the device planner and
the host capacity bound): exact coverage of every visible (query, row) pair by one item, one
partial slot per item, records that list their block's items, and the item_cap bound, over
random packed batches, chunks, ratios, windows and modes.  The enumeration is driven from the
host the way the planner drives it; the planner kernel itself is exercised by the GPU parity
tests of the backward and the indexer loss."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_keys_enumeration_covers_every_pair_once():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "keys_enumeration_check")
        subprocess.run(["g++", "-O2", "-std=c++17", "-o", exe,
                        os.path.join(HERE, "keys_enumeration_check.cpp")], check=True)
        out = subprocess.run([exe, "30"], capture_output=True, text=True, timeout=300)
    print(out.stdout)
    assert out.returncode == 0, out.stdout
    pairs = int(out.stdout.split("pairs ")[1].split()[0])
    assert pairs > 1_000_000

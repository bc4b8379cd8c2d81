"""The chunk-attention work list on the host (no GPU): the header the kernel uses to
cut the weighted (query block, key tile) list into workgroup shares
(csrc/attn_plan.h), built with g++ and checked over random cache shapes, query
counts, head counts and grids: every tile in exactly one share, every share
non-empty, the holders of a cut block's earlier tiles where the merging workgroup
looks for them, publishers' ranges processed first and mergers' last."""

import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "host_checks", "attn_partition.cpp")


@pytest.fixture(scope="module")
def prog(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("part") / "attn_partition")
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-o", exe, SRC], check=True)
    return exe


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_attention_partition(prog, seed):
    out = subprocess.run([prog, "3000", str(seed)], capture_output=True, text=True)
    print(out.stdout)
    assert out.returncode == 0, out.stdout
    assert "3000 cases, 0 failures" in out.stdout

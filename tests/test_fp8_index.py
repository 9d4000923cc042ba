"""Every block of the FP8-weight FFN's two launches, walked on the CPU.

tests/native/fp8_index_check.cpp is built (g++) from the index code the
kernel itself uses (top_expert_routing_amd/csrc/item_plan.h: the work-item
lookup of block_find_item and the FP8 code addresses) and run at the launch
geometry the library picks: it checks that every block's work item is valid,
that every code, scale, token-row and output access stays inside its buffer,
and that both phases write every output element exactly once.  The cases
include the GPT-OSS-shaped mixed batch's own routing (16640 rows, 256 groups,
d = I = 2880, 64-row tiles, a priority segment), the one configuration in
which an FP8 run ended in a GPU memory fault - and which the library now
refuses - and the shapes the GPU parity tests run.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import workloads
from oracle import moe_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "native", "fp8_index_check.cpp")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("fp8") / "fp8_index_check")
    subprocess.run([cxx, "-O2", "-std=c++17", "-Wall", "-Werror", SRC, "-o", exe], check=True)
    return exe


def _mf(n_rows, G):
    """The library's tile height for an average group size (16, 32 or 64 rows)."""
    avg = n_rows // G if G else n_rows
    return 1 if avg <= 8 else 2 if avg <= 24 else 4


def _run(exe, offs, rows, d, I, E, S, nseg, n_x, packed):
    N = int(offs[-1])
    G = nseg * E + S
    hdr = [d, I, E, S, nseg, N, n_x, _mf(N, G), int(packed), int(rows is not None)]
    body = " ".join(map(str, hdr)) + "\n" + " ".join(map(str, np.asarray(offs).tolist())) + "\n"
    if rows is not None:
        body += " ".join(map(str, np.asarray(rows).tolist())) + "\n"
    r = subprocess.run([exe], input=body, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout.strip()


@pytest.mark.timeout(900)
def test_fp8_launch_addresses_gptoss_mixed(checker):
    wl = workloads.make("gptoss_mixed", "cpu", with_weights=False)
    s = wl.spec
    ids, _ = O.gate(wl.logits.numpy(), s.k)
    p = O.permute(ids, s.E, s.S, s.n_priority)
    for packed in (True, False):
        rc, out = _run(checker, p["group_offsets"], p["sorted_token"], s.d, s.I, s.E, s.S, 2, s.T, packed)
        assert rc == 0 and out.startswith("ok"), out


CASES = [
    # (T, E, k, S, P, d, I): the FP8 parity cases' shapes and decode shapes
    (128, 64, 8, 0, 0, 2048, 1024), (16, 64, 6, 2, 0, 2048, 1408), (96, 16, 4, 0, 0, 144, 208),
    (300, 8, 2, 1, 20, 256, 192), (100, 16, 4, 0, 30, 128, 96), (64, 512, 8, 2, 0, 64, 48),
    (80, 512, 4, 2, 30, 32, 16), (1, 4, 1, 0, 0, 16, 16), (256, 64, 6, 2, 0, 2048, 1408),
]


@pytest.mark.parametrize("T,E,k,S,P,d,I", CASES)
def test_fp8_launch_addresses(checker, T, E, k, S, P, d, I):
    ids = workloads.random_ids(T, E, k, seed=T + E)[0].numpy()
    p = O.permute(ids, E, S, P)
    packed = d % 64 == 0 and I % 64 == 0
    for rows in (p["sorted_token"], None):
        rc, out = _run(checker, p["group_offsets"], rows, d, I, E, S, 2 if P else 1, T, packed)
        assert rc == 0 and out.startswith("ok"), out


def test_fp8_checker_detects_a_bad_offset(checker):
    """The walk does fail: group offsets that overlap (a precondition violation)
    make two blocks write the same output rows."""
    ids = workloads.random_ids(64, 8, 2, seed=3)[0].numpy()
    offs = O.permute(ids, 8, 0, 0)["group_offsets"].copy()
    offs[3] = offs[2] - 2              # group 3 starts inside group 1: two rows are written twice
    rc, out = _run(checker, offs, None, 64, 64, 8, 0, 1, 64, True)
    assert rc != 0 and out.startswith("FAIL"), out

"""Tile order of the persistent single-launch FFN, checked on the CPU.

tests/native/queue_check.cpp is built (g++) from the same header the GPU
kernel uses (top_expert_routing_amd/csrc/queue_plan.h) and run over routings:
every (phase, unit, column chunk) tile is listed exactly once over all
queues, the units tile each expert's rows exactly, flag indices stay inside
the workspace the host allocates, and with ONE block per queue popping in
order (a waiting block stalls its whole queue) every queue drains - so no
phase-2 wait of the kernel can stall on a phase-1 tile that is never popped.
The shapes mirror the library's: 128-row units, 128 SwiGLU / 256 output
columns per tile, 8 queues and a lag of one round of blocks (64), plus other
unit heights, queue counts and lags.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import workloads
from oracle import moe_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "native", "queue_check.cpp")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("qc") / "queue_check")
    subprocess.run([cxx, "-O2", "-std=c++17", "-Wall", "-Werror", SRC, "-o", exe], check=True)
    return exe


def _run(exe, offs, E, S, nseg, d, I, bm=128, nq=8, lag=64, units_cap=None):
    N = int(offs[-1])
    nch1, nch2 = -(-I // 128), -(-d // 256)
    cap = -(-N // bm) + E + S if units_cap is None else units_cap
    hdr = [E, S, nseg, N, bm, nch1, nch2, nq, lag, cap]
    inp = " ".join(map(str, hdr)) + "\n" + " ".join(map(str, np.asarray(offs).tolist())) + "\n"
    r = subprocess.run([exe], input=inp, capture_output=True, text=True)
    return r.returncode, r.stdout.strip()


def _offsets(T, E, k, S, P, kind, seed):
    rng = np.random.default_rng(seed)
    if kind == "zipf":
        lg = rng.standard_normal((T, E)) - 1.0 * np.log(np.arange(1, E + 1))[rng.permutation(E)]
    elif kind == "one_hot":
        lg = np.zeros((T, E))
        lg[:, E // 2] = 10.0
    else:
        lg = rng.standard_normal((T, E))
    ids, _ = O.gate(lg.astype(np.float32), k)
    return O.permute(ids, E, S, P)["group_offsets"]


CASES = [
    # (T, E, k, S, P, d, I, kind)
    (600, 8, 2, 0, 50, 256, 320, "random"),
    (4160, 128, 4, 0, 64, 256, 320, "zipf"),
    (2000, 64, 4, 2, 300, 128, 96, "zipf"),
    (1300, 512, 4, 256, 10, 64, 32, "random"),
    (900, 12, 3, 1, 100, 96, 160, "zipf"),
    (700, 8, 2, 0, 3, 128, 128, "random"),
    (3000, 4, 2, 1, 200, 128, 192, "zipf"),
    (500, 16, 2, 0, 500, 64, 64, "random"),      # every token in the priority segment
    (777, 8, 1, 0, 1, 64, 64, "one_hot"),        # one expert takes everything
    (40, 32, 2, 0, 7, 64, 2880, "zipf"),         # almost all experts empty, many chunks
]


@pytest.mark.parametrize("T,E,k,S,P,d,I,kind", CASES)
@pytest.mark.parametrize("bm,nq,lag", [(128, 8, 64), (128, 8, 0), (64, 8, 64), (128, 1, 1), (128, 3, 5),
                                       (16, 8, 1 << 20)])
def test_queue_order(checker, T, E, k, S, P, d, I, kind, bm, nq, lag):
    offs = _offsets(T, E, k, S, P, kind, seed=T + E)
    rc, out = _run(checker, offs, E, S, 2 if P else 1, d, I, bm, nq, lag)
    assert rc == 0 and out.startswith("ok"), out


def test_queue_order_gptoss_shape(checker):
    """The GPT-OSS-shaped mixed batch's own routing (64 decode + 4096 prefill
    tokens, Zipf-skewed, d = I = 2880), at the launch's queue count and lag."""
    wl = workloads.make("gptoss_mixed", "cpu", with_weights=False)
    s = wl.spec
    ids, _ = O.gate(wl.logits.numpy(), s.k)
    offs = O.permute(ids, s.E, s.S, s.n_priority)["group_offsets"]
    for lag in (64, 0):
        rc, out = _run(checker, offs, s.E, s.S, 2, s.d, s.I, 128, 8, lag)
        assert rc == 0 and out.startswith("ok"), out


def test_queue_checker_rejects_small_capacity(checker):
    """The checker does fail: a flag area smaller than the units needs."""
    offs = _offsets(600, 8, 2, 0, 50, "random", seed=1)
    rc, out = _run(checker, offs, 8, 0, 2, 256, 320, units_cap=3)
    assert rc != 0 and out.startswith("FAIL"), out

"""moe_grouped_ffn_noalloc: the FFN on the library's per-device scratch array
(no workspace argument, nothing allocated by the call) gives moe_grouped_ffn's
results bit for bit - the same kernels on the same inputs - over consecutive
calls that share the array, the later ones smaller, on the decode, split-K and
persistent-queue paths; a call whose workspace would exceed the array is
refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

from oracle import moe_oracle as O
from helpers import TOL, announce, f64_of, np_of, rel_max_err, require_gpu
import workloads

import top_expert_routing_amd as moe
from top_expert_routing_amd import _lib

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    # (T, E, k, S, P, d, I, kind): consecutive calls, each smaller than the one before
    (128, 64, 8, 0, 0, 2048, 1024, "random"),    # OLMoE decode shape (32-row decode tiles)
    (600, 8, 2, 0, 50, 256, 320, "random"),      # priority segment, large groups: persistent queue
    (40, 16, 2, 1, 6, 96, 160, "random"),        # split-K decode kernel, shared expert, priority segment
]


def _inputs(T, E, k, S, P, d, I, kind, seed):
    wl = workloads.custom(T=T, E=E, k=k, d=d, I=I, dtype="bf16", S=S, n_priority=P, seed=seed, device="cpu",
                          w_std=0.08)
    ids = workloads.random_ids(T, E, k, seed)[0].contiguous()
    return wl, ids


def test_ffn_noalloc_matches_workspace_call():
    require_gpu()
    lib = _lib.load()
    for case in CASES:
        T, E, k, S, P, d, I, kind = case
        announce(f"ffn noalloc T={T} E={E} k={k} S={S} P={P} d={d} I={I}")
        wl, ids = _inputs(*case, seed=T + 3 * E)
        nseg = 2 if P else 1
        p = O.permute(ids.numpy(), E, S, P, np_of(wl.x))
        N = int(p["group_offsets"][-1])
        offs = torch.from_numpy(p["group_offsets"]).to(DEV)
        rows = torch.from_numpy(p["sorted_token"]).to(DEV)
        x = wl.x.to(DEV)
        w = [t.to(DEV) for t in (wl.w_gate, wl.w_up, wl.w_down)]
        h_ref = moe.grouped_ffn(x, offs, E, S, nseg, *w, x_rows=rows)
        h = torch.full((N, d), float("nan"), dtype=torch.bfloat16, device=DEV)
        # straight through the C ABI
        st = lib.moe_grouped_ffn_noalloc(x.data_ptr(), rows.data_ptr(), T, offs.data_ptr(), N, E, S, nseg, d, I,
                                         w[0].data_ptr(), w[1].data_ptr(), w[2].data_ptr(), _lib.MOE_BF16,
                                         h.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert st == _lib.MOE_OK, _lib.STATUS_NAMES.get(st, st)
        torch.cuda.synchronize()
        assert torch.equal(h, h_ref)
        ref = O.grouped_ffn(p["x_sorted"], p["group_offsets"], E, S, nseg, np_of(wl.w_gate), np_of(wl.w_up),
                            np_of(wl.w_down), "bf16")
        assert rel_max_err(f64_of(h), ref) <= TOL["bf16"]


def test_ffn_noalloc_refuses_workspace_above_the_array():
    require_gpu()
    lib = _lib.load()
    # the Qwen3-shaped prefill needs ~96 MiB of SwiGLU intermediate: refused, nothing enqueued
    N, E, d, I = 65536, 128, 2048, 768
    assert moe.ffn_workspace_bytes(N, E, 0, 1, d, I) > moe.NOALLOC_SCRATCH_BYTES
    fake = 1 << 20
    st = lib.moe_grouped_ffn_noalloc(fake, None, 0, fake, N, E, 0, 1, d, I, fake, fake, fake, _lib.MOE_BF16, fake,
                                     None)
    assert st == _lib.MOE_ERR_WORKSPACE

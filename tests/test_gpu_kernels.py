"""GPU parity of each libmoe call against the CPU oracle, through the C ABI.

Integer outputs (ids, permutation, offsets, counts, union, affinity, request
counts) must match bit for bit; gate weights within 1e-6 absolute; FFN and
combine within 1e-2 (bf16) / 1e-5 (fp32) of max |reference|; signatures within
1e-6 relative.  Inputs are small enough for the oracle to finish in seconds
but span several tiles and ragged tails; edge cases cover empty batches,
empty groups, one hot expert, k = E, E = 1, E = 512 and priority segments.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import moe_oracle as O
from helpers import GATE_W_ATOL, SIG_RTOL, TOL, announce, f64_of, np_of, rel_max_err, require_gpu

import top_expert_routing_amd as moe

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _poison(shape, dtype):
    t = torch.empty(shape, dtype=dtype, device=DEV)
    t.view(torch.uint8).fill_(0xFF) if t.numel() else None
    return t


# ------------------------------------------------------------------ router
ROUTER_CASES = [
    # (T, d, E, dtype)
    (1, 8, 1, "bf16"),            # one token, one expert, a single partial K-step
    (37, 136, 70, "bf16"),        # token tail, K tail (136 = 128 + 8), experts past one 64-wide tile
    (128, 2048, 64, "bf16"),      # OLMoE decode shape
    (300, 256, 512, "bf16"),      # E = 512: eight expert tiles
    (4100, 264, 500, "bf16"),     # >= 1024 tiles of 32 tokens: the two-slab tile, with T, d and E tails
    (64, 128, 8, "f32"),          # the tiny config's shape
    (33, 72, 13, "f32"),          # fp32 tails
]


@pytest.mark.parametrize("T,d,E,dtype", ROUTER_CASES)
def test_router_parity(T, d, E, dtype):
    announce(f"router T={T} d={d} E={E} {dtype}")
    g = torch.Generator().manual_seed(T * 7 + d + E)
    xf = torch.randn((T, d), generator=g, dtype=torch.float64)
    wf = torch.randn((E, d), generator=g, dtype=torch.float64) * 0.05
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    x, w = xf.to(tdt), wf.to(tdt)
    ref = O.router(np_of(x), np_of(w), dtype)
    # fp32 accumulation of d products (exact for bf16 inputs, one rounding each
    # for fp32 inputs), in any order: |err| <= (d + 1) * 2^-24 * sum_i |x_i w_i|
    bound = (d + 1) * 2.0 ** -24 * (np.abs(O.to_f64(np_of(x), dtype)) @ np.abs(O.to_f64(np_of(w), dtype)).T)
    logits = _poison((T, E), torch.float32)
    moe.router(x.to(DEV), w.to(DEV), logits)
    torch.cuda.synchronize()
    got = np_of(logits).astype(np.float64)
    assert np.all(np.abs(got - ref) <= bound + 1e-30), float(np.max(np.abs(got - ref) - bound))


def test_router_then_gate_matches_oracle_on_gpu_logits():
    # the gate's ids are decided on the logits the GPU produced (both sides in fp32)
    wl = workloads.custom(T=96, E=64, k=8, d=2048, I=64, dtype="bf16", seed=5, device=DEV, w_std=0.08)
    w_r = (torch.randn((64, 2048), generator=torch.Generator().manual_seed(9)) * 0.02).to(torch.bfloat16).to(DEV)
    logits = moe.router(wl.x, w_r)
    ids, wts = moe.gate(logits, 8)
    torch.cuda.synchronize()
    ids_ref, w_ref = O.gate(np_of(logits), 8)
    np.testing.assert_array_equal(np_of(ids), ids_ref)
    assert np.abs(np_of(wts).astype(np.float64) - w_ref).max() <= GATE_W_ATOL


# ------------------------------------------------------------------ gate
GATE_CASES = [
    # (T, E, k, renormalize, kind)
    (1, 8, 2, 1, "normal"), (300, 64, 8, 1, "normal"), (257, 128, 8, 1, "normal"),
    (64, 8, 8, 1, "normal"), (33, 1, 1, 1, "normal"), (100, 512, 16, 1, "normal"),
    (129, 96, 5, 0, "normal"), (50, 16, 16, 0, "normal"), (200, 64, 6, 1, "ties"),
    (200, 130, 7, 1, "ties"), (64, 32, 4, 1, "zeros_nan"), (77, 512, 512, 1, "ties"),
]


def _gate_logits(T, E, kind, seed):
    g = torch.Generator().manual_seed(seed)
    lg = torch.randn((T, E), generator=g)
    if kind == "ties":
        lg = torch.floor(lg * 2) / 2
    if kind == "zeros_nan":
        lg = torch.floor(lg)
        lg[lg == 0] = -0.0
        lg[:, ::3] = 0.0
        lg[::5, 1] = float("nan")
        lg[::7, 2] = float("-inf")
    return lg


@pytest.mark.parametrize("T,E,k,renorm,kind", GATE_CASES)
def test_gate_parity(T, E, k, renorm, kind):
    announce(f"gate T={T} E={E} k={k} renorm={renorm} {kind}")
    lg = _gate_logits(T, E, kind, seed=T * 1000 + E + k)
    ids_ref, w_ref = O.gate(lg.numpy(), k, bool(renorm))
    ids = _poison((T, k), torch.int32)
    w = _poison((T, k), torch.float32)
    moe.gate(lg.to(DEV), k, bool(renorm), ids, w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(np_of(ids), ids_ref)
    got = np_of(w)
    finite = np.isfinite(w_ref)
    assert np.abs(got[finite].astype(np.float64) - w_ref[finite]).max(initial=0.0) <= GATE_W_ATOL


def test_gate_config_logits_bit_exact():
    for name in ("tiny", "olmoe_decode", "qwen3_prefill", "dsv2_decode_t256", "gptoss_mixed"):
        wl = workloads.make(name, DEV, with_weights=False)
        announce(f"gate {name}")
        for l in range(wl.stats_logits.shape[0]):
            lg = wl.stats_logits[l].contiguous()
            ids, w = moe.gate(lg, wl.spec.k)
            ids_ref, w_ref = O.gate(np_of(lg), wl.spec.k)
            np.testing.assert_array_equal(np_of(ids), ids_ref)
            assert np.abs(np_of(w).astype(np.float64) - w_ref).max() <= GATE_W_ATOL


GATE_RECORD_CASES = [
    # (T, E, k, renormalize, kind, block_tokens, L)
    (1000, 64, 6, 1, "normal", 16, 2),      # KV blocks of 16, ragged last block
    (37, 512, 8, 1, "ties", 7, 3),          # E = 512, an odd block size, ties
    (64, 8, 2, 1, "normal", 1, 1),          # one token per block
    (50, 32, 4, 0, "zeros_nan", 64, 1),     # one block longer than the batch
    (300, 96, 3, 1, "ties", 33, 2),         # E not a multiple of 64
    (200, 130, 130, 1, "normal", 40, 1),    # k = E: every block's row counts its tokens
]


@pytest.mark.parametrize("T,E,k,renorm,kind,bt,L", GATE_RECORD_CASES)
def test_gate_record_parity(T, E, k, renorm, kind, bt, L):
    """moe_gate_record: ids and weights bit-identical to moe_gate's, and the
    KV-block record equal to the oracle's request counts over block offsets,
    every row of every layer written (the buffer starts poisoned)."""
    announce(f"gate_record T={T} E={E} k={k} bt={bt} L={L} {kind}")
    nb = -(-T // bt)
    lgs = [_gate_logits(T, E, kind, seed=T * 7 + E + l) for l in range(L)]
    rec = _poison((nb, L, E), torch.int32)
    ids_all = []
    for l, lg in enumerate(lgs):
        ids = _poison((T, k), torch.int32)
        w = _poison((T, k), torch.float32)
        moe.gate_record(lg.to(DEV), k, bt, l, rec, bool(renorm), ids, w)
        ids0, w0 = moe.gate(lg.to(DEV), k, bool(renorm))
        torch.cuda.synchronize()
        assert torch.equal(ids, ids0) and torch.equal(w.view(torch.int32), w0.view(torch.int32))
        ids_ref, _ = O.gate(lg.numpy(), k, bool(renorm))
        np.testing.assert_array_equal(np_of(ids), ids_ref)
        ids_all.append(ids_ref)
    boffs = np.minimum(np.arange(nb + 1, dtype=np.int64) * bt, T).astype(np.int32)
    ref = O.stats(np.stack(ids_all), E, boffs)["req_counts"]          # [nb][L][E]
    np.testing.assert_array_equal(np_of(rec), ref)


def test_gate_record_touches_only_its_layer():
    T, E, k, bt, L = 100, 64, 4, 16, 3
    lg = _gate_logits(T, E, "normal", seed=5).to(DEV)
    rec = torch.full((-(-T // bt), L, E), -7, dtype=torch.int32, device=DEV)
    moe.gate_record(lg, k, bt, 1, rec)
    torch.cuda.synchronize()
    assert bool((rec[:, 0] == -7).all()) and bool((rec[:, 2] == -7).all())
    assert int(rec[:, 1].sum().item()) == T * k


def test_stage_to_host():
    """The record staged into pinned host memory with moe_stage_to_host equals
    the device copy; a pageable destination is refused."""
    announce("stage_to_host")
    src = torch.randint(-1000, 1000, (512, 8, 128), dtype=torch.int32, device=DEV)
    dst = torch.empty(src.shape, dtype=torch.int32, pin_memory=True)
    moe.stage_to_host(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(dst, src.cpu())
    with pytest.raises(moe.MoeError):
        moe.stage_to_host(src, torch.empty(src.shape, dtype=torch.int32))


def test_gate_empty_batch():
    ids = torch.empty((0, 2), dtype=torch.int32, device=DEV)
    w = torch.empty((0, 2), dtype=torch.float32, device=DEV)
    moe.gate(torch.empty((0, 8), device=DEV), 2, True, ids, w)
    torch.cuda.synchronize()


# ------------------------------------------------------------------ permute
PERM_CASES = [
    # (T, E, k, S, P, d, dtype, kind)
    (3, 3, 2, 0, 0, 8, torch.float32, "random"),
    (128, 64, 8, 0, 0, 2048, torch.bfloat16, "random"),
    (256, 64, 6, 2, 0, 64, torch.bfloat16, "zipf"),
    (600, 32, 8, 0, 0, 72, torch.float32, "random"),        # 4800 assignments: two chunks, ragged
    (4160, 128, 4, 0, 64, 40, torch.bfloat16, "zipf"),     # priority segment, 17 chunks
    (5000, 16, 2, 1, 5000, 16, torch.bfloat16, "random"),  # every token in the priority segment
    (777, 8, 1, 0, 1, 24, torch.float32, "one_hot"),       # all tokens to one expert
    (1100, 512, 4, 3, 0, 8, torch.bfloat16, "random"),
    (2, 4, 4, 0, 0, 8, torch.float32, "random"),           # k = E
    (10, 1, 1, 0, 0, 8, torch.float32, "random"),          # E = 1
    (9000, 8, 8, 0, 0, 0, None, "random"),                 # no row gather, k = E, 71 chunks: scan launch
    (8192, 128, 8, 0, 0, 0, None, "random"),               # 64 chunks: the most the scatter scans itself
    (8200, 16, 8, 2, 8, 0, None, "zipf"),                  # 65 chunks: scan launch, shared + priority
]


def _ids(T, E, k, kind, seed):
    if kind == "one_hot":
        return torch.full((T, k), E // 2, dtype=torch.int32)
    if kind == "zipf":
        lg = torch.randn((T, E), generator=torch.Generator().manual_seed(seed)) - 1.5 * torch.log(
            torch.arange(1, E + 1, dtype=torch.float32))
        return torch.topk(lg, k, dim=1).indices.to(torch.int32)
    return workloads.random_ids(T, E, k, seed)[0]


@pytest.mark.parametrize("T,E,k,S,P,d,dtype,kind", PERM_CASES)
def test_permute_parity(T, E, k, S, P, d, dtype, kind):
    announce(f"permute T={T} E={E} k={k} S={S} P={P} d={d} {kind}")
    ids = _ids(T, E, k, kind, seed=T + 7 * E).contiguous()
    x = None
    if dtype is not None:
        x = torch.randn((T, d), generator=torch.Generator().manual_seed(T)).to(dtype)
    ref = O.permute(ids.numpy(), E, S, P, np_of(x) if x is not None else None)
    N = T * (k + S)
    G = (2 if P > 0 else 1) * E + S
    out = {"group_offsets": _poison(G + 1, torch.int32), "sorted_to_flat": _poison(N, torch.int32),
           "flat_to_sorted": _poison(N, torch.int32), "sorted_token": _poison(N, torch.int32)}
    if x is not None:
        out["x_sorted"] = _poison((N, d), dtype)
    got = moe.permute(ids.to(DEV), E, S, P, x.to(DEV) if x is not None else None, out=out)
    torch.cuda.synchronize()
    for key in ("group_offsets", "sorted_to_flat", "flat_to_sorted", "sorted_token"):
        np.testing.assert_array_equal(np_of(got[key]), ref[key], err_msg=key)
    if x is not None:
        assert np.array_equal(np_of(got["x_sorted"]), ref["x_sorted"])


def test_permute_empty_batch_writes_zero_offsets():
    out = {"group_offsets": _poison(8 + 1 + 1, torch.int32),
           "sorted_to_flat": torch.empty(0, dtype=torch.int32, device=DEV),
           "flat_to_sorted": torch.empty(0, dtype=torch.int32, device=DEV)}
    moe.permute(torch.empty((0, 2), dtype=torch.int32, device=DEV), 8, 1, 0, None, out=out)
    torch.cuda.synchronize()
    assert (np_of(out["group_offsets"])[:9 + 1] == 0).all()


def test_permute_deterministic():
    ids = workloads.random_ids(8192, 128, 8, seed=11)[0].to(DEV)
    a = moe.permute(ids, 128, 0, 0)
    b = moe.permute(ids, 128, 0, 0)
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key


# ------------------------------------------------------------------ grouped FFN
FFN_CASES = [
    # (T, E, k, S, P, d, I, dtype, kind)
    (64, 8, 2, 0, 0, 128, 256, "f32", "random"),          # the tiny config's shape
    (40, 6, 2, 1, 9, 40, 24, "f32", "random"),            # tails in d and I, shared + priority
    (96, 16, 4, 0, 0, 136, 200, "bf16", "random"),        # K and N tails (136 = 2*64 + 8)
    (300, 8, 2, 0, 0, 256, 192, "bf16", "random"),        # groups far above one tile
    (50, 64, 8, 2, 0, 128, 88, "bf16", "zipf"),           # hot/cold, empty groups, shared
    (33, 4, 1, 0, 1, 64, 64, "bf16", "one_hot"),          # one expert takes everything
    (17, 128, 4, 0, 5, 72, 136, "bf16", "random"),        # priority segment, mostly empty groups
    # groups of <= 4 rows on average: the split-K decode kernel
    (40, 32, 2, 0, 0, 200, 136, "bf16", "zipf"),          # K tails in both phases, a hot group over two tiles
    (24, 16, 2, 1, 6, 96, 160, "bf16", "random"),         # priority segment + shared expert
    # large groups with a priority segment: one persistent launch, per-XCD queues
    (600, 8, 2, 0, 50, 256, 320, "bf16", "random"),       # column tail in I (320 = 2*128 + 64)
    (900, 12, 3, 1, 100, 96, 160, "bf16", "zipf"),        # shared expert, hot/cold, small d
    (4000, 16, 4, 0, 256, 512, 384, "bf16", "random"),    # many units per XCD
    (700, 8, 2, 0, 3, 128, 128, "bf16", "random"),        # priority units on few XCDs only
    # groups averaging >= 256 rows: the 256 x 256, eight-wave GEMM tile
    (2000, 8, 2, 0, 0, 256, 320, "bf16", "random"),       # ragged last m-tile, column tail
    (3000, 4, 2, 1, 200, 128, 192, "bf16", "zipf"),       # priority segment + shared expert
    # the largest group count (2*512 routed + 256 shared = 1280) on each kernel
    (4, 512, 4, 256, 2, 64, 32, "bf16", "random"),         # decode kernel
    (300, 512, 4, 256, 10, 64, 32, "bf16", "random"),      # 128 x 256 GEMM
    (1300, 512, 4, 256, 10, 64, 32, "bf16", "random"),     # 256 x 256 persistent GEMM
]


def _ffn_inputs(T, E, k, S, P, d, I, dtype, kind, seed):
    wl = workloads.custom(T=T, E=E, k=k, d=d, I=I, dtype=dtype, S=S, n_priority=P, seed=seed, device="cpu",
                          w_std=0.08)
    ids = _ids(T, E, k, kind, seed).contiguous()
    return wl, ids


@pytest.mark.parametrize("T,E,k,S,P,d,I,dtype,kind", FFN_CASES)
def test_grouped_ffn_parity(T, E, k, S, P, d, I, dtype, kind):
    announce(f"ffn T={T} E={E} k={k} S={S} P={P} d={d} I={I} {dtype} {kind}")
    wl, ids = _ffn_inputs(T, E, k, S, P, d, I, dtype, kind, seed=T + E)
    nseg = 2 if P > 0 else 1
    p_ref = O.permute(ids.numpy(), E, S, P, np_of(wl.x))
    h_ref = O.grouped_ffn(p_ref["x_sorted"], p_ref["group_offsets"], E, S, nseg, np_of(wl.w_gate),
                          np_of(wl.w_up), np_of(wl.w_down), dtype)
    xs = torch.from_numpy(p_ref["x_sorted"].view(np.int16) if dtype == "bf16" else p_ref["x_sorted"])
    xs = (xs.view(torch.bfloat16) if dtype == "bf16" else xs).to(DEV)
    offs = torch.from_numpy(p_ref["group_offsets"]).to(DEV)
    nbytes = moe.ffn_workspace_bytes(xs.shape[0], E, S, nseg, d, I, xs.dtype)
    ws = torch.full((nbytes,), 0x5a, dtype=torch.uint8, device=DEV)
    h = moe.grouped_ffn(xs, offs, E, S, nseg, wl.w_gate.to(DEV), wl.w_up.to(DEV), wl.w_down.to(DEV),
                        h_sorted=_poison((xs.shape[0], d), xs.dtype), workspace=ws)
    torch.cuda.synchronize()
    assert int(ws[-4:].view(torch.int32).item()) == 0, "a tile-queue wait gave up"
    err = rel_max_err(f64_of(h), h_ref)
    assert err <= TOL[dtype], err
    # the same FFN reading the token rows through the permutation's row list
    # (gather folded into the loads) gives the same bits
    x_dev = wl.x.to(DEV)
    rows = torch.from_numpy(p_ref["sorted_token"]).to(DEV)
    h2 = moe.grouped_ffn(x_dev, offs, E, S, nseg, wl.w_gate.to(DEV), wl.w_up.to(DEV), wl.w_down.to(DEV),
                         h_sorted=_poison((xs.shape[0], d), xs.dtype), x_rows=rows)
    torch.cuda.synchronize()
    assert torch.equal(h2, h)


# ------------------------------------------------------------------ combine
COMBINE_CASES = [
    (64, 2, 0, 128, "f32"), (128, 8, 0, 2048, "bf16"), (256, 6, 2, 2048, "bf16"),
    (4160, 4, 0, 2880, "bf16"), (7, 3, 1, 24, "f32"), (1, 1, 0, 8, "bf16"),
]


@pytest.mark.parametrize("T,k,S,d,dtype", COMBINE_CASES)
def test_combine_parity(T, k, S, d, dtype):
    announce(f"combine T={T} k={k} S={S} d={d} {dtype}")
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    gen = torch.Generator().manual_seed(T * 31 + d)
    N = T * (k + S)
    h = torch.randn((N, d), generator=gen).to(tdt)
    f2s = torch.randperm(N, generator=gen).to(torch.int32)
    w = torch.rand((T, k), generator=gen)
    y_ref = O.combine(O.to_f64(np_of(h), dtype), f2s.numpy(), w.numpy(), T, k, S)
    y = moe.combine(h.to(DEV), f2s.to(DEV), w.to(DEV), S, y=_poison((T, d), tdt))
    torch.cuda.synchronize()
    assert rel_max_err(f64_of(y), y_ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_combine_identity_experts_k1_returns_input(dtype):
    """k = 1 and h_sorted := x_sorted: y equals x bit for bit."""
    announce(f"combine identity {dtype}")
    T, E, d = 300, 16, 64
    x = torch.randn((T, d), generator=torch.Generator().manual_seed(5)).to(dtype).to(DEV)
    lg = torch.randn((T, E), generator=torch.Generator().manual_seed(6)).to(DEV)
    ids, w = moe.gate(lg, 1)
    p = moe.permute(ids, E, 0, 0, x)
    y = moe.combine(p["x_sorted"], p["flat_to_sorted"], w, 0)
    torch.cuda.synchronize()
    assert torch.equal(y, x)


# ------------------------------------------------------------------ stats
STATS_CASES = [
    # (L, T, E, k, req_len, with_idf)
    (1, 64, 8, 2, 0, False), (8, 8192, 128, 8, 64, False), (1, 128, 64, 8, 1, False),
    (2, 300, 256, 4, 7, False), (1, 1000, 512, 6, 100, True), (3, 50, 5, 5, 3, False),
    (1, 0, 16, 2, 1, False),
    # several token splits with an odd E*E (scalar partial sums) and many requests
    (2, 3000, 129, 3, 5, False),
]


@pytest.mark.parametrize("L,T,E,k,req_len,with_idf", STATS_CASES)
def test_stats_parity(L, T, E, k, req_len, with_idf):
    announce(f"stats L={L} T={T} E={E} k={k} req_len={req_len} idf={with_idf}")
    ids = workloads.random_ids(T, E, k, seed=T + E, L=L)
    if req_len:
        offs = list(range(0, T, req_len)) + [T]
        if T == 0:
            offs = [0, 0]
    else:
        offs = [0, T]
    req = torch.tensor(offs, dtype=torch.int32)
    idf = torch.rand((L, E), generator=torch.Generator().manual_seed(3)) if with_idf else None
    ref = O.stats(ids.numpy(), E, req.numpy(), idf.numpy() if idf is not None else None)
    R = len(offs) - 1
    out = {"counts": _poison((L, E), torch.int32), "union_size": _poison(L, torch.int32),
           "union_mask": _poison((L, E), torch.uint8), "affinity": _poison((L, E, E), torch.int32),
           "req_counts": _poison((R, L, E), torch.int32), "signature": _poison((R, L, E), torch.float32)}
    got = moe.stats(ids.to(DEV), E, req.to(DEV), idf.to(DEV) if idf is not None else None, out=out)
    torch.cuda.synchronize()
    for key in ("counts", "union_size", "union_mask", "affinity", "req_counts"):
        np.testing.assert_array_equal(np_of(got[key]), ref[key], err_msg=key)
    sig, sref = np_of(got["signature"]).astype(np.float64), ref["signature"].astype(np.float64)
    assert np.all(np.abs(sig - sref) <= SIG_RTOL * np.abs(sref))


@pytest.mark.parametrize("L,T,E,k,seed", [(1, 2500, 96, 6, 1), (3, 700, 200, 4, 2), (1, 40, 16, 2, 3)])
def test_stats_irregular_requests(L, T, E, k, seed):
    """Requests of random lengths, empty ones included, that leave tokens at
    both ends of the batch outside every request."""
    announce(f"stats irregular L={L} T={T} E={E} k={k}")
    ids = workloads.random_ids(T, E, k, seed=seed, L=L)
    g = np.random.default_rng(seed)
    cuts = np.sort(g.integers(T // 10, T - T // 10, size=max(1, T // 30)))
    offs = np.concatenate([[T // 10], cuts, cuts[-1:], [T - T // 10]]).astype(np.int32)
    ref = O.stats(ids.numpy(), E, offs)
    got = moe.stats(ids.to(DEV), E, torch.from_numpy(offs).to(DEV))
    torch.cuda.synchronize()
    for key in ("counts", "union_size", "union_mask", "affinity", "req_counts"):
        np.testing.assert_array_equal(np_of(got[key]), ref[key], err_msg=key)
    sig, sref = np_of(got["signature"]).astype(np.float64), ref["signature"].astype(np.float64)
    assert np.all(np.abs(sig - sref) <= SIG_RTOL * np.abs(sref))


def test_stats_split_without_affinity():
    """Several token splits, no affinity output: counts and union still exact."""
    ids = workloads.random_ids(5000, 200, 4, seed=11, L=2)
    ref = O.stats(ids.numpy(), 200)
    got = moe.stats(ids.to(DEV), 200, None, affinity=False)
    torch.cuda.synchronize()
    for key in ("counts", "union_size", "union_mask"):
        np.testing.assert_array_equal(np_of(got[key]), ref[key], err_msg=key)


def test_stats_without_optional_outputs():
    ids = workloads.random_ids(200, 32, 4, seed=9, L=2)
    ref = O.stats(ids.numpy(), 32)
    got = moe.stats(ids.to(DEV), 32, None, affinity=False)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(np_of(got["counts"]), ref["counts"])
    np.testing.assert_array_equal(np_of(got["union_size"]), ref["union_size"])


QUEUE_CASES = [
    # (T, E, k, S, P, d, I, kind): priority segment, groups averaging > 48 rows,
    # so both phases run in the one persistent launch
    (600, 8, 2, 0, 50, 256, 320, "random"),       # GEMM units only, column tail in I
    (4160, 128, 4, 0, 64, 256, 320, "zipf"),      # GPT-OSS-like routing: many one-unit experts, a few large
    (2000, 64, 4, 2, 300, 128, 96, "zipf"),       # shared experts, many priority units
    (1300, 512, 4, 256, 10, 64, 32, "random"),    # 768 sequences: one block per CU fits in LDS
]


@pytest.mark.parametrize("packed", [False, True], ids=["rowmajor", "packed"])
@pytest.mark.parametrize("T,E,k,S,P,d,I,kind", QUEUE_CASES)
def test_grouped_ffn_queue_path(T, E, k, S, P, d, I, kind, packed):
    """The persistent single-launch FFN (device-side tile queues, priority
    tiles first), on row-major and on pre-packed weights: every row within the
    bf16 tolerance of the oracle, the diagnostic word 0, the two-launch path
    within the tolerance too, and a per-tile timeline in which every tile ran
    once, the priority units' phase-1 tiles were popped first in each queue,
    and every phase-2 tile ended after every phase-1 tile of its unit."""
    import os
    announce(f"ffn queue T={T} E={E} k={k} S={S} P={P} d={d} I={I} {kind} packed={packed}")
    wl, ids = _ffn_inputs(T, E, k, S, P, d, I, "bf16", kind, seed=T + E + 11)
    p_ref = O.permute(ids.numpy(), E, S, P, np_of(wl.x))
    N = int(p_ref["group_offsets"][-1])
    h_ref = O.grouped_ffn(p_ref["x_sorted"], p_ref["group_offsets"], E, S, 2, np_of(wl.w_gate),
                          np_of(wl.w_up), np_of(wl.w_down), "bf16")
    offs = torch.from_numpy(p_ref["group_offsets"]).to(DEV)
    rows = torch.from_numpy(p_ref["sorted_token"]).to(DEV)
    w = [t.to(DEV) for t in (wl.w_gate, wl.w_up, wl.w_down)]
    if packed:
        w = [moe.pack_weights(t) for t in w]
    ffn = moe.grouped_ffn_packed if packed else moe.grouped_ffn
    x = wl.x.to(DEV)
    nbytes = moe.ffn_workspace_bytes(N, E, S, 2, d, I)
    ws = torch.full((nbytes,), 0x5a, dtype=torch.uint8, device=DEV)
    trace = torch.zeros((1 << 16, 4), dtype=torch.int64, device=DEV)
    h = ffn(x, offs, E, S, 2, *w, h_sorted=_poison((N, d), torch.bfloat16), workspace=ws, x_rows=rows, trace=trace)
    torch.cuda.synchronize()
    assert int(ws[-4:].view(torch.int32).item()) == 0, "a tile-queue wait gave up"
    err = rel_max_err(f64_of(h), h_ref)
    assert err <= TOL["bf16"], err
    os.environ["LIBMOE_FFN_QUEUE"] = "0"
    try:
        h2 = ffn(x, offs, E, S, 2, *w, h_sorted=_poison((N, d), torch.bfloat16), x_rows=rows)
        torch.cuda.synchronize()
    finally:
        os.environ.pop("LIBMOE_FFN_QUEUE", None)
    # the two-launch path (GEMM tiles for every group) is checked against the
    # oracle too; the persistent path streams small experts' weights on the
    # decode-shaped MFMA, so the two agree within the tolerance, not bit for bit
    err2 = rel_max_err(f64_of(h2), h_ref)
    assert err2 <= TOL["bf16"], err2
    # the timeline
    tr = trace.cpu().numpy().view(np.uint64)
    rec = tr[tr[:, 1] != 0]
    assert len(rec) > 0
    assert np.all(rec[:, 1] >= rec[:, 0])
    info = rec[:, 2]
    phase = (info & 1).astype(np.int64) + 1
    prio = ((info >> 1) & 1).astype(np.int64)
    chunk = ((info >> 8) & 0xFFFFFF).astype(np.int64)
    unit = (info >> 32).astype(np.int64)
    keys = set(zip(phase.tolist(), unit.tolist(), chunk.tolist()))
    assert len(keys) == len(rec), "a tile ran twice"
    nq = 8                                    # one queue per group of blocks, both tile kinds
    per_q = trace.shape[0] // nq
    slot = np.nonzero(tr[:, 1] != 0)[0]
    q_of, t_of = slot // per_q, slot % per_q
    assert np.array_equal(q_of, (rec[:, 3] >> 32).astype(np.int64)), "record in another queue's slots"
    assert np.array_equal((rec[:, 3] & 0xFFFFFFFF).astype(np.int64) % nq, q_of), "block took another group's queue"
    for q in range(nq):
        sel = q_of == q
        if not sel.any():
            continue
        t_sorted = np.sort(t_of[sel])
        assert len(t_sorted) < per_q, "trace too small for this queue"
        assert np.array_equal(t_sorted, np.arange(len(t_sorted))), "queue positions are not contiguous"
        p1 = t_of[sel & (phase == 1) & (prio == 1)]
        if len(p1):
            assert p1.max() == len(p1) - 1, "priority phase-1 tiles are not first in their queue"
    end1 = {}
    for u, e in zip(unit[phase == 1].tolist(), rec[phase == 1, 1].tolist()):
        end1[u] = max(end1.get(u, 0), e)
    for u, e in zip(unit[phase == 2].tolist(), rec[phase == 2, 1].tolist()):
        assert e > end1[u], "a phase-2 tile ended before a phase-1 tile of its unit"


COMBINE_CASES = [
    # (T, E, k, S, P, d, I): decode-shaped batches (groups averaging <= 48 rows)
    (16, 64, 6, 2, 0, 256, 128),      # groups of ~2 rows: the split-K kernel
    (96, 16, 4, 1, 0, 136, 200),      # 32-row tiles, d and I not multiples of 32, a column tail
    (100, 16, 4, 0, 30, 128, 96),     # priority segment: two row ranges per tile
    (300, 32, 4, 0, 0, 256, 192),     # 64-row tiles
    (128, 64, 8, 0, 0, 2048, 1024),   # OLMoE decode shape
]


@pytest.mark.parametrize("packed", [False, True], ids=["rowmajor", "packed"])
@pytest.mark.parametrize("T,E,k,S,P,d,I", COMBINE_CASES)
def test_grouped_ffn_combine_parity(T, E, k, S, P, d, I, packed):
    """moe_grouped_ffn_combine (the combine folded into the down projection):
    every token of y within the bf16 tolerance of the oracle's FFN + combine
    and of the two-call GPU path, twice on one workspace (the second call
    starts from its own cleared sums)."""
    if packed and (d % 32 or I % 32):
        pytest.skip("packed weights need d and I multiples of 32")
    announce(f"ffn+combine T={T} E={E} k={k} S={S} P={P} d={d} I={I} packed={packed}")
    wl, ids = _ffn_inputs(T, E, k, S, P, d, I, "bf16", "random", seed=T + E + 5)
    nseg = 2 if P > 0 else 1
    g = torch.Generator().manual_seed(T * 3 + k)
    w = torch.rand((T, k), generator=g) + 0.05
    w = (w / w.sum(dim=1, keepdim=True)).to(torch.float32)
    p_ref = O.permute(ids.numpy(), E, S, P, np_of(wl.x))
    h_ref = O.grouped_ffn(p_ref["x_sorted"], p_ref["group_offsets"], E, S, nseg, np_of(wl.w_gate),
                          np_of(wl.w_up), np_of(wl.w_down), "bf16")
    y_ref = O.combine(h_ref, p_ref["flat_to_sorted"], w.numpy(), T, k, S)
    wts = [t.to(DEV) for t in (wl.w_gate, wl.w_up, wl.w_down)]
    if packed:
        wts = [moe.pack_weights(t) for t in wts]
    x = wl.x.to(DEV)
    offs = torch.from_numpy(p_ref["group_offsets"]).to(DEV)
    rows = torch.from_numpy(p_ref["sorted_token"]).to(DEV)
    s2f = torch.from_numpy(p_ref["sorted_to_flat"]).to(DEV)
    f2s = torch.from_numpy(p_ref["flat_to_sorted"]).to(DEV)
    wd = w.to(DEV)
    nbytes = moe.ffn_combine_workspace_bytes(T * (k + S), E, S, nseg, d, I, T, k, packed)
    ws = torch.full((nbytes,), 0x5a, dtype=torch.uint8, device=DEV)
    for rep in range(2):
        y = moe.grouped_ffn_combine(x, offs, E, S, nseg, *wts, s2f, wd, y=_poison((T, d), torch.bfloat16),
                                    workspace=ws, x_rows=rows, packed=packed)
        torch.cuda.synchronize()
        assert int(ws[-4:].view(torch.int32).item()) == 0
        err = rel_max_err(f64_of(y), y_ref)
        assert err <= TOL["bf16"], (rep, err)
    ffn = moe.grouped_ffn_packed if packed else moe.grouped_ffn
    h = ffn(x, offs, E, S, nseg, *wts, x_rows=rows)
    y2 = moe.combine(h, f2s, wd, S)
    torch.cuda.synchronize()
    assert rel_max_err(f64_of(y), f64_of(y2)) <= TOL["bf16"]


def test_grouped_ffn_combine_refuses_prefill_batches():
    with pytest.raises(moe.MoeError):
        moe.ffn_combine_workspace_bytes(65536, 128, 0, 1, 2048, 768, 8192, 8)


# ------------------------------------------------------------------ KV-block signature recording
def test_kv_block_recording_and_host_staging():
    """Expert counts per 16-token KV block over the Qwen3-shaped 8-layer id stack,
    staged into pinned host memory: equal to the oracle's per-block counts, and
    a request's counts are the sum of its blocks' (the blocks tile the request)."""
    wl = workloads.make("qwen3_prefill", DEV, with_weights=False)
    s = wl.spec
    announce("kv-block recording")
    ids = torch.stack([moe.gate(wl.stats_logits[l].contiguous(), s.k)[0] for l in range(s.stats_layers)])
    block = 16
    boffs = torch.arange(0, s.T + 1, block, dtype=torch.int32, device=DEV)
    o = moe.stats(ids.contiguous(), s.E, boffs, affinity=False, signature=False)
    host = torch.empty(o["req_counts"].shape, dtype=torch.int32, pin_memory=True)
    host.copy_(o["req_counts"], non_blocking=True)
    torch.cuda.synchronize()
    ids_np = np_of(ids)
    ref = O.stats(ids_np, s.E, np_of(boffs))
    np.testing.assert_array_equal(host.numpy(), ref["req_counts"])
    req = O.stats(ids_np, s.E, np_of(wl.req_offsets))["req_counts"]
    ro = np_of(wl.req_offsets)
    summed = np.stack([host.numpy()[ro[r] // block:ro[r + 1] // block].sum(axis=0) for r in range(len(ro) - 1)])
    np.testing.assert_array_equal(summed, req)


# ------------------------------------------------------------------ continuous signature
def _prob_sig_case(L, T, E, seed):
    g = torch.Generator().manual_seed(seed)
    lg = torch.randn((L, T, E), generator=g) * 3.0
    cuts = sorted(torch.randint(0, T + 1, (5,), generator=g).tolist())
    offs = torch.tensor([0] + cuts + [T], dtype=torch.int32)
    return lg, offs


@pytest.mark.parametrize("L,T,E,seed", [(1, 1, 1, 0), (3, 600, 70, 1), (2, 40, 512, 2), (4, 257, 9, 3)])
def test_prob_signature_parity(L, T, E, seed):
    announce(f"prob signature L={L} T={T} E={E}")
    lg, offs = _prob_sig_case(L, T, E, seed)
    if T > 3:                       # special rows: one finite logit, NaNs, all -inf
        lg[0, 1, :] = -float("inf")
        lg[0, 1, 0] = 2.0
        lg[0, 2, ::2] = float("nan")
        lg[0, 3, :] = -float("inf")
    ref = O.prob_signature(lg.numpy(), offs.numpy())
    out = _poison(ref.shape, torch.float32)
    moe.prob_signature(lg.to(DEV), offs.to(DEV), out)
    torch.cuda.synchronize()
    got = np_of(out).astype(np.float64)
    # everything in double, one rounding to fp32 at the end: within 4 ulp of fp32
    assert np.all(np.abs(got - ref) <= 2.0 ** -22 * np.abs(ref) + 1e-30), float(np.max(np.abs(got - ref)))


def test_prob_signature_qwen3_stack():
    wl = workloads.make("qwen3_prefill", DEV, with_weights=False)
    announce("prob signature qwen3 stack")
    lg = wl.stats_logits.contiguous()
    out = moe.prob_signature(lg, wl.req_offsets)
    torch.cuda.synchronize()
    ref = O.prob_signature(np_of(lg), np_of(wl.req_offsets))
    got = np_of(out).astype(np.float64)
    assert np.all(np.abs(got - ref) <= 2.0 ** -22 * np.abs(ref) + 1e-30)
    sizes = np.diff(np_of(wl.req_offsets)).astype(np.float64)
    assert np.allclose(got.sum(axis=2), sizes[:, None], rtol=1e-5)


# ------------------------------------------------------------------ FP8-weight expert FFN
FP8_CASES = [
    # (T, E, k, S, P, d, I, kind)
    (128, 64, 8, 0, 0, 2048, 1024, "random"),   # OLMoE decode shape: 32-row tiles, 512-wide K chunks
    (16, 64, 6, 2, 0, 2048, 1408, "zipf"),      # DSv2-Lite decode shape: 16-row tiles, shared experts
    (96, 16, 4, 0, 0, 144, 208, "random"),      # K tails (144 = 128 + 16) and column tails in both phases
    (300, 8, 2, 1, 20, 256, 192, "random"),     # 64-row tiles (256-wide chunks), priority segment + shared
    (100, 16, 4, 0, 30, 128, 96, "random"),     # 32-row tiles (384-wide chunks) with a priority segment
    (64, 512, 8, 2, 0, 64, 48, "random"),       # the most routed experts, two shared, K shorter than a chunk
    (80, 512, 4, 2, 30, 32, 16, "zipf"),        # 1026 groups (priority segment at E = 512), one column chunk
    (1, 4, 1, 0, 0, 16, 16, "random"),          # one token, the smallest d and I
]


FP8_GEMM_CASES = [
    # (T, E, k, S, P, d, I, kind): packed codes, groups averaging > 48 rows ->
    # the 256 x 256 GEMM on FP8 codes
    (600, 8, 2, 0, 0, 256, 320, "random"),     # partial m-tiles, a half column chunk in phase 1
    (2048, 16, 4, 0, 0, 512, 256, "random"),   # ~512 rows per expert: two full m-tiles each
    (1500, 8, 3, 1, 0, 192, 448, "random"),    # a shared expert of 1500 rows, K = 192 (three code blocks)
    (3000, 32, 2, 0, 0, 128, 128, "zipf"),     # one hot expert, many nearly empty ones
    (600, 8, 2, 0, 50, 256, 320, "random"),    # a priority segment (its groups are tiles of their own)
    (2000, 64, 4, 2, 300, 128, 192, "zipf"),   # priority segment, two shared experts, Zipf routing
]


@pytest.mark.parametrize("T,E,k,S,P,d,I,kind", FP8_GEMM_CASES)
def test_grouped_ffn_fp8w_gemm_parity(T, E, k, S, P, d, I, kind):
    """FP8 codes on the GEMM (pre-packed codes, prefill-sized groups): every
    row within the bf16 tolerance of the oracle's FP8 FFN, directly and through
    the row list, and of the decode-shaped FP8 kernel on row-major codes."""
    announce(f"ffn fp8 gemm T={T} E={E} k={k} S={S} P={P} d={d} I={I} {kind}")
    wl, ids = _ffn_inputs(T, E, k, S, P, d, I, "bf16", kind, seed=T + E + 9)
    nseg = 2 if P > 0 else 1
    q = [moe.quantize_fp8_rows(w) for w in (wl.w_gate, wl.w_up, wl.w_down)]
    p_ref = O.permute(ids.numpy(), E, S, P, np_of(wl.x))
    h_ref = O.grouped_ffn_fp8w(p_ref["x_sorted"], p_ref["group_offsets"], E, S, nseg, q[0][0].numpy(),
                               q[0][1].numpy(), q[1][0].numpy(), q[1][1].numpy(), q[2][0].numpy(), q[2][1].numpy(),
                               "bf16")
    offs = torch.from_numpy(p_ref["group_offsets"]).to(DEV)
    rows = torch.from_numpy(p_ref["sorted_token"]).to(DEV)
    packed = []
    for c, sc in q:
        packed += [moe.pack_fp8_codes(c.to(DEV)), sc.to(DEV)]
    N = int(p_ref["group_offsets"][-1])
    nbytes = moe.ffn_fp8w_workspace_bytes(N, I, E, S, nseg, d, packed=True)
    ws = torch.full((max(nbytes, 256),), 0x5a, dtype=torch.uint8, device=DEV)
    h = moe.grouped_ffn_fp8w(wl.x.to(DEV), offs, E, S, nseg, *packed, h_sorted=_poison((N, d), torch.bfloat16),
                             workspace=ws, x_rows=rows, packed=True)
    torch.cuda.synchronize()
    assert int(ws[nbytes - 4:nbytes].view(torch.int32).item()) == 0
    err = rel_max_err(f64_of(h), h_ref)
    assert err <= TOL["bf16"], err
    xs = torch.from_numpy(p_ref["x_sorted"].view(np.int16)).view(torch.bfloat16).to(DEV)
    h2 = moe.grouped_ffn_fp8w(xs, offs, E, S, nseg, *packed, h_sorted=_poison((N, d), torch.bfloat16), packed=True)
    torch.cuda.synchronize()
    assert torch.equal(h2, h)
    rowmajor = [t.to(DEV) for pair in q for t in pair]
    h3 = moe.grouped_ffn_fp8w(wl.x.to(DEV), offs, E, S, nseg, *rowmajor, x_rows=rows)
    torch.cuda.synchronize()
    assert rel_max_err(f64_of(h3), f64_of(h)) <= TOL["bf16"]


@pytest.mark.parametrize("T,E,k,S,P,d,I,kind", FP8_CASES)
def test_grouped_ffn_fp8w_parity(T, E, k, S, P, d, I, kind):
    announce(f"ffn fp8 T={T} E={E} k={k} S={S} P={P} d={d} I={I} {kind}")
    wl, ids = _ffn_inputs(T, E, k, S, P, d, I, "bf16", kind, seed=T + E + 7)
    nseg = 2 if P > 0 else 1
    qg, sg = moe.quantize_fp8_rows(wl.w_gate)
    qu, su = moe.quantize_fp8_rows(wl.w_up)
    qd, sd = moe.quantize_fp8_rows(wl.w_down)
    p_ref = O.permute(ids.numpy(), E, S, P, np_of(wl.x))
    h_ref = O.grouped_ffn_fp8w(p_ref["x_sorted"], p_ref["group_offsets"], E, S, nseg, qg.numpy(), sg.numpy(),
                               qu.numpy(), su.numpy(), qd.numpy(), sd.numpy(), "bf16")
    xs = torch.from_numpy(p_ref["x_sorted"].view(np.int16)).view(torch.bfloat16).to(DEV)
    offs = torch.from_numpy(p_ref["group_offsets"]).to(DEV)
    h = moe.grouped_ffn_fp8w(xs, offs, E, S, nseg, qg.to(DEV), sg.to(DEV), qu.to(DEV), su.to(DEV), qd.to(DEV),
                             sd.to(DEV), h_sorted=_poison((xs.shape[0], d), torch.bfloat16))
    torch.cuda.synchronize()
    err = rel_max_err(f64_of(h), h_ref)
    assert err <= TOL["bf16"], err
    # through the row list: the same bits
    rows = torch.from_numpy(p_ref["sorted_token"]).to(DEV)
    h2 = moe.grouped_ffn_fp8w(wl.x.to(DEV), offs, E, S, nseg, qg.to(DEV), sg.to(DEV), qu.to(DEV), su.to(DEV),
                              qd.to(DEV), sd.to(DEV), h_sorted=_poison((xs.shape[0], d), torch.bfloat16), x_rows=rows)
    torch.cuda.synchronize()
    assert torch.equal(h2, h)
    if d % 64 == 0 and I % 64 == 0:
        h3 = moe.grouped_ffn_fp8w(wl.x.to(DEV), offs, E, S, nseg, moe.pack_fp8_codes(qg.to(DEV)), sg.to(DEV),
                                  moe.pack_fp8_codes(qu.to(DEV)), su.to(DEV), moe.pack_fp8_codes(qd.to(DEV)),
                                  sd.to(DEV), h_sorted=_poison((xs.shape[0], d), torch.bfloat16), x_rows=rows,
                                  packed=True)
        torch.cuda.synchronize()
        G = nseg * E + S
        if xs.shape[0] // G > 48 and d >= 128 and I >= 128:
            # prefill-sized groups on packed codes run on the FP8 GEMM: other sum order
            assert rel_max_err(f64_of(h3), h_ref) <= TOL["bf16"]
        else:
            # pre-packed codes on the same kernel: the same products in the same order, so the same bits
            assert torch.equal(h3, h)


def test_ffn_bindings_reject_mismatched_shapes():
    """The FFN bindings refuse weights, scales, offsets or outputs whose shapes do
    not match the call's sizes (before anything is enqueued)."""
    E, S, d, I, N = 4, 1, 32, 48, 10
    dev = DEV
    x = torch.zeros((N, d), dtype=torch.bfloat16, device=dev)
    offs = torch.zeros(E + S + 1, dtype=torch.int32, device=dev)
    wg = torch.zeros((E + S, I, d), dtype=torch.bfloat16, device=dev)
    wd = torch.zeros((E + S, d, I), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        moe.grouped_ffn(x, offs, E, S, 1, wg, wg, wg)                     # down has the wrong shape
    with pytest.raises(ValueError):
        moe.grouped_ffn(x, offs[:-1], E, S, 1, wg, wg, wd)                # too few offsets
    with pytest.raises(ValueError):
        moe.grouped_ffn(x, offs, E, S, 1, wg, wg, wd, h_sorted=torch.empty((N - 1, d), dtype=torch.bfloat16,
                                                                           device=dev))
    qg = torch.zeros((E + S, I, d), dtype=torch.uint8, device=dev)
    qd = torch.zeros((E + S, d, I), dtype=torch.uint8, device=dev)
    sg = torch.ones((E + S, I), dtype=torch.float32, device=dev)
    sd = torch.ones((E + S, d), dtype=torch.float32, device=dev)
    with pytest.raises(ValueError):
        moe.grouped_ffn_fp8w(x, offs, E, S, 1, qg, sg, qg, sg, qg, sd)    # down codes have the wrong shape
    with pytest.raises(ValueError):
        moe.grouped_ffn_fp8w(x, offs, E, S, 1, qg, sg, qg, sg, qd, sg)    # down scales have the wrong shape
    with pytest.raises(ValueError):
        moe.grouped_ffn_fp8w(x, offs, E + 1, S, 1, qg, sg, qg, sg, qd, sd)  # E does not match the weights
    with pytest.raises(ValueError):
        moe.grouped_ffn_fp8w(x, offs, E, S, 1, qg, sg, qg, sg, qd, sd,
                             h_sorted=torch.empty((N, d + 16), dtype=torch.bfloat16, device=dev))


def test_bindings_reject_mismatched_outputs():
    """Caller-supplied outputs of the wrong shape (or inputs whose sizes disagree)
    are refused before anything is enqueued."""
    T, E, k, d = 8, 16, 2, 32
    dev = DEV
    logits = torch.zeros((T, E), dtype=torch.float32, device=dev)
    ids = torch.zeros((T, k), dtype=torch.int32, device=dev)
    with pytest.raises(ValueError):
        moe.gate(logits, k, True, ids, torch.empty((T, k + 1), dtype=torch.float32, device=dev))
    with pytest.raises(ValueError):
        moe.gate(logits, k, True, torch.empty((T - 1, k), dtype=torch.int32, device=dev))
    with pytest.raises(ValueError):
        moe.permute(ids, E, x=torch.zeros((T + 1, d), dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError):
        moe.permute(ids, E, out={"group_offsets": torch.empty(E, dtype=torch.int32, device=dev)})
    with pytest.raises(ValueError):
        moe.stats(ids.view(1, T, k), E, out={"counts": torch.empty((1, E - 1), dtype=torch.int32, device=dev)})
    offs = torch.tensor([0, 4, 8], dtype=torch.int32, device=dev)
    with pytest.raises(ValueError):
        moe.prob_signature(logits.view(1, T, E), offs, torch.empty((2, 1, E + 1), dtype=torch.float32, device=dev))
    with pytest.raises(ValueError):
        moe.router(torch.zeros((T, d), dtype=torch.bfloat16, device=dev),
                   torch.zeros((E, d), dtype=torch.bfloat16, device=dev), torch.empty((T, E - 1), device=dev))


PACKED_CASES = [
    # (T, E, k, S, P, d, I, kind)
    (128, 64, 8, 0, 0, 2048, 1024, "random"),   # OLMoE decode shape: 32-row tiles
    (256, 64, 6, 2, 0, 2048, 1408, "zipf"),     # DSv2-Lite T=256 shape: 64-row tiles, shared experts
    (16, 64, 6, 2, 0, 2048, 1408, "zipf"),      # DSv2-Lite T=16 shape: split-K kernel
    (24, 16, 2, 1, 6, 96, 160, "random"),       # split-K with a priority segment and a shared expert
    (300, 8, 2, 0, 20, 256, 192, "random"),     # 64-row tiles with a priority segment, column tail
    (4, 512, 4, 256, 2, 64, 32, "random"),      # the largest group count (1280)
    # GEMM-sized groups: the GEMM kernels copy the packed blocks into LDS
    (300, 8, 2, 0, 0, 256, 192, "random"),      # 128 x 256 tiles, column tail in I
    (2000, 8, 2, 0, 0, 256, 320, "random"),     # 256 x 256 persistent tiles, column tail in I
    (4160, 128, 4, 0, 64, 256, 320, "zipf"),    # priority segment: the persistent queue (GEMM + stream tiles)
    (1300, 512, 4, 256, 10, 64, 32, "random"),  # the largest group count on the queue
]


@pytest.mark.parametrize("T,E,k,S,P,d,I,kind", PACKED_CASES)
def test_grouped_ffn_packed_parity(T, E, k, S, P, d, I, kind):
    """Pre-packed weights: every row within the bf16 tolerance of the oracle, and
    bit for bit the unpacked call's result (the same products in the same
    order, only read from other addresses), directly and through the row list."""
    announce(f"ffn packed T={T} E={E} k={k} S={S} P={P} d={d} I={I} {kind}")
    wl, ids = _ffn_inputs(T, E, k, S, P, d, I, "bf16", kind, seed=T + E + 3)
    nseg = 2 if P > 0 else 1
    p_ref = O.permute(ids.numpy(), E, S, P, np_of(wl.x))
    N = int(p_ref["group_offsets"][-1])
    h_ref = O.grouped_ffn(p_ref["x_sorted"], p_ref["group_offsets"], E, S, nseg, np_of(wl.w_gate),
                          np_of(wl.w_up), np_of(wl.w_down), "bf16")
    xs = torch.from_numpy(p_ref["x_sorted"].view(np.int16)).view(torch.bfloat16).to(DEV)
    offs = torch.from_numpy(p_ref["group_offsets"]).to(DEV)
    w = [t.to(DEV) for t in (wl.w_gate, wl.w_up, wl.w_down)]
    wp = [moe.pack_weights(t) for t in w]
    h_plain = moe.grouped_ffn(xs, offs, E, S, nseg, *w, h_sorted=_poison((N, d), torch.bfloat16))
    h = moe.grouped_ffn_packed(xs, offs, E, S, nseg, *wp, h_sorted=_poison((N, d), torch.bfloat16))
    tok = torch.from_numpy(p_ref["sorted_token"]).to(DEV)
    h2 = moe.grouped_ffn_packed(wl.x.to(DEV), offs, E, S, nseg, *wp, h_sorted=_poison((N, d), torch.bfloat16),
                                x_rows=tok)
    torch.cuda.synchronize()
    err = rel_max_err(f64_of(h), h_ref)
    assert err <= TOL["bf16"], err
    assert torch.equal(h, h_plain)
    assert torch.equal(h2, h)

"""The C ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before touching a GPU (CPU-only; no compute calls)."""
import ctypes
import os
import re

import pytest

import top_expert_routing_amd as m
from top_expert_routing_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libmoe.h")

INV, UNS, WS = _lib.MOE_ERR_INVALID_ARG, _lib.MOE_ERR_UNSUPPORTED, _lib.MOE_ERR_WORKSPACE
FAKE = 1 << 20          # a non-NULL, 16-byte aligned address that is never dereferenced


@pytest.fixture(scope="module")
def lib():
    return m.load()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:moe_status|const char\*)\s+(moe_\w+)\s*\(", text, re.M)))


def test_header_declares_the_calls():
    assert _declared() == sorted(["moe_router", "moe_gate", "moe_gate_record", "moe_stage_to_host", "moe_permute",
                                  "moe_grouped_ffn", "moe_grouped_ffn_traced", "moe_grouped_ffn_combine",
                                  "moe_grouped_ffn_noalloc",
                                  "moe_grouped_ffn_packed", "moe_grouped_ffn_fp8w", "moe_grouped_ffn_fp8w_packed",
                                  "moe_combine", "moe_stats", "moe_prob_signature", "moe_status_string"])


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    assert tuple(sorted(_lib.EXPORTS)) == tuple(_declared())


def test_status_strings(lib):
    for code, name in _lib.STATUS_NAMES.items():
        assert lib.moe_status_string(code).decode() == name
    assert lib.moe_status_string(99).decode() == "MOE_ERR_UNKNOWN"


def test_router_validation(lib):
    f = lib.moe_router
    assert f(FAKE, FAKE, -1, 64, 8, _lib.MOE_BF16, FAKE, None) == INV
    assert f(FAKE, FAKE, 4, 64, 0, _lib.MOE_BF16, FAKE, None) == INV
    assert f(FAKE, FAKE, 4, 0, 8, _lib.MOE_BF16, FAKE, None) == INV
    assert f(FAKE, FAKE, 4, 60, 8, _lib.MOE_BF16, FAKE, None) == UNS          # d not a multiple of 8
    assert f(FAKE, FAKE, 4, 64, 513, _lib.MOE_BF16, FAKE, None) == UNS        # E > 512
    assert f(FAKE, FAKE, 4, 64, 8, 7, FAKE, None) == UNS                      # unknown dtype
    assert f(FAKE, FAKE, 1 << 20, 1 << 12, 8, _lib.MOE_BF16, FAKE, None) == UNS   # T*d overflows int32
    assert f(None, FAKE, 4, 64, 8, _lib.MOE_BF16, FAKE, None) == INV
    assert f(FAKE, None, 4, 64, 8, _lib.MOE_BF16, FAKE, None) == INV
    assert f(FAKE, FAKE, 4, 64, 8, _lib.MOE_BF16, None, None) == INV
    assert f(FAKE + 4, FAKE, 4, 64, 8, _lib.MOE_BF16, FAKE, None) == INV      # misaligned
    assert f(None, None, 0, 64, 8, _lib.MOE_BF16, None, None) == 0            # T = 0: nothing to do


def test_prob_signature_validation(lib):
    f = lib.moe_prob_signature
    assert f(FAKE, 0, 4, 8, FAKE, 2, FAKE, None) == INV                # L < 1
    assert f(FAKE, 1, -1, 8, FAKE, 2, FAKE, None) == INV               # T < 0
    assert f(FAKE, 1, 4, 0, FAKE, 2, FAKE, None) == INV                # E < 1
    assert f(FAKE, 1, 4, 8, FAKE, -1, FAKE, None) == INV               # R < 0
    assert f(FAKE, 1, 4, 513, FAKE, 2, FAKE, None) == UNS              # E > 512
    assert f(FAKE, 1 << 12, 1 << 12, 512, FAKE, 2, FAKE, None) == UNS  # L*T*E overflows int32
    assert f(FAKE, 1, 4, 8, None, 2, FAKE, None) == INV                # NULL offsets
    assert f(FAKE, 1, 4, 8, FAKE, 2, None, None) == INV                # NULL output
    assert f(None, 1, 4, 8, FAKE, 2, FAKE, None) == INV                # NULL logits with T > 0
    assert f(FAKE + 2, 1, 4, 8, FAKE, 2, FAKE, None) == INV            # misaligned
    assert f(None, 1, 4, 8, None, 0, None, None) == 0                  # R = 0: nothing to do


def test_ffn_fp8w_validation_and_query(lib):
    f = lib.moe_grouped_ffn_fp8w
    n = ctypes.c_size_t(0)
    args = lambda **kw: [kw.get(f"a{i}", v) for i, v in enumerate(
        [FAKE, None, 0, FAKE, 64, 8, 0, 1, 256, 512, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
         ctypes.byref(n), None])]
    assert f(*args()) == 0 and n.value >= 64 * 512 * 2           # query
    assert f(*args(a8=264)) == UNS                                 # d not a multiple of 16
    assert f(*args(a9=520)) == UNS                                 # I not a multiple of 16
    assert f(*args(a7=3)) == INV                                   # nseg
    assert f(*args(a7=2)) == 0                                     # a priority segment: same query
    assert f(*args(a5=513)) == UNS                                 # E > 512
    small = ctypes.c_size_t(16)
    assert f(*args(a17=FAKE, a18=ctypes.byref(small))) == WS       # workspace too small
    big = ctypes.c_size_t(1 << 30)
    assert f(*args(a17=FAKE, a18=ctypes.byref(big), a11=None)) == INV   # NULL scale
    assert f(*args(a17=FAKE, a18=ctypes.byref(big), a10=FAKE + 8)) == INV   # misaligned weights
    fp = lib.moe_grouped_ffn_fp8w_packed
    assert fp(*args()) == 0                                        # d = 256, I = 512: multiples of 64
    assert fp(*args(a8=272)) == UNS                                # d a multiple of 16 but not of 64
    assert fp(*args(a9=528)) == UNS                                # I a multiple of 16 but not of 64
    assert fp(*args(a7=2)) == 0                                    # a priority segment, decode-sized groups
    assert fp(*args(a7=2, a4=8192)) == 0                           # ... and GEMM-sized ones


def test_ffn_fp8w_packed_workspace_follows_the_path(lib, monkeypatch):
    """The packed FP8 call reserves the persistent queue's heads and phase-1
    flags (the same layout as the bf16 call's) exactly when a batch with a
    priority segment runs in the queue: packed codes, groups of 49-255 rows
    on average, d and I multiples of 64 and at least 128.  Otherwise the
    workspace is the bf16 SwiGLU intermediate plus the diagnostic word."""
    def fp8(packed, n_rows, nseg, d=256, I=512, E=8):
        n = ctypes.c_size_t(0)
        f = lib.moe_grouped_ffn_fp8w_packed if packed else lib.moe_grouped_ffn_fp8w
        assert f(FAKE, None, 0, FAKE, n_rows, E, 0, nseg, d, I, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                 ctypes.byref(n), None) == 0
        return n.value

    def bf16(n_rows, nseg, d=256, I=512, E=8):
        n = ctypes.c_size_t(0)
        assert lib.moe_grouped_ffn_packed(FAKE, None, 0, FAKE, n_rows, E, 0, nseg, d, I, FAKE, FAKE, FAKE, FAKE,
                                          None, ctypes.byref(n), None) == 0
        return n.value

    plain = lambda n_rows, I=512: (n_rows * I * 2 + 255) // 256 * 256 + 256
    G2 = 2 * 8
    queue_rows = 100 * G2                          # 100 rows per group on average
    assert fp8(True, queue_rows, 2) == bf16(queue_rows, 2) > plain(queue_rows)
    assert fp8(True, queue_rows, 1) == plain(queue_rows)          # no priority segment: two launches
    assert fp8(False, queue_rows, 2) == plain(queue_rows)         # row-major codes: decode-shaped kernel
    assert fp8(True, 300 * G2, 2) == plain(300 * G2)              # 256-row tiles: two launches
    assert fp8(True, 40 * G2, 2) == plain(40 * G2)                # decode-sized groups
    assert fp8(True, queue_rows, 2, d=64) == plain(queue_rows)    # K below 128 in phase 2
    monkeypatch.setenv("LIBMOE_FFN_QUEUE", "0")
    assert fp8(True, queue_rows, 2) == bf16(queue_rows, 2) == plain(queue_rows)


def test_ffn_packed_validation_and_query(lib):
    f = lib.moe_grouped_ffn_packed
    n = ctypes.c_size_t(0)
    args = lambda **kw: [kw.get(f"a{i}", v) for i, v in enumerate(
        [FAKE, None, 0, FAKE, 64, 8, 0, 1, 256, 512, FAKE, FAKE, FAKE, FAKE, None, ctypes.byref(n), None])]
    assert f(*args()) == 0 and n.value >= 64 * 512 * 2            # query (workspace of moe_grouped_ffn)
    assert f(*args(a8=272)) == UNS                                 # d not a multiple of 32
    assert f(*args(a9=528)) == UNS                                 # I not a multiple of 32
    assert f(*args(a4=49 * 8 + 1)) == 0                            # GEMM-sized groups: the GEMM kernels read it too
    assert f(*args(a7=3)) == INV                                   # nseg
    big = ctypes.c_size_t(1 << 30)
    assert f(*args(a14=FAKE, a15=ctypes.byref(big), a12=None)) == INV       # NULL w_down
    assert f(*args(a14=FAKE, a15=ctypes.byref(big), a10=FAKE + 8)) == INV   # misaligned weights


def test_gate_validation(lib):
    g = lib.moe_gate
    assert g(FAKE, 4, 8, 9, 1, FAKE, FAKE, None) == INV          # k > E
    assert g(FAKE, 4, 8, 0, 1, FAKE, FAKE, None) == INV          # k < 1
    assert g(FAKE, -1, 8, 2, 1, FAKE, FAKE, None) == INV         # T < 0
    assert g(FAKE, 4, 8, 2, 2, FAKE, FAKE, None) == INV          # renormalize not 0/1
    assert g(FAKE, 4, 513, 2, 1, FAKE, FAKE, None) == UNS        # E > 512
    assert g(None, 4, 8, 2, 1, FAKE, FAKE, None) == INV          # NULL logits
    assert g(FAKE + 2, 4, 8, 2, 1, FAKE, FAKE, None) == INV      # misaligned
    assert g(None, 0, 8, 2, 1, None, None, None) == 0            # T = 0 is a no-op


def test_gate_record_validation(lib):
    g = lib.moe_gate_record
    ok = [FAKE, 64, 8, 2, 1, FAKE, FAKE, 16, 0, 1, FAKE, None]
    a = lambda **kw: [kw.get(f"a{i}", v) for i, v in enumerate(ok)]
    assert g(*a(a3=9)) == INV                  # k > E (moe_gate's checks apply)
    assert g(*a(a7=0)) == INV                  # block_tokens < 1
    assert g(*a(a9=0)) == INV                  # L < 1
    assert g(*a(a8=1)) == INV                  # layer >= L
    assert g(*a(a8=-1)) == INV                 # layer < 0
    assert g(*a(a10=None)) == INV              # NULL block_counts
    assert g(*a(a10=FAKE + 2)) == INV          # misaligned block_counts
    assert g(*a(a2=513)) == UNS                # E > 512
    assert g(*a(a1=0, a0=None, a5=None, a6=None, a10=None)) == 0     # T = 0 is a no-op


def test_stage_to_host_validation(lib):
    s = lib.moe_stage_to_host
    assert s(None, None, 0, None) == 0                               # nothing to copy
    assert s(None, FAKE, 64, None) == INV
    assert s(FAKE, None, 64, None) == INV


def _perm(lib, T=4, E=8, k=2, S=0, P=0, x=FAKE, dt=1, d=64, ws=FAKE, nbytes=1 << 30, **kw):
    n = ctypes.c_size_t(nbytes)
    ptrs = dict(ids=FAKE, go=FAKE, s2f=FAKE, f2s=FAKE, tok=FAKE, xs=FAKE)
    ptrs.update(kw)
    return lib.moe_permute(ptrs["ids"], T, E, k, S, P, x, dt, d, ptrs["go"], ptrs["s2f"], ptrs["f2s"],
                           ptrs["tok"], ptrs["xs"], ws, ctypes.byref(n), None), n.value


def test_permute_validation_and_query(lib):
    assert _perm(lib, k=9)[0] == INV
    assert _perm(lib, P=5)[0] == INV                 # n_priority > T
    assert _perm(lib, S=-1)[0] == INV
    assert _perm(lib, d=12)[0] == UNS                # d % 8
    assert _perm(lib, dt=7)[0] == UNS                # unknown dtype
    assert _perm(lib, go=None)[0] == INV
    assert _perm(lib, xs=None)[0] == INV             # x given without x_sorted
    assert _perm(lib, xs=FAKE + 8)[0] == INV         # misaligned x_sorted
    assert _perm(lib, tok=FAKE + 2)[0] == INV        # misaligned sorted_token
    assert _perm(lib, tok=None, x=None, xs=None, ws=None, nbytes=0)[0] == 0   # optional outputs
    st, need = _perm(lib, T=8192, E=128, k=8, ws=None, nbytes=0)
    assert st == 0 and need > 0
    assert _perm(lib, T=8192, E=128, k=8, nbytes=need - 1)[0] == WS
    st, need_small = _perm(lib, T=4, ws=None, nbytes=0)
    assert st == 0 and need_small > 0


def _ffn(lib, N=64, E=8, S=0, nseg=1, d=64, I=128, dt=1, ws=FAKE, nbytes=1 << 40, n_x=0, **kw):
    n = ctypes.c_size_t(nbytes)
    p = dict(xs=FAKE, rows=None, go=FAKE, wg=FAKE, wu=FAKE, wd=FAKE, h=FAKE)
    p.update(kw)
    return lib.moe_grouped_ffn(p["xs"], p["rows"], n_x, p["go"], N, E, S, nseg, d, I, p["wg"], p["wu"], p["wd"],
                               dt, p["h"], ws, ctypes.byref(n), None), n.value


def test_ffn_validation_and_query(lib):
    assert _ffn(lib, nseg=3)[0] == INV
    assert _ffn(lib, E=0)[0] == INV
    assert _ffn(lib, d=100)[0] == UNS
    assert _ffn(lib, I=12)[0] == UNS
    assert _ffn(lib, dt=5)[0] == UNS
    assert _ffn(lib, E=600)[0] == UNS
    assert _ffn(lib, wd=None)[0] == INV
    assert _ffn(lib, wg=FAKE + 4)[0] == INV
    assert _ffn(lib, rows=FAKE, n_x=0)[0] == INV          # row list without a row count
    assert _ffn(lib, rows=FAKE + 2, n_x=16)[0] == INV     # misaligned row list
    st, need = _ffn(lib, N=65536, E=128, d=2048, I=768, ws=None, nbytes=0)
    assert st == 0 and need >= 65536 * 768 * 2           # holds the bf16 intermediate
    assert _ffn(lib, N=65536, E=128, d=2048, I=768, nbytes=need - 1)[0] == WS
    assert _ffn(lib, N=0, ws=FAKE)[0] == 0               # no rows: no-op


def test_ffn_traced_validation_and_query(lib):
    f = lib.moe_grouped_ffn_traced
    n = ctypes.c_size_t(0)
    args = lambda **kw: [kw.get(f"a{i}", v) for i, v in enumerate(
        [FAKE, None, 0, FAKE, 4160 * 4, 128, 0, 2, 2880, 2880, FAKE, FAKE, FAKE, 1, FAKE, None, ctypes.byref(n),
         FAKE, 1024, 0, None])]
    assert f(*args()) == 0                                          # query
    st, need = _ffn(lib, N=4160 * 4, E=128, nseg=2, d=2880, I=2880, ws=None, nbytes=0)
    assert st == 0 and n.value == need                              # the same workspace as moe_grouped_ffn
    big = ctypes.c_size_t(1 << 40)
    assert f(*args(a15=FAKE, a16=ctypes.byref(big), a18=-1)) == INV          # negative capacity
    assert f(*args(a15=FAKE, a16=ctypes.byref(big), a17=None)) == INV        # NULL trace
    assert f(*args(a15=FAKE, a16=ctypes.byref(big), a17=FAKE + 8)) == INV    # misaligned trace
    assert f(*args(a15=FAKE, a16=ctypes.byref(big), a8=100)) == UNS          # checks of moe_grouped_ffn apply
    assert f(*args(a15=FAKE, a16=ctypes.byref(big), a19=2)) == INV           # weights_packed is 0 or 1
    assert f(*args(a19=1)) == 0                                              # packed weights: same query
    assert f(*args(a15=FAKE, a16=ctypes.byref(big), a19=1, a13=0)) == UNS    # packed weights are bf16 only
    assert f(*args(a15=FAKE, a16=ctypes.byref(big), a19=1, a8=2888)) == UNS  # packed: d % 32 != 0


def test_ffn_combine_validation(lib):
    """The fused FFN + combine: argument errors, shape support and the
    workspace query, all before any GPU work."""
    f = lib.moe_grouped_ffn_combine
    n = ctypes.c_size_t(0)
    base = [FAKE, FAKE, 128, FAKE, 1024, 64, 0, 1, 2048, 1024, FAKE, FAKE, FAKE, 0, FAKE, FAKE, 128, 8, FAKE, None,
            ctypes.byref(n), None]
    a = lambda **kw: [kw.get(f"a{i}", v) for i, v in enumerate(base)]
    assert f(*a()) == 0 and n.value > 128 * 2048 * 4                # query: the fp32 sums + the FFN workspace
    big = ctypes.c_size_t(1 << 40)
    assert f(*a(a19=FAKE, a20=ctypes.byref(big), a4=1000)) == INV    # n_rows != T * (k + n_shared)
    assert f(*a(a19=FAKE, a20=ctypes.byref(big), a13=2)) == INV      # weights_packed not 0/1
    assert f(*a(a19=FAKE, a20=ctypes.byref(big), a17=0)) == INV      # k < 1
    assert f(*a(a19=FAKE, a20=ctypes.byref(big), a18=None)) == INV   # NULL y
    assert f(*a(a19=FAKE, a20=ctypes.byref(big), a18=FAKE + 8)) == INV   # misaligned y
    assert f(*a(a19=FAKE, a20=ctypes.byref(big), a13=1, a8=2056)) == UNS  # packed: d % 32 != 0
    assert f(*a(a4=65536, a5=128, a8=2048, a9=768, a16=8192, a17=8)) == UNS   # prefill-sized groups
    assert f(*a(a19=FAKE, a20=ctypes.byref(ctypes.c_size_t(16)))) == WS
    assert f(*a(a4=0, a16=0, a19=FAKE, a20=ctypes.byref(big))) == 0  # empty batch: nothing to do


def test_ffn_noalloc_validation(lib):
    """Argument errors and the scratch limit are reported before the library
    touches a GPU (the CPU here has none)."""
    f = lib.moe_grouped_ffn_noalloc
    args = lambda **kw: [kw.get(f"a{i}", v) for i, v in enumerate(
        [FAKE, None, 0, FAKE, 1024, 64, 0, 1, 2048, 1024, FAKE, FAKE, FAKE, 1, FAKE, None])]
    assert f(*args(a7=3)) == INV                                     # nseg
    assert f(*args(a8=100)) == UNS                                   # d not a multiple of 8
    assert f(*args(a13=5)) == UNS                                    # unknown dtype
    assert f(*args(a4=65536, a5=128, a8=2048, a9=768)) == WS         # Qwen3-shaped: above the 64 MiB array
    assert f(*args(a4=0)) == 0                                       # no rows: nothing to do


def test_combine_validation(lib):
    c = lib.moe_combine
    assert c(FAKE, FAKE, FAKE, 4, 0, 0, 64, 1, FAKE, None) == INV
    assert c(FAKE, FAKE, FAKE, 4, 2, 0, 60, 1, FAKE, None) == UNS
    assert c(FAKE, FAKE, FAKE, 4, 2, 0, 64, 3, FAKE, None) == UNS
    assert c(None, FAKE, FAKE, 4, 2, 0, 64, 1, FAKE, None) == INV
    assert c(FAKE, FAKE, FAKE, 4, 2, 0, 64, 1, FAKE + 4, None) == INV
    assert c(None, None, None, 0, 2, 0, 64, 1, None, None) == 0


def _stats(lib, L=1, T=8, k=2, E=8, req=FAKE, R=2, ws=FAKE, nbytes=1 << 30, **kw):
    n = ctypes.c_size_t(nbytes)
    p = dict(ids=FAKE, idf=None, counts=FAKE, usize=FAKE, umask=FAKE, aff=FAKE, rc=FAKE, sig=FAKE)
    p.update(kw)
    return lib.moe_stats(p["ids"], L, T, k, E, req, R, p["idf"], p["counts"], p["usize"], p["umask"], p["aff"],
                         p["rc"], p["sig"], ws, ctypes.byref(n), None), n.value


def test_stats_validation_and_query(lib):
    assert _stats(lib, k=9)[0] == INV
    assert _stats(lib, R=-1)[0] == INV
    assert _stats(lib, E=1000, k=2)[0] == UNS
    assert _stats(lib, req=None)[0] == INV           # signature without requests
    assert _stats(lib, counts=None)[0] == INV
    st, need = _stats(lib, L=8, T=8192, k=8, E=128, R=128, ws=None, nbytes=0)
    assert st == 0 and need >= 128 * 8 * 128 * 4
    assert _stats(lib, L=8, T=8192, k=8, E=128, R=128, nbytes=need - 1)[0] == WS
    assert _stats(lib, L=0)[0] == 0

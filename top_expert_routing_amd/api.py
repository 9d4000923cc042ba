"""Thin torch wrappers over the libmoe calls (router projection, gate,
permutation, grouped FFN, combine, statistics).

Argument marshalling only: shapes, dtypes and contiguity are checked, outputs
and workspaces are allocated with torch on the input's device, and the call is
enqueued on torch's current stream.  Every step of the path runs in libmoe's
HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
from typing import Dict, Optional

import torch

from . import _lib
from ._lib import MOE_BF16, MOE_F32, check


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(t: torch.Tensor, name: str, dtype=None, ndim=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")


def _out(t: torch.Tensor, name: str, dtype, shape):
    """A caller-supplied output: a contiguous GPU tensor of exactly this dtype and shape."""
    _need(t, name, dtype, len(shape))
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _workspace(fn, args_before_ws, dev) -> torch.Tensor:
    """Query a call's workspace size (NULL workspace) and allocate it."""
    n = ctypes.c_size_t(0)
    check(fn.__name__, fn(*args_before_ws, None, ctypes.byref(n), None))
    return torch.empty(max(int(n.value), 256), dtype=torch.uint8, device=dev)


def router(x: torch.Tensor, w_router: torch.Tensor, logits: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp32 router logits [T][E] = x [T][d] . w_router [E][d]^T (bf16 or fp32 inputs)."""
    _need(x, "x", None, 2)
    _need(w_router, "w_router", x.dtype, 2)
    T, d = x.shape
    E = w_router.shape[0]
    if w_router.shape[1] != d:
        raise ValueError("w_router must be [E][d]")
    dev = x.device
    if logits is None:
        logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    _out(logits, "logits", torch.float32, (T, E))
    lib = _lib.load()
    check("moe_router", lib.moe_router(_ptr(x), _ptr(w_router), T, d, E, _dtype_code(x), _ptr(logits),
                                       _stream(dev)))
    return logits


def gate(logits: torch.Tensor, k: int, renormalize: bool = True,
         topk_ids: Optional[torch.Tensor] = None, topk_w: Optional[torch.Tensor] = None):
    _need(logits, "logits", torch.float32, 2)
    T, E = logits.shape
    dev = logits.device
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _out(topk_ids, "topk_ids", torch.int32, (T, k))
    _out(topk_w, "topk_w", torch.float32, (T, k))
    lib = _lib.load()
    check("moe_gate", lib.moe_gate(_ptr(logits), T, E, k, int(bool(renormalize)), _ptr(topk_ids),
                                   _ptr(topk_w), _stream(dev)))
    return topk_ids, topk_w


def gate_record(logits: torch.Tensor, k: int, block_tokens: int, layer: int, block_counts: torch.Tensor,
                renormalize: bool = True, topk_ids: Optional[torch.Tensor] = None,
                topk_w: Optional[torch.Tensor] = None):
    """gate() that also fills row `layer` of the KV-block record block_counts
    [ceil(T / block_tokens)][L][E] int32 (moe_gate_record)."""
    _need(logits, "logits", torch.float32, 2)
    T, E = logits.shape
    dev = logits.device
    if block_tokens < 1:
        raise ValueError("block_tokens must be >= 1")
    nb = -(-T // block_tokens)
    _need(block_counts, "block_counts", torch.int32, 3)
    L = block_counts.shape[1]
    _out(block_counts, "block_counts", torch.int32, (nb, L, E))
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _out(topk_ids, "topk_ids", torch.int32, (T, k))
    _out(topk_w, "topk_w", torch.float32, (T, k))
    lib = _lib.load()
    check("moe_gate_record", lib.moe_gate_record(_ptr(logits), T, E, k, int(bool(renormalize)), _ptr(topk_ids),
                                                 _ptr(topk_w), block_tokens, layer, L, _ptr(block_counts),
                                                 _stream(dev)))
    return topk_ids, topk_w


def stage_to_host(src: torch.Tensor, dst: torch.Tensor) -> torch.Tensor:
    """Enqueue the copy of GPU tensor `src` into the pinned host tensor `dst`
    (same dtype and shape) on the current stream (moe_stage_to_host); read
    `dst` after synchronising that stream."""
    _need(src, "src")
    if dst.is_cuda or not dst.is_contiguous():
        raise ValueError("dst must be a contiguous host tensor")
    if dst.dtype != src.dtype or dst.shape != src.shape:
        raise ValueError("dst must match src in dtype and shape")
    lib = _lib.load()
    check("moe_stage_to_host", lib.moe_stage_to_host(_ptr(src), ctypes.c_void_p(dst.data_ptr()),
                                                     src.numel() * src.element_size(), _stream(src.device)))
    return dst


def permute_workspace_bytes(T, E, k, n_shared=0, n_priority=0) -> int:
    lib = _lib.load()
    n = ctypes.c_size_t(0)
    check("moe_permute", lib.moe_permute(None, T, E, k, n_shared, n_priority, None, MOE_BF16, 8,
                                         None, None, None, None, None, None, ctypes.byref(n), None))
    return int(n.value)


def permute(topk_ids: torch.Tensor, E: int, n_shared: int = 0, n_priority: int = 0,
            x: Optional[torch.Tensor] = None, out: Optional[Dict[str, torch.Tensor]] = None,
            workspace: Optional[torch.Tensor] = None, sorted_token: bool = True) -> Dict[str, torch.Tensor]:
    """Counting sort of the assignments; `sorted_token` also writes the token
    of every sorted row (the row list moe_grouped_ffn can read x through)."""
    _need(topk_ids, "topk_ids", torch.int32, 2)
    T, k = topk_ids.shape
    dev = topk_ids.device
    nseg = 2 if n_priority > 0 else 1
    G = nseg * E + n_shared
    N = T * (k + n_shared)
    d = 8
    dt = MOE_BF16
    if x is not None:
        _need(x, "x", None, 2)
        if x.shape[0] != T:
            raise ValueError(f"x must have {T} rows, one per token")
        d = x.shape[1]
        dt = _dtype_code(x)
    o = {} if out is None else out
    if "group_offsets" not in o:
        o["group_offsets"] = torch.empty(G + 1, dtype=torch.int32, device=dev)
    if "sorted_to_flat" not in o:
        o["sorted_to_flat"] = torch.empty(N, dtype=torch.int32, device=dev)
    if "flat_to_sorted" not in o:
        o["flat_to_sorted"] = torch.empty(N, dtype=torch.int32, device=dev)
    if sorted_token and "sorted_token" not in o:
        o["sorted_token"] = torch.empty(N, dtype=torch.int32, device=dev)
    if x is not None and "x_sorted" not in o:
        o["x_sorted"] = torch.empty((N, d), dtype=x.dtype, device=dev)
    _out(o["group_offsets"], "group_offsets", torch.int32, (G + 1,))
    for key in ("sorted_to_flat", "flat_to_sorted") + (("sorted_token",) if sorted_token else ()):
        _out(o[key], key, torch.int32, (N,))
    if x is not None:
        _out(o["x_sorted"], "x_sorted", x.dtype, (N, d))
    if workspace is None:
        workspace = torch.empty(max(permute_workspace_bytes(T, E, k, n_shared, n_priority), 256),
                                dtype=torch.uint8, device=dev)
    lib = _lib.load()
    nbytes = ctypes.c_size_t(workspace.numel())
    check("moe_permute", lib.moe_permute(
        _ptr(topk_ids), T, E, k, n_shared, n_priority, _ptr(x), dt, d,
        _ptr(o["group_offsets"]), _ptr(o["sorted_to_flat"]), _ptr(o["flat_to_sorted"]),
        _ptr(o.get("sorted_token")) if sorted_token else None,
        _ptr(o.get("x_sorted")) if x is not None else None,
        _ptr(workspace), ctypes.byref(nbytes), _stream(dev)))
    return o


def ffn_workspace_bytes(n_rows, E, n_shared, nseg, d, I, dtype=torch.bfloat16) -> int:
    lib = _lib.load()
    n = ctypes.c_size_t(0)
    code = MOE_BF16 if dtype == torch.bfloat16 else MOE_F32
    check("moe_grouped_ffn", lib.moe_grouped_ffn(None, None, 0, None, n_rows, E, n_shared, nseg, d, I, None, None,
                                                 None, code, None, None, ctypes.byref(n), None))
    return int(n.value)


def grouped_ffn(x_sorted: torch.Tensor, group_offsets: torch.Tensor, E: int, n_shared: int, nseg: int,
                w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
                h_sorted: Optional[torch.Tensor] = None,
                workspace: Optional[torch.Tensor] = None,
                x_rows: Optional[torch.Tensor] = None,
                trace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Grouped SwiGLU FFN.  With `x_rows` ([N] int32, e.g. permute's
    sorted_token) `x_sorted` is the unsorted token matrix and sorted row n
    reads its row x_rows[n].  With `trace` ([R][4] int64, zero-filled by the
    caller) the persistent-queue path records one line per tile
    (moe_grouped_ffn_traced)."""
    _need(x_sorted, "x_sorted", None, 2)
    _need(group_offsets, "group_offsets", torch.int32, 1)
    for name, w in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _need(w, name, x_sorted.dtype, 3)
    n_x, d = x_sorted.shape
    N = n_x
    if x_rows is not None:
        _need(x_rows, "x_rows", torch.int32, 1)
        N = x_rows.numel()
    I = w_gate.shape[1]
    if w_gate.shape != (E + n_shared, I, d) or w_up.shape != w_gate.shape or w_down.shape != (E + n_shared, d, I):
        raise ValueError("expert weight shapes do not match [E+S][I][d] / [E+S][d][I]")
    if group_offsets.numel() != nseg * E + n_shared + 1:
        raise ValueError("group_offsets must have nseg*E + n_shared + 1 entries")
    dev = x_sorted.device
    if h_sorted is None:
        h_sorted = torch.empty((N, d), dtype=x_sorted.dtype, device=dev)
    _need(h_sorted, "h_sorted", x_sorted.dtype, 2)
    if h_sorted.shape != (N, d):
        raise ValueError(f"h_sorted must be [{N}][{d}]")
    if workspace is None:
        workspace = torch.empty(max(ffn_workspace_bytes(N, E, n_shared, nseg, d, I, x_sorted.dtype), 256),
                                dtype=torch.uint8, device=dev)
    lib = _lib.load()
    nbytes = ctypes.c_size_t(workspace.numel())
    args = (_ptr(x_sorted), _ptr(x_rows), n_x, _ptr(group_offsets), N, E, n_shared, nseg, d, I, _ptr(w_gate),
            _ptr(w_up), _ptr(w_down), _dtype_code(x_sorted), _ptr(h_sorted), _ptr(workspace), ctypes.byref(nbytes))
    if trace is None:
        check("moe_grouped_ffn", lib.moe_grouped_ffn(*args, _stream(dev)))
    else:
        _need_trace(trace)
        check("moe_grouped_ffn_traced", lib.moe_grouped_ffn_traced(*args, _ptr(trace), trace.shape[0], 0,
                                                                   _stream(dev)))
    return h_sorted


def _need_trace(trace: torch.Tensor):
    _need(trace, "trace", torch.int64, 2)
    if trace.shape[1] != 4:
        raise ValueError("trace must be [records][4] int64")


def ffn_combine_workspace_bytes(N, E, n_shared, nseg, d, I, T, k, packed=False) -> int:
    """Workspace of moe_grouped_ffn_combine (raises MoeError for a batch it
    does not serve)."""
    lib = _lib.load()
    n = ctypes.c_size_t(0)
    check("moe_grouped_ffn_combine", lib.moe_grouped_ffn_combine(
        None, None, 0, None, N, E, n_shared, nseg, d, I, None, None, None, int(bool(packed)), None, None, T, k,
        None, None, ctypes.byref(n), None))
    return int(n.value)


def grouped_ffn_combine(x_sorted: torch.Tensor, group_offsets: torch.Tensor, E: int, n_shared: int, nseg: int,
                        w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
                        sorted_to_flat: torch.Tensor, topk_w: torch.Tensor, y: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None, x_rows: Optional[torch.Tensor] = None,
                        packed: bool = False) -> torch.Tensor:
    """grouped_ffn then combine in one call, the combine folded into the down
    projection (moe_grouped_ffn_combine; bf16, decode-sized batches).  With
    `packed` the weights come from pack_weights."""
    _need(x_sorted, "x_sorted", torch.bfloat16, 2)
    _need(group_offsets, "group_offsets", torch.int32, 1)
    for name, w in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _need(w, name, torch.bfloat16, 3)
    _need(sorted_to_flat, "sorted_to_flat", torch.int32, 1)
    _need(topk_w, "topk_w", torch.float32, 2)
    n_x, d = x_sorted.shape
    N = sorted_to_flat.numel()
    if x_rows is not None:
        _need(x_rows, "x_rows", torch.int32, 1)
        if x_rows.numel() != N:
            raise ValueError("x_rows and sorted_to_flat must have one entry per sorted row")
    elif n_x != N:
        raise ValueError("x_sorted must have one row per sorted row")
    T, k = topk_w.shape
    I = w_gate.shape[1]
    if w_gate.shape != (E + n_shared, I, d) or w_up.shape != w_gate.shape or w_down.shape != (E + n_shared, d, I):
        raise ValueError("expert weight shapes do not match [E+S][I][d] / [E+S][d][I]")
    if group_offsets.numel() != nseg * E + n_shared + 1:
        raise ValueError("group_offsets must have nseg*E + n_shared + 1 entries")
    dev = x_sorted.device
    if y is None:
        y = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    _out(y, "y", torch.bfloat16, (T, d))
    if workspace is None:
        workspace = torch.empty(max(ffn_combine_workspace_bytes(N, E, n_shared, nseg, d, I, T, k, packed), 256),
                                dtype=torch.uint8, device=dev)
    lib = _lib.load()
    nbytes = ctypes.c_size_t(workspace.numel())
    check("moe_grouped_ffn_combine", lib.moe_grouped_ffn_combine(
        _ptr(x_sorted), _ptr(x_rows), n_x, _ptr(group_offsets), N, E, n_shared, nseg, d, I, _ptr(w_gate),
        _ptr(w_up), _ptr(w_down), int(bool(packed)), _ptr(sorted_to_flat), _ptr(topk_w), T, k, _ptr(y),
        _ptr(workspace), ctypes.byref(nbytes), _stream(dev)))
    return y


NOALLOC_SCRATCH_BYTES = 64 << 20


def grouped_ffn_noalloc(x_sorted: torch.Tensor, group_offsets: torch.Tensor, E: int, n_shared: int, nseg: int,
                        w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor, h_sorted: torch.Tensor,
                        x_rows: Optional[torch.Tensor] = None) -> torch.Tensor:
    """grouped_ffn on the library's per-device scratch array
    (moe_grouped_ffn_noalloc): no workspace, nothing allocated by the call.
    The caller passes the output; calls on one GPU must not overlap."""
    _need(x_sorted, "x_sorted", None, 2)
    _need(group_offsets, "group_offsets", torch.int32, 1)
    for name, w in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _need(w, name, x_sorted.dtype, 3)
    n_x, d = x_sorted.shape
    N = n_x
    if x_rows is not None:
        _need(x_rows, "x_rows", torch.int32, 1)
        N = x_rows.numel()
    I = w_gate.shape[1]
    if w_gate.shape != (E + n_shared, I, d) or w_up.shape != w_gate.shape or w_down.shape != (E + n_shared, d, I):
        raise ValueError("expert weight shapes do not match [E+S][I][d] / [E+S][d][I]")
    if group_offsets.numel() != nseg * E + n_shared + 1:
        raise ValueError("group_offsets must have nseg*E + n_shared + 1 entries")
    _out(h_sorted, "h_sorted", x_sorted.dtype, (N, d))
    lib = _lib.load()
    check("moe_grouped_ffn_noalloc", lib.moe_grouped_ffn_noalloc(
        _ptr(x_sorted), _ptr(x_rows), n_x, _ptr(group_offsets), N, E, n_shared, nseg, d, I, _ptr(w_gate),
        _ptr(w_up), _ptr(w_down), _dtype_code(x_sorted), _ptr(h_sorted), _stream(x_sorted.device)))
    return h_sorted


def pack_weights(w: torch.Tensor) -> torch.Tensor:
    """Expert matrices [..][R][K] in the layout moe_grouped_ffn_packed reads:
    blocks of 16 rows x 32 K values, block (r/16, k/32) at element offset
    ((r/16) * (K/32) + k/32) * 512 of each matrix, and W[r][k] at
    (((k%32)/8) * 16 + r%16) * 8 + k%8 inside its block.  The result keeps the
    input's shape (and each matrix its place); a one-time weight preparation."""
    *lead, R, K = w.shape
    if R % 16 != 0 or K % 32 != 0:
        raise ValueError("packing needs rows % 16 == 0 and K % 32 == 0")
    v = w.reshape(*lead, R // 16, 16, K // 32, 4, 8)       # r = 16 rb + r16, k = 32 kb + 8 q + t
    n = len(lead)
    return v.permute(*range(n), n, n + 2, n + 3, n + 1, n + 4).contiguous().reshape(w.shape)


def grouped_ffn_packed(x_sorted: torch.Tensor, group_offsets: torch.Tensor, E: int, n_shared: int, nseg: int,
                       w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor,
                       h_sorted: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                       x_rows: Optional[torch.Tensor] = None,
                       trace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """grouped_ffn (bf16, any batch size) with weights from pack_weights;
    `trace` as in grouped_ffn (moe_grouped_ffn_traced with packed weights)."""
    _need(x_sorted, "x_sorted", torch.bfloat16, 2)
    _need(group_offsets, "group_offsets", torch.int32, 1)
    for name, w in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down)):
        _need(w, name, torch.bfloat16, 3)
    n_x, d = x_sorted.shape
    N = n_x
    if x_rows is not None:
        _need(x_rows, "x_rows", torch.int32, 1)
        N = x_rows.numel()
    I = w_gate.shape[1]
    if w_gate.shape != (E + n_shared, I, d) or w_up.shape != w_gate.shape or w_down.shape != (E + n_shared, d, I):
        raise ValueError("expert weight shapes do not match [E+S][I][d] / [E+S][d][I]")
    if group_offsets.numel() != nseg * E + n_shared + 1:
        raise ValueError("group_offsets must have nseg*E + n_shared + 1 entries")
    dev = x_sorted.device
    if h_sorted is None:
        h_sorted = torch.empty((N, d), dtype=torch.bfloat16, device=dev)
    _out(h_sorted, "h_sorted", torch.bfloat16, (N, d))
    if workspace is None:
        workspace = torch.empty(max(ffn_workspace_bytes(N, E, n_shared, nseg, d, I, torch.bfloat16), 256),
                                dtype=torch.uint8, device=dev)
    lib = _lib.load()
    nbytes = ctypes.c_size_t(workspace.numel())
    if trace is None:
        check("moe_grouped_ffn_packed", lib.moe_grouped_ffn_packed(
            _ptr(x_sorted), _ptr(x_rows), n_x, _ptr(group_offsets), N, E, n_shared, nseg, d, I, _ptr(w_gate),
            _ptr(w_up), _ptr(w_down), _ptr(h_sorted), _ptr(workspace), ctypes.byref(nbytes), _stream(dev)))
    else:
        _need_trace(trace)
        check("moe_grouped_ffn_traced", lib.moe_grouped_ffn_traced(
            _ptr(x_sorted), _ptr(x_rows), n_x, _ptr(group_offsets), N, E, n_shared, nseg, d, I, _ptr(w_gate),
            _ptr(w_up), _ptr(w_down), _dtype_code(x_sorted), _ptr(h_sorted), _ptr(workspace), ctypes.byref(nbytes),
            _ptr(trace), trace.shape[0], 1, _stream(dev)))
    return h_sorted


def ffn_fp8w_workspace_bytes(n_rows, I, E=1, n_shared=0, nseg=1, d=64, packed=False) -> int:
    """Workspace of the FP8-weight FFN (the SwiGLU intermediate, plus the
    persistent queue's state for the batches that may run on it)."""
    lib = _lib.load()
    n = ctypes.c_size_t(0)
    name = "moe_grouped_ffn_fp8w_packed" if packed else "moe_grouped_ffn_fp8w"
    check(name, getattr(lib, name)(None, None, 0, None, n_rows, E, n_shared, nseg, d, I, None, None, None, None,
                                   None, None, None, None, ctypes.byref(n), None))
    return int(n.value)


def quantize_fp8_rows(w: torch.Tensor):
    """Per-row E4M3 quantisation of [..][rows][cols] weights: scale = max|row| / 448
    (1 for an all-zero row), codes = round-to-nearest-even(w / scale).  Input
    preparation for moe_grouped_ffn_fp8w; returns (codes uint8, scales fp32)."""
    wf = w.float()
    s = wf.abs().amax(dim=-1) / 448.0
    s = torch.where(s > 0, s, torch.ones_like(s))
    q = (wf / s.unsqueeze(-1)).to(torch.float8_e4m3fn).view(torch.uint8)
    return q.contiguous(), s.contiguous()


def pack_fp8_codes(q: torch.Tensor) -> torch.Tensor:
    """E4M3 code matrices [..][R][K] (uint8) in the layout
    moe_grouped_ffn_fp8w_packed reads: blocks of 16 rows x 64 codes, block
    (r/16, k/64) at byte ((r/16) * (K/64) + k/64) * 1024 of each matrix and
    C[r][k] at (((k%64)/16) * 16 + r%16) * 16 + k%16 inside it; same shape."""
    *lead, R, K = q.shape
    if R % 16 != 0 or K % 64 != 0:
        raise ValueError("packing needs rows % 16 == 0 and K % 64 == 0")
    v = q.reshape(*lead, R // 16, 16, K // 64, 4, 16)      # r = 16 rb + r16, k = 64 kb + 16 j + t
    n = len(lead)
    return v.permute(*range(n), n, n + 2, n + 3, n + 1, n + 4).contiguous().reshape(q.shape)


def grouped_ffn_fp8w(x: torch.Tensor, group_offsets: torch.Tensor, E: int, n_shared: int, nseg: int,
                     w_gate: torch.Tensor, s_gate: torch.Tensor, w_up: torch.Tensor, s_up: torch.Tensor,
                     w_down: torch.Tensor, s_down: torch.Tensor, h_sorted: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, x_rows: Optional[torch.Tensor] = None,
                     packed: bool = False) -> torch.Tensor:
    """The expert FFN with E4M3 weight codes (uint8) and fp32 per-row scales;
    bf16 token rows, read directly or through `x_rows`.  packed: the codes come
    from pack_fp8_codes (moe_grouped_ffn_fp8w_packed)."""
    _need(x, "x", torch.bfloat16, 2)
    for t, n in ((w_gate, "w_gate"), (w_up, "w_up"), (w_down, "w_down")):
        _need(t, n, torch.uint8, 3)
    for t, n in ((s_gate, "s_gate"), (s_up, "s_up"), (s_down, "s_down")):
        _need(t, n, torch.float32, 2)
    _need(group_offsets, "group_offsets", torch.int32, 1)
    if x_rows is not None:
        _need(x_rows, "x_rows", torch.int32, 1)
    n_rows = int(x_rows.numel()) if x_rows is not None else x.shape[0]
    d = x.shape[1]
    I = w_gate.shape[1]
    G = E + n_shared
    if w_gate.shape != (G, I, d) or w_up.shape != w_gate.shape or w_down.shape != (G, d, I):
        raise ValueError("expert weight codes must be [E+S][I][d] (gate, up) and [E+S][d][I] (down)")
    if s_gate.shape != (G, I) or s_up.shape != (G, I) or s_down.shape != (G, d):
        raise ValueError("row scales must be [E+S][I] (gate, up) and [E+S][d] (down)")
    if group_offsets.numel() != nseg * E + n_shared + 1:
        raise ValueError("group_offsets must have nseg*E + n_shared + 1 entries")
    dev = x.device
    if h_sorted is None:
        h_sorted = torch.empty((n_rows, d), dtype=torch.bfloat16, device=dev)
    _need(h_sorted, "h_sorted", torch.bfloat16, 2)
    if h_sorted.shape != (n_rows, d):
        raise ValueError(f"h_sorted must be [{n_rows}][{d}]")
    if workspace is None:
        workspace = torch.empty(max(ffn_fp8w_workspace_bytes(n_rows, I, E, n_shared, nseg, d, packed), 256),
                                dtype=torch.uint8, device=dev)
    lib = _lib.load()
    nbytes = ctypes.c_size_t(workspace.numel())
    name = "moe_grouped_ffn_fp8w_packed" if packed else "moe_grouped_ffn_fp8w"
    check(name, getattr(lib, name)(
        _ptr(x), _ptr(x_rows), x.shape[0] if x_rows is not None else 0, _ptr(group_offsets), n_rows, E, n_shared,
        nseg, d, I, _ptr(w_gate), _ptr(s_gate), _ptr(w_up), _ptr(s_up), _ptr(w_down), _ptr(s_down), _ptr(h_sorted),
        _ptr(workspace), ctypes.byref(nbytes), _stream(dev)))
    return h_sorted


def combine(h_sorted: torch.Tensor, flat_to_sorted: torch.Tensor, topk_w: torch.Tensor, n_shared: int = 0,
            y: Optional[torch.Tensor] = None) -> torch.Tensor:
    _need(h_sorted, "h_sorted", None, 2)
    _need(flat_to_sorted, "flat_to_sorted", torch.int32, 1)
    _need(topk_w, "topk_w", torch.float32, 2)
    T, k = topk_w.shape
    d = h_sorted.shape[1]
    if flat_to_sorted.numel() != T * (k + n_shared) or h_sorted.shape[0] != T * (k + n_shared):
        raise ValueError("h_sorted / flat_to_sorted must have T*(k+n_shared) rows")
    dev = h_sorted.device
    if y is None:
        y = torch.empty((T, d), dtype=h_sorted.dtype, device=dev)
    lib = _lib.load()
    check("moe_combine", lib.moe_combine(_ptr(h_sorted), _ptr(flat_to_sorted), _ptr(topk_w), T, k, n_shared,
                                         d, _dtype_code(h_sorted), _ptr(y), _stream(dev)))
    return y


def stats_workspace_bytes(L, T, k, E, R) -> int:
    lib = _lib.load()
    n = ctypes.c_size_t(0)
    check("moe_stats", lib.moe_stats(None, L, T, k, E, None, R, None, None, None, None, None, None, None,
                                     None, ctypes.byref(n), None))
    return int(n.value)


def stats(topk_ids: torch.Tensor, E: int, req_offsets: Optional[torch.Tensor] = None,
          idf: Optional[torch.Tensor] = None, affinity: bool = True, signature: bool = True,
          out: Optional[Dict[str, torch.Tensor]] = None,
          workspace: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    _need(topk_ids, "topk_ids", torch.int32, 3)
    L, T, k = topk_ids.shape
    dev = topk_ids.device
    R = 0
    if req_offsets is not None:
        _need(req_offsets, "req_offsets", torch.int32, 1)
        R = req_offsets.numel() - 1
    if idf is not None:
        _out(idf, "idf", torch.float32, (L, E))
    o = {} if out is None else out
    o.setdefault("counts", torch.empty((L, E), dtype=torch.int32, device=dev))
    o.setdefault("union_size", torch.empty(L, dtype=torch.int32, device=dev))
    o.setdefault("union_mask", torch.empty((L, E), dtype=torch.uint8, device=dev))
    if affinity:
        o.setdefault("affinity", torch.empty((L, E, E), dtype=torch.int32, device=dev))
    if R > 0:
        o.setdefault("req_counts", torch.empty((R, L, E), dtype=torch.int32, device=dev))
        if signature:
            o.setdefault("signature", torch.empty((R, L, E), dtype=torch.float32, device=dev))
    shapes = {"counts": ((L, E), torch.int32), "union_size": ((L,), torch.int32),
              "union_mask": ((L, E), torch.uint8), "affinity": ((L, E, E), torch.int32),
              "req_counts": ((R, L, E), torch.int32), "signature": ((R, L, E), torch.float32)}
    for key, (shape, dt) in shapes.items():
        if key in o and (R > 0 or key not in ("req_counts", "signature")):
            _out(o[key], key, dt, shape)
    if workspace is None:
        workspace = torch.empty(max(stats_workspace_bytes(L, T, k, E, R), 256), dtype=torch.uint8, device=dev)
    lib = _lib.load()
    nbytes = ctypes.c_size_t(workspace.numel())
    check("moe_stats", lib.moe_stats(
        _ptr(topk_ids), L, T, k, E, _ptr(req_offsets), R, _ptr(idf), _ptr(o["counts"]),
        _ptr(o["union_size"]), _ptr(o["union_mask"]), _ptr(o.get("affinity")), _ptr(o.get("req_counts")),
        _ptr(o.get("signature")), _ptr(workspace), ctypes.byref(nbytes), _stream(dev)))
    return o


def prob_signature(logits: torch.Tensor, req_offsets: torch.Tensor,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Continuous request signature [R][L][E]: per request, the sum of its
    tokens' full-E softmax probabilities, from fp32 logits [L][T][E]."""
    _need(logits, "logits", torch.float32, 3)
    _need(req_offsets, "req_offsets", torch.int32, 1)
    L, T, E = logits.shape
    R = req_offsets.numel() - 1
    dev = logits.device
    if out is None:
        out = torch.empty((R, L, E), dtype=torch.float32, device=dev)
    _out(out, "out", torch.float32, (R, L, E))
    lib = _lib.load()
    check("moe_prob_signature", lib.moe_prob_signature(_ptr(logits), L, T, E, _ptr(req_offsets), R, _ptr(out),
                                                       _stream(dev)))
    return out


class MoeLayer:
    """One MoE layer's expert path with every buffer allocated up front.

    `forward()` enqueues gate -> permute -> grouped FFN -> combine and, when
    `stats_ids` is given, the statistics over that [L][T][k] id stack (the
    routing layer's own ids are written into stats_ids[0] by the gate).  With
    `w_router` ([E][d], the input dtype) the router projection runs first and
    the gate reads its logits; `forward` then ignores the logits argument.
    Nothing is allocated per call.
    """

    def __init__(self, E, k, d, I, T, dtype, w_gate, w_up, w_down, n_shared=0, n_priority=0,
                 renormalize=True, stats_layers=0, req_offsets=None, device="cuda", topk_ids=None,
                 fused_gather=True, w_router=None, fp8_weights=None, packed_weights=False, fused_combine=False):
        dev = torch.device(device)
        # fp8_weights = (codes_gate, scales_gate, codes_up, scales_up, codes_down, scales_down):
        # the FFN runs moe_grouped_ffn_fp8w on them instead of w_gate / w_up / w_down
        self.fp8_weights = fp8_weights
        # packed_weights: w_gate / w_up / w_down come from pack_weights and the FFN
        # runs moe_grouped_ffn_packed (bf16, decode-sized batches); with
        # fp8_weights, the codes come from pack_fp8_codes (moe_grouped_ffn_fp8w_packed)
        self.packed = bool(packed_weights)
        # fused_combine: the FFN and the combine run as one moe_grouped_ffn_combine
        # call (bf16 decode-sized batches; h_sorted is then not written)
        self.fused_combine = bool(fused_combine)
        if self.fused_combine and (fp8_weights is not None or dtype != torch.bfloat16):
            raise ValueError("fused_combine serves bf16 expert weights only")
        self.w_router = w_router
        self.logits = torch.empty((T, E), dtype=torch.float32, device=dev) if w_router is not None else None
        self.E, self.k, self.d, self.I, self.T = E, k, d, I, T
        self.S, self.P = n_shared, n_priority
        self.nseg = 2 if n_priority > 0 else 1
        self.renormalize = renormalize
        self.w_gate, self.w_up, self.w_down = w_gate, w_up, w_down
        N = T * (k + n_shared)
        G = self.nseg * E + n_shared
        self.N, self.G = N, G
        # the gate may write straight into a caller buffer (e.g. one layer of a
        # statistics id stack)
        self.topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev) if topk_ids is None else topk_ids
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
        # fused_gather: the permutation writes only the row list and the FFN
        # reads the token rows through it; otherwise x_sorted is materialised
        self.fused_gather = fused_gather
        self.perm = {"group_offsets": torch.empty(G + 1, dtype=torch.int32, device=dev),
                     "sorted_to_flat": torch.empty(N, dtype=torch.int32, device=dev),
                     "flat_to_sorted": torch.empty(N, dtype=torch.int32, device=dev),
                     "sorted_token": torch.empty(N, dtype=torch.int32, device=dev)}
        if not fused_gather:
            self.perm["x_sorted"] = torch.empty((N, d), dtype=dtype, device=dev)
        self.perm_ws = torch.empty(max(permute_workspace_bytes(T, E, k, n_shared, n_priority), 256),
                                   dtype=torch.uint8, device=dev)
        self.h_sorted = torch.empty((N, d), dtype=dtype, device=dev)
        if self.fused_combine:
            ws_bytes = ffn_combine_workspace_bytes(N, E, n_shared, self.nseg, d, I, T, k, self.packed)
        elif fp8_weights is not None:
            ws_bytes = ffn_fp8w_workspace_bytes(N, I, E, n_shared, self.nseg, d, self.packed)
        else:
            ws_bytes = ffn_workspace_bytes(N, E, n_shared, self.nseg, d, I, dtype)
        self.ffn_ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
        self.y = torch.empty((T, d), dtype=dtype, device=dev)
        self.stats_out = None
        self.req_offsets = req_offsets
        if stats_layers:
            R = 0 if req_offsets is None else req_offsets.numel() - 1
            self.stats_out = {}
            self.stats_ws = torch.empty(max(stats_workspace_bytes(stats_layers, T, k, E, R), 256),
                                        dtype=torch.uint8, device=dev)

    def route(self, x):
        return router(x, self.w_router, self.logits)

    def gate(self, logits):
        return gate(logits, self.k, self.renormalize, self.topk_ids, self.topk_w)

    def permute(self, x):
        return permute(self.topk_ids, self.E, self.S, self.P, None if self.fused_gather else x, out=self.perm,
                       workspace=self.perm_ws)

    def ffn_combine(self, x):
        src = x if self.fused_gather else self.perm["x_sorted"]
        return grouped_ffn_combine(src, self.perm["group_offsets"], self.E, self.S, self.nseg, self.w_gate,
                                   self.w_up, self.w_down, self.perm["sorted_to_flat"], self.topk_w, self.y,
                                   self.ffn_ws, x_rows=self.perm["sorted_token"] if self.fused_gather else None,
                                   packed=self.packed)

    def ffn(self, x):
        if self.fp8_weights is not None:
            src = x if self.fused_gather else self.perm["x_sorted"]
            return grouped_ffn_fp8w(src, self.perm["group_offsets"], self.E, self.S, self.nseg, *self.fp8_weights,
                                    h_sorted=self.h_sorted, workspace=self.ffn_ws,
                                    x_rows=self.perm["sorted_token"] if self.fused_gather else None,
                                    packed=self.packed)
        if self.packed:
            src = x if self.fused_gather else self.perm["x_sorted"]
            return grouped_ffn_packed(src, self.perm["group_offsets"], self.E, self.S, self.nseg, self.w_gate,
                                      self.w_up, self.w_down, self.h_sorted, self.ffn_ws,
                                      x_rows=self.perm["sorted_token"] if self.fused_gather else None)
        if self.fused_gather:
            return grouped_ffn(x, self.perm["group_offsets"], self.E, self.S, self.nseg, self.w_gate, self.w_up,
                               self.w_down, self.h_sorted, self.ffn_ws, x_rows=self.perm["sorted_token"])
        return grouped_ffn(self.perm["x_sorted"], self.perm["group_offsets"], self.E, self.S, self.nseg,
                           self.w_gate, self.w_up, self.w_down, self.h_sorted, self.ffn_ws)

    def combine(self):
        return combine(self.h_sorted, self.perm["flat_to_sorted"], self.topk_w, self.S, self.y)

    def stats(self, stats_ids):
        return stats(stats_ids, self.E, self.req_offsets, out=self.stats_out, workspace=self.stats_ws)

    def bound_calls(self, logits, x, stats_ids=None, stream=None, stats_stream=None):
        """Pre-marshalled raw C calls for one forward over fixed buffers.

        Returns a list of (name, fn, args) whose arguments are plain integers,
        so a timing loop pays only the ctypes call per step.  Each entry is one
        of the libmoe calls, in path order (the router first when the layer has
        router weights; the gate then reads the router's logits).  `stats_stream` (a raw stream
        handle) puts the statistics call on its own stream; the caller orders it
        after the gate.
        """
        lib = _lib.load()
        dev = logits.device
        st = _stream(dev) if stream is None else stream
        k, T, E = self.k, self.T, self.E
        dt = _dtype_code(x)
        fused = self.fused_gather
        n_perm = ctypes.c_size_t(self.perm_ws.numel())
        n_ffn = ctypes.c_size_t(self.ffn_ws.numel())
        calls = []
        if self.w_router is not None:
            logits = self.logits
            calls.append(("moe_router", lib.moe_router, (x.data_ptr(), self.w_router.data_ptr(), T, self.d, E, dt,
                                                         logits.data_ptr(), st)))
        calls += [
            ("moe_gate", lib.moe_gate, (logits.data_ptr(), T, E, k, int(bool(self.renormalize)),
                                        self.topk_ids.data_ptr(), self.topk_w.data_ptr(), st)),
            ("moe_permute", lib.moe_permute, (self.topk_ids.data_ptr(), T, E, k, self.S, self.P,
                                              None if fused else x.data_ptr(), dt,
                                              self.d, self.perm["group_offsets"].data_ptr(),
                                              self.perm["sorted_to_flat"].data_ptr(),
                                              self.perm["flat_to_sorted"].data_ptr(),
                                              self.perm["sorted_token"].data_ptr(),
                                              None if fused else self.perm["x_sorted"].data_ptr(),
                                              self.perm_ws.data_ptr(), ctypes.byref(n_perm), st)),
        ]
        if self.fused_combine:
            src = x.data_ptr() if fused else self.perm["x_sorted"].data_ptr()
            calls.append(("moe_grouped_ffn_combine", lib.moe_grouped_ffn_combine, (
                src, self.perm["sorted_token"].data_ptr() if fused else None, T, self.perm["group_offsets"].data_ptr(),
                self.N, E, self.S, self.nseg, self.d, self.I, self.w_gate.data_ptr(), self.w_up.data_ptr(),
                self.w_down.data_ptr(), int(self.packed), self.perm["sorted_to_flat"].data_ptr(),
                self.topk_w.data_ptr(), T, k, self.y.data_ptr(), self.ffn_ws.data_ptr(), ctypes.byref(n_ffn), st)))
        else:
            calls += [
                self._ffn_call(lib, x, fused, dt, n_ffn, st),
                ("moe_combine", lib.moe_combine, (self.h_sorted.data_ptr(), self.perm["flat_to_sorted"].data_ptr(),
                                                  self.topk_w.data_ptr(), T, k, self.S, self.d, dt,
                                                  self.y.data_ptr(), st)),
            ]
        if stats_ids is not None and self.stats_out is not None:
            o = self.stats(stats_ids)          # allocates the outputs once
            L = stats_ids.shape[0]
            R = 0 if self.req_offsets is None else self.req_offsets.numel() - 1
            n_st = ctypes.c_size_t(self.stats_ws.numel())

            def p(key):
                return o[key].data_ptr() if key in o else None
            calls.append(("moe_stats", lib.moe_stats, (
                stats_ids.data_ptr(), L, T, k, E,
                self.req_offsets.data_ptr() if self.req_offsets is not None else None, R, None,
                p("counts"), p("union_size"), p("union_mask"), p("affinity"), p("req_counts"), p("signature"),
                self.stats_ws.data_ptr(), ctypes.byref(n_st), st if stats_stream is None else stats_stream)))
        self._keep = (n_perm, n_ffn, n_st if stats_ids is not None and self.stats_out is not None else None)
        return calls

    def _ffn_call(self, lib, x, fused, dt, n_ffn, st):
        src = x.data_ptr() if fused else self.perm["x_sorted"].data_ptr()
        rows = self.perm["sorted_token"].data_ptr() if fused else None
        offs = self.perm["group_offsets"].data_ptr()
        if self.fp8_weights is not None:
            qg, sg, qu, su, qd, sd = (t.data_ptr() for t in self.fp8_weights)
            name = "moe_grouped_ffn_fp8w_packed" if self.packed else "moe_grouped_ffn_fp8w"
            return (name, getattr(lib, name), (
                src, rows, self.T, offs, self.N, self.E, self.S, self.nseg, self.d, self.I, qg, sg, qu, su, qd, sd,
                self.h_sorted.data_ptr(), self.ffn_ws.data_ptr(), ctypes.byref(n_ffn), st))
        if self.packed:
            return ("moe_grouped_ffn_packed", lib.moe_grouped_ffn_packed, (
                src, rows, self.T, offs, self.N, self.E, self.S, self.nseg, self.d, self.I, self.w_gate.data_ptr(),
                self.w_up.data_ptr(), self.w_down.data_ptr(), self.h_sorted.data_ptr(), self.ffn_ws.data_ptr(),
                ctypes.byref(n_ffn), st))
        return ("moe_grouped_ffn", lib.moe_grouped_ffn, (
            src, rows, self.T, offs, self.N, self.E, self.S, self.nseg, self.d, self.I, self.w_gate.data_ptr(),
            self.w_up.data_ptr(), self.w_down.data_ptr(), dt, self.h_sorted.data_ptr(), self.ffn_ws.data_ptr(),
            ctypes.byref(n_ffn), st))

    def forward(self, logits, x, stats_ids=None, stats_stream=None):
        """Enqueue the layer on the current stream.  With `stats_stream` (a
        torch stream) the statistics run there, concurrently with the permute /
        FFN / combine chain; the current stream waits for them at the end."""
        if self.w_router is not None:
            logits = self.route(x)
        self.gate(logits)
        side = stats_ids is not None and self.stats_out is not None
        if side and stats_stream is not None:
            main = torch.cuda.current_stream(logits.device)
            stats_stream.wait_stream(main)
            with torch.cuda.stream(stats_stream):
                self.stats(stats_ids)
            side = False
        self.permute(x)
        if self.fused_combine:
            self.ffn_combine(x)
        else:
            self.ffn(x)
            self.combine()
        if side:
            self.stats(stats_ids)
        elif stats_ids is not None and self.stats_out is not None:
            torch.cuda.current_stream(logits.device).wait_stream(stats_stream)
        return self.y

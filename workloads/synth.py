"""Seeded synthetic inputs for one MoE layer's expert path.

This module only draws inputs: router logits, hidden states, expert weights and
request boundaries.  It holds none of the layer's arithmetic (no top-k, no
permutation, no FFN, no combine, no statistics), so both the HIP path and the
CPU oracle can consume what it makes without sharing code with each other.

The shapes follow the model table of the GRACE-MoE page ("Experiments":
OLMoE top-8 of 64, DeepSeek-V2-Lite top-6 of 64, Qwen3-30B-A3B top-8 of 128,
batch 128, prefill 64, decode 16), the GPT-OSS-120B scale named on the ELDR page
("Evidence") and the ~6.4 GB-per-layer expert footprint that implies.  The
structure follows what the pages report about expert usage:

* domain locality - same-domain tokens activate a shared expert subset (ELDR
  page, "What it solves"), modelled as a +2.0 bias on a fixed expert subset per
  synthetic domain;
* hot/cold skew - a few experts take most tokens (GRACE-MoE page, section 2 and
  section 3), modelled as a Zipf prior b_e = -s*ln(rank_e) on the logits.

Every tensor comes from a torch.Generator seeded from (workload, tensor name), on
the device asked for.  The same seed gives the same values on the same device
type; tests that compare two implementations generate once and hand the same
tensors to both.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Dict, List, Optional

import torch

SEED_BASE = 0x4D4F4500

# Stats layers for the Qwen3-shaped prefill: 8 of the model's 48 MoE layers,
# evenly spaced (the pages' greedy layer choice needs trained weights).
QWEN3_STATS_LAYERS = (0, 6, 12, 18, 24, 30, 36, 42)


@dataclasses.dataclass(frozen=True)
class Spec:
    """Shape and structure of one synthetic workload."""

    name: str
    index: int              # seeds derive from this
    T: int                  # tokens in the batch
    E: int                  # routed experts
    k: int                  # experts per token
    d: int                  # hidden size
    I: int                  # expert intermediate size
    dtype: str              # "f32" | "bf16": x, expert weights, h, y
    S: int = 0              # always-on shared experts (ids E..E+S-1)
    n_priority: int = 0     # first P tokens form the priority (decode) segment
    renormalize: int = 1
    x_std: float = 1.0
    w_std: Optional[float] = 0.02   # None: N(0, 1/fan_in)
    router_std: Optional[float] = 0.02
    domains: int = 0        # number of synthetic domains (0 = none)
    domain_size: int = 0    # experts per domain subset
    domain_bias: float = 2.0
    token_domain: str = "token"     # "token": t mod D; "request": request r mod D; "one": all 0
    zipf_s: float = 0.0
    stats_layers: int = 1
    req_len: int = 1        # tokens per request (0: one request for the batch)
    pool_T: int = 0         # draw x for this many tokens and take the first T
    mixed_prefill_req: bool = False  # priority tokens are 1-token requests, the rest one request

    @property
    def N(self) -> int:
        return self.T * (self.k + self.S)

    @property
    def nseg(self) -> int:
        return 2 if self.n_priority > 0 else 1

    @property
    def G(self) -> int:
        return self.nseg * self.E + self.S


def _specs() -> Dict[str, Spec]:
    s: Dict[str, Spec] = {}
    s["tiny"] = Spec("tiny", 1, T=64, E=8, k=2, d=128, I=256, dtype="f32",
                     x_std=1.0, w_std=None, router_std=None, req_len=0)
    s["olmoe_decode"] = Spec("olmoe_decode", 2, T=128, E=64, k=8, d=2048, I=1024,
                             dtype="bf16", domains=4, domain_size=16,
                             token_domain="token", req_len=1)
    # same shape, every token from domain 0: shows the union shrinking
    s["olmoe_decode_local"] = dataclasses.replace(
        s["olmoe_decode"], name="olmoe_decode_local", token_domain="one")
    s["qwen3_prefill"] = Spec("qwen3_prefill", 3, T=8192, E=128, k=8, d=2048, I=768,
                              dtype="bf16", domains=16, domain_size=8,
                              token_domain="request", stats_layers=8, req_len=64)
    for t in (16, 64, 128, 256):
        s[f"dsv2_decode_t{t}"] = Spec(f"dsv2_decode_t{t}", 4, T=t, E=64, k=6, d=2048,
                                      I=1408, dtype="bf16", S=2, zipf_s=1.1,
                                      req_len=1, pool_T=256)
    s["gptoss_mixed"] = Spec("gptoss_mixed", 5, T=4160, E=128, k=4, d=2880, I=2880,
                             dtype="bf16", n_priority=64, zipf_s=1.0,
                             mixed_prefill_req=True)
    return s


SPECS: Dict[str, Spec] = _specs()


@dataclasses.dataclass
class Workload:
    spec: Spec
    logits: torch.Tensor            # [T][E] fp32, the layer whose FFN runs
    x: torch.Tensor                 # [T][d] dtype
    w_gate: torch.Tensor            # [E+S][I][d] dtype
    w_up: torch.Tensor              # [E+S][I][d] dtype
    w_down: torch.Tensor            # [E+S][d][I] dtype
    stats_logits: torch.Tensor      # [L][T][E] fp32 (layer 0 is `logits`)
    req_offsets: torch.Tensor       # [R+1] int32
    token_domain: Optional[torch.Tensor] = None   # [T] int64 or None

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.spec.dtype == "f32" else torch.bfloat16


def _seed(spec: Spec, tensor: str, layer: int = 0) -> int:
    h = hashlib.sha256(f"{spec.index}/{tensor}/{layer}".encode()).digest()
    return (SEED_BASE + spec.index) ^ int.from_bytes(h[:6], "little")


def _gen(spec: Spec, tensor: str, device, layer: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(spec, tensor, layer))
    return g


def _normal(shape, std: float, g: torch.Generator, device) -> torch.Tensor:
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return t.mul_(std)


def _expert_weights(spec: Spec, name: str, out_f: int, in_f: int, device,
                    tdt: torch.dtype) -> torch.Tensor:
    """[E+S][out][in], one expert at a time so fp32 staging stays small."""
    n = spec.E + spec.S
    std = spec.w_std if spec.w_std is not None else 1.0 / math.sqrt(in_f)
    w = torch.empty((n, out_f, in_f), dtype=tdt, device=device)
    g = _gen(spec, name, device)
    for e in range(n):
        w[e].copy_(_normal((out_f, in_f), std, g, device))
    return w


def token_domains(spec: Spec, device) -> Optional[torch.Tensor]:
    if spec.domains == 0:
        return None
    t = torch.arange(spec.T, device=device)
    if spec.token_domain == "token":
        return t % spec.domains
    if spec.token_domain == "request":
        return (t // spec.req_len) % spec.domains
    return torch.zeros_like(t)


def request_offsets(spec: Spec) -> torch.Tensor:
    """Request boundaries [R+1] (CPU int32)."""
    T = spec.T
    if spec.mixed_prefill_req:
        offs = list(range(spec.n_priority + 1)) + [T]
    elif spec.req_len == 0:
        offs = [0, T]
    else:
        offs = list(range(0, T + 1, spec.req_len))
        if offs[-1] != T:
            offs.append(T)
    return torch.tensor(offs, dtype=torch.int32)


def _layer_logits(spec: Spec, x: torch.Tensor, layer: int, device,
                  dom: Optional[torch.Tensor]) -> torch.Tensor:
    """Router logits for one layer: fp32(x . W_r^T accumulated in fp64) + bias.

    The router projection sits in front of the path; its output is an input here.
    """
    E, d = spec.E, spec.d
    rstd = spec.router_std if spec.router_std is not None else 1.0 / math.sqrt(d)
    w_r = _normal((E, d), rstd, _gen(spec, "w_router", device, layer), device)
    logits = (x.double() @ w_r.double().t()).float()
    bias = torch.zeros((spec.T, E), dtype=torch.float32, device=device)
    if spec.domains:
        perm = torch.randperm(E, generator=_gen(spec, "domain_perm", "cpu", layer)).to(device)
        subsets = perm[: spec.domains * spec.domain_size].view(spec.domains, spec.domain_size)
        rows = torch.arange(spec.T, device=device).unsqueeze(1).expand(-1, spec.domain_size)
        bias[rows, subsets[dom]] = spec.domain_bias
    if spec.zipf_s:
        rank = torch.randperm(E, generator=_gen(spec, "zipf_rank", "cpu", layer)) + 1
        b = (-spec.zipf_s * torch.log(rank.double())).float().to(device)
        bias += b.unsqueeze(0)
    return logits + bias


def make(name: str, device="cpu", with_weights: bool = True) -> Workload:
    """Build the named workload on `device` (a torch device string)."""
    spec = SPECS[name]
    tdt = torch.float32 if spec.dtype == "f32" else torch.bfloat16
    pool = spec.pool_T or spec.T
    x = _normal((pool, spec.d), spec.x_std, _gen(spec, "x", device), device)[: spec.T]
    x = x.to(tdt).contiguous()
    dom = token_domains(spec, device)
    layers = [_layer_logits(spec, x, l, device, dom) for l in range(spec.stats_layers)]
    stats_logits = torch.stack(layers).contiguous()
    if with_weights:
        w_gate = _expert_weights(spec, "w_gate", spec.I, spec.d, device, tdt)
        w_up = _expert_weights(spec, "w_up", spec.I, spec.d, device, tdt)
        w_down = _expert_weights(spec, "w_down", spec.d, spec.I, device, tdt)
    else:
        empty = torch.empty((0,), dtype=tdt, device=device)
        w_gate = w_up = w_down = empty
    return Workload(spec=spec, logits=stats_logits[0].contiguous(), x=x,
                    w_gate=w_gate, w_up=w_up, w_down=w_down,
                    stats_logits=stats_logits,
                    req_offsets=request_offsets(spec).to(device),
                    token_domain=dom)


def custom(T: int, E: int, k: int, d: int, I: int, dtype: str = "bf16", S: int = 0,
           n_priority: int = 0, seed: int = 0, device="cpu", logit_levels: int = 0,
           zipf_s: float = 0.0, w_std: float = 0.05, stats_layers: int = 1,
           req_len: int = 1) -> Workload:
    """A small workload of any shape, for edge cases and ragged tails.

    logit_levels > 0 quantises the logits to that many values, which makes ties
    between experts common.
    """
    spec = Spec(f"custom{seed}", 100 + seed, T=T, E=E, k=k, d=d, I=I, dtype=dtype, S=S,
                n_priority=n_priority, x_std=1.0, w_std=w_std, router_std=None,
                zipf_s=zipf_s, stats_layers=stats_layers, req_len=req_len)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    x = _normal((T, d), 1.0, _gen(spec, "x", device), device).to(tdt).contiguous()
    layers = []
    for l in range(stats_layers):
        lg = _normal((T, E), 1.0, _gen(spec, "logits", device, l), device)
        if zipf_s:
            rank = torch.randperm(E, generator=_gen(spec, "zipf_rank", "cpu", l)) + 1
            lg = lg + (-zipf_s * torch.log(rank.double())).float().to(device)
        if logit_levels:
            lg = torch.floor(lg * (logit_levels / 4.0)).clamp_(-logit_levels, logit_levels)
        layers.append(lg)
    stats_logits = torch.stack(layers).contiguous()
    w_gate = _expert_weights(spec, "w_gate", I, d, device, tdt)
    w_up = _expert_weights(spec, "w_up", I, d, device, tdt)
    w_down = _expert_weights(spec, "w_down", d, I, device, tdt)
    return Workload(spec=spec, logits=stats_logits[0].contiguous(), x=x, w_gate=w_gate,
                    w_up=w_up, w_down=w_down, stats_logits=stats_logits,
                    req_offsets=request_offsets(spec).to(device))


def random_ids(T: int, E: int, k: int, seed: int, L: int = 1, device="cpu",
               distinct: bool = True) -> torch.Tensor:
    """[L][T][k] int32 expert ids drawn at random (distinct per token if asked)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(SEED_BASE ^ (seed * 7919 + 17))
    if distinct:
        ids = torch.argsort(torch.rand((L, T, E), generator=g), dim=-1)[..., :k]
    else:
        ids = torch.randint(0, E, (L, T, k), generator=g)
    return ids.to(torch.int32).contiguous().to(device)


def content_hash(*tensors: torch.Tensor) -> str:
    """SHA-256 over the raw bytes of the tensors (moved to host)."""
    h = hashlib.sha256()
    for t in tensors:
        c = t.detach().contiguous().cpu()
        if c.dtype == torch.bfloat16:
            c = c.view(torch.int16)
        h.update(c.numpy().tobytes())
    return h.hexdigest()


def names() -> List[str]:
    return list(SPECS)

"""Seeded synthetic inputs for one decode step.

This module only draws random tensors and plants structure in them; it holds
none of the method's arithmetic (no summaries, scores, selection or softmax).
Both the HIP path (through its tests and the benchmark) and the CPU oracle
(through the tests) consume what it produces; neither side generates inputs
of its own.

The workloads stand in for the KV caches of the pages' long reasoning traces
(16K-32K-token AIME / LiveCodeBench generations on Qwen3 models in the Kinetics
news page, section on Qwen3-0.6B throughput; 20K-token traces with 32 heads in
the LessIsMore explainer, section 一).  No dataset or trained weight is used.

Recipe (all normals are float32 N(0,1) rounded to the KV dtype at the end):
* q, K, V ~ N(0,1).
* Planted blocks: for a chosen set of blocks of each (sequence, KV head), each
  key of the block becomes  rho*sqrt(D)*u + sqrt(1-rho^2)*z  where z is its own
  normal draw and u is the unit vector along the sum of that KV group's query
  heads; the cosine between such a key and u is about rho.
* Planted tokens (vote-union workloads): the same, for a chosen set of history
  positions shared by every KV head of a sequence (heads of different groups
  agree on important tokens).
* Outlier channels: a seeded set of channels of every key is multiplied by a
  constant after planting.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    T: int
    dtype: str                 # "f32" or "bf16"
    Bs: int = 16               # block size (block top-k workloads)
    top_k: int = 0             # blocks per (sequence, KV head)
    token_budget: int = 0      # N (vote-union workloads)
    recent_window: int = 0     # W (vote-union workloads)
    plant: str = "none"        # "blocks", "tokens" or "none"
    plant_count: int = 0       # planted blocks per (b, g) or planted positions per b
    rho: float = 0.0
    outlier_channels: int = 0
    outlier_scale: float = 1.0
    seed: int = 0
    Tcap: int = 0              # token capacity of the cache (0: equal to T)
    description: str = ""

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def cap(self) -> int:
        return self.Tcap if self.Tcap else self.T

    @property
    def NB(self) -> int:
        return (self.T + self.Bs - 1) // self.Bs

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads of the build (seed i for workload ci).
WORKLOADS = {
    "c1": Workload("c1", B=2, Hq=4, Hkv=2, D=64, T=1024, dtype="f32", Bs=16, top_k=8, seed=1,
                   description="tiny decode step, fp32, GQA group 2, 64 blocks of 16, top-8"),
    "c2": Workload("c2", B=64, Hq=16, Hkv=8, D=128, T=16384, dtype="bf16", Bs=16, top_k=64,
                   plant="blocks", plant_count=32, rho=0.5, outlier_channels=4, outlier_scale=8.0,
                   seed=2, description="Qwen3-0.6B-shaped layer, block 16, top-64 blocks (1024 tokens)"),
    "c3": Workload("c3", B=32, Hq=32, Hkv=8, D=128, T=32768, dtype="bf16", Bs=32, top_k=64,
                   plant="blocks", plant_count=51, rho=0.3, seed=3,
                   description="Qwen3-8B-shaped layer, block 32, top-64 blocks (2048 tokens)"),
    "c4": Workload("c4", B=16, Hq=32, Hkv=8, D=128, T=20000, dtype="bf16", token_budget=2048,
                   recent_window=512, plant="tokens", plant_count=974, rho=0.3, seed=4,
                   description="vote-union, Qwen3-8B shape, budget 2048 = 1536 voted + 512 recent"),
    "c5": Workload("c5", B=256, Hq=64, Hkv=8, D=128, T=32768, dtype="bf16", Bs=16, top_k=128,
                   plant="blocks", plant_count=102, rho=0.3, seed=5,
                   description="one GPU's per-layer share of batch 2048 x ctx 32768, "
                               "Qwen3-32B shape, block 16, top-128 blocks"),
}


def _normal(gen: torch.Generator, shape, device) -> torch.Tensor:
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def _group_direction(qf: torch.Tensor, Hkv: int) -> torch.Tensor:
    """Unit vector along the sum of each KV group's query heads: [B, Hkv, D]."""
    B, Hq, D = qf.shape
    s = qf.view(B, Hkv, Hq // Hkv, D).sum(dim=2)
    return s / s.norm(dim=-1, keepdim=True).clamp_min(1e-12)


def make_inputs(w: Workload, device: str | torch.device = "cpu", seed: Optional[int] = None,
                batch_slice: Optional[slice] = None):
    """Return dict(q, k, v) for workload `w` on `device`.

    q: [B, Hq, D]; k, v: [B, Hkv, cap, D] in the workload's dtype.  Draws are
    made per sequence in a fixed order from one torch.Generator on `device`,
    so a given (workload, seed, device type) always yields the same bytes.
    Tokens in [T, cap) are drawn too (they are never read).
    ``batch_slice`` builds only those sequences (same bytes as the full build).
    """
    device = torch.device(device)
    seed = w.seed if seed is None else seed
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    B, Hq, Hkv, D, cap = w.B, w.Hq, w.Hkv, w.D, w.cap
    dt = w.torch_dtype

    qf = _normal(gen, (B, Hq, D), device)
    u = _group_direction(qf, Hkv)                      # [B, Hkv, D]
    if w.outlier_channels:
        perm = torch.randperm(D, generator=gen, device=device)
        outl = perm[: w.outlier_channels]
    else:
        outl = None

    bsel = range(B) if batch_slice is None else range(*batch_slice.indices(B))
    nb_out = len(bsel)
    k = torch.empty((nb_out, Hkv, cap, D), dtype=dt, device=device)
    v = torch.empty((nb_out, Hkv, cap, D), dtype=dt, device=device)
    a = w.rho * math.sqrt(D)
    c = math.sqrt(max(0.0, 1.0 - w.rho * w.rho))
    out_i = 0
    for b in range(B):
        kb = _normal(gen, (Hkv, cap, D), device)
        vb = _normal(gen, (Hkv, cap, D), device)
        if w.plant == "blocks" and w.plant_count > 0:
            nb = (w.T + w.Bs - 1) // w.Bs
            mask = torch.zeros((Hkv, cap), dtype=torch.bool, device=device)
            for g in range(Hkv):
                blocks = torch.randperm(nb, generator=gen, device=device)[: w.plant_count]
                tok = (blocks[:, None] * w.Bs + torch.arange(w.Bs, device=device)[None, :]).reshape(-1)
                tok = tok[tok < w.T]
                mask[g, tok] = True
            planted = a * u[b][:, None, :] + c * kb
            kb = torch.where(mask[:, :, None], planted, kb)
        elif w.plant == "tokens" and w.plant_count > 0:
            hist = w.T - w.recent_window
            pos = torch.randperm(hist, generator=gen, device=device)[: w.plant_count]
            mask = torch.zeros((cap,), dtype=torch.bool, device=device)
            mask[pos] = True
            planted = a * u[b][:, None, :] + c * kb
            kb = torch.where(mask[None, :, None], planted, kb)
        if outl is not None:
            kb[:, :, outl] *= w.outlier_scale
        if b in bsel:
            k[out_i] = kb.to(dt)
            v[out_i] = vb.to(dt)
            out_i += 1
    q = qf.to(dt)
    if batch_slice is not None:
        q = q[batch_slice].contiguous()
    return {"q": q.contiguous(), "k": k, "v": v}


def small_workload(**kw) -> Workload:
    """A workload built from keyword arguments (tests use it for small shapes)."""
    base = dict(name="custom", B=1, Hq=2, Hkv=1, D=64, T=64, dtype="bf16", Bs=16, top_k=2, seed=0)
    base.update(kw)
    return Workload(**base)


def integer_inputs(w: Workload, lo: int = -2, hi: int = 2, device="cpu", seed: Optional[int] = None):
    """q, K, V with small integer entries in [lo, hi].  Every dot product and
    every mean of a power-of-two block of them is exact in fp32 and bf16, so
    rankings computed on the GPU and in fp64 agree exactly, ties included."""
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed if seed is None else seed)
    dt = w.torch_dtype
    q = torch.randint(lo, hi + 1, (w.B, w.Hq, w.D), generator=gen, device=device).to(dt)
    k = torch.randint(lo, hi + 1, (w.B, w.Hkv, w.cap, w.D), generator=gen, device=device).to(dt)
    v = torch.randint(lo, hi + 1, (w.B, w.Hkv, w.cap, w.D), generator=gen, device=device).to(dt)
    return {"q": q, "k": k, "v": v}


def to_paged(k: torch.Tensor, v: torch.Tensor, block_size: int, seed: int = 0,
             spare_pages: int = 0):
    """Store contiguous caches k, v [B, Hkv, cap, D] as page pools
    [num_pages, Hkv, Bs, D] (cap a multiple of Bs) with a seeded random page
    order: block j of sequence b goes to page block_table[b, j].  Returns
    (k_pool, v_pool, block_table [B, cap/Bs] int32); the pool has
    `spare_pages` extra pages of noise that no sequence uses.  Only moves
    bytes: the paged cache holds exactly the contiguous cache's tokens."""
    B, Hkv, cap, D = k.shape
    if cap % block_size:
        raise ValueError("cap must be a multiple of the block size")
    nbc = cap // block_size
    num_pages = B * nbc + spare_pages
    gen = torch.Generator(device=k.device)
    gen.manual_seed(seed)
    perm = torch.randperm(num_pages, generator=gen, device=k.device)
    table = perm[: B * nbc].view(B, nbc).to(torch.int32).contiguous()
    spare = perm[B * nbc:].long()
    pools = []
    for x in (k, v):
        pool = torch.empty((num_pages, Hkv, block_size, D), dtype=x.dtype, device=k.device)
        blocks = x.view(B, Hkv, nbc, block_size, D).permute(0, 2, 1, 3, 4)  # [B, nbc, Hkv, Bs, D]
        pool[table.view(-1).long()] = blocks.reshape(B * nbc, Hkv, block_size, D)
        if spare_pages:
            pool[spare] = _normal(gen, (spare_pages, Hkv, block_size, D), k.device).to(x.dtype)
        pools.append(pool)
    return pools[0], pools[1], table


def as_numpy_bits(t: torch.Tensor):
    """CPU numpy view of a tensor's exact bytes: float32 stays float32, bf16
    becomes its uint16 bit patterns (the form the oracle takes)."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    if t.dtype == torch.float32:
        return t.numpy()
    raise TypeError(t.dtype)


def kv_bytes_per_token_per_layer(Hkv: int, D: int, elem_bytes: int = 2) -> int:
    """KV-cache bytes one token adds to one layer: K and V, Hkv heads, D each."""
    return 2 * Hkv * D * elem_bytes

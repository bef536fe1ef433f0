"""Seeded synthetic inputs shaped like the workloads on the reference pages.

This module only draws random inputs and lays out paging metadata (lengths,
block tables, slot mappings).  It contains none of the method's arithmetic (no
scales, no quantization, no attention) and is the only code shared by the GPU
path's tests and the CPU oracle.

Workloads (sizes from the pages' scenarios; the distributions are readings):
  tiny        2 sequences (300, 517 tokens), Hq 4 / Hkv 2, D 64; Q, K, V ~ N(0,1),
              1% of K/V elements x8 (outliers).
  gptoss65k   one gpt-oss-20b-shaped full-attention layer (Hq 64 / Hkv 8, D 64)
              at 65,536 tokens; 0.5% of K/V elements x10.  The video's KV byte
              math (24,576 B/token in BF16 = 12 such layers x 8 heads x 64 dims
              x K,V x 2 B) fixes the head geometry.
  agents126k  4 coding agents x 126,976 tokens, Hq 24 / Hkv 4, D 256; K/V =
              N(0,1) x a per-(head, dim) factor ~ LogUniform(0.1, 4); scales
              calibrated on a separate 8,192-token sample with the same factors.
  mixed64     64 sequences, lengths log-uniform in [1,024, 131,072], Hq 32 /
              Hkv 8, D 128.
  nvfp4_131k  the gptoss65k layer at 131,072 tokens, batch 2.
Every workload uses block size 16 and a random permutation of physical blocks
(make(..., contiguous=True): physical blocks in logical order instead, for
measuring what the scattered placement costs).
The last token of each sequence is the one a decode step writes.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import torch

BLOCK_SIZE = 16


@dataclass
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    block_size: int
    seq_lens: List[int]
    q: torch.Tensor                 # bf16 [B][Hq][D]
    k: torch.Tensor                 # bf16 [T][Hkv][D], sequences back to back
    v: torch.Tensor                 # bf16 [T][Hkv][D]
    slot_mapping: torch.Tensor      # int64 [T]
    block_tables: torch.Tensor      # int32 [B][max_blocks]
    num_blocks: int
    seq_starts: List[int]           # first row of each sequence in k / v
    calib_k: Optional[torch.Tensor] = None  # separate calibration sample, bf16 [Tc][Hkv][D]
    calib_v: Optional[torch.Tensor] = None
    meta: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return int(self.k.shape[0])

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_seq_len(self) -> int:
        return max(self.seq_lens) if self.seq_lens else 0

    def last_token_rows(self) -> torch.Tensor:
        """Row index in k / v of each sequence's newest token (-1 if empty)."""
        return torch.tensor([s + L - 1 if L > 0 else -1 for s, L in zip(self.seq_starts, self.seq_lens)],
                            dtype=torch.int64)

    def prefill_slots(self) -> torch.Tensor:
        """slot_mapping with each sequence's newest token masked out (-1)."""
        sm = self.slot_mapping.clone()
        rows = self.last_token_rows()
        rows = rows[rows >= 0].to(sm.device)
        sm[rows] = -1
        return sm


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, g, device) -> torch.Tensor:
    return torch.randn(*shape, generator=g, device=device, dtype=torch.float32)


def _add_outliers(x: torch.Tensor, frac: float, factor: float, g) -> torch.Tensor:
    """Multiply exactly round(frac * numel) elements, picked by a seeded
    permutation, by `factor` (in fp32, before the single cast to bf16)."""
    n = x.numel()
    cnt = int(round(frac * n))
    if cnt:
        idx = torch.randperm(n, generator=g, device=x.device)[:cnt]
        flat = x.view(-1)
        flat[idx] = flat[idx] * factor
    return x


def _paging(seq_lens: List[int], bs: int, g, device, contiguous: bool = False):
    nblk = [(L + bs - 1) // bs for L in seq_lens]
    num_blocks = max(sum(nblk), 1)
    if contiguous:
        perm = torch.arange(num_blocks)
    else:
        perm = torch.randperm(num_blocks, generator=g, device="cpu" if g.device.type == "cpu" else g.device)
        perm = perm.to("cpu")
    max_blocks = max(max(nblk) if nblk else 1, 1)
    bt = torch.zeros(len(seq_lens), max_blocks, dtype=torch.int32)
    slots = []
    starts = []
    cur_blk = 0
    row = 0
    for b, L in enumerate(seq_lens):
        starts.append(row)
        ids = perm[cur_blk:cur_blk + nblk[b]]
        bt[b, :nblk[b]] = ids.to(torch.int32)
        if L:
            pos = torch.arange(L, dtype=torch.int64)
            slots.append(ids.to(torch.int64)[pos // bs] * bs + pos % bs)
        cur_blk += nblk[b]
        row += L
    slot_mapping = torch.cat(slots) if slots else torch.zeros(0, dtype=torch.int64)
    return bt.to(device), slot_mapping.to(device), num_blocks, starts


def make(name: str, device="cpu", seed: int = 0, seq_lens: Optional[List[int]] = None,
         shape: Optional[dict] = None, contiguous: bool = False) -> Workload:
    """Build a named workload.  `seq_lens` and `shape` (Hq/Hkv/D/B) override the
    defaults to get small instances of the same recipe for parity tests;
    `contiguous` lays the physical blocks out in logical order."""
    device = torch.device(device)
    g = _gen(seed, device)
    cfg = dict(_DEFAULTS[name])
    if shape:
        cfg.update(shape)
    if seq_lens is None:
        seq_lens = _lengths(name, cfg, seed)
    B = len(seq_lens)
    Hq, Hkv, D = cfg["Hq"], cfg["Hkv"], cfg["D"]
    T = sum(seq_lens)
    q = _normal((B, Hq, D), g, device).to(torch.bfloat16)
    calib_k = calib_v = None
    if name == "agents126k":
        fk = torch.exp(torch.empty(Hkv, D, device=device).uniform_(math.log(0.1), math.log(4.0), generator=g))
        fv = torch.exp(torch.empty(Hkv, D, device=device).uniform_(math.log(0.1), math.log(4.0), generator=g))
        k = (_normal((T, Hkv, D), g, device) * fk).to(torch.bfloat16)
        v = (_normal((T, Hkv, D), g, device) * fv).to(torch.bfloat16)
        tc = cfg.get("calib_tokens", 8192)
        calib_k = (_normal((tc, Hkv, D), g, device) * fk).to(torch.bfloat16)
        calib_v = (_normal((tc, Hkv, D), g, device) * fv).to(torch.bfloat16)
    else:
        k = _normal((T, Hkv, D), g, device)
        v = _normal((T, Hkv, D), g, device)
        if cfg.get("outlier_frac"):
            k = _add_outliers(k, cfg["outlier_frac"], cfg["outlier_factor"], g)
            v = _add_outliers(v, cfg["outlier_frac"], cfg["outlier_factor"], g)
        k = k.to(torch.bfloat16)
        v = v.to(torch.bfloat16)
    gp = _gen(seed + 1, torch.device("cpu"))
    bt, sm, nb, starts = _paging(seq_lens, BLOCK_SIZE, gp, device, contiguous)
    return Workload(name=name, B=B, Hq=Hq, Hkv=Hkv, D=D, block_size=BLOCK_SIZE, seq_lens=list(seq_lens),
                    q=q, k=k, v=v, slot_mapping=sm, block_tables=bt, num_blocks=nb, seq_starts=starts,
                    calib_k=calib_k, calib_v=calib_v, meta=dict(cfg))


_DEFAULTS = {
    "tiny": dict(Hq=4, Hkv=2, D=64, outlier_frac=0.01, outlier_factor=8.0),
    "gptoss65k": dict(Hq=64, Hkv=8, D=64, outlier_frac=0.005, outlier_factor=10.0),
    "agents126k": dict(Hq=24, Hkv=4, D=256, calib_tokens=8192),
    "mixed64": dict(Hq=32, Hkv=8, D=128),
    "nvfp4_131k": dict(Hq=64, Hkv=8, D=64, outlier_frac=0.005, outlier_factor=10.0),
}


def _lengths(name: str, cfg: dict, seed: int) -> List[int]:
    if name == "tiny":
        return [300, 517]
    if name == "gptoss65k":
        return [65536]
    if name == "agents126k":
        return [126976] * 4
    if name == "nvfp4_131k":
        return [131072] * 2
    if name == "mixed64":
        gl = _gen(seed + 2, torch.device("cpu"))
        u = torch.rand(64, generator=gl, dtype=torch.float64)
        lo, hi = math.log(1024.0), math.log(131072.0)
        return [int(round(math.exp(lo + (hi - lo) * float(x)))) for x in u]
    raise KeyError(name)


NAMES = tuple(_DEFAULTS)


def mq_queries(w: Workload, q_len: int, seed: int = 0, device=None) -> torch.Tensor:
    """Queries of a multi-query decode step (speculative-decoding
    verification): bf16 [B][q_len][Hq][D] ~ N(0,1), one row per new token.
    The new tokens are the last q_len of each sequence in w (already in the
    cache); row q_len - 1 is w.q."""
    device = w.q.device if device is None else torch.device(device)
    g = _gen(seed + 3, device)
    q = _normal((w.B, q_len, w.Hq, w.D), g, device).to(torch.bfloat16)
    q[:, q_len - 1] = w.q.to(device)
    return q

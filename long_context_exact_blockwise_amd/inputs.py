"""Seeded synthetic inputs for the ring-attention forward, shared by the HIP path's
tests/bench and by the oracle's callers.

This module holds no part of the method's arithmetic: it only draws Gaussian
tensors, casts them and cuts the key/value sequence into position blocks.  It
imports nothing from the HIP binding or from the oracle.

Recipe (one torch.Generator on the target device, seeded): draw Q as fp32
randn in [B, Sq, H, D] order, then all P key blocks as one [B, P*Ck, H, D]
fp32 randn tensor, then the values the same way; multiply by the config's
input scale in fp32; round to the input dtype (round-to-nearest-even for
bf16).  Block j is the slice of positions [j*Ck, (j+1)*Ck).  The local query
chunk sits at block index q_idx, so its global positions start at q_idx*Sq.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "f32" or "bf16" (inputs and output)
    heads: int
    head_dim: int
    q_len: int          # rows of the local query chunk
    kv_len: int         # keys per KV block
    num_blocks: int     # P, the ring size
    causal: bool
    q_idx: int          # block index of the local query chunk
    in_scale: float = 1.0
    batch: int = 1
    host_streamed: bool = False
    q_pos_base: Optional[int] = None  # global position of query row 0 when it is not q_idx * q_len

    @property
    def q_pos0(self) -> int:
        return self.q_idx * self.q_len if self.q_pos_base is None else self.q_pos_base

    def kv_pos0(self, j: int) -> int:
        return j * self.kv_len


# The five workloads: one device's share of the ring at the shapes the pages
# discuss (a 1.3B model at 512K tokens over 4 devices; a 1M-token pass over 128
# devices), plus a small fp32 case the oracle finishes in seconds.
CONFIGS = {
    1: Workload("f32 H1 D64 Q256 P4x256 noncausal", "f32", 1, 64, 256, 256, 4, False, 0),
    2: Workload("bf16 H16 D128 Q32768 P8x32768 causal q_idx7", "bf16", 16, 128, 32768, 32768, 8,
                True, 7, in_scale=1.0 / math.sqrt(2.0)),
    3: Workload("bf16 H16 D128 Q131072 P4x131072 causal q_idx3", "bf16", 16, 128, 131072, 131072, 4,
                True, 3),
    4: Workload("bf16 H32 D128 Q8192 P128x8192 causal q_idx127", "bf16", 32, 128, 8192, 8192, 128,
                True, 127),
    5: Workload("bf16 H16 D128 Q32768 P8x32768 causal q_idx7 host-streamed", "bf16", 16, 128, 32768,
                32768, 8, True, 7, in_scale=1.0 / math.sqrt(2.0), host_streamed=True),
}


def torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


@dataclasses.dataclass
class Inputs:
    wl: Workload
    q: torch.Tensor          # [B, Sq, H, D]
    k: torch.Tensor          # [B, P*Ck, H, D], block j = positions [j*Ck, (j+1)*Ck)
    v: torch.Tensor

    def k_block(self, j: int) -> torch.Tensor:
        return self.k[:, j * self.wl.kv_len:(j + 1) * self.wl.kv_len]

    def v_block(self, j: int) -> torch.Tensor:
        return self.v[:, j * self.wl.kv_len:(j + 1) * self.wl.kv_len]


def make_inputs(wl: Workload, device="cpu", seed: int = 0, q_mult: float = 1.0,
                k_block_mult: Optional[dict] = None) -> Inputs:
    """Draw the workload's Q, K, V.

    q_mult multiplies Q before the cast (a "peaked" softmax variant);
    k_block_mult maps a block index to a multiplier applied to that block's
    keys before the cast (a late jump of the running max).
    """
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    b, h, d = wl.batch, wl.heads, wl.head_dim
    nk = wl.num_blocks * wl.kv_len
    q = torch.randn((b, wl.q_len, h, d), generator=g, device=device, dtype=torch.float32)
    k = torch.randn((b, nk, h, d), generator=g, device=device, dtype=torch.float32)
    v = torch.randn((b, nk, h, d), generator=g, device=device, dtype=torch.float32)
    if wl.in_scale != 1.0:
        q.mul_(wl.in_scale)
        k.mul_(wl.in_scale)
        v.mul_(wl.in_scale)
    if q_mult != 1.0:
        q.mul_(q_mult)
    for j, f in (k_block_mult or {}).items():
        k[:, j * wl.kv_len:(j + 1) * wl.kv_len].mul_(f)
    dt = torch_dtype(wl.dtype)
    return Inputs(wl, q.to(dt), k.to(dt), v.to(dt))


def make_grad(wl: Workload, device="cpu", seed: int = 0) -> torch.Tensor:
    """Upstream gradient dO for the backward pass: fp32 randn in Q's shape
    [B, Sq, H, D] from its own seeded generator, rounded to the input dtype."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    do = torch.randn((wl.batch, wl.q_len, wl.heads, wl.head_dim), generator=g, device=device, dtype=torch.float32)
    return do.to(torch_dtype(wl.dtype))


@dataclasses.dataclass(frozen=True)
class FfnWorkload:
    name: str
    rows: int
    d_model: int
    d_ff: int
    block_rows: int


# The feedforward of the 1.3B model's layer (hidden dim 2048, 4x expansion)
# over the 128K-token chunk of a 512K sequence on 4 devices, in blocks of 16K
# rows (a 256 MiB hidden activation per block instead of 2 GiB for the chunk).
FFN_CONFIG = FfnWorkload("bf16 FFN rows131072 d2048 f8192 block16384", 131072, 2048, 8192, 16384)


def make_ffn_inputs(rows: int, d_model: int, d_ff: int, device="cpu", seed: int = 0):
    """x [rows, d] ~ N(0, 1); W1 [F, d] ~ N(0, 1/d); b1 [F] ~ N(0, 0.1^2);
    W2 [d, F] ~ N(0, 1/F); b2 [d] ~ N(0, 0.1^2): fp32 randn in that order
    from one seeded generator, scaled in fp32, rounded to bf16."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn((rows, d_model), generator=g, device=device, dtype=torch.float32)
    w1 = torch.randn((d_ff, d_model), generator=g, device=device, dtype=torch.float32) / math.sqrt(d_model)
    b1 = torch.randn((d_ff,), generator=g, device=device, dtype=torch.float32) * 0.1
    w2 = torch.randn((d_model, d_ff), generator=g, device=device, dtype=torch.float32) / math.sqrt(d_ff)
    b2 = torch.randn((d_model,), generator=g, device=device, dtype=torch.float32) * 0.1
    return tuple(t.to(torch.bfloat16) for t in (x, w1, b1, w2, b2))


def sample_rows(q_len: int, extra: int = 8, seed: int = 1):
    """Rows checked at full size: the first, the last and `extra` seeded rows."""
    import numpy as np
    rng = np.random.default_rng(seed)
    rows = {0, q_len - 1}
    rows.update(int(r) for r in rng.integers(0, q_len, size=extra))
    return sorted(rows)


def to_f64(t: torch.Tensor):
    """Exact widening of a (CPU or GPU) tensor to a float64 numpy array."""
    return t.detach().to("cpu", torch.float32).double().numpy()

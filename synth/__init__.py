"""Seeded synthetic workloads for NABLA attention.

This module is shared by the HIP path's tests/bench and by the oracle's tests.
It holds workload shapes and a seeded random-field generator only: no step of
the attention method (no reorder, pooling, masking or attention arithmetic)
lives here.

Inputs imitate the attention shapes of the Wan 2.1 14B video DiT that the
NABLA pages evaluate on (40 heads, head_dim 128, 720p and 480p latents); the
model weights are not used.  Each of Q, K, V is a smooth spatio-temporal random
field (an N(0,1) control grid upsampled trilinearly with align_corners=True)
scaled by a gain, plus 0.5 * N(0,1) per-token noise, drawn per head.

Tensors are produced in the natural layout ``[B, heads, T, H, W, d]`` (valid
extents only; padding to a multiple of the patch side is the attention
library's business) and rounded once to the config dtype.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence, Tuple

import numpy as np
import torch

__all__ = ["Config", "CONFIGS", "config", "make_qkv", "make_tensor", "sampled_heads"]


@dataclasses.dataclass(frozen=True)
class Config:
    """One workload: geometry, dtype, threshold, STA window and generator knobs."""

    name: str
    batch: int
    heads: int
    head_dim: int
    dtype: str            # "fp32" or "bf16"
    T: int                # frames
    H: int                # valid latent height
    W: int                # valid latent width
    P: int                # patch side; blocks hold P*P tokens
    thr: float
    sta: Tuple[int, int, int]   # STA window in blocks (t, h, w); (0,0,0) = off
    seed: int
    ctrl: Tuple[int, int, int]  # control-grid size (t, h, w)
    gain_qk: float        # field gain for Q and K
    gain_v: float         # field gain for V
    noise: float = 0.5
    oracle_heads: int = 0  # heads the oracle checks at full size (0 = all)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16

    @property
    def Hp(self) -> int:
        return -(-self.H // self.P) * self.P

    @property
    def Wp(self) -> int:
        return -(-self.W // self.P) * self.P

    @property
    def nblocks(self) -> int:
        return self.T * (self.Hp // self.P) * (self.Wp // self.P)

    @property
    def seq_padded(self) -> int:
        return self.nblocks * self.P * self.P

    def with_(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


# Field gain for Q/K.  The configs fix the generator's form but not its
# amplitude except for Tiny (an N(0,1) field); 2.5 puts the 720p layer near the
# ~80% block sparsity it targets at thr=0.7 (calibrated with the oracle).
_G = 2.5

CONFIGS = {
    "tiny": Config("tiny", 1, 2, 64, "fp32", 4, 16, 16, 8, 0.8, (0, 0, 0), 0,
                   (4, 4, 4), 1.0, 1.0),
    "small": Config("small", 1, 8, 128, "bf16", 8, 32, 32, 8, 0.8, (0, 0, 0), 1,
                    (8, 8, 8), _G, 1.0),
    "480p": Config("480p", 1, 40, 128, "bf16", 21, 30, 52, 8, 0.9, (3, 3, 3), 2,
                   (8, 8, 8), _G, 1.0, oracle_heads=4),
    "720p": Config("720p", 1, 40, 128, "bf16", 21, 45, 80, 8, 0.7, (3, 3, 3), 3,
                   (8, 8, 8), _G, 1.0, oracle_heads=4),
    "long": Config("long", 1, 40, 128, "bf16", 41, 45, 80, 8, 0.7, (3, 3, 3), 4,
                   (8, 8, 8), _G, 1.0, oracle_heads=2),
}


def config(name: str, **overrides) -> Config:
    c = CONFIGS[name]
    return c.with_(**overrides) if overrides else c


def _field_head(gen: torch.Generator, cfg: Config, gain: float, device) -> torch.Tensor:
    """One head's smooth field + noise, float32, shape [T, H, W, d]."""
    d = cfg.head_dim
    ct, ch, cw = cfg.ctrl
    grid = torch.randn((1, d, ct, ch, cw), generator=gen, device=device, dtype=torch.float32)
    field = torch.nn.functional.interpolate(
        grid, size=(cfg.T, cfg.H, cfg.W), mode="trilinear", align_corners=True)[0]
    field = field.permute(1, 2, 3, 0)  # [T, H, W, d]
    noise = torch.randn((cfg.T, cfg.H, cfg.W, d), generator=gen, device=device,
                        dtype=torch.float32)
    return gain * field + cfg.noise * noise


def make_tensor(cfg: Config, tensor_id: int, device="cpu",
                heads: Optional[Sequence[int]] = None) -> torch.Tensor:
    """Seeded tensor ``tensor_id`` (0=Q, 1=K, 2=V) in layout [B, h, T, H, W, d].

    The stream is seeded by (config seed, tensor id); heads are drawn in order,
    so a given device always reproduces the same values.  ``heads`` restricts
    the output to a subset (still drawing the skipped heads' values so that the
    subset equals the corresponding slice of the full tensor).
    """
    gen = torch.Generator(device=device)
    gen.manual_seed(1_000_003 * cfg.seed + 7919 * tensor_id + 17)
    gain = cfg.gain_v if tensor_id == 2 else cfg.gain_qk
    want = list(range(cfg.heads)) if heads is None else sorted(heads)
    out = torch.empty((cfg.batch, len(want), cfg.T, cfg.H, cfg.W, cfg.head_dim),
                      dtype=cfg.torch_dtype, device=device)
    for b in range(cfg.batch):
        j = 0
        for h in range(cfg.heads):
            x = _field_head(gen, cfg, gain, device)
            if h in want:
                out[b, j] = x.to(cfg.torch_dtype)
                j += 1
    return out


def make_qkv(cfg: Config, device="cpu", heads: Optional[Sequence[int]] = None):
    """(Q, K, V) for ``cfg`` in layout [B, h, T, H, W, d] and the config dtype."""
    return tuple(make_tensor(cfg, i, device, heads) for i in range(3))


def sampled_heads(cfg: Config, n: Optional[int] = None) -> list:
    """Heads checked by the oracle at full size, drawn from the config seed."""
    n = cfg.oracle_heads if n is None else n
    if n <= 0 or n >= cfg.heads:
        return list(range(cfg.heads))
    rng = np.random.default_rng([cfg.seed, 99])
    return sorted(int(h) for h in rng.choice(cfg.heads, size=n, replace=False))

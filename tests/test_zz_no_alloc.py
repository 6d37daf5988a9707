"""nabla_forward_noalloc (library-owned scratch array, allocates nothing)
against nabla_forward (caller workspace), both through the C ABI: outputs
equal bit for bit, on calls in a row where the second input is smaller than
the first, then a larger batched one and a float32 call."""
import math

import pytest
import torch

import block_sparse_attention_flatten_amd as nabla
import synth
from gpu_helpers import geom_of, log

pytestmark = pytest.mark.gpu

CASES = [
    # 720p shape with 20 heads: more heads than the scratch array holds at once
    synth.config("720p", heads=20),
    # smaller, with ragged edge blocks
    synth.config("small", heads=3, T=3, H=20, W=28),
    # batch 2 x 6 heads at the 720p shape: a pass boundary inside the second
    # batch entry's heads
    synth.config("720p", batch=2, heads=6),
    # float32 inputs (no V^T part), no STA window
    synth.config("tiny"),
]


def _bits(x: torch.Tensor) -> torch.Tensor:
    return x.view(torch.int16 if x.dtype == torch.bfloat16 else torch.int32)


def test_noalloc_equals_forward():
    for cfg in CASES:
        log(f"noalloc: {cfg.name} heads={cfg.heads} THW=({cfg.T},{cfg.H},{cfg.W}) "
            f"d={cfg.head_dim} {cfg.dtype}")
        q, k, v = synth.make_qkv(cfg, device="cuda")
        g = geom_of(cfg)
        scale = 1.0 / math.sqrt(cfg.head_dim)
        o = torch.full(q.shape, float("nan"), dtype=g.odtype, device="cuda")
        nabla.nabla_forward_noalloc(g, q, k, v, cfg.thr, cfg.sta, scale, o)
        size, _ = nabla.nabla_forward_workspace_size(g)
        ws = torch.empty(size, dtype=torch.uint8, device="cuda")
        ref = torch.empty(q.shape, dtype=g.odtype, device="cuda")
        nabla.nabla_forward(g, q, k, v, cfg.thr, cfg.sta, scale, ref, ws)
        torch.cuda.synchronize()
        assert torch.isfinite(ref).all()
        assert torch.equal(_bits(o), _bits(ref)), cfg.name
        del ws
        log(f"noalloc: {cfg.name} equal")

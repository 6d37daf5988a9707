"""Shared helpers of the GPU parity tests (HIP path vs the float64 oracle)."""
from __future__ import annotations

import math
import sys
import time

import numpy as np
import torch

import block_sparse_attention_flatten_amd as nabla
import oracle as O
import synth

# tolerances fixed for bf16 inputs against the float64 oracle; float32 inputs
# are held to a bound derived from fp32 accumulation over a few thousand keys
BF16_MAX_ABS, BF16_MEAN_ABS = 1e-2, 1e-3
F32_MAX_ABS, F32_MEAN_ABS = 2e-5, 2e-6
BAND_EPS = 1e-5


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def geom_of(cfg: synth.Config, layout=nabla.LAYOUT_THW, out_dtype=None) -> nabla.Geometry:
    return nabla.Geometry(cfg.batch, cfg.heads, cfg.T, cfg.H, cfg.W, cfg.head_dim,
                          cfg.torch_dtype, layout, out_dtype=out_dtype)


def ogeom(cfg: synth.Config) -> O.Geometry:
    return O.Geometry(cfg.T, cfg.H, cfg.W, cfg.P)


def unpack_bits(words: torch.Tensor, nb: int) -> np.ndarray:
    """int32 words [..., nb, nw] -> bool [..., nb, nb]."""
    w = words.cpu().numpy().view(np.uint32)
    bits = np.unpackbits(w.view(np.uint8), axis=-1, bitorder="little")
    return bits[..., :nb].astype(bool)


def f64(x: torch.Tensor) -> np.ndarray:
    return x.detach().to(torch.float64).cpu().numpy()


def tol(dtype: torch.dtype):
    return (BF16_MAX_ABS, BF16_MEAN_ABS) if dtype == torch.bfloat16 else (F32_MAX_ABS, F32_MEAN_ABS)


def run_pipeline(cfg: synth.Config, q, k, v, layout=nabla.LAYOUT_THW, thr=None, sta=None,
                 out_dtype=torch.float32, also_bf16=False, attn="vt", fused=True):
    """Run mask construction and attention through the C ABI.  By default the
    launch sequence bench.py times: nabla_mask_build (pooling, mask and
    lists in one call) and, for bf16 inputs, nabla_transpose_v + nabla_attn_fwd_vt;
    fused=False calls nabla_pool, nabla_mask and nabla_compact one by one,
    attn="tr" selects nabla_attn_fwd.  The output is float32 by default (the
    kernel's result before any rounding to bf16); with ``also_bf16`` the
    attention is run a second time writing bf16 (o_bf16)."""
    g = geom_of(cfg, layout, out_dtype)
    thr = cfg.thr if thr is None else thr
    sta = cfg.sta if sta is None else sta
    dev = q.device
    B, h, nb, d = cfg.batch, cfg.heads, g.nb, cfg.head_dim
    qbar = torch.empty(nabla.qbar_shape(g), dtype=torch.float32, device=dev)
    kbar = torch.empty(nabla.kbar_shape(g), dtype=nabla.KBAR_DTYPE, device=dev)
    bits = torch.empty((B, h, nb, g.nw), dtype=torch.int32, device=dev)
    abits = torch.empty_like(bits)
    cnt = torch.empty((B, h, nb), dtype=torch.int32, device=dev)
    rp = torch.empty((B * h, nb + 1), dtype=torch.int32, device=dev)
    ci = torch.empty((B * h, nb * nb), dtype=torch.int32, device=dev)
    o = torch.empty(q.shape, dtype=g.odtype, device=dev)
    if fused:
        nabla.nabla_mask_build(g, q, k, thr, sta, qbar, kbar, bits, cnt, abits, rp, ci)
    else:
        nabla.nabla_pool(g, q, k, qbar, kbar)
        nabla.nabla_mask(g, qbar, kbar, thr, sta, bits, cnt, abits)
        nabla.nabla_compact(g, bits, cnt, rp, ci)
    use_vt = attn == "vt" and q.dtype == torch.bfloat16
    vt = None
    if use_vt:
        vt = torch.empty(nabla.vt_shape(g), dtype=q.dtype, device=dev)
        nabla.nabla_transpose_v(g, v, vt)

    def attention(geom, out):
        if use_vt:
            nabla.nabla_attn_fwd_vt(geom, q, k, vt, rp, ci, 1.0 / math.sqrt(d), out)
        else:
            nabla.nabla_attn_fwd(geom, q, k, v, rp, ci, 1.0 / math.sqrt(d), out)

    attention(g, o)
    out = dict(g=g, qbar=qbar, kbar=kbar, bits=bits, abits=abits, cnt=cnt, rp=rp, ci=ci, o=o)
    if also_bf16 and q.dtype == torch.bfloat16:
        gb = geom_of(cfg, layout, torch.bfloat16)
        ob = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
        attention(gb, ob)
        out["o_bf16"] = ob
    torch.cuda.synchronize()
    return out


def check_bf16_rounding(res) -> None:
    """The bf16 output is the float32 result rounded once to nearest even."""
    if "o_bf16" in res:
        want = res["o"].to(torch.bfloat16)
        assert torch.equal(res["o_bf16"].view(torch.int16), want.view(torch.int16)), \
            "bf16 output is not the float32 result rounded to nearest even"


def oracle_mask(cfg: synth.Config, q_h: np.ndarray, k_h: np.ndarray, thr=None, sta=None):
    """Oracle pooling + mask for one head ([T, H, W, d] float64 inputs)."""
    g = ogeom(cfg)
    valid = O.valid_tokens(g)
    qbar = O.pool(O.flatten(q_h, g), valid)
    kbar = O.pool(O.flatten(k_h, g), valid)
    thr = cfg.thr if thr is None else thr
    sta = cfg.sta if sta is None else sta
    m, m_ad, p = O.nabla_mask(qbar, kbar, thr, g, sta)
    band_a, band_b = O.band_rows(p, m_ad, thr, BAND_EPS)
    return dict(qbar=qbar, kbar=kbar, mask=m, mask_adaptive=m_ad, p=p, band=band_a | band_b,
                band_a=band_a, band_b=band_b, valid=valid)


def check_mask_rows(got_union, got_adapt, ref, thr, label=""):
    """Masks must agree bit for bit outside band rows.  On band rows that
    differ, the GPU's adaptive set must still be a valid cut under the
    oracle's probabilities to within the band.  Returns (#band rows, #differing)."""
    p = ref["p"]
    diff = (got_adapt != ref["mask_adaptive"]).any(1) | (got_union != ref["mask"]).any(1)
    bad = diff & ~ref["band"]
    assert not bad.any(), (f"{label}: mask differs outside the band on rows "
                           f"{np.flatnonzero(bad)[:10].tolist()}")
    for r in np.flatnonzero(diff):
        keep = got_adapt[r]
        mass = p[r][keep].sum()
        assert keep.any() and mass >= thr - BAND_EPS, (label, r, mass)
        assert mass - p[r][keep].min() < thr + BAND_EPS, (label, r)
    return int(ref["band"].sum()), int(diff.sum())


def check_output(got: np.ndarray, ref: np.ndarray, dtype, label=""):
    max_abs, mean_abs = tol(dtype)
    err = np.abs(got - ref)
    assert np.isfinite(got).all(), f"{label}: non-finite output"
    assert err.max() <= max_abs and err.mean() <= mean_abs, (
        f"{label}: max|err| {err.max():.3e} mean|err| {err.mean():.3e}")
    return float(err.max()), float(err.mean())


def gpu_mask_for_oracle(ref, union: np.ndarray) -> np.ndarray:
    """The mask the oracle's attention is compared under: the oracle's own
    mask, with the band rows where the GPU chose a different (valid) cut
    replaced by the GPU's rows, so that every output row can be compared."""
    m = ref["mask"].copy()
    diff = (union != m).any(1)
    assert not (diff & ~ref["band"]).any()
    m[diff] = union[diff]
    return m

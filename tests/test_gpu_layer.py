"""A DiT self-attention layer around NABLA with the token sequence kept in the
blocked (fractal-flattened) order across the network: QKV = X W_qkv (a
library GEMM), nabla_qkv_split (head-major q, k, V^T and block means in one
pass), mask, lists and attention in the blocked layout, then O W_o.  The
NABLA output is compared with the float64 oracle run on the projected q, k, v
of every head, masks included; the fused pass is checked bit for bit against
the separate calls it replaces (copies, nabla_transpose_v, nabla_pool)."""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_flatten_amd as nabla
import oracle as O
import synth
from gpu_helpers import (BAND_EPS, check_mask_rows, check_output, f64, gpu_mask_for_oracle, log,
                         ogeom, unpack_bits)

pytestmark = pytest.mark.gpu

CASES = {
    # ragged latent (H, W not multiples of 8), d = 128, STA window
    "ragged_d128": ("small", dict(heads=4, T=3, H=20, W=28, thr=0.7, sta=(3, 3, 3))),
    # batch 2, d = 64, asymmetric window
    "batch2_d64": ("small", dict(batch=2, heads=3, T=4, H=16, W=24, head_dim=64, thr=0.8,
                                 sta=(1, 3, 3))),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_layer(name):
    base, kw = CASES[name]
    cfg = synth.config(base, **kw)
    log(f"layer {name}: {cfg}")
    B, h, d = cfg.batch, cfg.heads, cfg.head_dim
    g = nabla.Geometry(B, h, cfg.T, cfg.H, cfg.W, d, torch.bfloat16, nabla.LAYOUT_BLOCKED,
                       out_dtype=torch.float32)
    nb, S, Dm = g.nb, g.nb * 64, h * d
    dev = "cuda"
    # X: the config's smooth synthetic field in the blocked token order
    # (token-major, pad slots zero), random N(0, 1/Dm) projection weights
    field = synth.make_tensor(cfg, 0, device=dev)
    xb = torch.zeros(g.tensor_shape(), dtype=torch.bfloat16, device=dev)
    nabla.nabla_flatten(g.with_layout(nabla.LAYOUT_THW), field, xb)
    X = xb.permute(0, 2, 3, 1, 4).reshape(B, S, Dm).contiguous()
    gen = torch.Generator(device=dev)
    gen.manual_seed(4321)
    Wqkv = (torch.randn(Dm, 3 * Dm, generator=gen, device=dev) / math.sqrt(Dm)).to(torch.bfloat16)
    Wo = (torch.randn(Dm, Dm, generator=gen, device=dev) / math.sqrt(Dm)).to(torch.bfloat16)
    qkv = torch.matmul(X, Wqkv).view(nabla.qkv_shape(g))

    q = torch.empty(g.tensor_shape(), dtype=torch.bfloat16, device=dev)
    k = torch.empty_like(q)
    vt = torch.empty(nabla.vt_shape(g), dtype=torch.bfloat16, device=dev)
    qbar = torch.empty(nabla.qbar_shape(g), dtype=torch.float32, device=dev)
    kbar = torch.empty(nabla.kbar_shape(g), dtype=nabla.KBAR_DTYPE, device=dev)
    nabla.nabla_qkv_split(g, qkv, q, k, vt, qbar, kbar)
    bits = torch.empty((B, h, nb, g.nw), dtype=torch.int32, device=dev)
    abits = torch.empty_like(bits)
    cnt = torch.empty((B, h, nb), dtype=torch.int32, device=dev)
    rp = torch.empty((B * h, nb + 1), dtype=torch.int32, device=dev)
    ci = torch.empty((B * h, nb * nb), dtype=torch.int32, device=dev)
    nabla.nabla_mask(g, qbar, kbar, cfg.thr, cfg.sta, bits, cnt, abits)
    nabla.nabla_compact(g, bits, cnt, rp, ci)
    o = torch.empty(g.tensor_shape(), dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(d)
    nabla.nabla_attn_fwd_vt(g, q, k, vt, rp, ci, scale, o)
    y = torch.matmul(o.to(torch.bfloat16).permute(0, 2, 3, 1, 4).reshape(B, S, Dm), Wo)

    # the separate calls the fused pass replaces
    heads_major = qkv.permute(2, 0, 3, 1, 4).reshape(3, B, h, nb, 64, d)
    v = heads_major[2].contiguous()
    vt_ref = torch.empty_like(vt)
    nabla.nabla_transpose_v(g, v, vt_ref)
    qbar_ref = torch.empty_like(qbar)
    kbar_ref = torch.empty_like(kbar)
    nabla.nabla_pool(g, heads_major[0].contiguous(), heads_major[1].contiguous(), qbar_ref,
                     kbar_ref)
    torch.cuda.synchronize()
    i16 = torch.int16
    assert torch.equal(q.view(i16), heads_major[0].contiguous().view(i16))
    assert torch.equal(k.view(i16), heads_major[1].contiguous().view(i16))
    assert torch.equal(vt.view(i16), vt_ref.view(i16))
    assert torch.equal(qbar.view(torch.int32), qbar_ref.view(torch.int32))
    # pooled keys: the rows of the blocks (rows past nb in the last tile are unwritten)
    assert torch.equal(nabla.kbar_untile(kbar, nb).contiguous().view(torch.int32),
                       nabla.kbar_untile(kbar_ref, nb).contiguous().view(torch.int32))

    og = ogeom(cfg)
    valid = O.valid_tokens(og)
    Wo64 = f64(Wo)
    for b in range(B):
        o_ref_tok = np.zeros((nb, 64, h, d))
        for hh in range(h):
            qh, kh, vh = (f64(x[b, hh]) for x in (q, k, v))     # [nb, 64, d], blocked order
            qb_, kb_ = O.pool(qh, valid), O.pool(kh, valid)
            assert np.abs(f64(qbar[b, hh]) - qb_).max() <= 64 * 2.0 ** -24 * np.abs(qh).max()
            m, m_ad, p = O.nabla_mask(qb_, kb_, cfg.thr, og, cfg.sta)
            band_a, band_b = O.band_rows(p, m_ad, cfg.thr, BAND_EPS)
            ref = dict(mask=m, mask_adaptive=m_ad, p=p, band=band_a | band_b, valid=valid)
            union = unpack_bits(bits[b, hh], nb)
            adapt = unpack_bits(abits[b, hh], nb)
            nbnd, ndf = check_mask_rows(union, adapt, ref, cfg.thr, f"{name} b{b} h{hh}")
            mm = gpu_mask_for_oracle(ref, union)
            ob = O.block_sparse_attention(qh, kh, vh, mm, valid)
            got = f64(o[b, hh])
            e = check_output(got[valid], ob[valid], torch.bfloat16, f"{name} b{b} h{hh}")
            assert np.all(got[~valid] == 0.0)        # pad queries of the blocked layout
            o_ref_tok[:, :, hh] = ob
            log(f"layer {name} b{b} h{hh}: sparsity {1 - union.mean():.3f} band {nbnd} "
                f"diff {ndf} max|err| {e[0]:.2e} mean|err| {e[1]:.2e}")
        # output projection of the layer: the bf16 rounding of O and the GEMM's
        # bf16 output bound the difference to a few bf16 ulps of |y|
        y_ref = o_ref_tok.reshape(S, Dm) @ Wo64
        yv = f64(y[b]).reshape(nb, 64, Dm)[valid]
        yr = y_ref.reshape(nb, 64, Dm)[valid]
        err = np.abs(yv - yr).max() / np.abs(yr).max()
        log(f"layer {name} b{b}: output projection max rel err {err:.2e}")
        assert err < 2e-2

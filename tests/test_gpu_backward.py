"""GPU parity of the gradient calls (mask held fixed) against the float64
oracle: transposed mask (bit-exact), key-major lists (bit-exact), the
forward's log-sum-exp, D = rowsum(dO * O), and dq, dk, dv.

The oracle differentiates the attention under its own mask.  Mask rows may
differ only inside the band (the CDF crossing within 1e-5 of thr, checked
here and in test_gpu_parity.py); as for the forward, such a row is taken from
the GPU's mask for the gradient comparison.

Gradient tolerances.  bf16: every gradient element is an fp32 sum of bf16
products, and the weights p and dS enter the matrix cores rounded to bf16
(relative error 2^-9 each), as do the outputs; over n kept keys the rounding
errors add up like a random walk, so the expected relative error is a few
2^-9 of the gradient's scale.  The bars, relative to max|reference| of each
tensor: max |err| <= 2e-2, mean |err| <= 2e-3 (about 10 and 1 units of 2^-9).
float32: max |err| <= 1e-4 and mean <= 1e-5 relative (fp32 sums over a few
thousand terms)."""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_flatten_amd as nabla
import oracle as O
import synth
from gpu_helpers import (check_mask_rows, f64, geom_of, log, ogeom, oracle_mask, run_pipeline,
                         unpack_bits)

pytestmark = pytest.mark.gpu

CASES = {
    "tiny_f32": ("tiny", {}),
    "ragged_bf16": ("small", dict(batch=2, heads=2, T=3, H=13, W=21, thr=0.6, sta=(1, 3, 3))),
    "small_bf16": ("small", dict(heads=2)),
    "d64_bf16": ("small", dict(heads=2, T=4, H=24, W=40, head_dim=64, thr=0.8, sta=(3, 3, 3))),
    "ragged_f32": ("tiny", dict(batch=1, heads=2, T=2, H=11, W=17, head_dim=128, thr=0.7,
                                sta=(3, 3, 3))),
    "thr_one_bf16": ("small", dict(heads=1, T=2, H=16, W=24, thr=1.0)),
    "hot_bf16": ("small", dict(heads=2, T=3, H=16, W=24, thr=0.7, sta=(3, 3, 3), gain_qk=8.0)),
    "flat_bf16": ("small", dict(heads=1, T=2, H=16, W=24, thr=0.5, gain_qk=0.0, noise=0.0)),
}
REL = {torch.bfloat16: (2e-2, 2e-3), torch.float32: (1e-4, 1e-5)}


def _run(cfg, layout):
    q, k, v = synth.make_qkv(cfg, device="cuda")
    q_thw, k_thw = q, k
    dout = synth.make_tensor(cfg, 3, device="cuda")
    if layout == nabla.LAYOUT_BLOCKED:
        gt = geom_of(cfg)
        blk = lambda x: _to_blocked(gt, x)   # noqa: E731
        q, k, v, dout = blk(q), blk(k), blk(v), blk(dout)
    g = geom_of(cfg, layout, q.dtype)
    res = run_pipeline(cfg, q, k, v, layout=layout, out_dtype=q.dtype)
    d = cfg.head_dim
    scale = 1.0 / math.sqrt(d)
    o = torch.empty_like(q)
    lse = torch.full(nabla.lse_shape(g), 123.0, dtype=torch.float32, device="cuda")
    if q.dtype == torch.bfloat16:
        vt = torch.empty(nabla.vt_shape(g), dtype=q.dtype, device="cuda")
        nabla.nabla_transpose_v(g, v, vt)
        nabla.nabla_attn_fwd_vt_lse(g, q, k, vt, res["rp"], res["ci"], scale, o, lse)
    else:
        nabla.nabla_attn_fwd_lse(g, q, k, v, res["rp"], res["ci"], scale, o, lse)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16) if o.dtype == torch.bfloat16 else o,
                       res["o"].view(torch.int16) if o.dtype == torch.bfloat16 else res["o"]), \
        "the lse variant must write the same output"
    bw = nabla.backward(g, q, k, v, o, lse, dout, res["bits"], res["rp"], res["ci"], scale)
    torch.cuda.synchronize()
    return g, q, k, v, dout, o, lse, res, bw, q_thw, k_thw


def _to_blocked(g, x):
    xb = torch.zeros(g.tensor_shape(nabla.LAYOUT_BLOCKED), dtype=x.dtype, device=x.device)
    nabla.nabla_flatten(g, x, xb)
    return xb


def _blocked_np(cfg, layout, x, og):
    """[B, h, ...] device tensor -> float64 [B, h, nb, 64, d]."""
    a = f64(x)
    if layout == nabla.LAYOUT_BLOCKED:
        return a
    B, h = a.shape[:2]
    return np.stack([np.stack([O.flatten(a[b, i], og) for i in range(h)]) for b in range(B)])


def _rel_check(got, ref, dtype, label):
    mx, mn = REL[dtype]
    scale = max(float(np.abs(ref).max()), 1e-30)
    err = np.abs(got - ref)
    assert np.isfinite(got).all(), f"{label}: non-finite values"
    assert err.max() <= mx * scale and err.mean() <= mn * scale, (
        f"{label}: max|err| {err.max():.3e} mean|err| {err.mean():.3e} (scale {scale:.3e})")
    return err.max() / scale, err.mean() / scale


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("layout", [nabla.LAYOUT_THW, nabla.LAYOUT_BLOCKED],
                         ids=["thw", "blocked"])
def test_backward_matches_oracle(name, layout):
    base, kw = CASES[name]
    cfg = synth.config(base, **kw)
    log(f"backward case {name} layout {layout}: {cfg}")
    g, q, k, v, dout, o, lse, res, bw, q_thw, k_thw = _run(cfg, layout)
    og = ogeom(cfg)
    valid = O.valid_tokens(og)
    nb = g.nb
    bits = unpack_bits(res["bits"], nb)                          # [B, h, nb, nb]
    bits_t = torch.empty_like(res["bits"])
    cnt_t = torch.empty_like(res["cnt"])
    nabla.nabla_mask_transpose(g, res["bits"], bits_t, cnt_t)
    torch.cuda.synchronize()
    mt = unpack_bits(bits_t, nb)
    assert np.array_equal(mt, np.swapaxes(bits, -1, -2)), "transposed mask differs"
    assert np.array_equal(cnt_t.cpu().numpy(), bits.sum(-2)), "transposed counts differ"
    cp, ri = bw.col_ptr.cpu().numpy(), bw.row_idx.cpu().numpy()
    qb, kb, vb, gb = (_blocked_np(cfg, layout, x, og) for x in (q, k, v, dout))
    dq, dk, dv = (_blocked_np(cfg, layout, x, og) for x in (bw.dq, bw.dk, bw.dv))
    lse_g, delta_g = lse.cpu().numpy().astype(np.float64), bw.delta.cpu().numpy()
    o_b = _blocked_np(cfg, layout, o, og)
    stats = []
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            bh = b * cfg.heads + h
            ref_m = oracle_mask(cfg, f64(q_thw[b, h]), f64(k_thw[b, h]))
            adapt = unpack_bits(res["abits"][b, h], nb)
            check_mask_rows(bits[b, h], adapt, ref_m, cfg.thr, f"{name} h{bh}")
            m = ref_m["mask"].copy()
            band = (bits[b, h] != m).any(1)        # band rows only (checked above)
            m[band] = bits[b, h][band]
            rp_ref, ci_ref = O.to_csr(m.T)
            assert np.array_equal(cp[bh], rp_ref), "col_ptr differs"
            assert np.array_equal(ri[bh, :len(ci_ref)], ci_ref), "row_idx differs"
            rdq, rdk, rdv, rlse = O.block_sparse_attention_backward(
                qb[b, h], kb[b, h], vb[b, h], m, valid, gb[b, h])
            vq = valid
            # log-sum-exp at valid queries; -inf at pad slots
            assert np.all(np.isneginf(lse_g[b, h][~vq]))
            fin = np.isfinite(rlse)
            assert np.array_equal(np.isfinite(lse_g[b, h]), fin)
            lse_bar = 1e-2 if q.dtype == torch.bfloat16 else 1e-5
            assert np.abs(lse_g[b, h][fin] - rlse[fin]).max() < lse_bar
            # D = rowsum(dO * O) of the forward's (rounded) output
            d_ref = (gb[b, h] * o_b[b, h]).sum(-1) * vq
            assert np.abs(delta_g[b, h] - d_ref).max() <= 1e-3 * max(1.0, np.abs(d_ref).max())
            for got, ref, lab in ((dq, rdq, "dq"), (dk, rdk, "dk"), (dv, rdv, "dv")):
                g_h = got[b, h]
                if layout == nabla.LAYOUT_BLOCKED:
                    assert np.all(g_h[~vq] == 0), f"{lab}: pad slots not zero"
                stats.append((lab,) + _rel_check(g_h[vq], ref[vq], q.dtype,
                                                 f"{name} {lab} h{bh}"))
    worst = {lab: max(s[1] for s in stats if s[0] == lab) for lab in ("dq", "dk", "dv")}
    log(f"{name}: worst relative max error {worst}")


def test_backward_rejects_mixed_dtypes():
    cfg = synth.config("small", heads=1, T=1, H=8, W=8)
    g = geom_of(cfg, nabla.LAYOUT_THW, torch.float32)    # bf16 inputs, float32 output
    x = torch.zeros(g.tensor_shape(), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros(nabla.lse_shape(g), dtype=torch.float32, device="cuda")
    rp = torch.zeros((1, g.nb + 1), dtype=torch.int32, device="cuda")
    ci = torch.zeros((1, g.nb * g.nb), dtype=torch.int32, device="cuda")
    with pytest.raises(nabla.NablaError) as e:   # the C ABI's dtype check, before any launch
        nabla.nabla_attn_bwd_dq(g, x, x, x, x, x, lse, rp, ci, 0.125, x, lse)
    assert e.value.status == -3


@pytest.mark.parametrize("name", ["ragged_bf16", "ragged_f32"])
def test_autograd_function_matches_explicit_calls(name):
    """nabla_attention as a torch autograd op: its output and the gradients
    autograd returns equal, bit for bit, the explicit forward-with-lse and
    backward calls on the same inputs."""
    base, kw = CASES[name]
    cfg = synth.config(base, **kw)
    q0, k0, v0 = synth.make_qkv(cfg, device="cuda")
    dout = synth.make_tensor(cfg, 3, device="cuda")
    q, k, v = (x.clone().requires_grad_(True) for x in (q0, k0, v0))
    o = nabla.nabla_attention(q, k, v, cfg.thr, cfg.sta)
    (o.float() * dout.float()).sum().backward()
    torch.cuda.synchronize()
    g, _, _, _, _, o_ref, _, _, bw, _, _ = _run(cfg, nabla.LAYOUT_THW)
    iv = torch.int16 if q0.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(o.detach().view(iv), o_ref.view(iv))
    for got, ref, lab in ((q.grad, bw.dq, "dq"), (k.grad, bw.dk, "dk"), (v.grad, bw.dv, "dv")):
        assert torch.equal(got.view(iv), ref.view(iv)), f"{name}: autograd {lab} differs"

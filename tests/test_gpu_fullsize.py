"""GPU parity at the full Wan-2.1-shaped sizes (480p, 720p, Long sweep), in the
launch configuration the bench times: all 40 heads run on the GPU; the oracle
checks the masks of sampled heads in full and the outputs of sampled query
blocks of those heads."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpu_helpers import (check_bf16_rounding, check_mask_rows, check_output, f64,
                         gpu_mask_for_oracle, log, ogeom, oracle_mask, run_pipeline, unpack_bits)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

ROWS_PER_HEAD = 24


def _sample_rows(cfg, nb):
    rng = np.random.default_rng([cfg.seed, 7])
    gt, gh, gw = cfg.T, -(-cfg.H // 8), -(-cfg.W // 8)
    must = {0, nb - 1, gh * gw - 1, (gh - 1) * gw}          # corners incl. padded edge blocks
    extra = rng.choice(nb, size=ROWS_PER_HEAD - len(must), replace=False).tolist()
    return sorted(must | set(int(x) for x in extra))


def _run(cfg, q, k, v, thr=None, sta=None, label=""):
    thr = cfg.thr if thr is None else thr
    sta = cfg.sta if sta is None else sta
    res = run_pipeline(cfg, q, k, v, thr=thr, sta=sta, also_bf16=True)
    check_bf16_rounding(res)
    nb = res["g"].nb
    og = ogeom(cfg)
    heads = synth.sampled_heads(cfg)
    stats = []
    for h in heads:
        qh, kh, vh = f64(q[0, h]), f64(k[0, h]), f64(v[0, h])
        ref = oracle_mask(cfg, qh, kh, thr, sta)
        union = unpack_bits(res["bits"][0, h], nb)
        adapt = unpack_bits(res["abits"][0, h], nb)
        nbnd, ndf = check_mask_rows(union, adapt, ref, thr, f"{label} h{h}")
        # sampled rows plus every band row where the GPU cut differently, those
        # compared under the GPU's row
        m = gpu_mask_for_oracle(ref, union)
        rows = sorted(set(_sample_rows(cfg, nb)) | set(np.flatnonzero((m != ref["mask"]).any(1))
                                                       .tolist()))
        ob = O.block_sparse_attention(O.flatten(qh, og), O.flatten(kh, og), O.flatten(vh, og),
                                      m, ref["valid"], rows=rows)
        got = O.flatten(f64(res["o"][0, h]), og)
        sel = np.zeros_like(ref["valid"])
        sel[rows] = ref["valid"][rows]
        e = check_output(got[sel], ob[sel], cfg.torch_dtype, f"{label} h{h}")
        stats.append((h, 1 - union.mean(), nbnd, ndf, e[0], e[1]))
        log(f"{label} h{h}: sparsity {1 - union.mean():.3f} band {nbnd} diff {ndf} "
            f"rows {len(rows)} max|err| {e[0]:.2e} mean|err| {e[1]:.2e}")
    return stats


@pytest.mark.parametrize("name", ["480p", "720p"])
def test_fullsize(name):
    cfg = synth.config(name)
    log(f"{name}: generating inputs {cfg}")
    q, k, v = synth.make_qkv(cfg, device="cuda")
    _run(cfg, q, k, v, label=name)


@pytest.fixture(scope="module")
def long_inputs():
    cfg = synth.config("long")
    log(f"long: generating inputs {cfg}")
    return cfg, synth.make_qkv(cfg, device="cuda")


@pytest.mark.parametrize("thr", [0.5, 0.7, 0.9])
@pytest.mark.parametrize("sta", [(3, 3, 3), (0, 0, 0)], ids=["sta", "nosta"])
def test_long_sweep(long_inputs, thr, sta):
    cfg, (q, k, v) = long_inputs
    _run(cfg, q, k, v, thr=thr, sta=sta, label=f"long thr={thr} sta={sta}")


def test_max_blocks():
    """3840 blocks per head (64 frames at 720p), close to the library's 4096:
    the longest kept lists and union schedules, and the widest mask row."""
    cfg = synth.config("long", T=64, heads=2, thr=0.9)
    log(f"max_blocks: generating inputs {cfg}")
    q, k, v = synth.make_qkv(cfg, device="cuda")
    _run(cfg, q, k, v, label="max_blocks")


def _backward_sampled(cfg, n_rows, n_cols, label):
    """Gradients in the bench's launch configuration (every head on the GPU,
    the forward through nabla_attn_fwd_vt_lse): one sampled head's mask checked
    in full, dq and lse of sampled query blocks, dk and dv of sampled key
    blocks (the oracle over every query block that keeps them)."""
    import math
    import block_sparse_attention_flatten_amd as nabla
    from gpu_helpers import geom_of
    log(f"{label}: generating inputs {cfg}")
    q, k, v = synth.make_qkv(cfg, device="cuda")
    dout = synth.make_tensor(cfg, 3, device="cuda")
    res = run_pipeline(cfg, q, k, v, out_dtype=torch.bfloat16)
    g = geom_of(cfg, out_dtype=torch.bfloat16)
    scale = 1.0 / math.sqrt(cfg.head_dim)
    vt = torch.empty(nabla.vt_shape(g), dtype=q.dtype, device="cuda")
    nabla.nabla_transpose_v(g, v, vt)
    o = torch.empty_like(q)
    lse = torch.empty(nabla.lse_shape(g), dtype=torch.float32, device="cuda")
    nabla.nabla_attn_fwd_vt_lse(g, q, k, vt, res["rp"], res["ci"], scale, o, lse)
    bw = nabla.backward(g, q, k, v, o, lse, dout, res["bits"], res["rp"], res["ci"], scale)
    torch.cuda.synchronize()
    log(f"{label}: GPU done")
    og = ogeom(cfg)
    nb = g.nb
    h = synth.sampled_heads(cfg)[0]
    qh, kh, vh, gh = f64(q[0, h]), f64(k[0, h]), f64(v[0, h]), f64(dout[0, h])
    ref = oracle_mask(cfg, qh, kh)
    union = unpack_bits(res["bits"][0, h], nb)
    adapt = unpack_bits(res["abits"][0, h], nb)
    check_mask_rows(union, adapt, ref, cfg.thr, f"{label} h{h}")
    m = gpu_mask_for_oracle(ref, union)
    valid = ref["valid"]
    qb, kb, vb, gb = (O.flatten(x, og) for x in (qh, kh, vh, gh))
    rng = np.random.default_rng([cfg.seed, 11])
    qrows = sorted(set([0, nb - 1] + rng.choice(nb, n_rows, replace=False).tolist()))
    kcols = sorted(set([nb - 1] + rng.choice(nb, n_cols, replace=False).tolist()))
    rows = sorted(set(qrows) | set(np.flatnonzero(m[:, kcols].any(1)).tolist()))
    log(f"{label}: oracle over {len(rows)} query blocks")
    rdq, rdk, rdv, rlse = O.block_sparse_attention_backward(qb, kb, vb, m, valid, gb, rows=rows)
    dq, dk, dv = (O.flatten(f64(x[0, h]), og) for x in (bw.dq, bw.dk, bw.dv))
    lse_h = lse[0, h].cpu().numpy().astype(np.float64)
    for r in qrows:
        vr = valid[r]
        assert np.abs(lse_h[r][vr] - rlse[r][vr]).max() < 1e-2
    sel_q = np.zeros_like(valid)
    sel_q[qrows] = valid[qrows]
    sel_k = np.zeros_like(valid)
    sel_k[kcols] = valid[kcols]
    for got, want, sel, lab in ((dq, rdq, sel_q, "dq"), (dk, rdk, sel_k, "dk"),
                                (dv, rdv, sel_k, "dv")):
        sc = np.abs(want[sel]).max()
        err = np.abs(got[sel] - want[sel])
        log(f"{label} {lab}: max|err| {err.max() / sc:.2e} mean {err.mean() / sc:.2e} "
            f"(relative to {sc:.3e})")
        assert np.isfinite(got[sel]).all()
        assert err.max() <= 2e-2 * sc and err.mean() <= 2e-3 * sc, lab


def test_backward_720p_sampled():
    """Gradients at the 720p bench shape, all 40 heads."""
    _backward_sampled(synth.config("720p"), 4, 1, "720p backward")


def test_backward_max_blocks_sampled():
    """Gradients at 3840 blocks per head (64 frames at 720p): the longest
    transposed mask rows and key-major lists."""
    _backward_sampled(synth.config("long", T=64, heads=2, thr=0.5), 2, 1, "max_blocks backward")


@pytest.mark.parametrize("shape", ["720p", "max_blocks"])
def test_dense_sampled(shape):
    """nabla_dense_attn_fwd at the 720p bench shape (all 40 heads) and at 3840
    blocks per head (64 frames at 720p, close to the 4096-block limit):
    sampled query blocks of sampled heads against the oracle's attention over
    every valid key (the all-kept mask), lse included."""
    import math
    import block_sparse_attention_flatten_amd as nabla
    from gpu_helpers import geom_of
    cfg = synth.config("720p") if shape == "720p" else synth.config("long", T=64, heads=2)
    log(f"dense {shape}: generating inputs {cfg}")
    q, k, v = synth.make_qkv(cfg, device="cuda")
    g = geom_of(cfg, out_dtype=torch.float32)
    nb = g.nb
    scale = 1.0 / math.sqrt(cfg.head_dim)
    vt = torch.empty(nabla.vt_shape(g), dtype=q.dtype, device="cuda")
    nabla.nabla_transpose_v(g, v, vt)
    o = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    lse = torch.empty(nabla.lse_shape(g), dtype=torch.float32, device="cuda")
    nabla.nabla_dense_attn_fwd(g, q, k, vt, scale, o, lse)
    torch.cuda.synchronize()
    log(f"dense {shape}: GPU done")
    og = ogeom(cfg)
    valid = O.valid_tokens(og)
    full = np.ones((nb, nb), dtype=bool)
    for h in synth.sampled_heads(cfg):
        qb, kb, vb = (O.flatten(f64(x[0, h]), og) for x in (q, k, v))
        rows = _sample_rows(cfg, nb) if shape == "720p" else [0, 1234, nb - 1]
        ref = O.block_sparse_attention(qb, kb, vb, full, valid, rows=rows)
        got = O.flatten(f64(o[0, h]), og)
        sel = np.zeros_like(valid)
        sel[rows] = valid[rows]
        e = check_output(got[sel], ref[sel], cfg.torch_dtype, f"dense {shape} h{h}")
        kv = kb[valid]
        lse_h = lse[0, h].cpu().numpy().astype(np.float64)
        for r in rows[:6]:
            s = qb[r][valid[r]] @ kv.T * scale
            m = s.max(1)
            want = m + np.log(np.exp(s - m[:, None]).sum(1))
            assert np.abs(lse_h[r][valid[r]] - want).max() < 1e-2
        log(f"dense {shape} h{h}: rows {len(rows)} max|err| {e[0]:.2e} mean|err| {e[1]:.2e}")


def test_layer_720p_sampled():
    """The DiT-layer path at the 720p shape, as bench.py's layer leg runs it:
    QKV = X W_qkv (library GEMM, 80640 x 5120 x 15360), nabla_qkv_split, mask,
    lists and attention on all 40 heads; for sampled heads the pooled means,
    the mask (bit-exact outside band rows) and sampled query blocks of the
    output against the oracle on the projected q, k, v."""
    import math
    import block_sparse_attention_flatten_amd as nabla
    cfg = synth.config("720p")
    B, h, d = cfg.batch, cfg.heads, cfg.head_dim
    g = nabla.Geometry(B, h, cfg.T, cfg.H, cfg.W, d, torch.bfloat16, nabla.LAYOUT_BLOCKED,
                       out_dtype=torch.float32)
    nb, S, Dm = g.nb, g.nb * 64, h * d
    dev = "cuda"
    log("layer 720p: generating inputs")
    field = synth.make_tensor(cfg, 0, device=dev)
    xb = torch.zeros(g.tensor_shape(), dtype=torch.bfloat16, device=dev)
    nabla.nabla_flatten(g.with_layout(nabla.LAYOUT_THW), field, xb)
    X = xb.permute(0, 2, 3, 1, 4).reshape(B, S, Dm).contiguous()
    del field, xb
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    Wqkv = (torch.randn(Dm, 3 * Dm, generator=gen, device=dev) / math.sqrt(Dm)).to(torch.bfloat16)
    qkv = torch.matmul(X, Wqkv).view(nabla.qkv_shape(g))
    del X
    q = torch.empty(g.tensor_shape(), dtype=torch.bfloat16, device=dev)
    k = torch.empty_like(q)
    vt = torch.empty(nabla.vt_shape(g), dtype=torch.bfloat16, device=dev)
    qbar = torch.empty(nabla.qbar_shape(g), dtype=torch.float32, device=dev)
    kbar = torch.empty(nabla.kbar_shape(g), dtype=nabla.KBAR_DTYPE, device=dev)
    bits = torch.empty((B, h, nb, g.nw), dtype=torch.int32, device=dev)
    abits = torch.empty_like(bits)
    cnt = torch.empty((B, h, nb), dtype=torch.int32, device=dev)
    rp = torch.empty((B * h, nb + 1), dtype=torch.int32, device=dev)
    ci = torch.empty((B * h, nb * nb), dtype=torch.int32, device=dev)
    o = torch.empty(g.tensor_shape(), dtype=torch.float32, device=dev)
    nabla.nabla_qkv_split(g, qkv, q, k, vt, qbar, kbar)
    nabla.nabla_mask(g, qbar, kbar, cfg.thr, cfg.sta, bits, cnt, abits)
    nabla.nabla_compact(g, bits, cnt, rp, ci)
    nabla.nabla_attn_fwd_vt(g, q, k, vt, rp, ci, 1.0 / math.sqrt(d), o)
    torch.cuda.synchronize()
    log("layer 720p: GPU done")
    og = ogeom(cfg)
    valid = O.valid_tokens(og)
    kb_rows = nabla.kbar_untile(kbar, nb)
    v = qkv[0, :, 2]                                          # [S, h, d], token-major
    for hh in synth.sampled_heads(cfg)[:2]:
        qh = f64(q[0, hh]).reshape(nb, 64, d)
        kh = f64(k[0, hh]).reshape(nb, 64, d)
        vh = f64(v[:, hh]).reshape(nb, 64, d)
        qb_, kb_ = O.pool(qh, valid), O.pool(kh, valid)
        for got, want, x in ((f64(qbar[0, hh]), qb_, qh), (f64(kb_rows[0, hh]), kb_, kh)):
            assert np.abs(got - want).max() <= 64 * 2.0 ** -24 * np.abs(x).max()
        m, m_ad, p = O.nabla_mask(qb_, kb_, cfg.thr, og, cfg.sta)
        band_a, band_b = O.band_rows(p, m_ad, cfg.thr, 1e-5)
        ref = dict(mask=m, mask_adaptive=m_ad, p=p, band=band_a | band_b, valid=valid)
        union = unpack_bits(bits[0, hh], nb)
        adapt = unpack_bits(abits[0, hh], nb)
        nbnd, ndf = check_mask_rows(union, adapt, ref, cfg.thr, f"layer 720p h{hh}")
        mm = gpu_mask_for_oracle(ref, union)
        rows = sorted(set(_sample_rows(cfg, nb)) | set(np.flatnonzero((mm != m).any(1)).tolist()))
        ob = O.block_sparse_attention(qh, kh, vh, mm, valid, rows=rows)
        got = f64(o[0, hh]).reshape(nb, 64, d)
        sel = np.zeros_like(valid)
        sel[rows] = valid[rows]
        e = check_output(got[sel], ob[sel], torch.bfloat16, f"layer 720p h{hh}")
        log(f"layer 720p h{hh}: sparsity {1 - union.mean():.3f} band {nbnd} diff {ndf} "
            f"rows {len(rows)} max|err| {e[0]:.2e} mean|err| {e[1]:.2e}")

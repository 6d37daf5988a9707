"""GPU parity, small and ragged workloads: every kernel of the HIP path
against the float64 oracle on the same seeded inputs, element by element."""
import math

import numpy as np
import pytest
import torch

import block_sparse_attention_flatten_amd as nabla
import oracle as O
import synth
from gpu_helpers import (check_bf16_rounding, check_mask_rows, check_output, f64, geom_of,
                         gpu_mask_for_oracle, log, ogeom, oracle_mask, run_pipeline, unpack_bits)

pytestmark = pytest.mark.gpu

# (name, config overrides): full Tiny and Small configs, plus ragged latents
# (H, W not multiples of 8, W < 8), batch > 1, d = 64 in bf16, a one-block latent
CASES = {
    "tiny": ("tiny", {}),
    "small": ("small", {}),
    "ragged_bf16": ("small", dict(batch=2, heads=3, T=3, H=13, W=21, thr=0.6, sta=(1, 3, 3))),
    "ragged_f32": ("tiny", dict(batch=2, heads=2, T=2, H=11, W=17, head_dim=128, thr=0.7,
                                sta=(3, 3, 3))),
    "narrow": ("small", dict(heads=2, T=4, H=5, W=3, thr=0.5)),
    "one_block": ("small", dict(heads=2, T=1, H=8, W=8, thr=0.5)),
    "d64_bf16": ("small", dict(heads=2, T=4, H=24, W=40, head_dim=64, thr=0.8, sta=(3, 3, 3))),
    "thr_one": ("small", dict(heads=2, T=2, H=16, W=24, thr=1.0)),
    "thr_low": ("small", dict(heads=2, T=3, H=24, W=24, thr=0.05)),
    "pure_sta": ("small", dict(heads=2, T=3, H=21, W=24, thr=0.0, sta=(3, 3, 3))),
    # large-magnitude scores (gain 8 on the Q and K fields): deep online-softmax
    # rescaling, weights spanning many orders of magnitude
    "hot": ("small", dict(heads=2, T=3, H=16, W=24, thr=0.7, sta=(3, 3, 3), gain_qk=8.0)),
    # nearly flat scores (gain 0.02 on the Q and K fields, no noise): the cut
    # falls among near-ties, most rows keep about thr * nb blocks
    "cold": ("small", dict(heads=2, T=3, H=16, W=24, thr=0.6, gain_qk=0.02, noise=0.0)),
    # asymmetric STA window wider than the grid in some directions
    "wide_sta": ("small", dict(heads=2, T=5, H=24, W=40, thr=0.3, sta=(5, 1, 7))),
    # Q = K = 0: every score is exactly 0, so every row is a tie of nb blocks
    # broken by block index, and O is the mean of V over the kept keys
    "flat": ("small", dict(heads=2, T=2, H=16, W=24, thr=0.5, gain_qk=0.0, noise=0.0)),
}


def _cfg(name):
    base, kw = CASES[name]
    return synth.config(base, **kw)


@pytest.fixture(scope="module", params=sorted(CASES))
def case(request):
    name = request.param
    cfg = _cfg(name)
    log(f"case {name}: {cfg}")
    q, k, v = synth.make_qkv(cfg, device="cuda")
    return name, cfg, q, k, v


def test_flatten_bit_exact(case):
    name, cfg, q, _, _ = case
    g = geom_of(cfg)
    xb = torch.full(g.tensor_shape(nabla.LAYOUT_BLOCKED), 7.0, dtype=q.dtype, device="cuda")
    nabla.nabla_flatten(g, q, xb)
    back = torch.full_like(q, 3.0)
    nabla.nabla_unflatten(g, xb, back)
    torch.cuda.synchronize()
    og = ogeom(cfg)
    ref = O.flatten(q.cpu().view(torch.int16 if q.dtype == torch.bfloat16 else torch.int32)
                    .numpy(), og)
    got = xb.cpu().view(torch.int16 if q.dtype == torch.bfloat16 else torch.int32).numpy()
    assert np.array_equal(got, ref), f"{name}: flatten differs"
    assert torch.equal(back.view(torch.int16 if q.dtype == torch.bfloat16 else torch.int32),
                       q.view(torch.int16 if q.dtype == torch.bfloat16 else torch.int32))


@pytest.mark.parametrize("layout", [nabla.LAYOUT_THW, nabla.LAYOUT_BLOCKED])
def test_pool(case, layout):
    name, cfg, q, k, _ = case
    g = geom_of(cfg, layout)
    if layout == nabla.LAYOUT_BLOCKED:
        qi = torch.empty(g.tensor_shape(), dtype=q.dtype, device="cuda")
        ki = torch.empty_like(qi)
        nabla.nabla_flatten(g, q, qi)
        nabla.nabla_flatten(g, k, ki)
    else:
        qi, ki = q, k
    qbar = torch.empty(nabla.qbar_shape(g), device="cuda")
    kbar = torch.full(nabla.kbar_shape(g), float("nan"), dtype=nabla.KBAR_DTYPE, device="cuda")
    nabla.nabla_pool(g, qi, ki, qbar, kbar)
    torch.cuda.synchronize()
    og = ogeom(cfg)
    valid = O.valid_tokens(og)
    # pooled keys come split and tiled for the mask kernel (every row written)
    for x, xbar in ((q, qbar), (k, nabla.kbar_untile(kbar, g.nb))):
        ref = O.pool(O.flatten(f64(x), og), valid)
        got = f64(xbar)
        bound = 64 * 2.0 ** -24 * np.abs(f64(x)).max() + 1e-30
        assert np.abs(got - ref).max() <= bound, (name, np.abs(got - ref).max(), bound)


# One call per row-group shape of the mask kernel that the cases above do
# not reach: blocks per head in (256, 512], (1280, 1536], (1536, 2048] and
# (2496, 3072] (the 480p, 720p, Long and 3840-block shapes are covered by
# test_gpu_fullsize.py).  One head, masks and lists only.
MASK_SHAPES = {
    "nb320_d64": dict(heads=1, T=4, H=64, W=80, head_dim=64, thr=0.7, sta=(3, 3, 3)),
    "nb1440": dict(heads=1, T=6, H=96, W=160, thr=0.7, sta=(3, 3, 3)),
    "nb1920": dict(heads=1, T=8, H=90, W=160, thr=0.8, sta=(1, 3, 3)),
    "nb2880": dict(heads=1, T=12, H=96, W=153, thr=0.6, sta=(3, 3, 3)),
}


@pytest.mark.parametrize("name", sorted(MASK_SHAPES))
def test_mask_shapes(name):
    cfg = synth.config("small", **MASK_SHAPES[name])
    log(f"mask shape {name}: {cfg}")
    q, k, v = synth.make_qkv(cfg, device="cuda")
    res = run_pipeline(cfg, q, k, v)
    nb = res["g"].nb
    union = unpack_bits(res["bits"], nb)[0, 0]
    adapt = unpack_bits(res["abits"], nb)[0, 0]
    cnt = res["cnt"].cpu().numpy()[0, 0]
    rp = res["rp"].cpu().numpy()[0]
    ci = res["ci"].cpu().numpy()[0]
    ref = oracle_mask(cfg, f64(q[0, 0]), f64(k[0, 0]))
    nbnd, ndf = check_mask_rows(union, adapt, ref, cfg.thr, name)
    assert np.array_equal(cnt, union.sum(1))
    assert rp[0] == 0 and np.array_equal(np.diff(rp), cnt)
    for r in range(nb):
        assert np.array_equal(ci[rp[r]:rp[r + 1]], np.flatnonzero(union[r])), (name, r)
    log(f"mask shape {name}: nb {nb}, kept {union.mean():.3f}, band {nbnd}, differing {ndf}")


def test_mask_and_forward(case):
    """pool -> mask -> compact -> attention through the C ABI vs the oracle."""
    name, cfg, q, k, v = case
    res = run_pipeline(cfg, q, k, v, also_bf16=True)
    check_bf16_rounding(res)
    g = res["g"]
    nb = g.nb
    union = unpack_bits(res["bits"], nb)
    adapt = unpack_bits(res["abits"], nb)
    rp = res["rp"].cpu().numpy()
    ci = res["ci"].cpu().numpy()
    cnt = res["cnt"].cpu().numpy()
    og = ogeom(cfg)
    n_band = n_diff = 0
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            qh, kh, vh = f64(q[b, h]), f64(k[b, h]), f64(v[b, h])
            ref = oracle_mask(cfg, qh, kh)
            nbnd, ndf = check_mask_rows(union[b, h], adapt[b, h], ref, cfg.thr, f"{name} b{b} h{h}")
            n_band += nbnd
            n_diff += ndf
            # row counts and CSR describe the GPU's own mask exactly
            bh = b * cfg.heads + h
            assert np.array_equal(cnt[b, h], union[b, h].sum(1))
            assert rp[bh, 0] == 0 and np.array_equal(np.diff(rp[bh]), cnt[b, h])
            for r in range(nb):
                cols = ci[bh, rp[bh, r]:rp[bh, r + 1]]
                assert np.array_equal(cols, np.flatnonzero(union[b, h, r])), (name, b, h, r)
            # output of every row vs the oracle's attention (band rows where the
            # GPU cut differently: under the GPU's row)
            m = gpu_mask_for_oracle(ref, union[b, h])
            ob = O.block_sparse_attention(O.flatten(qh, og), O.flatten(kh, og), O.flatten(vh, og),
                                          m, ref["valid"])
            got = O.flatten(f64(res["o"][b, h]), og)
            sel = ref["valid"]
            e = check_output(got[sel], ob[sel], cfg.torch_dtype, f"{name} b{b} h{h}")
            log(f"{name} b{b} h{h}: kept {union[b, h].mean():.3f} band {nbnd} "
                f"diff {ndf} max|err| {e[0]:.2e} mean|err| {e[1]:.2e}")
    log(f"{name}: band rows {n_band}, differing rows {n_diff}")


@pytest.mark.parametrize("layout", [nabla.LAYOUT_THW, nabla.LAYOUT_BLOCKED])
def test_mask_build_equals_separate_calls(case, layout):
    """nabla_mask_build (pooling, mask and lists in one call) writes exactly
    what nabla_pool, nabla_mask and nabla_compact write one by one."""
    name, cfg, q, k, v = case
    if layout == nabla.LAYOUT_BLOCKED:
        g = geom_of(cfg)
        blk = [torch.empty(g.tensor_shape(nabla.LAYOUT_BLOCKED), dtype=q.dtype, device="cuda")
               for _ in range(3)]
        for x, xb in zip((q, k, v), blk):
            nabla.nabla_flatten(g, x, xb)
        q, k, v = blk
    a = run_pipeline(cfg, q, k, v, layout=layout, fused=True)
    b = run_pipeline(cfg, q, k, v, layout=layout, fused=False)
    nb = a["g"].nb
    for key in ("qbar", "kbar", "bits", "abits", "cnt", "rp"):
        x, y = a[key], b[key]
        if key == "kbar":            # rows past nb in the last tile are unwritten
            x, y = nabla.kbar_untile(x, nb).contiguous(), nabla.kbar_untile(y, nb).contiguous()
        assert torch.equal(x.view(torch.int32), y.view(torch.int32)), (name, key)
    nnz = a["cnt"].to(torch.int64).sum(-1).flatten()
    for i in range(nnz.numel()):
        n = int(nnz[i])
        assert torch.equal(a["ci"][i, :n], b["ci"][i, :n]), (name, "ci", i)
    assert torch.equal(a["o"].view(torch.int32), b["o"].view(torch.int32)), (name, "o")


def test_attention_with_oracle_masks(case):
    """Attention kernel alone, fed the oracle's mask (and random masks with
    one-block, empty-ish and full rows) as CSR."""
    name, cfg, q, k, v = case
    g = geom_of(cfg, out_dtype=torch.float32)
    og = ogeom(cfg)
    nb = g.nb
    rng = np.random.default_rng(11)
    masks = []
    for b in range(cfg.batch):
        row = []
        for h in range(cfg.heads):
            m = rng.random((nb, nb)) < 0.3
            m[np.arange(nb), rng.integers(0, nb, nb)] = True   # >= 1 per row
            if nb > 2:
                m[0] = True                                     # a full row
                m[1] = False
                m[1, nb - 1] = True                             # a one-block row
            row.append(m)
        masks.append(row)
    rp = np.zeros((cfg.batch * cfg.heads, nb + 1), np.int32)
    ci = np.zeros((cfg.batch * cfg.heads, nb * nb), np.int32)
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            p_, c_ = O.to_csr(masks[b][h])
            rp[b * cfg.heads + h] = p_
            ci[b * cfg.heads + h, :len(c_)] = c_
    rp_d, ci_d = torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda()
    scale = 1.0 / math.sqrt(cfg.head_dim)
    outs = {"attn_fwd": torch.empty(q.shape, dtype=torch.float32, device="cuda")}
    nabla.nabla_attn_fwd(g, q, k, v, rp_d, ci_d, scale, outs["attn_fwd"])
    if q.dtype == torch.bfloat16:
        vt = torch.empty(nabla.vt_shape(g), dtype=q.dtype, device="cuda")
        nabla.nabla_transpose_v(g, v, vt)
        outs["attn_fwd_vt"] = torch.empty(q.shape, dtype=torch.float32, device="cuda")
        nabla.nabla_attn_fwd_vt(g, q, k, vt, rp_d, ci_d, scale, outs["attn_fwd_vt"])
    torch.cuda.synchronize()
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            ob = O.block_sparse_attention(O.flatten(f64(q[b, h]), og), O.flatten(f64(k[b, h]), og),
                                          O.flatten(f64(v[b, h]), og), masks[b][h],
                                          O.valid_tokens(og))
            got = O.unflatten(ob, og)
            for which, o in outs.items():
                check_output(f64(o[b, h]), got, cfg.torch_dtype,
                             f"{name} random-mask {which} b{b} h{h}")


def test_compact_against_oracle_csr():
    """Compaction alone: random masks (some empty and full rows) -> CSR, bit-exact."""
    cfg = synth.config("small", batch=2, heads=3, T=5, H=24, W=40)
    g = geom_of(cfg)
    nb = g.nb
    rng = np.random.default_rng(5)
    m = rng.random((cfg.batch, cfg.heads, nb, nb)) < rng.random((1, 1, nb, 1))
    m[0, 0, 3] = False
    m[0, 1, 4] = True
    words = np.packbits(np.pad(m, [(0, 0)] * 3 + [(0, g.nw * 32 - nb)]), axis=-1,
                        bitorder="little").view(np.uint32).view(np.int32)
    bits = torch.from_numpy(np.ascontiguousarray(words)).cuda()
    cnt = torch.from_numpy(m.sum(-1).astype(np.int32)).cuda()
    rp = torch.full((cfg.batch * cfg.heads, nb + 1), -1, dtype=torch.int32, device="cuda")
    ci = torch.full((cfg.batch * cfg.heads, nb * nb), -1, dtype=torch.int32, device="cuda")
    nabla.nabla_compact(g, bits, cnt, rp, ci)
    torch.cuda.synchronize()
    rp, ci = rp.cpu().numpy(), ci.cpu().numpy()
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            p_, c_ = O.to_csr(m[b, h])
            i = b * cfg.heads + h
            assert np.array_equal(rp[i], p_)
            assert np.array_equal(ci[i, :len(c_)], c_)
            assert np.all(ci[i, len(c_):] == -1)


def test_forward_entry_point_matches_stepwise():
    """nabla_forward (one call, V^T path for bf16) == the entry points called
    one by one (on-chip transposing attention), bit for bit."""
    cfg = synth.config("small", heads=3, T=3, H=21, W=30, thr=0.75, sta=(3, 3, 3))
    q, k, v = synth.make_qkv(cfg, device="cuda")
    step = run_pipeline(cfg, q, k, v, out_dtype=torch.bfloat16, attn="tr")
    res = nabla.forward(q, k, v, cfg.thr, cfg.sta)
    torch.cuda.synchronize()
    assert torch.equal(res.o.view(torch.int16), step["o"].view(torch.int16))
    res32 = nabla.forward(q, k, v, cfg.thr, cfg.sta, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(res32.o.to(torch.bfloat16).view(torch.int16), res.o.view(torch.int16))
    assert torch.equal(res.mask_bits, step["bits"])
    assert torch.equal(res.row_ptr, step["rp"])


def test_blocked_layout_forward_matches_thw():
    cfg = synth.config("small", heads=2, T=3, H=19, W=27, thr=0.7, sta=(3, 3, 3))
    q, k, v = synth.make_qkv(cfg, device="cuda")
    g = geom_of(cfg)
    blk = [torch.empty(g.tensor_shape(nabla.LAYOUT_BLOCKED), dtype=q.dtype, device="cuda")
           for _ in range(3)]
    for x, xb in zip((q, k, v), blk):
        nabla.nabla_flatten(g, x, xb)
    r_thw = nabla.forward(q, k, v, cfg.thr, cfg.sta)
    r_blk = nabla.forward(*blk, cfg.thr, cfg.sta, layout=nabla.LAYOUT_BLOCKED, T=cfg.T, H=cfg.H,
                          W=cfg.W)
    back = torch.empty_like(q)
    nabla.nabla_unflatten(g, r_blk.o, back)
    torch.cuda.synchronize()
    assert torch.equal(r_thw.mask_bits, r_blk.mask_bits)
    assert torch.equal(back.view(torch.int16), r_thw.o.view(torch.int16))
    # pad query slots of the blocked output are zero
    valid = torch.from_numpy(O.valid_tokens(ogeom(cfg))).cuda()
    assert (r_blk.o[:, :, ~valid] == 0).all()


def test_empty_batch_is_a_no_op():
    cfg = synth.config("small", batch=0, heads=4, T=2, H=16, W=16)
    g = geom_of(cfg)
    q = torch.empty(g.tensor_shape(), dtype=torch.bfloat16, device="cuda")
    res = nabla.forward(q, q, q, 0.5, (3, 3, 3))
    torch.cuda.synchronize()
    assert res.o.numel() == 0


def _vt_reference(v: torch.Tensor, cfg) -> np.ndarray:
    """V^T layout from its definition: block b, row c = channel c of the 64 key
    slots, slot order with bits 2 and 3 of the position swapped; pads zero."""
    og = ogeom(cfg)
    vb = O.flatten(v.cpu().view(torch.int16).numpy(), og)          # [B, h, nb, 64, d]
    pos = np.arange(64)
    key = (pos & ~12) | ((pos & 4) << 1) | ((pos & 8) >> 1)
    return np.ascontiguousarray(np.swapaxes(vb[..., key, :], -1, -2))   # [B, h, nb, d, 64]


def test_transpose_v_and_attn_fwd_vt(case):
    name, cfg, q, k, v = case
    if q.dtype != torch.bfloat16:
        pytest.skip("the V^T path is bf16-only")
    g = geom_of(cfg)
    vt = torch.full((cfg.batch, cfg.heads, g.nb, cfg.head_dim, 64), 5.0, dtype=v.dtype,
                    device="cuda")
    nabla.nabla_transpose_v(g, v, vt)
    torch.cuda.synchronize()
    assert np.array_equal(vt.cpu().view(torch.int16).numpy(), _vt_reference(v, cfg))
    # the attention reading V^T is bit-identical to the one transposing on chip
    res = run_pipeline(cfg, q, k, v, out_dtype=torch.float32)
    for odt in (torch.float32, torch.bfloat16):
        gg = geom_of(cfg, out_dtype=odt)
        o_vt = torch.empty(q.shape, dtype=odt, device="cuda")
        o_tr = torch.empty(q.shape, dtype=odt, device="cuda")
        nabla.nabla_attn_fwd_vt(gg, q, k, vt, res["rp"], res["ci"], 1.0 / math.sqrt(cfg.head_dim),
                                o_vt)
        nabla.nabla_attn_fwd(gg, q, k, v, res["rp"], res["ci"], 1.0 / math.sqrt(cfg.head_dim),
                             o_tr)
        torch.cuda.synchronize()
        iv = torch.int32 if odt == torch.float32 else torch.int16
        assert torch.equal(o_vt.view(iv), o_tr.view(iv)), f"{name}: V^T path differs ({odt})"


@pytest.mark.parametrize("path", ["vt", "tr", "f32"])
def test_out_of_range_list_entries_are_skipped(path):
    """The attention kernels skip list entries outside [0, nb) and treat a row
    whose end pointer lies past the list capacity as empty: corrupted lists
    give exactly the output of the same lists with those entries removed
    (and that row emptied)."""
    f32 = path == "f32"
    cfg = synth.config("tiny" if f32 else "small", heads=2, T=3, H=16, W=24, thr=0.6,
                       sta=(3, 3, 3), head_dim=64 if f32 else 128)
    q, k, v = synth.make_qkv(cfg, device="cuda")
    res = run_pipeline(cfg, q, k, v, out_dtype=q.dtype, attn="tr" if path == "tr" else "vt")
    g = res["g"]
    nb = g.nb
    rp, ci = res["rp"].cpu().numpy(), res["ci"].cpu().numpy()
    bad_rp, bad_ci = rp.copy(), ci.copy()
    clean_rp, clean_ci = np.zeros_like(rp), np.full_like(ci, -7)
    for i in range(rp.shape[0]):
        rows = []
        for r in range(nb):
            lst = ci[i, rp[i, r]:rp[i, r + 1]].tolist()
            keep = list(lst)
            if r in (1, 5, 7) and len(lst) >= 2:          # overwrite the second entry
                bad_ci[i, rp[i, r] + 1] = {1: -1, 5: nb, 7: 1 << 30}[r]
                keep = lst[:1] + lst[2:]
            if r == nb - 1:                                # end pointer past the capacity
                bad_rp[i, nb] = nb * nb + 5
                keep = []
            rows.append(keep)
        pos = 0
        for r, keep in enumerate(rows):
            clean_rp[i, r] = pos
            clean_ci[i, pos:pos + len(keep)] = keep
            pos += len(keep)
        clean_rp[i, nb] = pos
    d = cfg.head_dim
    scale = 1.0 / math.sqrt(d)
    outs = []
    for p_, c_ in ((bad_rp, bad_ci), (clean_rp, clean_ci)):
        rpt, cit = torch.from_numpy(p_).cuda(), torch.from_numpy(c_).cuda()
        o = torch.full_like(q, 3.0)
        if path == "vt":
            vt = torch.empty(nabla.vt_shape(g), dtype=q.dtype, device="cuda")
            nabla.nabla_transpose_v(g, v, vt)
            nabla.nabla_attn_fwd_vt(g, q, k, vt, rpt, cit, scale, o)
        else:
            nabla.nabla_attn_fwd(g, q, k, v, rpt, cit, scale, o)
        torch.cuda.synchronize()
        outs.append(o)
    iv = torch.int16 if q.dtype == torch.bfloat16 else torch.int32
    assert torch.equal(outs[0].view(iv), outs[1].view(iv)), f"{path}: corrupted lists differ"
    # the emptied last row gives zeros at its valid queries
    og = ogeom(cfg)
    last = O.flatten(f64(outs[1][0, 0]), og)[nb - 1][O.valid_tokens(og)[nb - 1]]
    assert np.all(last == 0)


@pytest.mark.parametrize("layout", [nabla.LAYOUT_THW, nabla.LAYOUT_BLOCKED])
def test_dense_attention(case, layout):
    """nabla_dense_attn_fwd (no mask, no lists) against the oracle's attention
    on the all-kept mask (pinned to textbook softmax attention), lse included;
    and bit-equal to the sparse kernel walking the all-kept lists."""
    name, cfg, q, k, v = case
    if cfg.torch_dtype != torch.bfloat16:
        pytest.skip("the dense kernel reads V^T (bf16 inputs only)")
    g = geom_of(cfg, layout, out_dtype=torch.float32)
    if layout == nabla.LAYOUT_BLOCKED:
        qb, kb, vb = (torch.empty(g.tensor_shape(layout), dtype=q.dtype, device="cuda")
                      for _ in range(3))
        for src, dst in ((q, qb), (k, kb), (v, vb)):
            nabla.nabla_flatten(geom_of(cfg), src, dst)
        q, k, v = qb, kb, vb
    nb = g.nb
    bh = cfg.batch * cfg.heads
    scale = 1.0 / math.sqrt(cfg.head_dim)
    vt = torch.empty(nabla.vt_shape(g), dtype=q.dtype, device="cuda")
    nabla.nabla_transpose_v(g, v, vt)
    o = torch.full(g.tensor_shape(layout), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.empty(nabla.lse_shape(g), dtype=torch.float32, device="cuda")
    nabla.nabla_dense_attn_fwd(g, q, k, vt, scale, o, lse)
    # the sparse kernel over every block
    rp = (torch.arange(nb + 1, dtype=torch.int32, device="cuda") * nb).repeat(bh, 1).contiguous()
    ci = torch.arange(nb, dtype=torch.int32, device="cuda").repeat(bh, nb).contiguous()
    o_sp = torch.empty_like(o)
    lse_sp = torch.empty_like(lse)
    nabla.nabla_attn_fwd_vt_lse(g, q, k, vt, rp, ci, scale, o_sp, lse_sp)
    ob = torch.empty(g.tensor_shape(layout), dtype=torch.bfloat16, device="cuda")
    gb = geom_of(cfg, layout, out_dtype=torch.bfloat16)
    nabla.nabla_dense_attn_fwd(gb, q, k, vt, scale, ob, None)
    torch.cuda.synchronize()
    og = ogeom(cfg)
    valid = O.valid_tokens(og)
    full = np.ones((nb, nb), dtype=bool)
    for b in range(cfg.batch):
        for h in range(cfg.heads):
            if layout == nabla.LAYOUT_THW:
                qh, kh, vh = (O.flatten(f64(x[b, h]), og) for x in (q, k, v))
                got = O.flatten(f64(o[b, h]), og)
            else:
                qh, kh, vh = (f64(x[b, h]).reshape(nb, 64, -1) for x in (q, k, v))
                got = f64(o[b, h]).reshape(nb, 64, -1)
            ref = O.block_sparse_attention(qh, kh, vh, full, valid)
            check_output(got[valid], ref[valid], cfg.torch_dtype, f"{name} dense b{b} h{h}")
            # lse against ln sum exp over every valid key
            s = np.einsum("qd,kd->qk", qh[valid], kh[valid]) * scale
            m = s.max(1, keepdims=True)
            want = (m[:, 0] + np.log(np.exp(s - m).sum(1)))
            assert np.abs(lse[b, h].cpu().numpy()[valid] - want).max() < 1e-2
    assert torch.equal(o.view(torch.int32), o_sp.view(torch.int32)), name
    assert torch.equal(lse.view(torch.int32), lse_sp.view(torch.int32)), name
    # the bf16 output is the float32 result rounded to nearest even
    assert torch.equal(ob.view(torch.int16), o.to(torch.bfloat16).view(torch.int16)), name

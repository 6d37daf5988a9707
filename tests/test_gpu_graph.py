"""The NABLA call inside a HIP graph.  The library's calls only launch
kernels on the given stream (no allocation, memset or synchronisation), so
nabla_forward can be captured once and replayed on new inputs; each replay
must give exactly the eager result for the same inputs (bit-exact output,
mask, counts and lists).  Eager calls and synchronisations run between the
replays."""
import math

import pytest
import torch

import block_sparse_attention_flatten_amd as nabla
import synth
from gpu_helpers import log

pytestmark = pytest.mark.gpu


def _views(g, ws, offs):
    bh = g.batch * g.heads
    def part(i, shape):
        n = math.prod(shape)
        return ws[offs[i]:offs[i] + 4 * n].view(torch.int32).view(shape)
    return (part(2, (bh, g.nb, g.nw)), part(3, (bh, g.nb)), part(4, (bh, g.nb + 1)),
            part(5, (bh, g.nb * g.nb)))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_forward_graph_replays_match_eager(dtype):
    base = "480p" if dtype == torch.bfloat16 else "tiny"
    cfg = synth.config(base, heads=2, T=3, dtype="bf16" if dtype == torch.bfloat16 else "fp32")
    log(f"graph test {cfg}")
    g = nabla.Geometry(cfg.batch, cfg.heads, cfg.T, cfg.H, cfg.W, cfg.head_dim, dtype)
    size, offs = nabla.nabla_forward_workspace_size(g)
    shp = g.tensor_shape()
    q, k, v = (torch.zeros(shp, dtype=dtype, device="cuda") for _ in range(3))
    o, o_e = torch.zeros_like(q), torch.zeros_like(q)
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    ws_e = torch.zeros_like(ws)
    scale = 1.0 / math.sqrt(cfg.head_dim)

    def fill(seed):
        qq, kk, vv = synth.make_qkv(cfg.with_(seed=seed), device="cuda")
        q.copy_(qq)
        k.copy_(kk)
        v.copy_(vv)

    def call(out, work, stream):
        nabla.nabla_forward(g, q, k, v, cfg.thr, cfg.sta, scale, out, work, stream)

    fill(cfg.seed)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):    # one eager call on a side stream before capture
        call(o, ws, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(o, ws, torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep, seed in enumerate([101, 102, 103]):
        fill(seed)
        call(o_e, ws_e, torch.cuda.current_stream())         # eager reference
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        if dtype == torch.bfloat16:
            assert torch.equal(o.view(torch.int16), o_e.view(torch.int16)), f"replay {rep}: o"
        else:
            assert torch.equal(o, o_e), f"replay {rep}: o"
        got, ref = _views(g, ws, offs), _views(g, ws_e, offs)
        for name, a, b in zip(("mask_bits", "row_count", "row_ptr"), got[:3], ref[:3]):
            assert torch.equal(a, b), f"replay {rep}: {name}"
        nnz = ref[2][:, -1].tolist()
        for hh, n in enumerate(nnz):
            assert torch.equal(got[3][hh, :n], ref[3][hh, :n]), f"replay {rep}: col_idx head {hh}"
        log(f"replay {rep} matches the eager call (nnz per head {nnz})")


def test_forward_and_backward_graph_replays_match_eager():
    """The whole training-side sequence (mask construction, the forward with
    its log-sum-exp, then dQ, dK, dV with the mask held fixed) in one graph;
    torch allocations inside the capture come from the graph's pool."""
    cfg = synth.config("480p", heads=2, T=3)
    log(f"graph test (forward + backward) {cfg}")
    g = nabla.Geometry(cfg.batch, cfg.heads, cfg.T, cfg.H, cfg.W, cfg.head_dim, torch.bfloat16)
    B, h, nb, d = cfg.batch, cfg.heads, g.nb, cfg.head_dim
    shp = g.tensor_shape()
    q, k, v, dout = (torch.zeros(shp, dtype=torch.bfloat16, device="cuda") for _ in range(4))
    scale = 1.0 / math.sqrt(d)

    def fill(seed):
        c = cfg.with_(seed=seed)
        qq, kk, vv = synth.make_qkv(c, device="cuda")
        q.copy_(qq)
        k.copy_(kk)
        v.copy_(vv)
        dout.copy_(synth.make_tensor(c, 3, device="cuda"))

    def step():
        dev = q.device
        qbar = torch.empty(nabla.qbar_shape(g), dtype=torch.float32, device=dev)
        kbar = torch.empty(nabla.kbar_shape(g), dtype=nabla.KBAR_DTYPE, device=dev)
        bits = torch.empty((B, h, nb, g.nw), dtype=torch.int32, device=dev)
        cnt = torch.empty((B, h, nb), dtype=torch.int32, device=dev)
        rp = torch.empty((B * h, nb + 1), dtype=torch.int32, device=dev)
        ci = torch.empty((B * h, nb * nb), dtype=torch.int32, device=dev)
        vt = torch.empty(nabla.vt_shape(g), dtype=torch.bfloat16, device=dev)
        o = torch.empty_like(q)
        lse = torch.empty(nabla.lse_shape(g), dtype=torch.float32, device=dev)
        nabla.nabla_pool(g, q, k, qbar, kbar)
        nabla.nabla_mask(g, qbar, kbar, cfg.thr, cfg.sta, bits, cnt, None)
        nabla.nabla_compact(g, bits, cnt, rp, ci)
        nabla.nabla_transpose_v(g, v, vt)
        nabla.nabla_attn_fwd_vt_lse(g, q, k, vt, rp, ci, scale, o, lse)
        bw = nabla.backward(g, q, k, v, o, lse, dout, bits, rp, ci, scale)
        return {"o": o, "lse": lse, "dq": bw.dq, "dk": bw.dk, "dv": bw.dv, "delta": bw.delta}

    fill(cfg.seed)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = step()
    torch.cuda.synchronize()
    for rep, seed in enumerate([201, 202, 203]):
        fill(seed)
        ref = step()                                           # eager reference
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a in out.items():
            b = ref[name]
            same = (torch.equal(a.view(torch.int16), b.view(torch.int16))
                    if a.dtype == torch.bfloat16 else torch.equal(a, b))
            assert same, f"replay {rep}: {name} differs from the eager call"
        log(f"replay {rep}: o, lse, dq, dk, dv, delta match the eager call")


def test_noalloc_and_layer_calls_graph_replays_match_eager():
    """nabla_forward_noalloc (library scratch array), and the layer path
    (nabla_qkv_split, mask, lists, attention) with the dense kernel, captured
    in one graph and replayed on new inputs: every replay equals the eager
    calls bit for bit."""
    cfg = synth.config("480p", heads=3, T=3)
    log(f"graph test (no-alloc + layer path) {cfg}")
    g = nabla.Geometry(cfg.batch, cfg.heads, cfg.T, cfg.H, cfg.W, cfg.head_dim, torch.bfloat16)
    gb = g.with_layout(nabla.LAYOUT_BLOCKED)
    B, h, nb, d = cfg.batch, cfg.heads, g.nb, cfg.head_dim
    scale = 1.0 / math.sqrt(d)
    q, k, v = (torch.zeros(g.tensor_shape(), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    qkv = torch.zeros(nabla.qkv_shape(gb), dtype=torch.bfloat16, device="cuda")

    def fill(seed):
        c = cfg.with_(seed=seed)
        qq, kk, vv = synth.make_qkv(c, device="cuda")
        q.copy_(qq)
        k.copy_(kk)
        v.copy_(vv)
        # the same fields as a token-major projection output in the blocked order
        for i, x in enumerate((qq, kk, vv)):
            xb = torch.empty(gb.tensor_shape(), dtype=torch.bfloat16, device="cuda")
            nabla.nabla_flatten(g, x, xb)
            qkv[:, :, i] = xb.permute(0, 2, 3, 1, 4).reshape(B, nb * 64, h, d)

    def step():
        dev = q.device
        o1 = torch.empty_like(q)
        nabla.nabla_forward_noalloc(g, q, k, v, cfg.thr, cfg.sta, scale, o1)
        qb = torch.empty(gb.tensor_shape(), dtype=torch.bfloat16, device=dev)
        kb = torch.empty_like(qb)
        vt = torch.empty(nabla.vt_shape(gb), dtype=torch.bfloat16, device=dev)
        qbar = torch.empty(nabla.qbar_shape(g), dtype=torch.float32, device=dev)
        kbar = torch.empty(nabla.kbar_shape(g), dtype=nabla.KBAR_DTYPE, device=dev)
        bits = torch.empty((B, h, nb, g.nw), dtype=torch.int32, device=dev)
        cnt = torch.empty((B, h, nb), dtype=torch.int32, device=dev)
        rp = torch.empty((B * h, nb + 1), dtype=torch.int32, device=dev)
        ci = torch.empty((B * h, nb * nb), dtype=torch.int32, device=dev)
        o2 = torch.empty_like(qb)
        o3 = torch.empty_like(qb)
        nabla.nabla_qkv_split(gb, qkv, qb, kb, vt, qbar, kbar)
        nabla.nabla_mask(gb, qbar, kbar, cfg.thr, cfg.sta, bits, cnt, None)
        nabla.nabla_compact(gb, bits, cnt, rp, ci)
        nabla.nabla_attn_fwd_vt(gb, qb, kb, vt, rp, ci, scale, o2)
        nabla.nabla_dense_attn_fwd(gb, qb, kb, vt, scale, o3, None)
        return {"noalloc": o1, "layer": o2, "dense": o3, "qbar": qbar, "bits": bits}

    fill(cfg.seed)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = step()
    torch.cuda.synchronize()
    for rep, seed in enumerate([301, 302, 303]):
        fill(seed)
        ref = step()                                           # eager reference
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a in out.items():
            b = ref[name]
            same = (torch.equal(a.view(torch.int16), b.view(torch.int16))
                    if a.dtype == torch.bfloat16 else torch.equal(a, b))
            assert same, f"replay {rep}: {name} differs from the eager call"
        log(f"replay {rep}: no-alloc, layer-path and dense outputs match the eager calls")

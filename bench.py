"""Benchmark of one NABLA attention call on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 720p]

A step is one pass of the whole hot path over one batch of synthetic input:
nabla_pool -> nabla_mask -> nabla_compact (the calls of nabla_mask_build),
with nabla_transpose_v on a second stream beside the mask and compaction ->
nabla_attn_fwd_vt (float32 inputs: nabla_attn_fwd),
called through the C ABI
on torch's current stream, with the fractal flatten applied inside the
pooling, transpose and attention loaders (inputs and output stay in the
natural [B, heads, T, H, W, d] layout).  Inputs are resident in HBM before
timing.
Prints ONE JSON line (plus progress on stderr).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NABLA attn ms/call + effective TFLOP/s (kept blocks) at 720p Wan-shape, 1 GPU"
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak

WORKLOAD_NAMES = {
    "tiny": "Tiny NABLA attention (1x2 heads, d=64, fp32, 4x16x16)",
    "small": "Small NABLA attention (1x8 heads, d=128, bf16, 8x32x32)",
    "480p": "Wan-2.1-14B-shaped 480p NABLA attention layer (40 heads, d=128, 21x30x52)",
    "720p": "Wan-2.1-14B-shaped 720p NABLA attention layer (40 heads, d=128, 21x45x80)",
    "long": "Long 720p NABLA attention layer (40 heads, d=128, 41x45x80)",
}


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="720p", choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--thr", type=float, default=None)
    ap.add_argument("--sta", type=str, default=None, help="e.g. 3,3,3 or 0,0,0")
    ap.add_argument("--heads", type=int, default=None, help="override the head count")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--thr-sweep", default="0,0.5,0.7,0.9",
                    help="thresholds for the sparsity/speed sweep (0 = pure STA); '' skips it")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the gradient calls (dq, dk, dv with the mask held fixed)")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the dense references (nabla_dense_attn_fwd, the sparse kernel "
                         "with every block kept, torch flash SDPA)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the 480p and Long summaries (720p runs only)")
    ap.add_argument("--no-layer", action="store_true",
                    help="skip the Wan-shaped attention layer (QKV and output projections on "
                         "hipBLASLt around the NABLA call, tokens in the blocked order)")
    ap.add_argument("--serial", action="store_true",
                    help="run every stage of the step on one stream (no V^T overlap)")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the achievable matrix-core / copy rate measurements")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 2 GiB device copy (reference for HBM counters)")
    return ap.parse_args()


def copy_calibration():
    """A plain device-to-device copy of known size: its FETCH_SIZE / WRITE_SIZE
    counter readings calibrate the counters of the NABLA kernels."""
    import torch
    n = 1 << 29                                   # 2 GiB of float32
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "launches": 3}))


PEAKS_SRC = os.path.join(ROOT, "bench_peaks.hip")
PEAKS_LIB = os.path.join(ROOT, "bench_peaks.so")


def build_peaks(verbose: bool = False) -> str:
    """Compile the benchmark's rate probe (bench_peaks.hip) into its own small
    library beside this file; the NABLA library does not contain it."""
    from block_sparse_attention_flatten_amd.build import HIP_FLAGS, _run, hipcc
    tmp = PEAKS_LIB + ".tmp"
    _run([hipcc(), *HIP_FLAGS, "-shared", "-o", tmp, PEAKS_SRC], verbose)
    os.replace(tmp, PEAKS_LIB)
    return PEAKS_LIB


def achievable_peaks(torch, stream, ev):
    """What this GPU sustains right now, for reading the roofline fractions:
    back-to-back bf16 matrix instructions on every CU (bench_peaks.hip, its own
    library) and a plain 2 GiB device copy.  None if the probe library is not
    built."""
    import ctypes
    path = PEAKS_LIB
    if not os.path.exists(path):
        log("achievable peaks skipped: bench_peaks.so not built")
        return None
    lib = ctypes.CDLL(path)
    lib.nabla_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                          ctypes.c_void_p]
    lib.nabla_probe_mfma_bf16.restype = ctypes.c_int
    lib.nabla_probe_mfma_bf16_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.nabla_probe_mfma_bf16_flops.restype = ctypes.c_double
    grid, iters = 256 * 3, 40000        # 3 workgroups per CU: all resident at once
    out = torch.empty(grid * 256, dtype=torch.float32, device="cuda")

    def probe():
        st = lib.nabla_probe_mfma_bf16(grid, iters, ctypes.c_void_p(out.data_ptr()),
                                       ctypes.c_void_p(stream.cuda_stream))
        if st != 0:
            raise RuntimeError(f"mfma probe launch failed ({st})")

    def timed(fn, reps):
        fn()
        a, b = ev(), ev()
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    mfma_ms = timed(probe, 3)
    lib.nabla_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                     ctypes.c_int, ctypes.c_void_p]
    lib.nabla_probe_copy.restype = ctypes.c_int
    n = 1 << 29                         # 2 GiB of float32 each way
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)

    def copy():
        st = lib.nabla_probe_copy(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(y.data_ptr()),
                                  4 * n, 256 * 32, ctypes.c_void_p(stream.cuda_stream))
        if st != 0:
            raise RuntimeError(f"copy probe launch failed ({st})")

    copy_ms = timed(copy, 3)
    torch_copy_ms = timed(lambda: y.copy_(x), 3)
    del x, y, out
    return {
        "mfma_bf16_tflops": round(lib.nabla_probe_mfma_bf16_flops(grid, iters)
                                  / (mfma_ms * 1e-3) / 1e12, 1),
        "hbm_copy_gbs": round(2 * 4 * n / (copy_ms * 1e-3) / 1e9, 1),
        "torch_copy_gbs": round(2 * 4 * n / (torch_copy_ms * 1e-3) / 1e9, 1),
        "how": "back-to-back v_mfma_f32_32x32x16_bf16 on all CUs; streaming 2 GiB device copy "
               "(bench_peaks.hip) and torch's copy_, read + write bytes",
    }


def torch_flash_reference(torch, cfg, q, k, v, time_call, attn_ms):
    """torch's flash-attention backend (no mask, all valid tokens) on the same
    Q, K, V as a tuned dense kernel of this box.  Only the flash backend is
    allowed: the math backend would materialise the S x S scores.  None when
    it is unavailable or the inputs are not bf16."""
    if cfg.torch_dtype != torch.bfloat16:
        return None
    from torch.nn.attention import SDPBackend, sdpa_kernel
    B, h, d = cfg.batch, cfg.heads, cfg.head_dim
    S = cfg.T * cfg.H * cfg.W                    # THW tensors hold valid tokens only
    qs, ks, vs = (x.reshape(B, h, S, d) for x in (q, k, v))
    try:
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            ms = time_call(lambda: torch.nn.functional.scaled_dot_product_attention(qs, ks, vs),
                           reps=3)
            # its backward on a synthetic dO (graph kept, gradients accumulate)
            qg, kg, vg = (x.detach().clone().requires_grad_(True) for x in (qs, ks, vs))
            og = torch.nn.functional.scaled_dot_product_attention(qg, kg, vg)
            dout = torch.ones_like(og)
            bwd_ms = time_call(lambda: og.backward(dout, retain_graph=True), reps=2)
            del qg, kg, vg, og, dout
    except RuntimeError as e:
        log(f"torch flash reference unavailable: {e}")
        return None
    flops = 4 * S * S * d * B * h
    out = {"what": "torch scaled_dot_product_attention, flash backend, full attention over "
                   "the valid tokens", "ms": round(ms, 3),
           "tflops_valid_tokens": round(flops / (ms * 1e-3) / 1e12, 1),
           "speedup_sparse_vs_torch_flash": round(ms / attn_ms, 3),
           "backward_ms": round(bwd_ms, 3),
           "backward_tflops_valid_tokens": round(2.5 * flops / (bwd_ms * 1e-3) / 1e12, 1)}
    log(f"torch flash reference: {out}")
    return out


def layer_leg(torch, nabla, cfg, g, x_field, thr, sta, scale, time_call, dev):
    """One self-attention layer of a Wan-shaped DiT around the NABLA call,
    with the token sequence kept in the blocked (fractal-flattened) order
    across the network, so no reorder runs per layer: X [S, h d] ->
    QKV = X W_qkv (one hipBLASLt GEMM through torch.matmul) ->
    nabla_qkv_split (head-major q, k, V^T and the block means in one pass) ->
    mask, lists, attention (blocked layout) -> token-major copy -> O W_o.
    Random weights; X is the bench's synthetic Q field, reordered once; pad
    tokens of the blocked order are zero.  Timed beside it: the same layer
    with the separate passes the split replaces (head-major copy, nabla_pool,
    nabla_transpose_v), and with torch's flash SDPA in place of NABLA (tokens
    of the valid set only)."""
    from torch.nn.attention import SDPBackend, sdpa_kernel
    if cfg.torch_dtype != torch.bfloat16 or cfg.batch != 1:
        return None
    h, d, nb = cfg.heads, cfg.head_dim, g.nb
    S = nb * 64                                   # blocked order, pad slots included
    D = h * d
    # X: the smooth spatio-temporal synthetic field of the bench's Q (40 x 128
    # channels) in the blocked token order, so that the projected Q and K keep
    # a latent-local structure; random N(0, 1/D) weights
    xb = torch.zeros(g.tensor_shape(nabla.LAYOUT_BLOCKED), dtype=torch.bfloat16, device=dev)
    nabla.nabla_flatten(g, x_field, xb)
    X = xb.view(h, S, d).permute(1, 0, 2).reshape(S, D).contiguous()
    del xb
    gen = torch.Generator(device=dev)
    gen.manual_seed(1234)
    Wqkv = (torch.randn(D, 3 * D, generator=gen, device=dev) / math.sqrt(D)).to(torch.bfloat16)
    Wo = (torch.randn(D, D, generator=gen, device=dev) / math.sqrt(D)).to(torch.bfloat16)
    gb = g.with_layout(nabla.LAYOUT_BLOCKED)
    qbar = torch.empty(nabla.qbar_shape(gb), dtype=torch.float32, device=dev)
    kbar = torch.empty(nabla.kbar_shape(gb), dtype=nabla.KBAR_DTYPE, device=dev)
    bits = torch.empty((1, h, nb, g.nw), dtype=torch.int32, device=dev)
    cnt = torch.empty((1, h, nb), dtype=torch.int32, device=dev)
    rp = torch.empty((h, nb + 1), dtype=torch.int32, device=dev)
    ci = torch.empty((h, nb * nb), dtype=torch.int32, device=dev)
    vt = torch.empty(nabla.vt_shape(gb), dtype=torch.bfloat16, device=dev)
    q = torch.empty(gb.tensor_shape(), dtype=torch.bfloat16, device=dev)
    k = torch.empty_like(q)
    o = torch.empty_like(q)
    st = {}

    def proj_in():
        st["qkv"] = torch.matmul(X, Wqkv).view(nabla.qkv_shape(gb))   # [1, S, 3, h, d]

    def split():
        nabla.nabla_qkv_split(gb, st["qkv"], q, k, vt, qbar, kbar)

    def split_separate():                         # what the split replaces
        hm = st["qkv"].permute(2, 0, 3, 1, 4).contiguous().view(3, *gb.tensor_shape())
        nabla.nabla_pool(gb, hm[0], hm[1], qbar, kbar)
        nabla.nabla_transpose_v(gb, hm[2], vt)
        st["hm"] = hm

    def attention():
        split()
        nabla.nabla_mask(gb, qbar, kbar, thr, sta, bits, cnt, None)
        nabla.nabla_compact(gb, bits, cnt, rp, ci)
        nabla.nabla_attn_fwd_vt(gb, q, k, vt, rp, ci, scale, o)
        st["o"] = o

    def proj_out():
        st["y"] = st["o"].view(h, S, d).permute(1, 0, 2).reshape(S, D) @ Wo

    def layer():
        proj_in()
        attention()
        proj_out()

    layer()
    ms = {"qkv_projection": time_call(proj_in, reps=3),
          "qkv_split_with_pooling": time_call(split, reps=3),
          "nabla_attention_incl_split": time_call(attention, reps=3),
          "token_major_copy_and_output_projection": time_call(proj_out, reps=3),
          "layer": time_call(layer, reps=3)}
    separate_ms = time_call(split_separate, reps=3)
    st.pop("hm", None)
    # the same layer with dense flash attention over the valid tokens
    valid = torch.from_numpy(np.ascontiguousarray(valid_slots(cfg, nb))).to(dev)

    def dense_attention():
        qkv = st["qkv"][0]                        # [S, 3, h, d]
        qd, kd, vd = (qkv[valid, i].permute(1, 0, 2).unsqueeze(0).contiguous()
                      for i in range(3))          # [1, h, Sv, d]
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            od = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd)
        out = torch.zeros((h, S, d), dtype=torch.bfloat16, device=dev)
        out[:, valid] = od[0]
        st["o"] = out

    def dense_layer():
        proj_in()
        dense_attention()
        proj_out()

    try:
        dense_ms = time_call(dense_layer, reps=2)
    except RuntimeError as e:
        log(f"dense layer reference unavailable: {e}")
        dense_ms = None
    layer()                                       # the call's own mask, for its sparsity
    torch.cuda.synchronize()
    sparsity = 1.0 - int(cnt.to(torch.int64).sum()) / (h * nb * nb)
    out = {"what": "Wan-shaped self-attention layer, tokens in the blocked order (flattened "
                   "once per network): QKV projection, nabla_qkv_split (q, k, V^T, block "
                   "means), mask + lists + attention, output projection",
           "tokens_blocked": S, "model_dim": D, "sparsity": round(sparsity, 4),
           "ms": {k_: round(v_, 3) for k_, v_ in ms.items()},
           "separate_copy_pool_transpose_ms": round(separate_ms, 3),
           "attention_share": round(ms["nabla_attention_incl_split"] / ms["layer"], 3),
           "dense_flash_layer_ms": None if dense_ms is None else round(dense_ms, 3),
           "layer_speedup_vs_dense_flash": None if dense_ms is None
           else round(dense_ms / ms["layer"], 3)}
    log(f"dit layer: {out}")
    del X, Wqkv, Wo, st, q, k, o, vt
    return out


def valid_slots(cfg, nb):
    """Valid-token flags of the blocked order, [nb * 64] (pad slots False)."""
    gh, gw = -(-cfg.H // 8), -(-cfg.W // 8)
    b = np.arange(nb)
    hb, wb = (b // gw) % gh, b % gw
    s = np.arange(64)
    rows = hb[:, None] * 8 + s[None, :] // 8
    cols = wb[:, None] * 8 + s[None, :] % 8
    return ((rows < cfg.H) & (cols < cfg.W)).reshape(-1)


KERNEL_SOURCES = ("attn_fwd_vt.hip", "attn_common.hpp", "nabla_common.hpp")


def kernel_source_digest():
    """First 16 hex digits of the sha256 of the attention kernel's sources with
    // comments and all white space removed (an edit to comments or layout does
    not change it); None if a source is missing."""
    import hashlib
    import re
    csrc = os.path.join(ROOT, "block_sparse_attention_flatten_amd", "csrc")
    try:
        text = "".join(open(os.path.join(csrc, n)).read() for n in KERNEL_SOURCES)
    except OSError:
        return None
    code = re.sub(r"\s+", "", re.sub(r"//[^\n]*", "", text))
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def traffic_record(workload_is_default):
    """HBM bytes per launch of the attention kernel, from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary of the 720p workload.  Valid only
    while the kernel's code (sources without comments) hashes to the value
    recorded there and the workload is that default one; otherwise None."""
    import re
    if not workload_is_default:
        return None
    path = os.path.join(ROOT, "profiles", "attn_fwd_720p.md")
    try:
        text = open(path).read()
    except OSError:
        return None
    m = re.search(r"<!-- traffic-record: (\{.*?\}) -->", text)
    if not m:
        return None
    rec = json.loads(m.group(1))
    digest = kernel_source_digest()
    if digest is None or rec.get("code_sha256_16") != digest:
        return None
    return float(rec["traffic_bytes"])


def algorithmic_bytes(cfg, nb, nnz_total):
    """HBM bytes each mask-construction stage must move at minimum."""
    bh = cfg.batch * cfg.heads
    es = 2 if cfg.dtype == "bf16" else 4
    d = cfg.head_dim
    nw = -(-nb // 32)
    tokens = cfg.T * cfg.H * cfg.W
    pool = 2 * bh * tokens * d * es + 2 * bh * nb * d * 4
    mask = 2 * bh * nb * d * 4 + bh * nb * nw * 4 + bh * nb * 4
    compact = bh * nb * nw * 4 + bh * nb * 4 + bh * (nb + 1) * 4 + nnz_total * 4
    return pool, mask, compact


def cpu_baseline(cfg, q, k, v, thr, sta, budget_s, gpu_bits=None, gpu_o=None):
    """Time the float64 oracle on a bounded sample of the same workload: one
    head's full mask construction plus attention for as many query blocks as
    fit in the time budget, extrapolated to the whole call.  Given the GPU's
    mask words and output of head 0, also report (after the timing) how they
    compare with the oracle's: band rows, differing rows, output error on the
    sampled query blocks."""
    import numpy as np
    import oracle as O
    try:
        import threadpoolctl
        threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    g = O.Geometry(cfg.T, cfg.H, cfg.W, cfg.P)
    h = 0
    qh = q[0, h].double().cpu().numpy()
    kh = k[0, h].double().cpu().numpy()
    vh = v[0, h].double().cpu().numpy()
    t0 = time.perf_counter()
    valid = O.valid_tokens(g)
    qb, kb, vb = O.flatten(qh, g), O.flatten(kh, g), O.flatten(vh, g)
    m, m_ad, p = O.nabla_mask(O.pool(qb, valid), O.pool(kb, valid), thr, g, sta)
    t_mask = time.perf_counter() - t0
    rng = np.random.default_rng(0)
    order = rng.permutation(g.nb)
    done, t_attn, kept_pairs = 0, 0.0, 0
    outs = []
    while done < g.nb and t_mask + t_attn < budget_s:
        rows = order[done:done + 16]
        t1 = time.perf_counter()
        ob = O.block_sparse_attention(qb, kb, vb, m, valid, rows=rows)
        t_attn += time.perf_counter() - t1
        outs.append((rows, ob))
        kept_pairs += int(m[rows].sum())
        done += len(rows)
    per_head = t_mask + t_attn * g.nb / done
    seconds = per_head * cfg.heads * cfg.batch
    flops_head = int(m.sum()) * 4 * 64 * 64 * cfg.head_dim
    accuracy = None
    if gpu_bits is not None and gpu_o is not None:
        words = gpu_bits.astype(np.uint32)
        gm = ((words[:, np.arange(g.nb) >> 5] >> (np.arange(g.nb) & 31)) & 1).astype(bool)
        band_a, band_b = O.band_rows(p, m_ad, thr)
        band = band_a | band_b
        diff = (gm != m).any(1)
        got = O.flatten(gpu_o, g)
        errs = []
        for rows, ob in outs:
            for r in rows:
                if not diff[r]:                       # rows whose masks agree
                    errs.append(np.abs(got[r][valid[r]] - ob[r][valid[r]]))
        e = np.concatenate([x.ravel() for x in errs]) if errs else np.zeros(1)
        accuracy = {"head": h, "band_rows_a": int(band_a.sum()), "band_rows_b": int(band_b.sum()),
                    "differing_rows": int(diff.sum()),
                    "differing_rows_outside_band": int((diff & ~band).sum()),
                    "output_rows_compared": int(sum(1 for rows, _ in outs for r in rows
                                                    if not diff[r])),
                    "max_abs_err": float(e.max()), "mean_abs_err": float(e.mean())}
    return {
        "value": flops_head * cfg.heads * cfg.batch / seconds / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "accuracy_vs_gpu": accuracy,
        "sample": (f"float64 oracle, head 0 of {cfg.heads}: full mask construction "
                   f"({g.nb} rows) + attention for {done} of {g.nb} query blocks "
                   f"({t_mask + t_attn:.1f} s CPU); extrapolated to the whole call "
                   f"= {seconds:.0f} s"),
        "seconds_per_call_extrapolated": seconds,
        "cpu": cpu_model(),
        "os_cpu_count": os.cpu_count(),
        "cores_note": "cores = BLAS threads the oracle ran with (threadpoolctl)",
    }


def popcount_rows(torch, words, nb):
    """Set bits per row of mask words [..., nb, nw] (bits past nb ignored)."""
    w = words.cpu().numpy().view(np.uint32)
    bits = np.unpackbits(w.view(np.uint8), axis=-1, bitorder="little")[..., :nb]
    return bits.sum(-1, dtype=np.int64)


def valid_token_flops(torch, cfg, nb, rp, ci, d):
    """FLOPs of the kept pairs counted over valid tokens only:
    4 d * sum over kept (a, b) of valid(a) * valid(b)."""
    nval = torch.from_numpy(valid_slots(cfg, nb).reshape(nb, 64).sum(1)).to(rp.device)
    nval = nval.to(torch.float64)
    total = 0.0
    for hh in range(rp.shape[0]):
        nnz_h = int(rp[hh, nb])
        cs = torch.zeros(nnz_h + 1, dtype=torch.float64, device=rp.device)
        cs[1:] = torch.cumsum(nval[ci[hh, :nnz_h].long()], 0)
        row = cs[rp[hh, 1:].long()] - cs[rp[hh, :-1].long()]
        total += float((row * nval).sum())
    return 4.0 * d * total


def config_summary(torch, nabla, synth, name, time_call, stream):
    """Stage times, roofline fractions and sparsity of another workload in the
    same launch configuration (mask construction, V^T, attention)."""
    cfg = synth.config(name)
    q, k, v = synth.make_qkv(cfg, device="cuda")
    g = nabla.Geometry(cfg.batch, cfg.heads, cfg.T, cfg.H, cfg.W, cfg.head_dim, cfg.torch_dtype)
    B, h, nb, d = cfg.batch, cfg.heads, g.nb, cfg.head_dim
    dev = q.device
    qbar = torch.empty(nabla.qbar_shape(g), dtype=torch.float32, device=dev)
    kbar = torch.empty(nabla.kbar_shape(g), dtype=nabla.KBAR_DTYPE, device=dev)
    bits = torch.empty((B, h, nb, g.nw), dtype=torch.int32, device=dev)
    abits = torch.empty_like(bits)
    cnt = torch.empty((B, h, nb), dtype=torch.int32, device=dev)
    rp = torch.empty((B * h, nb + 1), dtype=torch.int32, device=dev)
    ci = torch.empty((B * h, nb * nb), dtype=torch.int32, device=dev)
    vt = torch.empty(nabla.vt_shape(g), dtype=q.dtype, device=dev)
    o = torch.empty_like(q)
    scale = 1.0 / math.sqrt(d)
    mc_ms = time_call(lambda: nabla.nabla_mask_build(g, q, k, cfg.thr, cfg.sta, qbar, kbar, bits,
                                                     cnt, abits, rp, ci, stream), reps=3)
    vt_ms = time_call(lambda: nabla.nabla_transpose_v(g, v, vt, stream), reps=3)
    at_ms = time_call(lambda: nabla.nabla_attn_fwd_vt(g, q, k, vt, rp, ci, scale, o, stream),
                      reps=3)
    torch.cuda.synchronize()
    nnz = int(cnt.to(torch.int64).sum())
    n_ad = int(popcount_rows(torch, abits, nb).sum())
    flops = nnz * 4 * 64 * 64 * d
    mc_bytes = sum(algorithmic_bytes(cfg, nb, nnz))
    out = {"workload": WORKLOAD_NAMES[name], "thr": cfg.thr, "sta": list(cfg.sta),
           "blocks_per_head": nb,
           "sparsity": round(1.0 - nnz / (B * h * nb * nb), 4),
           "sparsity_adaptive_only": round(1.0 - n_ad / (B * h * nb * nb), 4),
           "mask_construction_ms": round(mc_ms, 4),
           "mask_construction_frac": round(mc_bytes / (mc_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "transpose_v_ms": round(vt_ms, 4),
           "attn_ms": round(at_ms, 3),
           "attn_tflops": round(flops / (at_ms * 1e-3) / 1e12, 1),
           "attn_frac": round(flops / (at_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}
    del q, k, v, qbar, kbar, bits, abits, cnt, rp, ci, vt, o
    torch.cuda.empty_cache()
    return out


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def mask_accuracy(cfg, q, k, thr, sta, heads, gpu_bits):
    """Band rows and differing rows of the GPU's mask against the oracle's on
    the given heads (float64 oracle, CPU)."""
    import oracle as O
    g = O.Geometry(cfg.T, cfg.H, cfg.W, cfg.P)
    valid = O.valid_tokens(g)
    out = []
    for hh in heads:
        qb = O.flatten(q[0, hh].double().cpu().numpy(), g)
        kb = O.flatten(k[0, hh].double().cpu().numpy(), g)
        m, m_ad, p = O.nabla_mask(O.pool(qb, valid), O.pool(kb, valid), thr, g, sta)
        band_a, band_b = O.band_rows(p, m_ad, thr)
        words = gpu_bits[hh].astype(np.uint32)
        gm = ((words[:, np.arange(g.nb) >> 5] >> (np.arange(g.nb) & 31)) & 1).astype(bool)
        diff = (gm != m).any(1)
        out.append({"head": int(hh), "band_rows_a": int(band_a.sum()),
                    "band_rows_b": int(band_b.sum()), "differing_rows": int(diff.sum()),
                    "differing_rows_outside_band": int((diff & ~(band_a | band_b)).sum())})
    return out


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the NABLA call "
              "shards by head with no communication, so run it per GPU.", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_attention_flatten_amd as nabla
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    cfg = synth.config(args.config)
    if args.heads is not None:
        cfg = cfg.with_(heads=args.heads)
    thr = cfg.thr if args.thr is None else args.thr
    sta = cfg.sta if args.sta is None else tuple(int(x) for x in args.sta.split(","))
    log(f"config {cfg.name}: {cfg} thr={thr} sta={sta}")
    q, k, v = synth.make_qkv(cfg, device="cuda")
    torch.cuda.synchronize()

    g = nabla.Geometry(cfg.batch, cfg.heads, cfg.T, cfg.H, cfg.W, cfg.head_dim, cfg.torch_dtype)
    B, h, nb, d = cfg.batch, cfg.heads, g.nb, cfg.head_dim
    dev = q.device
    qbar = torch.empty(nabla.qbar_shape(g), dtype=torch.float32, device=dev)
    kbar = torch.empty(nabla.kbar_shape(g), dtype=nabla.KBAR_DTYPE, device=dev)
    bits = torch.empty((B, h, nb, g.nw), dtype=torch.int32, device=dev)
    cnt = torch.empty((B, h, nb), dtype=torch.int32, device=dev)
    rp = torch.empty((B * h, nb + 1), dtype=torch.int32, device=dev)
    ci = torch.empty((B * h, nb * nb), dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    vt_path = cfg.torch_dtype == torch.bfloat16
    vt = (torch.empty((B, h, nb, d, 64), dtype=q.dtype, device=dev) if vt_path else None)
    scale = 1.0 / math.sqrt(d)
    stream = torch.cuda.current_stream()

    ev = lambda: torch.cuda.Event(enable_timing=True)   # noqa: E731

    def attention():
        if vt_path:
            nabla.nabla_attn_fwd_vt(g, q, k, vt, rp, ci, scale, o, stream)
        else:
            nabla.nabla_attn_fwd(g, q, k, v, rp, ci, scale, o, stream)

    # V^T is written on a second stream (default priority) beside the mask
    # kernel and the compaction.  It starts after the step's pooling, which
    # also orders it after the previous step's attention (the last reader of
    # V^T).
    side = torch.cuda.Stream() if vt_path and not args.serial else None
    started, vt_done = torch.cuda.Event(), torch.cuda.Event()

    def step(marks=None):
        if marks is not None:
            marks[0].record(stream)
        # the three calls of nabla_mask_build, with V^T's HBM stream started
        # once pooling (the other HBM-bound stage) is done, beside the mask
        # and the compaction
        nabla.nabla_pool(g, q, k, qbar, kbar, stream)
        if side is not None:
            started.record(stream)
            side.wait_event(started)
            nabla.nabla_transpose_v(g, v, vt, side)
            vt_done.record(side)
        nabla.nabla_mask(g, qbar, kbar, thr, sta, bits, cnt, None, stream)
        nabla.nabla_compact(g, bits, cnt, rp, ci, stream)
        if side is not None:
            stream.wait_event(vt_done)
        elif vt_path:
            nabla.nabla_transpose_v(g, v, vt, stream)
        if marks is not None:
            marks[1].record(stream)
        attention()
        if marks is not None:
            marks[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    marks = [[ev(), ev(), ev()] for _ in range(args.steps)]
    t_start, t_end = ev(), ev()
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(marks[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    mask_ms = sorted(m[0].elapsed_time(m[1]) for m in marks)   # incl. transpose_v
    attn_ms = sorted(m[1].elapsed_time(m[2]) for m in marks)
    attn_avg = sum(attn_ms) / len(attn_ms)
    mask_avg = sum(mask_ms) / len(mask_ms)
    log(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step (mask {mask_avg:.3f}, "
        f"attn {attn_avg:.3f})")

    achievable = None if args.no_peaks else achievable_peaks(torch, stream, ev)
    if achievable is not None:
        log(f"achievable peaks: {achievable}")

    # per-stage breakdown (separate, untimed-region runs) and the explicit reorder
    def time_call(fn, reps=5):
        a, b = ev(), ev()
        fn()
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    xb = torch.empty(g.tensor_shape(nabla.LAYOUT_BLOCKED), dtype=q.dtype, device=dev)
    stages = {
        "mask_build": time_call(lambda: nabla.nabla_mask_build(g, q, k, thr, sta, qbar, kbar, bits,
                                                               cnt, None, rp, ci, stream)),
        "pool": time_call(lambda: nabla.nabla_pool(g, q, k, qbar, kbar, stream)),
        "mask": time_call(lambda: nabla.nabla_mask(g, qbar, kbar, thr, sta, bits, cnt, None,
                                                   stream)),
        "compact": time_call(lambda: nabla.nabla_compact(g, bits, cnt, rp, ci, stream)),
        "transpose_v": (time_call(lambda: nabla.nabla_transpose_v(g, v, vt, stream))
                        if vt_path else 0.0),
        "attn_fwd": attn_avg,
        "flatten_one_tensor": time_call(lambda: nabla.nabla_flatten(g, q, xb, stream)),
        "unflatten_one_tensor": time_call(lambda: nabla.nabla_unflatten(g, xb, o, stream)),
    }
    # restore o (the unflatten timing overwrote it) and measure the mask statistics
    step()
    torch.cuda.synchronize()
    counts = cnt.to(torch.int64)
    nnz = int(counts.sum())
    kept_flops = nnz * 4 * 64 * 64 * d
    sparsity = 1.0 - nnz / (B * h * nb * nb)
    per_row = counts.flatten().float()
    abits = torch.empty_like(bits)
    nabla.nabla_mask(g, qbar, kbar, thr, sta, bits, cnt, abits, stream)
    torch.cuda.synchronize()
    n_adaptive = int(popcount_rows(torch, abits, nb).sum())
    del abits
    valid_flops = valid_token_flops(torch, cfg, nb, rp, ci, d)
    pool_b, mask_b, compact_b = algorithmic_bytes(cfg, nb, nnz)
    mc_bytes = pool_b + mask_b + compact_b
    mc_ms = stages["mask_build"]

    attn_tflops = kept_flops / (attn_avg * 1e-3) / 1e12
    value = kept_flops / (ms_per_step * 1e-3) / 1e12
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded smooth spatio-temporal fields + noise; no weights)",
        "config": {
            "workload": WORKLOAD_NAMES[cfg.name] + (
                f" [heads overridden to {cfg.heads}]" if args.heads is not None else ""),
            "batch": B, "heads": h, "head_dim": d, "latent_THW": [cfg.T, cfg.H, cfg.W],
            "patch": cfg.P, "blocks_per_head": nb, "tokens_padded": nb * 64,
            "thr": thr, "sta": list(sta),
        },
        "roofline": {
            "kernel": ("nabla_attn_fwd_vt (attn_fwd_vt_kernel)" if vt_path
                       else "nabla_attn_fwd (attn_fwd_f32_kernel)"),
            "bound": "mfma",
            "achieved": round(attn_tflops, 2),
            "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / BF16_PEAK_TFLOPS, 4),
            "traffic": traffic_record(vt_path and cfg.name == "720p" and args.heads is None
                                      and args.thr is None and args.sta is None),
            "traffic_unit": "bytes per launch fetched and written beyond L2 (Infinity Cache "
                            "and HBM; FETCH_SIZE / WRITE_SIZE, copy-calibrated)",
            "work_per_launch": f"{nnz} kept 64x64 block pairs x 4*64*64*{d} flop = "
                               f"{kept_flops / 1e12:.3f} TFLOP (pad slots of edge blocks "
                               "included: the kernel computes whole blocks)",
            "valid_token_tflop": round(valid_flops / 1e12, 3),
            "valid_token_tflops": round(valid_flops / (attn_avg * 1e-3) / 1e12, 2),
            "avg_launch_ms": round(attn_avg, 4),
        },
        "mask_construction": {
            "what": "nabla_mask_build: pooling, reduced map + CDF cut + STA, compressed lists",
            "bound": "hbm",
            "ms": round(mc_ms, 4),
            "algorithmic_bytes": mc_bytes,
            "achieved": round(mc_bytes / (mc_ms * 1e-3) / 1e9, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(mc_bytes / (mc_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        },
        "achievable_peaks": achievable,
        "stages_ms": {k_: round(v_, 4) for k_, v_ in stages.items()},
        "attn_ms_min_median": [round(attn_ms[0], 4), round(attn_ms[len(attn_ms) // 2], 4)],
        "sparsity": round(sparsity, 4),
        "sparsity_adaptive_only": round(1.0 - n_adaptive / (B * h * nb * nb), 4),
        "kept_per_row_min_mean_max": [int(per_row.min()), round(float(per_row.mean()), 1),
                                      int(per_row.max())],
        "gpu": torch.cuda.get_device_name(0),
    }
    if args.thr_sweep:
        # sparsity and attention time against thr with the same inputs and STA
        # window; thr = 0 is the pure STA mask (adaptive part off)
        sweep = []
        for t in [float(x) for x in args.thr_sweep.split(",")]:
            if t == 0.0 and not any(sta):
                continue
            nabla.nabla_mask(g, qbar, kbar, t, sta, bits, cnt, None, stream)
            nabla.nabla_compact(g, bits, cnt, rp, ci, stream)
            t_ms = time_call(attention, reps=3)
            n_t = int(cnt.to(torch.int64).sum())
            f_t = n_t * 4 * 64 * 64 * d
            sweep.append({"thr": t, "sparsity": round(1.0 - n_t / (B * h * nb * nb), 4),
                          "attn_ms": round(t_ms, 3),
                          "tflops": round(f_t / (t_ms * 1e-3) / 1e12, 1)})
        result["thr_sweep"] = sweep
        log(f"thr sweep: {sweep}")
        step()                       # restore the call's own mask and lists
        torch.cuda.synchronize()
    if not args.no_backward:
        # gradients with the mask held fixed: the forward with its log-sum-exp,
        # the key-major lists, then dQ (and D) and dK/dV; incoming gradient
        # dO is a synthetic field of the same shape
        dout = synth.make_tensor(cfg, 3, device="cuda")
        lse = torch.empty(nabla.lse_shape(g), dtype=torch.float32, device=dev)
        if vt_path:
            nabla.nabla_attn_fwd_vt_lse(g, q, k, vt, rp, ci, scale, o, lse, stream)
        else:
            nabla.nabla_attn_fwd_lse(g, q, k, v, rp, ci, scale, o, lse, stream)
        bits_t = torch.empty_like(bits)
        cnt_t = torch.empty_like(cnt)
        cp = torch.empty_like(rp)
        ri = torch.empty_like(ci)
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        delta = torch.empty_like(lse)
        bstages = {
            "mask_transpose": time_call(lambda: nabla.nabla_mask_transpose(g, bits, bits_t,
                                                                           cnt_t, stream)),
            "compact_transposed": time_call(lambda: nabla.nabla_compact(g, bits_t, cnt_t, cp, ri,
                                                                        stream)),
            "dq": time_call(lambda: nabla.nabla_attn_bwd_dq(g, q, k, v, o, dout, lse, rp, ci,
                                                            scale, dq, delta, stream), reps=3),
            "dkdv": time_call(lambda: nabla.nabla_attn_bwd_dkdv(g, q, k, v, dout, lse, delta, cp,
                                                                ri, scale, dk, dv, stream),
                              reps=3),
        }
        bwd_ms = sum(bstages.values())
        bwd_flops = 2.5 * kept_flops         # five 64x64xd products per kept pair vs two
        result["backward"] = {
            "what": "dq, dk, dv with the mask held fixed (transposed lists + dQ + dK/dV)",
            "ms": round(bwd_ms, 3),
            "stages_ms": {k_: round(v_, 4) for k_, v_ in bstages.items()},
            "algorithmic_tflop": round(bwd_flops / 1e12, 3),
            "tflops": round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 1),
            "frac": round(bwd_flops / (bwd_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
        }
        log(f"backward: {bwd_ms:.2f} ms {bstages}")
        del dout, lse, bits_t, cnt_t, cp, ri, dq, dk, dv, delta
    if not args.no_dense:
        # dense reference: nabla_dense_attn_fwd, full attention over every
        # valid key (no mask, no lists); the sparse kernel walking the
        # all-kept lists is timed beside it
        rp_full = (torch.arange(nb + 1, dtype=torch.int32, device=dev) * nb).expand(B * h, nb + 1)
        rp_full = rp_full.contiguous()
        ci_full = torch.arange(nb, dtype=torch.int32, device=dev).repeat(B * h, nb).contiguous()
        dense_flops = B * h * nb * nb * 4 * 64 * 64 * d

        def all_kept():
            if vt_path:
                nabla.nabla_attn_fwd_vt(g, q, k, vt, rp_full, ci_full, scale, o, stream)
            else:
                nabla.nabla_attn_fwd(g, q, k, v, rp_full, ci_full, scale, o, stream)
        kept_ms = time_call(all_kept, reps=3)
        del rp_full, ci_full
        result["dense_reference"] = {}
        if vt_path:
            dense_ms = time_call(
                lambda: nabla.nabla_dense_attn_fwd(g, q, k, vt, scale, o, None, stream), reps=3)
            result["dense_reference"] = {
                "what": "nabla_dense_attn_fwd: full attention, every valid key, no mask or lists",
                "ms": round(dense_ms, 3),
                "tflops": round(dense_flops / (dense_ms * 1e-3) / 1e12, 1),
                "frac": round(dense_flops / (dense_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                "speedup_sparse_vs_dense": round(dense_ms / attn_avg, 3),
            }
            log(f"dense: {dense_ms:.2f} ms ({result['dense_reference']['tflops']} TFLOP/s)")
        result["dense_reference"]["sparse_kernel_all_kept"] = {
            "what": "the sparse kernel walking every block (thr = 1, no STA)",
            "ms": round(kept_ms, 3),
            "tflops": round(dense_flops / (kept_ms * 1e-3) / 1e12, 1),
        }
        tf = torch_flash_reference(torch, cfg, q, k, v, time_call, attn_avg)
        if tf is not None and "backward" in result:
            tf["speedup_sparse_backward_vs_torch_flash"] = round(
                tf["backward_ms"] / result["backward"]["ms"], 3)
        result["dense_reference"]["torch_sdpa_flash"] = tf
    if not args.no_layer:
        result["dit_layer"] = layer_leg(torch, nabla, cfg, g, q, thr, sta, scale, time_call, dev)
    if not args.no_configs and cfg.name == "720p" and args.heads is None:
        result["other_configs"] = {}
        for name in ("480p", "long"):
            result["other_configs"][name] = config_summary(torch, nabla, synth, name, time_call,
                                                           stream)
            log(f"{name}: {result['other_configs'][name]}")
    if not args.no_cpu_baseline:
        step()                       # the call's own mask and output again (the legs above
        torch.cuda.synchronize()     # reused the buffers)
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(
            cfg, q, k, v, thr, sta, args.cpu_seconds,
            gpu_bits=bits[0, 0].cpu().numpy(), gpu_o=o[0, 0].double().cpu().numpy())
        log(f"cpu baseline done: {result['cpu_baseline']['value']:.6f} TFLOP/s; "
            f"head 0 vs the oracle: {result['cpu_baseline']['accuracy_vs_gpu']}")
        heads = sorted(set(synth.sampled_heads(cfg)) - {0})
        acc = mask_accuracy(cfg, q, k, thr, sta, heads, bits[0].cpu().numpy())
        result["cpu_baseline"]["mask_vs_oracle_other_sampled_heads"] = acc
        log(f"mask vs oracle: {acc}")
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

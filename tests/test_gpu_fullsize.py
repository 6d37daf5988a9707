"""GPU parity at the full Wan-2.1-shaped sizes (480p, 720p, Long sweep), in the
launch configuration the bench times: all 40 heads run on the GPU; the oracle
checks the masks of sampled heads in full and the outputs of sampled query
blocks of those heads."""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from gpu_helpers import (check_bf16_rounding, check_mask_rows, check_output, f64, log, ogeom,
                         oracle_mask, run_pipeline, unpack_bits)

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
        rows = [r for r in _sample_rows(cfg, nb) if not (union[r] != ref["mask"][r]).any()]
        ob = O.block_sparse_attention(O.flatten(qh, og), O.flatten(kh, og), O.flatten(vh, og),
                                      ref["mask"], ref["valid"], rows=rows)
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

"""Plant plausible mistakes in the oracle (CPU only) and check that the pins
catch every one of them.  Each mutation replaces one function of the oracle
module for the duration of one test."""
import math
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(__file__))

import oracle.nabla_oracle as M  # noqa: E402
from oracle_pins import ALL_PINS  # noqa: E402


def _positions(order):
    def f(g):
        P = g.P
        _, gh, gw = g.grid
        pos = np.empty((g.T, g.H, g.W), dtype=np.int64)
        for t in range(g.T):
            for h in range(g.H):
                for w in range(g.W):
                    pos[t, h, w] = order(g, P, gh, gw, t, h, w)
        return pos
    return f


def _col_major(g, P, gh, gw, t, h, w):
    return ((t * gh + h // P) * gw + w // P) * P * P + (w % P) * P + (h % P)


def _time_inner(g, P, gh, gw, t, h, w):
    return (((h // P) * gw + w // P) * g.T + t) * P * P + (h % P) * P + (w % P)


def _patch_col_major(g, P, gh, gw, t, h, w):
    return ((t * gw + w // P) * gh + h // P) * P * P + (h % P) * P + (w % P)


def _pool_div_n(xb, valid):
    return (np.asarray(xb, np.float64) * valid[..., None]).sum(-2) / valid.shape[-1]


def _map_no_scale(qbar, kbar):
    s = np.matmul(qbar, np.swapaxes(kbar, -1, -2))
    e = np.exp(s - s.max(-1, keepdims=True))
    return e / e.sum(-1, keepdims=True)


def _map_wrong_axis(qbar, kbar):
    s = np.matmul(qbar, np.swapaxes(kbar, -1, -2)) / math.sqrt(qbar.shape[-1])
    e = np.exp(s - s.max(-2, keepdims=True))
    return e / e.sum(-2, keepdims=True)


def _cdf_ge(p, thr):
    if thr >= 1:
        return np.ones(p.shape[0], bool)
    order = np.lexsort((-np.arange(p.shape[0]), p))
    keep = np.zeros(p.shape[0], bool)
    keep[order] = np.cumsum(p[order]) >= 1.0 - thr
    return keep


def _cdf_tail(p, thr):
    # "keep where the (descending) cumulative probability exceeds thr"
    order = np.argsort(-p, kind="stable")
    keep = np.zeros(p.shape[0], bool)
    keep[order] = np.cumsum(p[order]) > thr
    return keep


def _cdf_tie_high(p, thr):
    if thr >= 1:
        return np.ones(p.shape[0], bool)
    order = np.lexsort((np.arange(p.shape[0]), p))
    keep = np.zeros(p.shape[0], bool)
    keep[order] = np.cumsum(p[order]) > 1.0 - thr
    return keep


def _cdf_no_full(p, thr):
    # no special case for thr >= 1: blocks of zero probability get dropped
    order = np.lexsort((-np.arange(p.shape[0]), p))
    keep = np.zeros(p.shape[0], bool)
    keep[order] = np.cumsum(p[order]) > 1.0 - thr
    return keep


def _sta_wide(g, window):
    wt, wh, ww = window
    if not (wt or wh or ww):
        return np.zeros((g.nb, g.nb), bool)
    gt, gh, gw = g.grid
    c = np.array([(t, h, w) for t in range(gt) for h in range(gh) for w in range(gw)])
    return np.all(np.abs(c[:, None] - c[None]) <= np.array(window) // 2 + 1, -1)


def _sta_periodic(g, window):
    wt, wh, ww = window
    if not (wt or wh or ww):
        return np.zeros((g.nb, g.nb), bool)
    gt, gh, gw = g.grid
    c = np.array([(t, h, w) for t in range(gt) for h in range(gh) for w in range(gw)])
    d = np.abs(c[:, None] - c[None])
    d = np.minimum(d, np.array(g.grid) - d)
    return np.all(d <= np.array(window) // 2, -1)


def _union_and(qbar, kbar, thr, g, window=(0, 0, 0)):
    p = M.reduced_map(qbar, kbar)
    m_ad = M.cdf_keep(p, thr)
    sta = M.sta_mask(g, window)
    return (m_ad & sta) if sta.any() else m_ad, m_ad, p


def _attn_variant(pad_keys=False, scale=True, axis=1):
    def f(qb, kb, vb, m, valid, rows=None, scale_=None, **kw):
        qb, kb, vb = (np.asarray(x, np.float64) for x in (qb, kb, vb))
        nb, N, d = qb.shape
        out = np.zeros((nb, N, d))
        for a in (range(nb) if rows is None else rows):
            cols = np.flatnonzero(m[a])
            sel = np.ones_like(valid[cols]) if pad_keys else valid[cols]
            keys, vals = kb[cols][sel], vb[cols][sel]
            s = qb[a][valid[a]] @ keys.T * ((1 / math.sqrt(d)) if scale else 1.0)
            s = s - s.max(axis=axis, keepdims=True)
            w = np.exp(s)
            w = w / w.sum(axis=axis, keepdims=True)
            out[a][valid[a]] = w @ vals
        return out
    return f


def _csr_desc(m):
    counts = m.sum(1)
    rp = np.concatenate([[0], np.cumsum(counts)])
    return rp, np.concatenate([np.flatnonzero(r)[::-1] for r in m])


def _band_first_kept(p, m_ad, thr, eps=1e-5):
    fp, fm = p.reshape(-1, p.shape[-1]), m_ad.reshape(-1, p.shape[-1])
    a = np.zeros(fp.shape[0], bool)
    b = np.zeros(fp.shape[0], bool)
    for i, (row, keep) in enumerate(zip(fp, fm)):
        kept = np.sort(row[keep])[::-1]
        dropped = np.sort(row[~keep])[::-1]
        dk = kept.sum()
        a[i] = abs(dk - thr) < eps or abs(dk - kept[0] - thr) < eps
        if dropped.size:
            b[i] = (kept[0] - dropped[0]) < eps * kept[0]
    return a, b


def _bwd_variant(no_rowsum=False, dk_scale=True, dp_keys=False):
    def f(qb, kb, vb, m, valid, dob, scale=None):
        qb, kb, vb, dob = (np.asarray(x, np.float64) for x in (qb, kb, vb, dob))
        nb, N, d = qb.shape
        sc = 1 / math.sqrt(d) if scale is None else scale
        dq, dk, dv = (np.zeros((nb, N, d)) for _ in range(3))
        lse = np.full((nb, N), -np.inf)
        slot = np.arange(N)
        for a in range(nb):
            cols = np.flatnonzero(m[a])
            kblk = np.repeat(cols, N)[valid[cols].ravel()]
            kslot = np.tile(slot, len(cols))[valid[cols].ravel()]
            keys, vals = kb[kblk, kslot], vb[kblk, kslot]
            qi = np.flatnonzero(valid[a])
            q, do = qb[a, qi], dob[a, qi]
            s = q @ keys.T * sc
            w = np.exp(s - s.max(1, keepdims=True))
            p = w / w.sum(1, keepdims=True)
            lse[a, qi] = scipy_lse(s)
            o = p @ vals
            dp = do @ (keys if dp_keys else vals).T
            ds = p * dp if no_rowsum else p * (dp - (do * o).sum(1, keepdims=True))
            dq[a, qi] = ds @ keys * sc
            np.add.at(dk, (kblk, kslot), ds.T @ q * (sc if dk_scale else 1.0))
            np.add.at(dv, (kblk, kslot), p.T @ do)
        return dq, dk, dv, lse
    return f


def scipy_lse(s):
    import scipy.special
    return scipy.special.logsumexp(s, axis=1)


MUTATIONS = {
    "flatten_col_major_in_patch": ("flatten_positions", _positions(_col_major)),
    "flatten_time_innermost": ("flatten_positions", _positions(_time_inner)),
    "flatten_patches_col_major": ("flatten_positions", _positions(_patch_col_major)),
    "pool_divides_by_N": ("pool", _pool_div_n),
    "map_without_scale": ("reduced_map", _map_no_scale),
    "map_softmax_wrong_axis": ("reduced_map", _map_wrong_axis),
    "cdf_ge_instead_of_gt": ("cdf_keep_row", _cdf_ge),
    "cdf_keeps_tail": ("cdf_keep_row", _cdf_tail),
    "cdf_ties_high_index": ("cdf_keep_row", _cdf_tie_high),
    "cdf_thr1_not_full": ("cdf_keep_row", _cdf_no_full),
    "sta_one_block_wider": ("sta_mask", _sta_wide),
    "sta_periodic_borders": ("sta_mask", _sta_periodic),
    "union_is_and": ("nabla_mask", _union_and),
    "attn_pad_keys_weighted": ("block_sparse_attention", _attn_variant(pad_keys=True)),
    "attn_no_scale": ("block_sparse_attention", _attn_variant(scale=False)),
    "attn_softmax_wrong_axis": ("block_sparse_attention", _attn_variant(axis=0)),
    "csr_descending": ("to_csr", _csr_desc),
    "band_uses_top_block": ("band_rows", _band_first_kept),
    "bwd_without_rowsum_term": ("block_sparse_attention_backward", _bwd_variant(no_rowsum=True)),
    "bwd_dk_unscaled": ("block_sparse_attention_backward", _bwd_variant(dk_scale=False)),
    "bwd_dp_uses_keys": ("block_sparse_attention_backward", _bwd_variant(dp_keys=True)),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(M, attr, fn)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(M)
        except Exception as e:  # AssertionError, or a shape error from the planted bug
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught mutation {name}"

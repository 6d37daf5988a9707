"""NABLA oracle: a plain, slow, float64 CPU implementation of one NABLA
self-attention call.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run this module.  It shares
no code, constants or helpers with the HIP library, and the library never
calls it.

Sources (pages as titled; section named):
  [GZ] "NABLA: Neighborhood Adaptive Block-Level Attention", gist.science
       (Chinese), technical summary -> "Methodology: NABLA" (token reordering,
       adaptive mask construction, hybrid STA union).
  [LS] lsdiaocha.cn article on NABLA (Sber AI), section 2 "core innovations of
       the NABLA algorithm" and section 4 "technical principles", section 5
       "comparison with existing techniques" (compressed sparse storage).

Every step is written the way those pages state it, in their order:
fractal flatten -> average-pool Q and K into blocks -> full softmax attention
on the pooled blocks -> per-row CDF threshold -> (optional) union with a
sliding-tile window -> exact attention restricted to kept N x N token blocks.
Library primitives used as steps: numpy sort/cumsum/matmul/exp.

Readings of points the pages leave open (each is also listed with the
design notes):
  * flatten: one level of P x P patches, row-major inside a patch, time
    outermost; latent H, W padded up to multiples of P with pad tokens.
  * pooling: a block is N = P*P consecutive flattened tokens; its delegate is
    the mean over the block's *valid* (non-pad) tokens.
  * reduced map: scores q_bar . k_bar / sqrt(d), softmax along each row.
  * CDF cut: sort a row ascending, cumulate, keep blocks whose cumulative
    probability exceeds 1 - thr.  Equal probabilities: the lower block index is
    treated as the more important one (kept first).  thr >= 1 keeps every block;
    thr = 0 keeps none (pure STA when combined with a window).
  * STA: a window of (wt, wh, ww) blocks centred on the query block in
    (frame, block-row, block-column) coordinates, clipped at the borders.
  * attention: pad keys never receive weight; pad queries produce zeros.
  * gradients: the kept-block mask is held fixed (it is a threshold, so it
    has no useful derivative); pad slots receive zero gradient.

Pins: every function here is checked by tests against values the pages fix,
closed forms, library routines or brute force (tests/test_oracle_pins.py).
"""
from __future__ import annotations

import functools
import math
from dataclasses import dataclass
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "Geometry", "flatten_positions", "flatten", "unflatten", "valid_tokens",
    "pool", "reduced_map", "cdf_keep_row", "cdf_keep", "sta_mask", "nabla_mask",
    "to_csr", "block_sparse_attention", "block_sparse_attention_backward", "band_rows",
    "nabla_forward",
]


# ---------------------------------------------------------------------------
# geometry
# ---------------------------------------------------------------------------
@dataclass(frozen=True)
class Geometry:
    """Latent T x H x W (valid extents) cut into P x P spatial patches."""

    T: int
    H: int
    W: int
    P: int = 8

    @property
    def Hp(self) -> int:          # height padded to a multiple of P
        return -(-self.H // self.P) * self.P

    @property
    def Wp(self) -> int:
        return -(-self.W // self.P) * self.P

    @property
    def grid(self) -> Tuple[int, int, int]:   # block grid (t, h, w)
        return self.T, self.Hp // self.P, self.Wp // self.P

    @property
    def nb(self) -> int:                      # number of blocks
        t, h, w = self.grid
        return t * h * w

    @property
    def N(self) -> int:                       # tokens per block
        return self.P * self.P

    @property
    def S(self) -> int:                       # padded, flattened sequence
        return self.nb * self.N


# ---------------------------------------------------------------------------
# step 1: fractal flatten   ([GZ] Methodology, token reordering)
# ---------------------------------------------------------------------------
@functools.lru_cache(maxsize=16)
def flatten_positions(g: Geometry) -> np.ndarray:
    """Position in the flattened sequence of every valid token (t, h, w).

    Tokens of one P x P spatial patch of one frame become one contiguous run of
    P*P positions (row-major inside the patch); patches follow each other
    row-major over the frame, and frames keep their temporal order.
    Returns int64 array [T, H, W].
    """
    P = g.P
    _, gh, gw = g.grid
    pos = np.empty((g.T, g.H, g.W), dtype=np.int64)
    for t in range(g.T):
        for h in range(g.H):
            for w in range(g.W):
                patch = (t * gh + h // P) * gw + w // P
                pos[t, h, w] = patch * P * P + (h % P) * P + (w % P)
    pos.flags.writeable = False
    return pos


def valid_tokens(g: Geometry) -> np.ndarray:
    """Boolean [nb, N]: which slots of the flattened sequence hold real tokens."""
    v = np.zeros(g.S, dtype=bool)
    v[flatten_positions(g).ravel()] = True
    return v.reshape(g.nb, g.N)


def flatten(x: np.ndarray, g: Geometry) -> np.ndarray:
    """[..., T, H, W, d] -> [..., nb, N, d]; pad slots are zero."""
    lead = x.shape[:-4]
    d = x.shape[-1]
    out = np.zeros(lead + (g.S, d), dtype=x.dtype)
    out[..., flatten_positions(g).ravel(), :] = x.reshape(lead + (-1, d))
    return out.reshape(lead + (g.nb, g.N, d))


def unflatten(xb: np.ndarray, g: Geometry) -> np.ndarray:
    """Inverse of :func:`flatten` on the valid slots: [..., nb, N, d] -> [..., T, H, W, d]."""
    lead = xb.shape[:-3]
    d = xb.shape[-1]
    flat = xb.reshape(lead + (g.S, d))
    return flat[..., flatten_positions(g).ravel(), :].reshape(lead + (g.T, g.H, g.W, d))


# ---------------------------------------------------------------------------
# step 2: block average pooling   ([GZ] Methodology, downsampling; [LS] sec. 2)
# ---------------------------------------------------------------------------
def pool(xb: np.ndarray, valid: np.ndarray) -> np.ndarray:
    """Mean of each block's valid tokens: [..., nb, N, d] -> [..., nb, d] (float64)."""
    xb = np.asarray(xb, dtype=np.float64)
    w = valid.astype(np.float64)[..., None]                # [nb, N, 1]
    return (xb * w).sum(axis=-2) / w.sum(axis=-2)


# ---------------------------------------------------------------------------
# step 3: reduced attention map   ([GZ] Methodology, reduced attention)
# ---------------------------------------------------------------------------
def reduced_map(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """Full softmax attention between pooled blocks: [..., nb, d] x2 -> [..., nb, nb]."""
    d = qbar.shape[-1]
    s = np.matmul(qbar, np.swapaxes(kbar, -1, -2)) / math.sqrt(d)
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=-1, keepdims=True)


# ---------------------------------------------------------------------------
# step 4: CDF threshold   ([GZ] Methodology, CDF thresholding; [LS] sec. 2, 4)
# ---------------------------------------------------------------------------
def cdf_keep_row(p: np.ndarray, thr: float) -> np.ndarray:
    """Binarise one row of the reduced map.

    The row is sorted ascending and cumulated; a block is kept when its
    cumulative probability exceeds 1 - thr.  Among equal probabilities the
    higher block index sorts first in ascending order, so the lower index is
    kept first.  thr >= 1 keeps every block; thr = 0 keeps none (with an STA
    window this is the pure-STA mask, the pages' static baseline).
    """
    n = p.shape[0]
    if thr >= 1.0:
        return np.ones(n, dtype=bool)
    if thr <= 0.0:
        return np.zeros(n, dtype=bool)
    idx = np.arange(n)
    order = np.lexsort((-idx, p))          # ascending p; ties: descending index
    cdf = np.cumsum(p[order])
    keep = np.zeros(n, dtype=bool)
    keep[order] = cdf > 1.0 - thr
    return keep


def cdf_keep(p: np.ndarray, thr: float) -> np.ndarray:
    """Row-wise :func:`cdf_keep_row` over [..., nb, nb]."""
    flat = p.reshape(-1, p.shape[-1])
    out = np.stack([cdf_keep_row(r, thr) for r in flat])
    return out.reshape(p.shape)


# ---------------------------------------------------------------------------
# step 5: STA window and union   ([GZ] Methodology, hybrid integration with STA)
# ---------------------------------------------------------------------------
def sta_mask(g: Geometry, window: Sequence[int]) -> np.ndarray:
    """Sliding-tile mask [nb, nb]: query block and key block lie within a
    (wt, wh, ww) window of each other in block coordinates (clipped at borders).
    window (0, 0, 0) means no STA."""
    wt, wh, ww = window
    nb = g.nb
    if wt == 0 and wh == 0 and ww == 0:
        return np.zeros((nb, nb), dtype=bool)
    gt, gh, gw = g.grid
    coords = np.array([(t, h, w) for t in range(gt) for h in range(gh) for w in range(gw)])
    diff = np.abs(coords[:, None, :] - coords[None, :, :])
    half = np.array([wt // 2, wh // 2, ww // 2])
    return np.all(diff <= half, axis=-1)


def nabla_mask(qbar: np.ndarray, kbar: np.ndarray, thr: float, g: Geometry,
               window: Sequence[int] = (0, 0, 0)):
    """Adaptive mask, its union with STA, and the reduced probabilities.

    Returns (M, M_adaptive, p); M = M_adaptive OR M_STA, all [..., nb, nb]."""
    p = reduced_map(qbar, kbar)
    m_ad = cdf_keep(p, thr)
    return m_ad | sta_mask(g, window), m_ad, p


# ---------------------------------------------------------------------------
# step 6: compressed storage   ([LS] sec. 5, only the compressed sparse matrix)
# ---------------------------------------------------------------------------
def to_csr(m: np.ndarray):
    """Per-row ascending kept block indices of an [nb, nb] mask -> (row_ptr, col_idx)."""
    counts = m.sum(axis=1)
    row_ptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    col_idx = np.concatenate([np.flatnonzero(r) for r in m]).astype(np.int64)
    return row_ptr, col_idx


# ---------------------------------------------------------------------------
# step 7: exact attention on the kept token blocks
#         ([GZ] Methodology, expansion back to token resolution; [LS] sec. 2)
# ---------------------------------------------------------------------------
def block_sparse_attention(qb: np.ndarray, kb: np.ndarray, vb: np.ndarray,
                           m: np.ndarray, valid: np.ndarray,
                           rows: Optional[Iterable[int]] = None,
                           scale: Optional[float] = None) -> np.ndarray:
    """One head: softmax(q k^T * scale) v over the valid tokens of kept blocks.

    qb, kb, vb: [nb, N, d]; m: [nb, nb] bool; valid: [nb, N] bool.
    Returns [nb, N, d] float64 (rows not requested and pad queries are zero).
    """
    qb = np.asarray(qb, dtype=np.float64)
    kb = np.asarray(kb, dtype=np.float64)
    vb = np.asarray(vb, dtype=np.float64)
    nb, N, d = qb.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    out = np.zeros((nb, N, d))
    for a in (range(nb) if rows is None else rows):
        cols = np.flatnonzero(m[a])
        keys = kb[cols][valid[cols]]                 # [n_keys, d]
        vals = vb[cols][valid[cols]]
        q = qb[a][valid[a]]                          # [n_q, d]
        s = (q @ keys.T) * scale
        s = s - s.max(axis=1, keepdims=True)
        w = np.exp(s)
        w = w / w.sum(axis=1, keepdims=True)
        out[a][valid[a]] = w @ vals
    return out


# ---------------------------------------------------------------------------
# gradients of step 7 with the mask held fixed (training with NABLA:
# [GZ] core contributions, acceleration of pre-training / fine-tuning, and
# experimental results 2, pre-training of a 2B DiT; [LS] sec. 3)
# ---------------------------------------------------------------------------
def block_sparse_attention_backward(qb: np.ndarray, kb: np.ndarray, vb: np.ndarray,
                                    m: np.ndarray, valid: np.ndarray, dob: np.ndarray,
                                    scale: Optional[float] = None,
                                    rows: Optional[Iterable[int]] = None):
    """One head: gradients of L = sum(dob * o) for o = block_sparse_attention(...).

    The kept-block mask is a piecewise-constant function of q and k (a
    threshold on pooled scores), so it is held fixed: only the exact
    attention over the kept blocks is differentiated.  Plain definition:
    p = softmax(s), s = q k^T * scale over the valid keys of the kept blocks,
    o = p v; dv = p^T do, dp = do v^T, ds = p (dp - rowsum(do * o)),
    dq = ds k * scale, dk = ds^T q * scale.

    qb, kb, vb, dob: [nb, N, d]; m: [nb, nb] bool; valid: [nb, N] bool.
    Returns dq, dk, dv [nb, N, d] float64 (zero at pad slots) and lse [nb, N],
    the natural-log log-sum-exp of each valid query's scores (-inf for pad
    queries and for rows without keys).  With ``rows``, only those query blocks
    are processed: their dq and lse are exact, and dk, dv hold their
    contributions only (exact for a key block when rows covers every query
    block that keeps it).
    """
    qb = np.asarray(qb, dtype=np.float64)
    kb = np.asarray(kb, dtype=np.float64)
    vb = np.asarray(vb, dtype=np.float64)
    dob = np.asarray(dob, dtype=np.float64)
    nb, N, d = qb.shape
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    dq = np.zeros((nb, N, d))
    dk = np.zeros((nb, N, d))
    dv = np.zeros((nb, N, d))
    lse = np.full((nb, N), -np.inf)
    slot = np.arange(N)
    for a in (range(nb) if rows is None else rows):
        cols = np.flatnonzero(m[a])
        kblk = np.repeat(cols, N)[valid[cols].ravel()]          # key token -> block
        kslot = np.tile(slot, len(cols))[valid[cols].ravel()]   # key token -> slot
        if kblk.size == 0:
            continue
        keys, vals = kb[kblk, kslot], vb[kblk, kslot]         # [n_keys, d]
        qi = np.flatnonzero(valid[a])
        q, do = qb[a, qi], dob[a, qi]                          # [n_q, d]
        s = (q @ keys.T) * scale
        mx = s.max(axis=1, keepdims=True)
        w = np.exp(s - mx)
        z = w.sum(axis=1, keepdims=True)
        p = w / z
        lse[a, qi] = (mx + np.log(z))[:, 0]
        o = p @ vals
        dp = do @ vals.T
        ds = p * (dp - (do * o).sum(axis=1, keepdims=True))
        dq[a, qi] = (ds @ keys) * scale
        # each key token appears once in a row's list: a plain indexed add
        dk[kblk, kslot] += (ds.T @ q) * scale
        dv[kblk, kslot] += p.T @ do
    return dq, dk, dv, lse


# ---------------------------------------------------------------------------
# tolerance classes for comparing masks computed in other precisions
# ---------------------------------------------------------------------------
def band_rows(p: np.ndarray, m_ad: np.ndarray, thr: float, eps: float = 1e-5):
    """Rows whose CDF cut an fp32 computation may legitimately place differently.

    For each row, with blocks ordered by descending probability: D_k is the
    kept mass and D_{k-1} the mass above the least kept block.  Class "a": either
    lies within ``eps`` of thr.  Class "b": the least kept and the most
    probable dropped block differ by less than ``eps`` relative (a near tie
    that can swap which of them is kept).  Returns two boolean arrays [...].
    """
    flat_p = p.reshape(-1, p.shape[-1])
    flat_m = m_ad.reshape(-1, p.shape[-1])
    a = np.zeros(flat_p.shape[0], dtype=bool)
    b = np.zeros(flat_p.shape[0], dtype=bool)
    if thr >= 1.0 or thr <= 0.0:
        return a.reshape(p.shape[:-1]), b.reshape(p.shape[:-1])
    for i, (row, keep) in enumerate(zip(flat_p, flat_m)):
        kept = np.sort(row[keep])[::-1]
        dropped = np.sort(row[~keep])[::-1]
        dk = kept.sum()
        dk1 = dk - kept[-1]
        a[i] = abs(dk - thr) < eps or abs(dk1 - thr) < eps
        if dropped.size:
            b[i] = (kept[-1] - dropped[0]) < eps * kept[-1]
    return a.reshape(p.shape[:-1]), b.reshape(p.shape[:-1])


# ---------------------------------------------------------------------------
# whole call
# ---------------------------------------------------------------------------
def nabla_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: Geometry,
                  thr: float, window: Sequence[int] = (0, 0, 0),
                  rows: Optional[Iterable[int]] = None):
    """One NABLA attention call for one head.

    q, k, v: [T, H, W, d] (any float dtype; computed in float64).
    Returns dict with o [T,H,W,d], mask, mask_adaptive, p, qbar, kbar, csr.
    """
    valid = valid_tokens(g)
    qb = flatten(np.asarray(q, dtype=np.float64), g)
    kb = flatten(np.asarray(k, dtype=np.float64), g)
    vb = flatten(np.asarray(v, dtype=np.float64), g)
    qbar = pool(qb, valid)
    kbar = pool(kb, valid)
    m, m_ad, p = nabla_mask(qbar, kbar, thr, g, window)
    ob = block_sparse_attention(qb, kb, vb, m, valid, rows=rows)
    return {
        "o": unflatten(ob, g), "o_blocked": ob, "mask": m, "mask_adaptive": m_ad,
        "p": p, "qbar": qbar, "kbar": kbar, "csr": to_csr(m), "valid": valid,
    }

"""Pins that tie the NABLA oracle to facts outside itself.

Each ``pin_*`` takes the oracle module and raises AssertionError when the
oracle disagrees with a value the pages fix, a closed form, an independent
library routine, or brute force.  ``test_oracle_pins.py`` runs them on the
real oracle; ``test_oracle_mutations.py`` runs them on deliberately broken
copies to show that each plausible mistake is caught by at least one pin.
"""
from __future__ import annotations

import itertools
import math
import os

import numpy as np
import scipy.ndimage
import scipy.sparse
import scipy.special
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------- flatten
def pin_flatten_hand_positions(O):
    """Positions worked out by hand from the page's description of the reorder."""
    with open(os.path.join(GOLDEN, "flatten_positions.txt")) as f:
        rows = [ln.split("#")[0].split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(rows) >= 10
    for r in rows:
        T, H, W, P, t, h, w, want = map(int, r)
        got = int(O.flatten_positions(O.Geometry(T, H, W, P))[t, h, w])
        assert got == want, f"flatten position of {(t, h, w)} in {(T, H, W, P)}: {got} != {want}"


def pin_flatten_patch_structure(O):
    """Every block holds exactly one P x P patch of one frame, in row-major order;
    the map is injective; pad slots are exactly the out-of-range patch cells."""
    for (T, H, W, P) in [(2, 16, 24, 8), (3, 13, 10, 8), (1, 8, 8, 8), (2, 9, 7, 4)]:
        g = O.Geometry(T, H, W, P)
        pos = O.flatten_positions(g)
        assert len(set(pos.ravel().tolist())) == pos.size
        gh, gw = -(-H // P), -(-W // P)
        nb = T * gh * gw
        assert g.nb == nb and g.N == P * P
        inv = {int(pos[t, h, w]): (t, h, w) for t in range(T) for h in range(H) for w in range(W)}
        blk = 0
        for t in range(T):
            for bh in range(gh):
                for bw in range(gw):
                    for i in range(P):
                        for j in range(P):
                            slot = blk * P * P + i * P + j
                            hh, ww = bh * P + i, bw * P + j
                            if hh < H and ww < W:
                                assert inv.get(slot) == (t, hh, ww), (slot, inv.get(slot))
                            else:
                                assert slot not in inv
                    blk += 1
        valid = O.valid_tokens(g)
        assert valid.shape == (nb, P * P) and valid.sum() == T * H * W


def pin_flatten_roundtrip(O):
    g = O.Geometry(3, 13, 19, 8)
    x = _rng(1).standard_normal((2, 3, 13, 19, 5))
    xb = O.flatten(x, g)
    assert xb.shape == (2, g.nb, 64, 5)
    valid = O.valid_tokens(g)
    assert np.all(xb[:, ~valid] == 0)
    assert np.array_equal(O.unflatten(xb, g), x)
    # multiset of values is preserved
    assert np.array_equal(np.sort(xb[:, valid].ravel()), np.sort(x.ravel()))


# ------------------------------------------------------------------------ pool
def pin_pool_closed_forms(O):
    # constant input -> the constant, also in partially padded blocks
    g = O.Geometry(2, 11, 13, 8)
    x = np.full((2, 11, 13, 3), 1.75)
    qb = O.pool(O.flatten(x, g), O.valid_tokens(g))
    assert np.all(qb == 1.75)
    # ramp along h with H=12 padded to 16: block rows 0..7 -> 3.5, valid rows 8..11 -> 9.5
    g = O.Geometry(1, 12, 8, 8)
    x = np.broadcast_to(np.arange(12.0)[None, :, None, None], (1, 12, 8, 2)).copy()
    qb = O.pool(O.flatten(x, g), O.valid_tokens(g))
    assert np.allclose(qb[:, 0], [3.5, 9.5], rtol=0, atol=1e-15), qb
    # ramp along w with W=13 padded to 16: 0..7 -> 3.5, valid 8..12 -> 10
    g = O.Geometry(1, 8, 13, 8)
    x = np.broadcast_to(np.arange(13.0)[None, None, :, None], (1, 8, 13, 2)).copy()
    qb = O.pool(O.flatten(x, g), O.valid_tokens(g))
    assert np.allclose(qb[:, 0], [3.5, 10.0], rtol=0, atol=1e-15), qb
    # one distinct channel per block: mean equals that block's patch mean
    g = O.Geometry(1, 16, 16, 8)
    x = _rng(2).standard_normal((1, 16, 16, 4))
    qb = O.pool(O.flatten(x, g), O.valid_tokens(g))
    want = np.stack([x[0, 0:8, 0:8].mean((0, 1)), x[0, 0:8, 8:16].mean((0, 1)),
                     x[0, 8:16, 0:8].mean((0, 1)), x[0, 8:16, 8:16].mean((0, 1))])
    assert np.allclose(qb, want, rtol=0, atol=1e-14)


# -------------------------------------------------------------- reduced map
def pin_reduced_map(O):
    rng = _rng(3)
    # two blocks: p0 = logistic(s0 - s1) with s = q.k / sqrt(d)  (closed form)
    d = 16
    for a in [0.5, 1.0, 2.0]:
        q = np.zeros((1, d)); q[0, 3] = a
        k = np.zeros((2, d)); k[0, 3] = a
        p = O.reduced_map(q, k)
        want = 1.0 / (1.0 + math.exp(-(a * a) / math.sqrt(d)))
        assert abs(p[0, 0] - want) < 1e-14 and abs(p[0, 1] - (1 - want)) < 1e-14
    # asymmetric case: row i is the distribution of query block i over key blocks
    q = np.zeros((2, d)); q[0, 0] = 4.0
    k = np.zeros((3, d)); k[2, 0] = 4.0
    p = O.reduced_map(q, k)
    e = math.exp(16.0 / 4.0)
    assert np.allclose(p[0], [1 / (2 + e), 1 / (2 + e), e / (2 + e)], atol=1e-14)
    assert np.allclose(p[1], [1 / 3] * 3, atol=1e-15)
    # random: equals scipy's softmax of the score matrix; rows sum to 1
    qb = rng.standard_normal((3, 20, 32)) * 3
    kb = rng.standard_normal((3, 20, 32)) * 3
    p = O.reduced_map(qb, kb)
    s = np.einsum("hid,hjd->hij", qb, kb) / math.sqrt(32)
    assert np.allclose(p, scipy.special.softmax(s, axis=-1), rtol=1e-12, atol=1e-15)
    assert np.allclose(p.sum(-1), 1.0, atol=1e-13)


# ------------------------------------------------------------------- CDF cut
HAND_CDF = [
    # (p, thr, kept indices)   worked by hand: sort descending, keep until mass >= thr
    ([0.125, 0.5, 0.125, 0.25], 0.8, {1, 3, 0}),  # 0.5, 0.75, 0.875; tie -> lower index
    ([0.125, 0.5, 0.125, 0.25], 0.75, {1, 3}),    # 0.75 reaches 0.75 exactly
    ([0.125, 0.5, 0.125, 0.25], 0.5, {1}),        # 0.5 reaches 0.5
    ([0.125, 0.5, 0.125, 0.25], 0.3, {1}),
    ([0.5, 0.25, 0.25], 0.75, {0, 1}),          # tie at the cut: lower index kept
    ([0.25, 0.25, 0.25, 0.25], 0.5, {0, 1}),    # all tied: lowest indices
    ([0.25, 0.25, 0.25, 0.25], 0.51, {0, 1, 2}),
    ([0.7, 0.2, 0.1], 1.0, {0, 1, 2}),          # thr = 1: everything
    ([0.75, 0.0, 0.25], 1.0, {0, 1, 2}),        # thr = 1 keeps even zero-probability blocks
    ([0.0625] * 16, 0.125, {0, 1}),
]


def pin_cdf_hand_cases(O):
    for p, thr, want in HAND_CDF:
        got = set(np.flatnonzero(O.cdf_keep_row(np.array(p), thr)).tolist())
        assert got == want, (p, thr, got, want)


def pin_cdf_brute_force(O):
    """Kept set = a minimum-cardinality subset with mass >= thr, and of maximum
    mass among subsets of that size (checked over all 2^n subsets)."""
    rng = _rng(4)
    n = 16
    bits = ((np.arange(1 << n)[:, None] >> np.arange(n)[None, :]) & 1).astype(np.float64)
    card = bits.sum(1)
    for trial in range(40):
        p = rng.dirichlet(np.full(n, rng.choice([0.2, 1.0, 5.0])))
        thr = float(rng.choice([0.3, 0.5, 0.7, 0.8, 0.9, 0.95]))
        keep = O.cdf_keep_row(p, thr)
        mass = bits @ p
        ok = mass >= thr
        kmin = card[ok].min()
        assert keep.sum() == kmin, (trial, keep.sum(), kmin)
        best = mass[ok & (card == kmin)].max()
        assert abs(p[keep].sum() - best) < 1e-12
        assert p[keep].sum() >= thr
        if keep.sum() < n:
            assert p[keep].min() >= p[~keep].max()


def pin_cdf_invariants(O):
    rng = _rng(5)
    p = scipy.special.softmax(rng.standard_normal((30, 50)) * 3, axis=-1)
    prev = None
    for thr in [0.2, 0.5, 0.7, 0.9, 0.99, 1.0]:
        m = O.cdf_keep(p, thr)
        assert np.all(m.sum(1) >= 1)
        mass = (p * m).sum(1)
        assert np.all(mass >= thr - 1e-12)
        # minimality: dropping the least kept block falls below thr
        least = np.where(m, p, np.inf).min(1)
        assert np.all(mass - least < thr) or thr >= 1.0
        if prev is not None:
            assert np.all(prev <= m)          # nested in thr (smaller thr -> sparser)
        prev = m
    assert np.all(O.cdf_keep(p, 1.0))


# ------------------------------------------------------------------------ STA
def pin_sta(O):
    for grid, window in [((4, 3, 5), (3, 3, 3)), ((3, 6, 10), (3, 3, 3)), ((5, 2, 4), (1, 3, 5)),
                         ((2, 4, 4), (3, 1, 1))]:
        g = O.Geometry(grid[0], grid[1] * 8, grid[2] * 8, 8)
        m = O.sta_mask(g, window)
        nb = g.nb
        assert m.shape == (nb, nb)
        for a in range(nb):
            one = np.zeros(nb, dtype=bool); one[a] = True
            want = scipy.ndimage.binary_dilation(one.reshape(grid),
                                                 structure=np.ones(window, dtype=bool))
            assert np.array_equal(m[a].reshape(grid), want), (grid, window, a)
    g = O.Geometry(5, 40, 40, 8)
    m = O.sta_mask(g, (3, 3, 3))
    c = m.sum(1).reshape(5, 5, 5)
    assert c[2, 2, 2] == 27 and c[0, 0, 0] == 8 and c[0, 2, 2] == 18 and c[0, 0, 2] == 12
    assert not O.sta_mask(g, (0, 0, 0)).any()


def pin_pure_sta(O):
    """thr = 0 turns the adaptive part off: the mask is exactly the STA window
    (the static baseline the pages compare against)."""
    rng = _rng(15)
    g = O.Geometry(3, 16, 24, 8)
    qbar, kbar = rng.standard_normal((2, g.nb, 16))
    for win in [(3, 3, 3), (1, 3, 5)]:
        m, m_ad, _ = O.nabla_mask(qbar, kbar, 0.0, g, win)
        assert not m_ad.any()
        assert np.array_equal(m, O.sta_mask(g, win))


def pin_union(O):
    rng = _rng(6)
    g = O.Geometry(3, 24, 32, 8)
    qb = rng.standard_normal((g.nb, 16)) * 3
    kb = rng.standard_normal((g.nb, 16)) * 3
    m, m_ad, p = O.nabla_mask(qb, kb, 0.6, g, (3, 3, 3))
    sta = O.sta_mask(g, (3, 3, 3))
    assert np.array_equal(m, m_ad | sta)
    assert np.array_equal(m_ad, O.cdf_keep(O.reduced_map(qb, kb), 0.6))


# ------------------------------------------------------------------------ CSR
def pin_csr(O):
    rng = _rng(7)
    m = rng.random((37, 37)) < 0.3
    m[5] = False
    rp, ci = O.to_csr(m)
    ref = scipy.sparse.csr_matrix(m)
    assert np.array_equal(rp, ref.indptr) and np.array_equal(ci, ref.indices)


# ------------------------------------------------------------------ attention
def _sdpa(q, k, v, allow):
    """torch's scaled_dot_product_attention in float64 on the CPU."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    return torch.nn.functional.scaled_dot_product_attention(
        t(q)[None], t(k)[None], t(v)[None], attn_mask=t(allow)[None]).numpy()[0]


def pin_attention_dense_special_case(O):
    """thr = 1 without STA keeps every block: equals dense softmax attention."""
    rng = _rng(8)
    g = O.Geometry(2, 16, 16, 8)
    q, k, v = (rng.standard_normal((2, 16, 16, 32)) for _ in range(3))
    r = O.nabla_forward(q, k, v, g, 1.0)
    assert r["mask"].all()
    ref = _sdpa(q.reshape(-1, 32), k.reshape(-1, 32), v.reshape(-1, 32),
                np.ones((512, 512), dtype=bool)).reshape(q.shape)
    assert np.abs(r["o"] - ref).max() < 1e-12


def pin_attention_masked(O):
    """Sparse output = dense attention with non-kept blocks (and pad keys) at -inf."""
    rng = _rng(9)
    for (T, H, W, thr, win) in [(2, 16, 24, 0.6, (0, 0, 0)), (2, 13, 19, 0.5, (1, 3, 3)),
                                (3, 16, 16, 0.3, (0, 0, 0))]:
        g = O.Geometry(T, H, W, 8)
        q = rng.standard_normal((T, H, W, 16)) * 2
        k = rng.standard_normal((T, H, W, 16)) * 2
        v = rng.standard_normal((T, H, W, 16))
        r = O.nabla_forward(q, k, v, g, thr, win)
        m, valid = r["mask"], r["valid"]
        assert not m.all()
        allow = np.kron(m, np.ones((64, 64), dtype=bool)) & valid.reshape(1, -1)
        qb, kb, vb = (O.flatten(x, g).reshape(-1, 16) for x in (q, k, v))
        vq = valid.reshape(-1)
        ref = _sdpa(qb[vq], kb, vb, allow[vq])
        got = r["o_blocked"].reshape(-1, 16)[vq]
        assert np.abs(got - ref).max() < 1e-12
        assert np.all(r["o_blocked"].reshape(-1, 16)[~vq] == 0)


def pin_attention_special_values(O):
    rng = _rng(10)
    g = O.Geometry(2, 16, 16, 8)
    q, k = rng.standard_normal((2, 2, 16, 16, 8))
    v = np.full((2, 16, 16, 8), -0.625)
    r = O.nabla_forward(q, k, v, g, 0.5)
    assert np.abs(r["o"] + 0.625).max() < 1e-13          # V constant -> O constant
    # one kept block per row: plain 64-key softmax attention within that block
    valid = O.valid_tokens(g)
    qb, kb, vb = (O.flatten(x, g) for x in (q, k, rng.standard_normal((2, 16, 16, 8))))
    m = np.zeros((g.nb, g.nb), dtype=bool)
    m[np.arange(g.nb), (np.arange(g.nb) * 3) % g.nb] = True
    ob = O.block_sparse_attention(qb, kb, vb, m, valid)
    for a in range(g.nb):
        b = (a * 3) % g.nb
        s = qb[a] @ kb[b].T / math.sqrt(8)
        want = scipy.special.softmax(s, axis=1) @ vb[b]
        assert np.abs(ob[a] - want).max() < 1e-13


# ------------------------------------------------------------------ gradients
def _bwd_case(O, rng, T, H, W, d, density):
    """Blocked random inputs (pad slots random too) and a random mask with the
    diagonal kept, so every valid query sees at least one valid key."""
    g = O.Geometry(T, H, W, 8)
    valid = O.valid_tokens(g)
    qb, kb, vb, dob = (rng.standard_normal((g.nb, 64, d)) for _ in range(4))
    m = rng.random((g.nb, g.nb)) < density
    m[np.arange(g.nb), np.arange(g.nb)] = True
    return g, valid, qb, kb, vb, dob, m


def pin_backward_finite_differences(O):
    """Analytic gradients = central differences of L = sum(do * o), o the
    oracle's attention (itself pinned above); pad slots get zero gradient."""
    rng = _rng(11)
    g, valid, qb, kb, vb, dob, m = _bwd_case(O, rng, 1, 13, 16, 4, 0.5)
    assert not valid.all() and not m.all()
    dq, dk, dv, _ = O.block_sparse_attention_backward(qb, kb, vb, m, valid, dob)
    grads = {"q": dq, "k": dk, "v": dv}

    def loss(x):
        return float((dob * O.block_sparse_attention(x["q"], x["k"], x["v"], m, valid)).sum())
    h = 1e-6
    vb_idx = np.argwhere(valid)
    pad_idx = np.argwhere(~valid)
    for name in ("q", "k", "v"):
        picks = [tuple(vb_idx[i]) for i in rng.choice(len(vb_idx), 12, replace=False)]
        picks += [tuple(pad_idx[i]) for i in rng.choice(len(pad_idx), 3, replace=False)]
        for (b, t) in picks:
            c = int(rng.integers(qb.shape[-1]))
            x = {"q": qb.copy(), "k": kb.copy(), "v": vb.copy()}
            x[name][b, t, c] += h
            lp = loss(x)
            x[name][b, t, c] -= 2 * h
            lm = loss(x)
            num = (lp - lm) / (2 * h)
            ana = grads[name][b, t, c]
            assert abs(num - ana) <= 1e-7 + 1e-6 * abs(ana), (name, b, t, c, num, ana)
            if not valid[b, t]:
                assert ana == 0.0


def pin_backward_autograd(O):
    """Gradients and log-sum-exp = torch autograd of float64
    scaled_dot_product_attention with the kept blocks (and valid keys) as the
    attention mask; the dense case is the all-kept mask."""
    rng = _rng(12)
    for (T, H, W, d, density) in [(2, 13, 19, 16, 0.4), (2, 16, 16, 8, 1.0)]:
        g, valid, qb, kb, vb, dob, m = _bwd_case(O, rng, T, H, W, d, density)
        dq, dk, dv, lse = O.block_sparse_attention_backward(qb, kb, vb, m, valid, dob)
        vq = valid.reshape(-1)
        allow = (np.kron(m, np.ones((64, 64), dtype=bool)) & vq[None, :])[vq]
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a))  # noqa: E731
        q = t(qb.reshape(-1, d)[vq]).requires_grad_()
        k = t(kb.reshape(-1, d)).requires_grad_()
        v = t(vb.reshape(-1, d)).requires_grad_()
        o = torch.nn.functional.scaled_dot_product_attention(
            q[None], k[None], v[None], attn_mask=t(allow)[None])[0]
        (o * t(dob.reshape(-1, d)[vq])).sum().backward()
        assert np.abs(dq.reshape(-1, d)[vq] - q.grad.numpy()).max() < 1e-10
        assert np.abs(dk.reshape(-1, d) - k.grad.numpy()).max() < 1e-10
        assert np.abs(dv.reshape(-1, d) - v.grad.numpy()).max() < 1e-10
        assert np.all(dq.reshape(-1, d)[~vq] == 0)
        s = (qb.reshape(-1, d)[vq] @ kb.reshape(-1, d).T) / math.sqrt(d)
        want = scipy.special.logsumexp(np.where(allow, s, -np.inf), axis=1)
        assert np.abs(lse.reshape(-1)[vq] - want).max() < 1e-12
        assert np.all(np.isneginf(lse.reshape(-1)[~vq]))


def pin_backward_rows_subset(O):
    """Restricting to the query blocks that keep key block c reproduces c's
    full dk, dv and those rows' dq (the sums are the same terms)."""
    rng = _rng(14)
    g, valid, qb, kb, vb, dob, m = _bwd_case(O, rng, 2, 16, 16, 8, 0.35)
    dq, dk, dv, lse = O.block_sparse_attention_backward(qb, kb, vb, m, valid, dob)
    c = 3
    rows = np.flatnonzero(m[:, c])
    sq, sk, sv, sl = O.block_sparse_attention_backward(qb, kb, vb, m, valid, dob, rows=rows)
    assert np.abs(sk[c] - dk[c]).max() < 1e-12 and np.abs(sv[c] - dv[c]).max() < 1e-12
    assert np.abs(sq[rows] - dq[rows]).max() < 1e-12
    assert np.array_equal(sl[rows], lse[rows])


def pin_backward_invariants(O):
    """Rows of p sum to 1, so the dv rows add up to the do rows; rows of ds sum
    to 0, so the dk rows add up to 0 (per head)."""
    rng = _rng(13)
    g, valid, qb, kb, vb, dob, m = _bwd_case(O, rng, 2, 16, 24, 8, 0.3)
    dq, dk, dv, _ = O.block_sparse_attention_backward(qb, kb, vb, m, valid, dob)
    assert np.abs(dv.sum((0, 1)) - dob[valid].sum(0)).max() < 1e-10
    assert np.abs(dk.sum((0, 1))).max() < 1e-10
    assert np.abs(dq).max() > 1e-3 and np.abs(dk).max() > 1e-3


# ----------------------------------------------------------------- band rows
def pin_band_rows(O):
    p = np.array([[0.4, 0.2 + 3e-6, 0.15, 0.15, 0.1 - 3e-6],  # D_2 = thr + 3e-6: class a
                  [0.4, 0.3, 0.2, 0.1, 0.0],                   # D_1 = .4, D_2 = .7: clear
                  [0.45, 0.2, 0.2 - 1e-7, 0.15 + 1e-7, 0.0]])  # near tie at the cut: b
    m = O.cdf_keep(p, 0.6)
    assert m.sum(1).tolist() == [2, 2, 2]
    a, b = O.band_rows(p, m, 0.6)
    assert a.tolist() == [True, False, False]
    assert b.tolist() == [False, False, True]


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]

"""The oracle on the seeded workloads (CPU): the Tiny config end to end, and the
mask invariants on Small."""
import numpy as np
import torch

import oracle as O
import synth


def _geom(cfg):
    return O.Geometry(cfg.T, cfg.H, cfg.W, cfg.P)


def test_tiny_brute_force_and_dense_masked():
    cfg = synth.config("tiny")
    g = _geom(cfg)
    assert g.nb == 16
    q, k, v = synth.make_qkv(cfg)
    n = g.nb
    bits = ((np.arange(1 << n)[:, None] >> np.arange(n)[None, :]) & 1).astype(np.float64)
    card = bits.sum(1)
    for h in range(cfg.heads):
        r = O.nabla_forward(q[0, h].numpy(), k[0, h].numpy(), v[0, h].numpy(), g, cfg.thr)
        p, m = r["p"], r["mask"]
        for a in range(n):
            mass = bits @ p[a]
            ok = mass >= cfg.thr
            kmin = card[ok].min()
            assert m[a].sum() == kmin
            assert abs(p[a][m[a]].sum() - mass[ok & (card == kmin)].max()) < 1e-12
        # sparse output == dense attention with non-kept blocks at -inf (torch SDPA, float64)
        allow = torch.from_numpy(np.kron(m, np.ones((64, 64), dtype=bool)))
        qb, kb, vb = (torch.from_numpy(O.flatten(x[0, h].double().numpy(), g).reshape(-1, 64))
                      for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(
            qb[None], kb[None], vb[None], attn_mask=allow[None])[0].numpy()
        assert np.abs(r["o_blocked"].reshape(-1, 64) - ref).max() < 1e-12


def test_small_mask_invariants():
    cfg = synth.config("small", heads=2)
    g = _geom(cfg)
    q, k, _ = synth.make_qkv(cfg)
    valid = O.valid_tokens(g)
    for h in range(cfg.heads):
        qbar = O.pool(O.flatten(q[0, h].double().numpy(), g), valid)
        kbar = O.pool(O.flatten(k[0, h].double().numpy(), g), valid)
        m, m_ad, p = O.nabla_mask(qbar, kbar, cfg.thr, g, cfg.sta)
        mass = (p * m_ad).sum(1)
        assert np.all(mass >= cfg.thr) and np.all(m_ad.sum(1) >= 1)
        least = np.where(m_ad, p, np.inf).min(1)
        assert np.all(mass - least < cfg.thr)
        sparsity = 1 - m.mean()
        assert 0.3 < sparsity < 0.95
        m2 = O.cdf_keep(p, 0.5)
        assert np.all(m2 <= m_ad)

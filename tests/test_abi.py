"""C ABI contract on the CPU: the library loads, exports every call that
include/nabla.h declares, and rejects bad arguments with the documented status
before launching anything (no GPU is touched by these calls)."""
import ctypes
import os
import re
import subprocess

import pytest

from block_sparse_attention_flatten_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nabla.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|const char\s*\*)\s+(nabla_\w+)\s*\(", text, re.M)))


def test_header_declares_the_expected_calls():
    names = declared_functions()
    for want in ["nabla_flatten", "nabla_unflatten", "nabla_pool", "nabla_mask", "nabla_compact",
                 "nabla_attn_fwd", "nabla_forward", "nabla_forward_workspace_size"]:
        assert want in names
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(nabla_\w+)", out))
    for name in declared_functions():
        assert name in exported, f"{name} not exported"
        assert getattr(lib, name) is not None
    assert lib.nabla_abi_version() == 5


def G(**kw):
    base = dict(batch=1, heads=2, T=4, H=16, W=16, P=8, head_dim=64, dtype=1, layout=0,
                out_dtype=1)
    base.update(kw)
    return _lib.nabla_geom(*[base[f] for f, _ in _lib.nabla_geom._fields_])


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every case below fails validation


@pytest.mark.parametrize("geom,status", [
    (dict(batch=-1), -2), (dict(heads=-3), -2), (dict(T=0), -2), (dict(H=0), -2), (dict(W=-1), -2),
    (dict(P=4), -5), (dict(head_dim=96), -4), (dict(dtype=7), -3), (dict(layout=5), -9),
    (dict(out_dtype=2), -3), (dict(dtype=0, out_dtype=1), -3),
    (dict(T=100, H=64, W=64), -12), (dict(batch=300, heads=300), -2),
])
def test_geometry_validation(geom, status):
    lib = _lib.load()
    g = G(**geom)
    st = lib.nabla_pool(ctypes.byref(g), FAKE, FAKE, FAKE, FAKE, None)
    assert st == status, (geom, st)
    assert lib.nabla_status_string(st).decode() not in ("", "unknown status")


def test_argument_validation():
    lib = _lib.load()
    g = G()
    sta = (ctypes.c_int32 * 3)
    assert lib.nabla_pool(None, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert lib.nabla_pool(ctypes.byref(g), None, FAKE, FAKE, FAKE, None) == -1
    for bad in [0.0, -0.1, 1.5, float("nan"), float("inf")]:
        assert lib.nabla_mask(ctypes.byref(g), FAKE, FAKE, bad, None, FAKE, FAKE, None, None) == -6
    # thr = 0 (pure STA) needs a window; with one, validation passes on to the pointers
    assert lib.nabla_mask(ctypes.byref(g), FAKE, FAKE, 0.0, sta(0, 0, 0), FAKE, FAKE, None,
                          None) == -6
    assert lib.nabla_mask(ctypes.byref(g), None, FAKE, 0.0, sta(3, 3, 3), FAKE, FAKE, None,
                          None) == -1
    for bad in [(2, 3, 3), (3, 0, 3), (-1, 3, 3), (3, 3, 4)]:
        assert lib.nabla_mask(ctypes.byref(g), FAKE, FAKE, 0.5, sta(*bad), FAKE, FAKE, None,
                              None) == -7
    assert lib.nabla_mask(ctypes.byref(g), None, FAKE, 0.5, sta(3, 3, 3), FAKE, FAKE, None,
                          None) == -1
    for bad in [0.0, -1.0, float("nan")]:
        assert lib.nabla_attn_fwd(ctypes.byref(g), FAKE, FAKE, FAKE, FAKE, FAKE, bad, FAKE,
                                  None) == -11
    assert lib.nabla_attn_fwd(ctypes.byref(g), FAKE, FAKE, FAKE, FAKE, None, 0.1, FAKE, None) == -1
    assert lib.nabla_compact(ctypes.byref(g), FAKE, FAKE, FAKE, None, None) == -1
    assert lib.nabla_transpose_v(ctypes.byref(g), FAKE, None, None) == -1
    assert lib.nabla_transpose_v(ctypes.byref(G(dtype=0, out_dtype=0)), FAKE, FAKE, None) == -3
    assert lib.nabla_attn_fwd_vt(ctypes.byref(G(dtype=0, out_dtype=0)), FAKE, FAKE, FAKE, FAKE,
                                 FAKE, 0.1, FAKE, None) == -3
    assert lib.nabla_attn_fwd_vt(ctypes.byref(g), FAKE, FAKE, None, FAKE, FAKE, 0.1, FAKE,
                                 None) == -1
    assert lib.nabla_dense_attn_fwd(ctypes.byref(G(dtype=0, out_dtype=0)), FAKE, FAKE, FAKE, 0.1,
                                    FAKE, None, None) == -3
    assert lib.nabla_dense_attn_fwd(ctypes.byref(g), FAKE, FAKE, None, 0.1, FAKE, None,
                                    None) == -1
    assert lib.nabla_dense_attn_fwd(ctypes.byref(g), FAKE, FAKE, FAKE, 0.0, FAKE, None,
                                    None) == -11
    assert lib.nabla_qkv_split(ctypes.byref(g), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -9
    gbl = G(layout=1)
    assert lib.nabla_qkv_split(ctypes.byref(G(layout=1, dtype=0, out_dtype=0)), FAKE, FAKE, FAKE,
                               FAKE, FAKE, FAKE, None) == -3
    assert lib.nabla_qkv_split(ctypes.byref(gbl), FAKE, FAKE, FAKE, None, FAKE, FAKE, None) == -1
    assert lib.nabla_flatten(ctypes.byref(g), None, FAKE, None) == -1
    assert lib.nabla_unflatten(ctypes.byref(g), FAKE, None, None) == -1
    size = ctypes.c_size_t(0)
    assert lib.nabla_forward_workspace_size(ctypes.byref(g), ctypes.byref(size), None) == 0
    assert lib.nabla_forward(ctypes.byref(g), FAKE, FAKE, FAKE, 0.5, None, 0.125, FAKE, FAKE,
                             size.value - 1, None) == -8
    assert lib.nabla_forward(ctypes.byref(g), FAKE, FAKE, FAKE, 0.5, None, 0.125, FAKE, None,
                             size.value, None) == -1
    assert lib.nabla_forward(ctypes.byref(g), FAKE, FAKE, FAKE, 2.0, None, 0.125, FAKE, FAKE,
                             size.value, None) == -6
    assert lib.nabla_forward_noalloc(ctypes.byref(g), FAKE, FAKE, None, 0.5, None, 0.125, FAKE,
                                     None) == -1
    assert lib.nabla_forward_noalloc(ctypes.byref(g), FAKE, FAKE, FAKE, 2.0, None, 0.125, FAKE,
                                     None) == -6
    assert lib.nabla_forward_noalloc(ctypes.byref(g), FAKE, FAKE, FAKE, 0.5, None, -1.0, FAKE,
                                     None) == -11
    assert lib.nabla_forward_noalloc(ctypes.byref(G(head_dim=96)), FAKE, FAKE, FAKE, 0.5, None,
                                     0.125, FAKE, None) == -4


def test_empty_calls_launch_nothing():
    lib = _lib.load()
    for geom in [dict(batch=0), dict(heads=0)]:
        g = G(**geom)
        assert lib.nabla_pool(ctypes.byref(g), None, None, None, None, None) == 0
        assert lib.nabla_attn_fwd(ctypes.byref(g), None, None, None, None, None, 0.1, None,
                                  None) == 0
        assert lib.nabla_mask(ctypes.byref(g), None, None, 0.5, None, None, None, None, None) == 0
        assert lib.nabla_forward(ctypes.byref(g), None, None, None, 0.5, None, 0.1, None, None, 0,
                                 None) == 0
        assert lib.nabla_forward_noalloc(ctypes.byref(g), None, None, None, 0.5, None, 0.1, None,
                                         None) == 0


def test_workspace_layout_and_block_count():
    lib = _lib.load()
    # 720p Wan shape: 21 x 45 x 80 -> 21 x 6 x 10 blocks
    g = G(batch=1, heads=40, T=21, H=45, W=80, head_dim=128)
    nb = ctypes.c_int64(0)
    assert lib.nabla_num_blocks(ctypes.byref(g), ctypes.byref(nb)) == 0
    assert nb.value == 1260
    size = ctypes.c_size_t(0)
    offs = (ctypes.c_size_t * 7)()
    assert lib.nabla_forward_workspace_size(ctypes.byref(g), ctypes.byref(size), offs) == 0
    o = list(offs)
    assert o[0] == 0 and all(x % 256 == 0 for x in o) and o == sorted(o)
    bh, n, d = 40, 1260, 128
    assert o[1] >= bh * n * d * 4 and o[2] - o[1] >= bh * n * d * 4
    assert o[6] - o[5] >= bh * n * n * 4
    assert size.value - o[6] >= bh * n * 64 * d * 2      # V^T for bf16 inputs
    # Long: 41 x 45 x 80 -> 2460 blocks; 480p: 21 x 30 x 52 -> 21 x 4 x 7
    assert lib.nabla_num_blocks(ctypes.byref(G(T=41, H=45, W=80)), ctypes.byref(nb)) == 0
    assert nb.value == 2460
    assert lib.nabla_num_blocks(ctypes.byref(G(T=21, H=30, W=52)), ctypes.byref(nb)) == 0
    assert nb.value == 588


def test_status_strings():
    lib = _lib.load()
    for code in _lib.STATUS:
        assert lib.nabla_status_string(code).decode() != "unknown status"
    assert lib.nabla_status_string(12345).decode() == "unknown status"


def test_probe_library_exports():
    """The benchmark's rate probe (bench_peaks.hip) is built beside bench.py,
    outside the library, and exports its three calls; only bench.py loads it."""
    path = os.path.join(ROOT, "bench_peaks.so")
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT\s+(nabla_probe_\w+)", out))
    assert exported == {"nabla_probe_mfma_bf16", "nabla_probe_mfma_bf16_flops",
                        "nabla_probe_copy"}
    lib = ctypes.CDLL(path)
    lib.nabla_probe_mfma_bf16_flops.restype = ctypes.c_double
    lib.nabla_probe_mfma_bf16_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    assert lib.nabla_probe_mfma_bf16_flops(2, 3) == 2 * 4 * 3 * 4 * 2 * 32 * 32 * 16
    # argument checks fail before any launch (no GPU touched)
    lib.nabla_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                     ctypes.c_int, ctypes.c_void_p]
    assert lib.nabla_probe_copy(None, FAKE, 16, 1, None) == -1
    assert lib.nabla_probe_copy(FAKE, FAKE, 15, 1, None) == -1
    lib.nabla_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                          ctypes.c_void_p]
    assert lib.nabla_probe_mfma_bf16(0, 1, FAKE, None) == -1


def _split3(x):
    """Three-part bf16 encoding of float32 values, as include/nabla.h defines
    it: h = bf16(x), m = bf16(x - h), l = bf16(x - h - m), round to nearest
    even, differences in float32."""
    import torch
    h = x.to(torch.bfloat16)
    r = x - h.to(torch.float32)
    m = r.to(torch.bfloat16)
    lo = (r - m.to(torch.float32)).to(torch.bfloat16)
    return h, m, lo


def test_kbar_split_is_exact():
    """Every float32 mean survives its three-part encoding: h + m + l == x,
    and (h + m) + l in float32 gives x back (normal magnitudes, both signs)."""
    import torch
    g = torch.Generator().manual_seed(7)
    mant = torch.rand(200000, generator=g, dtype=torch.float64) + 1.0
    expo = torch.randint(-60, 60, (200000,), generator=g).to(torch.float64)
    sign = torch.where(torch.rand(200000, generator=g) < 0.5, -1.0, 1.0).to(torch.float64)
    x = (sign * mant * torch.pow(2.0, expo)).to(torch.float32)
    h, m, lo = _split3(x)
    exact = h.to(torch.float64) + m.to(torch.float64) + lo.to(torch.float64)
    assert torch.equal(exact, x.to(torch.float64))
    back = (h.to(torch.float32) + m.to(torch.float32)) + lo.to(torch.float32)
    assert torch.equal(back.view(torch.int32), x.view(torch.int32))


def test_kbar_untile_follows_the_header_order():
    """kbar_untile inverts the split, tiled encoding documented in
    include/nabla.h: part p of block 16 j + i, channel c at bf16 offset
    (((j * (d / 32) + c / 32) * 3 + p) * 64 + ((c / 8) % 4) * 16 + i) * 8 + c % 8."""
    import torch
    from block_sparse_attention_flatten_amd.api import kbar_untile
    g = torch.Generator().manual_seed(3)
    for nb, d in ((37, 64), (48, 128)):
        nb16 = -(-nb // 16) * 16
        want = torch.randn(nb, d, generator=g, dtype=torch.float32) * 3.0
        h, m, lo = _split3(want)
        flat = torch.full((3 * nb16 * d,), float("nan"), dtype=torch.bfloat16)
        for row in range(nb):
            for c in range(d):
                base = (((row // 16) * (d // 32) + c // 32) * 3 * 64 + ((c // 8) % 4) * 16
                        + row % 16) * 8 + c % 8
                for p, part in enumerate((h, m, lo)):
                    flat[base + p * 64 * 8] = part[row, c]
        got = kbar_untile(flat.view(1, 1, nb16, 3 * d), nb)[0, 0]
        assert torch.equal(got.view(torch.int32), want.view(torch.int32))

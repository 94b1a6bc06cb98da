"""Host-side checks of the C ABI (no GPU work): exports, geometry, argument validation.

Pointer arguments here are fake addresses; every call is rejected on the host
before anything is enqueued, so nothing dereferences them.
"""
import ctypes
import os
import re

import pytest
import numpy as np
import torch

import oracle
import spatially_sparse_incremental_amd as ssi
from spatially_sparse_incremental_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sige.h")

EINVAL, EDTYPE, EALIGN, ENODEV, ERANGE = L.SIGE_EINVAL, L.SIGE_EDTYPE, L.SIGE_EALIGN, L.SIGE_ENODEV, L.SIGE_ERANGE
A = 0x7F0000000000  # fake, 256-byte aligned device addresses, far apart
B = A + (1 << 36)
C = A + (2 << 36)
D = A + (3 << 36)
E = A + (4 << 36)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libsige.so not built")
    return L.lib()


def _g(n=1, h=256, w=256, ci=128, co=128, k=3, s=1, p=1, b=6):
    return L.Geom(n, h, w, ci, co, k, s, p, b)


def _v(x):
    return ctypes.c_void_p(x)


def test_every_declared_function_is_exported(lib):
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(sige_\w+)\s*\(", text, re.M))
    assert declared == set(L.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


@pytest.mark.parametrize("geom", [(256, 256, 3, 1, 1, 6), (13, 17, 3, 2, 1, 3), (64, 64, 3, 1, 1, 8),
                                  (16, 16, 1, 1, 0, 2), (11, 14, 5, 1, 2, 3), (32, 64, 3, 1, 1, 4)])
def test_geometry_matches_oracle(lib, geom):
    h, w, k, s, p, b = geom
    d = ssi.sige_geom_derive(_g(2, h, w, 8, 8, k, s, p, b))
    assert (d.ho, d.wo, d.nby, d.nbx, d.ib) == oracle.geometry(h, w, k, s, p, b)
    assert d.cap == 2 * d.nby * d.nbx == ssi.sige_max_blocks(_g(2, h, w, 8, 8, k, s, p, b))


@pytest.mark.parametrize("bad", [dict(n=0), dict(k=0), dict(k=8), dict(s=0), dict(p=3), dict(b=0), dict(b=65),
                                 dict(h=1, p=0), dict(b=40, s=2)])
def test_bad_geometry_is_einval(lib, bad):
    kw = dict(n=1, h=64, w=64, ci=8, co=8, k=3, s=1, p=1, b=6)
    kw.update(bad)
    with pytest.raises(ssi.SigeError) as e:
        ssi.sige_geom_derive(_g(**kw))
    assert e.value.code == EINVAL
    assert ssi.sige_max_blocks.__name__  # message path exercised above


def test_diff_validation(lib):
    f = lib.sige_diff_mask
    s = _v(0)
    assert f(_v(A), _v(B), 7, 1, 4, 4, 8, ctypes.c_float(1e-6), _v(C), s) == EDTYPE
    assert f(None, _v(B), 1, 1, 4, 4, 8, ctypes.c_float(1e-6), _v(C), s) == EINVAL
    assert f(_v(A), _v(B), 1, 1, 4, 4, 8, ctypes.c_float(float("nan")), _v(C), s) == EINVAL
    assert f(_v(A), _v(B), 1, 1, 4, 4, 8, ctypes.c_float(-1.0), _v(C), s) == EINVAL
    assert f(_v(A), _v(B), 1, 1, 4, 4, 12, ctypes.c_float(1e-6), _v(C), s) == EALIGN  # 24-byte rows
    assert f(_v(A), _v(B), 0, 1, 4, 4, 6, ctypes.c_float(1e-6), _v(C), s) == EALIGN  # fp32 c % 4
    assert f(_v(A + 8), _v(B), 1, 1, 4, 4, 8, ctypes.c_float(1e-6), _v(C), s) == EALIGN
    assert f(_v(A), _v(B), 1, 1, 4, 4, 8, ctypes.c_float(1e-6), _v(C + 2), s) == EALIGN
    assert f(_v(A), _v(B), 1, 1, 4, 4, 8, ctypes.c_float(1e-6), _v(A + 64), s) == EINVAL  # mask inside a_orig
    assert f(_v(A), _v(B), 1, 1, 4, 4, 12, ctypes.c_float(1e-6), _v(C), s) == EALIGN
    assert b"multiple of 16" in lib.sige_last_error()
    assert f(None, None, 1, 0, 4, 4, 8, ctypes.c_float(1e-6), None, s) == 0  # empty: nothing to do
    assert lib.sige_last_error() == b""


def test_bitset_validation(lib):
    s = _v(0)
    f = lib.sige_diff_mask_bits
    assert f(_v(A), _v(B), 1, 1, 4, 48, 8, ctypes.c_float(1e-6), _v(C), _v(D), s) == EINVAL  # w % 32
    assert b"multiple of 32" in lib.sige_last_error()
    assert f(_v(A), _v(B), 1, 1, 4, 32, 8, ctypes.c_float(1e-6), None, None, s) == EINVAL  # no output
    assert f(_v(A), _v(B), 1, 1, 4, 32, 8, ctypes.c_float(1e-6), None, _v(D + 2), s) == EALIGN
    assert f(_v(A), _v(B), 1, 1, 4, 32, 8, ctypes.c_float(1e-6), None, _v(A + 64), s) == EINVAL  # bits in a_orig
    assert f(_v(A), _v(B), 1, 1, 4, 32, 8, ctypes.c_float(1e-6), _v(C), _v(C + 64), s) == EINVAL  # bits in mask
    assert f(_v(A), _v(B), 7, 1, 4, 32, 8, ctypes.c_float(1e-6), None, _v(D), s) == EDTYPE
    assert f(_v(A), _v(B), 1, 1, 4, 32, 8, ctypes.c_float(1e-6), None, _v(D), s) == ENODEV
    g = _g()
    r = lib.sige_reduce_bits
    assert r(None, 256, 256, ctypes.byref(g), 1, _v(B), _v(C), s) == EINVAL
    assert r(_v(A + 2), 256, 256, ctypes.byref(g), 1, _v(B), _v(C), s) == EALIGN
    odd = _g(h=16, w=40, b=4)
    assert r(_v(A), 16, 40, ctypes.byref(odd), 1, _v(B), _v(C), s) == EINVAL  # mask width % 32
    assert r(_v(A), 256, 256, ctypes.byref(g), 1, _v(A + 64), _v(C), s) == EINVAL  # idx inside the bits
    rc = lib.sige_reduce_bits_copy
    assert rc(_v(A), 256, 256, ctypes.byref(g), 1, _v(B), _v(C), 1, _v(D), None, s) == EINVAL
    assert r(_v(A), 256, 256, ctypes.byref(g), 1, _v(B), _v(C), s) == ENODEV


def test_reduce_validation(lib):
    f = lib.sige_reduce_mask
    s = _v(0)
    g = _g()
    assert f(None, 256, 256, ctypes.byref(g), 1, _v(B), _v(C), s) == EINVAL
    assert f(_v(A), 300, 256, ctypes.byref(g), 1, _v(B), _v(C), s) == EINVAL  # not an integer multiple
    assert f(_v(A), 128, 128, ctypes.byref(g), 1, _v(B), _v(C), s) == EINVAL  # coarser than the input
    assert f(_v(A), 256, 256, ctypes.byref(g), -1, _v(B), _v(C), s) == EINVAL
    assert f(_v(A), 256, 256, ctypes.byref(g), 17, _v(B), _v(C), s) == EINVAL
    assert f(_v(A), 256, 256, ctypes.byref(g), 1, _v(B + 2), _v(C), s) == EALIGN
    assert f(_v(A), 256, 256, ctypes.byref(g), 1, _v(A + 128), _v(C), s) == EINVAL  # idx inside mask
    wide = _g(h=16, w=8200, b=32)  # conv input wider than 8192
    assert f(_v(A), 16, 8200, ctypes.byref(wide), 1, _v(B), _v(C), s) == ERANGE
    grid = _g(h=516, w=516, b=4)  # 129 x 129 blocks > 16384
    assert f(_v(A), 516, 516, ctypes.byref(grid), 1, _v(B), _v(C), s) == ERANGE
    grid2 = _g(n=2, h=512, w=256, b=4)  # 2 x 128 x 64 = 16384: the limit itself is accepted up to the device
    assert f(_v(A), 512, 256, ctypes.byref(grid2), 1, _v(B), _v(C), s) in (0, ENODEV)


def test_conv_step_validation(lib):
    s = _v(0)
    g = _g()
    assert lib.sige_gather(_v(A), 3, ctypes.byref(g), _v(B), _v(C), _v(D), s) == EDTYPE
    assert lib.sige_gather(_v(A), 1, ctypes.byref(g), None, _v(C), _v(D), s) == EINVAL
    assert lib.sige_gather(_v(A + 4), 1, ctypes.byref(g), _v(B), _v(C), _v(D), s) == EALIGN
    assert lib.sige_conv_blocks(_v(A), _v(B), None, 1, ctypes.byref(g), _v(C), _v(A + 32), s) == EINVAL  # overlap
    assert lib.sige_conv_blocks(_v(A), _v(B), _v(E + 2), 1, ctypes.byref(g), _v(C), _v(D), s) == EALIGN
    odd = _g(ci=12)
    assert lib.sige_conv_blocks(_v(A), _v(B), None, 1, ctypes.byref(odd), _v(C), _v(D), s) == EALIGN
    wide = _g(ci=8192)  # 16 KiB channel rows
    assert lib.sige_conv_blocks(_v(A), _v(B), None, 1, ctypes.byref(wide), _v(C), _v(D), s) == ERANGE
    assert lib.sige_scatter(_v(A), _v(B), _v(C), ctypes.byref(g), 1, _v(D), _v(D), 1, s) == EINVAL  # out == cached
    assert lib.sige_scatter(_v(A), _v(B), _v(C), ctypes.byref(g), 1, None, _v(D), 1, s) == EINVAL
    assert lib.sige_sparse_conv_layer(_v(A), _v(B), None, _v(C), _v(D), _v(E), 1, ctypes.byref(g), _v(A + 64), 1,
                                      s) == EINVAL  # out overlaps a_edit
    assert lib.sige_sparse_conv_layer(_v(A), _v(B), None, None, _v(D), _v(E), 1, ctypes.byref(g), _v(C), 1,
                                      s) == EINVAL  # copy without a cache
    huge = _g(h=128, w=128, ci=64, co=64, k=1, p=0, b=64)  # two 64x64 windows cannot fit in LDS
    assert lib.sige_sparse_conv_layer(_v(A), _v(B), None, _v(C), _v(D), _v(E), 1, ctypes.byref(huge), _v(B + (1 << 35)),
                                      1, s) == ERANGE


def test_outputs_overlapping_lists_weights_or_workspace_are_rejected(lib):
    """Every entry point checks what it writes against everything it reads: the
    block list, the count, the weights and the bias too."""
    s = _v(0)
    g = _g()
    far = _v(E + (1 << 35))
    conv = lib.sige_sparse_conv_layer
    assert conv(_v(A), _v(B), None, _v(C), _v(D), _v(E), 1, ctypes.byref(g), far, 1, s) == ENODEV  # valid
    assert conv(_v(A), _v(B), None, _v(C), _v(D), _v(E), 1, ctypes.byref(g), _v(D), 1, s) == EINVAL  # out = idx
    assert conv(_v(A), _v(B), None, _v(C), _v(D), _v(E), 1, ctypes.byref(g), _v(E), 1, s) == EINVAL  # out = count
    assert conv(_v(A), _v(B), None, _v(C), _v(D), _v(E), 1, ctypes.byref(g), _v(B + 256), 1, s) == EINVAL  # weights
    assert conv(_v(A), _v(B), _v(far.value + 64), _v(C), _v(D), _v(E), 1, ctypes.byref(g), far, 1,
                s) == EINVAL  # bias inside out
    sc = lib.sige_scatter
    assert sc(_v(A), _v(B), _v(C), ctypes.byref(g), 1, _v(D), far, 1, s) == ENODEV
    assert sc(_v(A), _v(B), _v(C), ctypes.byref(g), 1, _v(D), _v(B), 1, s) == EINVAL  # out = idx
    assert sc(_v(A), _v(B), _v(C), ctypes.byref(g), 1, _v(D), _v(C), 0, s) == EINVAL  # out = count
    assert lib.sige_gather(_v(A), 1, ctypes.byref(g), _v(B), _v(C), _v(B), s) == EINVAL  # blocks = idx
    assert lib.sige_conv_blocks(_v(A), _v(B), None, 1, ctypes.byref(g), _v(C), _v(B + 64), s) == EINVAL  # weights
    att = lib.sige_sparse_attention
    q, k, v, idx, cnt = A, B, D, A + (1 << 39), A + (1 << 40)

    def call(out=far.value, ws=C):
        return att(_v(q), _v(k), _v(v), _v(idx), _v(cnt), 2, 1, 64, 64, 5, 64, 4, ctypes.c_float(0.125), _v(E),
                   _v(out), 1, _v(ws), 1 << 30, s)

    assert call() == ENODEV
    assert call(ws=k) == EINVAL          # workspace overlaps k
    assert call(ws=idx) == EINVAL        # workspace overlaps idx
    assert call(ws=E) == EINVAL          # workspace overlaps cached
    assert call(out=idx) == EINVAL       # out overlaps idx
    assert call(ws=far.value + 64) == EINVAL  # workspace overlaps out
    rs = lib.sige_restore_blocks
    assert rs(_v(A), _v(B), _v(C), _v(D), ctypes.byref(g), 1, _v(E), far, s) == ENODEV
    assert rs(_v(A), _v(B), _v(C), _v(D), ctypes.byref(g), 1, _v(E), _v(A), s) == EINVAL  # out = prev_idx


def test_reduce_limits_match_between_one_layer_and_many(lib):
    """sige_reduce_bits_layers applies the single-layer reduce's limits per layer."""
    s = _v(0)
    many = _g(n=5, h=256, w=256)  # 5 * 1849 = 9245 blocks per launch: fine for both
    over = _g(n=9, h=256, w=256)  # 9 * 1849 = 16641 > 16384
    f1 = lib.sige_reduce_bits
    assert f1(_v(A), 256, 256, ctypes.byref(many), 1, _v(B), _v(C), s) == ENODEV
    assert f1(_v(A), 256, 256, ctypes.byref(over), 1, _v(B), _v(C), s) == ERANGE
    fl = lib.sige_reduce_bits_layers
    for geo, want in ((many, ENODEV), (over, ERANGE)):
        GA, IA, VA = L.Geom * 1, ctypes.c_int * 1, ctypes.c_void_p * 1
        rc = fl(_v(A), 256, 256, 1, GA(geo), IA(1), VA(B), VA(C), 1, None, None, s)
        assert rc == want, (geo.n, rc)


def test_binding_checks_list_capacity_and_shapes():
    """The binding refuses a block list shorter than the capacity (the kernels may
    read entries past *count) and tensors of the wrong shape or dtype."""
    g = ssi.geom(1, 64, 64, 32, 32, 3, 1, 1, 8)  # 8 x 8 = 64 blocks
    L._need_list(g, torch.zeros(64, dtype=torch.int32), torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError, match="idx"):
        L._need_list(g, torch.zeros(10, dtype=torch.int32), torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError, match="idx"):
        L._need_list(g, torch.zeros(64, dtype=torch.int64), torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError, match="count"):
        L._need_list(g, torch.zeros(64, dtype=torch.int32), torch.zeros(0, dtype=torch.int32))
    a = torch.zeros(1, 64, 64, 32, dtype=torch.bfloat16)
    w = torch.zeros(32, 3, 3, 32, dtype=torch.bfloat16)
    b = torch.zeros(32, dtype=torch.float32)
    L._need_layer(g, a, w, b, a, a)
    with pytest.raises(ValueError, match="w_krsc"):
        L._need_layer(g, a, w.permute(0, 3, 1, 2), b, None, None)
    with pytest.raises(ValueError, match="out"):
        L._need_layer(g, a, w, b, None, a[:, :32])
    with pytest.raises(ValueError, match="bias"):
        L._need_layer(g, a, w, b.double(), None, None)


def test_reduce_copy_validation(lib):
    s = _v(0)
    g = _g()
    f = lib.sige_reduce_mask_copy
    far = _v(E + (1 << 35))
    assert f(_v(A), 256, 256, ctypes.byref(g), 1, _v(B), _v(C), 1, None, far, s) == EINVAL
    assert f(_v(A), 256, 256, ctypes.byref(g), 1, _v(B), _v(C), 1, _v(D), None, s) == EINVAL
    assert f(_v(A), 256, 256, ctypes.byref(g), 1, _v(B), _v(C), 5, _v(D), far, s) == EDTYPE
    assert f(_v(A), 256, 256, ctypes.byref(g), 1, _v(B), _v(C), 1, _v(D + 8), far, s) == EALIGN
    assert f(_v(A), 256, 256, ctypes.byref(g), 1, _v(B), _v(C), 1, _v(D), _v(D + 256), s) == EINVAL  # overlap
    assert f(_v(A), 255, 256, ctypes.byref(g), 1, _v(B), _v(C), 1, _v(D), far, s) == EINVAL  # not a multiple


def test_split_layer_validation(lib):
    s = _v(0)
    g = _g(h=16, w=16, ci=1280, co=1280, b=2)
    f = lib.sige_sparse_conv_layer_split
    far = _v(E + (1 << 35))
    ws = 0x7F9000000000
    assert f(_v(A), _v(B), None, _v(C), _v(D), _v(E), 2, ctypes.byref(g), far, 1, None, 1 << 30, s) == EINVAL
    assert f(_v(A), _v(B), None, None, _v(D), _v(E), 2, ctypes.byref(g), far, 1, _v(ws), 1 << 30, s) == EINVAL
    assert f(_v(A), _v(B), None, _v(C), _v(D), _v(E), 7, ctypes.byref(g), far, 1, _v(ws), 1 << 30, s) == EDTYPE
    assert f(_v(A), _v(B), None, _v(C), _v(D), _v(E), 2, ctypes.byref(g), far, 1, _v(ws + 8), 1 << 30, s) == EALIGN
    assert f(_v(A), _v(B), None, _v(C), _v(D), _v(E), 2, ctypes.byref(g), _v(A + 64), 1, _v(ws), 1 << 30,
             s) == EINVAL  # out overlaps a_edit
    assert lib.sige_sparse_conv_layer_split_workspace(ctypes.byref(g), 2) > 0
    assert lib.sige_sparse_conv_layer_split_workspace(ctypes.byref(g), 9) == EDTYPE
    assert f(_v(A), _v(B), None, _v(C), _v(D), _v(E), 2, ctypes.byref(g), far, 1, _v(ws), 1 << 30, s) == ENODEV


def test_split_noalloc_limit_and_validation(lib):
    s = _v(0)
    f = lib.sige_sparse_conv_layer_split_noalloc
    far = _v(E + (1 << 35))
    assert lib.sige_noalloc_scratch_bytes() == 64 << 20
    # the 64x128x1024 -> 512 GauGAN-shaped layer needs 128 MiB of partial tiles: past the static scratch
    big = _g(h=64, w=128, ci=1024, co=512, b=4)
    assert lib.sige_sparse_conv_layer_split_workspace(ctypes.byref(big), 1) > lib.sige_noalloc_scratch_bytes()
    assert f(_v(A), _v(B), None, _v(C), _v(D), _v(E), 1, ctypes.byref(big), far, 1, s) == ERANGE
    assert b"scratch" in lib.sige_last_error()
    g = _g(h=16, w=16, ci=1280, co=1280, b=2)
    assert f(_v(A), _v(B), None, _v(C), _v(D), _v(E), 7, ctypes.byref(g), far, 1, s) == EDTYPE
    assert f(_v(A), _v(B), None, None, _v(D), _v(E), 2, ctypes.byref(g), far, 1, s) == EINVAL
    assert f(_v(A), _v(B), None, _v(C), _v(D), _v(E), 2, ctypes.byref(g), _v(A + 64), 1, s) == EINVAL
    # within the limit, a valid call reaches the device check (no GPU here)
    assert f(_v(A), _v(B), None, _v(C), _v(D), _v(E), 2, ctypes.byref(g), far, 1, s) == ENODEV


def test_restore_validation(lib):
    s = _v(0)
    g = _g()
    f = lib.sige_restore_blocks
    assert f(_v(A), _v(B), _v(C), _v(D), ctypes.byref(g), 3, _v(E), _v(E + (1 << 35)), s) == EDTYPE
    assert f(None, _v(B), _v(C), _v(D), ctypes.byref(g), 1, _v(E), _v(E + (1 << 35)), s) == EINVAL
    assert f(_v(A), _v(B), _v(C), None, ctypes.byref(g), 1, _v(E), _v(E + (1 << 35)), s) == EINVAL  # idx, no count
    assert f(_v(A), _v(B), _v(C), _v(D), ctypes.byref(g), 1, _v(E), _v(E + 64), s) == EINVAL  # out overlaps cached
    assert f(_v(A), _v(B), _v(C), _v(D), ctypes.byref(g), 1, _v(E + 8), _v(E + (1 << 35)), s) == EALIGN
    assert f(_v(A), _v(B), _v(C), _v(D), ctypes.byref(_g(co=12)), 1, _v(E), _v(E + (1 << 35)), s) == EALIGN
    assert f(_v(A), _v(B), None, None, ctypes.byref(_g(k=9)), 1, _v(E), _v(E + (1 << 35)), s) == EINVAL
    h = lib.sige_sparse_conv_layer_restore
    far = _v(E + (1 << 35))
    assert h(_v(A), _v(B), None, _v(C), _v(D), _v(D + 64), None, _v(E), 1, ctypes.byref(g), far, s) == EINVAL
    assert h(_v(A), _v(B), None, _v(C), _v(D), _v(D + 64), _v(E), _v(E + 64), 1, ctypes.byref(g), _v(A + 64),
             s) == EINVAL  # out overlaps a_edit
    assert h(_v(A), _v(B), None, _v(C), _v(D), _v(D + 64), _v(E), _v(E + 64), 1, ctypes.byref(g), _v(C), s) == EINVAL
    assert h(_v(A), _v(B + 4), None, _v(C), _v(D), _v(D + 64), _v(E), _v(E + 64), 1, ctypes.byref(g), far,
             s) == EALIGN


def test_attention_validation(lib):
    s = _v(0)
    f = lib.sige_sparse_attention
    far = _v(E + (1 << 35))

    def call(dtype=2, n=1, h=64, w=64, heads=5, hd=64, b=4, q=A, out=far, ws=C, wsb=1 << 30, scale=0.125):
        return f(_v(q), _v(B), _v(D), _v(A + (1 << 39)), _v(A + (1 << 40)), dtype, n, h, w, heads, hd, b,
                 ctypes.c_float(scale), _v(E), out, 1, _v(ws), wsb, s)

    assert call(dtype=0) == EDTYPE
    assert call(hd=32) == ERANGE
    assert call(n=9) == ERANGE
    assert call(heads=0) == EINVAL
    assert call(b=0) == EINVAL
    assert call(q=A + 8) == EALIGN
    assert call(out=_v(A + 64)) == EINVAL  # overlaps q
    assert call(scale=0.0) == EINVAL
    assert lib.sige_sparse_attention_workspace(1, 64, 64, 5, 32, 4) == ERANGE
    assert lib.sige_sparse_attention_workspace(1, 64, 64, 5, 64, 4) >= 64 * 68 * 4


def test_strerror_names_every_code(lib):
    for code, name in [(0, b"SIGE_OK"), (EINVAL, b"SIGE_EINVAL"), (EDTYPE, b"SIGE_EDTYPE"), (EALIGN, b"SIGE_EALIGN"),
                       (L.SIGE_EHIP, b"SIGE_EHIP"), (ENODEV, b"SIGE_ENODEV"), (ERANGE, b"SIGE_ERANGE")]:
        assert lib.sige_strerror(code).startswith(name)


def test_binding_raises_with_message(lib):
    with pytest.raises(ssi.SigeError) as e:
        ssi.sige_geom_derive(_g(k=9))
    assert "k=9" in str(e.value)


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="checks the no-GPU path")
def test_valid_call_without_gpu_is_enodev(lib):
    g = _g()
    assert lib.sige_diff_mask(_v(A), _v(B), 1, 1, 4, 4, 8, ctypes.c_float(1e-6), _v(C), _v(0)) == ENODEV
    assert lib.sige_reduce_mask(_v(A), 256, 256, ctypes.byref(g), 1, _v(B), _v(C), _v(0)) == ENODEV
    assert lib.sige_sparse_conv_layer(_v(A), _v(B), None, _v(C), _v(D), _v(E), 1, ctypes.byref(g),
                                      _v(E + (1 << 35)), 1, _v(0)) == ENODEV
    assert lib.sige_restore_blocks(_v(A), _v(B), None, None, ctypes.byref(g), 1, _v(E), _v(E + (1 << 35)),
                                   _v(0)) == ENODEV
    assert lib.sige_sparse_conv_layer_restore(_v(A), _v(B), None, _v(C), _v(D), _v(D + 64), _v(E), _v(E + 64), 1,
                                              ctypes.byref(g), _v(E + (1 << 35)), _v(0)) == ENODEV


def test_reduce_layers_validation(lib):
    """sige_reduce_bits_layers: host arrays of per-layer geometries, lists and copies."""
    f = lib.sige_reduce_bits_layers
    s = _v(0)
    gs = [_g(), _g(h=128, w=128, ci=128, co=256), _g(h=64, w=64, ci=256, co=256, b=4)]
    n = len(gs)
    step = 1 << 30

    def call(nl=n, geoms=gs, dil=(1, 1, 1), idx=None, cnt=None, dt=1, cached=None, out=None, mw=256, bits=A):
        GA, IA, VA = L.Geom * len(geoms), ctypes.c_int * len(dil), ctypes.c_void_p * n
        idx = idx or [B + i * step for i in range(n)]
        cnt = cnt or [C + i * 256 for i in range(n)]
        ca = VA(*cached) if cached is not None else None
        oa = VA(*out) if out is not None else None
        return f(_v(bits), 256, mw, nl, GA(*geoms), IA(*dil), VA(*idx), VA(*cnt), dt, ca, oa, s)

    cached = [D + i * step for i in range(n)]
    out = [E + i * step for i in range(n)]
    assert call() == ENODEV                                   # valid, no GPU here
    assert call(cached=cached, out=out) == ENODEV
    assert call(nl=0) == EINVAL
    assert call(nl=17) == EINVAL
    assert call(mw=250) == EINVAL                             # packed rows need whole words
    assert call(bits=A + 2) == EALIGN
    assert call(dil=(1, 17, 1)) == EINVAL
    assert call(geoms=[gs[0], _g(h=96, w=96), gs[2]]) == EINVAL  # 256 is not a multiple of 96
    assert call(geoms=[gs[0], _g(n=2, h=128, w=128), gs[2]]) == EINVAL  # one mask: the same n everywhere
    assert call(idx=[B, B + 64, B + 2 * step]) == EINVAL      # two layers' lists overlap
    assert call(cnt=[C, C, C + 512]) == EINVAL                # shared count
    assert call(cached=[cached[0], None, cached[2]], out=out) == EINVAL  # copy half given
    assert call(cached=[cached[0], None, cached[2]], out=[out[0], None, out[2]]) == ENODEV  # layer 1 not copied
    assert call(cached=cached, out=[out[0], out[0] + 256, out[2]]) == EINVAL  # outputs overlap
    assert call(cached=cached, out=[out[0], cached[1], out[2]]) == EINVAL     # output is another layer's cache
    assert call(cached=cached, out=out, dt=7) == EDTYPE
    assert call(cached=[cached[0] + 8, cached[1], cached[2]], out=out) == EALIGN
    assert call(geoms=[gs[0], _g(h=256, w=256, b=1), gs[2]]) == ERANGE  # 65536 blocks: beyond one workgroup



def test_layer_plan_without_a_gpu(lib):
    """sige_sparse_conv_layer_plan needs no device: the threshold lies in [-1, cap],
    a workspace is asked for exactly when the split can run, and a deep
    low-resolution layer goes to the split for its smallest lists."""
    for g, dt in ((_g(), torch.bfloat16), (_g(1, 16, 16, 1280, 1280, 3, 1, 1, 2), torch.float16),
                  (_g(1, 64, 128, 1024, 512), torch.bfloat16), (_g(1, 16, 16, 1280, 1280, 1, 1, 0, 2), torch.float16),
                  (_g(1, 64, 64, 64, 64, 3, 1, 1, 8), torch.float32)):
        p = ssi.sige_sparse_conv_layer_plan(g, dt)
        assert -1 <= p.split_max <= p.cap == ssi.sige_max_blocks(g)
        assert (p.workspace_bytes > 0) == (p.split_max >= 0)
        assert p.chunks >= 1 and p.steps >= 1 and p.slots >= 1 and p.n_tiles >= 1
    assert ssi.sige_sparse_conv_layer_plan(_g(1, 16, 16, 1280, 1280, 3, 1, 1, 2), torch.float16).split_max >= 1
    plan = L.LayerPlan()
    assert lib.sige_sparse_conv_layer_plan(ctypes.byref(_g()), 7, ctypes.byref(plan)) == EDTYPE
    assert lib.sige_sparse_conv_layer_plan(ctypes.byref(_g()), 1, None) == EINVAL


def test_layer_plan_wide_tiles_without_a_gpu():
    """The wide tiles' range in the plan: after the split's, within the capacity,
    for 16-bit types with k <= 3 only (not fp32, not 5x5, not where two staging
    buffers exceed the LDS: stride 2, 2x2 blocks); 16-channel stages and their
    1 KiB staging loads as the kernel issues them (windows of the <= 9 slots a
    256-row tile of 6x6 blocks touches, two 8x8 window rows per load, plus 4
    loads per tap for 128 columns of weights)."""
    p = ssi.sige_sparse_conv_layer_plan(_g(1, 256, 256, 128, 128, 3, 1, 1, 6), torch.bfloat16)
    assert p.wide_stages == 8 and p.wide_loads == 9 * 4 + 4 * 9 and p.wide_n_tiles == 1
    # from several hundred blocks on, to the longest list of one round (256 tiles of
    # 256 rows on 256 CUs): a list one tile longer takes two rounds and k_layer leads
    assert p.split_max < p.wide_min <= p.wide_max == 256 * 256 // 36 < p.cap
    # 8 stages: at most 2 K parts of 4 stages
    assert p.wide_parts_max == 2
    p = ssi.sige_sparse_conv_layer_plan(_g(1, 256, 512, 256, 128, 3, 1, 1, 6), torch.bfloat16)
    assert p.wide_stages == 16 and p.split_max < p.wide_min <= p.cap and p.wide_parts_max == 4
    p = ssi.sige_sparse_conv_layer_plan(_g(1, 32, 64, 1024, 1024, 3, 1, 1, 4), torch.bfloat16)
    assert p.wide_stages == 64 and p.wide_parts_max == 16
    for g, dt in ((_g(1, 256, 256, 128, 128, 3, 1, 1, 6), torch.float32),
                  (_g(1, 64, 64, 64, 64, 5, 1, 2, 6), torch.bfloat16),
                  (_g(1, 64, 64, 64, 128, 3, 2, 1, 4), torch.float16),
                  (_g(1, 16, 16, 1280, 1280, 3, 1, 1, 2), torch.float16)):
        p = ssi.sige_sparse_conv_layer_plan(g, dt)
        assert p.wide_stages == 0 and p.wide_min == p.wide_max == 0x7FFFFFFF, (g.k, g.s, g.b)
        assert p.wide_parts_max == 0


def test_layer_plan_ranges_over_random_geometries():
    """For any valid geometry and 16-bit or fp32 type the plan's ranges are
    ordered and disjoint (split up to split_max, wide tiles wide_min..wide_max
    after it, never past the capacity when present), the workspace is asked
    for exactly when the split can run, and the wide tiles appear only where
    their kernel can run (16-bit, k <= 3, stride 1 here)."""
    rng = np.random.default_rng(5)
    for _ in range(60):
        k = int(rng.choice([1, 3, 5]))
        s = int(rng.choice([1, 1, 2]))
        b = int(rng.integers(2, 9))
        h, w = int(rng.integers(8, 257)), int(rng.integers(8, 257))
        cin, cout = 8 * int(rng.integers(1, 41)), 8 * int(rng.integers(1, 41))
        dt = [torch.bfloat16, torch.float16, torch.float32][int(rng.integers(0, 3))]
        g = _g(1, h, w, cin, cout, k, s, k // 2, b)
        try:
            p = ssi.sige_sparse_conv_layer_plan(g, dt)
        except ssi.SigeError:
            continue  # a geometry some kernel's limits exclude (the call says which)
        assert -1 <= p.split_max <= p.cap
        assert (p.workspace_bytes > 0) == (p.split_max >= 0)
        if p.wide_min <= p.cap:
            assert dt != torch.float32 and k <= 3 and p.wide_stages == (cin + 15) // 16
            assert p.split_max < p.wide_min <= p.wide_max
        else:
            assert p.wide_min == 0x7FFFFFFF


def test_auto_layer_validation(lib):
    """Checks before any device work: a workspace smaller than the plan's is
    SIGE_ERANGE, overlaps and NULL pointers SIGE_EINVAL."""
    f = lib.sige_sparse_conv_layer_auto
    g = _g(1, 16, 16, 1280, 1280, 3, 1, 1, 2)
    need = ssi.sige_sparse_conv_layer_plan(g, torch.float16).workspace_bytes
    assert need > 0
    s = _v(0)
    args = (_v(A), _v(B), None, None, _v(C), _v(C + 4096), 2, ctypes.byref(g), _v(D), 0)
    assert f(*args, _v(E), need - 16, s) == ERANGE
    assert f(*args, None, 0, s) == ERANGE
    assert f(_v(A), _v(B), None, None, _v(C), _v(C + 4096), 2, ctypes.byref(g), _v(A + 64), 0, _v(E), need,
             s) == EINVAL  # out overlaps a_edit
    assert f(*args, _v(D + 4096), need, s) == EINVAL  # the workspace overlaps out
    assert f(None, _v(B), None, None, _v(C), _v(C + 4096), 2, ctypes.byref(g), _v(D), 0, _v(E), need, s) == EINVAL
    assert f(*args[:6], 7, *args[7:], _v(E), need, s) == EDTYPE


def test_packed_weights_validation(lib):
    """The packed weight copy: its size (the single-range kernel's section, one
    1 KiB load per chunk, N tile, K step and N subtile -- the KRSC size when
    nothing is padded -- then, from a 256-byte boundary, the wide tiles'
    section for 16-bit types where they run), and the checks of the pack call
    and of the packed layer entry points before any device work (short buffers
    SIGE_ERANGE, NULL and overlapping pointers SIGE_EINVAL, misalignment
    SIGE_EALIGN; a valid call without a GPU SIGE_ENODEV)."""
    def size(g, dt):
        return lib.sige_packed_weights_bytes(ctypes.byref(g), dt)

    def layer_part(g, dt):
        p = ssi.sige_sparse_conv_layer_plan(g, {0: torch.float32, 1: torch.bfloat16, 2: torch.float16}[dt])
        nsub = 2 if p.n_tiles * 32 >= g.c_out else 1  # 16 x NT output channels per N tile
        return p.chunks * p.n_tiles * p.steps * nsub * 1024
    g = _g(1, 256, 256, 128, 128, 3, 1, 1, 6)
    krsc = 128 * 9 * 128 * 2
    assert layer_part(g, 1) == krsc
    assert size(g, 1) == 3 * krsc  # the three sections, nothing padded
    assert layer_part(g, 0) == 2 * krsc and size(g, 0) == 4 * krsc  # fp32: no wide tiles; split chunks of 64
    g2 = _g(1, 64, 64, 24, 136, 3, 1, 1, 6)  # c_out 136: 5 N tiles of 32; c_in 24: one 32-channel slice
    lp = (layer_part(g2, 2) + 255) // 256 * 256
    wide = 2 * 2 * 9 * 256 * 16
    split = 1 * 5 * 9 * 1 * 2 * 1024  # one chunk, 5 N tiles, 9 taps x 1 slice, 2 subtiles
    assert size(g2, 2) == lp + wide + split
    gs = _g(1, 16, 16, 1280, 1280, 3, 1, 1, 2)  # no wide tiles (2x2 blocks)
    k2 = 1280 * 9 * 1280 * 2
    assert layer_part(gs, 2) == k2 and size(gs, 2) == 2 * k2
    assert size(g, 7) == EDTYPE
    need = size(g, 1)
    s = _v(0)
    pack = lib.sige_pack_weights
    assert pack(_v(A), 1, ctypes.byref(g), _v(B), need, s) == ENODEV
    assert pack(_v(A), 1, ctypes.byref(g), _v(B), need - 16, s) == ERANGE
    assert pack(None, 1, ctypes.byref(g), _v(B), need, s) == EINVAL
    assert pack(_v(A), 1, ctypes.byref(g), None, need, s) == EINVAL
    assert pack(_v(A), 1, ctypes.byref(g), _v(A + 4096), need, s) == EINVAL  # overlaps the KRSC weights
    assert pack(_v(A + 8), 1, ctypes.byref(g), _v(B), need, s) == EALIGN
    assert pack(_v(A), 1, ctypes.byref(g), _v(B + 16), need, s) == EALIGN  # 256-byte alignment

    W = A + (5 << 36)
    f = lib.sige_sparse_conv_layer_packed
    args = (_v(A), _v(B), None, None, _v(C), _v(C + 4096), 1, ctypes.byref(g), _v(D), 0)
    assert f(*args, _v(W), need, s) == ENODEV
    assert f(*args, None, need, s) == EINVAL
    assert f(*args, _v(W), need - 16, s) == ERANGE
    assert f(*args, _v(W + 16), need, s) == EALIGN
    assert f(*args, _v(D + 256), need, s) == EINVAL  # overlaps out

    f = lib.sige_conv_blocks_packed
    args = (_v(A), _v(B), None, 1, ctypes.byref(g), _v(C), _v(D))
    assert f(*args, _v(W), need, s) == ENODEV
    assert f(*args, None, need, s) == EINVAL
    assert f(*args, _v(W), need - 16, s) == ERANGE
    assert f(*args, _v(D + 256), need, s) == EINVAL  # overlaps out_blocks

    f = lib.sige_sparse_conv_layer_auto_packed
    g3 = _g(1, 32, 64, 1024, 1024, 3, 1, 1, 4)
    need3 = size(g3, 1)
    ws = ssi.sige_sparse_conv_layer_plan(g3, torch.bfloat16).workspace_bytes
    args = (_v(A), _v(B), None, None, _v(C), _v(C + 4096), 1, ctypes.byref(g3), _v(D), 0, _v(E), ws)
    assert f(*args, _v(W), need3, s) == ENODEV
    assert f(*args, None, need3, s) == EINVAL
    assert f(*args, _v(W), need3 - 16, s) == ERANGE
    assert f(*args, _v(W + 16), need3, s) == EALIGN
    assert f(*args, _v(D + 256), need3, s) == EINVAL  # overlaps out
    assert f(*args, _v(E + 256), need3, s) == EINVAL  # overlaps the workspace

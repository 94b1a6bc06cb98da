"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: a closed form, a library routine
that the case reduces to (torch fp64 conv2d, max_pool2d, numpy/torch casts), an
invariant of the mathematics, brute force on tiny inputs, or a fact printed on
the pages (tests/golden).  CPU only.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DTS = [torch.float32, torch.bfloat16, torch.float16]


def _rand(shape, dtype, seed, std=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g, dtype=torch.float32) * std).to(dtype)


def _torch_conv_f64(a_nhwc, w_oihw, bias, s, p):
    """Library reference: torch conv2d in fp64 on the exactly-widened stored values."""
    x = oracle.decode(a_nhwc).permute(0, 3, 1, 2)
    y = F.conv2d(x, oracle.decode(w_oihw), None if bias is None else bias.double(), stride=s, padding=p)
    return y.permute(0, 2, 3, 1).contiguous()


def _pixel_block_mask(active, b, ho, wo):
    """[n, ho, wo] bool: pixel lies in an active block (nearest-neighbour upsampling)."""
    up = active.bool().repeat_interleave(b, 1).repeat_interleave(b, 2)
    return up[:, :ho, :wo]


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------
def test_round_known_bit_patterns():
    # IEEE 754 binary16 and bfloat16 encodings worked out by hand
    x = torch.tensor([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 65504.0, 65520.0, 2 ** -24, 2 ** -25,
                      3 * 2 ** -25, -2.0, 0.0, 1e30], dtype=torch.float64)
    bf = oracle.round_to(x, torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    hf = oracle.round_to(x, torch.float16).view(torch.int16).numpy().astype(np.uint16)
    assert [hex(v) for v in bf] == ["0x3f80", "0x3f80", "0x3f82", "0x4780", "0x4780", "0x3380", "0x3300",
                                    "0x33c0", "0xc000", "0x0", "0x714a"]
    assert [hex(v) for v in hf] == ["0x3c00", "0x3c04", "0x3c0c", "0x7bff", "0x7c00", "0x1", "0x0",
                                    "0x2", "0xc000", "0x0", "0x7c00"]


def test_round_f16_matches_numpy_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-9, 6, 20000),
                        rng.uniform(-7e4, 7e4, 2000), [6.1e-5, -5.96e-8, 2.98e-8, 65519.99, 65520.0]])
    ours = oracle.round_to(torch.from_numpy(x), torch.float16).view(torch.int16).numpy()
    ref = x.astype(np.float16).view(np.int16)
    assert np.array_equal(ours, ref)


def test_round_bf16_matches_torch_cast_on_f32_values():
    x32 = _rand((50000,), torch.float32, 1) * torch.exp(_rand((50000,), torch.float32, 2) * 20)
    ours = oracle.round_to(x32.double(), torch.bfloat16).view(torch.int16)
    ref = x32.to(torch.bfloat16).view(torch.int16)
    assert torch.equal(ours, ref)


def test_decode_is_exact_widening():
    for dt in DTS:
        t = _rand((4096,), dt, 3, 100.0)
        assert torch.equal(oracle.decode(t), t.double())


# ---------------------------------------------------------------------------
# step 1: diff
# ---------------------------------------------------------------------------
def test_diff_strict_threshold_boundary():
    tau = np.float32(1e-6)
    a_o = torch.zeros((1, 2, 3, 5), dtype=torch.float32)
    a_e = a_o.clone()
    a_e[0, 0, 0, 4] = float(tau)  # exactly tau: not flagged (strict >)
    a_e[0, 0, 1, 4] = float(np.nextafter(tau, np.float32(1)))  # one ulp above
    a_e[0, 1, 2, 0] = -float(np.nextafter(tau, np.float32(1)))  # negative change, first channel
    a_e[0, 1, 0, 3] = float(np.nextafter(tau, np.float32(0)))  # below
    m = oracle.diff_mask(a_o, a_e, float(tau))
    assert m.tolist() == [[[0, 1, 0], [0, 0, 1]]]


def test_diff_small_bf16_change_is_seen():
    a_o = torch.ones((1, 1, 2, 8), dtype=torch.bfloat16)
    a_e = a_o.clone()
    a_e[0, 0, 1, 7] = 1.0078125  # next bf16 above 1: a change of 2^-7
    assert oracle.diff_mask(a_o, a_e).tolist() == [[[0, 1]]]


@pytest.mark.parametrize("name", ["rect_64x64x64_f32", "unet_256x256x128_bf16"])
def test_diff_recovers_generated_edit_region(name):
    # the generator changes every channel of exactly the masked pixels
    wl = synth.workload(name)
    L = wl.layers[0]
    if wl.edit == "rect":
        m, _ = synth.rectangle_mask(5, L.h, L.w)
    else:
        m = synth.edit_shape(wl, 5).raster(L.h, L.w)
    a_o = synth.make_activation(1, L.h, L.w, L.c_in, L.dtype, 5, wl.layout)
    a_e = synth.make_edit(a_o, m, wl.edit_kind, 5, wl.layout)
    got = oracle.diff_mask(a_o, a_e, wl.tau, wl.layout)
    assert np.array_equal(got[0].numpy(), m)


def test_diff_same_mask_in_nchw_and_nhwc():
    a_o = _rand((2, 9, 11, 24), torch.float16, 4)
    a_e = a_o.clone()
    a_e[1, 3, 4, 17] += 1
    a_e[0, 8, 10, 0] -= 1
    m1 = oracle.diff_mask(a_o, a_e, 1e-6, "NHWC")
    m2 = oracle.diff_mask(a_o.permute(0, 3, 1, 2).contiguous(), a_e.permute(0, 3, 1, 2).contiguous(), 1e-6,
                          "NCHW")
    assert torch.equal(m1, m2) and int(m1.sum()) == 2


# ---------------------------------------------------------------------------
# step 2: reduce
# ---------------------------------------------------------------------------
def test_rectangle_blocks_closed_form():
    # 10x12 rectangle rows [y0, y0+9], cols [x0, x0+11]; 3x3 s1 p1 conv, 8x8 blocks,
    # 10x10 windows starting at 8i-1: block row i is hit iff 8i-1 <= y0+9 and 8i+8 >= y0.
    for seed in range(60):
        m, (y0, x0) = synth.rectangle_mask(seed)
        act = oracle.block_activity(torch.from_numpy(m), 64, 64, 3, 1, 1, 8, 0)[0].numpy()
        rows = [i for i in range(8) if math.ceil((y0 - 8) / 8) <= i <= math.floor((y0 + 10) / 8)]
        cols = [j for j in range(8) if math.ceil((x0 - 8) / 8) <= j <= math.floor((x0 + 12) / 8)]
        want = np.zeros((8, 8), np.uint8)
        want[np.ix_(rows, cols)] = 1
        assert np.array_equal(act, want), seed
        assert 4 <= act.sum() <= 9


GEOMS = [  # (h, w, k, s, p, b); all satisfy (ho-1)*s - p + k >= h (every input row feeds an output)
    (13, 17, 3, 1, 1, 2), (13, 17, 3, 1, 1, 4), (16, 20, 3, 1, 1, 6), (13, 15, 3, 2, 1, 3),
    (14, 18, 3, 2, 1, 2), (12, 11, 1, 1, 0, 4), (11, 14, 5, 1, 2, 3), (9, 9, 3, 1, 1, 9),
]


@pytest.mark.parametrize("geom", GEOMS)
def test_activity_equals_blocks_whose_output_changes(geom):
    # brute force: a block must be recomputed iff some output pixel of it changes
    # when the marked input pixels change (random fp64 data: no accidental cancellation)
    h, w, k, s, p, b = geom
    ho, wo, nby, nbx, _ = oracle.geometry(h, w, k, s, p, b)
    assert (ho - 1) * s - p + k >= h and (wo - 1) * s - p + k >= w
    rng = np.random.default_rng(h * 131 + w * 7 + k + s + b)
    for trial in range(6):
        m = (rng.random((h, w)) < [0.01, 0.03, 0.08, 0.0, 0.2, 0.02][trial]).astype(np.uint8)
        a_o = torch.randn((1, h, w, 3), dtype=torch.float64)
        a_e = a_o + torch.from_numpy(m).double()[None, :, :, None] * torch.randn((1, h, w, 3),
                                                                                   dtype=torch.float64)
        wt = torch.randn((2, 3, k, k), dtype=torch.float64)
        y_o = F.conv2d(a_o.permute(0, 3, 1, 2), wt, stride=s, padding=p)
        y_e = F.conv2d(a_e.permute(0, 3, 1, 2), wt, stride=s, padding=p)
        changed = (y_o != y_e).any(1)[0].numpy()
        want = np.zeros((nby, nbx), np.uint8)
        for y, x in zip(*np.nonzero(changed)):
            want[y // b, x // b] = 1
        got = oracle.block_activity(torch.from_numpy(m), h, w, k, s, p, b, 0)[0].numpy()
        assert np.array_equal(got, want), (geom, trial)


@pytest.mark.parametrize("f", [2, 4, 8])
def test_pooling_is_max_pool(f):
    rng = np.random.default_rng(f)
    h, w = 12, 20
    m = torch.from_numpy((rng.random((2, h * f, w * f)) < 0.004).astype(np.uint8))
    pooled = F.max_pool2d(m.float()[:, None], f)[:, 0].to(torch.uint8)
    for k, s, p, b in [(3, 1, 1, 4), (3, 2, 1, 2), (1, 1, 0, 3)]:
        got = oracle.block_activity(m, h, w, k, s, p, b, 1)
        ref = oracle.block_activity(pooled, h, w, k, s, p, b, 1)
        assert torch.equal(got, ref)


@pytest.mark.parametrize("d", [1, 2, 3])
def test_dilation_is_square_max_pool(d):
    rng = np.random.default_rng(10 + d)
    m = torch.from_numpy((rng.random((2, 40, 52)) < 0.01).astype(np.uint8))
    a0 = oracle.block_activity(m, 40, 52, 3, 1, 1, 4, 0)
    ad = oracle.block_activity(m, 40, 52, 3, 1, 1, 4, d)
    ref = F.max_pool2d(a0.float()[:, None], 2 * d + 1, stride=1, padding=d)[:, 0].to(torch.uint8)
    assert torch.equal(ad, ref)
    assert bool((ad >= a0).all())  # monotone


def test_index_list_is_ascending_nonzero():
    rng = np.random.default_rng(3)
    act = torch.from_numpy((rng.random((3, 7, 9)) < 0.3).astype(np.uint8))
    idx = oracle.index_list(act)
    assert torch.equal(idx.long(), torch.nonzero(act.flatten())[:, 0])
    assert oracle.index_list(torch.zeros((1, 4, 4), dtype=torch.uint8)).numel() == 0


def test_empty_mask_gives_no_blocks():
    m = torch.zeros((1, 256, 256), dtype=torch.uint8)
    assert int(oracle.block_activity(m, 256, 256, 3, 1, 1, 6, 1).sum()) == 0


# ---------------------------------------------------------------------------
# steps 3-5: the edited output
# ---------------------------------------------------------------------------
CONV_CASES = [  # (n, h, w, cin, cout, k, s, p, dtype)
    (1, 11, 13, 8, 16, 3, 1, 1, torch.float32),
    (2, 10, 9, 16, 8, 3, 2, 1, torch.bfloat16),
    (1, 7, 12, 24, 16, 1, 1, 0, torch.float16),
    (1, 9, 9, 8, 8, 5, 1, 2, torch.bfloat16),
    (1, 12, 10, 32, 16, 3, 2, 0, torch.float32),
]


@pytest.mark.parametrize("case", CONV_CASES)
def test_dense_conv_matches_torch_fp64(case):
    n, h, w, cin, cout, k, s, p, dt = case
    a = _rand((n, h, w, cin), dt, 11)
    wt = _rand((cout, cin, k, k), dt, 12, 0.2)
    bias = _rand((cout,), torch.float32, 13, 0.1)
    got = oracle.dense_conv(a, wt, bias, k, s, p, out_f64=True)
    ref = _torch_conv_f64(a, wt, bias, s, p)
    assert got.shape == ref.shape
    assert (got - ref).abs().max() <= 1e-12 * ref.abs().max()
    # the rounded output is the fp64 output rounded once (nearest even)
    rounded = oracle.dense_conv(a, wt, bias, k, s, p)
    assert torch.equal(rounded.view(torch.int16) if dt != torch.float32 else rounded,
                       oracle.round_to(got, dt).view(torch.int16) if dt != torch.float32
                       else oracle.round_to(got, dt))


def test_nchw_and_nhwc_agree():
    a = _rand((1, 9, 10, 8), torch.float32, 21)
    wt = _rand((8, 8, 3, 3), torch.float32, 22)
    y1 = oracle.dense_conv(a, wt, None, 3, 1, 1, "NHWC")
    y2 = oracle.dense_conv(a.permute(0, 3, 1, 2).contiguous(), wt, None, 3, 1, 1, "NCHW")
    assert torch.equal(y1, y2.permute(0, 2, 3, 1))


def test_linearity_without_bias():
    # conv(A_e) = conv(A_o) + conv(A_e - A_o) (mer.dev notes, 3.1), in fp64
    a_o = torch.randn((1, 10, 12, 16), dtype=torch.float64)
    a_e = a_o.clone()
    a_e[0, 3:6, 4:9] += torch.randn((3, 5, 16), dtype=torch.float64)
    wt = torch.randn((8, 16, 3, 3), dtype=torch.float64)
    c = lambda x: oracle.sparse_layer(x, wt, None, 3, 1, 1, 1, None, None, out_f64=True)  # noqa: E731
    assert (c(a_e) - (c(a_o) + c(a_e - a_o))).abs().max() <= 1e-12 * c(a_e).abs().max()


def _pipeline(a_o, a_e, wt, bias, k, s, p, b, d, tau=1e-6):
    """diff -> reduce -> edited output, with the cache = conv(A_o) (all oracle)."""
    cache = oracle.dense_conv(a_o, wt, bias, k, s, p)
    m = oracle.diff_mask(a_o, a_e, tau)
    _, _, h, w = (None, None) + tuple(a_o.shape[1:3])
    act = oracle.block_activity(m, h, w, k, s, p, b, d)
    return oracle.sparse_layer(a_e, wt, bias, k, s, p, b, act, cache), cache, act


@pytest.mark.parametrize("dt", DTS)
def test_empty_edit_returns_cache_bit_for_bit(dt):
    a = _rand((1, 18, 22, 16), dt, 31)
    wt = _rand((16, 16, 3, 3), dt, 32, 0.1)
    out, cache, act = _pipeline(a, a.clone(), wt, _rand((16,), torch.float32, 33), 3, 1, 1, 6, 1)
    assert int(act.sum()) == 0
    assert torch.equal(out.view(torch.uint8), cache.view(torch.uint8))


@pytest.mark.parametrize("dt,k,s,p,b,d", [(torch.float32, 3, 1, 1, 8, 0), (torch.bfloat16, 3, 1, 1, 6, 1),
                                          (torch.float16, 3, 2, 1, 3, 0), (torch.bfloat16, 1, 1, 0, 4, 1),
                                          (torch.float16, 5, 1, 2, 4, 0)])
def test_single_layer_sparse_equals_dense_edited(dt, k, s, p, b, d):
    # with the input-window activity rule the sparse result is the dense conv of
    # A_e at every pixel, bit for bit (unchanged receptive field => same bits)
    a_o = _rand((1, 30, 26, 16), dt, 41)
    m = np.zeros((30, 26), np.uint8)
    m[7:11, 5:9] = 1
    m[20, 20] = 1
    a_e = synth.make_edit(a_o, m, "replace", 42)
    wt = _rand((16, 16, k, k), dt, 43, 0.2)
    bias = _rand((16,), torch.float32, 44)
    out, cache, act = _pipeline(a_o, a_e, wt, bias, k, s, p, b, d)
    dense = oracle.dense_conv(a_e, wt, bias, k, s, p)
    assert 0 < int(act.sum()) < act.numel()
    assert torch.equal(out.view(torch.uint8), dense.view(torch.uint8))
    assert not torch.equal(out.view(torch.uint8), cache.view(torch.uint8))


@pytest.mark.parametrize("dt", DTS)
def test_delta_kernel_copies_edited_input(dt):
    # W = centre-tap identity, zero bias: active pixels equal A_e exactly, others the cache
    c = 16
    wt = torch.zeros((c, c, 3, 3), dtype=torch.float32)
    wt[torch.arange(c), torch.arange(c), 1, 1] = 1.0
    wt = wt.to(dt)
    a_e = _rand((1, 14, 19, c), dt, 51)
    cache = _rand((1, 14, 19, c), dt, 52)
    act = torch.zeros((1, 3, 4), dtype=torch.uint8)
    act[0, 1, 2] = act[0, 2, 3] = act[0, 0, 0] = 1
    out = oracle.sparse_layer(a_e, wt, None, 3, 1, 1, 5, act, cache)
    pm = _pixel_block_mask(act, 5, 14, 19)[0]
    assert torch.equal(out[0][pm].view(torch.uint8), a_e[0][pm].view(torch.uint8))
    assert torch.equal(out[0][~pm].view(torch.uint8), cache[0][~pm].view(torch.uint8))


def test_integer_data_is_exact_in_fp32():
    g = torch.Generator().manual_seed(61)
    a = torch.randint(-2, 3, (1, 9, 10, 8), generator=g).float()
    wt = torch.randint(-2, 3, (8, 8, 3, 3), generator=g).float()
    got = oracle.dense_conv(a, wt, None, 3, 1, 1)
    ref = F.conv2d(a.permute(0, 3, 1, 2).double(), wt.double(), padding=1).permute(0, 2, 3, 1)
    assert torch.equal(got.double(), ref)


def test_brute_force_every_block_subset_tiny():
    # 1x7x9x3 input, 3x3 s1 p1, 2x2 blocks -> a 4x5 grid with partial last row and column;
    # all 64 subsets of the 2x3 sub-grid rows {2,3} x cols {2,3,4} (the partial edge):
    # the output is conv(A_e) on selected blocks' pixels and the cache elsewhere
    a_e = torch.randn((1, 7, 9, 3), dtype=torch.float64)
    cache = torch.randn((1, 7, 9, 4), dtype=torch.float64)
    wt = torch.randn((4, 3, 3, 3), dtype=torch.float64)
    bias = torch.randn((4,), dtype=torch.float32)
    dense = _torch_conv_f64(a_e, wt, bias, 1, 1)
    cells = [(i, j) for i in (2, 3) for j in (2, 3, 4)]
    for bits in itertools.product([0, 1], repeat=len(cells)):
        act = torch.zeros((1, 4, 5), dtype=torch.uint8)
        for on, (i, j) in zip(bits, cells):
            act[0, i, j] = on
        out = oracle.sparse_layer(a_e, wt, bias, 3, 1, 1, 2, act, cache, out_f64=True)
        pm = _pixel_block_mask(act, 2, 7, 9)[..., None]
        ref = torch.where(pm, dense, cache)
        assert (out - ref).abs().max() <= 1e-12 * dense.abs().max()
        assert torch.equal(out[~pm.expand_as(out)], cache[~pm.expand_as(out)])


# ---------------------------------------------------------------------------
# the three separate steps
# ---------------------------------------------------------------------------
def test_gather_is_zero_padded_slice():
    a = _rand((2, 11, 13, 8), torch.bfloat16, 71)
    k, s, p, b = 3, 2, 1, 3
    ho, wo, nby, nbx, ib = oracle.geometry(11, 13, k, s, p, b)
    assert ib == 2 * b + 1
    idx = torch.tensor([0, 3, nby * nbx - 1, nby * nbx + 5, 2 * nby * nbx - 1], dtype=torch.int32)
    blocks = oracle.gather(a, k, s, p, b, idx)
    pad = 20
    ap = F.pad(a.float().permute(0, 3, 1, 2), (pad, pad, pad, pad)).permute(0, 2, 3, 1)
    for slot, lin in enumerate(idx.tolist()):
        n, i, j = lin // (nby * nbx), (lin // nbx) % nby, lin % nbx
        y0, x0 = i * b * s - p + pad, j * b * s - p + pad
        assert torch.equal(blocks[slot].float(), ap[n, y0:y0 + ib, x0:x0 + ib])


def test_gather_overlap_matches_readme():
    # golden: gathered blocks of a 3x3 stride-1 conv overlap by a strip 2 px wide
    g = json.load(open(os.path.join(GOLDEN, "readme_overview_overlap.json")))
    k, s, b = g["k"], g["stride"], 6
    a = _rand((1, 24, 24, 4), torch.float32, 72)
    ho, wo, nby, nbx, ib = oracle.geometry(24, 24, k, s, (k - 1) // 2, b)
    idx = torch.tensor([nbx + 1, nbx + 2, 2 * nbx + 1], dtype=torch.int32)
    bl = oracle.gather(a, k, s, (k - 1) // 2, b, idx)
    ov = g["overlap"]
    assert ib - b * s == ov
    assert torch.equal(bl[0][:, ib - ov:], bl[1][:, :ov])  # horizontal neighbours
    assert torch.equal(bl[0][ib - ov:, :], bl[2][:ov, :])  # vertical neighbours
    assert not torch.equal(bl[0][:, ib - ov - 1], bl[1][:, ov])  # and no wider


@pytest.mark.parametrize("k,s,b", [(3, 1, 4), (3, 2, 3), (1, 1, 4), (5, 1, 2)])
def test_conv_blocks_is_valid_conv(k, s, b):
    ib = (b - 1) * s + k
    blocks = _rand((5, ib, ib, 16), torch.float16, 81)
    wt = _rand((8, 16, k, k), torch.float16, 82, 0.2)
    bias = _rand((8,), torch.float32, 83)
    got = oracle.conv_blocks(blocks, wt, bias, k, s, b, out_f64=True)
    ref = _torch_conv_f64(blocks, wt, bias, s, 0)
    assert got.shape == ref.shape == (5, b, b, 8)
    assert (got - ref).abs().max() <= 1e-12 * ref.abs().max()


def test_scatter_is_block_overwrite():
    cache = _rand((2, 10, 11, 8), torch.bfloat16, 91)
    b = 4
    nby, nbx = 3, 3
    idx = torch.tensor([0, 4, 8, 9 + 5], dtype=torch.int32)
    ob = _rand((4, b, b, 8), torch.bfloat16, 92)
    out = oracle.scatter(ob, idx, cache, b)
    ref = cache.clone()
    for slot, lin in enumerate(idx.tolist()):
        n, i, j = lin // (nby * nbx), (lin // nbx) % nby, lin % nbx
        hh, ww = min(b, 10 - i * b), min(b, 11 - j * b)
        ref[n, i * b:i * b + hh, j * b:j * b + ww] = ob[slot, :hh, :ww]
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("dt,k,s,p,b", [(torch.bfloat16, 3, 1, 1, 6), (torch.float16, 3, 2, 1, 4),
                                        (torch.float32, 1, 1, 0, 3)])
def test_three_steps_compose_to_the_layer(dt, k, s, p, b):
    a_e = _rand((2, 26, 23, 16), dt, 101)
    wt = _rand((8, 16, k, k), dt, 102, 0.2)
    bias = _rand((8,), torch.float32, 103)
    ho, wo, nby, nbx, ib = oracle.geometry(26, 23, k, s, p, b)
    cache = _rand((2, ho, wo, 8), dt, 104)
    rng = np.random.default_rng(105)
    act = torch.from_numpy((rng.random((2, nby, nbx)) < 0.35).astype(np.uint8))
    idx = oracle.index_list(act)
    out3 = oracle.scatter(oracle.conv_blocks(oracle.gather(a_e, k, s, p, b, idx), wt, bias, k, s, b), idx, cache, b)
    out1 = oracle.sparse_layer(a_e, wt, bias, k, s, p, b, act, cache)
    assert torch.equal(out3.view(torch.uint8), out1.view(torch.uint8))


# ---------------------------------------------------------------------------
# sequential edits: restore the previous edit's blocks, then write the new ones
# ---------------------------------------------------------------------------
def _seq_case(dt, seed, h=29, w=23, k=3, s=1, p=1, b=4, cin=16, cout=8):
    a_o = _rand((1, h, w, cin), dt, seed)
    wt = _rand((cout, cin, k, k), dt, seed + 1, 0.2)
    bias = _rand((cout,), torch.float32, seed + 2)
    cache = oracle.dense_conv(a_o, wt, bias, k, s, p)
    return a_o, wt, bias, cache


@pytest.mark.parametrize("dt", DTS)
def test_sequential_edits_through_restore_equal_fresh_layers(dt):
    # out_k by restore(prev -> cache) + writing list k's blocks into a persistent
    # buffer == the layer computed from scratch with the cache copy, bit for bit,
    # over three edits with overlapping and disjoint block lists (partial edge blocks)
    k, s, p, b = 3, 1, 1, 4
    a_o, wt, bias, cache = _seq_case(dt, 111)
    ho, wo = cache.shape[1:3]
    rects = [(3, 9, 2, 8), (5, 14, 6, 12), (20, 29, 15, 23)]  # rows [y0, y1), cols [x0, x1)
    out = cache.clone()
    prev = torch.zeros(0, dtype=torch.int32)
    for r, (y0, y1, x0, x1) in enumerate(rects):
        m = np.zeros((29, 23), np.uint8)
        m[y0:y1, x0:x1] = 1
        a_e = synth.make_edit(a_o, m, "replace", 120 + r)
        act = oracle.block_activity(oracle.diff_mask(a_o, a_e), 29, 23, k, s, p, b, 1)
        idx = oracle.index_list(act)
        fresh = oracle.sparse_layer(a_e, wt, bias, k, s, p, b, act, cache)
        oracle.restore_blocks(prev, idx, cache, out, b)
        blocks = oracle.conv_blocks(oracle.gather(a_e, k, s, p, b, idx), wt, bias, k, s, b)
        oracle.scatter(blocks, idx, cache, b, copy_cached=False, out=out)
        assert torch.equal(out.view(torch.uint8), fresh.view(torch.uint8)), f"edit {r}"
        prev = idx


def test_restore_touches_exactly_the_blocks_left_behind():
    # brute force on the block grid: pixels of blocks in prev and not in new take
    # the cache; every other pixel keeps its value
    dt = torch.bfloat16
    n, ho, wo, c, b = 2, 13, 18, 8, 4
    nby, nbx = -(-ho // b), -(-wo // b)
    cache = _rand((n, ho, wo, c), dt, 131)
    rng = np.random.default_rng(132)
    for trial in range(20):
        prev_act = rng.random((n, nby, nbx)) < 0.4
        new_act = rng.random((n, nby, nbx)) < 0.4
        before = _rand((n, ho, wo, c), dt, 140 + trial)
        out = before.clone()
        prev_idx = oracle.index_list(torch.from_numpy(prev_act.astype(np.uint8)))
        new_idx = oracle.index_list(torch.from_numpy(new_act.astype(np.uint8)))
        oracle.restore_blocks(prev_idx, new_idx, cache, out, b)
        gone = torch.from_numpy(prev_act & ~new_act)
        pix = _pixel_block_mask(gone, b, ho, wo)[..., None].expand_as(out)
        expect = torch.where(pix, cache, before)
        assert torch.equal(out.view(torch.int16), expect.view(torch.int16)), f"trial {trial}"


def test_restore_special_cases():
    dt = torch.float16
    cache = _rand((1, 16, 16, 8), dt, 151)
    out = _rand((1, 16, 16, 8), dt, 152)
    idx = torch.tensor([0, 5, 6, 15], dtype=torch.int32)
    same = oracle.restore_blocks(idx, idx, cache, out.clone(), 4)
    assert torch.equal(same.view(torch.int16), out.view(torch.int16))  # prev == new: nothing to do
    act = torch.ones((1, 4, 4), dtype=torch.uint8)
    allb = oracle.restore_blocks(oracle.index_list(act), None, cache, out.clone(), 4)
    assert torch.equal(allb.view(torch.int16), cache.view(torch.int16))  # no new list: all back to the cache


# ---------------------------------------------------------------------------
# query-pruned self-attention
# ---------------------------------------------------------------------------
def _attn_torch_f64(q, k, v, heads, scale):
    """Library reference: torch softmax and matmul in fp64, per image and head."""
    n, h, w, C = q.shape
    d = C // heads
    qd, kd, vd = (oracle.decode(t).reshape(n, h * w, heads, d).permute(0, 2, 1, 3) for t in (q, k, v))
    p = torch.softmax(scale * qd @ kd.transpose(-1, -2), dim=-1)
    return (p @ vd).permute(0, 2, 1, 3).reshape(n, h, w, C)


@pytest.mark.parametrize("dt", DTS)
def test_attention_dense_matches_torch_fp64(dt):
    n, h, w, heads, d = 2, 6, 7, 2, 8
    q, k, v = (_rand((n, h, w, heads * d), dt, 501 + i) for i in range(3))
    ref = _attn_torch_f64(q, k, v, heads, d ** -0.5)
    got = oracle.sparse_attention(q, k, v, heads, 2, None, None, out_f64=True)
    assert (got - ref).abs().max() <= 1e-12 * ref.abs().max()
    rounded = oracle.sparse_attention(q, k, v, heads, 2, None, None)
    assert torch.equal(rounded.view(torch.uint8), oracle.round_to(got, dt).view(torch.uint8))


def test_attention_uniform_keys_average_the_values():
    n, h, w, heads, d = 1, 5, 6, 3, 4
    dt = torch.float32
    q = _rand((n, h, w, heads * d), dt, 511)
    k = _rand((1, 1, 1, heads * d), dt, 512).expand(n, h, w, heads * d).contiguous()  # every key the same
    v = _rand((n, h, w, heads * d), dt, 513)
    got = oracle.sparse_attention(q, k, v, heads, 2, None, None, out_f64=True)
    mean = v.double().reshape(n, h * w, heads * d).mean(dim=1)
    assert (got.reshape(n, h * w, -1) - mean[:, None, :]).abs().max() <= 1e-12


def test_attention_dominant_key_selects_its_value():
    n, h, w, heads, d = 1, 4, 4, 1, 16
    dt = torch.float32
    eye = torch.eye(16)
    k = (eye * 40.0).reshape(1, 4, 4, 16)  # key j = 40 e_j: q = e_j scores 40 against 0 for every other key
    q = eye.reshape(1, 4, 4, 16)
    v = _rand((n, h, w, 16), dt, 521)
    got = oracle.sparse_attention(q, k, v, heads, 4, None, None, out_f64=True, scale=1.0)
    e = math.exp(-40.0)
    vv = v.double().reshape(16, 16)
    expect = (vv + e * (vv.sum(0, keepdim=True) - vv)) / (1 + 15 * e)  # closed form of the softmax mixture
    assert (got.reshape(16, 16) - expect).abs().max() <= 1e-12


def test_attention_is_invariant_to_a_joint_key_value_permutation_and_images_are_independent():
    n, h, w, heads, d = 2, 5, 5, 2, 8
    dt = torch.float64
    q, k, v = (_rand((n, h, w, heads * d), dt, 531 + i) for i in range(3))
    base = oracle.sparse_attention(q, k, v, heads, 2, None, None)
    perm = torch.randperm(h * w, generator=torch.Generator().manual_seed(5))
    kp = k.reshape(n, h * w, -1)[:, perm].reshape(k.shape)
    vp = v.reshape(n, h * w, -1)[:, perm].reshape(v.shape)
    assert (oracle.sparse_attention(q, kp, vp, heads, 2, None, None) - base).abs().max() <= 1e-12
    one = oracle.sparse_attention(q[1:].clone(), k[1:].clone(), v[1:].clone(), heads, 2, None, None)
    assert torch.equal(one, base[1:])


@pytest.mark.parametrize("dt", DTS)
def test_attention_pruned_queries_keep_the_cache(dt):
    n, h, w, heads, d, b = 1, 9, 10, 2, 8, 4
    q, k, v = (_rand((n, h, w, heads * d), dt, 541 + i) for i in range(3))
    cache = _rand((n, h, w, heads * d), dt, 545)
    act = torch.zeros((n, 3, 3), dtype=torch.uint8)
    act[0, 0, 1] = act[0, 2, 2] = 1  # the second includes the clipped corner block
    got = oracle.sparse_attention(q, k, v, heads, b, act, cache)
    dense = oracle.sparse_attention(q, k, v, heads, b, None, None)
    sel = _pixel_block_mask(act, b, h, w)[..., None].expand_as(got)
    assert torch.equal(got[sel].view(torch.uint8), dense[sel].view(torch.uint8))
    assert torch.equal(got[~sel].view(torch.uint8), cache[~sel].view(torch.uint8))
    empty = oracle.sparse_attention(q, k, v, heads, b, torch.zeros_like(act), cache)
    assert torch.equal(empty.view(torch.uint8), cache.view(torch.uint8))


# ---------------------------------------------------------------------------
# the chain
# ---------------------------------------------------------------------------
def _small_chain(dt=torch.bfloat16):
    specs = [(8, 16, 3, 1, 1, 3), (16, 16, 3, 2, 1, 2), (16, 24, 3, 1, 1, 2)]  # (cin, cout, k, s, p, b)
    layers = []
    for li, (cin, cout, k, s, p, b) in enumerate(specs):
        layers.append(dict(weight=_rand((cout, cin, k, k), dt, 200 + li, math.sqrt(2 / (cin * k * k))),
                           bias=_rand((cout,), torch.float32, 210 + li, 0.01), k=k, s=s, p=p, b=b, dilate=1))
    return layers


def _chain_dense_torch(x, layers, dt):
    outs = []
    for L in layers:
        y = _torch_conv_f64(x, L["weight"], L["bias"], L["s"], L["p"])
        x = oracle.round_to(y, dt)
        outs.append(x)
    return outs


def test_chain_all_active_is_dense_chain_and_empty_edit_is_caches():
    dt = torch.bfloat16
    layers = _small_chain(dt)
    a_o = _rand((1, 24, 24, 8), dt, 220)
    caches = _chain_dense_torch(a_o, layers, dt)
    # empty edit: every layer returns its cache bit for bit
    outs = oracle.sparse_chain(a_o, layers, caches, torch.zeros((1, 24, 24), dtype=torch.uint8))
    for o, c in zip(outs, caches):
        assert torch.equal(o.view(torch.int16), c.view(torch.int16))
    # all-active: the dense chain (within one bf16 rounding step per layer)
    a_e = _rand((1, 24, 24, 8), dt, 221)
    outs = oracle.sparse_chain(a_e, layers, caches, torch.ones((1, 24, 24), dtype=torch.uint8))
    dense = _chain_dense_torch(a_e, layers, dt)
    for o, r in zip(outs, dense):
        assert (o.double() - r.double()).abs().max() <= 2 ** -7 * r.double().abs().max()


def test_chain_with_wide_dilation_is_dense_edited_chain():
    # dilation wider than the chain's cumulative halo makes the layer-wise result
    # equal the dense edited chain
    dt = torch.float32
    layers = _small_chain(dt)
    for L in layers:
        L["dilate"] = 3
    a_o = _rand((1, 24, 24, 8), dt, 230)
    m = np.zeros((24, 24), np.uint8)
    m[9:12, 10:13] = 1
    a_e = synth.make_edit(a_o, m, "replace", 231)
    caches = _chain_dense_torch(a_o, layers, dt)
    outs = oracle.sparse_chain(a_e, layers, caches, torch.from_numpy(m)[None])
    dense = _chain_dense_torch(a_e, layers, dt)
    for o, r in zip(outs, dense):
        assert (o.double() - r.double()).abs().max() <= 1e-5 * r.double().abs().max()


# ---------------------------------------------------------------------------
# generators
# ---------------------------------------------------------------------------
def test_generators_are_deterministic_and_hit_the_area():
    g = json.load(open(os.path.join(GOLDEN, "edit_area.json")))
    for seed in range(3):
        m1 = synth.blob_mask(seed, 256, 256, g["area"])
        assert np.array_equal(m1, synth.blob_mask(seed, 256, 256, g["area"]))
        assert abs(m1.mean() - g["area"]) * 100 <= g["tolerance_pp"]
        p1 = synth.polygon_mask(seed, 256, 512, g["area"])
        assert abs(p1.mean() - g["area"]) * 100 <= g["tolerance_pp"]
    a = synth.make_activation(1, 8, 8, 16, "bf16", 7)
    assert torch.equal(a.view(torch.int16), synth.make_activation(1, 8, 8, 16, "bf16", 7).view(torch.int16))

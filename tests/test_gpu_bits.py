"""The change mask packed one bit per pixel (sige_diff_mask_bits) and the block
list reduced from it (sige_reduce_bits, sige_reduce_bits_copy).

Expected values: the oracle's change mask packed on the host (bit p % 32 of
32-bit word p / 32 for pixel p), the oracle's block list, and, bit for bit,
the byte-mask calls on the same inputs: same list, same count, same copy, same
layer output.
"""
import numpy as np
import pytest
import torch

import oracle
import spatially_sparse_incremental_amd as ssi
import synth
from _parity import DT, bits, gpu, layer_inputs, rand, random_mask

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def pack(mask):
    """uint8 [..] (0/1) -> int32 words, bit p % 32 of word p / 32 (host-side packing of a mask)."""
    flat = np.ascontiguousarray(np.asarray(mask, dtype=np.uint8).reshape(-1))
    assert flat.size % 32 == 0
    return torch.from_numpy(np.packbits(flat, bitorder="little").view("<i4").copy())


def _geom(n, h, w, cin, cout, k, s, p, b):
    return ssi.geom(n, h, w, cin, cout, k, s, p, b)


@pytest.mark.parametrize("shape,dts", [((1, 64, 64, 64), "f32"), ((2, 7, 32, 8), "bf16"), ((1, 5, 96, 320), "f16"),
                                       ((3, 2, 32, 16), "f16"), ((1, 256, 256, 128), "bf16")])
def test_diff_bits_against_the_packed_oracle_mask(shape, dts):
    dt = DT[dts]
    n, h, w, c = shape
    print(f"\n[diff bits] {shape} {dts}", flush=True)
    mask = random_mask(n, h, w, 0.1, 191)
    a_o = rand(shape, dt, 192)
    a_e = synth.make_edit(a_o, mask, "replace", 193)
    a_e[0, 0, 0, c - 1] = a_o[0, 0, 0, c - 1] + 1  # a single channel, at the first pixel
    a_e[-1, -1, -1, 0] = a_o[-1, -1, -1, 0] + 1  # and at the last
    ref = oracle.diff_mask(a_o, a_e, 1e-6)
    got = ssi.sige_diff_mask_bits(gpu(a_o), gpu(a_e), 1e-6)  # bits only
    m = torch.full((n, h, w), 7, dtype=torch.uint8, device="cuda")
    got2 = ssi.sige_diff_mask_bits(gpu(a_o), gpu(a_e), 1e-6, mask=m)  # bits and bytes
    torch.cuda.synchronize()
    assert torch.equal(got.cpu(), pack(ref))
    assert torch.equal(got2.cpu(), pack(ref))
    assert torch.equal(m.cpu(), ref)


# (n, h, w, f, k, s, p, b, dilate, frac): mask_w = f * w is a multiple of 32
REDUCE_BITS = [
    (1, 256, 256, 1, 3, 1, 1, 6, 1, 0.002),
    (1, 128, 128, 2, 3, 2, 1, 6, 1, 0.001),
    (1, 32, 32, 8, 3, 1, 1, 4, 1, 0.0005),
    (1, 16, 16, 4, 1, 1, 0, 2, 1, 0.002),
    (1, 32, 32, 3, 3, 1, 1, 4, 1, 0.004),      # fx = 3: pooled pixels straddle bitset words
    (1, 64, 96, 1, 5, 1, 2, 3, 3, 0.001),
    (2, 40, 64, 2, 1, 3, 0, 2, 2, 0.01),       # windows with gaps, two images, pooled
    (3, 32, 32, 1, 3, 1, 1, 1, 0, 0.05),       # three images, 1-pixel blocks
    (1, 256, 512, 1, 3, 1, 1, 6, 1, 0.001),
    (1, 512, 1024, 1, 3, 1, 1, 6, 1, 0.0005),  # pooled bits exceed one workgroup's LDS: two-launch path
    (2, 96, 640, 2, 3, 2, 1, 4, 2, 0.001),     # two-launch path, two images, stride 2, pooled
    (1, 128, 64, 1, 3, 1, 1, 8, 1, 0.3),       # dense edit
]


@pytest.mark.parametrize("case", REDUCE_BITS)
def test_reduce_bits_matches_the_oracle_and_the_byte_mask(case):
    n, h, w, f, k, s, p, b, d, frac = case
    print(f"\n[reduce bits] {case}", flush=True)
    m = random_mask(n, h * f, w * f, frac, 301 + h + w)
    g = _geom(n, h, w, 8, 8, k, s, p, b)
    idx, count = ssi.sige_reduce_bits(gpu(pack(m)), h * f, w * f, g, d)
    bidx, bcount = ssi.sige_reduce_mask(gpu(torch.from_numpy(m)), g, d)
    torch.cuda.synchronize()
    cnt = int(count.item())
    ref = oracle.index_list(oracle.block_activity(torch.from_numpy(m), h, w, k, s, p, b, d))
    assert cnt == ref.numel() == int(bcount.item())
    assert torch.equal(idx[:cnt].cpu(), ref)
    assert torch.equal(idx[:cnt], bidx[:cnt])
    # empty and full masks
    z = np.zeros_like(m)
    idx, count = ssi.sige_reduce_bits(gpu(pack(z)), h * f, w * f, g, d)
    assert int(count.item()) == 0
    idx, count = ssi.sige_reduce_bits(gpu(pack(z + 1)), h * f, w * f, g, d)
    cap = ssi.sige_max_blocks(g)
    assert int(count.item()) == cap
    assert torch.equal(idx[:cap].cpu(), torch.arange(cap, dtype=torch.int32))


@pytest.mark.parametrize("case", [REDUCE_BITS[0], REDUCE_BITS[4], REDUCE_BITS[6], REDUCE_BITS[9]])
def test_reduce_bits_copy(case):
    # the same list as sige_reduce_bits and out == cached bit for bit (one- and two-launch paths)
    n, h, w, f, k, s, p, b, d, frac = case
    print(f"\n[reduce bits+copy] {case}", flush=True)
    wb = gpu(pack(random_mask(n, h * f, w * f, frac, 301 + h + w)))
    cout = 24
    g = _geom(n, h, w, 8, cout, k, s, p, b)
    ho, wo, _, _, _ = oracle.geometry(h, w, k, s, p, b)
    cache = rand((n, ho, wo, cout), torch.bfloat16, 377).cuda()
    ref_idx, ref_cnt = ssi.sige_reduce_bits(wb, h * f, w * f, g, d)
    idx, cnt, out = ssi.sige_reduce_bits_copy(wb, h * f, w * f, g, d, cache)
    torch.cuda.synchronize()
    c = int(cnt.item())
    assert c == int(ref_cnt.item())
    assert torch.equal(idx[:c], ref_idx[:c])
    assert torch.equal(bits(out), bits(cache))


@pytest.mark.parametrize("dts", ["bf16", "f16"])
def test_step_through_the_bitset_equals_the_byte_mask_step(dts):
    # diff_bits -> reduce_bits_copy -> fused conv (copy_cached = 0) ==
    # diff -> reduce -> fused conv (copy_cached = 1), bit for bit
    dt = DT[dts]
    n, h, w, cin, cout, k, s, p, b, d = 1, 64, 96, 64, 48, 3, 1, 1, 6, 1
    mask = random_mask(n, h, w, 0.01, 401)
    a_o, a_e, wt, bias = layer_inputs(n, h, w, cin, cout, k, dt, 402, mask)
    cache = rand((n, h, w, cout), dt, 403).cuda()
    g = _geom(n, h, w, cin, cout, k, s, p, b)
    ao, ae, wk, bs = a_o.cuda(), a_e.cuda(), ssi.weight_to_krsc(wt).cuda(), bias.cuda()
    wb = ssi.sige_diff_mask_bits(ao, ae, 1e-6)
    idx, cnt, out = ssi.sige_reduce_bits_copy(wb, h, w, g, d, cache)
    out = ssi.sige_sparse_conv_layer(ae, wk, bs, None, idx, cnt, g, out=out, copy_cached=False)
    mk = ssi.sige_diff_mask(ao, ae, 1e-6)
    ridx, rcnt = ssi.sige_reduce_mask(mk, g, d)
    ref = ssi.sige_sparse_conv_layer(ae, wk, bs, cache, ridx, rcnt, g)
    torch.cuda.synchronize()
    assert int(cnt.item()) == int(rcnt.item()) > 0
    assert torch.equal(bits(out), bits(ref))

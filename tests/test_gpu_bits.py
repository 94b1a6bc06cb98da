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



def _layers_case(wl, layers, m, seed, copy_mask):
    """One sige_reduce_bits_layers call over `layers` of the workload for the
    change mask m (at the first layer's input): every list against the oracle's
    (bit-exact, pooled from the one mask), nothing written past a count, and
    every copy equal to its cache bit for bit."""
    first = wl.layers[0]
    mbits = pack(m).cuda()
    geoms, dil, idx, cnt, cached, out = [], [], [], [], [], []
    for li, L in enumerate(layers):
        g = ssi.geom(1, L.h, L.w, L.c_in, L.c_out, L.k, L.stride, L.pad, L.block)
        d = ssi.sige_geom_derive(g)
        geoms.append(g)
        dil.append(L.dilate)
        idx.append(torch.full((d.cap,), -7, dtype=torch.int32, device="cuda"))
        cnt.append(torch.full((1,), -7, dtype=torch.int32, device="cuda"))
        dt = synth.DTYPES[L.dtype]
        cached.append(rand((1, d.ho, d.wo, L.c_out), dt, seed * 10 + li).cuda() if copy_mask[li] else None)
        out.append(rand((1, d.ho, d.wo, L.c_out), dt, seed * 10 + li + 5).cuda() if copy_mask[li] else None)
    print(f"\n[case] reduce layers: {len(layers)} layers, {int(m.sum())} changed pixels, seed {seed}", flush=True)
    ssi.sige_reduce_bits_layers(mbits, first.h, first.w, geoms, dil, idx, cnt, cached, out)
    torch.cuda.synchronize()
    for li, L in enumerate(layers):
        act = oracle.block_activity(torch.from_numpy(m).unsqueeze(0), L.h, L.w, L.k, L.stride, L.pad, L.block,
                                    L.dilate)
        ref = oracle.index_list(act)
        k = int(cnt[li].item())
        assert k == ref.numel(), (L.name, k, ref.numel())
        assert torch.equal(idx[li][:k].cpu(), ref.to(torch.int32)), L.name
        assert bool((idx[li][k:] == -7).all()), L.name  # nothing written past the count
        if copy_mask[li]:
            assert torch.equal(bits(out[li].cpu()), bits(cached[li].cpu())), L.name


def test_reduce_layers_builds_every_chain_list_and_copy():
    """All 12 layers of the U-Net chain in one launch at the 1.2% blob; the
    deeper layers at a 5% blob with one layer left without a copy; one layer at
    an empty edit."""
    wl = synth.workload("unet_chain_12conv_bf16")
    first = wl.layers[0]
    m = synth.edit_shape(wl, 5).raster(first.h, first.w)
    _layers_case(wl, wl.layers, m, 5, [True] * 12)
    m5 = synth.edit_shape(wl, 6, 0.05).raster(first.h, first.w)
    _layers_case(wl, wl.layers[5:], m5, 6, [True, True, False, True, True, True, True])
    _layers_case(wl, wl.layers[:1], np.zeros_like(m), 7, [True])


def test_chain_with_all_lists_in_one_launch_equals_the_per_layer_chain():
    """The 12-conv chain run as one diff, one sige_reduce_bits_layers launch and
    12 fused layers equals, at every layer and bit for bit, the chain run with a
    sige_reduce_bits_copy before each layer (itself checked against the oracle
    layer by layer in the full-size workload tests)."""
    wl = synth.workload("unet_chain_12conv_bf16")
    seed = 8
    first = wl.layers[0]
    m = synth.edit_shape(wl, seed).raster(first.h, first.w)
    a_o = synth.make_activation(1, first.h, first.w, first.c_in, first.dtype, seed).cuda()
    a_e = synth.make_edit(a_o.cpu(), m, wl.edit_kind, seed).cuda()
    mbits = ssi.sige_diff_mask_bits(a_o, a_e, wl.tau)
    lay = []
    for li, L in enumerate(wl.layers):
        wt, bias = synth.make_layer_tensors(L, seed * 100 + li)
        g = ssi.geom(1, L.h, L.w, L.c_in, L.c_out, L.k, L.stride, L.pad, L.block)
        d = ssi.sige_geom_derive(g)
        cache = synth.make_activation(1, d.ho, d.wo, L.c_out, L.dtype, seed * 100 + li + 50).cuda()
        lay.append(dict(L=L, g=g, wk=ssi.weight_to_krsc(wt).cuda(), bias=bias.cuda(), cache=cache, cap=d.cap))

    def run(batched):
        idx = [torch.empty((ly["cap"],), dtype=torch.int32, device="cuda") for ly in lay]
        cnt = [torch.empty((1,), dtype=torch.int32, device="cuda") for ly in lay]
        out = [torch.empty_like(ly["cache"]) for ly in lay]
        if batched:
            ssi.sige_reduce_bits_layers(mbits, first.h, first.w, [ly["g"] for ly in lay],
                                        [ly["L"].dilate for ly in lay], idx, cnt, [ly["cache"] for ly in lay], out)
        x = a_e
        for i, ly in enumerate(lay):
            if not batched:
                ssi.sige_reduce_bits_copy(mbits, first.h, first.w, ly["g"], ly["L"].dilate, ly["cache"], out=out[i],
                                          idx=idx[i], count=cnt[i])
            ssi.sige_sparse_conv_layer(x, ly["wk"], ly["bias"], None, idx[i], cnt[i], ly["g"], out=out[i],
                                       copy_cached=False)
            x = out[i]
        torch.cuda.synchronize()
        return [o.cpu() for o in out], [int(c.item()) for c in cnt]

    print(f"\n[case] chain, lists in one launch vs per layer, seed {seed}", flush=True)
    ref, ref_cnt = run(False)
    got, got_cnt = run(True)
    assert got_cnt == ref_cnt
    for li in range(len(lay)):
        assert torch.equal(bits(got[li]), bits(ref[li])), wl.layers[li].name

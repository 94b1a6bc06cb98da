"""The fused layer split over input channels (sige_sparse_conv_layer_split)
against the oracle: the latent-diffusion layers of the workload (few blocks,
640-1280 channels, where the split engages), every low-resolution point of
the block-size sweep, small shapes that force either a split or one range per
tile, the persistent-buffer mode, an empty edit, repeated calls and graph
replays.

Expected values: the oracle (listed pixels within tolerance, every other pixel
equal to the cache bit for bit) and, for repeated calls and replays, the
first result bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import spatially_sparse_incremental_amd as ssi
import synth
from _parity import DT, active_pixels, assert_close, bits, check_layer_sampled, layer_inputs, rand, random_mask
from _parity import run_layer_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _split_full(a_e, wt, bias, cache, L, mask):
    g = ssi.geom(1, L.h, L.w, L.c_in, L.c_out, L.k, L.stride, L.pad, L.block)
    idx, cnt = ssi.sige_reduce_mask(mask, g, L.dilate)
    out = ssi.sige_sparse_conv_layer_split(a_e, ssi.weight_to_krsc(wt).cuda(), bias.cuda(), cache, idx, cnt, g)
    torch.cuda.synchronize()
    return out, idx[:int(cnt.item())].cpu()


LDM = [L for L in synth.workload("ldm_64x64x320_f16").layers if L.h <= 32]
LOWRES = [L for w, L in synth.SWEEP if w == "ldm_64x64x320_f16"]


@pytest.mark.parametrize("area", [0.012, 0.10])
@pytest.mark.parametrize("L", LDM, ids=[L.name for L in LDM])
def test_split_ldm_layers(L, area):
    wl = synth.workload("ldm_64x64x320_f16")
    seed = 3
    m = synth.edit_shape(wl, seed, area).raster(L.h, L.w)
    a_o = synth.make_activation(1, L.h, L.w, L.c_in, L.dtype, seed)
    a_e = synth.make_edit(a_o, m, wl.edit_kind, seed)
    wt, bias = synth.make_layer_tensors(L, seed)
    cache = synth.make_activation(1, L.h, L.w, L.c_out, L.dtype, seed + 50)
    mask = ssi.sige_diff_mask(a_o.cuda(), a_e.cuda(), wl.tau)
    out, idx = _split_full(a_e.cuda(), wt, bias, cache.cuda(), L, mask)
    print(f"\n[case] {L.name} area {area}: {idx.numel()} blocks", flush=True)
    check_layer_sampled(L.name, a_e, wt, bias, cache, out.cpu(), idx, L, mask.cpu(), seed, sample=10)


@pytest.mark.parametrize("L", LOWRES, ids=[L.name for L in LOWRES])
def test_split_sweep_points(L):
    wl = synth.workload("ldm_64x64x320_f16")
    seed = 9
    m = synth.edit_shape(wl, seed).raster(L.h, L.w)
    a_o = synth.make_activation(1, L.h, L.w, L.c_in, L.dtype, seed)
    a_e = synth.make_edit(a_o, m, wl.edit_kind, seed)
    wt, bias = synth.make_layer_tensors(L, seed)
    cache = synth.make_activation(1, L.h, L.w, L.c_out, L.dtype, seed + 50)
    mask = ssi.sige_diff_mask(a_o.cuda(), a_e.cuda(), wl.tau)
    out, idx = _split_full(a_e.cuda(), wt, bias, cache.cuda(), L, mask)
    print(f"\n[case] {L.name}: {idx.numel()} blocks", flush=True)
    check_layer_sampled(L.name, a_e, wt, bias, cache, out.cpu(), idx, L, mask.cpu(), seed)


# (name, n, h, w, cin, cout, k, s, p, b, dtype, dilate, edit fraction): a split
# over many channels with a handful of blocks; a ragged stride-2 case; fp32 and
# bf16; many tiles (one range per tile); a two-image batch
SMALL = [
    ("split_f16", 1, 12, 12, 512, 256, 3, 1, 1, 4, "f16", 0, 0.02),
    ("split_stride2_bf16", 1, 15, 13, 384, 96, 3, 2, 1, 3, "bf16", 1, 0.03),
    ("split_f32", 1, 10, 10, 256, 64, 3, 1, 1, 4, "f32", 0, 0.03),
    ("split_1x1_f16", 1, 16, 16, 1024, 512, 1, 1, 0, 2, "f16", 1, 0.02),
    ("many_tiles_bf16", 1, 64, 64, 64, 64, 3, 1, 1, 4, "bf16", 1, 0.2),
    ("two_images_f16", 2, 12, 14, 320, 160, 3, 1, 1, 4, "f16", 1, 0.03),
]


@pytest.mark.parametrize("copy", [True, False], ids=["copy", "persistent"])
@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_split_small_shapes_against_oracle(case, copy):
    name, n, h, w, cin, cout, k, s, p, b, dts, d, frac = case
    dt = DT[dts]
    print(f"\n[case] {name} copy={copy}", flush=True)
    mask = random_mask(n, h, w, frac, 17)
    a_o, a_e, wt, bias = layer_inputs(n, h, w, cin, cout, k, dt, 21, mask)
    ho, wo, _, _, _ = oracle.geometry(h, w, k, s, p, b)
    cache = rand((n, ho, wo, cout), dt, 23)
    base = rand((n, ho, wo, cout), dt, 24)
    g = ssi.geom(n, h, w, cin, cout, k, s, p, b)
    ao, ae, wk, bs, cg = a_o.cuda(), a_e.cuda(), ssi.weight_to_krsc(wt).cuda(), bias.cuda(), cache.cuda()
    mk = ssi.sige_diff_mask(ao, ae, 1e-6)
    idx, cnt = ssi.sige_reduce_mask(mk, g, d)
    out = None if copy else base.cuda()
    out = ssi.sige_sparse_conv_layer_split(ae, wk, bs, cg if copy else None, idx, cnt, g, out=out, copy_cached=copy)
    torch.cuda.synchronize()
    ref = run_layer_oracle(a_o, a_e, wt, bias, cache, k, s, p, b, d)
    assert torch.equal(idx[:int(cnt.item())].cpu(), ref["idx"])
    sel = active_pixels(ref["act"], b, ho, wo)
    keep = ~sel.expand_as(cache)
    expect = cache if copy else base
    assert torch.equal(out.cpu()[keep].view(torch.uint8), expect[keep].view(torch.uint8))
    assert_close(out.cpu(), ref["out64"], dt, sel, name)


def test_split_is_deterministic_and_empty_edit_keeps_the_cache():
    n, h, w, cin, cout, b = 1, 12, 12, 512, 256, 4
    dt = torch.float16
    mask = random_mask(n, h, w, 0.03, 31)
    a_o, a_e, wt, bias = layer_inputs(n, h, w, cin, cout, 3, dt, 32, mask)
    cache = rand((n, h, w, cout), dt, 33).cuda()
    g = ssi.geom(n, h, w, cin, cout, 3, 1, 1, b)
    ao, ae, wk, bs = a_o.cuda(), a_e.cuda(), ssi.weight_to_krsc(wt).cuda(), bias.cuda()
    idx, cnt = ssi.sige_reduce_mask(ssi.sige_diff_mask(ao, ae, 1e-6), g, 1)
    ws = torch.empty(ssi.sige_sparse_conv_layer_split_workspace(g, dt), dtype=torch.uint8, device="cuda")
    first = ssi.sige_sparse_conv_layer_split(ae, wk, bs, cache, idx, cnt, g, workspace=ws)
    for _ in range(5):
        again = ssi.sige_sparse_conv_layer_split(ae, wk, bs, cache, idx, cnt, g, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(bits(again), bits(first))
    zero = torch.zeros(1, dtype=torch.int32, device="cuda")
    empty = ssi.sige_sparse_conv_layer_split(ae, wk, bs, cache, idx, zero, g, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(bits(empty), bits(cache))


def test_split_graph_replays_match_eager():
    n, h, w, cin, cout, b = 1, 16, 16, 640, 320, 4
    dt = torch.float16
    a_o = rand((n, h, w, cin), dt, 41).cuda()
    a_e = a_o.clone()
    wt = rand((cout, cin, 3, 3), dt, 42, (2.0 / (9 * cin)) ** 0.5)
    wk, bs = ssi.weight_to_krsc(wt).cuda(), rand((cout,), torch.float32, 43, 0.01).cuda()
    cache = rand((n, h, w, cout), dt, 44).cuda()
    g = ssi.geom(n, h, w, cin, cout, 3, 1, 1, b)
    d = ssi.sige_geom_derive(g)
    m = torch.empty((n, h, w), dtype=torch.uint8, device="cuda")
    idx = torch.empty((d.cap,), dtype=torch.int32, device="cuda")
    cnt = torch.empty((1,), dtype=torch.int32, device="cuda")
    out = torch.empty_like(cache)
    ws = torch.empty(ssi.sige_sparse_conv_layer_split_workspace(g, dt), dtype=torch.uint8, device="cuda")

    def step():
        ssi.sige_diff_mask(a_o, a_e, 1e-6, mask=m)
        ssi.sige_reduce_mask(m, g, 1, idx=idx, count=cnt)
        ssi.sige_sparse_conv_layer_split(a_e, wk, bs, cache, idx, cnt, g, out=out, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    rng = np.random.default_rng(45)
    for rep in range(4):
        mk = (rng.random((n, h, w)) < 0.03).astype(np.uint8)
        a_e.copy_(synth.make_edit(a_o.cpu(), mk, "replace", 46 + rep).cuda())
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        print(f"[case] replay {rep}: {int(cnt.item())} blocks", flush=True)
        out.zero_()
        step()
        torch.cuda.synchronize()
        assert torch.equal(bits(got), bits(out)), rep


@pytest.mark.parametrize("area", [0.005, 0.012, 0.05, 0.15, 0.30])
def test_split_gaugan_layers(area):
    # the four GauGAN-shaped bf16 convs (18.9 MB of weights at 32x64x1024): list and
    # untouched pixels bit for bit, sampled blocks against the oracle, and every
    # listed pixel against the single-range layer (an independently written kernel
    # that the oracle checks on the same layers) within the bf16 tolerance
    wl = synth.workload("gaugan_4conv_bf16")
    seed = 6
    shape = synth.edit_shape(wl, seed, area)
    for li, L in enumerate(wl.layers):
        m = shape.raster(L.h, L.w)
        a_o = synth.make_activation(1, L.h, L.w, L.c_in, L.dtype, seed + li)
        a_e = synth.make_edit(a_o, m, wl.edit_kind, seed + li)
        wt, bias = synth.make_layer_tensors(L, seed + li)
        cache = synth.make_activation(1, L.h, L.w, L.c_out, L.dtype, seed + li + 50)
        mask = ssi.sige_diff_mask(a_o.cuda(), a_e.cuda(), wl.tau)
        out, idx = _split_full(a_e.cuda(), wt, bias, cache.cuda(), L, mask)
        print(f"\n[case] gaugan split {L.name} area {area}: {idx.numel()} blocks", flush=True)
        check_layer_sampled(f"gaugan split {L.name} area {area}", a_e, wt, bias, cache, out.cpu(), idx, L,
                            mask.cpu(), li, sample=None if area <= 0.012 else 10)
        g = ssi.geom(1, L.h, L.w, L.c_in, L.c_out, L.k, L.stride, L.pad, L.block)
        i2, c2 = ssi.sige_reduce_mask(mask, g, L.dilate)
        single = ssi.sige_sparse_conv_layer(a_e.cuda(), ssi.weight_to_krsc(wt).cuda(), bias.cuda(), cache.cuda(),
                                            i2, c2, g).cpu()
        act = torch.zeros(1, *oracle.geometry(L.h, L.w, L.k, L.stride, L.pad, L.block)[2:4], dtype=torch.uint8)
        act.view(-1)[idx.long()] = 1
        sel = active_pixels(act, L.block, L.h, L.w).expand_as(out)
        assert_close(out.cpu(), single.double(), out.dtype, sel, f"gaugan split vs single {L.name} area {area}")


def test_split_unet_chain_12conv_layerwise():
    """The split on every layer of the 12-conv U-Net chain (stride-1 and stride-2
    layers, 128 to 512 channels), layer by layer as the chain runs: the bench
    times the faster of the two layer kernels per layer of this chain."""
    wl = synth.workload("unet_chain_12conv_bf16")
    seed = 4
    first = wl.layers[0]
    m = synth.edit_shape(wl, seed).raster(first.h, first.w)
    a_o = synth.make_activation(1, first.h, first.w, first.c_in, first.dtype, seed)
    a_e = synth.make_edit(a_o, m, wl.edit_kind, seed)
    mask = ssi.sige_diff_mask(a_o.cuda(), a_e.cuda(), wl.tau)  # one diff at 256x256, pooled per layer
    x = a_e.cuda()
    for li, L in enumerate(wl.layers):
        wt, bias = synth.make_layer_tensors(L, seed * 100 + li)
        ho, wo, _, _, _ = oracle.geometry(L.h, L.w, L.k, L.stride, L.pad, L.block)
        cache = synth.make_activation(1, ho, wo, L.c_out, L.dtype, seed * 100 + li + 50)
        out, idx = _split_full(x, wt, bias, cache.cuda(), L, mask)
        print(f"\n[case] chain split {L.name}: {idx.numel()} blocks", flush=True)
        check_layer_sampled(f"chain split {L.name}", x.cpu(), wt, bias, cache, out.cpu(), idx, L, mask.cpu(),
                            seed + li)
        x = out  # layer l+1 takes layer l's edited output

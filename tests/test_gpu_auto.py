"""The layer entry point that picks its kernel (sige_sparse_conv_layer_auto):
every chain, GauGAN and latent-diffusion layer against the oracle, and bit for
bit against the kernel the plan names for the list length (the other kernel
must leave `out` alone, cache copy included)."""
import pytest
import torch

import oracle
import spatially_sparse_incremental_amd as ssi
import synth
from synth.gen import DTYPES
from _parity import active_pixels, assert_close, check_layer_sampled, run_layer_full

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _check_choice(name, a_e_gpu, wt, bias, cache_gpu, L, mask_gpu, out):
    """`out` (auto) equals, bit for bit, the kernel the plan picks for this list;
    the wide tiles (no entry point of their own) equal the single-range kernel
    within the dtype's tolerance, and bit for bit outside the listed blocks."""
    g = ssi.geom(1, L.h, L.w, L.c_in, L.c_out, L.k, L.stride, L.pad, L.block)
    plan = ssi.sige_sparse_conv_layer_plan(g, DTYPES[L.dtype])
    assert -1 <= plan.split_max <= plan.cap == ssi.sige_max_blocks(g)
    assert plan.split_max < plan.wide_min <= plan.wide_max
    idx, count = ssi.sige_reduce_mask(mask_gpu, g, L.dilate)
    n = int(count.item())
    wk = ssi.weight_to_krsc(wt).cuda()
    path = "split" if n <= plan.split_max else ("wide" if plan.wide_min <= n <= plan.wide_max else "single")
    if path == "split":
        ref = ssi.sige_sparse_conv_layer_split(a_e_gpu, wk, bias.cuda(), cache_gpu, idx, count, g)
    else:
        ref = ssi.sige_sparse_conv_layer(a_e_gpu, wk, bias.cuda(), cache_gpu, idx, count, g)
    torch.cuda.synchronize()
    if path != "wide":
        assert torch.equal(out.view(torch.uint8), ref.view(torch.uint8)), f"{name}: auto differs from the {path} kernel"
    else:
        d = ssi.sige_geom_derive(g)
        act = torch.zeros(d.nby * d.nbx, dtype=torch.uint8)
        act[idx[:n].long().cpu()] = 1
        sel = active_pixels(act.view(1, d.nby, d.nbx), L.block, d.ho, d.wo).expand_as(out.cpu())
        o, r = out.cpu(), ref.cpu()
        assert torch.equal(o[~sel].view(torch.uint8), r[~sel].view(torch.uint8)), f"{name}: untouched pixels"
        assert_close(o, r.double(), o.dtype, sel, f"{name}: wide tiles against the single-range kernel")
    return path


@pytest.mark.parametrize("area", [0.005, 0.012, 0.15])
def test_auto_unet_chain_every_layer(area):
    wl = synth.workload("unet_chain_12conv_bf16")
    seed = 3
    first = wl.layers[0]
    m = synth.edit_shape(wl, seed, area).raster(first.h, first.w)
    a_o = synth.make_activation(1, first.h, first.w, first.c_in, first.dtype, seed)
    a_e = synth.make_edit(a_o, m, wl.edit_kind, seed)
    mask = ssi.sige_diff_mask(a_o.cuda(), a_e.cuda(), wl.tau)
    x = a_e.cuda()
    paths = []
    for li, L in enumerate(wl.layers):
        wt, bias = synth.make_layer_tensors(L, seed * 100 + li)
        ho, wo, _, _, _ = oracle.geometry(L.h, L.w, L.k, L.stride, L.pad, L.block)
        cache = synth.make_activation(1, ho, wo, L.c_out, L.dtype, seed * 100 + li + 50)
        out, idx = run_layer_full(x, wt, bias, cache.cuda(), L, mask, layer=ssi.sige_sparse_conv_layer_auto)
        check_layer_sampled(f"auto chain {L.name} area {area}", x.cpu(), wt, bias, cache, out.cpu(), idx, L,
                            mask.cpu(), seed + li, sample=None if area <= 0.012 else 8)
        paths.append(_check_choice(f"auto chain {L.name}", x, wt, bias, cache.cuda(), L, mask, out))
        x = out
    print(f"chain area {area}: {paths}")


@pytest.mark.parametrize("area", [0.005, 0.05, 0.30])
def test_auto_gaugan_layers(area):
    wl = synth.workload("gaugan_4conv_bf16")
    seed = 4
    shape = synth.edit_shape(wl, seed, area)
    for li, L in enumerate(wl.layers):
        m = shape.raster(L.h, L.w)
        a_o = synth.make_activation(1, L.h, L.w, L.c_in, L.dtype, seed + li)
        a_e = synth.make_edit(a_o, m, wl.edit_kind, seed + li)
        wt, bias = synth.make_layer_tensors(L, seed + li)
        cache = synth.make_activation(1, L.h, L.w, L.c_out, L.dtype, seed + li + 50)
        mask = ssi.sige_diff_mask(a_o.cuda(), a_e.cuda(), wl.tau)
        out, idx = run_layer_full(a_e.cuda(), wt, bias, cache.cuda(), L, mask, layer=ssi.sige_sparse_conv_layer_auto)
        check_layer_sampled(f"auto gaugan {L.name} area {area}", a_e, wt, bias, cache, out.cpu(), idx, L,
                            mask.cpu(), li, sample=None if area <= 0.012 else 8)
        _check_choice(f"auto gaugan {L.name}", a_e.cuda(), wt, bias, cache.cuda(), L, mask, out)


@pytest.mark.parametrize("area", [0.012, 0.30])
def test_auto_latent_diffusion_layers(area):
    wname = "ldm_64x64x320_f16"
    wl = synth.workload(wname)
    seed = 5
    shape = synth.edit_shape(wl, seed, area)
    for li, L in enumerate(wl.layers):
        m = shape.raster(L.h, L.w)
        a_o = synth.make_activation(1, L.h, L.w, L.c_in, L.dtype, seed + li)
        a_e = synth.make_edit(a_o, m, wl.edit_kind, seed + li)
        wt, bias = synth.make_layer_tensors(L, seed + li)
        cache = synth.make_activation(1, L.h, L.w, L.c_out, L.dtype, seed + li + 50)
        mask = ssi.sige_diff_mask(a_o.cuda(), a_e.cuda(), wl.tau)
        out, idx = run_layer_full(a_e.cuda(), wt, bias, cache.cuda(), L, mask, layer=ssi.sige_sparse_conv_layer_auto)
        check_layer_sampled(f"auto {wname} {L.name} area {area}", a_e, wt, bias, cache, out.cpu(), idx, L,
                            mask.cpu(), li)
        _check_choice(f"auto {wname} {L.name}", a_e.cuda(), wt, bias, cache.cuda(), L, mask, out)


def test_auto_persistent_buffer_and_empty_list():
    """copy_cached = 0 writes only the listed blocks; an empty list writes nothing
    (copy_cached = 0) or the cache (copy_cached = 1), on every side of the plan
    (bit for bit against the kernel the plan names; the wide tiles against the
    single-range kernel within tolerance on the listed blocks, bit for bit
    elsewhere)."""
    L = synth.workload("gaugan_4conv_bf16").layers[1]  # 64x128x1024 -> 512: the plan uses both kernels
    g = ssi.geom(1, L.h, L.w, L.c_in, L.c_out, L.k, L.stride, L.pad, L.block)
    plan = ssi.sige_sparse_conv_layer_plan(g, DTYPES[L.dtype])
    assert 0 <= plan.split_max < plan.cap, "this layer should exercise both gated kernels"
    wt, bias = synth.make_layer_tensors(L, 9)
    wk = ssi.weight_to_krsc(wt).cuda()
    a = synth.make_activation(1, L.h, L.w, L.c_in, L.dtype, 9).cuda()
    cache = synth.make_activation(1, L.h, L.w, L.c_out, L.dtype, 10).cuda()
    cap = plan.cap
    d = ssi.sige_geom_derive(g)
    lengths = sorted({0, 1, plan.split_max, plan.split_max + 1, min(plan.wide_min - 1, cap), min(plan.wide_min, cap),
                      cap})
    for n in lengths:
        idx = torch.arange(cap, dtype=torch.int32, device="cuda")  # ascending, the first n listed
        count = torch.tensor([n], dtype=torch.int32, device="cuda")
        wide = plan.wide_min <= n <= plan.wide_max
        act = torch.zeros(cap, dtype=torch.uint8)
        act[:n] = 1
        sel = active_pixels(act.view(1, d.nby, d.nbx), L.block, d.ho, d.wo).expand_as(cache.cpu())

        def same(got, ref, what):
            o, r = got.cpu(), ref.cpu()
            if not wide:
                assert torch.equal(o.view(torch.uint8), r.view(torch.uint8)), what
                return
            assert torch.equal(o[~sel].view(torch.uint8), r[~sel].view(torch.uint8)), what + ": untouched pixels"
            assert_close(o, r.double(), o.dtype, sel, what + ": wide tiles against the single-range kernel")

        sentinel = torch.full_like(cache, 7.0)
        got = ssi.sige_sparse_conv_layer_auto(a, wk, bias.cuda(), None, idx, count, g, out=sentinel.clone(),
                                              copy_cached=False)
        ref_fn = ssi.sige_sparse_conv_layer_split if n <= plan.split_max else ssi.sige_sparse_conv_layer
        ref = ref_fn(a, wk, bias.cuda(), None, idx, count, g, out=sentinel.clone(), copy_cached=False)
        torch.cuda.synchronize()
        same(got, ref, f"copy_cached=0, {n} blocks")
        got = ssi.sige_sparse_conv_layer_auto(a, wk, bias.cuda(), cache, idx, count, g)
        ref = ref_fn(a, wk, bias.cuda(), cache, idx, count, g)
        torch.cuda.synchronize()
        same(got, ref, f"copy_cached=1, {n} blocks")
        if n == 0:
            assert torch.equal(got.view(torch.uint8), cache.view(torch.uint8))


# (name, n, h, w, cin, cout, k, s, p, b, dtype, dilate, edit fraction): small shapes with
# ragged tiles, two images, stride 2, 1x1 and 5x5 kernels, fp32
SMALL = [
    ("f32_nhwc", 1, 64, 64, 64, 64, 3, 1, 1, 8, "f32", 0, 0.01),
    ("two_images_bf16", 2, 13, 17, 40, 24, 3, 1, 1, 4, "bf16", 1, 0.02),
    ("stride2_f16", 1, 30, 26, 32, 48, 3, 2, 1, 3, "f16", 1, 0.02),
    ("pointwise_f16", 1, 20, 20, 320, 64, 1, 1, 0, 4, "f16", 1, 0.02),
    ("k5_f32", 1, 19, 23, 16, 16, 5, 1, 2, 3, "f32", 0, 0.02),
    ("deep_small_f16", 1, 16, 16, 640, 640, 3, 1, 1, 2, "f16", 1, 0.05),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_auto_small_shapes_against_the_oracle(case):
    from _parity import DT, active_pixels, assert_close, bits, layer_inputs, rand, random_mask, run_layer_oracle
    name, n, h, w, cin, cout, k, s, p, b, dts, d, frac = case
    dt = DT[dts]
    mask = random_mask(n, h, w, frac, 17)
    a_o, a_e, wt, bias = layer_inputs(n, h, w, cin, cout, k, dt, 18, mask)
    ho, wo, _, _, _ = oracle.geometry(h, w, k, s, p, b)
    cache = rand((n, ho, wo, cout), dt, 19)
    g = ssi.geom(n, h, w, cin, cout, k, s, p, b)
    ref = run_layer_oracle(a_o, a_e, wt, bias, cache, k, s, p, b, d)
    plan = ssi.sige_sparse_conv_layer_plan(g, dt)
    ae, wk, bs, cg = a_e.cuda(), ssi.weight_to_krsc(wt).cuda(), bias.cuda(), cache.cuda()
    idx, count = ssi.sige_reduce_mask(ssi.sige_diff_mask(a_o.cuda(), ae, 1e-6), g, d)
    out = ssi.sige_sparse_conv_layer_auto(ae, wk, bs, cg, idx, count, g)
    torch.cuda.synchronize()
    cnt = int(count.item())
    assert torch.equal(idx[:cnt].cpu(), ref["idx"]) and cnt > 0
    sel = active_pixels(ref["act"], b, ho, wo)
    keep = ~sel.expand_as(cache)
    assert torch.equal(out.cpu()[keep].view(torch.uint8), cache[keep].view(torch.uint8))
    assert_close(out.cpu(), ref["out64"], dt, sel, f"auto {name}")
    fn = ssi.sige_sparse_conv_layer_split if cnt <= plan.split_max else ssi.sige_sparse_conv_layer
    chosen = fn(ae, wk, bs, cg, idx, count, g)
    torch.cuda.synchronize()
    assert torch.equal(bits(out.cpu()), bits(chosen.cpu())), f"{name}: auto differs from the planned kernel"

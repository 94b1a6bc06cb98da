"""The single-range layer kernel with its weights packed in load order
(sige_pack_weights, sige_sparse_conv_layer_packed, sige_conv_blocks_packed)
against the same kernel on
the KRSC weights, bit for bit: the packed copy holds exactly the 16 bytes each
lane would load from the KRSC weights (clamped columns and channels included),
so every MFMA sees the same operands in the same order.  Geometries: 16-bit
32x32 MFMAs and fp32 16x16 ones, 16-column tiles (7x7 kernels), two K chunks
with a partial second one (c_in = 200), a partial last N tile (c_out = 136,
40), stride 2, two images; lists of 0, 1, a third and every block, with and
without the cache copy; the pack's writes stay inside its buffer; and the
bench's layer (256x256x128 bf16, 1.2% blob) at full size, also against the
oracle on sampled blocks."""
import pytest
import torch

import oracle
import spatially_sparse_incremental_amd as ssi
from _parity import DT, active_pixels, assert_close, layer_inputs, rand, random_mask

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# (name, n, h, w, cin, cout, k, s, p, b, dtype)
CASES = [
    ("bf16_3x3_b6", 1, 40, 44, 128, 128, 3, 1, 1, 6, "bf16"),
    ("f16_cin200_cout136_two_chunks", 1, 40, 44, 200, 136, 3, 1, 1, 6, "f16"),
    ("f32_b8_16x16_mfma", 1, 36, 36, 64, 64, 3, 1, 1, 8, "f32"),
    ("bf16_5x5_cout40", 1, 30, 30, 48, 40, 5, 1, 2, 4, "bf16"),
    ("bf16_7x7_16_column_tiles", 1, 30, 30, 32, 48, 7, 1, 3, 4, "bf16"),
    ("f16_stride2", 1, 33, 35, 64, 96, 3, 2, 1, 4, "f16"),
    ("bf16_two_images", 2, 30, 30, 32, 64, 3, 1, 1, 4, "bf16"),
]


def _pack_guarded(wk, g):
    need = ssi.sige_packed_weights_bytes(g, wk.dtype)
    buf = torch.full((need + 4096,), 0x5A, dtype=torch.uint8, device="cuda")
    wp = ssi.sige_pack_weights(wk, g, out=buf[:need])
    torch.cuda.synchronize()
    assert (buf[need:] == 0x5A).all(), "writes past the packed copy"
    return wp


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_packed_single_range_layer_equals_krsc(case):
    name, n, h, w, cin, cout, k, s, p, b, dts = case
    dt = DT[dts]
    g = ssi.geom(n, h, w, cin, cout, k, s, p, b)
    ho, wo, nby, nbx, _ = oracle.geometry(h, w, k, s, p, b)
    cap = n * nby * nbx
    mask = random_mask(n, h, w, 0.5, 91)
    _, a_e, wt, bias = layer_inputs(n, h, w, cin, cout, k, dt, 93, mask)
    cache = rand((n, ho, wo, cout), dt, 95).cuda()
    ag, wk, bg = a_e.cuda(), ssi.weight_to_krsc(wt).cuda(), bias.cuda()
    wp = _pack_guarded(wk, g)
    gen = torch.Generator().manual_seed(97)
    for cnt in sorted({0, 1, max(1, cap // 3), cap}):
        lst = torch.randperm(cap, generator=gen)[:cnt].sort().values.to(torch.int32)
        idx = torch.zeros(cap, dtype=torch.int32)
        idx[:cnt] = lst
        idx, count = idx.cuda(), torch.tensor([cnt], dtype=torch.int32, device="cuda")
        print(f"[case] {name}: {cnt} of {cap} blocks", flush=True)
        for copy in (True, False):
            o1, o2 = cache.clone(), cache.clone()
            ssi.sige_sparse_conv_layer(ag, wk, bg, cache if copy else None, idx, count, g, out=o1, copy_cached=copy)
            ssi.sige_sparse_conv_layer(ag, wk, bg, cache if copy else None, idx, count, g, out=o2, copy_cached=copy,
                                       w_packed=wp)
            assert torch.equal(o1.view(torch.uint8), o2.view(torch.uint8)), f"{name} {cnt} blocks copy={copy}"
        # the three-call path's block convolution on the same list
        blocks = ssi.sige_gather(ag, g, idx, count)
        b1 = ssi.sige_conv_blocks(blocks, wk, bg, g, count)
        b2 = ssi.sige_conv_blocks(blocks, wk, bg, g, count, w_packed=wp)
        torch.cuda.synchronize()
        assert torch.equal(b1[:cnt].view(torch.uint8), b2[:cnt].view(torch.uint8)), f"{name} {cnt} blocks: conv_blocks"


def test_packed_bench_layer_at_full_size():
    """The bench's layer and edit (256x256x128 bf16, 1.2% blob, 74 blocks) and
    every block listed: packed equals KRSC bit for bit; the packed result equals
    the oracle on sampled blocks."""
    import synth

    wl = synth.workload("unet_256x256x128_bf16")
    L = wl.layers[0]
    g = ssi.geom(1, L.h, L.w, L.c_in, L.c_out, L.k, L.stride, L.pad, L.block)
    a_o = synth.make_activation(1, L.h, L.w, L.c_in, L.dtype, 1)
    a_e = synth.make_edit(a_o, synth.edit_shape(wl, 1).raster(L.h, L.w), wl.edit_kind, 1)
    wt, bias = synth.make_layer_tensors(L, 1)
    cache = synth.make_activation(1, L.h, L.w, L.c_out, L.dtype, 51)
    ag, ao, wk, bg, cg = a_e.cuda(), a_o.cuda(), ssi.weight_to_krsc(wt).cuda(), bias.cuda(), cache.cuda()
    wp = _pack_guarded(wk, g)
    idx, count = ssi.sige_reduce_mask(ssi.sige_diff_mask(ao, ag, wl.tau), g, L.dilate)
    cnt = int(count.item())
    assert 60 <= cnt <= 90
    o1 = ssi.sige_sparse_conv_layer(ag, wk, bg, cg, idx, count, g)
    o2 = ssi.sige_sparse_conv_layer(ag, wk, bg, cg, idx, count, g, w_packed=wp)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.uint8), o2.view(torch.uint8)), "1.2% edit"
    ho, wo, nby, nbx, _ = oracle.geometry(L.h, L.w, L.k, L.stride, L.pad, L.block)
    lst = idx[:cnt].cpu()
    sub = torch.zeros(nby * nbx, dtype=torch.uint8)
    sub[lst[torch.randperm(cnt, generator=torch.Generator().manual_seed(5))[:6]].long()] = 1
    sub = sub.view(1, nby, nbx)
    out = o2.cpu()
    r64 = oracle.sparse_layer(a_e, wt, bias, L.k, L.stride, L.pad, L.block, sub, out, out_f64=True)
    assert_close(out, r64, torch.bfloat16, active_pixels(sub, L.block, ho, wo), "packed, sampled blocks")
    cap = nby * nbx
    idx_all = torch.arange(cap, dtype=torch.int32, device="cuda")
    c_all = torch.tensor([cap], dtype=torch.int32, device="cuda")
    o1 = ssi.sige_sparse_conv_layer(ag, wk, bg, cg, idx_all, c_all, g)
    o2 = ssi.sige_sparse_conv_layer(ag, wk, bg, cg, idx_all, c_all, g, w_packed=wp)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.uint8), o2.view(torch.uint8)), "every block"


@pytest.mark.parametrize("workload,layer", [("ldm_64x64x320_f16", "l16_3x3"), ("ldm_64x64x320_f16", "l32_1x1"),
                                            ("gaugan_4conv_bf16", "g32x64"), ("unet_chain_12conv_bf16", "L32_down"),
                                            ("unet_chain_12conv_bf16", "L128_down")])
def test_packed_split_equals_krsc(workload, layer):
    """Lists the library's plan gives to the split (the low-resolution,
    weight-bound layers; stride 2; 1x1): sige_sparse_conv_layer_auto_packed
    (the split's weight fragments from the packed copy) equals the KRSC call
    bit for bit, with and without the copy, and the oracle on sampled blocks."""
    import synth

    L = [x for x in synth.workload(workload).layers if x.name == layer][0]
    dt = DT[L.dtype]
    g = ssi.geom(1, L.h, L.w, L.c_in, L.c_out, L.k, L.stride, L.pad, L.block)
    plan = ssi.sige_sparse_conv_layer_plan(g, dt)
    assert plan.split_max >= 1, plan.as_dict()
    ho, wo, nby, nbx, _ = oracle.geometry(L.h, L.w, L.k, L.stride, L.pad, L.block)
    a_e = synth.make_activation(1, L.h, L.w, L.c_in, L.dtype, 101)
    wt, bias = synth.make_layer_tensors(L, 103)
    cache = synth.make_activation(1, ho, wo, L.c_out, L.dtype, 105).cuda()
    ag, wk, bg = a_e.cuda(), ssi.weight_to_krsc(wt).cuda(), bias.cuda()
    wp = _pack_guarded(wk, g)
    ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    gen = torch.Generator().manual_seed(107)
    for cnt in sorted({1, max(1, plan.split_max // 2), min(plan.split_max, plan.cap)}):
        lst = torch.randperm(plan.cap, generator=gen)[:cnt].sort().values.to(torch.int32)
        idx = torch.zeros(plan.cap, dtype=torch.int32)
        idx[:cnt] = lst
        idx, count = idx.cuda(), torch.tensor([cnt], dtype=torch.int32, device="cuda")
        print(f"[case] {layer} split packed: {cnt} of {plan.cap} blocks", flush=True)
        for copy in (True, False):
            o1, o2 = cache.clone(), cache.clone()
            ssi.sige_sparse_conv_layer_auto(ag, wk, bg, cache if copy else None, idx, count, g, out=o1,
                                            copy_cached=copy, workspace=ws)
            ssi.sige_sparse_conv_layer_auto(ag, wk, bg, cache if copy else None, idx, count, g, out=o2,
                                            copy_cached=copy, workspace=ws, w_packed=wp)
            assert torch.equal(o1.view(torch.uint8), o2.view(torch.uint8)), f"{layer} {cnt} blocks copy={copy}"
        sub = torch.zeros(plan.cap, dtype=torch.uint8)
        sub[lst[torch.randperm(cnt, generator=gen)[:2]].long()] = 1
        sub = sub.view(1, nby, nbx)
        out = o2.cpu()
        r64 = oracle.sparse_layer(a_e, wt, bias, L.k, L.stride, L.pad, L.block, sub, out, out_f64=True)
        assert_close(out, r64, dt, active_pixels(sub, L.block, ho, wo), f"{layer} split packed, sampled blocks")

"""The bounding-box comparator on the GPU: dense conv of the crop (torch) and
the same rectangle through this library's tile path, against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import spatially_sparse_incremental_amd as ssi
import synth
from _parity import assert_close, bits, rand
from spatially_sparse_incremental_amd import comparators as cmp

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("dt,k,s,p,b", [(torch.bfloat16, 3, 1, 1, 4), (torch.float16, 3, 2, 1, 3),
                                        (torch.float32, 1, 1, 0, 4)])
def test_crop_conv_equals_dense_edited_conv(dt, k, s, p, b):
    n, h, w, cin, cout = 1, 40, 52, 32, 24
    a_o = rand((n, h, w, cin), dt, 401)
    m = np.zeros((n, h, w), np.uint8)
    m[:, 5:9, 6:11] = 1     # two separated edits: the box spans both
    m[:, 30:33, 40:47] = 1
    a_e = synth.make_edit(a_o, m, "replace", 402)
    wt = rand((cout, cin, k, k), dt, 403, (2.0 / (cin * k * k)) ** 0.5)
    bias = rand((cout,), torch.float32, 404, 0.01)
    cache = oracle.dense_conv(a_o, wt, bias, k, s, p)
    mask = ssi.sige_diff_mask(a_o.cuda(), a_e.cuda(), 1e-6)
    box = cmp.edit_bbox(mask)
    assert box == (5, 32, 6, 46)
    rect = cmp.bbox_out_rect(box, h, w, k, s, p)
    out = cmp.bbox_crop_conv(a_e.cuda(), wt.cuda(), bias.cuda(), cache.cuda(), rect, k, s, p)
    torch.cuda.synchronize()
    o = out.cpu()
    inside = torch.zeros(o.shape[:3], dtype=torch.bool)
    inside[:, rect[0]:rect[1] + 1, rect[2]:rect[3] + 1] = True
    keep = ~inside[..., None].expand_as(o)
    assert torch.equal(o[keep].view(torch.uint8), cache[keep].view(torch.uint8))
    assert_close(o, oracle.dense_conv(a_e, wt, bias, k, s, p, out_f64=True), dt, None, "bbox crop")


def test_bbox_rectangle_through_the_tile_path_on_the_unet_layer():
    wl = synth.workload("unet_256x256x128_bf16")
    L = wl.layers[0]
    a_o = synth.make_activation(1, L.h, L.w, L.c_in, L.dtype, 1)
    a_e = synth.make_edit(a_o, synth.edit_shape(wl, 1).raster(L.h, L.w), wl.edit_kind, 1)
    wt, bias = synth.make_layer_tensors(L, 1)
    g = ssi.geom(1, L.h, L.w, L.c_in, L.c_out, L.k, L.stride, L.pad, L.block)
    d = ssi.sige_geom_derive(g)
    cache = synth.make_activation(1, d.ho, d.wo, L.c_out, L.dtype, 7).cuda()
    ae = a_e.cuda()
    mask = ssi.sige_diff_mask(a_o.cuda(), ae, wl.tau)
    rect = cmp.bbox_out_rect(cmp.edit_bbox(mask), L.h, L.w, L.k, L.stride, L.pad)
    crop = cmp.bbox_crop_conv(ae, wt.cuda().contiguous(memory_format=torch.channels_last), bias.cuda(), cache, rect,
                              L.k, L.stride, L.pad)
    idx, cnt = cmp.bbox_block_list(rect, L.block, d.nby, d.nbx)
    tiles = ssi.sige_sparse_conv_layer(ae, ssi.weight_to_krsc(wt).cuda(), bias.cuda(), cache, idx, cnt, g)
    torch.cuda.synchronize()
    print(f"\n[case] bbox rows {rect[0]}..{rect[1]} cols {rect[2]}..{rect[3]}, {int(cnt)} blocks", flush=True)
    inside = torch.zeros((1, d.ho, d.wo), dtype=torch.bool, device="cuda")
    inside[:, rect[0]:rect[1] + 1, rect[2]:rect[3] + 1] = True
    keep = ~inside[..., None].expand_as(cache)
    assert torch.equal(bits(crop[keep]), bits(cache[keep]))
    # the tile path recomputes whole blocks: inside the rectangle both are the dense
    # edited conv (checked against the oracle at sampled pixels), outside it the
    # blocks' edge pixels equal the dense conv of an unchanged window
    sel = inside[..., None].expand_as(cache)
    assert_close(tiles[sel].float().cpu(), crop[sel].double().cpu(), torch.bfloat16, None, "tiles vs crop")
    ys = np.random.default_rng(3).integers(rect[0], rect[1] + 1, 6)
    xs = np.random.default_rng(4).integers(rect[2], rect[3] + 1, 6)
    act = torch.zeros((1, d.nby, d.nbx), dtype=torch.uint8)
    for y, x in zip(ys, xs):
        act[0, y // L.block, x // L.block] = 1
    ref = oracle.sparse_layer(a_e, wt, bias, L.k, L.stride, L.pad, L.block, act, cache.cpu(), out_f64=True)
    pts = torch.zeros((1, d.ho, d.wo, 1), dtype=torch.bool)
    for y, x in zip(ys, xs):
        pts[0, y, x] = True
    assert_close(crop.cpu(), ref, torch.bfloat16, pts, "crop vs oracle at sampled pixels")

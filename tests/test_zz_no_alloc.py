"""sige_sparse_conv_layer_split_noalloc (the split layer on the library's static
scratch) against sige_sparse_conv_layer_split with a caller workspace: the
same kernels on the same inputs, so the outputs must agree bit for bit.  Two
calls in a row on one GPU, the second with a smaller input, so the second runs
on scratch that the first left full of its own partial tiles.
"""
import pytest
import torch

import spatially_sparse_incremental_amd as ssi
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _case(h, w, c_in, c_out, k, block, area, seed, copy_cached):
    """Inputs of one layer, its block list, and both entry points' outputs."""
    dev = torch.device("cuda")
    L = synth.LayerSpec(f"noalloc_{h}x{w}x{c_in}", h, w, c_in, c_out, k, 1, k // 2, block, 1, "f16")
    mask_np = synth.Blob.draw(seed, h, w).fit_area(area).raster()
    a_o = synth.make_activation(1, h, w, c_in, "f16", seed)
    a_e = synth.make_edit(a_o, mask_np, "replace", seed).to(dev)
    wt, bias = synth.make_layer_tensors(L, seed)
    w_krsc, bias = ssi.weight_to_krsc(wt).to(dev), bias.to(dev)
    cache = synth.make_activation(1, h, w, c_out, "f16", seed + 7).to(dev)
    g = ssi.geom(1, h, w, c_in, c_out, k, 1, k // 2, block)
    mask = ssi.sige_diff_mask(a_o.to(dev), a_e)
    idx, count = ssi.sige_reduce_mask(mask, g, 1)
    assert ssi.sige_sparse_conv_layer_split_workspace(g, torch.float16) <= ssi.sige_noalloc_scratch_bytes()
    out_ws = cache.clone()
    ssi.sige_sparse_conv_layer_split(a_e, w_krsc, bias, cache, idx, count, g, out=out_ws, copy_cached=copy_cached)
    out_na = torch.full_like(cache, float("nan")) if copy_cached else cache.clone()
    ssi.sige_sparse_conv_layer_split_noalloc(a_e, w_krsc, bias, cache, idx, count, g, out_na,
                                             copy_cached=copy_cached)
    torch.cuda.synchronize()
    return out_ws, out_na, int(count.item())


@pytest.mark.parametrize("copy_cached", [True, False])
def test_noalloc_matches_the_workspace_call_twice(copy_cached):
    # first: the 16x16x1280 latent-diffusion layer at a 10% edit (12.5 MiB of partial tiles)
    out_ws, out_na, n1 = _case(16, 16, 1280, 1280, 3, 2, 0.10, 5, copy_cached)
    print(f"\n[case] 16x16x1280 b2: {n1} blocks", flush=True)
    assert n1 > 0
    assert torch.equal(out_ws.view(torch.int16), out_na.view(torch.int16))
    # second, smaller: 24x40x128 -> 64, 3x3, b 4, a 3% edit
    out_ws, out_na, n2 = _case(24, 40, 128, 64, 3, 4, 0.03, 6, copy_cached)
    print(f"[case] 24x40x128 b4: {n2} blocks", flush=True)
    assert 0 < n2
    assert torch.equal(out_ws.view(torch.int16), out_na.view(torch.int16))

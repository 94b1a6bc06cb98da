"""The bench's measured step at its full size, against the oracle on every
listed block: sige_diff_mask_bits -> sige_reduce_bits_copy ->
sige_sparse_conv_layer_packed(copy_cached = 0) (the weights packed once by
sige_pack_weights, as the bench does) on the 256x256x128 -> 128 bf16 U-Net
layer with the bench's own seeded 1.2% blob edit, run as replays of a captured
HIP graph (the launch configuration the bench times).

Expected values: the oracle's change mask (packed here one bit per pixel),
its block list and its fp64 sparse layer; the cache, bit for bit, outside the
listed blocks.
"""
import numpy as np
import pytest
import torch

import oracle
import spatially_sparse_incremental_amd as ssi
import synth
from _parity import active_pixels, assert_close, bits

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_bench_step_at_full_size_against_the_oracle():
    wl = synth.workload("unet_256x256x128_bf16")
    L = wl.layers[0]
    seed = 1  # the bench's inputs
    mask_np = synth.edit_shape(wl, seed).raster(L.h, L.w)
    a_o = synth.make_activation(1, L.h, L.w, L.c_in, L.dtype, seed)
    a_e = synth.make_edit(a_o, mask_np, wl.edit_kind, seed)
    wt, bias = synth.make_layer_tensors(L, seed)
    cache = oracle.dense_conv(a_o, wt, bias, L.k, L.stride, L.pad)  # conv(A_o), rounded to bf16
    g = ssi.geom(1, L.h, L.w, L.c_in, L.c_out, L.k, L.stride, L.pad, L.block)
    cap = ssi.sige_max_blocks(g)
    ao, ae, cg = a_o.cuda(), a_e.cuda(), cache.cuda()
    wk, bs = ssi.weight_to_krsc(wt).cuda(), bias.cuda()
    wp = ssi.sige_pack_weights(wk, g)
    mbits = torch.empty((L.h * L.w // 32,), dtype=torch.int32, device="cuda")
    idx = torch.empty((cap,), dtype=torch.int32, device="cuda")
    count = torch.empty((1,), dtype=torch.int32, device="cuda")
    out = torch.empty_like(cg)

    def step():
        ssi.sige_diff_mask_bits(ao, ae, wl.tau, bits=mbits)
        ssi.sige_reduce_bits_copy(mbits, L.h, L.w, g, L.dilate, cg, out=out, idx=idx, count=count)
        ssi.sige_sparse_conv_layer(ae, wk, bs, None, idx, count, g, out=out, copy_cached=False, w_packed=wp)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    m_ref = oracle.diff_mask(a_o, a_e, wl.tau)
    act = oracle.block_activity(m_ref, L.h, L.w, L.k, L.stride, L.pad, L.block, L.dilate)
    idx_ref = oracle.index_list(act)
    out64 = oracle.sparse_layer(a_e, wt, bias, L.k, L.stride, L.pad, L.block, act, cache, out_f64=True)
    # the packed oracle mask: bit p % 32 of word p / 32
    flat = m_ref.reshape(-1).numpy().astype(np.uint64)
    words = (flat.reshape(-1, 32) << np.arange(32, dtype=np.uint64)).sum(axis=1).astype(np.uint32)
    sel = active_pixels(act, L.block, L.h, L.w)
    for rep in range(3):
        out.fill_(7.0)
        idx.fill_(-5)
        graph.replay()
        torch.cuda.synchronize()
        print(f"\n[case] bench step replay {rep}: {int(count.item())} of {cap} blocks", flush=True)
        assert np.array_equal(mbits.cpu().numpy().view(np.uint32), words), "change mask"
        cnt = int(count.item())
        assert cnt == idx_ref.numel() and torch.equal(idx[:cnt].cpu(), idx_ref), "block list"
        got = out.cpu()
        keep = ~sel.expand_as(got)
        assert torch.equal(bits(got[keep]), bits(cache[keep])), "pixels outside the listed blocks"
        assert_close(got, out64, got.dtype, sel, f"bench step, every listed block, replay {rep}")

"""The hot path captured in a HIP graph: every replay equals the eager result.

Replays are interleaved with eager work, synchronisations and input changes,
and each one is compared bit for bit with an eager run on the same inputs.
"""
import numpy as np
import pytest
import torch

import spatially_sparse_incremental_amd as ssi
import synth
from _parity import active_pixels, assert_close, bits, layer_inputs, rand

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("copy", ["conv", "reduce", "none"])
def test_graph_replays_match_eager(copy):
    n, h, w, c, b = 1, 64, 72, 64, 6
    dt = torch.bfloat16
    blob = synth.Blob.draw(5, h, w).fit_area(0.02)
    mask0 = blob.raster()
    a_o, a_e, wt, bias = [t.cuda() for t in layer_inputs(n, h, w, c, c, 3, dt, 201, mask0)]
    wk = ssi.weight_to_krsc(wt)
    cache = rand((n, h, w, c), dt, 202).cuda()
    g = ssi.geom(n, h, w, c, c, 3, 1, 1, b)
    cap = ssi.sige_max_blocks(g)
    m = torch.empty((n, h, w), dtype=torch.uint8, device="cuda")
    idx = torch.empty((cap,), dtype=torch.int32, device="cuda")
    cnt = torch.empty((1,), dtype=torch.int32, device="cuda")
    out = cache.clone()

    def step():
        ssi.sige_diff_mask(a_o, a_e, 1e-6, mask=m)
        if copy == "reduce":  # the copy of the cache rides with the reduce
            ssi.sige_reduce_mask_copy(m, g, 1, cache, out=out, idx=idx, count=cnt)
        else:
            ssi.sige_reduce_mask(m, g, 1, idx=idx, count=cnt)
        if copy == "conv":
            ssi.sige_sparse_conv_layer(a_e, wk, bias, cache, idx, cnt, g, out=out, copy_cached=True)
        else:
            ssi.sige_sparse_conv_layer(a_e, wk, bias, None, idx, cnt, g, out=out, copy_cached=False)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    rng = np.random.default_rng(203)
    for rep in range(5):
        # a new edit, written in place into the captured input buffer; `out` holds
        # stale values where the graph must overwrite them
        mk = torch.from_numpy((rng.random((n, h, w)) < 0.01).astype(np.uint8))
        a_e.copy_(synth.make_edit(a_o.cpu(), mk.numpy(), "replace", 210 + rep).cuda())
        out.copy_(cache if copy == "none" else torch.zeros_like(cache))
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        got_idx = idx[:int(cnt.item())].clone()
        out.copy_(cache if copy == "none" else torch.zeros_like(cache))
        step()  # eager, same inputs
        torch.cuda.synchronize()
        assert torch.equal(got_idx, idx[:int(cnt.item())]), rep
        assert torch.equal(bits(got), bits(out)), rep
        assert int(cnt.item()) > 0


def test_graph_replays_of_the_auto_layer_follow_the_list_length():
    """sige_sparse_conv_layer_auto captured once on a layer whose plan enqueues all
    three kernels: replays with list lengths on every side of the thresholds
    (written in place) match an eager call bit for bit, and the kernel the plan
    names (the wide tiles: the single-range kernel within tolerance on the listed
    blocks, bit for bit elsewhere)."""
    L = synth.workload("gaugan_4conv_bf16").layers[1]  # 64x128x1024 -> 512: gated plan
    g = ssi.geom(1, L.h, L.w, L.c_in, L.c_out, L.k, L.stride, L.pad, L.block)
    plan = ssi.sige_sparse_conv_layer_plan(g, torch.bfloat16)
    assert 0 <= plan.split_max < plan.wide_min <= plan.cap
    wt, bias = synth.make_layer_tensors(L, 31)
    wk, bias = ssi.weight_to_krsc(wt).cuda(), bias.cuda()
    a = synth.make_activation(1, L.h, L.w, L.c_in, L.dtype, 32).cuda()
    cache = synth.make_activation(1, L.h, L.w, L.c_out, L.dtype, 33).cuda()
    idx = torch.zeros((plan.cap,), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((1,), dtype=torch.int32, device="cuda")
    ws = torch.empty((plan.workspace_bytes,), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(cache)

    def layer():
        ssi.sige_sparse_conv_layer_auto(a, wk, bias, cache, idx, cnt, g, out=out, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer()
    rng = np.random.default_rng(34)
    d = ssi.sige_geom_derive(g)
    for n in (7, plan.split_max, plan.split_max + 1, plan.wide_min - 1, plan.wide_min, plan.cap, 0,
              plan.split_max // 2):
        pick = np.sort(rng.choice(plan.cap, size=n, replace=False)).astype(np.int32)
        idx.zero_()
        idx[:n] = torch.from_numpy(pick).cuda()
        cnt.fill_(n)
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        out.zero_()
        layer()  # eager, same inputs
        ref_fn = ssi.sige_sparse_conv_layer_split if n <= plan.split_max else ssi.sige_sparse_conv_layer
        ref = ref_fn(a, wk, bias, cache, idx, cnt, g)
        torch.cuda.synchronize()
        assert torch.equal(bits(got), bits(out)), n
        if n < plan.wide_min:
            assert torch.equal(bits(got), bits(ref)), n
        else:
            act = torch.zeros(plan.cap, dtype=torch.uint8)
            act[torch.from_numpy(pick).long()] = 1
            sel = active_pixels(act.view(1, d.nby, d.nbx), L.block, d.ho, d.wo).expand_as(cache.cpu())
            o, r = got.cpu(), ref.cpu()
            assert torch.equal(o[~sel].view(torch.uint8), r[~sel].view(torch.uint8)), n
            assert_close(o, r.double(), o.dtype, sel, f"wide tiles in a graph replay, {n} blocks")

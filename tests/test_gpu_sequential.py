"""Sequential edits on the GPU: restore of the previous edit's blocks into a
persistent output buffer, then the new blocks written without the cache copy.

Expected values: the oracle's restore_blocks (bit for bit) and the oracle's
layer computed from scratch for each edit; the GPU's own copy_cached = 1 result
must match the persistent buffer bit for bit after every edit.
"""
import numpy as np
import pytest
import torch

import oracle
import spatially_sparse_incremental_amd as ssi
import synth
from _parity import assert_close, bits, rand

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("with_new", [True, False], ids=["new_list", "no_new_list"])
def test_restore_matches_oracle_bitwise(with_new):
    n, h, w, c, b = 2, 29, 23, 24, 4
    g = ssi.geom(n, h, w, 8, c, 3, 1, 1, b)
    d = ssi.sige_geom_derive(g)
    dt = torch.float16
    cache = rand((n, d.ho, d.wo, c), dt, 201)
    rng = np.random.default_rng(202)
    for trial in range(6):
        prev_act = rng.random((n, d.nby, d.nbx)) < 0.3
        new_act = rng.random((n, d.nby, d.nbx)) < 0.3
        before = rand((n, d.ho, d.wo, c), dt, 210 + trial)
        prev = oracle.index_list(torch.from_numpy(prev_act.astype(np.uint8)))
        new = oracle.index_list(torch.from_numpy(new_act.astype(np.uint8))) if with_new else None
        ref = oracle.restore_blocks(prev, new, cache, before.clone(), b)
        print(f"\n[case] restore trial {trial}: {prev.numel()} previous blocks", flush=True)
        buf = torch.zeros(d.cap, dtype=torch.int32)
        buf[:prev.numel()] = prev
        prev_g, prev_c = buf.cuda(), torch.tensor([prev.numel()], dtype=torch.int32).cuda()
        if with_new:
            nb = torch.zeros(d.cap, dtype=torch.int32)
            nb[:new.numel()] = new
            new_g, new_c = nb.cuda(), torch.tensor([new.numel()], dtype=torch.int32).cuda()
        else:
            new_g = new_c = None
        out = before.cuda()
        ssi.sige_restore_blocks(prev_g, prev_c, new_g, new_c, g, cache.cuda(), out)
        torch.cuda.synchronize()
        assert torch.equal(bits(out.cpu()), bits(ref)), f"trial {trial}"


@pytest.mark.parametrize("mode", ["one_call", "restore_then_fused", "three_step"])
def test_sequence_of_edits_through_a_persistent_buffer(mode):
    # four edits (overlapping, disjoint, empty, then a new one): after each, the
    # persistent buffer equals the copy_cached = 1 result bit for bit and the
    # oracle's layer computed from scratch
    n, h, w, cin, cout, k, s, p, b, dil = 1, 37, 45, 32, 40, 3, 1, 1, 5, 1
    dt = torch.bfloat16
    a_o = rand((n, h, w, cin), dt, 301)
    wt = rand((cout, cin, k, k), dt, 302, (2.0 / (cin * k * k)) ** 0.5)
    bias = rand((cout,), torch.float32, 303, 0.01)
    g = ssi.geom(n, h, w, cin, cout, k, s, p, b)
    d = ssi.sige_geom_derive(g)
    cache = rand((n, d.ho, d.wo, cout), dt, 304)
    wk, bs, cg, ao = ssi.weight_to_krsc(wt).cuda(), bias.cuda(), cache.cuda(), a_o.cuda()
    rects = [(4, 12, 3, 15), (8, 20, 10, 25), None, (25, 37, 30, 45)]
    persist = cg.clone()
    idx_buf = [torch.zeros(d.cap, dtype=torch.int32, device="cuda") for _ in range(2)]
    cnt_buf = [torch.zeros(1, dtype=torch.int32, device="cuda") for _ in range(2)]  # no previous edit at first
    for e, r in enumerate(rects):
        m = np.zeros((n, h, w), np.uint8)
        if r is not None:
            m[:, r[0]:r[1], r[2]:r[3]] = 1
        a_e = synth.make_edit(a_o, m, "replace", 310 + e) if r is not None else a_o.clone()
        ae = a_e.cuda()
        cur, prv = e % 2, (e + 1) % 2
        mask = ssi.sige_diff_mask(ao, ae, 1e-6)
        ssi.sige_reduce_mask(mask, g, dil, idx=idx_buf[cur], count=cnt_buf[cur])
        if mode == "one_call":
            ssi.sige_sparse_conv_layer_restore(ae, wk, bs, cg, idx_buf[prv], cnt_buf[prv], idx_buf[cur],
                                               cnt_buf[cur], g, persist)
        elif mode == "restore_then_fused":
            ssi.sige_restore_blocks(idx_buf[prv], cnt_buf[prv], idx_buf[cur], cnt_buf[cur], g, cg, persist)
            ssi.sige_sparse_conv_layer(ae, wk, bs, None, idx_buf[cur], cnt_buf[cur], g, out=persist,
                                       copy_cached=False)
        else:
            ssi.sige_restore_blocks(idx_buf[prv], cnt_buf[prv], idx_buf[cur], cnt_buf[cur], g, cg, persist)
            blocks = ssi.sige_gather(ae, g, idx_buf[cur], cnt_buf[cur])
            ob = ssi.sige_conv_blocks(blocks, wk, bs, g, cnt_buf[cur])
            ssi.sige_scatter(ob, idx_buf[cur], cnt_buf[cur], g, None, out=persist, copy_cached=False)
        literal = ssi.sige_sparse_conv_layer(ae, wk, bs, cg, idx_buf[cur], cnt_buf[cur], g)
        torch.cuda.synchronize()
        cnt = int(cnt_buf[cur].item())
        print(f"\n[case] edit {e}: {cnt} blocks", flush=True)
        assert torch.equal(bits(persist.cpu()), bits(literal.cpu())), f"edit {e}"
        act = oracle.block_activity(oracle.diff_mask(a_o, a_e), h, w, k, s, p, b, dil)
        assert torch.equal(idx_buf[cur][:cnt].cpu(), oracle.index_list(act))
        ref = oracle.sparse_layer(a_e, wt, bias, k, s, p, b, act, cache, out_f64=True)
        assert_close(persist.cpu(), ref, dt, None, f"edit {e}")


@pytest.mark.parametrize("one_call", [True, False], ids=["one_call", "two_calls"])
def test_unet_layer_alternating_edits_full_size(one_call):
    # the 256x256x128 bf16 layer: two blob edits alternate through one persistent
    # buffer; each step must equal the copy_cached = 1 result bit for bit
    wl = synth.workload("unet_256x256x128_bf16")
    L = wl.layers[0]
    a_o = synth.make_activation(1, L.h, L.w, L.c_in, L.dtype, 1)
    edits = [synth.make_edit(a_o, synth.edit_shape(wl, sd).raster(L.h, L.w), wl.edit_kind, sd).cuda()
             for sd in (1, 2)]
    wt, bias = synth.make_layer_tensors(L, 1)
    wk, bs = ssi.weight_to_krsc(wt).cuda(), bias.cuda()
    g = ssi.geom(1, L.h, L.w, L.c_in, L.c_out, L.k, L.stride, L.pad, L.block)
    d = ssi.sige_geom_derive(g)
    ao = a_o.cuda()
    cg = synth.make_activation(1, L.h, L.w, L.c_out, L.dtype, 5).cuda()
    persist = cg.clone()
    idx_buf = [torch.zeros(d.cap, dtype=torch.int32, device="cuda") for _ in range(2)]
    cnt_buf = [torch.zeros(1, dtype=torch.int32, device="cuda") for _ in range(2)]  # no previous edit at first
    for step in range(5):
        cur, prv = step % 2, (step + 1) % 2
        ae = edits[cur]
        mask = ssi.sige_diff_mask(ao, ae, wl.tau)
        ssi.sige_reduce_mask(mask, g, L.dilate, idx=idx_buf[cur], count=cnt_buf[cur])
        if one_call:
            ssi.sige_sparse_conv_layer_restore(ae, wk, bs, cg, idx_buf[prv], cnt_buf[prv], idx_buf[cur],
                                               cnt_buf[cur], g, persist)
        else:
            ssi.sige_restore_blocks(idx_buf[prv], cnt_buf[prv], idx_buf[cur], cnt_buf[cur], g, cg, persist)
            ssi.sige_sparse_conv_layer(ae, wk, bs, None, idx_buf[cur], cnt_buf[cur], g, out=persist,
                                       copy_cached=False)
        literal = ssi.sige_sparse_conv_layer(ae, wk, bs, cg, idx_buf[cur], cnt_buf[cur], g)
        torch.cuda.synchronize()
        print(f"\n[case] step {step}: {int(cnt_buf[cur].item())} blocks", flush=True)
        assert torch.equal(bits(persist), bits(literal)), f"step {step}"

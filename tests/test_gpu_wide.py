"""The wide tiles of the fused layer (k_layer_wide, run by
sige_sparse_conv_layer_auto for long lists) against the oracle.

SIGE_WIDE_MIN=0 makes the plan send every list of these geometries to the wide
tiles (the plan is made once per geometry, so the geometries here are used by
no other test).  Edge cases: a partial last 16-channel stage (c_in = 24, 200),
output channels past one or two 128-channel tiles (c_out = 136, 64), two
images, 1x1 and 3x3 kernels, blocks of 4, 5, 6 and 8 (one or two window rows
per staging load), windows over the image border, several 256-row tiles, the
empty list, one block, every block, with and without the cache copy; and
tiles split over K (c_in >= 128: these lists make fewer tiles than there are
compute units, so each tile's stages are split into 2-4 parts, of unequal
length for c_in = 200, whose fp32 partials a second launch adds up)."""
import os

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
    ("cin24_cout136_b6_bf16", 1, 40, 44, 24, 136, 3, 1, 1, 6, "bf16"),
    ("two_images_b4_f16", 2, 30, 30, 32, 64, 3, 1, 1, 4, "f16"),
    ("pointwise_b5_bf16", 1, 33, 35, 48, 128, 1, 1, 0, 5, "bf16"),
    ("b8_one_row_per_load_f16", 1, 48, 52, 40, 96, 3, 1, 1, 8, "f16"),
    ("parts3_cin200_cout136_b6_bf16", 1, 40, 44, 200, 136, 3, 1, 1, 6, "bf16"),
    ("parts4_cin256_two_images_b4_f16", 2, 30, 30, 256, 64, 3, 1, 1, 4, "f16"),
    ("parts2_pointwise_cin128_b5_bf16", 1, 33, 35, 128, 128, 1, 1, 0, 5, "bf16"),
]


def _parts_max(cin):
    """The most K parts of a wide tile: at least 4 stages of 16 channels each, at most 16 parts."""
    return max(1, min(16, ((cin + 15) // 16) // 4))


def _forced_plan(g, dt, monkeypatch):
    monkeypatch.setenv("SIGE_WIDE_MIN", "0")
    plan = ssi.sige_sparse_conv_layer_plan(g, dt)
    assert plan.wide_stages > 0 and plan.wide_min <= plan.split_max + 1, plan.as_dict()
    assert plan.wide_parts_max == _parts_max(g.c_in), plan.as_dict()
    if plan.wide_parts_max > 1:  # the partial tiles' workspace
        assert plan.workspace_bytes >= 2 * 256 * 128 * 4, plan.as_dict()
    return plan


def _lists(cap, seed):
    gen = torch.Generator().manual_seed(seed)
    sizes = sorted({0, 1, max(1, cap // 7), max(1, cap // 2), cap})
    for n in sizes:
        yield torch.randperm(cap, generator=gen)[:n].sort().values.to(torch.int32)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_wide_tiles_against_the_oracle(case, monkeypatch):
    name, n, h, w, cin, cout, k, s, p, b, dts = case
    dt = DT[dts]
    g = ssi.geom(n, h, w, cin, cout, k, s, p, b)
    plan = _forced_plan(g, dt, monkeypatch)
    ho, wo, nby, nbx, _ = oracle.geometry(h, w, k, s, p, b)
    cap = n * nby * nbx
    mask = random_mask(n, h, w, 0.5, 3)
    _, a_e, wt, bias = layer_inputs(n, h, w, cin, cout, k, dt, 5, mask)
    cache = rand((n, ho, wo, cout), dt, 7)
    wk, bg, ag, cg = ssi.weight_to_krsc(wt).cuda(), bias.cuda(), a_e.cuda(), cache.cuda()
    ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    for lst in _lists(cap, 11):
        cnt = lst.numel()
        idx = torch.zeros(cap, dtype=torch.int32)
        idx[:cnt] = lst
        idx_g, count = idx.cuda(), torch.tensor([cnt], dtype=torch.int32, device="cuda")
        act = torch.zeros(cap, dtype=torch.uint8)
        act[lst.long()] = 1
        act = act.view(n, nby, nbx)
        print(f"[case] {name}: {cnt} of {cap} blocks", flush=True)
        ref = oracle.sparse_layer(a_e, wt, bias, k, s, p, b, act, cache, out_f64=True)
        sel = active_pixels(act, b, ho, wo)
        keep = ~sel.expand_as(cache)
        out = ssi.sige_sparse_conv_layer_auto(ag, wk, bg, cg, idx_g, count, g, workspace=ws).cpu()
        assert torch.equal(out[keep].view(torch.uint8), cache[keep].view(torch.uint8)), f"{name}: copy"
        assert_close(out, ref, dt, sel, f"{name} {cnt} blocks")
        pers = cg.clone()
        ssi.sige_sparse_conv_layer_auto(ag, wk, bg, None, idx_g, count, g, out=pers, copy_cached=False,
                                        workspace=ws)
        assert torch.equal(pers.cpu().view(torch.uint8), out.view(torch.uint8)), f"{name}: persistent buffer"


@pytest.mark.parametrize("cin", [32, 256], ids=["one_part", "four_parts"])
def test_wide_tiles_in_a_graph_replay(cin, monkeypatch):
    """Replays of a captured wide-tile layer equal the eager result (each replay's
    output cleared in between), with and without the K split."""
    n, h, w, cout, k, s, p, b = 1, 36, 60, 128, 3, 1, 1, 6
    dt = torch.bfloat16
    g = ssi.geom(n, h, w, cin, cout, k, s, p, b)
    plan = _forced_plan(g, dt, monkeypatch)
    mask = random_mask(n, h, w, 0.3, 41)
    a_o, a_e, wt, bias = layer_inputs(n, h, w, cin, cout, k, dt, 43, mask)
    cache = rand((n, h, w, cout), dt, 45).cuda()
    ag, ao, wk, bg = a_e.cuda(), a_o.cuda(), ssi.weight_to_krsc(wt).cuda(), bias.cuda()
    ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    mk = ssi.sige_diff_mask(ao, ag, 1e-6)
    idx, count = ssi.sige_reduce_mask(mk, g, 1)
    out = torch.empty_like(cache)

    def step():
        ssi.sige_sparse_conv_layer_auto(ag, wk, bg, cache, idx, count, g, out=out, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = out.clone()
    assert int(count.item()) > 0
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        step()
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.uint8), eager.view(torch.uint8))


def test_wide_tiles_at_full_size():
    """The 256x256x128 bf16 layer with 1500 of its 1849 blocks listed: the
    library's own plan sends the list to the wide tiles; equal to the 64 x 32
    tiles within tolerance (untouched pixels bit for bit), and to the oracle on
    sampled blocks."""
    assert "SIGE_WIDE_MIN" not in os.environ
    n, h, w, cin, cout, k, s, p, b = 1, 256, 256, 128, 128, 3, 1, 1, 6
    dt = torch.bfloat16
    g = ssi.geom(n, h, w, cin, cout, k, s, p, b)
    plan = ssi.sige_sparse_conv_layer_plan(g, dt)
    cap, cnt = plan.cap, 1500
    assert plan.wide_min <= cnt <= plan.wide_max, plan.as_dict()
    mask = random_mask(n, h, w, 1.0, 51)
    _, a_e, wt, bias = layer_inputs(n, h, w, cin, cout, k, dt, 53, mask)
    cache = rand((n, h, w, cout), dt, 55)
    ag, wk, bg = a_e.cuda(), ssi.weight_to_krsc(wt).cuda(), bias.cuda()
    gen = torch.Generator().manual_seed(57)
    lst = torch.randperm(cap, generator=gen)[:cnt].sort().values.to(torch.int32)
    idx = torch.zeros(cap, dtype=torch.int32)
    idx[:cnt] = lst
    idx, count = idx.cuda(), torch.tensor([cnt], dtype=torch.int32, device="cuda")
    ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    out = ssi.sige_sparse_conv_layer_auto(ag, wk, bg, cache.cuda(), idx, count, g, workspace=ws).cpu()
    ref = ssi.sige_sparse_conv_layer(ag, wk, bg, cache.cuda(), idx, count, g).cpu()
    ho, wo, nby, nbx, _ = oracle.geometry(h, w, k, s, p, b)
    act = torch.zeros(cap, dtype=torch.uint8)
    act[lst.long()] = 1
    sel = active_pixels(act.view(1, nby, nbx), b, ho, wo).expand_as(out)
    assert torch.equal(out[~sel].view(torch.uint8), ref[~sel].view(torch.uint8)), "untouched pixels"
    assert_close(out, ref.double(), dt, sel, "wide vs 64x32 tiles, 1500 blocks")
    sub = torch.zeros(cap, dtype=torch.uint8)
    sub[lst[torch.randperm(cnt, generator=gen)[:6]].long()] = 1
    sub = sub.view(1, nby, nbx)
    r64 = oracle.sparse_layer(a_e, wt, bias, k, s, p, b, sub, out, out_f64=True)
    assert_close(out, r64, dt, active_pixels(sub, b, ho, wo), "wide tiles, sampled blocks against the oracle")


@pytest.mark.parametrize("cin", [40, 128], ids=["one_part", "two_parts"])
def test_wide_tiles_write_nothing_outside_out(cin, monkeypatch):
    """Guard canaries before and after `out` (and after the workspace): the wide
    tiles (every list of this geometry forced to them) write only inside the
    output and the workspace, with and without the cache copy and the K split,
    and leave the unlisted blocks alone without the copy."""
    n, h, w, cout, k, s, p, b = 1, 26, 34, 72, 3, 1, 1, 6
    dt = torch.bfloat16
    g = ssi.geom(n, h, w, cin, cout, k, s, p, b)
    plan = _forced_plan(g, dt, monkeypatch)
    ho, wo, nby, nbx, _ = oracle.geometry(h, w, k, s, p, b)
    cap = n * nby * nbx
    mask = random_mask(n, h, w, 0.5, 61)
    _, a_e, wt, bias = layer_inputs(n, h, w, cin, cout, k, dt, 63, mask)
    cache = rand((n, ho, wo, cout), dt, 65).cuda()
    ag, wk, bg = a_e.cuda(), ssi.weight_to_krsc(wt).cuda(), bias.cuda()
    nws = max(plan.workspace_bytes, 16)
    wbuf = torch.full((nws + 4096,), 0x5A, dtype=torch.uint8, device="cuda")
    ws = wbuf[:nws]
    G, nout = 4096, n * ho * wo * cout
    gen = torch.Generator().manual_seed(67)
    for cnt, copy in ((cap, True), (cap // 2, False), (1, True)):
        lst = torch.randperm(cap, generator=gen)[:cnt].sort().values.to(torch.int32)
        idx = torch.zeros(cap, dtype=torch.int32)
        idx[:cnt] = lst
        idx, count = idx.cuda(), torch.tensor([cnt], dtype=torch.int32, device="cuda")
        buf = torch.full((G + nout + G,), 3.0, dtype=dt, device="cuda")
        out = buf[G:G + nout].view(n, ho, wo, cout)
        if not copy:
            out.copy_(cache)
        ssi.sige_sparse_conv_layer_auto(ag, wk, bg, cache if copy else None, idx, count, g, out=out,
                                        copy_cached=copy, workspace=ws)
        torch.cuda.synchronize()
        assert (buf[:G] == 3.0).all() and (buf[G + nout:] == 3.0).all(), f"{cnt} blocks: stray writes"
        assert (wbuf[nws:] == 0x5A).all(), f"{cnt} blocks: writes past the workspace"
        act = torch.zeros(cap, dtype=torch.uint8)
        act[lst.long()] = 1
        sel = active_pixels(act.view(n, nby, nbx), b, ho, wo).expand_as(out).cuda()
        assert torch.equal(out[~sel].view(torch.uint8), cache[~sel].view(torch.uint8)), f"{cnt} blocks: unlisted"


def _packed_reference(wk, cin, cout, k):
    """The stage-major layout written out from its definition, on the CPU: unit
    ((tn * nst + s) * k*k + t) * 256 + 2n + (h xor (n/8 mod 2)) holds the 8
    channels 16s + 8h .. of output channel 128 tn + n at tap t, zeros outside
    the weights."""
    ntn, nst, k2 = (cout + 127) // 128, (cin + 15) // 16, k * k
    w = wk.view(cout, k2, cin)
    ref = torch.zeros(ntn, nst, k2, 256, 8, dtype=wk.dtype)
    for u in range(256):
        n = (u >> 1) & 127
        h = (u & 1) ^ ((n >> 3) & 1)
        for tn in range(ntn):
            col = tn * 128 + n
            if col >= cout:
                continue
            for s in range(nst):
                ch = s * 16 + h * 8
                if ch < cin:
                    ref[tn, s, :, u, :] = w[col, :, ch:ch + 8]
    return ref.reshape(-1)


@pytest.mark.parametrize("shape", [(24, 136, 3), (48, 128, 1), (200, 136, 3), (256, 64, 3)],
                         ids=["cin24_cout136", "pointwise", "cin200", "cin256_cout64"])
def test_packed_weights_wide_section_layout(shape):
    """The wide tiles' section of sige_pack_weights (from the 256-byte boundary
    after the single-range kernel's section; the split's section follows it)
    against the stage-major layout written out on the CPU, bit for bit, with a
    guard canary after the copy."""
    cin, cout, k = shape
    g = ssi.geom(1, 40, 44, cin, cout, k, 1, k // 2, 6)
    dt = torch.bfloat16
    wt = rand((cout, cin, k, k), dt, 71)
    wk = ssi.weight_to_krsc(wt)
    need = ssi.sige_packed_weights_bytes(g, dt)
    wide = ((cout + 127) // 128) * ((cin + 15) // 16) * k * k * 4096
    plan = ssi.sige_sparse_conv_layer_plan(g, dt)
    nsub = 2 if plan.n_tiles * 32 >= cout else 1  # the single-range kernel's N subtiles per tile
    off = (plan.chunks * plan.n_tiles * plan.steps * nsub * 1024 + 255) // 256 * 256  # after its section
    assert off + wide <= need
    buf = torch.full((need + 4096,), 0x5A, dtype=torch.uint8, device="cuda")
    ssi.sige_pack_weights(wk.cuda(), g, out=buf[:need])
    torch.cuda.synchronize()
    assert (buf[need:] == 0x5A).all(), "writes past the packed copy"
    got = buf[off:off + wide].cpu().view(torch.int16)
    ref = _packed_reference(wk, cin, cout, k).view(torch.int16)
    assert torch.equal(got, ref)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_packed_weights_give_the_same_layer(case, monkeypatch):
    """sige_sparse_conv_layer_auto_packed equals sige_sparse_conv_layer_auto bit
    for bit (the same weights reach the same registers and LDS slots), on every
    forced-wide geometry (K splits included) and list length, with and without
    the copy."""
    name, n, h, w, cin, cout, k, s, p, b, dts = case
    dt = DT[dts]
    g = ssi.geom(n, h, w, cin, cout, k, s, p, b)
    plan = _forced_plan(g, dt, monkeypatch)
    ho, wo, nby, nbx, _ = oracle.geometry(h, w, k, s, p, b)
    cap = n * nby * nbx
    mask = random_mask(n, h, w, 0.5, 3)
    _, a_e, wt, bias = layer_inputs(n, h, w, cin, cout, k, dt, 5, mask)
    cache = rand((n, ho, wo, cout), dt, 7)
    wk, bg, ag, cg = ssi.weight_to_krsc(wt).cuda(), bias.cuda(), a_e.cuda(), cache.cuda()
    ww = ssi.sige_pack_weights(wk, g)
    ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    for lst in _lists(cap, 13):
        cnt = lst.numel()
        idx = torch.zeros(cap, dtype=torch.int32)
        idx[:cnt] = lst
        idx_g, count = idx.cuda(), torch.tensor([cnt], dtype=torch.int32, device="cuda")
        print(f"[case] {name} packed: {cnt} of {cap} blocks", flush=True)
        for copy in (True, False):
            o1 = cg.clone()
            o2 = cg.clone()
            ssi.sige_sparse_conv_layer_auto(ag, wk, bg, cg if copy else None, idx_g, count, g, out=o1,
                                            copy_cached=copy, workspace=ws)
            ssi.sige_sparse_conv_layer_auto(ag, wk, bg, cg if copy else None, idx_g, count, g, out=o2,
                                            copy_cached=copy, workspace=ws, w_packed=ww)
            assert torch.equal(o1.view(torch.uint8), o2.view(torch.uint8)), f"{name} {cnt} blocks copy={copy}"


@pytest.mark.parametrize("layer,cnt", [("g32x64", 64), ("g64x128", 252), ("g256x512", 1400)])
def test_packed_weights_on_gaugan_layers(layer, cnt):
    """The GauGAN-shaped layers at the list lengths of the 15-30% edits, on the
    library's own plan (the wide tiles, split over K for the deep layers): the
    packed entry point equals the KRSC one bit for bit, and the oracle on
    sampled blocks."""
    import synth

    assert "SIGE_WIDE_MIN" not in os.environ
    L = [x for x in synth.workload("gaugan_4conv_bf16").layers if x.name == layer][0]
    dt = torch.bfloat16
    g = ssi.geom(1, L.h, L.w, L.c_in, L.c_out, L.k, L.stride, L.pad, L.block)
    plan = ssi.sige_sparse_conv_layer_plan(g, dt)
    assert plan.wide_min <= cnt <= plan.wide_max, plan.as_dict()
    ho, wo, nby, nbx, _ = oracle.geometry(L.h, L.w, L.k, L.stride, L.pad, L.block)
    a_e = synth.make_activation(1, L.h, L.w, L.c_in, "bf16", 81)
    wt, bias = synth.make_layer_tensors(L, 83)
    cache = synth.make_activation(1, ho, wo, L.c_out, "bf16", 85)
    ag, wk, bg, cg = a_e.cuda(), ssi.weight_to_krsc(wt).cuda(), bias.cuda(), cache.cuda()
    ww = ssi.sige_pack_weights(wk, g)
    gen = torch.Generator().manual_seed(87)
    lst = torch.randperm(plan.cap, generator=gen)[:cnt].sort().values.to(torch.int32)
    idx = torch.zeros(plan.cap, dtype=torch.int32)
    idx[:cnt] = lst
    idx, count = idx.cuda(), torch.tensor([cnt], dtype=torch.int32, device="cuda")
    ws = torch.empty(max(plan.workspace_bytes, 16), dtype=torch.uint8, device="cuda")
    print(f"[case] {layer} packed: {cnt} of {plan.cap} blocks", flush=True)
    o1 = ssi.sige_sparse_conv_layer_auto(ag, wk, bg, cg, idx, count, g, workspace=ws)
    o2 = ssi.sige_sparse_conv_layer_auto(ag, wk, bg, cg, idx, count, g, workspace=ws, w_packed=ww)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.uint8), o2.view(torch.uint8))
    sub = torch.zeros(plan.cap, dtype=torch.uint8)
    sub[lst[torch.randperm(cnt, generator=gen)[:4]].long()] = 1
    sub = sub.view(1, nby, nbx)
    out = o2.cpu()
    r64 = oracle.sparse_layer(a_e, wt, bias, L.k, L.stride, L.pad, L.block, sub, out, out_f64=True)
    assert_close(out, r64, dt, active_pixels(sub, L.block, ho, wo), f"{layer} packed, sampled blocks")

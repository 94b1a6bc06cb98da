"""GPU parity: every step of the HIP path against the CPU oracle, through the C ABI.

Bit-exact: change masks, block lists, counts, gathered blocks, scatter, and every
output pixel outside the recomputed blocks.  Within tolerance (max abs error
<= TOL[dtype] * max|out|, TOL in _parity.py): convolution values.
"""
import numpy as np
import pytest
import torch

import oracle
import spatially_sparse_incremental_amd as ssi
import synth
from _parity import (DT, active_pixels, assert_close, bits, gpu, layer_inputs, rand, random_mask,
                     run_layer_gpu, run_layer_oracle)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# (name, n, h, w, cin, cout, k, s, p, b, dtype, dilate, edit fraction)
CASES = [
    ("rect_64x64x64_shape_f32", 1, 64, 64, 64, 64, 3, 1, 1, 8, "f32", 0, 0.01),
    ("ragged_bf16", 2, 13, 17, 40, 24, 3, 1, 1, 4, "bf16", 1, 0.02),
    ("stride2_f16", 1, 30, 26, 32, 48, 3, 2, 1, 3, "f16", 1, 0.02),
    ("pointwise_f16", 1, 20, 20, 320, 64, 1, 1, 0, 4, "f16", 1, 0.02),
    ("k5_f32", 1, 19, 23, 16, 16, 5, 1, 2, 3, "f32", 0, 0.02),
    ("tiny_blocks_f16", 1, 16, 16, 128, 128, 3, 1, 1, 2, "f16", 1, 0.03),
    ("one_px_blocks_bf16", 1, 9, 9, 32, 32, 3, 1, 1, 1, "bf16", 0, 0.05),
    ("wide_bf16", 1, 24, 40, 256, 160, 3, 1, 1, 6, "bf16", 1, 0.01),
    # one chunk of 4 K slices over 96 channels: the last slice starts past c_in
    ("slice_past_cin_bf16", 1, 20, 28, 96, 48, 3, 1, 1, 4, "bf16", 1, 0.03),
    # more listed blocks than one workgroup's threads (the copy's block bitmap is completed in a second pass)
    ("many_blocks_f16", 1, 96, 96, 32, 32, 3, 1, 1, 2, "f16", 1, 0.10),
]


def _geom(n, h, w, cin, cout, k, s, p, b):
    return ssi.geom(n, h, w, cin, cout, k, s, p, b)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("fused", [True, False], ids=["fused", "three_step"])
def test_layer_parity(case, fused):
    name, n, h, w, cin, cout, k, s, p, b, dts, d, frac = case
    dt = DT[dts]
    print(f"\n[case] {name} fused={fused}", flush=True)
    mask = random_mask(n, h, w, frac, 7)
    a_o, a_e, wt, bias = layer_inputs(n, h, w, cin, cout, k, dt, 11, mask)
    ho, wo, nby, nbx, ib = oracle.geometry(h, w, k, s, p, b)
    cache = rand((n, ho, wo, cout), dt, 13)
    g = _geom(n, h, w, cin, cout, k, s, p, b)
    ref = run_layer_oracle(a_o, a_e, wt, bias, cache, k, s, p, b, d)
    got = run_layer_gpu(a_o, a_e, wt, bias, cache, g, d, fused=fused)
    assert torch.equal(got["mask"], ref["mask"])
    assert got["count"] == ref["idx"].numel() > 0
    assert torch.equal(got["idx"], ref["idx"])
    print(f"[case] {name}: {got['count']} listed blocks", flush=True)
    sel = active_pixels(ref["act"], b, ho, wo)
    keep = ~sel.expand_as(cache)
    assert torch.equal(got["out"][keep].view(torch.uint8), cache[keep].view(torch.uint8))
    assert_close(got["out"], ref["out64"], dt, sel, name)
    if not fused:
        assert torch.equal(bits(got["blocks"]), bits(oracle.gather(a_e, k, s, p, b, ref["idx"])))
        ob64 = oracle.conv_blocks(got["blocks"], wt, bias, k, s, b, out_f64=True)
        assert_close(got["out_blocks"], ob64, dt, None, name + " conv_blocks")
        sc = oracle.scatter(got["out_blocks"], ref["idx"], cache, b)
        assert torch.equal(bits(got["out"]), bits(sc))


@pytest.mark.parametrize("case", CASES[:4], ids=[c[0] for c in CASES[:4]])
def test_fused_equals_three_steps_and_is_deterministic(case):
    name, n, h, w, cin, cout, k, s, p, b, dts, d, frac = case
    dt = DT[dts]
    mask = random_mask(n, h, w, frac, 21)
    a_o, a_e, wt, bias = layer_inputs(n, h, w, cin, cout, k, dt, 23, mask)
    ho, wo, _, _, _ = oracle.geometry(h, w, k, s, p, b)
    cache = rand((n, ho, wo, cout), dt, 25)
    g = _geom(n, h, w, cin, cout, k, s, p, b)
    r1 = run_layer_gpu(a_o, a_e, wt, bias, cache, g, d, fused=True)
    r2 = run_layer_gpu(a_o, a_e, wt, bias, cache, g, d, fused=True)
    r3 = run_layer_gpu(a_o, a_e, wt, bias, cache, g, d, fused=False)
    assert torch.equal(bits(r1["out"]), bits(r2["out"]))
    assert torch.equal(bits(r1["out"]), bits(r3["out"]))


@pytest.mark.parametrize("fused", [True, False])
def test_persistent_buffer_mode(fused):
    # copy_cached = 0: only listed blocks are written into a buffer that holds the cache
    n, h, w, cin, cout, k, s, p, b = 1, 40, 36, 64, 32, 3, 1, 1, 6
    dt = torch.bfloat16
    mask = random_mask(n, h, w, 0.02, 31)
    a_o, a_e, wt, bias = layer_inputs(n, h, w, cin, cout, k, dt, 33, mask)
    cache = rand((n, h, w, cout), dt, 35)
    g = _geom(n, h, w, cin, cout, k, s, p, b)
    a = run_layer_gpu(a_o, a_e, wt, bias, cache, g, 1, fused=fused, copy=True)
    c = run_layer_gpu(a_o, a_e, wt, bias, cache, g, 1, fused=fused, copy=False)
    assert torch.equal(bits(a["out"]), bits(c["out"]))


@pytest.mark.parametrize("dts", ["f32", "bf16", "f16"])
def test_delta_kernel_is_bit_exact(dts):
    # centre-tap identity weights, zero bias: recomputed pixels equal A_e exactly
    dt = DT[dts]
    n, h, w, c, b = 1, 22, 27, 32, 5
    wt = torch.zeros((c, c, 3, 3))
    wt[torch.arange(c), torch.arange(c), 1, 1] = 1.0
    wt = wt.to(dt)
    mask = random_mask(n, h, w, 0.03, 41)
    a_o = rand((n, h, w, c), dt, 42)
    a_e = synth.make_edit(a_o, mask, "replace", 43)
    cache = rand((n, h, w, c), dt, 44)
    g = _geom(n, h, w, c, c, 3, 1, 1, b)
    got = run_layer_gpu(a_o, a_e, wt, None, cache, g, 1)
    ref = run_layer_oracle(a_o, a_e, wt, None, cache, 3, 1, 1, b, 1)
    assert torch.equal(bits(got["out"]), bits(oracle.round_to(ref["out64"], dt)))


def test_integer_valued_fp32_is_bit_exact():
    n, h, w, c, b = 1, 20, 18, 16, 4
    gen = torch.Generator().manual_seed(51)
    a_o = torch.randint(-2, 3, (n, h, w, c), generator=gen).float()
    mask = random_mask(n, h, w, 0.05, 52)
    a_e = torch.where(torch.from_numpy(mask).bool()[..., None],
                      torch.randint(-2, 3, (n, h, w, c), generator=gen).float(), a_o)
    wt = torch.randint(-2, 3, (c, c, 3, 3), generator=gen).float()
    bias = torch.randint(-2, 3, (c,), generator=gen).float()
    cache = torch.zeros((n, h, w, c))
    g = _geom(n, h, w, c, c, 3, 1, 1, b)
    got = run_layer_gpu(a_o, a_e, wt, bias, cache, g, 0)
    ref = run_layer_oracle(a_o, a_e, wt, bias, cache, 3, 1, 1, b, 0)
    assert torch.equal(got["out"].double(), ref["out64"])


@pytest.mark.parametrize("dts", ["bf16", "f16", "f32"])
def test_empty_edit_returns_cache_bit_for_bit(dts):
    dt = DT[dts]
    n, h, w, c = 1, 48, 40, 32
    a = rand((n, h, w, c), dt, 61)
    wt = rand((c, c, 3, 3), dt, 62, 0.1)
    cache = rand((n, h, w, c), dt, 63)
    g = _geom(n, h, w, c, c, 3, 1, 1, 6)
    for fused in (True, False):
        got = run_layer_gpu(a, a.clone(), wt, None, cache, g, 1, fused=fused)
        assert got["count"] == 0 and int(got["mask"].sum()) == 0
        assert torch.equal(bits(got["out"]), bits(cache))


def test_single_layer_sparse_equals_dense_edited():
    # cache = conv(A_o) from the oracle; the sparse result must equal conv(A_e)
    n, h, w, c, k, b = 1, 36, 30, 64, 3, 6
    dt = torch.bfloat16
    mask = np.zeros((n, h, w), np.uint8)
    mask[0, 10:14, 7:12] = 1
    mask[0, 30, 25] = 1
    a_o, a_e, wt, bias = layer_inputs(n, h, w, c, c, k, dt, 71, mask)
    cache = oracle.dense_conv(a_o, wt, bias, k, 1, 1)
    g = _geom(n, h, w, c, c, k, 1, 1, b)
    got = run_layer_gpu(a_o, a_e, wt, bias, cache, g, 0)
    dense64 = oracle.dense_conv(a_e, wt, bias, k, 1, 1, out_f64=True)
    assert_close(got["out"], dense64, dt, None, "sparse vs dense edited")


@pytest.mark.parametrize("fused", [True, False], ids=["fused", "three_step"])
def test_block_grid_beyond_the_reduce_limit(fused):
    # 200x200 one-pixel blocks: 40000 blocks, more than sige_reduce_mask takes, so
    # the list comes from the oracle; the copy marks listed blocks without the
    # static LDS bitmap
    n, h, w, c, k, s, p, b = 1, 200, 200, 16, 3, 1, 1, 1
    dt = torch.bfloat16
    mask = random_mask(n, h, w, 0.03, 17)
    a_o, a_e, wt, bias = layer_inputs(n, h, w, c, c, k, dt, 18, mask)
    cache = rand((n, h, w, c), dt, 19)
    act = oracle.block_activity(torch.from_numpy(mask), h, w, k, s, p, b, 0)
    ref_idx = oracle.index_list(act)
    cap = h * w
    idx = torch.zeros(cap, dtype=torch.int32)
    idx[:ref_idx.numel()] = ref_idx
    idx, count = idx.cuda(), torch.tensor([ref_idx.numel()], dtype=torch.int32).cuda()
    g = _geom(n, h, w, c, c, k, s, p, b)
    wk, bs, ae, cg = ssi.weight_to_krsc(wt).cuda(), bias.cuda(), a_e.cuda(), cache.cuda()
    if fused:
        out = ssi.sige_sparse_conv_layer(ae, wk, bs, cg, idx, count, g)
    else:
        blocks = ssi.sige_gather(ae, g, idx, count)
        out = ssi.sige_scatter(ssi.sige_conv_blocks(blocks, wk, bs, g, count), idx, count, g, cg)
    torch.cuda.synchronize()
    ref = oracle.sparse_layer(a_e, wt, bias, k, s, p, b, act, cache, out_f64=True)
    sel = active_pixels(act, b, h, w)
    o = out.cpu()
    keep = ~sel.expand_as(cache)
    assert torch.equal(o[keep].view(torch.uint8), cache[keep].view(torch.uint8))
    assert_close(o, ref, dt, sel, "40000-block grid")


def test_all_active_is_dense_conv():
    n, h, w, c = 1, 32, 32, 64
    dt = torch.float16
    mask = np.ones((n, h, w), np.uint8)
    a_o, a_e, wt, bias = layer_inputs(n, h, w, c, c, 3, dt, 81, mask)
    cache = rand((n, h, w, c), dt, 82)
    g = _geom(n, h, w, c, c, 3, 1, 1, 4)
    got = run_layer_gpu(a_o, a_e, wt, bias, cache, g, 1)
    assert got["count"] == 64
    assert_close(got["out"], oracle.dense_conv(a_e, wt, bias, 3, 1, 1, out_f64=True), dt, None, "all active")


# ---------------------------------------------------------------------------
# step 1 and step 2 on their own
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("shape,dts", [((1, 64, 64, 64), "f32"), ((2, 7, 9, 8), "bf16"), ((1, 5, 13, 320), "f16"),
                                       ((1, 3, 3, 1024), "bf16"), ((3, 11, 1, 16), "f16")])
def test_diff_parity(shape, dts):
    dt = DT[dts]
    n, h, w, c = shape
    mask = random_mask(n, h, w, 0.1, 91)
    a_o = rand(shape, dt, 92)
    a_e = synth.make_edit(a_o, mask, "replace", 93)
    # single-channel and boundary changes
    a_e[0, 0, 0, c - 1] = a_o[0, 0, 0, c - 1] + 1
    got = ssi.sige_diff_mask(gpu(a_o), gpu(a_e), 1e-6).cpu()
    assert torch.equal(got, oracle.diff_mask(a_o, a_e, 1e-6))


def test_diff_threshold_boundary_on_gpu():
    tau = np.float32(1e-6)
    a_o = torch.zeros((1, 2, 3, 4))
    a_e = a_o.clone()
    a_e[0, 0, 0, 3] = float(tau)
    a_e[0, 0, 1, 3] = float(np.nextafter(tau, np.float32(1)))
    a_e[0, 1, 2, 0] = -float(np.nextafter(tau, np.float32(1)))
    a_e[0, 1, 0, 2] = float(np.nextafter(tau, np.float32(0)))
    got = ssi.sige_diff_mask(gpu(a_o), gpu(a_e), float(tau)).cpu()
    assert got.tolist() == [[[0, 1, 0], [0, 0, 1]]]


REDUCE = [  # (n, h, w, f, k, s, p, b, dilate, frac)
    (1, 256, 256, 1, 3, 1, 1, 6, 1, 0.002),
    (2, 13, 17, 1, 3, 1, 1, 4, 2, 0.02),
    (1, 128, 128, 2, 3, 2, 1, 6, 1, 0.001),
    (1, 32, 32, 8, 3, 1, 1, 4, 1, 0.0005),
    (1, 16, 16, 4, 1, 1, 0, 2, 1, 0.002),
    (1, 21, 19, 3, 3, 1, 1, 5, 0, 0.003),  # mask width 57: byte path
    (1, 256, 512, 1, 3, 1, 1, 6, 1, 0.001),
    (1, 64, 64, 1, 5, 1, 2, 3, 3, 0.001),
    (1, 9, 9, 1, 3, 1, 1, 1, 0, 0.05),
    (1, 24, 20, 1, 1, 2, 0, 3, 1, 0.02),       # 1x1 stride 2: neighbouring windows do not touch
    (2, 30, 22, 2, 1, 3, 0, 2, 2, 0.01),       # windows with gaps, two images, pooled
    (1, 512, 1024, 1, 3, 1, 1, 6, 1, 0.0005),  # pooled bits exceed one workgroup's LDS: two-launch path
    (2, 96, 640, 2, 3, 2, 1, 4, 2, 0.001),    # two-launch path, two images, stride 2, pooled
]


@pytest.mark.parametrize("case", REDUCE)
def test_reduce_parity(case):
    n, h, w, f, k, s, p, b, d, frac = case
    print(f"\n[reduce] {case}", flush=True)
    m = torch.from_numpy(random_mask(n, h * f, w * f, frac, 101 + h + w))
    g = _geom(n, h, w, 8, 8, k, s, p, b)
    idx, count = ssi.sige_reduce_mask(gpu(m), g, d)
    torch.cuda.synchronize()
    cnt = int(count.item())
    ref = oracle.index_list(oracle.block_activity(m, h, w, k, s, p, b, d))
    assert cnt == ref.numel()
    assert torch.equal(idx[:cnt].cpu(), ref)
    # empty and full masks
    idx, count = ssi.sige_reduce_mask(gpu(torch.zeros_like(m)), g, d)
    assert int(count.item()) == 0
    idx, count = ssi.sige_reduce_mask(gpu(torch.ones_like(m)), g, d)
    cap = ssi.sige_max_blocks(g)
    assert int(count.item()) == cap
    assert torch.equal(idx[:cap].cpu(), torch.arange(cap, dtype=torch.int32))


@pytest.mark.parametrize("case", [REDUCE[0], REDUCE[1], REDUCE[5], REDUCE[10], REDUCE[11]])
def test_reduce_with_copy(case):
    # the same list as sige_reduce_mask, and out == cached bit for bit (one- and two-launch paths)
    n, h, w, f, k, s, p, b, d, frac = case
    print(f"\n[reduce+copy] {case}", flush=True)
    m = gpu(torch.from_numpy(random_mask(n, h * f, w * f, frac, 101 + h + w)))
    cout = 24
    g = _geom(n, h, w, 8, cout, k, s, p, b)
    ho, wo, _, _, _ = oracle.geometry(h, w, k, s, p, b)
    cache = rand((n, ho, wo, cout), torch.bfloat16, 77).cuda()
    ref_idx, ref_cnt = ssi.sige_reduce_mask(m, g, d)
    idx, cnt, out = ssi.sige_reduce_mask_copy(m, g, d, cache)
    torch.cuda.synchronize()
    c = int(cnt.item())
    assert c == int(ref_cnt.item())
    assert torch.equal(idx[:c], ref_idx[:c])
    assert torch.equal(bits(out), bits(cache))


@pytest.mark.parametrize("case", CASES[:4] + CASES[5:6], ids=[c[0] for c in CASES[:4] + CASES[5:6]])
def test_step_with_copy_in_the_reduce(case):
    # diff -> reduce+copy -> fused conv (copy_cached = 0) == diff -> reduce -> fused conv (copy_cached = 1)
    name, n, h, w, cin, cout, k, s, p, b, dts, d, frac = case
    dt = DT[dts]
    mask = random_mask(n, h, w, frac, 7)
    a_o, a_e, wt, bias = layer_inputs(n, h, w, cin, cout, k, dt, 11, mask)
    ho, wo, _, _, _ = oracle.geometry(h, w, k, s, p, b)
    cache = rand((n, ho, wo, cout), dt, 13).cuda()
    g = _geom(n, h, w, cin, cout, k, s, p, b)
    ae, wk, bs = a_e.cuda(), ssi.weight_to_krsc(wt).cuda(), bias.cuda()
    mk = ssi.sige_diff_mask(a_o.cuda(), ae, 1e-6)
    idx, cnt = ssi.sige_reduce_mask(mk, g, d)
    lit = ssi.sige_sparse_conv_layer(ae, wk, bs, cache, idx, cnt, g)
    idx2, cnt2, out = ssi.sige_reduce_mask_copy(mk, g, d, cache)
    ssi.sige_sparse_conv_layer(ae, wk, bs, None, idx2, cnt2, g, out=out, copy_cached=False)
    torch.cuda.synchronize()
    assert torch.equal(bits(out), bits(lit)), name


def test_reduce_at_its_limits():
    # widest conv input (8192) and largest block grid (16384) accepted, on both reduce paths
    for (h, w, b) in [(256, 1024, 16), (128, 128, 1), (16, 8192, 32), (1024, 8192, 32), (2048, 512, 8)]:
        g = _geom(1, h, w, 8, 8, 3, 1, 1, b)
        m = torch.from_numpy(random_mask(1, h, w, 0.0005, 111))
        idx, count = ssi.sige_reduce_mask(gpu(m), g, 1)
        torch.cuda.synchronize()
        ref = oracle.index_list(oracle.block_activity(m, h, w, 3, 1, 1, b, 1))
        assert torch.equal(idx[:int(count.item())].cpu(), ref)


def test_outputs_have_no_stray_writes():
    # guard canaries around every output of the fused and three-step paths
    n, h, w, c, b = 1, 30, 30, 64, 6
    dt = torch.bfloat16
    mask = random_mask(n, h, w, 0.03, 121)
    a_o, a_e, wt, bias = layer_inputs(n, h, w, c, c, 3, dt, 122, mask)
    g = _geom(n, h, w, c, c, 3, 1, 1, b)
    cap = ssi.sige_max_blocks(g)
    G = 4096
    cache = gpu(rand((n, h, w, c), dt, 123))
    ae, wk, bs = gpu(a_e), gpu(ssi.weight_to_krsc(wt)), gpu(bias)
    m = ssi.sige_diff_mask(gpu(a_o), ae)
    idx_buf = torch.full((cap + G,), -7, dtype=torch.int32, device="cuda")
    cnt_buf = torch.full((1 + G,), -7, dtype=torch.int32, device="cuda")
    idx, count = ssi.sige_reduce_mask(m, g, 1, idx=idx_buf[:cap], count=cnt_buf[:1])
    nout = n * h * w * c
    out_buf = torch.full((nout + G,), 3.0, dtype=dt, device="cuda")
    ssi.sige_sparse_conv_layer(ae, wk, bs, cache, idx, count, g, out=out_buf[:nout].view(n, h, w, c))
    ib = ssi.sige_geom_derive(g).ib
    nb = cap * ib * ib * c
    blk_buf = torch.full((nb + G,), 5.0, dtype=dt, device="cuda")
    ssi.sige_gather(ae, g, idx, count, blocks=blk_buf[:nb].view(cap, ib, ib, c))
    torch.cuda.synchronize()
    cnt = int(count.item())
    assert (idx_buf[cap:] == -7).all() and (cnt_buf[1:] == -7).all()
    assert (idx_buf[cnt:cap] == -7).all()  # unused list entries are untouched
    assert (out_buf[nout:] == 3.0).all() and (blk_buf[nb:] == 5.0).all()
    assert (blk_buf[cnt * ib * ib * c:nb] == 5.0).all()  # unused block slots untouched


def test_more_outputs_have_no_stray_writes():
    # guard canaries after the outputs of the block conv, the scatter, the split
    # layer (and its workspace), the restore and the attention
    n, h, w, c, b = 1, 30, 30, 64, 6
    dt = torch.bfloat16
    G = 4096
    mask = random_mask(n, h, w, 0.03, 141)
    a_o, a_e, wt, bias = layer_inputs(n, h, w, c, c, 3, dt, 142, mask)
    g = _geom(n, h, w, c, c, 3, 1, 1, b)
    d = ssi.sige_geom_derive(g)
    cap = d.cap
    cache = gpu(rand((n, h, w, c), dt, 143))
    ae, wk, bs = gpu(a_e), gpu(ssi.weight_to_krsc(wt)), gpu(bias)
    idx, count = ssi.sige_reduce_mask(ssi.sige_diff_mask(gpu(a_o), ae), g, 1)
    blocks = ssi.sige_gather(ae, g, idx, count)

    def guarded(numel, fill, dtype=dt):
        buf = torch.full((numel + G,), fill, dtype=dtype, device="cuda")
        return buf, buf[:numel]

    nob = cap * b * b * c
    ob_buf, ob = guarded(nob, 5.0)
    ssi.sige_conv_blocks(blocks, wk, bs, g, count, out_blocks=ob.view(cap, b, b, c))
    nout = n * h * w * c
    sc_buf, sc = guarded(nout, 3.0)
    ssi.sige_scatter(ob.view(cap, b, b, c), idx, count, g, cache, out=sc.view(n, h, w, c))
    sp_buf, sp = guarded(nout, 3.0)
    nws = ssi.sige_sparse_conv_layer_split_workspace(g, dt)
    ws_buf, ws = guarded(nws, 9, torch.uint8)
    ssi.sige_sparse_conv_layer_split(ae, wk, bs, cache, idx, count, g, out=sp.view(n, h, w, c), workspace=ws)
    rs_buf, rs = guarded(nout, 3.0)
    rs.copy_(cache.view(-1))
    ssi.sige_restore_blocks(idx, count, None, None, g, cache, rs.view(n, h, w, c))
    heads = 1
    q, k, v = (gpu(rand((n, h, w, 64), dt, 150 + i)) for i in range(3))
    ga = _geom(n, h, w, 64, 64, 1, 1, 0, 5)
    ia, ca = ssi.sige_reduce_mask(ssi.sige_diff_mask(gpu(a_o[..., :64].contiguous()), gpu(a_e[..., :64].contiguous())),
                                  ga, 1)
    at_buf, at = guarded(n * h * w * 64, 3.0)
    nwa = ssi.sige_sparse_attention_workspace(n, h, w, heads, 64, 5)
    wa_buf, wa = guarded(nwa, 9, torch.uint8)
    ssi.sige_sparse_attention(q, k, v, ia, ca, heads, 5, cached=gpu(rand((n, h, w, 64), dt, 154)),
                              out=at.view(n, h, w, 64), workspace=wa)
    torch.cuda.synchronize()
    cnt = int(count.item())
    assert cnt > 0 and int(ca.item()) > 0
    assert (ob_buf[nob:] == 5.0).all() and (ob_buf[cnt * b * b * c:nob] == 5.0).all()  # unused slots untouched
    assert (sc_buf[nout:] == 3.0).all() and (sp_buf[nout:] == 3.0).all() and (rs_buf[nout:] == 3.0).all()
    assert (ws_buf[nws:] == 9).all() and (wa_buf[nwa:] == 9).all()
    assert (at_buf[n * h * w * 64:] == 3.0).all()


def test_batch_of_two_images():
    n, h, w, c, b = 2, 24, 20, 32, 4
    dt = torch.float16
    mask = np.zeros((n, h, w), np.uint8)
    mask[1, 5:8, 6:9] = 1  # only the second image is edited
    a_o, a_e, wt, bias = layer_inputs(n, h, w, c, c, 3, dt, 131, mask)
    cache = rand((n, h, w, c), dt, 132)
    g = _geom(n, h, w, c, c, 3, 1, 1, b)
    got = run_layer_gpu(a_o, a_e, wt, bias, cache, g, 1)
    ref = run_layer_oracle(a_o, a_e, wt, bias, cache, 3, 1, 1, b, 1)
    assert torch.equal(got["idx"], ref["idx"]) and int(ref["idx"].min()) >= 30  # 5 x 6 blocks per image
    assert torch.equal(bits(got["out"][0]), bits(cache[0]))
    assert_close(got["out"], ref["out64"], dt, active_pixels(ref["act"], b, h, w), "batch")

"""Query-pruned self-attention on the GPU against the oracle (fp64)."""
import numpy as np
import pytest
import torch

import oracle
import spatially_sparse_incremental_amd as ssi
import synth
from _parity import TOL, bits, note_error, rand

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _list(act, cap):
    idx = oracle.index_list(act)
    buf = torch.zeros(cap, dtype=torch.int32)
    buf[:idx.numel()] = idx
    return buf.cuda(), torch.tensor([idx.numel()], dtype=torch.int32).cuda(), idx


def _check(got, ref64, cache, act, b, dt, what):
    n, h, w, c = got.shape
    sel = act.bool().repeat_interleave(b, 1).repeat_interleave(b, 2)[:, :h, :w, None].expand_as(got)
    assert torch.equal(got[~sel].view(torch.uint8), cache[~sel].view(torch.uint8)), what + ": pruned tokens"
    if sel.any():
        g64, r64 = got.double()[sel], ref64[sel]
        err = (g64 - r64).abs().max().item()
        scale = r64.abs().max().item()
        print(f"[case] {what}: max relative error {err / scale:.2e}", flush=True)
        note_error(dt, err / scale, what)
        assert err <= TOL[dt] * scale, f"{what}: max err {err:.3e} vs scale {scale:.3e}"
        return err / scale
    return 0.0


@pytest.mark.parametrize("n,h,w,heads,b,dts,frac", [
    (1, 16, 16, 2, 4, "f16", 0.3),    # 256 tokens: 4 key tiles
    (2, 13, 11, 3, 4, "bf16", 0.4),   # a ragged key tile, partial blocks, two images
    (1, 32, 24, 1, 2, "f16", 0.15),   # 4-token blocks
    (1, 9, 7, 2, 1, "bf16", 0.5),     # one-token blocks, 63 keys
    (3, 20, 20, 4, 5, "f16", 0.2),    # 25-token blocks over three images
])
def test_attention_parity(n, h, w, heads, b, dts, frac):
    dt = {"f16": torch.float16, "bf16": torch.bfloat16}[dts]
    c = heads * 64
    q, k, v = (rand((n, h, w, c), dt, 601 + i) for i in range(3))
    cache = rand((n, h, w, c), dt, 605)
    nby, nbx = -(-h // b), -(-w // b)
    rng = np.random.default_rng(606)
    act = torch.from_numpy((rng.random((n, nby, nbx)) < frac).astype(np.uint8))
    act.view(-1)[0] = 1
    idx_g, cnt_g, idx = _list(act, n * nby * nbx)
    print(f"\n[case] attention {n}x{h}x{w} heads {heads} b {b} {dts}: {idx.numel()} blocks", flush=True)
    out = ssi.sige_sparse_attention(q.cuda(), k.cuda(), v.cuda(), idx_g, cnt_g, heads, b, cached=cache.cuda())
    torch.cuda.synchronize()
    ref = oracle.sparse_attention(q, k, v, heads, b, act, cache, out_f64=True)
    _check(out.cpu(), ref, cache, act, b, dt, "attention")


def test_attention_all_blocks_and_no_block():
    n, h, w, heads, b = 1, 12, 12, 2, 4
    dt = torch.float16
    q, k, v = (rand((n, h, w, heads * 64), dt, 611 + i) for i in range(3))
    cache = rand((n, h, w, heads * 64), dt, 615)
    act = torch.ones((n, 3, 3), dtype=torch.uint8)
    idx_g, cnt_g, _ = _list(act, 9)
    out = ssi.sige_sparse_attention(q.cuda(), k.cuda(), v.cuda(), idx_g, cnt_g, heads, b, cached=cache.cuda())
    torch.cuda.synchronize()
    _check(out.cpu(), oracle.sparse_attention(q, k, v, heads, b, None, None, out_f64=True), cache, act, b, dt, "all")
    none = torch.zeros(1, dtype=torch.int32).cuda()
    out0 = ssi.sige_sparse_attention(q.cuda(), k.cuda(), v.cuda(), idx_g, none, heads, b, cached=cache.cuda())
    torch.cuda.synchronize()
    assert torch.equal(bits(out0.cpu()), bits(cache))


def test_attention_persistent_buffer_mode():
    n, h, w, heads, b = 1, 16, 16, 2, 4
    dt = torch.bfloat16
    q, k, v = (rand((n, h, w, heads * 64), dt, 621 + i) for i in range(3))
    cache = rand((n, h, w, heads * 64), dt, 625)
    act = torch.zeros((1, 4, 4), dtype=torch.uint8)
    act[0, 1, 2] = act[0, 3, 0] = 1
    idx_g, cnt_g, _ = _list(act, 16)
    lit = ssi.sige_sparse_attention(q.cuda(), k.cuda(), v.cuda(), idx_g, cnt_g, heads, b, cached=cache.cuda())
    per = cache.cuda()
    ssi.sige_sparse_attention(q.cuda(), k.cuda(), v.cuda(), idx_g, cnt_g, heads, b, out=per, copy_cached=False)
    torch.cuda.synchronize()
    assert torch.equal(bits(lit.cpu()), bits(per.cpu()))


def test_attention_latent_diffusion_shape_with_a_blob_edit():
    # 64x64 tokens, 5 heads of 64, fp16; query blocks of 4x4 tokens from the diff of
    # a 1.2% blob edit (k = 1 geometry, dilation 1), every listed token checked on a
    # sample of blocks against the oracle, the pruned tokens bit for bit
    wl = synth.workload("ldm_64x64x320_f16")
    h = w = 64
    heads, b, dt = 5, 4, torch.float16
    m = synth.edit_shape(wl, 3).raster(h, w)
    x_o = synth.make_activation(1, h, w, heads * 64, "f16", 31)
    x_e = synth.make_edit(x_o, m, "replace", 32)
    q, k, v = (rand((1, h, w, heads * 64), dt, 631 + i, 0.5) for i in range(3))
    cache = rand((1, h, w, heads * 64), dt, 635)
    g = ssi.geom(1, h, w, heads * 64, heads * 64, 1, 1, 0, b)
    mask = ssi.sige_diff_mask(x_o.cuda(), x_e.cuda(), wl.tau)
    idx, cnt = ssi.sige_reduce_mask(mask, g, 1)
    out = ssi.sige_sparse_attention(q.cuda(), k.cuda(), v.cuda(), idx, cnt, heads, b, cached=cache.cuda())
    torch.cuda.synchronize()
    count = int(cnt.item())
    lst = idx[:count].cpu()
    act = oracle.block_activity(mask.cpu(), h, w, 1, 1, 0, b, 1)
    assert torch.equal(lst, oracle.index_list(act))
    print(f"\n[case] ldm attention: {count} query blocks", flush=True)
    o = out.cpu()
    keep = ~act.bool().repeat_interleave(b, 1).repeat_interleave(b, 2)[..., None].expand_as(o)
    assert torch.equal(o[keep].view(torch.uint8), cache[keep].view(torch.uint8))
    pick = np.random.default_rng(7).choice(lst.numpy(), size=min(6, count), replace=False)
    sub = torch.zeros_like(act)
    sub.view(-1)[torch.from_numpy(pick).long()] = 1
    ref = oracle.sparse_attention(q, k, v, heads, b, sub, o, out_f64=True)
    _check(o, ref, o, sub, b, dt, "ldm attention sample")

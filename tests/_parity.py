"""Shared helpers of the GPU parity tests: inputs from `synth`, expected values
from `oracle` (CPU), results from the HIP library through its binding."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import spatially_sparse_incremental_amd as ssi
import synth

DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
# max |gpu - oracle| <= TOL * max |oracle| over the recomputed pixels.
# fp32 1e-4 and bf16 2e-2 are the bounds the method's statement gives.  fp16
# has none there; it is derived from the arithmetic: products of fp16 values
# are exact in fp32, so a recomputed value carries the one final rounding (at
# most 2^-11 = 4.9e-4 of |out|) plus the fp32 accumulation over K <= 11520
# terms (a few 2^-24 * sqrt(K) * sum|a w|), and the attention's probabilities
# are rounded to fp16 (2^-11 each) before their product with V.  3e-3 is six
# fp16 roundoff units: errors measured on every fp16 case stay below 1.5e-3.
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2, torch.float16: 3e-3}
# largest observed max|gpu - oracle| / max|oracle| per dtype in this session
# (reported at the end of the run by conftest.py)
WORST = {}


def note_error(dt, rel, what=""):
    """Records one case's relative error, for the end-of-session report."""
    cur = WORST.get(dt)
    if cur is None or rel > cur[0]:
        WORST[dt] = (rel, what)


def rand(shape, dtype, seed, std=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g, dtype=torch.float32) * std).to(dtype)


def bits(t):
    """Raw storage of a tensor, for bit-exact comparison."""
    return t.contiguous().view(torch.uint8)


def layer_inputs(n, h, w, cin, cout, k, dt, seed, mask, std=None):
    """A_o, A_e (differs exactly on `mask`), weight OIHW, bias, on the CPU."""
    a_o = rand((n, h, w, cin), dt, seed)
    a_e = synth.make_edit(a_o, mask, "replace", seed + 1)
    std = std if std is not None else (2.0 / (cin * k * k)) ** 0.5
    wt = rand((cout, cin, k, k), dt, seed + 2, std)
    bias = rand((cout,), torch.float32, seed + 3, 0.01)
    return a_o, a_e, wt, bias


def random_mask(n, h, w, frac, seed):
    rng = np.random.default_rng(seed)
    return (rng.random((n, h, w)) < frac).astype(np.uint8)


def gpu(t):
    return t.to("cuda") if t is not None else None


def active_pixels(act, b, ho, wo):
    """bool [n, ho, wo, 1]: output pixel lies in an active block."""
    up = act.bool().repeat_interleave(b, 1).repeat_interleave(b, 2)[:, :ho, :wo]
    return up[..., None]


def assert_close(got, ref64, dt, sel=None, what=""):
    """max |got - ref| <= TOL[dt] * max |ref| over the selected elements."""
    g = got.double()
    if sel is not None:
        sel = sel.expand_as(g)
        g, ref64 = g[sel], ref64[sel]
    if g.numel() == 0:
        return 0.0
    scale = ref64.abs().max().item()
    err = (g - ref64).abs().max().item()
    note_error(dt, err / max(scale, 1e-30), what)
    assert err <= TOL[dt] * max(scale, 1e-30), f"{what}: max err {err:.3e} vs scale {scale:.3e} (tol {TOL[dt]})"
    return err / max(scale, 1e-30)


def run_layer_gpu(a_o, a_e, wt, bias, cache, g, dilate, tau=1e-6, fused=True, copy=True):
    """diff -> reduce -> (fused | gather+conv+scatter) on the GPU; returns CPU tensors."""
    ao, ae = gpu(a_o), gpu(a_e)
    wk = gpu(ssi.weight_to_krsc(wt))
    bs = gpu(bias)
    cg = gpu(cache)
    mask = ssi.sige_diff_mask(ao, ae, tau)
    idx, count = ssi.sige_reduce_mask(mask, g, dilate)
    if fused:
        out = ssi.sige_sparse_conv_layer(ae, wk, bs, cg, idx, count, g, copy_cached=True) if copy else None
        if not copy:
            out = cg.clone()
            ssi.sige_sparse_conv_layer(ae, wk, bs, None, idx, count, g, out=out, copy_cached=False)
        blocks = ob = None
    else:
        blocks = ssi.sige_gather(ae, g, idx, count)
        ob = ssi.sige_conv_blocks(blocks, wk, bs, g, count)
        if copy:
            out = ssi.sige_scatter(ob, idx, count, g, cg)
        else:
            out = cg.clone()
            ssi.sige_scatter(ob, idx, count, g, None, out=out, copy_cached=False)
    torch.cuda.synchronize()
    cnt = int(count.item())
    res = dict(mask=mask.cpu(), idx=idx[:cnt].cpu(), count=cnt, out=out.cpu())
    if blocks is not None:
        res["blocks"] = blocks[:cnt].cpu()
        res["out_blocks"] = ob[:cnt].cpu()
    return res


def run_layer_oracle(a_o, a_e, wt, bias, cache, k, s, p, b, dilate, tau=1e-6):
    mask = oracle.diff_mask(a_o, a_e, tau)
    n, h, w, _ = a_o.shape
    act = oracle.block_activity(mask, h, w, k, s, p, b, dilate)
    idx = oracle.index_list(act)
    out64 = oracle.sparse_layer(a_e, wt, bias, k, s, p, b, act, cache, out_f64=True)
    return dict(mask=mask, act=act, idx=idx, out64=out64)


def check_layer_sampled(name, a_e, wt, bias, cache, out, idx, L, mask_full, seed, sample=6):
    """Full-size check of one layer: the block list bit for bit, every pixel outside
    the listed blocks equal to the cache bit for bit, and `sample` listed blocks
    (None: every listed block) recomputed by the oracle (fp64) within tolerance.
    a_e, cache, out: CPU NHWC; idx: the GPU's list; mask_full: [n, hm, wm] diff
    mask.  Returns the relative error."""
    n, h, w, _ = a_e.shape
    act = oracle.block_activity(mask_full, h, w, L.k, L.stride, L.pad, L.block, L.dilate)
    ref_idx = oracle.index_list(act)
    assert torch.equal(idx, ref_idx), f"{name}: block list differs"
    ho, wo, nby, nbx, _ = oracle.geometry(h, w, L.k, L.stride, L.pad, L.block)
    pm = act.bool().repeat_interleave(L.block, 1).repeat_interleave(L.block, 2)[:, :ho, :wo, None]
    keep = ~pm.expand_as(cache)
    assert torch.equal(out[keep].view(torch.uint8), cache[keep].view(torch.uint8)), f"{name}: untouched pixels"
    if ref_idx.numel() == 0:
        return 0.0
    rng = np.random.default_rng(seed)
    pick = ref_idx.numpy() if sample is None else \
        rng.choice(ref_idx.numpy(), size=min(sample, ref_idx.numel()), replace=False)
    sub = torch.zeros_like(act)
    sub.view(-1)[torch.from_numpy(pick).long()] = 1
    ref = oracle.sparse_layer(a_e, wt, bias, L.k, L.stride, L.pad, L.block, sub, out, out_f64=True)
    sel = sub.bool().repeat_interleave(L.block, 1).repeat_interleave(L.block, 2)[:, :ho, :wo, None].expand_as(out)
    g64, r64 = out.double()[sel], ref[sel]
    scale = r64.abs().max().item()
    err = (g64 - r64).abs().max().item()
    note_error(out.dtype, err / max(scale, 1e-30), name)
    assert err <= TOL[out.dtype] * scale, f"{name}: max err {err:.3e} vs scale {scale:.3e}"
    return err / scale


def run_layer_full(a_e_gpu, wt, bias, cache_gpu, L, mask_gpu, layer=None):
    """reduce + fused layer (copy_cached = 1) on the GPU for layer spec L; returns (out, CPU list).
    layer: the entry point (default sige_sparse_conv_layer)."""
    g = ssi.geom(a_e_gpu.shape[0], L.h, L.w, L.c_in, L.c_out, L.k, L.stride, L.pad, L.block)
    idx, count = ssi.sige_reduce_mask(mask_gpu, g, L.dilate)
    layer = layer or ssi.sige_sparse_conv_layer
    out = layer(a_e_gpu, ssi.weight_to_krsc(wt).cuda(), bias.cuda(), cache_gpu, idx, count, g)
    torch.cuda.synchronize()
    return out, idx[:int(count.item())].cpu()

"""CPU oracle for tile-sparse incremental convolution -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package.  It wraps ``liboracle.so`` (plain C, built from
``sige_oracle.c`` by ``oracle/build.py``) with ctypes and takes/returns torch
CPU tensors used purely as containers.  It shares no code with the GPU library.

Functions and the passages they follow (page title, section):

* ``diff_mask``        -- mer.dev notes on "Efficient Spatially Sparse Inference
  for Conditional GANs and Diffusion Models", section 3; SIGE README mirror,
  Overview.  Pinned: generator edit regions, the strict tau boundary.
* ``block_activity``, ``index_list`` -- mer.dev notes section 3.2 (downsample,
  dilate, select tiles); SIGE README Overview (reduce to active block indices).
  Pinned: closed-form rectangle blocks, brute-force output-change test,
  max-pool formulations of pooling and dilation.
* ``sparse_layer``, ``dense_conv`` -- SIGE README Overview (scatter into the
  cached output); mer.dev notes 3.1 (linearity).  Pinned: torch fp64 conv2d,
  linearity, empty edit, delta kernel, brute force over block subsets.
* ``gather``, ``conv_blocks``, ``scatter`` -- SIGE README Overview (gather with
  overlap 2 for 3x3 s1, stack on batch, F_l, scatter).  Pinned: zero-padded
  slicing, torch fp64 valid conv, slicing.
* ``sparse_chain``     -- mer.dev notes section 3.2 (the mask downsampled to
  each layer's scale); the layer-wise update of the README Overview applied
  conv after conv.  Pinned: all-active chain equals the dense chain, an empty
  edit returns the caches, a dilation wider than the chain's halo equals the
  dense edited chain.
* ``restore_blocks``   -- nubint.ai review, ABSTRACT (sequential edits) and
  Proposed method (state kept between edits).  Pinned: a sequence of edits
  through one buffer equals each edit computed from scratch; exactly the
  blocks listed before and not now change.
* ``sparse_attention`` -- nubint.ai review, Proposed method (attention prunes
  the queries of unedited tokens).  Pinned: every query listed equals torch
  fp64 softmax(QK^T/sqrt(d))V; identical keys give the mean value; one
  dominant key returns its value; permuting keys with values changes nothing;
  unlisted tokens keep the cache bit for bit.
* ``round_to``         -- IEEE 754 binary16 / bfloat16 round-to-nearest-even.
  Pinned: hand-listed bit patterns, numpy float16 and torch bfloat16 casts.

No function is unpinned.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

DT = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2, torch.float64: 3}
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python oracle/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        c_int, c_long, c_void = ctypes.c_int, ctypes.c_long, ctypes.c_void_p
        L.oracle_round.restype = ctypes.c_double
        L.oracle_round.argtypes = [ctypes.c_double, c_int]
        L.oracle_encode.argtypes = [c_void, c_long, c_int, c_void]
        L.oracle_decode.argtypes = [c_void, c_long, c_int, c_void]
        L.oracle_geometry.argtypes = [c_int] * 6 + [c_void]
        L.oracle_diff_mask.argtypes = [c_void, c_void, c_int, c_int, c_int, c_int, c_int,
                                       c_long, c_long, c_long, c_long, ctypes.c_float, c_void]
        L.oracle_block_activity.argtypes = [c_void] + [c_int] * 10 + [c_void]
        L.oracle_index_list.restype = c_long
        L.oracle_index_list.argtypes = [c_void, c_long, c_void]
        L.oracle_sparse_layer.argtypes = (
            [c_void, c_int, c_int, c_int, c_int, c_int, c_long, c_long, c_long, c_long,
             c_void, c_void, c_int, c_int, c_int, c_int, c_int,
             c_void, c_void, c_void, c_int, c_long, c_long, c_long, c_long])
        L.oracle_gather.argtypes = [c_void, c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                    c_void, c_long, c_void]
        L.oracle_conv_blocks.argtypes = [c_void, c_int, c_long, c_int, c_int, c_void, c_void,
                                         c_int, c_int, c_int, c_int, c_void, c_int]
        L.oracle_scatter.argtypes = [c_void, c_int, c_long, c_void, c_int, c_int, c_int, c_int,
                                     c_int, c_void, c_void, c_int]
        L.oracle_num_threads.restype = c_int
        L.oracle_restore_blocks.argtypes = [c_void, c_long, c_void, c_long, c_int, c_int, c_int, c_int, c_int,
                                            c_int, c_void, c_void]
        L.oracle_sparse_attention.argtypes = [c_void, c_void, c_void, c_int, c_int, c_int, c_int, c_int, c_int,
                                              ctypes.c_double, c_int, c_void, c_void, c_void, c_int]
        L.oracle_set_threads.argtypes = [c_int]
        _lib = L
    return _lib


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_threads(t: int) -> None:
    lib().oracle_set_threads(int(t))


def geometry(h, w, k, s, p, b):
    """(ho, wo, nby, nbx, ib) of a k x k / stride s / pad p conv with b x b output blocks."""
    out = (ctypes.c_int * 5)()
    _check(lib().oracle_geometry(h, w, k, s, p, b, out), "geometry")
    return tuple(out)


def _strides(shape, layout):
    """Element strides (sn, sh, sw, sc) of a contiguous NHWC or NCHW tensor."""
    if layout == "NHWC":
        n, h, w, c = shape
        return n, h, w, c, (h * w * c, w * c, c, 1)
    n, c, h, w = shape
    return n, h, w, c, (c * h * w, w, 1, h * w)


# ---------------------------------------------------------------------------
def round_to(x: torch.Tensor, dtype) -> torch.Tensor:
    """Round fp64 values to `dtype` (f32/bf16/f16), nearest-even, as raw storage."""
    x = x.to(torch.float64).contiguous()
    out = torch.empty(x.shape, dtype=dtype)
    lib().oracle_encode(_ptr(x), x.numel(), DT[dtype], _ptr(out))
    return out


def decode(x: torch.Tensor) -> torch.Tensor:
    """Exact fp64 values of stored elements."""
    x = x.contiguous()
    out = torch.empty(x.shape, dtype=torch.float64)
    lib().oracle_decode(_ptr(x), x.numel(), DT[x.dtype], _ptr(out))
    return out


def diff_mask(a_orig: torch.Tensor, a_edit: torch.Tensor, tau: float = 1e-6, layout: str = "NHWC"):
    """uint8 [n, h, w]: 1 where some channel differs by more than tau (fp32 difference)."""
    assert a_orig.shape == a_edit.shape and a_orig.dtype == a_edit.dtype
    a_orig, a_edit = a_orig.contiguous(), a_edit.contiguous()
    n, h, w, c, (sn, sh, sw, sc) = _strides(a_orig.shape, layout)
    mask = torch.empty((n, h, w), dtype=torch.uint8)
    rc = lib().oracle_diff_mask(_ptr(a_orig), _ptr(a_edit), DT[a_orig.dtype], n, h, w, c,
                                sn, sh, sw, sc, ctypes.c_float(tau), _ptr(mask))
    _check(rc, "diff_mask")
    return mask


def block_activity(mask: torch.Tensor, h, w, k, s, p, b, dilate) -> torch.Tensor:
    """uint8 [n, nby, nbx]: blocks whose input window touches the (OR-pooled) mask, dilated."""
    mask = torch.as_tensor(mask).to(torch.uint8).contiguous()
    if mask.dim() == 2:
        mask = mask.unsqueeze(0)
    n, hm, wm = mask.shape
    _, _, nby, nbx, _ = geometry(h, w, k, s, p, b)
    act = torch.empty((n, nby, nbx), dtype=torch.uint8)
    rc = lib().oracle_block_activity(_ptr(mask), n, hm, wm, h, w, k, s, p, b, dilate, _ptr(act))
    _check(rc, "block_activity")
    return act


def index_list(active: torch.Tensor) -> torch.Tensor:
    """int32 ascending linear indices (n*nby + by)*nbx + bx of active blocks."""
    active = active.to(torch.uint8).contiguous()
    idx = torch.empty(max(active.numel(), 1), dtype=torch.int32)
    cnt = lib().oracle_index_list(_ptr(active), active.numel(), _ptr(idx))
    return idx[:cnt].clone()


def sparse_layer(a_edit, weight_oihw, bias, k, s, p, b, active, cache, layout="NHWC", out_f64=False):
    """Edited layer output: conv(A_e) on pixels of active blocks, cache elsewhere.

    a_edit: [n,h,w,cin] (NHWC) or [n,cin,h,w] (NCHW), storage dtype.
    weight_oihw: [cout, cin, k, k] storage dtype; bias fp32 [cout] or None.
    active: uint8 [n, nby, nbx] or None (dense conv).  cache: output layout, or None.
    """
    a_edit = a_edit.contiguous()
    dt = a_edit.dtype
    n, h, w, cin, (sn, sh, sw, sc) = _strides(a_edit.shape, layout)
    cout = weight_oihw.shape[0]
    assert weight_oihw.shape == (cout, cin, k, k) and weight_oihw.dtype == dt
    ho, wo, nby, nbx, _ = geometry(h, w, k, s, p, b)
    oshape = (n, ho, wo, cout) if layout == "NHWC" else (n, cout, ho, wo)
    _, _, _, _, (osn, osh, osw, osc) = _strides(oshape, layout)
    out = torch.empty(oshape, dtype=torch.float64 if out_f64 else dt)
    if active is not None:
        active = active.to(torch.uint8).contiguous()
        assert active.shape == (n, nby, nbx)
        cache = cache.contiguous()
        assert cache.shape == oshape and cache.dtype == dt
    wt = weight_oihw.contiguous()
    bias_t = bias.to(torch.float32).contiguous() if bias is not None else None
    rc = lib().oracle_sparse_layer(_ptr(a_edit), DT[dt], n, h, w, cin, sn, sh, sw, sc,
                                   _ptr(wt), _ptr(bias_t), cout, k, s, p, b,
                                   _ptr(active), _ptr(cache), _ptr(out), DT[out.dtype],
                                   osn, osh, osw, osc)
    _check(rc, "sparse_layer")
    return out


def dense_conv(a, weight_oihw, bias, k, s, p, layout="NHWC", out_f64=False):
    """The plain dense conv (every block active)."""
    return sparse_layer(a, weight_oihw, bias, k, s, p, 1, None, None, layout, out_f64)


def gather(a_nhwc, k, s, p, b, idx) -> torch.Tensor:
    """[count, ib, ib, cin] input windows of the listed blocks, zero outside the image."""
    a = a_nhwc.contiguous()
    n, h, w, cin = a.shape
    ib = geometry(h, w, k, s, p, b)[4]
    idx = idx.to(torch.int32).contiguous()
    blocks = torch.empty((idx.numel(), ib, ib, cin), dtype=a.dtype)
    rc = lib().oracle_gather(_ptr(a), DT[a.dtype], n, h, w, cin, k, s, p, b, _ptr(idx), idx.numel(),
                             _ptr(blocks))
    _check(rc, "gather")
    return blocks


def conv_blocks(blocks, weight_oihw, bias, k, s, b, out_f64=False) -> torch.Tensor:
    """[count, b, b, cout]: valid conv of each stacked block, plus bias."""
    blocks = blocks.contiguous()
    count, ib, _, cin = blocks.shape
    cout = weight_oihw.shape[0]
    out = torch.empty((count, b, b, cout), dtype=torch.float64 if out_f64 else blocks.dtype)
    bias_t = bias.to(torch.float32).contiguous() if bias is not None else None
    wt = weight_oihw.contiguous()
    rc = lib().oracle_conv_blocks(_ptr(blocks), DT[blocks.dtype], count, ib, cin, _ptr(wt), _ptr(bias_t),
                                  cout, k, s, b, _ptr(out), DT[out.dtype])
    _check(rc, "conv_blocks")
    return out


def scatter(out_blocks, idx, cache, b, copy_cached=True, out=None) -> torch.Tensor:
    """Cached output with each listed block's valid pixels overwritten (NHWC)."""
    out_blocks = out_blocks.contiguous()
    cache = cache.contiguous()
    n, ho, wo, cout = cache.shape
    if out is None:
        out = torch.empty_like(cache)
        assert copy_cached
    idx = idx.to(torch.int32).contiguous()
    rc = lib().oracle_scatter(_ptr(out_blocks), DT[cache.dtype], idx.numel(), _ptr(idx), n, ho, wo, cout, b,
                              _ptr(cache), _ptr(out), int(copy_cached))
    _check(rc, "scatter")
    return out


def restore_blocks(prev_idx, idx, cache, out, b) -> torch.Tensor:
    """In place on `out` (NHWC, the previous edit's result): blocks listed in
    prev_idx and not in idx get their cached pixels back.  idx may be None."""
    cache = cache.contiguous()
    assert out.is_contiguous() and out.shape == cache.shape and out.dtype == cache.dtype
    n, ho, wo, cout = cache.shape
    prev_idx = prev_idx.to(torch.int32).contiguous()
    new = (idx if idx is not None else torch.zeros(0)).to(torch.int32).contiguous()
    rc = lib().oracle_restore_blocks(_ptr(prev_idx), prev_idx.numel(), _ptr(new) if new.numel() else None,
                                     new.numel(), n, ho, wo, cout, b, DT[cache.dtype], _ptr(cache), _ptr(out))
    _check(rc, "restore_blocks")
    return out


def sparse_attention(q, k, v, heads, b, active, cache, scale=None, out_f64=False) -> torch.Tensor:
    """Query-pruned self-attention over a token grid.

    q, k, v, cache: [n, h, w, heads*d] (tokens row-major), storage dtype.
    active: uint8 [n, ceil(h/b), ceil(w/b)] blocks of query tokens, or None (all).
    scale defaults to 1/sqrt(d).  Tokens outside active blocks keep the cache.
    """
    q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
    n, h, w, C = q.shape
    assert k.shape == q.shape == v.shape and k.dtype == q.dtype == v.dtype and C % heads == 0
    d = C // heads
    scale = d ** -0.5 if scale is None else scale
    out = torch.empty(q.shape, dtype=torch.float64 if out_f64 else q.dtype)
    if active is not None:
        active = active.to(torch.uint8).contiguous()
        assert active.shape == (n, -(-h // b), -(-w // b))
        cache = cache.contiguous()
        assert cache.shape == q.shape and cache.dtype == q.dtype
    rc = lib().oracle_sparse_attention(_ptr(q), _ptr(k), _ptr(v), DT[q.dtype], n, h, w, heads, d, float(scale), b,
                                       _ptr(active), _ptr(cache), _ptr(out), DT[out.dtype])
    _check(rc, "sparse_attention")
    return out


def sparse_chain(a_edit, layers, caches, mask):
    """Layer-wise edited outputs of a conv chain (NHWC).

    layers: list of dicts with keys weight (OIHW), bias, k, s, p, b, dilate.
    caches: cached outputs of the original chain, one per layer.
    mask:   [n, hm, wm] diff mask at the first layer's input resolution (or finer);
            each layer OR-pools it to its own input resolution.
    Layer l+1 takes layer l's edited output (already rounded to the storage
    dtype) as its edited input; the caches are inputs, not recomputed.
    """
    outs, x = [], a_edit
    for L, cache in zip(layers, caches):
        n, h, w, _ = x.shape
        act = block_activity(mask, h, w, L["k"], L["s"], L["p"], L["b"], L["dilate"])
        x = sparse_layer(x, L["weight"], L["bias"], L["k"], L["s"], L["p"], L["b"], act, cache)
        outs.append(x)
    return outs

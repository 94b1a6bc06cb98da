"""ctypes binding of libsige.so -- argument marshalling only.

Each function has the name of the C entry point it calls (include/sige.h) and
passes torch tensors' device pointers plus the current HIP stream.  Every step
of the computation runs in the HIP kernels; there is no other code path, and a
missing library raises instead of falling back.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsige.so")

SIGE_OK, SIGE_EINVAL, SIGE_EDTYPE, SIGE_EALIGN, SIGE_EHIP, SIGE_ENODEV, SIGE_ERANGE = 0, -1, -2, -3, -4, -5, -6
DTYPE_CODE = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}

EXPORTS = ("sige_geom_derive", "sige_max_blocks", "sige_diff_mask", "sige_reduce_mask", "sige_reduce_mask_copy",
           "sige_diff_mask_bits", "sige_reduce_bits", "sige_reduce_bits_copy", "sige_reduce_bits_layers",
           "sige_sparse_conv_layer_split", "sige_sparse_conv_layer_split_workspace",
           "sige_sparse_conv_layer_split_noalloc", "sige_noalloc_scratch_bytes",
           "sige_sparse_conv_layer_plan", "sige_sparse_conv_layer_auto",
           "sige_packed_weights_bytes", "sige_pack_weights", "sige_sparse_conv_layer_packed",
           "sige_conv_blocks_packed",
           "sige_sparse_conv_layer_auto_packed",
           "sige_gather",
           "sige_conv_blocks", "sige_scatter", "sige_sparse_conv_layer", "sige_restore_blocks", "sige_sparse_conv_layer_restore",
           "sige_sparse_attention_workspace", "sige_sparse_attention", "sige_strerror",
           "sige_last_error")


class SigeError(RuntimeError):
    def __init__(self, code: int, fn: str, msg: str):
        super().__init__(f"{fn}: {msg} (code {code})")
        self.code = code


class Geom(ctypes.Structure):
    """sige_geom: input [n, h, w, c_in], k x k kernel, stride, pad, output block edge."""
    _fields_ = [(f, ctypes.c_int32) for f in ("n", "h", "w", "c_in", "c_out", "k", "stride", "pad", "block")]


class LayerPlan(ctypes.Structure):
    """sige_layer_plan: which kernel sige_sparse_conv_layer_auto runs for which list lengths."""
    _fields_ = [("split_max", ctypes.c_int32), ("cap", ctypes.c_int32), ("workspace_bytes", ctypes.c_int64),
                ("chunks", ctypes.c_int32), ("steps", ctypes.c_int32), ("stage_groups", ctypes.c_int32),
                ("slots", ctypes.c_int32), ("n_tiles", ctypes.c_int32), ("split_chunks", ctypes.c_int32),
                ("split_slots", ctypes.c_int32), ("split_stage_kb", ctypes.c_double), ("weight_mb", ctypes.c_double),
                ("gflop_per_block", ctypes.c_double), ("wide_min", ctypes.c_int32), ("wide_stages", ctypes.c_int32),
                ("wide_loads", ctypes.c_int32), ("wide_n_tiles", ctypes.c_int32), ("wide_max", ctypes.c_int32),
                ("wide_parts_max", ctypes.c_int32)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}


class Derived(ctypes.Structure):
    _fields_ = [("ho", ctypes.c_int32), ("wo", ctypes.c_int32), ("nby", ctypes.c_int32), ("nbx", ctypes.c_int32),
                ("ib", ctypes.c_int32), ("cap", ctypes.c_int64)]


_lib = None


def lib():
    """Load libsige.so (built in-tree by `python -m spatially_sparse_incremental_amd.build`)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m spatially_sparse_incremental_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        V, I, P = ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(Geom)
        L.sige_geom_derive.argtypes = [P, ctypes.POINTER(Derived)]
        L.sige_max_blocks.argtypes = [P]
        L.sige_max_blocks.restype = ctypes.c_int64
        L.sige_diff_mask.argtypes = [V, V, I, I, I, I, I, ctypes.c_float, V, V]
        L.sige_reduce_mask.argtypes = [V, I, I, P, I, V, V, V]
        L.sige_reduce_mask_copy.argtypes = [V, I, I, P, I, V, V, I, V, V, V]
        L.sige_diff_mask_bits.argtypes = [V, V, I, I, I, I, I, ctypes.c_float, V, V, V]
        L.sige_reduce_bits.argtypes = [V, I, I, P, I, V, V, V]
        L.sige_reduce_bits_copy.argtypes = [V, I, I, P, I, V, V, I, V, V, V]
        L.sige_reduce_bits_layers.argtypes = [V, I, I, I, P, ctypes.POINTER(I), ctypes.POINTER(V), ctypes.POINTER(V),
                                              I, ctypes.POINTER(V), ctypes.POINTER(V), V]
        L.sige_gather.argtypes = [V, I, P, V, V, V, V]
        L.sige_conv_blocks.argtypes = [V, V, V, I, P, V, V, V]
        L.sige_scatter.argtypes = [V, V, V, P, I, V, V, I, V]
        L.sige_sparse_conv_layer.argtypes = [V, V, V, V, V, V, I, P, V, I, V]
        L.sige_sparse_conv_layer_split_workspace.argtypes = [P, I]
        L.sige_sparse_conv_layer_split_workspace.restype = ctypes.c_int64
        L.sige_sparse_conv_layer_split.argtypes = [V, V, V, V, V, V, I, P, V, I, V, ctypes.c_int64, V]
        L.sige_sparse_conv_layer_split_noalloc.argtypes = [V, V, V, V, V, V, I, P, V, I, V]
        L.sige_sparse_conv_layer_plan.argtypes = [P, I, ctypes.POINTER(LayerPlan)]
        L.sige_sparse_conv_layer_auto.argtypes = [V, V, V, V, V, V, I, P, V, I, V, ctypes.c_int64, V]
        L.sige_packed_weights_bytes.argtypes = [P, I]
        L.sige_packed_weights_bytes.restype = ctypes.c_int64
        L.sige_pack_weights.argtypes = [V, I, P, V, ctypes.c_int64, V]
        L.sige_sparse_conv_layer_packed.argtypes = [V, V, V, V, V, V, I, P, V, I, V, ctypes.c_int64, V]
        L.sige_conv_blocks_packed.argtypes = [V, V, V, I, P, V, V, V, ctypes.c_int64, V]
        L.sige_sparse_conv_layer_auto_packed.argtypes = [V, V, V, V, V, V, I, P, V, I, V, ctypes.c_int64, V,
                                                         ctypes.c_int64, V]
        L.sige_noalloc_scratch_bytes.argtypes = []
        L.sige_noalloc_scratch_bytes.restype = ctypes.c_int64
        L.sige_restore_blocks.argtypes = [V, V, V, V, P, I, V, V, V]
        L.sige_sparse_conv_layer_restore.argtypes = [V, V, V, V, V, V, V, V, I, P, V, V]
        L.sige_sparse_attention_workspace.argtypes = [I] * 6
        L.sige_sparse_attention_workspace.restype = ctypes.c_int64
        L.sige_sparse_attention.argtypes = [V, V, V, V, V, I, I, I, I, I, I, I, ctypes.c_float, V, V, I, V,
                                            ctypes.c_int64, V]
        L.sige_strerror.restype = ctypes.c_char_p
        L.sige_strerror.argtypes = [I]
        L.sige_last_error.restype = ctypes.c_char_p
        for f in EXPORTS:
            if f not in ("sige_strerror", "sige_last_error", "sige_max_blocks", "sige_sparse_attention_workspace",
                         "sige_sparse_conv_layer_split_workspace", "sige_noalloc_scratch_bytes",
                         "sige_packed_weights_bytes"):
                getattr(L, f).restype = I
        _lib = L
    return _lib


def _check(rc: int, fn: str):
    if rc != SIGE_OK:
        msg = lib().sige_last_error().decode() or lib().sige_strerror(rc).decode()
        raise SigeError(rc, fn, msg)


def _p(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise ValueError("tensors must live on the GPU")
            if not t.is_contiguous():
                raise ValueError("tensors must be contiguous")


def _dt(t):
    try:
        return DTYPE_CODE[t.dtype]
    except KeyError:
        raise SigeError(SIGE_EDTYPE, "dtype", f"unsupported dtype {t.dtype}") from None


def _need(t, what, dtype=None, shape=None, numel=None):
    """Checks a caller tensor's dtype, shape or size before its pointer goes to the library."""
    if t is None:
        return
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{what}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{what}: {t.numel()} elements, at least {numel} needed")


def _need_list(g, idx, count):
    """A block list holds sige_max_blocks(g) int32 entries (the kernels may read past *count) and
    its count one int32."""
    _need(idx, "idx", dtype=torch.int32, numel=sige_max_blocks(g))
    _need(count, "count", dtype=torch.int32, numel=1)


def _need_layer(g, a_edit, w_krsc, bias, cached, out):
    """Shapes of a layer's tensors: NHWC activation and outputs, KRSC weights, fp32 bias."""
    d = sige_geom_derive(g)
    _need(a_edit, "a_edit", shape=(g.n, g.h, g.w, g.c_in))
    _need(w_krsc, "w_krsc", dtype=a_edit.dtype, shape=(g.c_out, g.k, g.k, g.c_in))
    _need(bias, "bias", dtype=torch.float32, shape=(g.c_out,))
    _need(cached, "cached", dtype=a_edit.dtype, shape=(g.n, d.ho, d.wo, g.c_out))
    _need(out, "out", dtype=a_edit.dtype, shape=(g.n, d.ho, d.wo, g.c_out))
    return d


# ---------------------------------------------------------------------------
def geom(n, h, w, c_in, c_out, k=3, stride=1, pad=1, block=6) -> Geom:
    return Geom(n, h, w, c_in, c_out, k, stride, pad, block)


def sige_geom_derive(g: Geom) -> Derived:
    d = Derived()
    _check(lib().sige_geom_derive(ctypes.byref(g), ctypes.byref(d)), "sige_geom_derive")
    return d


def sige_max_blocks(g: Geom) -> int:
    v = lib().sige_max_blocks(ctypes.byref(g))
    if v < 0:
        _check(int(v), "sige_max_blocks")
    return int(v)


def sige_diff_mask(a_orig, a_edit, thresh=1e-6, mask=None, stream=None):
    """uint8 [n, h, w] change mask of two NHWC activations."""
    _dev(a_orig, a_edit, mask)
    if a_orig.shape != a_edit.shape or a_orig.dtype != a_edit.dtype or a_orig.dim() != 4:
        raise ValueError("a_orig and a_edit must be NHWC tensors of one shape and dtype")
    n, h, w, c = a_orig.shape
    if mask is None:
        mask = torch.empty((n, h, w), dtype=torch.uint8, device=a_orig.device)
    rc = lib().sige_diff_mask(_p(a_orig), _p(a_edit), _dt(a_orig), n, h, w, c, ctypes.c_float(thresh), _p(mask),
                              _stream(stream))
    _check(rc, "sige_diff_mask")
    return mask


def sige_diff_mask_bits(a_orig, a_edit, thresh=1e-6, bits=None, mask=None, stream=None):
    """The change mask packed one bit per pixel: int32 [n*h*w/32] (bit p % 32 of
    word p / 32 for pixel p); also the uint8 [n, h, w] mask when `mask` is given
    (a tensor to fill).  w must be a multiple of 32."""
    _dev(a_orig, a_edit, bits, mask)
    if a_orig.shape != a_edit.shape or a_orig.dtype != a_edit.dtype or a_orig.dim() != 4:
        raise ValueError("a_orig and a_edit must be NHWC tensors of one shape and dtype")
    n, h, w, c = a_orig.shape
    if bits is None:
        bits = torch.empty((max(n * h * w // 32, 1),), dtype=torch.int32, device=a_orig.device)
    rc = lib().sige_diff_mask_bits(_p(a_orig), _p(a_edit), _dt(a_orig), n, h, w, c, ctypes.c_float(thresh),
                                   _p(mask), _p(bits), _stream(stream))
    _check(rc, "sige_diff_mask_bits")
    return bits


def sige_reduce_bits(bits, mask_h, mask_w, g: Geom, dilate_blocks=1, idx=None, count=None, stream=None):
    """sige_reduce_mask on a mask packed as sige_diff_mask_bits writes it (mask_h x mask_w per image)."""
    _dev(bits, idx, count)
    _need_list(g, idx, count)
    _need(bits, "bits", dtype=torch.int32, numel=g.n * mask_h * mask_w // 32)
    cap = sige_max_blocks(g)
    dev = bits.device
    if idx is None:
        idx = torch.empty((max(cap, 1),), dtype=torch.int32, device=dev)
    if count is None:
        count = torch.empty((1,), dtype=torch.int32, device=dev)
    rc = lib().sige_reduce_bits(_p(bits), mask_h, mask_w, ctypes.byref(g), dilate_blocks, _p(idx), _p(count),
                                _stream(stream))
    _check(rc, "sige_reduce_bits")
    return idx, count


def sige_reduce_bits_copy(bits, mask_h, mask_w, g: Geom, dilate_blocks, cached, out=None, idx=None, count=None,
                          stream=None):
    """sige_reduce_bits with `cached` copied into `out` by the same launch; returns (idx, count, out)."""
    _dev(bits, idx, count, cached, out)
    _need_list(g, idx, count)
    _need(bits, "bits", dtype=torch.int32, numel=g.n * mask_h * mask_w // 32)
    d = sige_geom_derive(g)
    _need(cached, "cached", shape=(g.n, d.ho, d.wo, g.c_out))
    _need(out, "out", dtype=cached.dtype, shape=(g.n, d.ho, d.wo, g.c_out))
    cap = sige_max_blocks(g)
    dev = bits.device
    if idx is None:
        idx = torch.empty((max(cap, 1),), dtype=torch.int32, device=dev)
    if count is None:
        count = torch.empty((1,), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty_like(cached)
    rc = lib().sige_reduce_bits_copy(_p(bits), mask_h, mask_w, ctypes.byref(g), dilate_blocks, _p(idx), _p(count),
                                     _dt(cached), _p(cached), _p(out), _stream(stream))
    _check(rc, "sige_reduce_bits_copy")
    return idx, count, out


def sige_reduce_bits_layers(bits, mask_h, mask_w, geoms, dilate_blocks, idx, count, cached=None, out=None,
                            stream=None):
    """Every layer's block list from one packed mask in one launch, with the
    layers' cache copies (cached[l] -> out[l]) on its other workgroups.
    geoms, dilate_blocks, idx, count (and cached, out, or None) are lists with
    one entry per layer; cached[l] and out[l] may both be None."""
    n = len(geoms)
    _dev(bits, *idx, *count, *(cached or []), *(out or []))
    if not (len(dilate_blocks) == len(idx) == len(count) == n) or (cached and len(cached) != n) or \
            (out and len(out) != n):
        raise ValueError("geoms, dilate_blocks, idx, count (and cached, out) need one entry per layer")
    for l, gl in enumerate(geoms):
        _need_list(gl, idx[l], count[l])
        if cached and out and cached[l] is not None:
            dl = sige_geom_derive(gl)
            _need(cached[l], f"cached[{l}]", shape=(gl.n, dl.ho, dl.wo, gl.c_out))
            _need(out[l], f"out[{l}]", dtype=cached[l].dtype, shape=(gl.n, dl.ho, dl.wo, gl.c_out))
    GA = Geom * n
    IA = ctypes.c_int * n
    VA = ctypes.c_void_p * n
    cached = cached or [None] * n
    out = out or [None] * n
    dt = next((_dt(c) for c in cached if c is not None), 0)
    rc = lib().sige_reduce_bits_layers(_p(bits), mask_h, mask_w, n, GA(*geoms), IA(*dilate_blocks),
                                       VA(*[t.data_ptr() for t in idx]), VA(*[t.data_ptr() for t in count]), dt,
                                       VA(*[t.data_ptr() if t is not None else 0 for t in cached]),
                                       VA(*[t.data_ptr() if t is not None else 0 for t in out]), _stream(stream))
    _check(rc, "sige_reduce_bits_layers")
    return idx, count, out


def sige_reduce_mask(mask, g: Geom, dilate_blocks=1, idx=None, count=None, stream=None):
    """(idx int32 [cap], count int32 [1]) on the device; idx[:count] are the active blocks, ascending."""
    if mask.dim() == 2:
        mask = mask.unsqueeze(0)
    _dev(mask, idx, count)
    _need_list(g, idx, count)
    _need(mask, "mask", dtype=torch.uint8)
    cap = sige_max_blocks(g)
    dev = mask.device
    if idx is None:
        idx = torch.empty((max(cap, 1),), dtype=torch.int32, device=dev)
    if count is None:
        count = torch.empty((1,), dtype=torch.int32, device=dev)
    rc = lib().sige_reduce_mask(_p(mask), mask.shape[-2], mask.shape[-1], ctypes.byref(g), dilate_blocks, _p(idx),
                                _p(count), _stream(stream))
    _check(rc, "sige_reduce_mask")
    return idx, count


def sige_reduce_mask_copy(mask, g: Geom, dilate_blocks, cached, out=None, idx=None, count=None, stream=None):
    """sige_reduce_mask, with `cached` copied into `out` (all of it) by the same
    launch; returns (idx, count, out)."""
    if mask.dim() == 2:
        mask = mask.unsqueeze(0)
    _dev(mask, idx, count, cached, out)
    _need_list(g, idx, count)
    _need(mask, "mask", dtype=torch.uint8)
    d = sige_geom_derive(g)
    _need(cached, "cached", shape=(g.n, d.ho, d.wo, g.c_out))
    _need(out, "out", dtype=cached.dtype, shape=(g.n, d.ho, d.wo, g.c_out))
    cap = sige_max_blocks(g)
    dev = mask.device
    if idx is None:
        idx = torch.empty((max(cap, 1),), dtype=torch.int32, device=dev)
    if count is None:
        count = torch.empty((1,), dtype=torch.int32, device=dev)
    if out is None:
        out = torch.empty_like(cached)
    rc = lib().sige_reduce_mask_copy(_p(mask), mask.shape[-2], mask.shape[-1], ctypes.byref(g), dilate_blocks,
                                     _p(idx), _p(count), _dt(cached), _p(cached), _p(out), _stream(stream))
    _check(rc, "sige_reduce_mask_copy")
    return idx, count, out


def sige_gather(a_edit, g: Geom, idx, count, blocks=None, stream=None):
    """[cap, ib, ib, c_in]: input windows of the listed blocks (slots < count)."""
    _dev(a_edit, idx, count, blocks)
    _need_list(g, idx, count)
    d = sige_geom_derive(g)
    _need(a_edit, "a_edit", shape=(g.n, g.h, g.w, g.c_in))
    _need(blocks, "blocks", dtype=a_edit.dtype, shape=(max(d.cap, 1), d.ib, d.ib, g.c_in))
    if blocks is None:
        blocks = torch.empty((max(d.cap, 1), d.ib, d.ib, g.c_in), dtype=a_edit.dtype, device=a_edit.device)
    rc = lib().sige_gather(_p(a_edit), _dt(a_edit), ctypes.byref(g), _p(idx), _p(count), _p(blocks),
                           _stream(stream))
    _check(rc, "sige_gather")
    return blocks


def sige_conv_blocks(blocks, w_krsc, bias, g: Geom, count, out_blocks=None, stream=None, w_packed=None):
    """[cap, b, b, c_out]: conv of each stacked block (slots < count); with w_packed
    (sige_pack_weights of w_krsc) the weights come from the packed copy
    (sige_conv_blocks_packed)."""
    _dev(blocks, w_krsc, bias, count, out_blocks, w_packed)
    if w_krsc.dtype != blocks.dtype or (bias is not None and bias.dtype != torch.float32):
        raise ValueError("weights must match the activation dtype; bias must be fp32")
    d = sige_geom_derive(g)
    _need(count, "count", dtype=torch.int32, numel=1)
    _need(blocks, "blocks", shape=(max(d.cap, 1), d.ib, d.ib, g.c_in))
    _need(w_krsc, "w_krsc", shape=(g.c_out, g.k, g.k, g.c_in))
    _need(bias, "bias", shape=(g.c_out,))
    _need(out_blocks, "out_blocks", dtype=blocks.dtype, shape=(max(d.cap, 1), g.block, g.block, g.c_out))
    if out_blocks is None:
        out_blocks = torch.empty((max(d.cap, 1), g.block, g.block, g.c_out), dtype=blocks.dtype,
                                 device=blocks.device)
    args = (_p(blocks), _p(w_krsc), _p(bias), _dt(blocks), ctypes.byref(g), _p(count), _p(out_blocks))
    if w_packed is None:
        rc = lib().sige_conv_blocks(*args, _stream(stream))
        _check(rc, "sige_conv_blocks")
    else:
        rc = lib().sige_conv_blocks_packed(*args, _p(w_packed), w_packed.numel() * w_packed.element_size(),
                                           _stream(stream))
        _check(rc, "sige_conv_blocks_packed")
    return out_blocks


def sige_scatter(out_blocks, idx, count, g: Geom, cached, out=None, copy_cached=True, stream=None):
    """[n, ho, wo, c_out]: cached output with the listed blocks overwritten."""
    _dev(out_blocks, idx, count, cached, out)
    _need_list(g, idx, count)
    d = sige_geom_derive(g)
    _need(out_blocks, "out_blocks", shape=(max(d.cap, 1), g.block, g.block, g.c_out))
    _need(cached, "cached", dtype=out_blocks.dtype, shape=(g.n, d.ho, d.wo, g.c_out))
    _need(out, "out", dtype=out_blocks.dtype, shape=(g.n, d.ho, d.wo, g.c_out))
    if out is None:
        if not copy_cached:
            raise ValueError("copy_cached=False needs a persistent `out`")
        out = torch.empty((g.n, d.ho, d.wo, g.c_out), dtype=out_blocks.dtype, device=out_blocks.device)
    rc = lib().sige_scatter(_p(out_blocks), _p(idx), _p(count), ctypes.byref(g), _dt(out_blocks),
                            _p(cached if copy_cached else None), _p(out), int(bool(copy_cached)), _stream(stream))
    _check(rc, "sige_scatter")
    return out


def sige_sparse_conv_layer(a_edit, w_krsc, bias, cached, idx, count, g: Geom, out=None, copy_cached=True,
                           stream=None, w_packed=None):
    """Fused gather + conv + scatter into `out` (NHWC [n, ho, wo, c_out]); with w_packed
    (sige_pack_weights of w_krsc) the kernel loads its weights from the packed copy
    (sige_sparse_conv_layer_packed)."""
    _dev(a_edit, w_krsc, bias, cached, idx, count, out, w_packed)
    _need_list(g, idx, count)
    d = _need_layer(g, a_edit, w_krsc, bias, cached if copy_cached else None, out)
    if out is None:
        if not copy_cached:
            raise ValueError("copy_cached=False needs a persistent `out`")
        out = torch.empty((g.n, d.ho, d.wo, g.c_out), dtype=a_edit.dtype, device=a_edit.device)
    args = (_p(a_edit), _p(w_krsc), _p(bias), _p(cached if copy_cached else None), _p(idx), _p(count), _dt(a_edit),
            ctypes.byref(g), _p(out), int(bool(copy_cached)))
    if w_packed is None:
        rc = lib().sige_sparse_conv_layer(*args, _stream(stream))
        _check(rc, "sige_sparse_conv_layer")
    else:
        rc = lib().sige_sparse_conv_layer_packed(*args, _p(w_packed), w_packed.numel() * w_packed.element_size(),
                                                 _stream(stream))
        _check(rc, "sige_sparse_conv_layer_packed")
    return out


def sige_sparse_conv_layer_split_workspace(g: Geom, dtype) -> int:
    """Bytes of the workspace of sige_sparse_conv_layer_split for g and a torch dtype."""
    nbytes = lib().sige_sparse_conv_layer_split_workspace(ctypes.byref(g), DTYPE_CODE[dtype])
    if nbytes < 0:
        _check(int(nbytes), "sige_sparse_conv_layer_split_workspace")
    return int(nbytes)


def sige_sparse_conv_layer_split(a_edit, w_krsc, bias, cached, idx, count, g: Geom, out=None, copy_cached=True,
                                 workspace=None, stream=None):
    """The fused layer split over input channels (weight-bound layers); the
    workspace is allocated here when not given."""
    _dev(a_edit, w_krsc, bias, cached, idx, count, out, workspace)
    _need_list(g, idx, count)
    d = _need_layer(g, a_edit, w_krsc, bias, cached if copy_cached else None, out)
    if out is None:
        if not copy_cached:
            raise ValueError("copy_cached=False needs a persistent `out`")
        out = torch.empty((g.n, d.ho, d.wo, g.c_out), dtype=a_edit.dtype, device=a_edit.device)
    if workspace is None:
        workspace = torch.empty(sige_sparse_conv_layer_split_workspace(g, a_edit.dtype), dtype=torch.uint8,
                                device=a_edit.device)
    rc = lib().sige_sparse_conv_layer_split(_p(a_edit), _p(w_krsc), _p(bias), _p(cached if copy_cached else None),
                                            _p(idx), _p(count), _dt(a_edit), ctypes.byref(g), _p(out),
                                            int(bool(copy_cached)), _p(workspace), workspace.numel(),
                                            _stream(stream))
    _check(rc, "sige_sparse_conv_layer_split")
    return out


def sige_sparse_conv_layer_plan(g: Geom, dtype) -> LayerPlan:
    """The kernel choice of sige_sparse_conv_layer_auto for g and a torch dtype:
    the split takes lists of at most .split_max blocks (-1: never), the
    single-range kernel the longer ones; .workspace_bytes for the split."""
    plan = LayerPlan()
    _check(lib().sige_sparse_conv_layer_plan(ctypes.byref(g), DTYPE_CODE[dtype], ctypes.byref(plan)),
           "sige_sparse_conv_layer_plan")
    return plan


def sige_packed_weights_bytes(g: Geom, dtype) -> int:
    """Bytes of the packed copy of a layer's weights for g and a torch dtype (sige_pack_weights)."""
    n = int(lib().sige_packed_weights_bytes(ctypes.byref(g), DTYPE_CODE[dtype]))
    if n < 0:
        _check(n, "sige_packed_weights_bytes")
    return n


def sige_pack_weights(w_krsc, g: Geom, out=None, stream=None):
    """The packed copy of KRSC weights in the layer kernels' load order (made once per layer),
    for sige_sparse_conv_layer(..., w_packed=) and sige_sparse_conv_layer_auto(..., w_packed=);
    allocated here when `out` is not given (256-byte aligned)."""
    _dev(w_krsc, out)
    need = sige_packed_weights_bytes(g, w_krsc.dtype)
    if out is None:
        out = torch.empty(need, dtype=torch.uint8, device=w_krsc.device)
    rc = lib().sige_pack_weights(_p(w_krsc), _dt(w_krsc), ctypes.byref(g), _p(out),
                                 out.numel() * out.element_size(), _stream(stream))
    _check(rc, "sige_pack_weights")
    return out


def sige_sparse_conv_layer_auto(a_edit, w_krsc, bias, cached, idx, count, g: Geom, out=None, copy_cached=True,
                                workspace=None, stream=None, w_packed=None):
    """The fused layer on the kernel the library picks for *count (see
    sige_sparse_conv_layer_plan); the workspace is allocated here when the
    plan needs one and none is given.  With w_packed (sige_pack_weights of
    w_krsc) the single-range kernel and the wide tiles load their weights
    from it (sige_sparse_conv_layer_auto_packed)."""
    _dev(a_edit, w_krsc, bias, cached, idx, count, out, workspace, w_packed)
    _need_list(g, idx, count)
    d = _need_layer(g, a_edit, w_krsc, bias, cached if copy_cached else None, out)
    if out is None:
        if not copy_cached:
            raise ValueError("copy_cached=False needs a persistent `out`")
        out = torch.empty((g.n, d.ho, d.wo, g.c_out), dtype=a_edit.dtype, device=a_edit.device)
    if workspace is None:
        need = sige_sparse_conv_layer_plan(g, a_edit.dtype).workspace_bytes
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=a_edit.device)
    args = (_p(a_edit), _p(w_krsc), _p(bias), _p(cached if copy_cached else None), _p(idx), _p(count), _dt(a_edit),
            ctypes.byref(g), _p(out), int(bool(copy_cached)), _p(workspace),
            workspace.numel() if workspace is not None else 0)
    if w_packed is None:
        rc = lib().sige_sparse_conv_layer_auto(*args, _stream(stream))
        _check(rc, "sige_sparse_conv_layer_auto")
    else:
        rc = lib().sige_sparse_conv_layer_auto_packed(*args, _p(w_packed), w_packed.numel() * w_packed.element_size(),
                                                      _stream(stream))
        _check(rc, "sige_sparse_conv_layer_auto_packed")
    return out


def sige_noalloc_scratch_bytes() -> int:
    """Bytes of the library's static scratch (per GPU) used by sige_sparse_conv_layer_split_noalloc."""
    return int(lib().sige_noalloc_scratch_bytes())


def sige_sparse_conv_layer_split_noalloc(a_edit, w_krsc, bias, cached, idx, count, g: Geom, out, copy_cached=True,
                                         stream=None):
    """sige_sparse_conv_layer_split on the library's static scratch: no workspace, and the
    call allocates nothing (`out` is required)."""
    _dev(a_edit, w_krsc, bias, cached, idx, count, out)
    _need_list(g, idx, count)
    _need_layer(g, a_edit, w_krsc, bias, cached if copy_cached else None, out)
    rc = lib().sige_sparse_conv_layer_split_noalloc(_p(a_edit), _p(w_krsc), _p(bias),
                                                    _p(cached if copy_cached else None), _p(idx), _p(count),
                                                    _dt(a_edit), ctypes.byref(g), _p(out), int(bool(copy_cached)),
                                                    _stream(stream))
    _check(rc, "sige_sparse_conv_layer_split_noalloc")
    return out


def weight_to_krsc(w_oihw: torch.Tensor) -> torch.Tensor:
    """Repack PyTorch OIHW weights to the library's KRSC layout (once, at load time)."""
    return w_oihw.permute(0, 2, 3, 1).contiguous()


def sige_restore_blocks(prev_idx, prev_count, idx, count, g: Geom, cached, out, stream=None):
    """Sequential edits: in the persistent buffer `out`, the blocks of the
    previous list that the new list (idx, count; both None: empty) does not
    hold get the cache back.  Returns `out`."""
    _dev(prev_idx, prev_count, idx, count, cached, out)
    if (idx is None) != (count is None):
        raise ValueError("idx and count must both be given or both be None")
    _need_list(g, prev_idx, prev_count)
    _need_list(g, idx, count)
    d = sige_geom_derive(g)
    _need(cached, "cached", shape=(g.n, d.ho, d.wo, g.c_out))
    _need(out, "out", dtype=cached.dtype, shape=(g.n, d.ho, d.wo, g.c_out))
    rc = lib().sige_restore_blocks(_p(prev_idx), _p(prev_count), _p(idx), _p(count), ctypes.byref(g), _dt(cached),
                                   _p(cached), _p(out), _stream(stream))
    _check(rc, "sige_restore_blocks")
    return out


def sige_sparse_conv_layer_restore(a_edit, w_krsc, bias, cached, prev_idx, prev_count, idx, count, g: Geom, out,
                                   stream=None):
    """Sequential edits in one launch: restore the previous list's blocks that
    the new list does not hold, and write the new blocks, into `out`."""
    _dev(a_edit, w_krsc, bias, cached, prev_idx, prev_count, idx, count, out)
    _need_list(g, prev_idx, prev_count)
    _need_list(g, idx, count)
    _need_layer(g, a_edit, w_krsc, bias, cached, out)
    rc = lib().sige_sparse_conv_layer_restore(_p(a_edit), _p(w_krsc), _p(bias), _p(cached), _p(prev_idx),
                                              _p(prev_count), _p(idx), _p(count), _dt(a_edit), ctypes.byref(g),
                                              _p(out), _stream(stream))
    _check(rc, "sige_sparse_conv_layer_restore")
    return out


def sige_sparse_attention_workspace(n, h, w, heads, head_dim, block) -> int:
    nbytes = lib().sige_sparse_attention_workspace(n, h, w, heads, head_dim, block)
    if nbytes < 0:
        _check(int(nbytes), "sige_sparse_attention_workspace")
    return int(nbytes)


def sige_sparse_attention(q, k, v, idx, count, heads, block, scale=None, cached=None, out=None, copy_cached=True,
                          workspace=None, stream=None):
    """Query-pruned self-attention over a token grid: q, k, v, cached, out are
    [n, h, w, heads*head_dim] (NHWC = tokens row-major).  The workspace is
    allocated here when not given."""
    _dev(q, k, v, idx, count, cached, out, workspace)
    n, h, w, c = q.shape
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype or c % heads:
        raise ValueError("q, k and v must match, with heads dividing the channels")
    d = c // heads
    scale = d ** -0.5 if scale is None else scale
    _need_list(geom(n, h, w, c, c, 1, 1, 0, block), idx, count)
    _need(cached, "cached", dtype=q.dtype, shape=q.shape)
    _need(out, "out", dtype=q.dtype, shape=q.shape)
    if out is None:
        if not copy_cached:
            raise ValueError("copy_cached=False needs a persistent `out`")
        out = torch.empty_like(q)
    if workspace is None:
        nbytes = sige_sparse_attention_workspace(n, h, w, heads, d, block)
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    rc = lib().sige_sparse_attention(_p(q), _p(k), _p(v), _p(idx), _p(count), _dt(q), n, h, w, heads, d, block,
                                     ctypes.c_float(scale), _p(cached if copy_cached else None), _p(out),
                                     int(bool(copy_cached)), _p(workspace), workspace.numel(), _stream(stream))
    _check(rc, "sige_sparse_attention")
    return out

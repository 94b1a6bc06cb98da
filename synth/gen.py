"""Seeded generators for the synthetic edit workloads.

What is drawn here, and why it has these shapes:

* Activations are N(0, 1) in fp32 from ``torch.Generator().manual_seed(seed)``,
  then rounded once (round-to-nearest-even) to the workload's storage dtype.
* Edits are local and small.  The pages measure at about 1.2 % edited area
  (mer.dev notes on "Efficient Spatially Sparse Inference for Conditional GANs
  and Diffusion Models", abstract; SIGE README mirror, Efficiency section), and
  say user edits are local and structured (mer.dev notes, section 3.1).  The
  edit shapes are: a fixed-size rectangle, a blob made of three overlapping
  ellipses, and a 12-vertex star polygon.  Blob and polygon are continuous
  shapes in reference-pixel units; a common scale is bisected until the raster
  at the reference resolution covers the target area within 0.02 percentage
  points.  The same continuous shape can then be rasterised at any resolution
  (pixel centres, even-odd rule for the polygon).
* Weights: N(0, 0.05) for the small fp32 layer, He-normal
  (std = sqrt(2 / (Cin k^2))) elsewhere; bias N(0, 0.01) in fp32.

Nothing in this module computes a diff, a pooled mask, a block list or a
convolution.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


# ----------------------------------------------------------------------------
# edit shapes
# ----------------------------------------------------------------------------
def rectangle_mask(seed: int, h: int = 64, w: int = 64, rows: int = 10, cols: int = 12):
    """A rows x cols rectangle with a seeded top-left corner, fully inside the image.

    Returns (mask uint8 [h, w], (y0, x0)).
    """
    rng = np.random.default_rng(seed)
    y0 = int(rng.integers(0, h - rows + 1))
    x0 = int(rng.integers(0, w - cols + 1))
    m = np.zeros((h, w), np.uint8)
    m[y0:y0 + rows, x0:x0 + cols] = 1
    return m, (y0, x0)


def _pixel_centres(h: int, w: int, ref_h: int, ref_w: int):
    ys = (np.arange(h, dtype=np.float64) + 0.5) * (ref_h / h)
    xs = (np.arange(w, dtype=np.float64) + 0.5) * (ref_w / w)
    return np.meshgrid(ys, xs, indexing="ij")


@dataclass
class _Shape:
    """A continuous edit region in reference-pixel units, with a bisected scale."""

    ref_h: int
    ref_w: int
    scale: float = 1.0

    def inside(self, yy, xx, scale):  # pragma: no cover - overridden
        raise NotImplementedError

    def raster(self, h: int | None = None, w: int | None = None) -> np.ndarray:
        h = self.ref_h if h is None else h
        w = self.ref_w if w is None else w
        yy, xx = _pixel_centres(h, w, self.ref_h, self.ref_w)
        return self.inside(yy, xx, self.scale).astype(np.uint8)

    def fit_area(self, area: float, tol: float = 2e-4, iters: int = 80):
        yy, xx = _pixel_centres(self.ref_h, self.ref_w, self.ref_h, self.ref_w)
        npix = self.ref_h * self.ref_w
        lo, hi = 0.0, 1.0
        while self.inside(yy, xx, hi).mean() < area and hi < 1e4:
            hi *= 2.0
        best, best_err = hi, abs(self.inside(yy, xx, hi).mean() - area)
        for _ in range(iters):
            mid = 0.5 * (lo + hi)
            frac = self.inside(yy, xx, mid).sum() / npix
            err = abs(frac - area)
            if err < best_err:
                best, best_err = mid, err
            if err <= tol:
                break
            if frac < area:
                lo = mid
            else:
                hi = mid
        self.scale = best
        return self


@dataclass
class Blob(_Shape):
    """Union of three random ellipses clustered around one seeded centre."""

    centres: np.ndarray = field(default_factory=lambda: np.zeros((3, 2)))
    axes: np.ndarray = field(default_factory=lambda: np.ones((3, 2)))
    angles: np.ndarray = field(default_factory=lambda: np.zeros(3))

    @classmethod
    def draw(cls, seed: int, ref_h: int, ref_w: int, n: int = 3):
        rng = np.random.default_rng(seed)
        size = min(ref_h, ref_w)
        c0 = np.array([rng.uniform(0.25, 0.75) * ref_h, rng.uniform(0.25, 0.75) * ref_w])
        centres = [c0] + [c0 + rng.uniform(-0.08, 0.08, 2) * size for _ in range(n - 1)]
        axes = rng.uniform(0.5, 1.5, (n, 2)) * (0.05 * size)
        angles = rng.uniform(0.0, math.pi, n)
        return cls(ref_h=ref_h, ref_w=ref_w, centres=np.array(centres), axes=axes, angles=angles)

    def inside(self, yy, xx, scale):
        out = np.zeros(yy.shape, bool)
        for (cy, cx), (ay, ax), th in zip(self.centres, self.axes, self.angles):
            dy, dx = yy - cy, xx - cx
            u = dx * math.cos(th) + dy * math.sin(th)
            v = -dx * math.sin(th) + dy * math.cos(th)
            out |= (u / (ax * scale)) ** 2 + (v / (ay * scale)) ** 2 <= 1.0
        return out


@dataclass
class StarPolygon(_Shape):
    """A 12-vertex polygon, star-shaped about its centre (so area grows with scale)."""

    centre: np.ndarray = field(default_factory=lambda: np.zeros(2))
    angles: np.ndarray = field(default_factory=lambda: np.zeros(12))
    radii: np.ndarray = field(default_factory=lambda: np.ones(12))

    @classmethod
    def draw(cls, seed: int, ref_h: int, ref_w: int, n: int = 12):
        rng = np.random.default_rng(seed)
        size = min(ref_h, ref_w)
        centre = np.array([rng.uniform(0.25, 0.75) * ref_h, rng.uniform(0.25, 0.75) * ref_w])
        base = np.linspace(0.0, 2 * math.pi, n, endpoint=False)
        angles = base + rng.uniform(-0.35, 0.35, n) * (2 * math.pi / n)
        radii = np.where(np.arange(n) % 2 == 0, rng.uniform(0.7, 1.0, n), rng.uniform(0.3, 0.6, n))
        return cls(ref_h=ref_h, ref_w=ref_w, centre=centre, angles=angles, radii=radii * 0.1 * size)

    def inside(self, yy, xx, scale):
        vy = self.centre[0] + scale * self.radii * np.sin(self.angles)
        vx = self.centre[1] + scale * self.radii * np.cos(self.angles)
        inside = np.zeros(yy.shape, bool)
        n = len(vy)
        for i in range(n):  # even-odd rule, one edge at a time
            y1, x1, y2, x2 = vy[i], vx[i], vy[(i + 1) % n], vx[(i + 1) % n]
            crosses = (y1 > yy) != (y2 > yy)
            with np.errstate(divide="ignore", invalid="ignore"):
                xint = x1 + (yy - y1) * (x2 - x1) / (y2 - y1)
            inside ^= crosses & (xx < xint)
        return inside


def blob_mask(seed: int, h: int, w: int, area: float) -> np.ndarray:
    """Three-ellipse blob rasterised at (h, w), covering `area` of the pixels."""
    return Blob.draw(seed, h, w).fit_area(area).raster()


def polygon_mask(seed: int, h: int, w: int, area: float) -> np.ndarray:
    """12-vertex star polygon rasterised at (h, w), covering `area` of the pixels."""
    return StarPolygon.draw(seed, h, w).fit_area(area).raster()


# ----------------------------------------------------------------------------
# tensors
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class LayerSpec:
    """One convolution: input (h, w, c_in) -> c_out, k x k kernel, stride, pad,
    output block size `block`, block-grid dilation `dilate`, storage dtype."""

    name: str
    h: int
    w: int
    c_in: int
    c_out: int
    k: int = 3
    stride: int = 1
    pad: int = 1
    block: int = 6
    dilate: int = 1
    dtype: str = "bf16"
    w_std: float | None = None  # None -> He-normal

    @property
    def std(self) -> float:
        return self.w_std if self.w_std is not None else math.sqrt(2.0 / (self.c_in * self.k * self.k))


def _randn(shape, seed: int, std: float = 1.0) -> torch.Tensor:
    g = torch.Generator().manual_seed(int(seed))
    return torch.randn(shape, generator=g, dtype=torch.float32) * std


def make_layer_tensors(spec: LayerSpec, seed: int):
    """Weight (OIHW, storage dtype) and bias (fp32) for one layer."""
    dt = DTYPES[spec.dtype]
    w = _randn((spec.c_out, spec.c_in, spec.k, spec.k), seed * 7919 + 11, spec.std).to(dt)
    b = _randn((spec.c_out,), seed * 7919 + 13, 0.01)
    return w, b


def make_activation(n: int, h: int, w: int, c: int, dtype: str, seed: int, layout: str = "NHWC"):
    """A ~ N(0, 1), rounded to the storage dtype; NHWC unless layout == 'NCHW'."""
    shape = (n, h, w, c) if layout == "NHWC" else (n, c, h, w)
    return _randn(shape, seed * 104729 + 3).to(DTYPES[dtype])


def make_edit(a_orig: torch.Tensor, mask: np.ndarray, kind: str, seed: int, layout: str = "NHWC"):
    """Edited activation that differs from `a_orig` exactly on the pixels of `mask`.

    kind == 'add':     A_e = A_o + N(0, 1) on the masked pixels (all channels), in fp32.
    kind == 'replace': masked pixels get fresh N(0, 1) values.
    mask is [h, w] (shared by every image) or [n, h, w].
    """
    m = torch.from_numpy(np.ascontiguousarray(mask).astype(bool))
    if m.dim() == 2:
        m = m.unsqueeze(0).expand(a_orig.shape[0], -1, -1)
    m = m.unsqueeze(-1) if layout == "NHWC" else m.unsqueeze(1)
    noise = _randn(a_orig.shape, seed * 15485863 + 5)
    if kind == "add":
        new = (a_orig.float() + noise).to(a_orig.dtype)
    elif kind == "replace":
        new = noise.to(a_orig.dtype)
    else:
        raise ValueError(kind)
    return torch.where(m, new, a_orig)


# ----------------------------------------------------------------------------
# the workloads
# ----------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    description: str
    layers: tuple
    n: int = 1
    chain: bool = False  # layer l+1 consumes layer l's output
    edit: str = "blob"  # rect | blob | polygon
    area: float = 0.012
    edit_kind: str = "replace"
    layout: str = "NHWC"
    tau: float = 1e-6
    mask_hw: tuple = (256, 256)  # resolution the edit shape is fitted at


def _chain_layers():
    # levels 256/128/64/32 with 128/256/256/512 channels; two 3x3 s1 convs and one
    # 3x3 s2 downsample per level; output block size 6/6/4/4.
    out, cin = [], 128
    for res, c, b in ((256, 128, 6), (128, 256, 6), (64, 256, 4), (32, 512, 4)):
        out.append(LayerSpec(f"L{res}_a", res, res, cin, c, 3, 1, 1, b, 1))
        out.append(LayerSpec(f"L{res}_b", res, res, c, c, 3, 1, 1, b, 1))
        out.append(LayerSpec(f"L{res}_down", res, res, c, c, 3, 2, 1, b, 1))
        cin = c
    return tuple(out)


WORKLOADS = {
    "rect_64x64x64_f32": Workload(
        "rect_64x64x64_f32",
        "3x3 s1 p1 conv, fp32, NCHW 1x64x64x64 -> 64; 10x12 rectangle edit; 8x8 output blocks",
        (LayerSpec("conv", 64, 64, 64, 64, 3, 1, 1, 8, 0, "f32", 0.05),),
        edit="rect", area=120 / 4096, edit_kind="add", layout="NCHW", mask_hw=(64, 64)),
    "unet_256x256x128_bf16": Workload(
        "unet_256x256x128_bf16",
        "U-Net-shaped 3x3 s1 conv, bf16 NHWC 1x256x256x128 -> 128; 1.2% blob; 6x6 blocks, dilate 1",
        (LayerSpec("conv", 256, 256, 128, 128, 3, 1, 1, 6, 1, "bf16"),)),
    "unet_chain_12conv_bf16": Workload(
        "unet_chain_12conv_bf16",
        "U-Net conv chain 256/128/64/32 x 128/256/256/512, bf16; mask pooled per scale",
        _chain_layers(), chain=True),
    "gaugan_4conv_bf16": Workload(
        "gaugan_4conv_bf16",
        "GauGAN-like standalone 3x3 convs, bf16, 1.2% polygon (area sweep 0.5-30%)",
        (LayerSpec("g32x64", 32, 64, 1024, 1024, 3, 1, 1, 4, 1),
         LayerSpec("g64x128", 64, 128, 1024, 512, 3, 1, 1, 4, 1),
         LayerSpec("g128x256", 128, 256, 512, 256, 3, 1, 1, 6, 1),
         LayerSpec("g256x512", 256, 512, 256, 128, 3, 1, 1, 6, 1)),
        edit="polygon", mask_hw=(256, 512)),
    "ldm_64x64x320_f16": Workload(
        "ldm_64x64x320_f16",
        "latent-diffusion-shaped 3x3 and 1x1 convs, fp16, 64^2x320 / 32^2x640 / 16^2x1280",
        (LayerSpec("l64_3x3", 64, 64, 320, 320, 3, 1, 1, 4, 1, "f16"),
         LayerSpec("l64_1x1", 64, 64, 320, 320, 1, 1, 0, 4, 1, "f16"),
         LayerSpec("l32_3x3", 32, 32, 640, 640, 3, 1, 1, 4, 1, "f16"),
         LayerSpec("l32_1x1", 32, 32, 640, 640, 1, 1, 0, 4, 1, "f16"),
         LayerSpec("l16_3x3", 16, 16, 1280, 1280, 3, 1, 1, 2, 1, "f16"),
         LayerSpec("l16_1x1", 16, 16, 1280, 1280, 1, 1, 0, 2, 1, "f16")),
        mask_hw=(64, 64)),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def _sweep_points():
    """Block size and dilation sweep: (workload name, layer with the swept
    block size and dilation).  The U-Net layer at 256x256, and the latent-
    diffusion 3x3 layers at the low resolutions (32x32, 16x16) where only
    1-2 pixel blocks keep the update sparse."""
    pts = []
    base = WORKLOADS["unet_256x256x128_bf16"].layers[0]
    for b in (2, 4, 6, 8, 12, 16):
        for d in (0, 1, 2):
            pts.append(("unet_256x256x128_bf16", dataclasses.replace(base, name=f"unet_b{b}_d{d}", block=b, dilate=d)))
    for lname, blocks in (("l32_3x3", (1, 2, 4, 8)), ("l16_3x3", (1, 2, 4))):
        lay = next(x for x in WORKLOADS["ldm_64x64x320_f16"].layers if x.name == lname)
        for b in blocks:
            for d in (0, 1):
                pts.append(("ldm_64x64x320_f16", dataclasses.replace(lay, name=f"{lname}_b{b}_d{d}", block=b, dilate=d)))
    return tuple(pts)


SWEEP = _sweep_points()


def edit_shape(wl: Workload, seed: int, area: float | None = None):
    """The continuous edit shape of a blob/polygon workload, fitted at wl.mask_hw."""
    a = wl.area if area is None else area
    h, w = wl.mask_hw
    if wl.edit == "blob":
        return Blob.draw(seed, h, w).fit_area(a)
    if wl.edit == "polygon":
        return StarPolygon.draw(seed, h, w).fit_area(a)
    raise ValueError(wl.edit)

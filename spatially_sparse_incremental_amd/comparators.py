"""The bounding-box crop, the alternative to tiles that the mer.dev notes
("Efficient Spatially Sparse Inference...", section 3.2) describe and set
aside: recompute a dense convolution on the smallest rectangle that holds the
change (plus the kernel's reach), keep the cache elsewhere.

Used by the benchmarks as a comparator, on the GPU:
  * `edit_bbox`: the changed pixels' bounding box, from a diff mask;
  * `bbox_out_rect`: the output pixels that box can reach;
  * `bbox_crop_conv`: dense conv of that output rectangle (torch, i.e. MIOpen)
    written into a copy of the cache;
  * `bbox_block_list`: every block touching that output rectangle, for running
    the same rectangle through this library's tile path.
"""
from __future__ import annotations

import torch
import torch.nn.functional as F


def edit_bbox(mask: torch.Tensor):
    """(y0, y1, x0, x1), inclusive, of the set pixels of a [n, h, w] mask over
    all images, or None when nothing changed.  Synchronises with the device."""
    rows = mask.amax(dim=(0, 2)).nonzero()
    if rows.numel() == 0:
        return None
    cols = mask.amax(dim=(0, 1)).nonzero()
    return int(rows[0]), int(rows[-1]), int(cols[0]), int(cols[-1])


def bbox_out_rect(bbox, h, w, k, s, p):
    """Output rows and columns (inclusive) whose input window meets the box."""
    y0, y1, x0, x1 = bbox
    ho, wo = (h + 2 * p - k) // s + 1, (w + 2 * p - k) // s + 1

    def span(a0, a1, no):
        lo = max(0, -(-(a0 + p - k + 1) // s))  # ceil((a0 + p - k + 1) / s)
        hi = min(no - 1, (a1 + p) // s)
        return lo, hi

    oy0, oy1 = span(y0, y1, ho)
    ox0, ox1 = span(x0, x1, wo)
    return oy0, oy1, ox0, ox1


def bbox_crop_conv(a_edit, weight_oihw, bias, cache, rect, k, s, p, out=None):
    """`out` (a copy of `cache` unless given) with the output rectangle
    recomputed by a dense conv of the cropped input (NHWC tensors; the weight
    in OIHW, ideally channels_last; bias fp32 or None)."""
    n, h, w, _ = a_edit.shape
    oy0, oy1, ox0, ox1 = rect
    if out is None:
        out = cache.clone()
    iy0, iy1 = oy0 * s - p, oy1 * s - p + k - 1
    ix0, ix1 = ox0 * s - p, ox1 * s - p + k - 1
    crop = a_edit[:, max(iy0, 0):min(iy1, h - 1) + 1, max(ix0, 0):min(ix1, w - 1) + 1, :].permute(0, 3, 1, 2)
    pads = (max(0, -ix0), max(0, ix1 - (w - 1)), max(0, -iy0), max(0, iy1 - (h - 1)))
    if any(pads):
        crop = F.pad(crop, pads)
    y = F.conv2d(crop, weight_oihw, None if bias is None else bias.to(a_edit.dtype), stride=s)
    out[:, oy0:oy1 + 1, ox0:ox1 + 1, :] = y.permute(0, 2, 3, 1)
    return out


def bbox_block_list(rect, b, nby, nbx, n=1, device="cuda"):
    """Ascending linear indices of the blocks that touch the output rectangle,
    in every image, and their count (both int32 on `device`)."""
    oy0, oy1, ox0, ox1 = rect
    by = torch.arange(oy0 // b, oy1 // b + 1)
    bx = torch.arange(ox0 // b, ox1 // b + 1)
    per = (by[:, None] * nbx + bx[None, :]).reshape(-1)
    lin = torch.cat([img * nby * nbx + per for img in range(n)]).to(torch.int32)
    idx = torch.zeros(n * nby * nbx, dtype=torch.int32)
    idx[:lin.numel()] = lin
    return idx.to(device), torch.tensor([lin.numel()], dtype=torch.int32, device=device)

"""Host logic of the bounding-box comparator (CPU): the output rectangle a
changed input box can reach, against brute force, and the block list of a
rectangle."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from spatially_sparse_incremental_amd import comparators as cmp


@pytest.mark.parametrize("h,w,k,s,p", [(20, 17, 3, 1, 1), (21, 18, 3, 2, 1), (15, 15, 1, 1, 0), (19, 23, 5, 1, 2),
                                       (16, 16, 5, 2, 2)])
def test_out_rect_is_the_reach_of_the_box(h, w, k, s, p):
    rng = np.random.default_rng(h * 100 + w + k + s)
    for _ in range(25):
        y0, x0 = rng.integers(0, h), rng.integers(0, w)
        y1, x1 = rng.integers(y0, h), rng.integers(x0, w)
        img = torch.zeros((1, 1, h, w), dtype=torch.float64)
        img[0, 0, y0:y1 + 1, x0:x1 + 1] = 1.0
        reach = F.conv2d(img, torch.ones((1, 1, k, k), dtype=torch.float64), stride=s, padding=p)[0, 0] > 0
        ys, xs = reach.nonzero(as_tuple=True)
        assert cmp.bbox_out_rect((y0, y1, x0, x1), h, w, k, s, p) == (int(ys.min()), int(ys.max()),
                                                                       int(xs.min()), int(xs.max()))


def test_edit_bbox_of_a_mask():
    m = torch.zeros((2, 9, 11), dtype=torch.uint8)
    assert cmp.edit_bbox(m) is None
    m[0, 2, 3] = 1
    m[1, 6, 8] = 1
    assert cmp.edit_bbox(m) == (2, 6, 3, 8)


def test_block_list_of_a_rectangle():
    idx, cnt = cmp.bbox_block_list((5, 12, 0, 6), 4, 4, 3, n=2, device="cpu")
    blocks = {(0, by, bx) for by in range(1, 4) for bx in range(0, 2)} | {(1, by, bx) for by in range(1, 4)
                                                                          for bx in range(0, 2)}
    want = sorted((img * 4 + by) * 3 + bx for img, by, bx in blocks)
    assert int(cnt) == len(want)
    assert idx[:len(want)].tolist() == want

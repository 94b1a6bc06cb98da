"""Block size and dilation sweep at full size: every point of the sweep grid
(the 256x256 U-Net layer, b = 2..16 and d = 0..2; the 32x32 and 16x16
latent-diffusion 3x3 layers down to 1-pixel blocks) checked like the
workload configs: list and untouched pixels bit for bit, sampled blocks
against the oracle."""
import pytest
import torch

import spatially_sparse_incremental_amd as ssi
import synth
from _parity import check_layer_sampled, run_layer_full

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("point", synth.SWEEP, ids=[L.name for _, L in synth.SWEEP])
def test_sweep_point(point):
    wname, L = point
    wl = synth.workload(wname)
    seed = 9
    m = synth.edit_shape(wl, seed).raster(L.h, L.w)
    a_o = synth.make_activation(1, L.h, L.w, L.c_in, L.dtype, seed)
    a_e = synth.make_edit(a_o, m, wl.edit_kind, seed)
    wt, bias = synth.make_layer_tensors(L, seed)
    cache = synth.make_activation(1, L.h, L.w, L.c_out, L.dtype, seed + 50)
    mask = ssi.sige_diff_mask(a_o.cuda(), a_e.cuda(), wl.tau)
    out, idx = run_layer_full(a_e.cuda(), wt, bias, cache.cuda(), L, mask)
    print(f"\n[case] {L.name}: {idx.numel()} blocks", flush=True)
    check_layer_sampled(L.name, a_e, wt, bias, cache, out.cpu(), idx, L, mask.cpu(), seed)

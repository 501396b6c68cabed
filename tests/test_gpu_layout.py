"""Device layout maps against the oracle, bit-exact (GPU)."""

import random

import numpy as np
import pytest
import torch

from oracle import layout as ol

pytestmark = pytest.mark.gpu


def _lib():
    from layout_algebra_tiled_amd import Layout, gemm
    return Layout, gemm


def test_device_is_gfx950():
    _, g = _lib()
    assert g.device_check().startswith("gfx950")


def test_zipped_divide_eval_all_32768():
    """The device evaluates zipped_divide((256,128):(128,1),(16,16)) at every
    index exactly as the oracle does (the page's 32,768-element gate)."""
    Layout, g = _lib()
    zd = Layout.parse("(256,128):(128,1)").zipped_divide((16, 16))
    out = torch.empty(32768, dtype=torch.int64, device="cuda")
    g.layout_eval_device(zd, out)
    torch.cuda.synchronize()
    want = ol.enumerate_offsets(ol.zipped_divide(ol.parse_layout("(256,128):(128,1)"), (16, 16)))
    assert out.cpu().tolist() == want


def test_device_gather_32768():
    """dst[x] = src[zd(x)]: the matrix gathered tile by tile through the layout."""
    Layout, g = _lib()
    zd = Layout.parse("(256,128):(128,1)").zipped_divide((16, 16))
    src = torch.arange(32768, dtype=torch.int32, device="cuda") * 3 + 1
    dst = torch.full((32768,), -1, dtype=torch.int32, device="cuda")
    g.gather_device(zd, src, dst)
    torch.cuda.synchronize()
    o = ol.zipped_divide(ol.parse_layout("(256,128):(128,1)"), (16, 16))
    want = [3 * o(x) + 1 for x in range(32768)]
    assert dst.cpu().tolist() == want


@pytest.mark.parametrize("elem", [torch.uint8, torch.int16, torch.int32, torch.int64])
def test_random_layouts_eval_and_gather(elem):
    Layout, g = _lib()
    rng = random.Random(7)
    for _ in range(40):
        k = rng.randint(1, 4)
        shape = tuple(rng.randint(1, 9) for _ in range(k))
        stride = tuple(rng.randint(0, 40) for _ in range(k))
        lay = ol.Layout(shape, stride)
        want = ol.enumerate_offsets(lay)
        L = Layout.parse(str(lay))
        out = torch.empty(len(want), dtype=torch.int64, device="cuda")
        g.layout_eval_device(L, out)
        src = (torch.arange(ol.cosize(lay), device="cuda") % 101).to(elem)
        dst = torch.empty(len(want), dtype=elem, device="cuda")
        g.gather_device(L, src, dst)
        torch.cuda.synchronize()
        assert out.cpu().tolist() == want
        assert dst.cpu().tolist() == [v % 101 for v in want]


def test_wide_layout_uses_64bit_offsets():
    """cosize above 2^31: offsets are computed in 64 bits (sampled check)."""
    Layout, g = _lib()
    lay = ol.Layout((1024, 64, 8), (1, 1024, 1 << 31))
    L = Layout.parse(str(lay))
    n = 1024 * 64 * 8
    out = torch.empty(n, dtype=torch.int64, device="cuda")
    g.layout_eval_device(L, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    rng = np.random.default_rng(0)
    for x in list(rng.integers(0, n, 3000)) + [0, n - 1]:
        assert int(got[x]) == ol.evaluate(lay, int(x))


def test_partial_and_empty_and_refused():
    Layout, g = _lib()
    from layout_algebra_tiled_amd import LtError
    L = Layout.parse("(8,4):(4,1)")
    out = torch.full((32,), -1, dtype=torch.int64, device="cuda")
    g.layout_eval_device(L, out, n=10)
    g.layout_eval_device(L, out, n=0)
    torch.cuda.synchronize()
    assert out.cpu().tolist()[:10] == [L(x) for x in range(10)] and out.cpu().tolist()[10:] == [-1] * 22
    with pytest.raises(LtError):
        g.layout_eval_device(L, out, n=33)

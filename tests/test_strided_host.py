"""Host logic of the strided binding, without a GPU: ``strided_dims`` must
describe a view so that the element (n, c, h, w) of the (N, C, H, W)
description sits at n*s0 + c*s1 + h*s2 + w*s3 from the view's pointer -- the
addressing the strided C calls document.  Checked against torch's own
storage offsets: a base tensor holding 0, 1, 2, ... gives each element of a
view its offset as its value."""
import ctypes

import pytest
import torch

import normalization_gn_stats_amd as gn


def _offsets_ok(view, N, C, H, W, s):
    vals = (view - view.storage_offset()).reshape(N, C, H * W)   # logical order; spatial flattened row-major
    n = torch.arange(N).view(N, 1, 1)
    c = torch.arange(C).view(1, C, 1)
    p = torch.arange(H * W).view(1, 1, H * W)
    want = n * s[0] + c * s[1] + (p // W) * s[2] + (p % W) * s[3]
    return torch.equal(vals, want.expand_as(vals))


def _base(*shape, channels_last=False):
    """A dense tensor whose values are their own storage offsets."""
    n = torch.Size(shape).numel()
    if not channels_last:
        return torch.arange(n, dtype=torch.int64).reshape(shape)
    mem = (shape[0], *shape[2:], shape[1])          # memory order: n, spatial..., c
    return torch.arange(n, dtype=torch.int64).reshape(mem).permute(0, len(shape) - 1, *range(1, len(shape) - 1))


VIEWS = {
    "crop_w": lambda: _base(2, 5, 6, 9)[..., 2:7],
    "crop_hw": lambda: _base(2, 3, 8, 9)[..., 1:-1, 2:-1],
    "channel_slice": lambda: _base(2, 10, 4, 4)[:, 3:8],
    "sample_step": lambda: _base(5, 3, 4, 4)[::2],
    "steps": lambda: _base(2, 3, 9, 10)[:, :, ::2, ::3],
    "transposed": lambda: _base(2, 3, 5, 7).transpose(2, 3),
    "nc_swapped": lambda: _base(3, 2, 4, 5).transpose(0, 1),
    "broadcast_n": lambda: _base(1, 3, 4, 5).expand(4, 3, 4, 5),
    "broadcast_w": lambda: _base(2, 3, 4, 1).expand(2, 3, 4, 6),
    "nhwc_crop": lambda: _base(2, 6, 5, 7, channels_last=True)[:, :, 1:, :-2],
    "rows_2d": lambda: _base(6, 20)[:, 3:15],
    "one_spatial": lambda: _base(2, 4, 30)[..., 5:25],
    "spatial_3d_crop": lambda: _base(2, 3, 4, 6, 10)[..., 1:5],
    "spatial_3d_nhwc": lambda: _base(2, 4, 3, 5, 6, channels_last=True)[:, :, :, 1:4],
    "unit_dims": lambda: _base(2, 3, 1, 7, 1)[:, :, :, 1:6],
}


@pytest.mark.parametrize("name", sorted(VIEWS))
def test_strided_dims_addresses_every_element(name):
    v = VIEWS[name]()
    N, C, H, W, (s,) = gn.strided_dims(v)
    assert (N, C) == tuple(v.shape[:2]) and H * W == v[0, 0].numel()
    assert _offsets_ok(v, N, C, H, W, list(s))


def test_strided_dims_uses_one_grouping_for_all_tensors():
    x = _base(2, 3, 4, 6, 10)[..., 1:5]          # dims (4, 6) mergeable, the last not
    y = torch.empty(2, 3, 4, 6, 4).transpose(2, 3).contiguous().transpose(2, 3)   # (4, 6) not mergeable in y
    with pytest.raises(ValueError):
        gn.strided_dims(x, y)                    # three groups would be needed
    N, C, H, W, (sx, sy) = gn.strided_dims(x, torch.empty(2, 3, 4, 6, 4))
    assert (H, W) == (24, 4)
    assert _offsets_ok(x, N, C, H, W, list(sx))


def test_strided_dims_rejects_three_spatial_groups():
    with pytest.raises(ValueError):
        gn.strided_dims(_base(2, 3, 4, 6, 10)[:, :, ::2, ::2, ::3])


def test_strided_dims_shapes_must_match():
    with pytest.raises(ValueError):
        gn.strided_dims(_base(2, 3, 4, 4), _base(2, 3, 4, 5))


def test_common_layout():
    a = torch.empty(2, 8, 4, 4)
    b = a.contiguous(memory_format=torch.channels_last)
    assert gn.common_layout(a, a, None) == gn.GN_NCHW
    assert gn.common_layout(b, b) == gn.GN_NHWC
    assert gn.common_layout(a, b) is None
    assert gn.common_layout(a[..., 1:]) is None


def test_stride_arrays_are_int64x4():
    *_, (s,) = gn.strided_dims(_base(2, 3, 4, 5)[..., 1:])
    assert isinstance(s, ctypes.Array) and len(s) == 4 and s._type_ is ctypes.c_int64

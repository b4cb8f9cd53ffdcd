"""The C-ABI library on the host: it loads, exports every symbol include/gn.h
declares, and rejects bad arguments before enqueuing anything.  None of these
calls reaches the GPU (validation returns first), so they run without one.

The rejected cases follow the argument checks of the baracuda-kernels
GroupNorm backward plan (non-negative sizes, G > 0 dividing C, supported
dtype, affine parameters all-or-none, workspace at least the queried size,
zero extent is a successful no-op) and the output mask of ROCm/pytorch
PR #3564's tests.
"""
import ctypes
import os
import re
import subprocess

import pytest

from normalization_gn_stats_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gn.h")

F32, F16, BF16 = _lib.GN_F32, _lib.GN_F16, _lib.GN_BF16
NCHW, NHWC = _lib.GN_NCHW, _lib.GN_NHWC
FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: every case below is rejected on the host


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("library not built")
    return _lib.lib()


def header_symbols():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\w[\w\s\*]*?\b(gn_\w+)\s*\(", txt, flags=re.M)))


def test_header_declares_the_binding_list():
    assert header_symbols() == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
    defined = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for s in header_symbols():
        assert s in defined, s
        assert getattr(L, s) is not None


def test_status_strings(L):
    for s in range(6):
        assert L.gn_status_string(s)
    assert L.gn_status_string(_lib.GN_ERR_WAIT) != L.gn_status_string(99)
    assert L.gn_version() >= 100


def test_read_status_rejects_null_word(L):
    # checked before any HIP call
    assert L.gn_read_status(None, None, 0, None) == _lib.GN_ERR_INVALID


def test_options_layout_matches_header():
    """The binding's gn_options mirrors the header's struct (size and field
    offsets), checked against a C program compiled from include/gn.h."""
    import tempfile
    names = [f[0] for f in _lib.Options._fields_]
    src = "#include <stdio.h>\n#include <stddef.h>\n#include \"gn.h\"\nint main(void){printf(\"%zu\\n\", sizeof(gn_options));"
    for n in names:
        src += f'printf("%zu\\n", offsetof(gn_options, {n}));'
    src += "return 0;}\n"
    with tempfile.TemporaryDirectory() as d:
        c, exe = os.path.join(d, "o.c"), os.path.join(d, "o")
        open(c, "w").write(src)
        subprocess.check_call(["gcc", "-I", os.path.dirname(HEADER), c, "-o", exe])
        got = [int(v) for v in subprocess.check_output([exe], text=True).split()]
    assert got[0] == ctypes.sizeof(_lib.Options)
    assert got[1:] == [getattr(_lib.Options, n).offset for n in names]


def fwd(L, x=FAKE, g=None, b=None, y=FAKE, m=FAKE, r=FAKE, N=2, C=8, HW=4, G=2, eps=1e-5, dt=F32, lay=NCHW,
        ws=None, wsb=0):
    return L.gn_forward(x, g, b, y, m, r, N, C, HW, G, eps, dt, lay, ws, wsb, None, None)


def bwd(L, dy=FAKE, x=FAKE, m=FAKE, r=FAKE, g=FAKE, dx=FAKE, dg=FAKE, db=FAKE, mask=7, N=2, C=8, HW=4, G=2,
        dt=F32, lay=NCHW, ws=None, wsb=0):
    return L.gn_backward(dy, x, m, r, g, dx, dg, db, mask, N, C, HW, G, dt, lay, ws, wsb, None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(N=-1), _lib.GN_ERR_INVALID),
    (dict(C=-8), _lib.GN_ERR_INVALID),
    (dict(HW=-4), _lib.GN_ERR_INVALID),
    (dict(G=0), _lib.GN_ERR_INVALID),
    (dict(G=3), _lib.GN_ERR_INVALID),           # 3 does not divide 8
    (dict(dt=7), _lib.GN_ERR_UNSUPPORTED),
    (dict(lay=5), _lib.GN_ERR_UNSUPPORTED),
    (dict(g=FAKE), _lib.GN_ERR_INVALID),        # gamma without beta
    (dict(b=FAKE), _lib.GN_ERR_INVALID),        # beta without gamma
    (dict(x=None), _lib.GN_ERR_INVALID),
    (dict(m=None), _lib.GN_ERR_INVALID),
    (dict(eps=-1.0), _lib.GN_ERR_INVALID),
    (dict(eps=float("nan")), _lib.GN_ERR_INVALID),
    (dict(N=1 << 40, C=1 << 20, HW=1 << 20, G=1), _lib.GN_ERR_INVALID),   # element count overflows
])
def test_forward_rejects(L, kw, status):
    assert fwd(L, **kw) == status


def test_forward_workspace_too_small(L):
    need = L.gn_forward_workspace_size(2, 8, 4, 2, F32, NCHW, None)
    assert need > 0
    assert fwd(L, ws=FAKE, wsb=need - 1) == _lib.GN_ERR_WORKSPACE
    assert fwd(L, ws=None, wsb=0) == _lib.GN_ERR_WORKSPACE


@pytest.mark.parametrize("kw,status", [
    (dict(mask=0), _lib.GN_ERR_INVALID),
    (dict(mask=8), _lib.GN_ERR_INVALID),
    (dict(dx=None), _lib.GN_ERR_INVALID),
    (dict(dg=None), _lib.GN_ERR_INVALID),
    (dict(db=None), _lib.GN_ERR_INVALID),
    (dict(g=None), _lib.GN_ERR_INVALID),             # dgamma/dbeta need gamma
    (dict(g=None, mask=1, dg=None, db=None, dx=FAKE, ws=FAKE, wsb=0), _lib.GN_ERR_WORKSPACE),
    (dict(dy=None), _lib.GN_ERR_INVALID),
    (dict(G=5), _lib.GN_ERR_INVALID),
    (dict(dt=3), _lib.GN_ERR_UNSUPPORTED),
])
def test_backward_rejects(L, kw, status):
    assert bwd(L, **kw) == status


@pytest.mark.parametrize("kw", [dict(N=0), dict(C=0), dict(HW=0)])
def test_zero_extent_is_a_noop(L, kw):
    # outputs are NULL-free fakes: a no-op must not touch them (and reach no GPU)
    assert fwd(L, **kw) == _lib.GN_OK
    assert bwd(L, **kw) == _lib.GN_OK
    assert L.gn_forward_workspace_size(kw.get("N", 2), kw.get("C", 8), kw.get("HW", 4), 2, F32, NCHW, None) == 0


def test_path_selection(L):
    sel = lambda bw, N, C, HW, G, dt, lay, force=0: L.gn_select_path(
        bw, N, C, HW, G, dt, lay, ctypes.byref(_lib.Options(force, 0, None, None, None)))
    assert sel(0, 4096, 1024, 1, 1, F16, NCHW) == _lib.GN_PATH_ROWS
    assert sel(1, 131072, 4096, 1, 1, BF16, NCHW) == _lib.GN_PATH_ROWS
    assert sel(0, 4, 36, 1, 1, F16, NCHW) == _lib.GN_PATH_GENERIC          # 36 not a multiple of 8
    assert sel(0, 4, 36, 1, 1, F16, NCHW, _lib.GN_PATH_ROWS) == -1         # forced path cannot serve
    assert sel(0, 2, 8, 4, 2, F32, NCHW, _lib.GN_PATH_GENERIC) == _lib.GN_PATH_GENERIC
    assert sel(0, 2, 8, 4, 3, F32, NCHW) == -1
    # NHWC streams at every size the stream kernels take (measured faster than
    # the cooperative slab kernels throughout); past their grid limit (more
    # than 65535 samples) the slab kernels take it; NCHW is cooperative
    for bw in (0, 1):
        assert sel(bw, 1, 128, 1024 * 2048, 16, F16, NHWC) == _lib.GN_PATH_STREAM
        assert sel(bw, 1, 128, 64 * 130, 16, F16, NHWC) == _lib.GN_PATH_STREAM
        assert sel(bw, 2, 32, 16 * 16, 8, F32, NHWC) == _lib.GN_PATH_STREAM
        assert sel(bw, 70000, 64, 16, 8, F16, NHWC) == _lib.GN_PATH_SLAB
        assert sel(bw, 112, 64, 512 * 512, 8, F32, NCHW) == _lib.GN_PATH_SLAB
        # NCHW slabs of one workgroup each (the small-slab kernel), however many planes
        assert sel(bw, 2, 32, 16 * 16, 8, F32, NCHW) == _lib.GN_PATH_SLAB
        assert sel(bw, 2, 640, 32 * 32, 32, F16, NCHW) == _lib.GN_PATH_SLAB
    assert sel(0, 1, 128, 64 * 130, 16, F16, NHWC, _lib.GN_PATH_STREAM) == _lib.GN_PATH_STREAM
    assert sel(0, 2, 16, 64, 4, F32, NCHW, _lib.GN_PATH_STREAM) == -1      # stream is NHWC only
    assert sel(0, 2, 96, 64, 4, F16, NHWC, _lib.GN_PATH_STREAM) == _lib.GN_PATH_STREAM   # 12 chunks per pixel
    assert sel(0, 2, 4100, 64, 4, F16, NHWC, _lib.GN_PATH_STREAM) == -1   # more chunks per pixel than threads
    assert sel(0, 2, 36, 64, 4, F16, NHWC, _lib.GN_PATH_STREAM) == -1     # pixel not whole 16-byte chunks
    # channel counts the slab kernels do not take (Stable Diffusion-like) stream
    for bw in (0, 1):
        assert sel(bw, 2, 320, 64 * 64, 32, F16, NHWC) == _lib.GN_PATH_STREAM
        assert sel(bw, 2, 1280, 32 * 32, 32, F16, NHWC) == _lib.GN_PATH_STREAM


def test_workspace_sizes_cover_every_mask(L):
    for mask in range(1, 8):
        n = L.gn_backward_workspace_size(4096, 1024, 1, 1, F16, NCHW, mask, None)
        assert n >= 0
    assert L.gn_backward_workspace_size(4096, 1024, 1, 1, F16, NCHW, 0, None) == 0


# ---- RMSNorm over rows -------------------------------------------------------
def rfwd(L, x=FAKE, g=None, y=FAKE, r=FAKE, N=4, C=64, G=1, eps=1e-5, dt=F16, ws=None, wsb=0, opts=None):
    return L.gn_rms_forward(x, g, y, r, N, C, G, eps, dt, ws, wsb, None, opts)


def rbwd(L, dy=FAKE, x=FAKE, r=FAKE, g=FAKE, dx=FAKE, dg=FAKE, mask=3, N=4, C=64, G=1, dt=F16, ws=None, wsb=0,
         opts=None):
    return L.gn_rms_backward(dy, x, r, g, dx, dg, mask, N, C, G, dt, ws, wsb, None, opts)


def _forced(path):
    return ctypes.byref(_lib.Options(path, 0, None, None, None))


@pytest.mark.parametrize("kw,status", [
    (dict(N=-1), _lib.GN_ERR_INVALID),
    (dict(G=0), _lib.GN_ERR_INVALID),
    (dict(G=3), _lib.GN_ERR_INVALID),                 # 3 does not divide 64
    (dict(dt=7), _lib.GN_ERR_UNSUPPORTED),
    (dict(x=None), _lib.GN_ERR_INVALID),
    (dict(r=None), _lib.GN_ERR_INVALID),
    (dict(eps=-1.0), _lib.GN_ERR_INVALID),
    (dict(C=36), _lib.GN_ERR_UNSUPPORTED),            # not a multiple of 8 fp16 elements
    (dict(C=32768), _lib.GN_ERR_UNSUPPORTED),         # wider than the rows kernels hold
    (dict(x=ctypes.c_void_p(0x10004)), _lib.GN_ERR_UNSUPPORTED),   # not 16-byte aligned
    (dict(opts=_forced(_lib.GN_PATH_SLAB)), _lib.GN_ERR_UNSUPPORTED),
])
def test_rms_forward_rejects(L, kw, status):
    assert rfwd(L, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(mask=0), _lib.GN_ERR_INVALID),
    (dict(mask=_lib.GN_GRAD_DBETA), _lib.GN_ERR_INVALID),      # no bias
    (dict(mask=7), _lib.GN_ERR_INVALID),
    (dict(dx=None), _lib.GN_ERR_INVALID),
    (dict(dg=None), _lib.GN_ERR_INVALID),
    (dict(g=None), _lib.GN_ERR_INVALID),                       # dgamma needs gamma
    (dict(dy=None), _lib.GN_ERR_INVALID),
    (dict(r=None), _lib.GN_ERR_INVALID),
    (dict(C=36), _lib.GN_ERR_UNSUPPORTED),
    (dict(mask=_lib.GN_GRAD_DGAMMA, ws=FAKE, wsb=8), _lib.GN_ERR_WORKSPACE),
])
def test_rms_backward_rejects(L, kw, status):
    assert rbwd(L, **kw) == status


def test_rms_zero_extent_and_sizes(L):
    assert rfwd(L, N=0) == _lib.GN_OK
    assert rbwd(L, N=0) == _lib.GN_OK
    assert L.gn_rms_forward_workspace_size(4096, 1024, 1, F16, None) == 0
    assert L.gn_rms_backward_workspace_size(4096, 1024, 1, F16, _lib.GN_GRAD_DX, None) == 0
    assert L.gn_rms_backward_workspace_size(4096, 1024, 1, F16, _lib.GN_GRAD_DGAMMA, None) > 0
    assert L.gn_rms_backward_workspace_size(4096, 1024, 1, F16, _lib.GN_GRAD_DBETA, None) == 0


# ---- strided tensors --------------------------------------------------------
I64x4 = ctypes.c_int64 * 4


def _st(*v):
    return I64x4(*v)


def dense_nchw(N, C, H, W):
    return _st(C * H * W, H * W, W, 1)


def dense_nhwc(N, C, H, W):
    return _st(H * W * C, 1, W * C, C)


def sfwd(L, x=FAKE, xs="crop", g=None, b=None, y=FAKE, ys="dense", m=FAKE, r=FAKE, N=2, C=8, H=4, W=6, G=2,
         eps=1e-5, dt=F32, ws=None, wsb=0, opts=None):
    if isinstance(xs, str):
        xs = _st(C * H * (W + 2), H * (W + 2), W + 2, 1)    # a crop of a wider NCHW buffer
    if isinstance(ys, str):
        ys = dense_nchw(N, C, H, W)
    return L.gn_forward_strided(x, xs, g, b, y, ys, m, r, N, C, H, W, G, eps, dt, ws, wsb, None, opts)


def sbwd(L, dy=FAKE, dys="crop", x=FAKE, xs="crop", m=FAKE, r=FAKE, g=FAKE, dx=FAKE, dxs="dense", dg=FAKE,
         db=FAKE, mask=7, N=2, C=8, H=4, W=6, G=2, dt=F32, ws=None, wsb=0, opts=None):
    crop = _st(C * H * (W + 2), H * (W + 2), W + 2, 1)
    dys = crop if isinstance(dys, str) else dys
    xs = crop if isinstance(xs, str) else xs
    dxs = dense_nchw(N, C, H, W) if isinstance(dxs, str) else dxs
    return L.gn_backward_strided(dy, dys, x, xs, m, r, g, dx, dxs, dg, db, mask, N, C, H, W, G, dt, ws, wsb, None,
                                 opts)


@pytest.mark.parametrize("kw,status", [
    (dict(N=-1), _lib.GN_ERR_INVALID),
    (dict(H=-1), _lib.GN_ERR_INVALID),
    (dict(W=-2), _lib.GN_ERR_INVALID),
    (dict(G=3), _lib.GN_ERR_INVALID),
    (dict(dt=9), _lib.GN_ERR_UNSUPPORTED),
    (dict(xs=None), _lib.GN_ERR_INVALID),                              # strides required
    (dict(ys=None), _lib.GN_ERR_INVALID),                              # ... for y too when y is given
    (dict(xs=_st(-1, 24, 6, 1)), _lib.GN_ERR_INVALID),                 # negative stride
    (dict(ys=_st(0, 24, 6, 1)), _lib.GN_ERR_INVALID),                  # output broadcast over n: overlap
    (dict(ys=_st(48, 1, 6, 1)), _lib.GN_ERR_INVALID),                  # c and w collide in the output
    (dict(xs=_st(1 << 62, 24, 6, 1)), _lib.GN_ERR_INVALID),            # offsets beyond 2^62
    (dict(g=FAKE), _lib.GN_ERR_INVALID),                               # affine all-or-none
    (dict(x=None), _lib.GN_ERR_INVALID),
    (dict(m=None), _lib.GN_ERR_INVALID),
    (dict(eps=-1.0), _lib.GN_ERR_INVALID),
    (dict(opts=_forced(_lib.GN_PATH_ROWS)), _lib.GN_ERR_UNSUPPORTED),  # only generic serves strides
    (dict(opts=_forced(_lib.GN_PATH_SLAB)), _lib.GN_ERR_UNSUPPORTED),
    (dict(ws=FAKE, wsb=16), _lib.GN_ERR_WORKSPACE),
])
def test_forward_strided_rejects(L, kw, status):
    assert sfwd(L, **kw) == status


def test_forward_strided_input_may_overlap(L):
    # a broadcast input (stride 0 over n) passes validation: only the workspace is missing
    assert sfwd(L, xs=_st(0, 24, 6, 1), ws=FAKE, wsb=16) == _lib.GN_ERR_WORKSPACE


@pytest.mark.parametrize("kw,status", [
    (dict(mask=0), _lib.GN_ERR_INVALID),
    (dict(dys=None), _lib.GN_ERR_INVALID),
    (dict(xs=None), _lib.GN_ERR_INVALID),
    (dict(dxs=None), _lib.GN_ERR_INVALID),                             # dx requested without strides
    (dict(dxs=_st(0, 24, 6, 1)), _lib.GN_ERR_INVALID),                 # overlapping dx
    (dict(dx=None), _lib.GN_ERR_INVALID),
    (dict(g=None), _lib.GN_ERR_INVALID),
    (dict(dy=None), _lib.GN_ERR_INVALID),
    (dict(opts=_forced(_lib.GN_PATH_STREAM)), _lib.GN_ERR_UNSUPPORTED),
    (dict(ws=FAKE, wsb=16), _lib.GN_ERR_WORKSPACE),
    (dict(mask=6, dxs=None, dx=None, ws=FAKE, wsb=16), _lib.GN_ERR_WORKSPACE),   # no dx: its strides unused
])
def test_backward_strided_rejects(L, kw, status):
    assert sbwd(L, **kw) == status


@pytest.mark.parametrize("kw", [dict(N=0), dict(C=0), dict(H=0), dict(W=0)])
def test_strided_zero_extent_is_a_noop(L, kw):
    assert sfwd(L, xs=None, ys=None, **kw) == _lib.GN_OK
    assert sbwd(L, dys=None, xs=None, dxs=None, **kw) == _lib.GN_OK


@pytest.mark.parametrize("N,C,H,W,G,dt", [(2, 8, 4, 6, 2, F32), (4, 1024, 1, 1, 1, F16), (1, 128, 1024, 2048, 16, F16),
                                          (112, 64, 512, 512, 8, F32), (2, 36, 3, 5, 4, BF16)])
def test_dense_strides_are_the_dense_call(L, N, C, H, W, G, dt):
    # dense strides describe exactly the dense call: same workspace, both layouts
    for lay, mk in ((NCHW, dense_nchw), (NHWC, dense_nhwc)):
        s = mk(N, C, H, W)
        assert (L.gn_forward_strided_workspace_size(N, C, H, W, G, dt, s, s, None) ==
                L.gn_forward_workspace_size(N, C, H * W, G, dt, lay, None))
        for mask in (1, 6, 7):
            assert (L.gn_backward_strided_workspace_size(N, C, H, W, G, dt, s, s, s, mask, None) ==
                    L.gn_backward_workspace_size(N, C, H * W, G, dt, lay, mask, None))


def test_strided_workspace_sizes(L):
    crop = _st(64 * 512 * 512, 512 * 512, 512, 1)
    dense = dense_nchw(112, 64, 510, 510)
    n = L.gn_forward_strided_workspace_size(112, 64, 510, 510, 8, F32, crop, dense, None)
    assert n > 0
    assert L.gn_forward_strided_workspace_size(112, 64, 510, 510, 8, F32, crop, dense, _forced(_lib.GN_PATH_SLAB)) == 0
    assert L.gn_forward_strided_workspace_size(112, 64, 510, 510, 8, F32, crop, dense,
                                               _forced(_lib.GN_PATH_GENERIC)) == n
    for mask in range(1, 8):
        assert L.gn_backward_strided_workspace_size(112, 64, 510, 510, 8, F32, crop, crop, dense, mask, None) > 0
    assert L.gn_backward_strided_workspace_size(112, 64, 510, 510, 8, F32, crop, crop, dense, 0, None) == 0


def test_scratch_backward_rejects_sizes_beyond_the_array(L):
    """gn_backward_scratch refuses, on the host, a call whose workspace would
    exceed the static array (rows bf16, 262144 channels in 16 segments: 64 MiB
    of column partials)."""
    N, C, G = 65536, 262144, 16
    assert L.gn_backward_workspace_size(N, C, 1, G, BF16, NCHW, 7, None) > _lib.GN_SCRATCH_BYTES
    assert L.gn_backward_scratch(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 7, N, C, 1, G, BF16, NCHW,
                                 None, None) == _lib.GN_ERR_WORKSPACE
    # argument checks come first, as in gn_backward
    assert L.gn_backward_scratch(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 7, 2, 8, 4, 2, F32, NCHW,
                                 None, None) == _lib.GN_ERR_INVALID


def test_scratch_size_matches_header():
    txt = open(HEADER).read()
    m = re.search(r"#define GN_SCRATCH_BYTES \((\d+)u << (\d+)\)", txt)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.GN_SCRATCH_BYTES

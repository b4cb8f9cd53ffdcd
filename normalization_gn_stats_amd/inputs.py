"""Seeded synthetic inputs and workload shapes shared by tests, smoke and bench.

This module holds no GroupNorm arithmetic: it only draws random tensors of
the workloads' shapes, dtypes and memory layouts, so that the HIP path and
the fp64 oracle see the very same quantised values.

Recipe (per workload, seed 0 unless stated):
  * one ``torch.Generator`` seeded with ``seed``; draw order x, dy, gamma, beta;
  * x and dy: float32 standard normal of logical shape (N, C, H, W), then cast
    to the workload dtype (round to nearest even);
  * gamma = 1 + 0.1*randn(C) and beta = 0.1*randn(C) (float32), except where the
    workload says gamma, beta ~ N(0, 1) (the NHWC image workload, as in the
    apex PR #2018 reproducer, which draws weight and bias with randn);
  * NHWC workloads are made dense in channels_last order, as that reproducer does;
  * a workload with crop = k > 0 draws x and dy over spatial extent
    (H + 2k, W + 2k) and uses their centre (H, W) crops: views whose rows are
    strided, read and written in place (a non-contiguous input);
  * ``draw`` / ``draw_affine``: the same distributions for tensors of any
    shape (the strided-view tests cut their views out of these).
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
ELEM_BYTES = {"f32": 4, "f16": 2, "bf16": 2}


@dataclass(frozen=True)
class Workload:
    name: str
    N: int
    C: int
    H: int
    W: int
    G: int
    dtype: str          # "f32" | "f16" | "bf16"
    layout: str         # "nchw" | "nhwc"
    affine: str = "n1"  # "n1": gamma ~ N(1, 0.1), beta ~ N(0, 0.1); "n01": both ~ N(0, 1)
    eps: float = 1e-5
    op: str = "gn"          # "gn": GroupNorm; "rms": RMSNorm over rows (HW == 1, no beta)
    crop: int = 0           # > 0: x, dy are centre (H, W) crops of (H + 2*crop, W + 2*crop) buffers

    @property
    def HW(self) -> int:
        return self.H * self.W

    @property
    def E(self) -> int:
        return self.N * self.C * self.H * self.W

    @property
    def s(self) -> int:
        return ELEM_BYTES[self.dtype]

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]

    def fwd_min_bytes(self) -> int:
        """Algorithmic bytes of one forward: read x, write y, read gamma/beta,
        write mean/rstd (RMSNorm: gamma only, rstd only)."""
        if self.op == "rms":
            return 2 * self.E * self.s + self.C * 4 + self.N * self.G * 4
        return 2 * self.E * self.s + 2 * self.C * 4 + 2 * self.N * self.G * 4

    def bwd_min_bytes(self, dx: bool = True, dparams: bool = True) -> int:
        """Algorithmic bytes of one backward: read dy, x, gamma, mean/rstd,
        write dx (if asked) and dgamma/dbeta (if asked); RMSNorm: rstd only
        and dgamma only."""
        nstat, nparam = (1, 1) if self.op == "rms" else (2, 2)
        b = 2 * self.E * self.s + self.C * 4 + nstat * self.N * self.G * 4
        if dx:
            b += self.E * self.s
        if dparams:
            b += nparam * self.C * 4
        return b

    def scaled(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


# The five benchmark configurations (the second one has two row shapes).
TINY = Workload("tiny_nchw_f32_2x32x16x16_g8", 2, 32, 16, 16, 8, "f32", "nchw")
ROWS_A = Workload("rows_f16_4096x1024", 4096, 1024, 1, 1, 1, "f16", "nchw")
ROWS_B = Workload("rows_f16_8192x768", 8192, 768, 1, 1, 1, "f16", "nchw")
NHWC_IMG = Workload("nhwc_f16_1x128x1024x2048_g16", 1, 128, 1024, 2048, 16, "f16", "nhwc", affine="n01")
NCHW_BIG = Workload("nchw_f32_112x64x512x512_g8", 112, 64, 512, 512, 8, "f32", "nchw")
ROWS_BIG = Workload("rows_bf16_131072x4096", 131072, 4096, 1, 1, 1, "bf16", "nchw")
# The NCHW configuration's shape in bf16 (the same slab kernels at 2-byte elements).
NCHW_BIG_BF16 = Workload("nchw_bf16_112x64x512x512_g8", 112, 64, 512, 512, 8, "bf16", "nchw")
# Narrow rows with many of them (the "huge M" LayerNorm shape of the same table).
ROWS_NARROW = Workload("rows_f16_131072x64", 131072, 64, 1, 1, 1, "f16", "nchw")

# RMSNorm at the three rms_norm shapes of that table (eps 1e-6: the table
# states none).
RMS_A = Workload("rms_f16_4096x1024", 4096, 1024, 1, 1, 1, "f16", "nchw", eps=1e-6, op="rms")
RMS_BIG = Workload("rms_bf16_131072x4096", 131072, 4096, 1, 1, 1, "bf16", "nchw", eps=1e-6, op="rms")
RMS_NARROW = Workload("rms_f16_131072x64", 131072, 64, 1, 1, 1, "f16", "nchw", eps=1e-6, op="rms")

# Non-contiguous input: the 112x64 images of the NCHW configuration with a
# one-pixel border cropped away (rows of 510 elements 512 apart), read and
# written in place; and a small case of the same kind for the oracle.
CROP_BIG = Workload("nchw_f32_112x64x510x510_g8_crop1", 112, 64, 510, 510, 8, "f32", "nchw", crop=1)
CROP_TINY = Workload("tiny_nchw_f32_2x32x14x14_g8_crop1", 2, 32, 14, 14, 8, "f32", "nchw", crop=1)

WORKLOADS = {w.name: w for w in (TINY, ROWS_A, ROWS_B, NHWC_IMG, NCHW_BIG, NCHW_BIG_BF16, ROWS_BIG, ROWS_NARROW,
                                 RMS_A, RMS_BIG, RMS_NARROW, CROP_BIG, CROP_TINY)}


def make_inputs(wl: Workload, seed: int = 0, device: str = "cpu"):
    """Returns dict(x, dy, gamma, beta) as torch tensors on ``device``.

    x, dy have logical shape (N, C, H, W), dtype ``wl.dtype`` and are dense in
    the workload's layout; gamma, beta are float32 of shape (C,)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    k = wl.crop
    shape = (wl.N, wl.C, wl.H + 2 * k, wl.W + 2 * k)
    out = {}
    for name in ("x", "dy"):
        t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        t = t.to(wl.torch_dtype)
        if wl.layout == "nhwc":
            t = t.contiguous(memory_format=torch.channels_last)
        out[name] = t[:, :, k:k + wl.H, k:k + wl.W] if k else t
    if wl.affine == "n01":
        out["gamma"] = torch.randn(wl.C, generator=gen, device=device, dtype=torch.float32)
        out["beta"] = torch.randn(wl.C, generator=gen, device=device, dtype=torch.float32)
    else:
        out["gamma"] = 1.0 + 0.1 * torch.randn(wl.C, generator=gen, device=device, dtype=torch.float32)
        out["beta"] = 0.1 * torch.randn(wl.C, generator=gen, device=device, dtype=torch.float32)
    return out


def draw(shape, dtype: str, seed: int, device: str = "cpu", channels_last: bool = False) -> torch.Tensor:
    """Standard normal float32 values of ``shape`` from a generator seeded with
    ``seed``, cast to ``dtype`` (round to nearest even); channels_last: dense
    with the channel dimension (1) innermost."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    t = torch.randn(tuple(shape), generator=gen, device=device, dtype=torch.float32).to(DTYPES[dtype])
    if channels_last:
        nd = len(shape)
        t = t.permute(0, *range(2, nd), 1).contiguous().permute(0, nd - 1, *range(1, nd - 1))
    return t


def draw_affine(C: int, seed: int, device: str = "cpu"):
    """gamma ~ N(1, 0.1), beta ~ N(0, 0.1), float32 (C,), seeded."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    g = 1.0 + 0.1 * torch.randn(C, generator=gen, device=device, dtype=torch.float32)
    b = 0.1 * torch.randn(C, generator=gen, device=device, dtype=torch.float32)
    return g, b


def memory_image(t: torch.Tensor, layout: str) -> torch.Tensor:
    """Flat view of a dense (N, C, H, W) tensor in its memory order."""
    if layout == "nhwc":
        return t.permute(0, 2, 3, 1).reshape(-1)
    return t.reshape(-1)


def from_memory_image(flat: torch.Tensor, N: int, C: int, H: int, W: int, layout: str) -> torch.Tensor:
    """Inverse of :func:`memory_image`: logical (N, C, H, W) view of a flat buffer."""
    if layout == "nhwc":
        return flat.reshape(N, H, W, C).permute(0, 3, 1, 2)
    return flat.reshape(N, C, H, W)

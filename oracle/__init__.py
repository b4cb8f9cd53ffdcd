"""fp64 CPU oracle for GroupNorm forward/backward -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package.  The product library never calls it, and it shares no
code with the HIP path: ``gn_oracle.c`` is plain C built with gcc, loaded here
through ctypes over numpy float64 arrays.

Definition followed (see the header of ``gn_oracle.c`` for the citations):
forward = per-(n, group) mean and biased variance, x_hat = (x - mean) /
sqrt(var + eps), y = gamma_c * x_hat + beta_c; backward = dbeta, dgamma column
sums, per-slice A = sum(gamma*dy), B = sum(gamma*dy*x_hat), and
dx = rstd * (gamma*dy - A/M - x_hat*B/M).  RMSNorm over rows (``rms_forward``,
``rms_backward``): r = 1/sqrt(mean(x^2) + eps), y = gamma_c * x * r,
dx = r * (gamma*dy - x_hat * sum(gamma*dy*x_hat)/D), dgamma = sum dy*x_hat.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gn_oracle.c")
LIB = os.path.join(HERE, "libgn_oracle.so")
LIB_MUT = os.path.join(HERE, "libgn_oracle_mutants.so")

NCHW = 0
NHWC = 1


def build(force: bool = True) -> None:
    """Compile the oracle (and its planted-mistake variant) with gcc."""
    for out, extra in ((LIB, []), (LIB_MUT, ["-DGNO_MUTANTS"])):
        if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(SRC):
            continue
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
               "-fno-fast-math", "-ffp-contract=off", *extra, SRC, "-o", out + ".tmp", "-lm"]
        subprocess.check_call(cmd)
        os.replace(out + ".tmp", out)


_libs: dict[str, ctypes.CDLL] = {}


def _load(path: str) -> ctypes.CDLL:
    if path in _libs:
        return _libs[path]
    if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(SRC):
        build(force=False)
    lib = ctypes.CDLL(path)
    i64, p, d, i = ctypes.c_int64, ctypes.c_void_p, ctypes.c_double, ctypes.c_int
    lib.gno_forward.argtypes = [i64, i64, i64, i64, i, p, p, p, d, p, p, p]
    lib.gno_forward.restype = i
    lib.gno_backward.argtypes = [i64, i64, i64, i64, i, p, p, p, d, p, p, p, p, p, p]
    lib.gno_backward.restype = i
    lib.gno_rms_forward.argtypes = [i64, i64, i64, p, p, d, p, p]
    lib.gno_rms_forward.restype = i
    lib.gno_rms_backward.argtypes = [i64, i64, i64, p, p, p, d, p, p, p]
    lib.gno_rms_backward.restype = i
    lib.gno_num_threads.restype = i
    lib.gno_set_num_threads.argtypes = [i]
    _libs[path] = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64)).reshape(-1)


def _layout(layout) -> int:
    if layout in (NCHW, "nchw", "NCHW"):
        return NCHW
    if layout in (NHWC, "nhwc", "NHWC"):
        return NHWC
    raise ValueError(f"unknown layout {layout!r}")


def forward(x, gamma, beta, N: int, C: int, HW: int, G: int, eps: float,
            layout=NCHW, want_y: bool = True, mutant: int = 0):
    """Returns (y or None, mean[N*G], rstd[N*G]) as float64 numpy arrays.

    ``x`` is the flat memory image of the tensor in ``layout``; ``y`` comes back
    in the same layout.  ``eps`` is used exactly as given (pass the float32
    value the device sees, widened)."""
    lib = _load(LIB_MUT if mutant else LIB)
    if mutant:
        ctypes.c_int.in_dll(lib, "gno_mutation").value = mutant
    x = _f64(x)
    g = _f64(gamma)
    b = _f64(beta)
    assert x.size == N * C * HW
    y = np.empty(N * C * HW, np.float64) if want_y else None
    mean = np.empty(N * G, np.float64)
    rstd = np.empty(N * G, np.float64)
    rc = lib.gno_forward(N, C, HW, G, _layout(layout), _ptr(x), _ptr(g), _ptr(b),
                         float(eps), _ptr(y), _ptr(mean), _ptr(rstd))
    if mutant:
        ctypes.c_int.in_dll(lib, "gno_mutation").value = 0
    if rc != 0:
        raise ValueError("oracle forward: invalid arguments")
    return y, mean, rstd


def backward(dy, x, gamma, N: int, C: int, HW: int, G: int, eps: float,
             layout=NCHW, want_dx: bool = True, want_dgamma: bool = True,
             want_dbeta: bool = True, mutant: int = 0):
    """Returns (dx or None, dgamma or None, dbeta or None, mean, rstd), float64."""
    lib = _load(LIB_MUT if mutant else LIB)
    if mutant:
        ctypes.c_int.in_dll(lib, "gno_mutation").value = mutant
    dy = _f64(dy)
    x = _f64(x)
    g = _f64(gamma)
    assert x.size == N * C * HW and dy.size == x.size
    dx = np.empty(N * C * HW, np.float64) if want_dx else None
    dgamma = np.empty(C, np.float64) if want_dgamma else None
    dbeta = np.empty(C, np.float64) if want_dbeta else None
    mean = np.empty(N * G, np.float64)
    rstd = np.empty(N * G, np.float64)
    work = np.empty(2 * N * G, np.float64)
    rc = lib.gno_backward(N, C, HW, G, _layout(layout), _ptr(dy), _ptr(x), _ptr(g),
                          float(eps), _ptr(dx), _ptr(dgamma), _ptr(dbeta),
                          _ptr(mean), _ptr(rstd), _ptr(work))
    if mutant:
        ctypes.c_int.in_dll(lib, "gno_mutation").value = 0
    if rc != 0:
        raise ValueError("oracle backward: invalid arguments")
    return dx, dgamma, dbeta, mean, rstd


def rms_forward(x, gamma, N: int, C: int, G: int, eps: float, want_y: bool = True, mutant: int = 0):
    """RMSNorm over rows of D = C/G channels of an [N, C] tensor.
    Returns (y or None, rstd[N*G]) as float64 numpy arrays."""
    lib = _load(LIB_MUT if mutant else LIB)
    if mutant:
        ctypes.c_int.in_dll(lib, "gno_mutation").value = mutant
    x = _f64(x)
    g = _f64(gamma)
    assert x.size == N * C
    y = np.empty(N * C, np.float64) if want_y else None
    rstd = np.empty(N * G, np.float64)
    rc = lib.gno_rms_forward(N, C, G, _ptr(x), _ptr(g), float(eps), _ptr(y), _ptr(rstd))
    if mutant:
        ctypes.c_int.in_dll(lib, "gno_mutation").value = 0
    if rc != 0:
        raise ValueError("oracle rms forward: invalid arguments")
    return y, rstd


def rms_backward(dy, x, gamma, N: int, C: int, G: int, eps: float, want_dx: bool = True,
                 want_dgamma: bool = True, mutant: int = 0):
    """Returns (dx or None, dgamma or None, rstd) as float64 numpy arrays."""
    lib = _load(LIB_MUT if mutant else LIB)
    if mutant:
        ctypes.c_int.in_dll(lib, "gno_mutation").value = mutant
    dy = _f64(dy)
    x = _f64(x)
    g = _f64(gamma)
    assert x.size == N * C and dy.size == x.size
    dx = np.empty(N * C, np.float64) if want_dx else None
    dgamma = np.empty(C, np.float64) if want_dgamma else None
    rstd = np.empty(N * G, np.float64)
    rc = lib.gno_rms_backward(N, C, G, _ptr(dy), _ptr(x), _ptr(g), float(eps), _ptr(dx), _ptr(dgamma), _ptr(rstd))
    if mutant:
        ctypes.c_int.in_dll(lib, "gno_mutation").value = 0
    if rc != 0:
        raise ValueError("oracle rms backward: invalid arguments")
    return dx, dgamma, rstd


def num_threads() -> int:
    return _load(LIB).gno_num_threads()


def set_num_threads(n: int) -> None:
    _load(LIB).gno_set_num_threads(n)

"""fp64 CPU oracle of the Mamba-2 SSD recurrence (ctypes wrapper of ssd_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The HIP library and
its Python binding never import, link or call it, and it imports nothing from
them.

The recurrence it runs is written out in ``ssd_oracle.c``'s header; it follows
"Compiler-First State Space Duality and Portable O(1) Autoregressive Caching
for Inference", section 2 (diagonal per-head state, chunkable recurrence, O(1)
on-device state cache).  Every argument is widened to fp64 before the call; the
callers widen bf16 inputs exactly (``ssd_inputs.widen``).

Parity pins (tests/test_oracle_pins.py): brute-force quadratic
(semiseparable-matrix) form, A = 0 prefix sums, the memoryless and pure-decay
limits, a closed-form geometric series, superposition, B/C rescaling, batch /
head permutation and group replication, chunk-size invariance of a separately
written chunked form, split continuity and the one-pass decode identity.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "ssd_oracle.c")
LIBRARY = os.path.join(_HERE, "libssd_oracle.so")
CFLAGS = ["-O2", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off", "-fno-fast-math"]

_lib = None


def build(source: str = SOURCE, out: str = LIBRARY) -> str:
    """Compile the oracle with gcc (fp64, no FMA contraction, no fast-math)."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, source, "-o", tmp, "-lm", "-lpthread"], check=True)
    os.replace(tmp, out)
    return out


def load(path: str | None = None):
    """Load the built oracle (building it first if nothing is built)."""
    global _lib
    if path is not None:
        lib = ctypes.CDLL(path)
    else:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIBRARY):
            build()
        lib = ctypes.CDLL(LIBRARY)
    f = lib.ssd_oracle_scan
    i64, dp = ctypes.c_int64, ctypes.POINTER(ctypes.c_double)
    f.argtypes = [i64] * 6 + [dp] * 9 + [ctypes.c_int]
    f.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def ssd_scan(x, dt, A, B, C, D, h0=None, nthreads: int = 1, lib=None):
    """Run the recurrence over x[b, L, H, P] (see ssd_oracle.c).

    Returns (y[b, L, H, P], final_state[b, H, P, N]) as fp64 arrays.
    """
    x, dt, A, B, C, D = map(_f64, (x, dt, A, B, C, D))
    bsz, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dt.shape == (bsz, L, H) and A.shape == (H,) and D.shape == (H,)
    assert B.shape == (bsz, L, G, N) and C.shape == B.shape
    if h0 is not None:
        h0 = _f64(h0)
        assert h0.shape == (bsz, H, P, N)
    y = np.zeros((bsz, L, H, P), dtype=np.float64)
    hL = np.zeros((bsz, H, P, N), dtype=np.float64)
    lib = lib or load()
    rc = lib.ssd_oracle_scan(bsz, L, H, P, N, G, _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                             _ptr(D), _ptr(h0), _ptr(y), _ptr(hL), int(nthreads))
    if rc != 0:
        raise ValueError(f"ssd_oracle_scan rejected the arguments (rc={rc})")
    return y, hL


def dt_softplus(u, bias=None):
    """Step size of the fused input prep: softplus(u + bias) = log(1 + exp(u + bias))
    in fp64, with bias per head (the last axis of u) or None.

    The workloads draw the step size through a softplus of a uniform u; the
    library can take u and a per-head bias instead of the step size and form
    it in its kernels.  Written as the plain definition with numpy's
    log(exp(0) + exp(v)), which is evaluated without overflow.
    """
    v = np.asarray(u, dtype=np.float64)
    if bias is not None:
        v = v + np.asarray(bias, dtype=np.float64)
    return np.logaddexp(0.0, v)


def ssd_decode_step(state, x, dt, A, B, C, D, nthreads: int = 1, lib=None):
    """One more iteration of the recurrence on a cached state.

    state [b, H, P, N], x [b, H, P], dt [b, H], B/C [b, G, N].
    Returns (y[b, H, P], new_state[b, H, P, N]).
    """
    x, dt, B, C = map(_f64, (x, dt, B, C))
    y, s = ssd_scan(x[:, None], dt[:, None], A, B[:, None], C[:, None], D, h0=state,
                    nthreads=nthreads, lib=lib)
    return y[:, 0], s

"""Shared helpers for the GPU parity tests: move seeded inputs to the device,
run the oracle on the same values, and compare.

Error metric: rel(a, r) = ||a - r||_F / ||r||_F in fp64, applied to the whole
tensor and to every (batch row, head) slice, so that one broken head cannot
hide in the norm.  Tolerances: 2e-2 for bf16 inputs with fp32 accumulation,
1e-5 for the fp32 path.
"""
from __future__ import annotations

import os

import numpy as np
import torch

import oracle
import ssd_inputs as si

TOL = {"bf16": 2e-2, "f32": 1e-5}
NTHREADS = min(16, os.cpu_count() or 1)


def dev(a: np.ndarray, io: str | None = None) -> torch.Tensor:
    """Host array (bf16 bit patterns when io == 'bf16') -> cuda tensor."""
    if io == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    """cuda tensor -> fp64 host array (exact widening)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def widen_inputs(inp: dict, io: str) -> dict:
    return {"x": si.widen(inp["x"], io), "dt": inp["dt"].astype(np.float64),
            "B": si.widen(inp["B"], io), "C": si.widen(inp["C"], io)}


def rel(a, r) -> float:
    a = np.asarray(a, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    n = np.linalg.norm(r.ravel())
    d = np.linalg.norm((a - r).ravel())
    return float(d / n) if n > 0 else float(d)


def check_y(y, yref, tol, what="y"):
    """y, yref: [b, L, H, P].  Whole tensor and every (b, h) slice within tol."""
    assert y.shape == yref.shape, (y.shape, yref.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite values"
    worst = rel(y, yref)
    assert worst <= tol, f"{what}: rel {worst:.3e} > {tol}"
    for b in range(y.shape[0]):
        for h in range(y.shape[2]):
            e = rel(y[b, :, h], yref[b, :, h])
            assert e <= tol, f"{what}[b={b}, h={h}]: rel {e:.3e} > {tol}"
    return worst


def check_state(s, sref, tol, what="state"):
    """s, sref: [b, H, P, N]."""
    assert s.shape == sref.shape, (s.shape, sref.shape)
    assert np.all(np.isfinite(s)), f"{what}: non-finite values"
    worst = rel(s, sref)
    assert worst <= tol, f"{what}: rel {worst:.3e} > {tol}"
    for b in range(s.shape[0]):
        for h in range(s.shape[1]):
            e = rel(s[b, h], sref[b, h])
            assert e <= tol, f"{what}[b={b}, h={h}]: rel {e:.3e} > {tol}"
    return worst


def oracle_heads(inp: dict, io: str, A, D, pairs, h0=None):
    """Oracle on selected (b, h) pairs only: returns y[len(pairs), L, P], s[len(pairs), P, N].

    ``inp`` holds the stored (not widened) inputs; each pair is widened and run
    as its own 1-batch, 1-head problem on that pair's inputs (head h reads group
    h // (H // G)), threaded over pairs.
    """
    from concurrent.futures import ThreadPoolExecutor

    H, G = inp["x"].shape[2], inp["B"].shape[2]

    def one(pair):
        b, h = pair
        g = h // (H // G)
        x = si.widen(inp["x"][b:b + 1, :, h:h + 1], io)
        dt = inp["dt"][b:b + 1, :, h:h + 1].astype(np.float64)
        Bm = si.widen(inp["B"][b:b + 1, :, g:g + 1], io)
        Cm = si.widen(inp["C"][b:b + 1, :, g:g + 1], io)
        s0 = None if h0 is None else np.asarray(h0[b:b + 1, h:h + 1], dtype=np.float64)
        y, s = oracle.ssd_scan(x, dt, np.array([A[h]]), Bm, Cm, np.array([D[h]]), h0=s0)
        return y[0, :, 0], s[0, 0]

    with ThreadPoolExecutor(NTHREADS) as ex:
        res = list(ex.map(one, pairs))
    return np.stack([r[0] for r in res]), np.stack([r[1] for r in res])


def sample_pairs(bsz, H, n, seed):
    rng = np.random.default_rng(seed)
    pairs = {(0, 0), (bsz - 1, H - 1)}
    while len(pairs) < min(n, bsz * H):
        pairs.add((int(rng.integers(bsz)), int(rng.integers(H))))
    return sorted(pairs)

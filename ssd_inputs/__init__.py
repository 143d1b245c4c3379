"""Seeded synthetic inputs for the Mamba-2 SSD layer workloads.

This module is shared by the fp64 oracle (``oracle/``) and the HIP path
(``state_space_model_mamba_amd``) and by nothing else of either side.  It
holds none of the method's arithmetic: it only draws random numbers, applies
the input-side transforms the workloads prescribe (dt = softplus(u),
A = -exp(A_log), bf16 quantisation of x/B/C) and lays the arrays out as the
layer expects them:

    x  [batch, seqlen, nheads, headdim]      bf16 (or fp32)
    dt [batch, seqlen, nheads]               fp32, already softplus-ed
    A  [nheads]                              fp32, negative
    B  [batch, seqlen, ngroups, dstate]      bf16 (or fp32)
    C  [batch, seqlen, ngroups, dstate]      bf16 (or fp32)
    D  [nheads]                              fp32
    state [batch, nheads, headdim, dstate]   fp32

The pages ("Compiler-First State Space Duality and Portable O(1)
Autoregressive Caching for Inference", section 4, results) measure whole
Mamba-2 models at the 130M..2.7B scales on Wikitext-103; no dataset or trained
weight is available, so these seeded draws of the same layer shapes stand in
for them.

Draw recipe (one ``numpy.random.SeedSequence(seed)`` per workload, PCG64):
  child 0: A_log[H] ~ U(0, ln 16) then D[H] ~ N(0, 1)
  child 1: initial / cached state ~ N(0, 1)            (only where used)
  child 2: decode tokens; its child k holds step k's token, drawn with the
           per-token recipe below at seqlen 1
  child 3 + k: token block k (``TOKEN_BLOCK`` tokens), in this order:
           x ~ N(0,1), B ~ N(0,1)/sqrt(N), C ~ N(0,1)/sqrt(N),
           u ~ U(ln expm1(0.001), ln expm1(0.1)), dt = log1p(exp(u))
Blocks are independent, so any block (e.g. config 4's [0, 4096) prefix) can be
generated alone and blocks can be generated in parallel threads.

bf16 values are produced by round-to-nearest-even of the fp32 draw, done once
here; both sides then consume exactly the same values.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

TOKEN_BLOCK = 4096
DT_MIN, DT_MAX = 0.001, 0.1
A_LOG_MAX = math.log(16.0)


# --------------------------------------------------------------------------
# bf16 helpers (storage format only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 -> bf16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + (((u >> 16) & 1) + np.uint32(0x7FFF))) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def widen(a: np.ndarray, io: str) -> np.ndarray:
    """Exact widening of a stored array (bf16 bits or fp32) to fp64."""
    if io == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Workload table
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk: int
    io: str                      # "f32" or "bf16" (x, B, C, y); dt/A/D/state are fp32
    seed: int
    decode_steps: int = 0        # decode steps following the prefill (or alone)
    decode_batches: tuple = field(default_factory=tuple)
    random_state: bool = False   # decode-only workloads start from a N(0,1) state
    prefix: int = 0              # tokens checked in full against the oracle

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # Tiny fp32 layer; zero initial state; then 16 decode steps.
    "tiny_f32": Workload("tiny_f32", 1, 256, 4, 16, 16, 1, 64, "f32", seed=0, decode_steps=16),
    # Mamba-2-130M-shaped layer: d_inner 1536 = 24 heads x 64.
    "m2_130m": Workload("m2_130m", 8, 2048, 24, 64, 128, 1, 256, "bf16", seed=1),
    # Mamba-2-2.7B-shaped layer: d_inner 5120 = 80 heads x 64.
    "m2_2p7b": Workload("m2_2p7b", 4, 8192, 80, 64, 128, 1, 256, "bf16", seed=2),
    # Decode-only O(1) step at the 2.7B shape, 1000 in-place steps from a N(0,1) state.
    "decode_2p7b": Workload("decode_2p7b", 256, 0, 80, 64, 128, 1, 256, "bf16", seed=3,
                            decode_steps=1000, decode_batches=(1, 16, 64, 256),
                            random_state=True),
    # Long context: 131072 tokens, 8 B/C groups, then 256 decode steps.
    "longctx_2p7b": Workload("longctx_2p7b", 1, 131072, 80, 64, 128, 8, 256, "bf16", seed=4,
                             decode_steps=256, prefix=4096),
}


def _threads() -> int:
    env = os.environ.get("SSD_GEN_THREADS")
    if env:
        return max(1, int(env))
    return max(1, min(16, os.cpu_count() or 1))


def _rng(ss: np.random.SeedSequence) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(ss))


def _children(seed: int, nblk: int = 0):
    # A fresh SeedSequence each call, so child k is the same whatever nblk is.
    return np.random.SeedSequence(seed).spawn(3 + nblk)


def _store(a32: np.ndarray, io: str) -> np.ndarray:
    return f32_to_bf16_bits(a32) if io == "bf16" else np.ascontiguousarray(a32, dtype=np.float32)


def _draw_tokens(rng: np.random.Generator, batch: int, ntok: int, H: int, P: int, G: int,
                 N: int, io: str):
    x = rng.standard_normal((batch, ntok, H, P), dtype=np.float32)
    b = rng.standard_normal((batch, ntok, G, N), dtype=np.float32) / np.float32(math.sqrt(N))
    c = rng.standard_normal((batch, ntok, G, N), dtype=np.float32) / np.float32(math.sqrt(N))
    lo, hi = math.log(math.expm1(DT_MIN)), math.log(math.expm1(DT_MAX))
    u = rng.uniform(lo, hi, size=(batch, ntok, H))
    dt = np.log1p(np.exp(u)).astype(np.float32)          # softplus, fp64 -> fp32
    return _store(x, io), dt, _store(b, io), _store(c, io)


def head_params(w: Workload):
    """A[H] (fp32, in [-16, -1]) and D[H] (fp32)."""
    ss = _children(w.seed)[0]
    rng = _rng(ss)
    a_log = rng.uniform(0.0, A_LOG_MAX, size=w.nheads)
    A = (-np.exp(a_log)).astype(np.float32)
    D = rng.standard_normal(w.nheads).astype(np.float32)
    return A, D


def random_state(w: Workload, batch: int | None = None) -> np.ndarray:
    """N(0,1) fp32 state [batch, H, P, N] (decode-only workloads)."""
    bsz = w.batch if batch is None else batch
    ss = _children(w.seed)[1]
    return _rng(ss).standard_normal((bsz, w.nheads, w.headdim, w.dstate), dtype=np.float32)


def token_blocks(w: Workload, t0: int, t1: int):
    """Block indices covering tokens [t0, t1)."""
    return range(t0 // TOKEN_BLOCK, (t1 + TOKEN_BLOCK - 1) // TOKEN_BLOCK)


def prefill_inputs(w: Workload, t0: int = 0, t1: int | None = None, threads: int | None = None):
    """Token tensors for tokens [t0, t1) of the workload's prefill.

    Returns dict(x, dt, B, C) with the full batch; bf16 tensors are uint16 bit
    patterns.  Any sub-range gives exactly the values of the full draw.
    """
    t1 = w.seqlen if t1 is None else t1
    assert 0 <= t0 <= t1 <= w.seqlen
    H, P, G, N = w.nheads, w.headdim, w.ngroups, w.dstate
    nblk_total = (w.seqlen + TOKEN_BLOCK - 1) // TOKEN_BLOCK
    children = _children(w.seed, nblk_total)[3:]
    xdt = np.uint16 if w.io == "bf16" else np.float32
    L = t1 - t0
    x = np.empty((w.batch, L, H, P), dtype=xdt)
    dt = np.empty((w.batch, L, H), dtype=np.float32)
    B = np.empty((w.batch, L, G, N), dtype=xdt)
    C = np.empty((w.batch, L, G, N), dtype=xdt)

    def work(k):
        bs = k * TOKEN_BLOCK
        ntok = min(TOKEN_BLOCK, w.seqlen - bs)
        xb, dtb, bb, cb = _draw_tokens(_rng(children[k]), w.batch, ntok, H, P, G, N, w.io)
        lo, hi = max(t0, bs), min(t1, bs + ntok)
        if lo >= hi:
            return
        s = slice(lo - bs, hi - bs)
        d = slice(lo - t0, hi - t0)
        x[:, d] = xb[:, s]
        dt[:, d] = dtb[:, s]
        B[:, d] = bb[:, s]
        C[:, d] = cb[:, s]

    blocks = list(token_blocks(w, t0, t1)) if L > 0 else []
    nt = threads or _threads()
    if nt > 1 and len(blocks) > 1:
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(work, blocks))
    else:
        for k in blocks:
            work(k)
    return dict(x=x, dt=dt, B=B, C=C)


def decode_tokens(w: Workload, batch: int, s0: int, s1: int, threads: int | None = None):
    """Per-step decode tokens for steps [s0, s1): x[S,b,H,P], dt[S,b,H], B/C[S,b,G,N]."""
    H, P, G, N = w.nheads, w.headdim, w.ngroups, w.dstate
    children = _children(w.seed)[2].spawn(max(s1, 1))
    xdt = np.uint16 if w.io == "bf16" else np.float32
    S = s1 - s0
    x = np.empty((S, batch, H, P), dtype=xdt)
    dt = np.empty((S, batch, H), dtype=np.float32)
    B = np.empty((S, batch, G, N), dtype=xdt)
    C = np.empty((S, batch, G, N), dtype=xdt)

    def work(k):
        xb, dtb, bb, cb = _draw_tokens(_rng(children[k]), batch, 1, H, P, G, N, w.io)
        i = k - s0
        x[i], dt[i], B[i], C[i] = xb[:, 0], dtb[:, 0], bb[:, 0], cb[:, 0]

    nt = threads or _threads()
    if nt > 1 and S > 1:
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(work, range(s0, s1)))
    else:
        for k in range(s0, s1):
            work(k)
    return dict(x=x, dt=dt, B=B, C=C)


def small_workload(name="small", batch=2, seqlen=200, nheads=4, headdim=64, dstate=128,
                   ngroups=1, chunk=64, io="bf16", seed=100, **kw) -> Workload:
    """Ad-hoc workload with the same value distributions (for tests)."""
    return Workload(name, batch, seqlen, nheads, headdim, dstate, ngroups, chunk, io, seed, **kw)


# --------------------------------------------------------------------------
# Gated DeltaNet decode tokens (the FPGA decode page's second fixed-state
# recurrence).  The page fixes the shapes (2 MB of fp32 state over 32 value
# heads: dk = dv = 128; value heads grouped two per query/key head) and no
# value distributions; the draw below follows what the recurrence expects of
# its inputs: unit-norm keys and queries, a decay gate g in (0.8, 1) and a write
# strength beta in (0.1, 0.9), values ~ N(0, 1), the state ~ N(0, 1) / sqrt(dk).
# --------------------------------------------------------------------------
GDN_SHAPE = dict(qk_heads=16, v_heads=32, dk=128, dv=128)


def gdn_tokens(seed: int, steps: int, batch: int, qk_heads: int, v_heads: int, dk: int, dv: int,
               io: str = "bf16"):
    """q, k [T, b, Hk, dk], v [T, b, Hv, dv] (bf16 bits or fp32), g, beta [T, b, Hv] fp32,
    and state0 [b, Hv, dk, dv] fp32."""
    rng = _rng(np.random.SeedSequence(seed))
    q = rng.standard_normal((steps, batch, qk_heads, dk), dtype=np.float32)
    k = rng.standard_normal((steps, batch, qk_heads, dk), dtype=np.float32)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((steps, batch, v_heads, dv), dtype=np.float32)
    g = rng.uniform(0.8, 1.0, (steps, batch, v_heads)).astype(np.float32)
    beta = rng.uniform(0.1, 0.9, (steps, batch, v_heads)).astype(np.float32)
    state0 = (rng.standard_normal((batch, v_heads, dk, dv), dtype=np.float32)
              / np.float32(math.sqrt(dk)))
    return dict(q=_store(q, io), k=_store(k, io), v=_store(v, io), g=g, beta=beta,
                state0=state0)

"""fp64 CPU oracle of the Gated DeltaNet (GDN) decode step.

TEST INFRASTRUCTURE ONLY, under the same rule as the rest of ``oracle/``:
only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may use it; the HIP library never does.

"A Persistent-State Dataflow Accelerator for Memory-Bound Linear Attention
Decode on FPGA", section 2B: the standard GDN step makes three passes over the
recurrent state -- a read to retrieve the value stored under the key, a read
and write to update the state, a read to form the output.  This oracle makes
exactly those three passes, in fp64, one (batch row, value head) at a time:

    r   = S_{t-1}^T k                       (retrieval)
    dv  = beta (v - g r)                    (the delta)
    S_t = g S_{t-1} + k dv^T                (update)
    o   = S_t^T q                           (output)

S is [d_k, d_v] per value head.  The page writes the update and the output
identity but not the delta; the delta here is the gated delta rule's (the
value written is the new value minus what the decayed state already returns
for the key, scaled by the write strength beta).  Value head j reads query /
key head j // (Hv / Hk) (the page's grouped value heads, two per query/key
pair in its model).
"""
from __future__ import annotations

import numpy as np


def gdn_decode_step(S, q, k, v, g, beta):
    """One GDN decode step.

    S [B, Hv, dk, dv], q and k [B, Hk, dk], v [B, Hv, dv], g and beta [B, Hv].
    Returns (o [B, Hv, dv], S_new [B, Hv, dk, dv]) in fp64; S is not modified.
    """
    S = np.array(S, dtype=np.float64)
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    g, beta = np.asarray(g, dtype=np.float64), np.asarray(beta, dtype=np.float64)
    B, Hv, dk, dv = S.shape
    Hk = q.shape[1]
    assert Hv % Hk == 0 and q.shape == (B, Hk, dk) and k.shape == q.shape
    assert v.shape == (B, Hv, dv) and g.shape == (B, Hv) and beta.shape == (B, Hv)
    o = np.empty((B, Hv, dv))
    for b in range(B):
        for j in range(Hv):
            i = j // (Hv // Hk)
            s = S[b, j]
            r = s.T @ k[b, i]                                  # pass 1: retrieval
            delta = beta[b, j] * (v[b, j] - g[b, j] * r)
            s = g[b, j] * s + np.outer(k[b, i], delta)         # pass 2: update
            S[b, j] = s
            o[b, j] = s.T @ q[b, i]                            # pass 3: output
    return o, S


def gdn_decode_steps(S, q, k, v, g, beta):
    """T steps in order: q, k [T, B, Hk, dk], v [T, B, Hv, dv], g, beta [T, B, Hv].
    Returns (o [T, B, Hv, dv], S after the last step)."""
    out = []
    for t in range(len(q)):
        o, S = gdn_decode_step(S, q[t], k[t], v[t], g[t], beta[t])
        out.append(o)
    return np.stack(out), S

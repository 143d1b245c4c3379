"""GPU parity of the fused step-size prep (ssd_dims.flags = SSD_DT_SOFTPLUS):
the dt arguments hold u and the kernels form softplus(u + dt_bias[h]) in fp32.

The oracle takes the same fp32 u and bias, forms the step size in fp64
(oracle.dt_softplus) and runs the unchanged recurrence.  Ragged lengths and
forced segment / unit counts check that positions past the end of a sequence
still contribute nothing when u there is not zero.
"""
import numpy as np
import pytest
import torch

import oracle
import ssd_inputs as si
import state_space_model_mamba_amd as ssd
from parity import TOL, check_state, check_y, dev, host, oracle_heads, sample_pairs
from test_gpu_decode import oracle_decode

pytestmark = pytest.mark.gpu


def draw_u(shape, H, seed):
    """u such that softplus(u + bias) spans about 0.0003 .. 0.3, and a per-head bias."""
    rng = np.random.default_rng(seed)
    u = rng.uniform(-8.0, -2.0, shape).astype(np.float32)
    bias = rng.uniform(-0.5, 1.0, H).astype(np.float32)
    return u, bias


@pytest.mark.parametrize("L,nseg,with_bias", [(1100, None, True), (1100, 3, True),
                                              (700, 2, False), (257, 1, True)])
def test_scan_bf16_softplus(L, nseg, with_bias, monkeypatch):
    if nseg is not None:
        monkeypatch.setenv("SSD_NSEG", str(nseg))
    H, G = 8, 2
    w = si.small_workload(batch=2, seqlen=L, nheads=H, ngroups=G, chunk=128, seed=L + 3)
    inp = si.prefill_inputs(w)
    A, D = si.head_params(w)
    u, bias = draw_u(inp["dt"].shape, H, seed=L)
    b = bias if with_bias else None
    ref = dict(inp)
    ref["dt"] = oracle.dt_softplus(u, b)
    pairs = sample_pairs(2, H, 16, seed=L)
    fs_prev = None
    # with D and with D = 0 (D x is about 99% of |y|: only the D = 0 run holds
    # the step sizes' effect on the SSM part of y to the tolerance)
    for Dv, tag in ((D, ""), (np.zeros_like(D), " (D = 0)")):
        y, fs = ssd.ssd_chunk_scan(dev(inp["x"], "bf16"), dev(u), dev(A), dev(inp["B"], "bf16"),
                                   dev(inp["C"], "bf16"), dev(Dv), 128, dt_softplus=True,
                                   dt_bias=None if b is None else dev(b))
        torch.cuda.synchronize()
        yref, sref = oracle_heads(ref, "bf16", A, Dv, pairs)
        yh, sh = host(y), host(fs)
        ys = np.stack([yh[bb, :, h] for bb, h in pairs])[:, :, None]
        ss = np.stack([sh[bb, h] for bb, h in pairs])[:, None]
        check_y(ys, yref[:, :, None], TOL["bf16"], "softplus scan y" + tag)
        check_state(ss, sref[:, None], TOL["bf16"], "softplus scan state" + tag)
        if fs_prev is not None:
            assert np.array_equal(sh, fs_prev)
        fs_prev = sh


def test_scan_f32_softplus():
    w = si.WORKLOADS["tiny_f32"]
    inp = si.prefill_inputs(w)
    A, D = si.head_params(w)
    u, bias = draw_u(inp["dt"].shape, w.nheads, seed=9)
    y, fs = ssd.ssd_chunk_scan(dev(inp["x"]), dev(u), dev(A), dev(inp["B"]), dev(inp["C"]),
                               dev(D), w.chunk, dt_softplus=True, dt_bias=dev(bias))
    torch.cuda.synchronize()
    yref, sref = oracle.ssd_scan(inp["x"], oracle.dt_softplus(u, bias), A, inp["B"], inp["C"], D)
    check_y(host(y), yref, TOL["f32"], "softplus f32 scan y")
    check_state(host(fs), sref, TOL["f32"], "softplus f32 scan state")


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("N,batch", [(128, 3), (128, 40), (16, 5), (256, 4)])
def test_decode_softplus(io, N, batch):
    """One step per call (ssd_decode_step) and all steps in one launch
    (ssd_decode_steps; batch 40 at N = 128 takes its large row blocking)."""
    H, P, steps = 16, 64, 9
    w = si.small_workload(batch=batch, seqlen=0, nheads=H, headdim=P, dstate=N, ngroups=4,
                          io=io, seed=N + batch)
    tok = si.decode_tokens(w, batch, 0, steps)
    A, D = si.head_params(w)
    u, bias = draw_u(tok["dt"].shape, H, seed=N * batch)
    state0 = si.random_state(w, batch)
    x, B, C = dev(tok["x"], io), dev(tok["B"], io), dev(tok["C"], io)
    du, dA, dD, db = dev(u), dev(A), dev(D), dev(bias)
    st1 = dev(state0.copy())
    y1 = torch.empty_like(x)
    for k in range(steps):
        ssd.ssd_decode_step(x[k], du[k], dA, B[k], C[k], dD, st1, y=y1[k], dt_softplus=True,
                            dt_bias=db)
    st2 = dev(state0.copy())
    y2 = ssd.ssd_decode_steps(x, du, dA, B, C, dD, st2, dt_softplus=True, dt_bias=db)
    torch.cuda.synchronize()
    ref = dict(tok)
    ref["dt"] = oracle.dt_softplus(u, bias)
    seqs = list(range(min(batch, 6))) + ([batch - 1] if batch > 6 else [])
    yref, sref = oracle_decode(w, ref, A, D, state0, seqs)
    for name, y, s in (("decode_step", y1, st1), ("decode_steps", y2, st2)):
        check_y(host(y)[:, seqs].transpose(1, 0, 2, 3), yref, TOL[io], f"softplus {name} y")
        check_state(host(s)[seqs], sref, TOL[io], f"softplus {name} state")


def test_softplus_flag_matches_precomputed_dt():
    """The fused prep gives what passing softplus(u + bias) as dt gives, at the
    2.7B layer's head shape.  The two step sizes differ in their last fp32 bits,
    and the scan rounds dt-scaled MFMA operands to bf16, so such a difference
    can move an operand by one bf16 ulp (2^-8 relative): the tolerance is 2e-3,
    ten times below the bf16 parity bar against the oracle."""
    w = si.small_workload(batch=2, seqlen=640, nheads=8, chunk=256, seed=77)
    inp = si.prefill_inputs(w)
    A, D = si.head_params(w)
    u, bias = draw_u(inp["dt"].shape, 8, seed=78)
    dt = oracle.dt_softplus(u, bias).astype(np.float32)
    g = [dev(inp["x"], "bf16"), None, dev(A), dev(inp["B"], "bf16"), dev(inp["C"], "bf16"), dev(D)]
    g[1] = dev(u)
    y1, s1 = ssd.ssd_chunk_scan(*g, 256, dt_softplus=True, dt_bias=dev(bias))
    g[1] = dev(dt)
    y2, s2 = ssd.ssd_chunk_scan(*g, 256)
    torch.cuda.synchronize()
    check_y(host(y1), host(y2), 2e-3, "fused vs precomputed y")
    check_state(host(s1), host(s2), 2e-3, "fused vs precomputed state")

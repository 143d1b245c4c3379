"""GPU parity of ssd_gdn_decode_step (Gated DeltaNet decode, one read and one
write of the state) against the fp64 three-pass oracle (oracle.gdn).

Several consecutive steps are run and every output and the final state are
compared, so an error in the state carried from step to step shows too.
Tolerances as for the SSD paths: 2e-2 relative for bf16 I/O (o rounded to
bf16), 1e-5 for fp32; the state is fp32 on both sides.
"""
import numpy as np
import pytest
import torch

import ssd_inputs as si
import state_space_model_mamba_amd as ssd
from oracle import gdn
from parity import TOL, dev, host, rel

pytestmark = pytest.mark.gpu


def run(tok, io, steps):
    q, k, v = dev(tok["q"], io), dev(tok["k"], io), dev(tok["v"], io)
    g, beta = dev(tok["g"]), dev(tok["beta"])
    state = dev(tok["state0"].copy())
    outs = torch.empty_like(v)
    for t in range(steps):
        ssd.ssd_gdn_decode_step(q[t], k[t], v[t], g[t], beta[t], state, o=outs[t])
    torch.cuda.synchronize()
    return host(outs), host(state)


def oracle_run(tok, io):
    w = lambda a: si.widen(a, io)
    return gdn.gdn_decode_steps(tok["state0"], w(tok["q"]), w(tok["k"]), w(tok["v"]),
                                tok["g"].astype(np.float64), tok["beta"].astype(np.float64))


def check(o, s, oref, sref, tol, what):
    assert np.isfinite(o).all() and np.isfinite(s).all(), what
    assert rel(o, oref) <= tol, f"{what}: o rel {rel(o, oref):.3e}"
    assert rel(s, sref) <= tol, f"{what}: state rel {rel(s, sref):.3e}"
    T, B, Hv = o.shape[:3]
    for b in range(B):
        for j in range(Hv):
            eo, es = rel(o[:, b, j], oref[:, b, j]), rel(s[b, j], sref[b, j])
            assert eo <= tol and es <= tol, f"{what}[b={b}, head {j}]: o {eo:.3e}, state {es:.3e}"


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("batch", [1, 8])
def test_gdn_page_shape(io, batch):
    """The page's shape: 32 value heads over 16 query/key heads, 128 x 128 fp32
    state per value head (2 MB per sequence), 12 steps."""
    sh = si.GDN_SHAPE
    tok = si.gdn_tokens(300 + batch, 12, batch, sh["qk_heads"], sh["v_heads"], sh["dk"], sh["dv"], io)
    o, s = run(tok, io, 12)
    oref, sref = oracle_run(tok, io)
    check(o, s, oref, sref, TOL[io], f"gdn {io} b={batch}")


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv,Hk,Hv", [(64, 64, 2, 2), (64, 256, 1, 4), (256, 64, 3, 6),
                                         (256, 256, 2, 4), (128, 64, 4, 4)])
def test_gdn_shapes(io, dk, dv, Hk, Hv):
    tok = si.gdn_tokens(dk * 7 + dv + Hv, 5, 3, Hk, Hv, dk, dv, io)
    o, s = run(tok, io, 5)
    oref, sref = oracle_run(tok, io)
    check(o, s, oref, sref, TOL[io], f"gdn {io} dk={dk} dv={dv}")


def test_gdn_batch_256_sampled():
    """Batch 256 at the page's shape (537 MB of state), 3 steps; sampled sequences
    against the oracle and the whole batch finite and deterministic."""
    sh = si.GDN_SHAPE
    tok = si.gdn_tokens(311, 3, 256, sh["qk_heads"], sh["v_heads"], sh["dk"], sh["dv"], "bf16")
    o1, s1 = run(tok, "bf16", 3)
    o2, s2 = run(tok, "bf16", 3)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)
    seqs = [0, 77, 255]
    sub = {k: (v[:, seqs] if k != "state0" else v[seqs]) for k, v in tok.items()}
    oref, sref = oracle_run(sub, "bf16")
    check(o1[:, seqs], s1[seqs], oref, sref, TOL["bf16"], "gdn b=256")


def test_gdn_empty_batch():
    z = torch.empty((0, 16, 128), dtype=torch.bfloat16, device="cuda")
    v = torch.empty((0, 32, 128), dtype=torch.bfloat16, device="cuda")
    g = torch.empty((0, 32), dtype=torch.float32, device="cuda")
    st = torch.empty((0, 32, 128, 128), dtype=torch.float32, device="cuda")
    out = ssd.ssd_gdn_decode_step(z, z, v, g, g, st)
    assert out.shape == v.shape


def run_steps_launch(tok, io):
    q, k, v = dev(tok["q"], io), dev(tok["k"], io), dev(tok["v"], io)
    state = dev(tok["state0"].copy())
    o = ssd.ssd_gdn_decode_steps(q, k, v, dev(tok["g"]), dev(tok["beta"]), state)
    torch.cuda.synchronize()
    return host(o), host(state)


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("batch,steps", [(1, 40), (8, 17)])
def test_gdn_steps_page_shape(io, batch, steps):
    """ssd_gdn_decode_steps: every step's output and the final state against the
    oracle, and against the same number of single-step calls.  The launch holds
    the state as S / sc between steps (one multiply-add per element and step),
    so it rounds differently from the single-step kernel: the two agree within
    the same tolerance, not bit for bit."""
    sh = si.GDN_SHAPE
    tok = si.gdn_tokens(500 + batch, steps, batch, sh["qk_heads"], sh["v_heads"], sh["dk"], sh["dv"], io)
    o, s = run_steps_launch(tok, io)
    oref, sref = oracle_run(tok, io)
    check(o, s, oref, sref, TOL[io], f"gdn steps {io} b={batch}")
    o1, s1 = run(tok, io, steps)
    check(o, s, o1.astype(np.float64), s1.astype(np.float64), TOL[io], f"gdn steps vs single {io} b={batch}")


@pytest.mark.parametrize("dk,dv,Hk,Hv", [(64, 64, 2, 2), (256, 64, 3, 6), (256, 256, 2, 4),
                                         (64, 256, 1, 4), (128, 128, 2, 6)])
def test_gdn_steps_shapes(dk, dv, Hk, Hv):
    """Value heads per query/key head 1 and 3 (one value head per work-group)
    and 2 and 4 (pairs of value heads sharing the q/k datapath)."""
    tok = si.gdn_tokens(dk + 3 * dv + Hk, 6, 2, Hk, Hv, dk, dv, "bf16")
    o, s = run_steps_launch(tok, "bf16")
    oref, sref = oracle_run(tok, "bf16")
    check(o, s, oref, sref, TOL["bf16"], f"gdn steps dk={dk} dv={dv}")


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv,Hk,Hv,batch", [(128, 128, 16, 32, 16), (64, 256, 1, 4, 64),
                                               (256, 64, 3, 6, 86)])
def test_gdn_steps_value_head_pairs(io, dk, dv, Hk, Hv, batch):
    """Batches large enough that the launch pairs the value heads of each
    query/key head in one work-group (the pairs fill every CU), against the
    oracle: the page's shape, four value heads per query/key head over two
    128-column tiles, and dk = 256 on 64-column tiles."""
    steps = 7
    tok = si.gdn_tokens(600 + dk + dv + batch, steps, batch, Hk, Hv, dk, dv, io)
    o, s = run_steps_launch(tok, io)
    oref, sref = oracle_run(tok, io)
    check(o, s, oref, sref, TOL[io], f"gdn steps pairs {io} dk={dk} dv={dv} b={batch}")


def test_gdn_steps_zero_steps():
    sh = si.GDN_SHAPE
    tok = si.gdn_tokens(9, 1, 2, sh["qk_heads"], sh["v_heads"], sh["dk"], sh["dv"], "bf16")
    state = dev(tok["state0"].copy())
    q = dev(tok["q"], "bf16")[:0]
    v = dev(tok["v"], "bf16")[:0]
    g = dev(tok["g"])[:0]
    ssd.ssd_gdn_decode_steps(q, q, v, g, g, state)
    torch.cuda.synchronize()
    assert np.array_equal(host(state), tok["state0"])


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_gdn_steps_gate_extremes(io):
    """Gates that force the launch's renormalisation of S / sc: g = 0 (forget),
    g = 1e-12 and 1e-30 (sc leaves [2^-64, 2^64] within a few steps), g = 1,
    mixed over value heads and steps; every output and the final state against
    the oracle."""
    sh = si.GDN_SHAPE
    steps = 24
    tok = si.gdn_tokens(777, steps, 2, sh["qk_heads"], sh["v_heads"], sh["dk"], sh["dv"], io)
    choices = np.array([0.0, 1e-12, 1e-30, 1.0, 0.9], dtype=np.float32)
    pick = np.random.default_rng(778).integers(0, len(choices), tok["g"].shape)
    tok["g"] = choices[pick]
    tok["g"][:, 0, 0] = 1e-12          # one head renormalises every few steps
    tok["g"][:, 1, 3] = 1.0            # one never does
    o, s = run_steps_launch(tok, io)
    oref, sref = oracle_run(tok, io)
    check(o, s, oref, sref, TOL[io], f"gdn steps gate extremes {io}")


@pytest.mark.parametrize("steps", [1, 2, 3, 4])
@pytest.mark.parametrize("dk,dv,Hk,Hv", [(128, 128, 2, 4), (256, 64, 1, 1)])
def test_gdn_steps_few_steps(steps, dk, dv, Hk, Hv):
    """Launches of 1 to 4 steps: the start of the launch's pipeline (q and k
    two steps ahead through three LDS buffers, clamped fetches past the last
    step) against the oracle and single-step calls."""
    tok = si.gdn_tokens(900 + steps + dk, steps, 3, Hk, Hv, dk, dv, "bf16")
    o, s = run_steps_launch(tok, "bf16")
    oref, sref = oracle_run(tok, "bf16")
    check(o, s, oref, sref, TOL["bf16"], f"gdn {steps} steps dk={dk} dv={dv}")
    o1, s1 = run(tok, "bf16", steps)
    check(o, s, o1.astype(np.float64), s1.astype(np.float64), TOL["bf16"], f"gdn {steps} steps vs single")

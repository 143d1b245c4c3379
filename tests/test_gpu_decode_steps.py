"""GPU parity of ssd_decode_steps (S decode steps in one launch) against the
fp64 oracle.

S steps from a cached state are the oracle's scan over those S tokens started
from that state, as for ssd_decode_step; the same per-step tokens are fed to
both.  Shapes are chosen to reach both row blockings of the kernel (the small
one below about two waves per SIMD, the large one above), ragged P, every
supported N, and step counts that are and are not multiples of the kernel's
four-step prefetch.
"""
import numpy as np
import pytest
import torch

import ssd_inputs as si
import state_space_model_mamba_amd as ssd
from parity import TOL, check_state, check_y, dev, host
from test_gpu_decode import oracle_decode, run_decode

pytestmark = pytest.mark.gpu


def run_steps(w, batch, steps, state0):
    tok = si.decode_tokens(w, batch, 0, steps)
    A, D = si.head_params(w)
    io = w.io
    x, dt, B, C = dev(tok["x"], io), dev(tok["dt"]), dev(tok["B"], io), dev(tok["C"], io)
    state = dev(state0.copy())
    ys = ssd.ssd_decode_steps(x, dt, dev(A), B, C, dev(D), state)
    torch.cuda.synchronize()
    return tok, A, D, host(ys), host(state)


def check_steps(w, batch, steps, seqs):
    state0 = si.random_state(w, batch)
    tok, A, D, ys, s = run_steps(w, batch, steps, state0)
    yref, sref = oracle_decode(w, tok, A, D, state0, seqs)
    tol = TOL[w.io]
    check_y(ys[:, seqs].transpose(1, 0, 2, 3), yref, tol, f"decode_steps y (b={batch}, S={steps})")
    check_state(s[seqs], sref, tol, f"decode_steps state (b={batch}, S={steps})")


def test_decode_steps_tiny_f32():
    w = si.WORKLOADS["tiny_f32"].with_(random_state=True)
    check_steps(w, 1, 16, [0])


@pytest.mark.parametrize("batch,nseq", [(1, 1), (16, 6), (256, 8)])
def test_decode_steps_2p7b_1000_steps(batch, nseq):
    """The 2.7B decode shape, 1000 steps in one launch: batch 1 takes the small
    row blocking, 16 and 256 the large one."""
    w = si.WORKLOADS["decode_2p7b"]
    rng = np.random.default_rng(batch + 7)
    seqs = sorted(set([0, batch - 1] + list(rng.choice(batch, size=nseq, replace=False))))
    check_steps(w, batch, w.decode_steps, seqs)


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("P,N,H,G", [(37, 16, 3, 1), (64, 32, 4, 2), (16, 64, 6, 3), (8, 256, 2, 2),
                                     (128, 128, 2, 1), (5, 128, 3, 3)])
@pytest.mark.parametrize("steps", [1, 3, 4, 9])
def test_decode_steps_shapes(io, P, N, H, G, steps):
    w = si.small_workload(batch=5, seqlen=0, nheads=H, headdim=P, dstate=N, ngroups=G, io=io,
                          seed=P * N + steps)
    check_steps(w, 5, steps, list(range(5)))


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("P,N", [(64, 16), (64, 32), (64, 64), (50, 128), (64, 256)])
def test_decode_steps_large_blocking(io, P, N):
    """Enough (batch row, head) pairs (2560) for the large row blocking at every N."""
    H, G, batch = 16, 2, 160
    w = si.small_workload(batch=batch, seqlen=0, nheads=H, headdim=P, dstate=N, ngroups=G, io=io,
                          seed=N + P)
    check_steps(w, batch, 6, [0, 17, 41, batch - 1])


def test_decode_steps_match_decode_step():
    """Every sequence of batch 256 at the 2.7B shape: 24 steps in one launch agree
    with 24 ssd_decode_step calls (same recurrence, another summation order)."""
    w = si.WORKLOADS["decode_2p7b"]
    state0 = si.random_state(w, 256)
    _, _, _, y1, s1 = run_decode(w, 256, 24, state0)
    _, _, _, y2, s2 = run_steps(w, 256, 24, state0)
    tol = TOL[w.io]
    check_y(y2.transpose(1, 0, 2, 3), y1.transpose(1, 0, 2, 3), tol, "steps vs step: y")
    check_state(s2, s1, 1e-5, "steps vs step: state")


def test_decode_steps_empty_and_deterministic():
    w = si.WORKLOADS["decode_2p7b"]
    state0 = si.random_state(w, 4)
    A, D = si.head_params(w)
    state = dev(state0.copy())
    x = torch.empty((0, 4, w.nheads, w.headdim), dtype=torch.bfloat16, device="cuda")
    dt = torch.empty((0, 4, w.nheads), dtype=torch.float32, device="cuda")
    Bm = torch.empty((0, 4, w.ngroups, w.dstate), dtype=torch.bfloat16, device="cuda")
    ssd.ssd_decode_steps(x, dt, dev(A), Bm, Bm.clone(), dev(D), state)
    torch.cuda.synchronize()
    assert np.array_equal(host(state), state0)          # zero steps: state untouched
    _, _, _, y1, s1 = run_steps(w, 4, 7, state0)
    _, _, _, y2, s2 = run_steps(w, 4, 7, state0)
    assert np.array_equal(y1, y2) and np.array_equal(s1, s2)


def test_decode_steps_graph_replay():
    """One ssd_decode_steps launch captured into a HIP graph replays bit-identically
    to the eager call, with eager work and synchronisation between replays."""
    w = si.WORKLOADS["decode_2p7b"]
    batch, steps = 8, 40
    state0 = si.random_state(w, batch)
    _, _, _, y_ref, s_ref = run_steps(w, batch, steps, state0)
    tok = si.decode_tokens(w, batch, 0, steps)
    A, D = si.head_params(w)
    x, dt, B, C = dev(tok["x"], "bf16"), dev(tok["dt"]), dev(tok["B"], "bf16"), dev(tok["C"], "bf16")
    dA, dD = dev(A), dev(D)
    s0 = dev(state0.copy())
    state = s0.clone()
    ys = torch.empty_like(x)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            ssd.ssd_decode_steps(x, dt, dA, B, C, dD, state, y=ys)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        state.copy_(s0)
        ys.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(ys), y_ref), f"replay {rep}: y"
        assert np.array_equal(host(state), s_ref), f"replay {rep}: state"


def _steps_with_heads(A, dt_scale, seed, steps, io="bf16", batch=3):
    """decode_steps with chosen per-head A and dt scaled by dt_scale, against the
    oracle on the same values (all sequences)."""
    H = len(A)
    w = si.small_workload(batch=batch, seqlen=0, nheads=H, io=io, seed=seed)
    tok = si.decode_tokens(w, batch, 0, steps)
    tok["dt"] = (tok["dt"] * np.float32(dt_scale)).astype(np.float32)
    A = np.asarray(A, dtype=np.float32)
    _, D = si.head_params(w)
    state0 = si.random_state(w, batch)
    x, dt, B, C = dev(tok["x"], io), dev(tok["dt"]), dev(tok["B"], io), dev(tok["C"], io)
    state = dev(state0.copy())
    ys = ssd.ssd_decode_steps(x, dt, dev(A), B, C, dev(D), state)
    torch.cuda.synchronize()
    yref, sref = oracle_decode(w, tok, A.astype(np.float64), D, state0, list(range(batch)))
    y, s = host(ys), host(state)
    assert np.isfinite(y).all() and np.isfinite(s).all()
    check_y(y.transpose(1, 0, 2, 3), yref, TOL[io], "decay y")
    check_state(s, sref, TOL[io], "decay state")


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_decode_steps_extreme_decay(io):
    """A = -1e6: alpha underflows to 0 on every step, so every step folds the
    scale back and the state is memoryless: H_t = dt_t x_t (outer) B_t."""
    _steps_with_heads([-1e6, -1e6, -5e5, -1e6], 1.0, seed=41, steps=11, io=io)


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_decode_steps_no_decay(io):
    """A = 0: alpha = 1, the scale never moves and the state is a running sum."""
    _steps_with_heads([0.0, 0.0, 0.0], 1.0, seed=42, steps=300, io=io)


def test_decode_steps_decay_mix():
    """Heads from no decay to strong decay over many steps, so that the state
    scale is renormalised every few steps, rarely, or never, head by head."""
    _steps_with_heads([0.0, -0.05, -1.0, -16.0, -100.0, -3.0, -0.5, -40.0], 1.0, seed=43, steps=400)
    _steps_with_heads([-16.0, -8.0, -4.0, -1.0], 10.0, seed=44, steps=90)

"""GPU parity of ssd_decode_step against the fp64 oracle.

A decode step is one more iteration of the recurrence on the cached state, so a
run of S steps of one sequence equals the oracle's scan over those S tokens
started from the same state; the oracle is run that way on sampled sequences.
"""
import numpy as np
import pytest
import torch

import ssd_inputs as si
import state_space_model_mamba_amd as ssd
from parity import TOL, check_state, check_y, dev, host, oracle_heads, widen_inputs, rel
import oracle

pytestmark = pytest.mark.gpu


def run_decode(w, batch, steps, state0):
    tok = si.decode_tokens(w, batch, 0, steps)
    A, D = si.head_params(w)
    io = w.io
    x, dt, B, C = dev(tok["x"], io), dev(tok["dt"]), dev(tok["B"], io), dev(tok["C"], io)
    dA, dD = dev(A), dev(D)
    state = dev(state0.copy())
    ys = torch.empty((steps,) + tuple(x.shape[1:]), dtype=x.dtype, device="cuda")
    for k in range(steps):
        ssd.ssd_decode_step(x[k], dt[k], dA, B[k], C[k], dD, state, y=ys[k])
    torch.cuda.synchronize()
    return tok, A, D, host(ys), host(state)


def oracle_decode(w, tok, A, D, state0, seqs):
    """Oracle over the S decode tokens of the chosen sequences (scan from state0)."""
    io = w.io
    seq = {"x": si.widen(tok["x"][:, seqs], io).transpose(1, 0, 2, 3),
           "dt": tok["dt"][:, seqs].astype(np.float64).transpose(1, 0, 2),
           "B": si.widen(tok["B"][:, seqs], io).transpose(1, 0, 2, 3),
           "C": si.widen(tok["C"][:, seqs], io).transpose(1, 0, 2, 3)}
    return oracle.ssd_scan(seq["x"], seq["dt"], A, seq["B"], seq["C"], D,
                           h0=state0[seqs].astype(np.float64), nthreads=16)


def check_decode(w, batch, steps, seqs):
    state0 = si.random_state(w, batch)
    tok, A, D, ys, s = run_decode(w, batch, steps, state0)
    yref, sref = oracle_decode(w, tok, A, D, state0, seqs)
    tol = TOL[w.io]
    check_y(ys[:, seqs].transpose(1, 0, 2, 3), yref, tol, f"decode y (b={batch})")
    check_state(s[seqs], sref, tol, f"decode state (b={batch})")


def test_decode_tiny_f32():
    w = si.WORKLOADS["tiny_f32"].with_(random_state=True)
    check_decode(w, 1, 16, [0])


@pytest.mark.parametrize("batch,nseq", [(1, 1), (16, 16), (64, 8), (256, 16)])
def test_decode_2p7b_1000_steps(batch, nseq):
    w = si.WORKLOADS["decode_2p7b"]
    rng = np.random.default_rng(batch)
    seqs = sorted(set([0, batch - 1] + list(rng.choice(batch, size=nseq, replace=False))))[:max(nseq, 1)]
    check_decode(w, batch, w.decode_steps, seqs)


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("P,N,H,G", [(37, 16, 3, 1), (64, 32, 4, 2), (16, 64, 6, 3), (8, 256, 2, 2),
                                     (128, 128, 2, 1)])
def test_decode_shapes(io, P, N, H, G):
    w = si.small_workload(batch=5, seqlen=0, nheads=H, headdim=P, dstate=N, ngroups=G, io=io, seed=P * N)
    check_decode(w, 5, 7, list(range(5)))


def test_decode_deterministic_and_in_place():
    w = si.WORKLOADS["decode_2p7b"]
    state0 = si.random_state(w, 4)
    _, _, _, y1, s1 = run_decode(w, 4, 5, state0)
    _, _, _, y2, s2 = run_decode(w, 4, 5, state0)
    assert np.array_equal(y1, y2) and np.array_equal(s1, s2)


def test_decode_step_time_independent_of_context():
    """The O(1) cache: a step moves the same bytes whatever the context length, so
    the state after a long prefix is as cheap to advance as a fresh one (timed)."""
    w = si.WORKLOADS["decode_2p7b"]
    b = 64
    A, D = si.head_params(w)
    tok = si.decode_tokens(w, b, 0, 1)
    x, dt, B, C = dev(tok["x"][0], "bf16"), dev(tok["dt"][0]), dev(tok["B"][0], "bf16"), dev(tok["C"][0], "bf16")
    dA, dD = dev(A), dev(D)
    times = []
    for _ in range(2):
        state = torch.randn((b, w.nheads, w.headdim, w.dstate), device="cuda")
        for _ in range(3):
            ssd.ssd_decode_step(x, dt, dA, B, C, dD, state)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(50):
            ssd.ssd_decode_step(x, dt, dA, B, C, dD, state)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    assert max(times) < 3 * min(times)


@pytest.mark.parametrize("batch", [1, 256])
def test_decode_graph_replay(batch):
    """A run of decode steps captured into one HIP graph (per-step launches
    replaced by a replay) gives bit-identical y and state to the eager run, on
    every replay, with eager work and synchronisation between the replays
    (256: the non-temporal path; 1: the cache-resident one)."""
    w = si.WORKLOADS["decode_2p7b"]
    steps = 12
    state0 = si.random_state(w, batch)
    _, _, _, y_ref, s_ref = run_decode(w, batch, steps, state0)
    tok = si.decode_tokens(w, batch, 0, steps)
    A, D = si.head_params(w)
    x, dt, B, C = dev(tok["x"], "bf16"), dev(tok["dt"]), dev(tok["B"], "bf16"), dev(tok["C"], "bf16")
    dA, dD = dev(A), dev(D)
    s0 = dev(state0.copy())
    state = s0.clone()
    ys = torch.empty((steps,) + tuple(x.shape[1:]), dtype=x.dtype, device="cuda")
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for k in range(steps):
                ssd.ssd_decode_step(x[k], dt[k], dA, B[k], C[k], dD, state, y=ys[k])
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        state.copy_(s0)                         # eager reset between replays
        ys.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(ys), y_ref), f"replay {rep}: y"
        assert np.array_equal(host(state), s_ref), f"replay {rep}: state"

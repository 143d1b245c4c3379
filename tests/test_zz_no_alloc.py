"""GPU test of ssd_chunk_scan_noalloc, the scan entry point that allocates
nothing (its workspace is the library's per-device scratch array): called
through the C ABI, it must give what ssd_chunk_scan with a caller workspace
gives, on consecutive calls of different sizes (the second smaller, then the
first again over the scratch contents the smaller one left), and meet the
oracle's tolerance."""
import numpy as np
import pytest
import torch

import oracle
import ssd_inputs as si
import state_space_model_mamba_amd as ssd
from parity import TOL, check_state, check_y, dev, host, widen_inputs

pytestmark = pytest.mark.gpu


def inputs(w):
    inp = si.prefill_inputs(w)
    A, D = si.head_params(w)
    g = dict(x=dev(inp["x"], "bf16"), dt=dev(inp["dt"]), A=dev(A), B=dev(inp["B"], "bf16"),
             C=dev(inp["C"], "bf16"), D=dev(D))
    return inp, A, D, g


def both(w, g, h0=None, in_place=False, **kw):
    """(y, state) of ssd_chunk_scan with its own workspace and of the no-alloc
    entry point (outputs passed in: nothing is allocated around the call)."""
    args = (g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], w.chunk)
    init1 = None if h0 is None else dev(h0)
    y1, s1 = ssd.ssd_chunk_scan(*args, initial_state=init1,
                                final_state=init1 if in_place else None, **kw)
    init2 = None if h0 is None else dev(h0)
    y2 = torch.empty_like(g["x"])
    s2 = init2 if in_place else torch.empty((w.batch, w.nheads, 64, 128), device="cuda")
    out = ssd.ssd_chunk_scan_noalloc(*args, initial_state=init2, y=y2, final_state=s2, **kw)
    torch.cuda.synchronize()
    assert out[0] is y2 and out[1] is s2
    return host(y1), host(s1), host(y2), host(s2)


def against_oracle(w, inp, A, D, h0, y, s):
    wid = widen_inputs(inp, "bf16")
    yref, sref = oracle.ssd_scan(wid["x"], wid["dt"], A, wid["B"], wid["C"], D,
                                 h0=None if h0 is None else h0.astype(np.float64), nthreads=16)
    check_y(y, yref, TOL["bf16"], "no-alloc y")
    check_state(s, sref, TOL["bf16"], "no-alloc state")


def test_noalloc_matches_scan_on_consecutive_calls():
    big = si.small_workload(batch=2, seqlen=3000, nheads=8, ngroups=2, chunk=256, seed=301)
    small = si.small_workload(batch=1, seqlen=1000, nheads=4, ngroups=1, chunk=128, seed=302)
    # both use the scratch array (the planner cuts them into several segments)
    for w in (big, small):
        assert ssd.ssd_chunk_scan_workspace_size(w.batch, w.seqlen, w.nheads, 64, 128,
                                                 w.ngroups, w.chunk) > 0
    inp_b, A_b, D_b, g_b = inputs(big)
    y1, s1, y2, s2 = both(big, g_b)
    assert np.array_equal(y1, y2) and np.array_equal(s1, s2)
    against_oracle(big, inp_b, A_b, D_b, None, y2, s2)
    # second call, smaller, resuming a cache in place (the state kernel copies
    # the initial state into the scratch array's spare slot first)
    inp_s, A_s, D_s, g_s = inputs(small)
    h0 = np.random.default_rng(3).standard_normal((1, 4, 64, 128)).astype(np.float32)
    y1, s1, y2, s2 = both(small, g_s, h0=h0, in_place=True)
    assert np.array_equal(y1, y2) and np.array_equal(s1, s2)
    against_oracle(small, inp_s, A_s, D_s, h0, y2, s2)
    # the larger call again, over what the smaller one left in the scratch array
    y1b, s1b, y2b, s2b = both(big, g_b)
    assert np.array_equal(y1b, y2b) and np.array_equal(s1b, s2b)
    # D = 0 (the SSM part of y on its own)
    g0 = dict(g_b, D=torch.zeros_like(g_b["D"]))
    y1, s1, y2, s2 = both(big, g0)
    assert np.array_equal(y1, y2) and np.array_equal(s1, s2)
    against_oracle(big, inp_b, A_b, np.zeros_like(D_b), None, y2, s2)


def test_noalloc_fused_step_sizes():
    """With the fused step-size prep (u in place of dt, the step sizes formed
    inside the kernels): the same results as ssd_chunk_scan with its own
    workspace, on a fused call between two plain ones over the same scratch
    array, and the oracle's tolerance on the fp64 step sizes."""
    w = si.small_workload(batch=2, seqlen=3000, nheads=8, ngroups=2, chunk=256, seed=305)
    inp, A, D, g = inputs(w)
    u = np.random.default_rng(306).uniform(-8.0, -2.0, inp["dt"].shape).astype(np.float32)
    bias = np.random.default_rng(307).uniform(-0.5, 1.0, 8).astype(np.float32)
    gu = dict(g, dt=dev(u))
    y1, s1, y2, s2 = both(w, g)
    assert np.array_equal(y1, y2) and np.array_equal(s1, s2)
    y1, s1, y2, s2 = both(w, gu, dt_softplus=True, dt_bias=dev(bias))
    assert np.array_equal(y1, y2) and np.array_equal(s1, s2)
    ref = dict(inp)
    ref["dt"] = oracle.dt_softplus(u, bias).astype(np.float32)
    against_oracle(w, ref, A, D, None, y2, s2)
    y1, s1, y2, s2 = both(w, g)
    assert np.array_equal(y1, y2) and np.array_equal(s1, s2)


def test_noalloc_without_workspace_need():
    """A problem the planner runs as one segment needs no workspace: the entry
    point then never touches the scratch array."""
    w = si.small_workload(batch=1, seqlen=200, nheads=80, ngroups=1, chunk=256, seed=303)
    assert ssd.ssd_chunk_scan_workspace_size(w.batch, w.seqlen, w.nheads, 64, 128, w.ngroups,
                                             w.chunk) == 0
    _, _, _, g = inputs(w)
    y1, s1, y2, s2 = both(w, g)
    assert np.array_equal(y1, y2) and np.array_equal(s1, s2)


def test_noalloc_in_captured_graph():
    """The callers the entry point is for: it is captured once into a HIP graph
    (outputs passed in, no allocation anywhere in the call) and the graph is
    replayed three times, with new inputs copied into the captured buffers
    eagerly between replays; every replay must equal an eager ssd_chunk_scan
    with its own workspace on the same inputs, bit for bit."""
    w = si.small_workload(batch=2, seqlen=1500, nheads=8, ngroups=2, chunk=128, seed=311)
    assert ssd.ssd_chunk_scan_workspace_size(w.batch, w.seqlen, w.nheads, 64, 128,
                                             w.ngroups, w.chunk) > 0
    sets = []
    for k in range(3):
        _, _, _, g = inputs(si.small_workload(batch=2, seqlen=1500, nheads=8, ngroups=2,
                                              chunk=128, seed=312 + k))
        sets.append(g)
    buf = {k: v.clone() for k, v in sets[0].items()}
    y = torch.empty_like(buf["x"])
    s = torch.empty((w.batch, w.nheads, 64, 128), device="cuda")
    args = lambda g: (g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], w.chunk)
    ssd.ssd_chunk_scan_noalloc(*args(buf), y=y, final_state=s)     # first call: scratch address
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            ssd.ssd_chunk_scan_noalloc(*args(buf), y=y, final_state=s)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep, g in enumerate(sets):
        for k in buf:
            buf[k].copy_(g[k])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        y_ref, s_ref = ssd.ssd_chunk_scan(*args(g))
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), f"replay {rep}: y"
        assert torch.equal(s, s_ref), f"replay {rep}: final state"

"""GPU tests of ssd_state_init, the on-device cache initialisation (section 2
of the Compiler-First page: the cache lives on the device and is set there):
the zero state, a copy from another device buffer, src == state (a no-op), an
overlapping src (rejected before anything runs), and capture inside a HIP
graph (a fill/copy kernel, no memset), replayed several times with eager work
in between."""
import ctypes

import numpy as np
import pytest
import torch

import ssd_inputs as si
import state_space_model_mamba_amd as ssd
from parity import TOL, check_state, dev, host

pytestmark = pytest.mark.gpu

SHAPES = [(1, 1, 1, 1), (3, 5, 7, 11), (4, 80, 64, 128), (2, 3, 64, 16)]


@pytest.mark.parametrize("shape", SHAPES)
def test_zero_and_copy(shape):
    g = torch.Generator(device="cuda").manual_seed(sum(shape))
    state = torch.randn(shape, device="cuda", generator=g)
    ssd.ssd_state_init(state)
    torch.cuda.synchronize()
    assert torch.count_nonzero(state) == 0
    src = torch.randn(shape, device="cuda", generator=g)
    ssd.ssd_state_init(state, src)
    torch.cuda.synchronize()
    assert torch.equal(state, src)
    before = state.clone()
    ssd.ssd_state_init(state, state)           # src == state: nothing changes
    torch.cuda.synchronize()
    assert torch.equal(state, before)


def test_overlap_rejected():
    buf = torch.randn(2 * 4 * 8 * 16 + 16, device="cuda")
    state = buf[:2 * 4 * 8 * 16].view(2, 4, 8, 16)
    src = buf[16:].view(2, 4, 8, 16)           # overlaps state, not the same pointer
    before = buf.clone()
    with pytest.raises(ssd.SsdError) as e:
        ssd.ssd_state_init(state, src)
    assert e.value.code == 4                   # SSD_ERR_ALIAS
    torch.cuda.synchronize()
    assert torch.equal(buf, before)            # nothing was launched


def test_graph_captured_init_then_decode():
    """One captured graph holds an init from a saved cache and two decode steps;
    each replay (with eager work that scribbles over the state in between) must
    give the eager result bit for bit, and that result must match the oracle."""
    w = si.small_workload(batch=3, seqlen=0, nheads=8, headdim=64, dstate=128, ngroups=2, seed=71)
    A, D = si.head_params(w)
    tok = si.decode_tokens(w, w.batch, 0, 2)
    x, dt = dev(tok["x"], "bf16"), dev(tok["dt"])
    B, C = dev(tok["B"], "bf16"), dev(tok["C"], "bf16")
    dA, dD = dev(A), dev(D)
    saved = dev(si.random_state(w, w.batch))
    state = torch.empty_like(saved)
    ys = torch.empty((2,) + tuple(x.shape[1:]), dtype=torch.bfloat16, device="cuda")

    def work():
        ssd.ssd_state_init(state, saved)
        for k in range(2):
            ssd.ssd_decode_step(x[k], dt[k], dA, B[k], C[k], dD, state, y=ys[k])

    work()
    torch.cuda.synchronize()
    y_ref, s_ref = ys.clone(), state.clone()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            work()
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(4):
        state.normal_()                        # eager work between replays
        ys.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(state, s_ref), f"replay {rep}: state"
        assert torch.equal(ys, y_ref), f"replay {rep}: y"
    # and the zero-state form, captured on its own
    g0 = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g0, stream=side):
            ssd.ssd_state_init(state)
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        state.normal_()
        torch.cuda.synchronize()
        g0.replay()
        torch.cuda.synchronize()
        assert torch.count_nonzero(state) == 0, f"zero replay {rep}"
    # the eager result against the oracle (two steps from the saved state)
    import oracle
    seq = {"x": si.widen(tok["x"], "bf16").transpose(1, 0, 2, 3),
           "dt": tok["dt"].astype(np.float64).transpose(1, 0, 2),
           "B": si.widen(tok["B"], "bf16").transpose(1, 0, 2, 3),
           "C": si.widen(tok["C"], "bf16").transpose(1, 0, 2, 3)}
    _, sref = oracle.ssd_scan(seq["x"], seq["dt"], A, seq["B"], seq["C"], D,
                              h0=host(saved), nthreads=4)
    check_state(host(s_ref), sref, TOL["bf16"], "state after init + 2 steps")

"""GPU parity of ssd_chunk_scan (and prefill -> decode continuity) against the
fp64 oracle, on the five seeded workloads and on edge cases."""
import os

import numpy as np
import pytest
import torch

import oracle
import ssd_inputs as si
import state_space_model_mamba_amd as ssd
from parity import (TOL, check_state, check_y, dev, host, oracle_heads, rel, sample_pairs,
                    widen_inputs)

pytestmark = pytest.mark.gpu


def gpu_inputs(w, inp):
    A, D = si.head_params(w)
    return dict(x=dev(inp["x"], w.io), dt=dev(inp["dt"]), B=dev(inp["B"], w.io),
                C=dev(inp["C"], w.io), A=dev(A), D=dev(D)), A, D


def gpu_scan(g, chunk, D=None, init=None, **kw):
    y, s = ssd.ssd_chunk_scan(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"] if D is None else D,
                              chunk, initial_state=init, **kw)
    torch.cuda.synchronize()
    return y, s


def full_check(w, Q=None, h0=None, zero_D=True, in_place=False):
    """GPU scan vs the oracle over the whole input (small workloads).  With
    in_place, final_state is the initial-state buffer itself (a fresh copy of
    h0 for each run): the cache resumed in place."""
    Q = Q or w.chunk
    inp = si.prefill_inputs(w)
    g, A, D = gpu_inputs(w, inp)
    wid = widen_inputs(inp, w.io)
    tol = TOL[w.io]

    def run(Dv=None):
        init = None if h0 is None else dev(h0.astype(np.float32))
        kw = {"final_state": init} if (in_place and init is not None) else {}
        y, s = gpu_scan(g, Q, D=Dv, init=init, **kw)
        if kw:
            assert s.data_ptr() == init.data_ptr()
        return y, s

    y, s = run()
    h0d = None if h0 is None else h0.astype(np.float32).astype(np.float64)
    yref, sref = oracle.ssd_scan(wid["x"], wid["dt"], A, wid["B"], wid["C"], D, h0=h0d, nthreads=16)
    check_y(host(y), yref, tol)
    check_state(host(s), sref, tol)
    if zero_D:
        # D masks most of y (|y - D x| is under 1% of |y|); rerun with D = 0 so the
        # SSM part alone is held to the same tolerance.
        y0, s0 = run(torch.zeros_like(g["D"]))
        yref0, _ = oracle.ssd_scan(wid["x"], wid["dt"], A, wid["B"], wid["C"], np.zeros_like(D),
                                   h0=h0d, nthreads=16)
        check_y(host(y0), yref0, tol, "y (D = 0)")
        assert np.array_equal(host(s0), host(s))
    return g, A, D, y, s


# --------------------------------------------------------------------------
# the five workloads
# --------------------------------------------------------------------------
def test_tiny_f32_prefill_then_decode():
    """256-token fp32 prefill, then 16 decode steps from its final state; all
    272 outputs and the final state against the oracle's 272-token recurrence."""
    w = si.WORKLOADS["tiny_f32"]
    inp = si.prefill_inputs(w)
    g, A, D = gpu_inputs(w, inp)
    y, s = gpu_scan(g, w.chunk)
    tok = si.decode_tokens(w, w.batch, 0, w.decode_steps)
    ys = []
    for k in range(w.decode_steps):
        ys.append(ssd.ssd_decode_step(dev(tok["x"][k]), dev(tok["dt"][k]), g["A"], dev(tok["B"][k]),
                                      dev(tok["C"][k]), g["D"], s))
    torch.cuda.synchronize()
    y_all = np.concatenate([host(y), np.stack([host(t) for t in ys], axis=1)], axis=1)
    wid = widen_inputs(inp, "f32")
    seq = {k: np.concatenate([wid[k], (tok[k].astype(np.float64)).transpose(1, 0, *range(2, tok[k].ndim))], axis=1)
           for k in ("x", "dt", "B", "C")}
    yref, sref = oracle.ssd_scan(seq["x"], seq["dt"], A, seq["B"], seq["C"], D)
    check_y(y_all, yref, TOL["f32"], "y (prefill + decode)")
    check_state(host(s), sref, TOL["f32"], "state after decode")


def test_m2_130m_full():
    full_check(si.WORKLOADS["m2_130m"])


def test_m2_2p7b_sampled_heads():
    """Full-size 2.7B layer (B=4, L=8192, H=80); the oracle runs 16 sampled
    (b, h) sequences in full (each 8192 tokens), with and without D."""
    w = si.WORKLOADS["m2_2p7b"]
    inp = si.prefill_inputs(w)
    g, A, D = gpu_inputs(w, inp)
    y, s = gpu_scan(g, w.chunk)
    y0, _ = gpu_scan(g, w.chunk, D=torch.zeros_like(g["D"]))
    pairs = sample_pairs(w.batch, w.nheads, 16, seed=2)
    yref, sref = oracle_heads(inp, w.io, A, D, pairs)
    yref0, _ = oracle_heads(inp, w.io, A, np.zeros_like(D), pairs)
    yh, y0h, sh = host(y), host(y0), host(s)
    tol = TOL[w.io]
    for i, (b, h) in enumerate(pairs):
        assert rel(yh[b, :, h], yref[i]) <= tol, (b, h, rel(yh[b, :, h], yref[i]))
        assert rel(y0h[b, :, h], yref0[i]) <= tol, (b, h, rel(y0h[b, :, h], yref0[i]))
        assert rel(sh[b, h], sref[i]) <= tol, (b, h, rel(sh[b, h], sref[i]))
    assert np.all(np.isfinite(yh)) and np.all(np.isfinite(sh))


@pytest.mark.parametrize("batch,L,nseg", [(16, 700, 1), (13, 1500, 4)])
def test_multi_round_default_plan(batch, L, nseg):
    """Batches whose scan work-groups per segment (batch x 20 head quads) exceed
    the 256 CUs, so no plan fits one round and the planner's cost picks among
    multi-round plans: 16 x 700 tokens in one segment (320 work-groups, two
    rounds, no state kernel); 13 x 1500 tokens in 4 segments (1040 scan and
    780 state work-groups, several rounds of each).  The segment count is read
    back from the workspace size; 16 sampled (b, h) sequences, the last row
    and head among them, against the oracle, with and without D."""
    w = si.small_workload(batch=batch, seqlen=L, nheads=80, ngroups=1, chunk=256, seed=L + batch)
    need = ssd.ssd_chunk_scan_workspace_size(batch, L, 80, 64, 128, 1, 256)
    slots = batch * 80 * nseg if nseg > 1 else 0
    assert need == ((slots * 64 * 128 * 4 + 255) // 256 * 256 + (slots * 4 + 255) // 256 * 256
                    if slots else 0)
    inp = si.prefill_inputs(w)
    g, A, D = gpu_inputs(w, inp)
    y, s = gpu_scan(g, w.chunk)
    y0, s0 = gpu_scan(g, w.chunk, D=torch.zeros_like(g["D"]))
    assert torch.equal(s, s0), "the state does not depend on D"
    pairs = sorted(set(sample_pairs(batch, 80, 14, seed=L) + [(0, 0), (batch - 1, 79)]))
    yref, sref = oracle_heads(inp, w.io, A, D, pairs)
    yref0, _ = oracle_heads(inp, w.io, A, np.zeros_like(D), pairs)
    yh, y0h, sh = host(y), host(y0), host(s)
    tol = TOL[w.io]
    for i, (b, h) in enumerate(pairs):
        assert rel(yh[b, :, h], yref[i]) <= tol, (b, h, rel(yh[b, :, h], yref[i]))
        assert rel(y0h[b, :, h], yref0[i]) <= tol, (b, h, rel(y0h[b, :, h], yref0[i]))
        assert rel(sh[b, h], sref[i]) <= tol, (b, h, rel(sh[b, h], sref[i]))
    assert np.all(np.isfinite(yh)) and np.all(np.isfinite(sh))


def test_longctx_prefix_fullrun_and_decode_continuity():
    """131072 tokens, 8 groups: (1) the [0, 4096) prefix as its own scan against
    the oracle; (2) the full-length scan on 8 sampled heads against the oracle's
    131072-step recurrence; (3) 256 decode steps from the GPU's final state
    against the oracle started from that same state.  Each part is run with the
    workload's D and again with D = 0: D x is about 99% of |y|, so only the
    D = 0 run holds the scan's own output (entering states of every segment,
    the intra-chunk and state->output terms) to the tolerance."""
    w = si.WORKLOADS["longctx_2p7b"]
    A, D = si.head_params(w)
    D0 = np.zeros_like(D)
    tol = TOL[w.io]
    # (1) prefix
    pre = si.prefill_inputs(w, 0, w.prefix)
    gp, _, _ = gpu_inputs(w, pre)
    wp = widen_inputs(pre, w.io)
    sp = None
    for Dv, tag in ((D, ""), (D0, " (D = 0)")):
        yp, sp_v = gpu_scan(gp, w.chunk, D=dev(Dv))
        yref, sref = oracle.ssd_scan(wp["x"], wp["dt"], A, wp["B"], wp["C"], Dv, nthreads=16)
        check_y(host(yp), yref, tol, "prefix y" + tag)
        check_state(host(sp_v), sref, tol, "prefix state" + tag)
        if sp is not None:
            assert torch.equal(sp, sp_v), "the state does not depend on D"
        sp = sp_v
    del gp, yp, sp, sp_v, wp, yref, sref
    # (2) full length: the heads sit in 4 of the 8 groups, at both ends of a
    # group and in the last (two-head) quad of a group's 4 + 4 + 2 split
    inp = si.prefill_inputs(w)
    g, _, _ = gpu_inputs(w, inp)
    y, s = gpu_scan(g, w.chunk)
    y0, s0 = gpu_scan(g, w.chunk, D=dev(D0))
    assert torch.equal(s, s0), "the state does not depend on D"
    pairs = [(0, h) for h in (0, 9, 10, 37, 41, 63, 70, 79)]
    yr, sr = oracle_heads(inp, w.io, A, D, pairs)
    yr0, _ = oracle_heads(inp, w.io, A, D0, pairs)
    yh, y0h, sh = host(y), host(y0), host(s)
    for i, (b, h) in enumerate(pairs):
        assert rel(yh[b, :, h], yr[i]) <= tol, (h, rel(yh[b, :, h], yr[i]))
        assert rel(y0h[b, :, h], yr0[i]) <= tol, ("D = 0", h, rel(y0h[b, :, h], yr0[i]))
        assert rel(sh[b, h], sr[i]) <= tol, (h, rel(sh[b, h], sr[i]))
    # the last 4096 tokens alone: the part of y that the entering states of the
    # late segments dominate (the full-length norm is spread over 131072 tokens)
    tail = slice(w.seqlen - 4096, w.seqlen)
    for i, (b, h) in enumerate(pairs):
        e = rel(y0h[b, tail, h], yr0[i][tail])
        assert e <= tol, ("D = 0, last 4096 tokens", h, e)
    del g, y, y0, s0, inp, yh, y0h
    # (3) decode continuity from the GPU's own final state
    tok = si.decode_tokens(w, w.batch, 0, w.decode_steps)
    dA = dev(A)
    seq = {"x": si.widen(tok["x"], w.io).transpose(1, 0, 2, 3),
           "dt": tok["dt"].astype(np.float64).transpose(1, 0, 2),
           "B": si.widen(tok["B"], w.io).transpose(1, 0, 2, 3),
           "C": si.widen(tok["C"], w.io).transpose(1, 0, 2, 3)}
    for Dv, tag in ((D, ""), (D0, " (D = 0)")):
        dD = dev(Dv)
        ys = []
        s_run = s.clone()
        for k in range(w.decode_steps):
            ys.append(ssd.ssd_decode_step(dev(tok["x"][k], w.io), dev(tok["dt"][k]), dA,
                                          dev(tok["B"][k], w.io), dev(tok["C"][k], w.io), dD,
                                          s_run))
        torch.cuda.synchronize()
        yd = np.stack([host(t) for t in ys], axis=1)
        ydr, sdr = oracle.ssd_scan(seq["x"], seq["dt"], A, seq["B"], seq["C"], Dv, h0=sh,
                                   nthreads=16)
        check_y(yd, ydr, tol, "decode after long prefill" + tag)
        check_state(host(s_run), sdr, tol, "state after long prefill + decode" + tag)


# --------------------------------------------------------------------------
# chunk length, raggedness, groups, segments
# --------------------------------------------------------------------------
@pytest.mark.parametrize("Q", [64, 128, 256, 512])
def test_chunk_size_invariance(Q):
    w = si.small_workload(batch=2, seqlen=1000, nheads=4, ngroups=2, chunk=Q, seed=21)
    full_check(w, Q)


@pytest.mark.parametrize("L", [1, 17, 63, 64, 65, 130, 255, 257])
def test_ragged_lengths(L):
    w = si.small_workload(batch=2, seqlen=L, nheads=3, ngroups=1, chunk=128, seed=L)
    full_check(w)


@pytest.mark.parametrize("H,G", [(8, 8), (8, 2), (10, 5)])
def test_groups(H, G):
    w = si.small_workload(batch=1, seqlen=700, nheads=H, ngroups=G, chunk=64, seed=H * 31 + G)
    full_check(w)


@pytest.mark.parametrize("nseg", ["1", "2", "4096"])
def test_segment_count_extremes(nseg, monkeypatch):
    """One segment per sequence, two, and one segment per chunk."""
    monkeypatch.setenv("SSD_NSEG", nseg)
    w = si.small_workload(batch=2, seqlen=2048 + 77, nheads=2, chunk=64, seed=5)
    full_check(w)


@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("nsub", ["1", "2", "5"])
def test_state_kernel_units(nsub, in_place, monkeypatch):
    """Segments of the state kernel cut into 1, 2 and 5 units, with a ragged
    tail and a non-zero initial state; in_place: the final state is written
    over the initial state (which the state kernel first copies to the spare
    workspace slot that segment 0 of the scan kernel then reads)."""
    monkeypatch.setenv("SSD_NSEG", "3")
    monkeypatch.setenv("SSD_NSUB", nsub)
    w = si.small_workload(batch=2, seqlen=3 * 640 + 50, nheads=4, chunk=128, seed=21)
    h0 = np.random.default_rng(2).standard_normal((2, 4, 64, 128)).astype(np.float32)
    full_check(w, h0=h0, in_place=in_place)


def test_initial_state_and_split_continuity():
    """scan(L) == scan(k) then scan(L - k, initial_state = that final state), for
    a given non-zero initial state; and final_state may alias initial_state."""
    w = si.small_workload(batch=2, seqlen=900, nheads=4, chunk=128, seed=9)
    h0 = np.random.default_rng(1).standard_normal((2, 4, 64, 128)).astype(np.float32)
    g, A, D, y, s = full_check(w, h0=h0, zero_D=False)
    inp = si.prefill_inputs(w)
    for k in (128, 333):
        a = {key: v[:, :k] for key, v in inp.items()}
        b = {key: v[:, k:] for key, v in inp.items()}
        ga, _, _ = gpu_inputs(w, a)
        gb, _, _ = gpu_inputs(w, b)
        state = dev(h0.copy())
        ya, _ = gpu_scan(ga, w.chunk, init=state, final_state=state)    # in place
        yb, _ = gpu_scan(gb, w.chunk, init=state, final_state=state)
        yab = np.concatenate([host(ya), host(yb)], axis=1)
        assert rel(yab, host(y)) < TOL["bf16"] and rel(host(state), host(s)) < TOL["bf16"]


def test_empty_inputs():
    w = si.small_workload(batch=2, seqlen=0, nheads=4, chunk=64, seed=3)
    x = torch.empty((2, 0, 4, 64), dtype=torch.bfloat16, device="cuda")
    dt = torch.empty((2, 0, 4), device="cuda")
    Bm = torch.empty((2, 0, 1, 128), dtype=torch.bfloat16, device="cuda")
    A = torch.full((4,), -1.0, device="cuda")
    D = torch.ones(4, device="cuda")
    h0 = torch.randn((2, 4, 64, 128), device="cuda")
    y, s = ssd.ssd_chunk_scan(x, dt, A, Bm, Bm, D, 64, initial_state=h0)
    y2, s2 = ssd.ssd_chunk_scan(x, dt, A, Bm, Bm, D, 64)
    torch.cuda.synchronize()
    assert y.numel() == 0 and torch.equal(s, h0) and torch.count_nonzero(s2) == 0
    xb = torch.empty((0, 10, 4, 64), dtype=torch.bfloat16, device="cuda")
    yb, sb = ssd.ssd_chunk_scan(xb, torch.empty((0, 10, 4), device="cuda"), A,
                                torch.empty((0, 10, 1, 128), dtype=torch.bfloat16, device="cuda"),
                                torch.empty((0, 10, 1, 128), dtype=torch.bfloat16, device="cuda"), D, 64)
    assert yb.numel() == 0 and sb.numel() == 0


@pytest.mark.parametrize("P,N,Q,L", [(64, 128, 256, 600), (16, 16, 64, 256), (32, 64, 100, 333),
                                     (7, 5, 16, 50)])
def test_f32_path_shapes(P, N, Q, L):
    w = si.small_workload(batch=2, seqlen=L, nheads=4, headdim=P, dstate=N, ngroups=2, chunk=Q,
                          io="f32", seed=P + N + Q)
    full_check(w)


def test_bitwise_deterministic():
    w = si.small_workload(batch=2, seqlen=3000, nheads=8, chunk=256, seed=77)
    inp = si.prefill_inputs(w)
    g, _, _ = gpu_inputs(w, inp)
    y1, s1 = gpu_scan(g, 256)
    y2, s2 = gpu_scan(g, 256)
    assert torch.equal(y1, y2) and torch.equal(s1, s2)


def test_timed_entry_point_matches():
    w = si.small_workload(batch=2, seqlen=3000, nheads=8, chunk=256, seed=78)
    inp = si.prefill_inputs(w)
    g, _, _ = gpu_inputs(w, inp)
    y1, s1 = gpu_scan(g, 256)
    y2, s2, times = ssd.ssd_chunk_scan_timed(g["x"], g["dt"], g["A"], g["B"], g["C"], g["D"], 256)
    assert torch.equal(y1, y2) and torch.equal(s1, s2)
    assert [n for n, _ in times][-1] == "chunk_scan_kernel" and all(ms > 0 for _, ms in times)


def _scan_with_heads(A, dt_scale, seed, L=1100, h0=True):
    """Scan with chosen per-head A (fp32) and dt scaled by dt_scale, against the
    oracle on the same (rounded) values."""
    H = len(A)
    w = si.small_workload(batch=2, seqlen=L, nheads=H, chunk=128, seed=seed)
    inp = si.prefill_inputs(w)
    inp["dt"] = (inp["dt"] * np.float32(dt_scale)).astype(np.float32)
    A = np.asarray(A, dtype=np.float32)
    _, D = si.head_params(w)
    g = dict(x=dev(inp["x"], "bf16"), dt=dev(inp["dt"]), B=dev(inp["B"], "bf16"),
             C=dev(inp["C"], "bf16"), A=dev(A), D=dev(D))
    s0 = (np.random.default_rng(seed).standard_normal((2, H, 64, 128)).astype(np.float32)
          if h0 else None)
    wid = widen_inputs(inp, "bf16")
    for Dv in (D, np.zeros_like(D)):
        y, s = gpu_scan(g, 128, D=dev(Dv), init=None if s0 is None else dev(s0))
        yref, sref = oracle.ssd_scan(wid["x"], wid["dt"], A.astype(np.float64), wid["B"], wid["C"],
                                     Dv.astype(np.float64),
                                     h0=None if s0 is None else s0.astype(np.float64), nthreads=16)
        assert np.isfinite(host(y)).all() and np.isfinite(host(s)).all()
        check_y(host(y), yref, TOL["bf16"])
        if np.abs(sref).max() > 0:
            check_state(host(s), sref, TOL["bf16"])


def test_extreme_decay_memoryless():
    """A = -1e6: every tile's decay underflows, so y_t = dt_t (B_t . C_t) x_t + D x_t
    (the direct-decay path on every tile, and the masked exponents at -inf)."""
    _scan_with_heads([-1e6, -1e6, -5e5, -1e6], 1.0, seed=31)


def test_no_decay():
    """A = 0: the state is a plain prefix sum that grows along the sequence (the
    lazy scale never moves)."""
    _scan_with_heads([0.0, 0.0, 0.0, 0.0], 1.0, seed=32)


def test_decay_mix_renormalisation():
    """Heads from no decay to strong decay with long tiles' worth of tokens, so
    that the lazily applied state scale is renormalised, applied directly, or
    left alone, head by head."""
    _scan_with_heads([0.0, -0.05, -1.0, -16.0, -100.0, -3.0, -0.5, -40.0], 1.0, seed=33, L=2300)
    _scan_with_heads([-16.0, -8.0, -4.0, -1.0], 10.0, seed=34, L=700)

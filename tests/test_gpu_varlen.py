"""GPU parity of ssd_chunk_scan_varlen (packed batches of sequences of
different lengths) against the fp64 oracle, sequence by sequence.

Each sequence of the packed batch is its own recurrence, so the oracle runs on
each sequence's slice of the packed inputs with that sequence's initial state.
"""
import numpy as np
import pytest
import torch

import ssd_inputs as si
import state_space_model_mamba_amd as ssd
from parity import TOL, check_state, check_y, dev, host, oracle_heads

pytestmark = pytest.mark.gpu


def packed(T, H, G, seed, chunk=128):
    w = si.small_workload(batch=1, seqlen=T, nheads=H, ngroups=G, chunk=chunk, seed=seed)
    inp = si.prefill_inputs(w)
    A, D = si.head_params(w)
    return w, {k: v[0] for k, v in inp.items()}, A, D


def run_varlen(inp, A, D, cu, chunk, init=None, **kw):
    y, fs = ssd.ssd_chunk_scan_varlen(dev(inp["x"], "bf16"), dev(inp["dt"]), dev(A),
                                      dev(inp["B"], "bf16"), dev(inp["C"], "bf16"), dev(D), cu,
                                      chunk, initial_states=init, **kw)
    torch.cuda.synchronize()
    return host(y), host(fs)


def check_sequences(inp, A, D, cu, y, fs, init0, heads, what):
    for i in range(len(cu) - 1):
        a, b = cu[i], cu[i + 1]
        if b == a:     # an empty sequence hands its state through
            want = init0[i] if init0 is not None else np.zeros_like(fs[i])
            assert np.array_equal(fs[i], want), f"{what}: empty sequence {i}"
            continue
        seq = {k: v[None, a:b] for k, v in inp.items()}
        h0 = None if init0 is None else init0[i:i + 1]
        pairs = [(0, h) for h in heads]
        yref, sref = oracle_heads(seq, "bf16", A, D, pairs, h0=h0)
        ys = np.stack([y[a:b, h] for h in heads])[:, :, None]
        ss = np.stack([fs[i, h] for h in heads])[:, None]
        check_y(ys, yref[:, :, None], TOL["bf16"], f"{what} y (sequence {i}, {b - a} tokens)")
        check_state(ss, sref[:, None], TOL["bf16"], f"{what} state (sequence {i})")


def run_and_check(inp, A, D, cu, chunk, init0, heads, what):
    """The packed scan with the workload's D and again with D = 0, each against
    the oracle sequence by sequence (D x is about 99% of |y|, so only the D = 0
    run holds the SSM part of y to the tolerance); the states agree bit for bit."""
    init = None if init0 is None else dev(init0)
    y, fs = run_varlen(inp, A, D, cu, chunk, init=init)
    check_sequences(inp, A, D, cu, y, fs, init0, heads, what)
    init = None if init0 is None else dev(init0)
    y0, fs0 = run_varlen(inp, A, np.zeros_like(D), cu, chunk, init=init)
    check_sequences(inp, A, np.zeros_like(D), cu, y0, fs0, init0, heads, what + " (D = 0)")
    assert np.array_equal(fs, fs0)
    return y, fs


@pytest.mark.parametrize("with_init", [False, True])
def test_varlen_mixed_lengths(with_init):
    """Lengths with an empty sequence, a one-token one, a ragged one and a run of
    two equal lengths (one batched call)."""
    lengths = [700, 0, 64, 1300, 1300, 1, 257]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    H, G = 8, 2
    w, inp, A, D = packed(int(cu[-1]), H, G, seed=101)
    init0 = (np.random.default_rng(5).standard_normal((len(lengths), H, 64, 128))
             .astype(np.float32) if with_init else None)
    run_and_check(inp, A, D, cu, 128, init0, [0, 3, 7], "varlen")


def test_varlen_equal_lengths_match_batched():
    """A packed batch of equal lengths is the batched scan: bit-identical."""
    H, G, L, nseq = 8, 1, 1024, 4
    w = si.small_workload(batch=nseq, seqlen=L, nheads=H, ngroups=G, chunk=256, seed=102)
    inp = si.prefill_inputs(w)
    A, D = si.head_params(w)
    y1, s1 = ssd.ssd_chunk_scan(dev(inp["x"], "bf16"), dev(inp["dt"]), dev(A),
                                dev(inp["B"], "bf16"), dev(inp["C"], "bf16"), dev(D), 256)
    flat = {k: v.reshape((nseq * L,) + v.shape[2:]) for k, v in inp.items()}
    y2, s2 = run_varlen(flat, A, D, np.arange(nseq + 1) * L, 256)
    assert np.array_equal(host(y1).reshape(y2.shape), y2)
    assert np.array_equal(host(s1), s2)


def test_varlen_in_place_cache():
    """final_states may be initial_states (each sequence's cache resumed in
    place): the same result as separate buffers."""
    lengths = [300, 129, 129, 0, 900]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    H = 4
    w, inp, A, D = packed(int(cu[-1]), H, 1, seed=103)
    init0 = np.random.default_rng(6).standard_normal((len(lengths), H, 64, 128)).astype(np.float32)
    y1, s1 = run_varlen(inp, A, D, cu, 128, init=dev(init0))
    cache = dev(init0.copy())
    y2, s2 = run_varlen(inp, A, D, cu, 128, init=cache, final_states=cache)
    assert np.array_equal(y1, y2) and np.array_equal(s1, s2)


def test_varlen_2p7b_heads():
    """The 2.7B layer's head shape (80 heads x 64, dstate 128, chunk 256) with a
    continuous-batching mix of prompt lengths; sampled heads of every sequence."""
    lengths = [8192, 2048, 4096, 512, 1536]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    w, inp, A, D = packed(int(cu[-1]), 80, 1, seed=104, chunk=256)
    run_and_check(inp, A, D, cu, 256, None, [0, 41, 79], "varlen 2.7B")


def test_varlen_more_runs_than_one_launch():
    """Ten runs of distinct lengths (two launch groups of at most eight runs),
    from a 1-token sequence to 3000 tokens, with segment counts from the group
    planner; sampled heads of every sequence against the oracle."""
    lengths = [3000, 1, 130, 2500, 640, 1999, 64, 900, 1200, 257]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int64)
    H = 12
    w, inp, A, D = packed(int(cu[-1]), H, 3, seed=105, chunk=128)
    init0 = np.random.default_rng(9).standard_normal((len(lengths), H, 64, 128)).astype(np.float32)
    run_and_check(inp, A, D, cu, 128, init0, [0, 5, 11], "varlen 10 runs")

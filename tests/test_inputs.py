"""The seeded input generator: determinism, sub-range consistency, value ranges and
bf16 rounding (CPU only)."""
import math

import numpy as np
import torch

import ssd_inputs as si


def test_bf16_round_to_nearest_even_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100_000).astype(np.float32),
                        np.array([1.0, -2.5, 3.0e-30, 1.00390625, 1.01171875], np.float32)])
    # ties: 1 + 2^-8 rounds down to 1 (even), 1 + 3*2^-8 rounds up
    bits = si.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    back = si.bf16_bits_to_f32(bits)
    assert np.array_equal(back, torch.from_numpy(a).to(torch.bfloat16).float().numpy())
    assert back[-2] == 1.0 and back[-1] == np.float32(1.015625)


def test_deterministic_and_subrange_consistent():
    w = si.small_workload(batch=2, seqlen=9000, nheads=3, headdim=4, dstate=5, ngroups=1, seed=7)
    full = si.prefill_inputs(w, threads=3)
    again = si.prefill_inputs(w, threads=1)
    for k in full:
        assert np.array_equal(full[k], again[k])
    part = si.prefill_inputs(w, 4000, 8500)
    for k in full:
        assert np.array_equal(part[k], full[k][:, 4000:8500])
    A1, D1 = si.head_params(w)
    A2, D2 = si.head_params(w)
    assert np.array_equal(A1, A2) and np.array_equal(D1, D2)


def test_value_ranges():
    w = si.small_workload(batch=2, seqlen=4096, nheads=16, headdim=8, dstate=128, seed=3)
    inp = si.prefill_inputs(w)
    dt = inp["dt"]
    assert dt.dtype == np.float32 and dt.min() >= 0.001 * (1 - 1e-6) and dt.max() <= 0.1 * (1 + 1e-6)
    A, D = si.head_params(w)
    assert A.dtype == np.float32 and np.all(A <= -1.0 + 1e-6) and np.all(A >= -16.0 - 1e-5)
    B = si.widen(inp["B"], "bf16")
    assert abs(B.std() * math.sqrt(128) - 1.0) < 0.02
    x = si.widen(inp["x"], "bf16")
    assert abs(x.std() - 1.0) < 0.02 and abs(x.mean()) < 0.02


def test_decode_tokens_and_state():
    w = si.WORKLOADS["decode_2p7b"].with_(nheads=4, headdim=8, dstate=16)
    a = si.decode_tokens(w, 3, 0, 6)
    b = si.decode_tokens(w, 3, 2, 5)
    for k in a:
        assert np.array_equal(a[k][2:5], b[k])
    s = si.random_state(w, 3)
    assert s.shape == (3, 4, 8, 16) and s.dtype == np.float32
    assert np.array_equal(s, si.random_state(w, 3))


def test_workload_table_shapes():
    W = si.WORKLOADS
    assert (W["m2_2p7b"].nheads * W["m2_2p7b"].headdim) == 5120
    assert (W["m2_130m"].nheads * W["m2_130m"].headdim) == 1536
    assert W["longctx_2p7b"].nheads // W["longctx_2p7b"].ngroups == 10
    for w in W.values():
        assert w.nheads % w.ngroups == 0

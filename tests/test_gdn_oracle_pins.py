"""Pins of the fp64 Gated DeltaNet decode oracle (CPU only).

"A Persistent-State Dataflow Accelerator for Memory-Bound Linear Attention
Decode on FPGA" (section 2B) gives the update S_t = g S_{t-1} + k dv^T and the
output identity S_t^T q = g S_{t-1}^T q + (q^T k) dv, and prints no worked
example.  The pins are what the delta rule fixes by algebra: a unit key
written with g = beta = 1 reads back its value; orthonormal keys store
independent values; g = 0 forgets, beta = 0 only decays; the classical matrix
form g (I - beta k k^T) S + beta k v^T; the page's output identity; and the
grouping of value heads onto query/key heads.  ``test_gdn_mutants_are_caught``
checks that plausible mistakes fail at least one pin.
"""
import numpy as np
import pytest

from oracle import gdn


def rand_problem(seed, B=2, Hk=2, Hv=4, dk=8, dv=6):
    rng = np.random.default_rng(seed)
    S = rng.standard_normal((B, Hv, dk, dv))
    q = rng.standard_normal((B, Hk, dk))
    k = rng.standard_normal((B, Hk, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, Hv, dv))
    g = rng.uniform(0.5, 1.0, (B, Hv))
    beta = rng.uniform(0.0, 1.0, (B, Hv))
    return S, q, k, v, g, beta


def pin_write_read(f):
    """g = beta = 1 and |k| = 1: the step stores v under k, S_t^T k = v."""
    S, q, k, v, g, beta = rand_problem(1)
    _, S1 = f(S, q, k, v, np.ones_like(g), np.ones_like(beta))
    for b in range(S.shape[0]):
        for j in range(S.shape[1]):
            assert np.allclose(S1[b, j].T @ k[b, j // 2], v[b, j], atol=1e-12)


def pin_orthonormal_memory(f):
    """Two orthonormal keys written in turn from a zero state keep both values."""
    dk, dv = 8, 5
    basis = np.linalg.qr(np.random.default_rng(2).standard_normal((dk, dk)))[0]
    ka, kb = basis[:, 0], basis[:, 3]
    va, vb = np.arange(dv, dtype=float), -np.ones(dv)
    S = np.zeros((1, 1, dk, dv))
    one = np.ones((1, 1))
    q = np.zeros((1, 1, dk))
    _, S = f(S, q, ka[None, None], va[None, None], one, one)
    _, S = f(S, q, kb[None, None], vb[None, None], one, one)
    assert np.allclose(S[0, 0].T @ ka, va, atol=1e-12)
    assert np.allclose(S[0, 0].T @ kb, vb, atol=1e-12)


def pin_forget_and_decay(f):
    """g = 0: S_t = beta k v^T and o = beta (q.k) v.  beta = 0: S_t = g S, o = g S^T q."""
    S, q, k, v, g, beta = rand_problem(3)
    o, S1 = f(S, q, k, v, np.zeros_like(g), beta)
    for b in range(2):
        for j in range(4):
            i = j // 2
            assert np.allclose(S1[b, j], beta[b, j] * np.outer(k[b, i], v[b, j]), atol=1e-13)
            assert np.allclose(o[b, j], beta[b, j] * (q[b, i] @ k[b, i]) * v[b, j], atol=1e-12)
    o, S1 = f(S, q, k, v, g, np.zeros_like(beta))
    for b in range(2):
        for j in range(4):
            assert np.allclose(S1[b, j], g[b, j] * S[b, j], atol=1e-13)
            assert np.allclose(o[b, j], g[b, j] * S[b, j].T @ q[b, j // 2], atol=1e-12)


def pin_matrix_form(f):
    """The delta rule as a matrix: S_t = g (I - beta k k^T) S_{t-1} + beta k v^T."""
    S, q, k, v, g, beta = rand_problem(4)
    o, S1 = f(S, q, k, v, g, beta)
    for b in range(2):
        for j in range(4):
            kk = k[b, j // 2]
            want = g[b, j] * (np.eye(8) - beta[b, j] * np.outer(kk, kk)) @ S[b, j] \
                + beta[b, j] * np.outer(kk, v[b, j])
            assert np.allclose(S1[b, j], want, atol=1e-12)
            assert np.allclose(o[b, j], want.T @ q[b, j // 2], atol=1e-12)


def pin_output_identity(f):
    """The page's identity: o = g S_{t-1}^T q + (q^T k) dv, dv = beta (v - g S_{t-1}^T k)."""
    S, q, k, v, g, beta = rand_problem(5)
    o, _ = f(S, q, k, v, g, beta)
    for b in range(2):
        for j in range(4):
            qq, kk = q[b, j // 2], k[b, j // 2]
            dv = beta[b, j] * (v[b, j] - g[b, j] * S[b, j].T @ kk)
            assert np.allclose(o[b, j], g[b, j] * S[b, j].T @ qq + (qq @ kk) * dv, atol=1e-12)


def pin_head_groups(f):
    """Value head j reads query/key head j // (Hv / Hk): with the query/key heads
    replicated per value head the result is the same."""
    S, q, k, v, g, beta = rand_problem(6)
    o1, S1 = f(S, q, k, v, g, beta)
    o2, S2 = f(S, np.repeat(q, 2, axis=1), np.repeat(k, 2, axis=1), v, g, beta)
    assert np.allclose(o1, o2, atol=1e-14) and np.allclose(S1, S2, atol=1e-14)


PINS = [pin_write_read, pin_orthonormal_memory, pin_forget_and_decay, pin_matrix_form,
        pin_output_identity, pin_head_groups]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_gdn_pin(pin):
    pin(gdn.gdn_decode_step)


def test_gdn_steps_is_steps_in_order():
    rng = np.random.default_rng(7)
    T, (S, *_) = 5, rand_problem(8)
    q = rng.standard_normal((T, 2, 2, 8))
    k = rng.standard_normal((T, 2, 2, 8))
    v = rng.standard_normal((T, 2, 4, 6))
    g = rng.uniform(0.5, 1, (T, 2, 4))
    beta = rng.uniform(0, 1, (T, 2, 4))
    o, Sn = gdn.gdn_decode_steps(S, q, k, v, g, beta)
    s = S
    for t in range(T):
        ot, s = gdn.gdn_decode_step(s, q[t], k[t], v[t], g[t], beta[t])
        assert np.array_equal(o[t], ot)
    assert np.array_equal(Sn, s)


def _mutant(kind):
    def f(S, q, k, v, g, beta):
        S = np.array(S, dtype=np.float64)
        B, Hv, dk, dv = S.shape
        Hk = q.shape[1]
        o = np.empty((B, Hv, dv))
        for b in range(B):
            for j in range(Hv):
                i = j // (Hv // Hk)
                s = S[b, j]
                r = s.T @ k[b, i]
                if kind == "no_gate_in_delta":
                    delta = beta[b, j] * (v[b, j] - r)
                else:
                    delta = beta[b, j] * (v[b, j] - g[b, j] * r)
                s = g[b, j] * s + np.outer(k[b, i], delta)
                S[b, j] = s
                if kind == "output_from_old_state":
                    o[b, j] = S[b, j].T @ q[b, i] - np.outer(k[b, i], delta).T @ q[b, i]
                elif kind == "head_group_modulo":
                    o[b, j] = s.T @ q[b, j % Hk]
                else:
                    o[b, j] = s.T @ q[b, i]
        return o, S
    return f


@pytest.mark.parametrize("kind", ["no_gate_in_delta", "output_from_old_state", "head_group_modulo"])
def test_gdn_mutants_are_caught(kind):
    caught = 0
    for pin in PINS:
        try:
            pin(_mutant(kind))
        except AssertionError:
            caught += 1
    assert caught >= 1, f"mutant {kind} passed every pin"

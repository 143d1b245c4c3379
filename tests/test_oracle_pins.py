"""Pins of the fp64 oracle against what mathematics fixes (CPU only).

The pages ("Compiler-First State Space Duality and Portable O(1)
Autoregressive Caching for Inference", sections 2-4) print no worked numeric
SSD example, so every pin here is mathematical: a brute-force quadratic
(semiseparable matrix) form, closed forms (A = 0 prefix sums, a geometric
series, the memoryless and pure-decay limits), linear-algebra invariants, a
separately written chunked form (the decomposition the GPU kernels use) with
several chunk lengths, split continuity of the state cache (section 2, the O(1)
cache) and the one-pass decode identity.  ``test_mutants_are_caught`` plants
plausible mistakes in copies of the oracle and checks each one fails a pin.
"""
import math
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle


# ----------------------------------------------------------------------------
# small random problems with the workloads' value distributions
# ----------------------------------------------------------------------------
def problem(seed, bsz=2, L=17, H=4, P=3, N=5, G=2, h0=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((bsz, L, H, P))
    B = rng.standard_normal((bsz, L, G, N)) / math.sqrt(N)
    C = rng.standard_normal((bsz, L, G, N)) / math.sqrt(N)
    u = rng.uniform(math.log(math.expm1(0.001)), math.log(math.expm1(0.1)), (bsz, L, H))
    dt = np.log1p(np.exp(u))
    A = -np.exp(rng.uniform(0, math.log(16), H))
    D = rng.standard_normal(H)
    s0 = rng.standard_normal((bsz, H, P, N)) if h0 else None
    return dict(x=x, dt=dt, A=A, B=B, C=C, D=D, h0=s0)


def run(p, lib=None, **kw):
    q = dict(p)
    q.update(kw)
    return oracle.ssd_scan(q["x"], q["dt"], q["A"], q["B"], q["C"], q["D"], h0=q["h0"], lib=lib)


def rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    d = np.linalg.norm((a - b).ravel())
    n = np.linalg.norm(b.ravel())
    return d / n if n > 0 else d


# ----------------------------------------------------------------------------
# independent forms
# ----------------------------------------------------------------------------
def brute_force(x, dt, A, B, C, D, h0=None):
    """Materialised semiseparable form, decay sums taken term by term.

    y[t] = sum_{s<=t} (C_t . B_s) * exp(sum_{r=s+1..t} dt_r A) * dt_s * x_s
           + D x_t + exp(sum_{r=1..t} dt_r A) * (H0 C_t)
    H_L  = exp(sum_{r=1..L} dt_r A) H0 + sum_s exp(sum_{r=s+1..L} dt_r A) dt_s x_s B_s^T
    """
    bsz, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    y = np.zeros_like(x)
    hL = np.zeros((bsz, H, P, N))
    for b in range(bsz):
        for h in range(H):
            g = h // (H // G)
            a = dt[b, :, h] * A[h]

            def decay(s, t):          # exp(sum_{r=s+1..t} a_r), tokens are 0-based
                tot = 0.0
                for r in range(s + 1, t + 1):
                    tot += a[r]
                return math.exp(tot)

            M = np.zeros((L, L))
            for t in range(L):
                for s in range(t + 1):
                    M[t, s] = float(C[b, t, g] @ B[b, s, g]) * decay(s, t) * dt[b, s, h]
            y[b, :, h] = M @ x[b, :, h] + D[h] * x[b, :, h]
            S = np.zeros((P, N))
            for s in range(L):
                S += decay(s, L - 1) * dt[b, s, h] * np.outer(x[b, s, h], B[b, s, g])
            if h0 is not None:
                for t in range(L):
                    y[b, t, h] += decay(-1, t) * (h0[b, h] @ C[b, t, g])
                S += decay(-1, L - 1) * h0[b, h]
            hL[b, h] = S
    return y, hL


def chunked_form(x, dt, A, B, C, D, h0, Q):
    """The chunked SSD decomposition (intra-chunk quadratic block + chunk state
    + state passing + state-to-output), chunk length Q, last chunk may be short."""
    bsz, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    y = np.zeros_like(x)
    hL = np.zeros((bsz, H, P, N))
    for b in range(bsz):
        for h in range(H):
            g = h // (H // G)
            S = np.zeros((P, N)) if h0 is None else h0[b, h].copy()
            for c0 in range(0, L, Q):
                c1 = min(c0 + Q, L)
                a = dt[b, c0:c1, h] * A[h]
                lam = np.cumsum(a)
                seg = lam[:, None] - lam[None, :]
                Lmat = np.where(np.tril(np.ones((c1 - c0, c1 - c0), bool)), np.exp(np.minimum(seg, 0)), 0.0)
                Cc, Bc, xc, dtc = C[b, c0:c1, g], B[b, c0:c1, g], x[b, c0:c1, h], dt[b, c0:c1, h]
                y_diag = ((Cc @ Bc.T) * Lmat * dtc[None, :]) @ xc
                y_off = np.exp(lam)[:, None] * (Cc @ S.T)
                y[b, c0:c1, h] = y_diag + y_off + D[h] * xc
                w = np.exp(lam[-1] - lam) * dtc
                S = math.exp(lam[-1]) * S + (xc * w[:, None]).T @ Bc
            hL[b, h] = S
    return y, hL


# ----------------------------------------------------------------------------
# pins: each takes the oracle library (so mutants can be run through them)
# ----------------------------------------------------------------------------
def pin_bruteforce(lib=None):
    for seed, shape in [(1, dict(bsz=2, L=13, H=4, P=3, N=5, G=2)),
                        (2, dict(bsz=1, L=24, H=3, P=4, N=2, G=1)),
                        (3, dict(bsz=1, L=9, H=2, P=2, N=3, G=2, h0=False))]:
        p = problem(seed, **shape)
        y, hL = run(p, lib)
        yb, hb = brute_force(**p)
        assert rel(y, yb) < 1e-12 and rel(hL, hb) < 1e-12, (seed, rel(y, yb), rel(hL, hb))


def pin_a_zero_prefix_sums(lib=None):
    p = problem(4, bsz=2, L=20, H=2, P=3, N=4, G=1)
    p["A"] = np.zeros_like(p["A"])
    y, hL = run(p, lib)
    x, dt, B, C, D, h0 = p["x"], p["dt"], p["B"], p["C"], p["D"], p["h0"]
    # H_t = H0 + cumulative sum of dt_s x_s B_s^T
    inc = np.einsum("blh,blhp,bln->blhpn", dt, x, B[:, :, 0])
    Ht = h0[:, None] + np.cumsum(inc, axis=1)
    yref = np.einsum("blhpn,bln->blhp", Ht, C[:, :, 0]) + D[None, None, :, None] * x
    assert rel(y, yref) < 1e-12 and rel(hL, Ht[:, -1]) < 1e-12


def pin_memoryless(lib=None):
    # dt >= 0.001, A = -1e6: exp(dt A) <= exp(-1000) == 0.0 in fp64
    p = problem(5, bsz=1, L=10, H=2, P=3, N=4, G=1)
    p["A"] = np.full_like(p["A"], -1e6)
    y, hL = run(p, lib)
    x, dt, B, C, D = p["x"], p["dt"], p["B"], p["C"], p["D"]
    bc = np.einsum("bln,bln->bl", B[:, :, 0], C[:, :, 0])
    yref = dt[..., None] * bc[:, :, None, None] * x + D[None, None, :, None] * x
    href = dt[:, -1, :, None, None] * x[:, -1, :, :, None] * B[:, -1, 0][:, None, None, :]
    assert rel(y, yref) < 1e-13 and rel(hL, href) < 1e-13


def pin_pure_decay(lib=None):
    p = problem(6, bsz=2, L=15, H=3, P=2, N=3, G=3)
    p["x"] = np.zeros_like(p["x"])
    y, hL = run(p, lib)
    a = p["dt"] * p["A"][None, None, :]
    cum = np.cumsum(a, axis=1)                              # sum_{r<=t} a_r
    g = np.arange(3)                                        # G == H here
    yref = np.exp(cum)[..., None] * np.einsum("bhpn,blhn->blhp", p["h0"], p["C"][:, :, g])
    href = np.exp(cum[:, -1])[..., None, None] * p["h0"]
    assert rel(y, yref) < 1e-12 and rel(hL, href) < 1e-12


def pin_single_step(lib=None):
    p = problem(7, bsz=2, L=1, H=2, P=3, N=2, G=1)
    y, hL = run(p, lib)
    al = np.exp(p["dt"][:, 0] * p["A"])                     # [b, H]
    href = al[..., None, None] * p["h0"] + \
        (p["dt"][:, 0, :, None] * p["x"][:, 0])[..., None] * p["B"][:, 0, 0][:, None, None, :]
    yref = np.einsum("bhpn,bn->bhp", href, p["C"][:, 0, 0]) + p["D"][None, :, None] * p["x"][:, 0]
    assert rel(hL, href) < 1e-14 and rel(y[:, 0], yref) < 1e-14


def pin_geometric_series(lib=None):
    # P = N = 1, dt = 1, A = -ln 2 (alpha = 1/2), x_t = t (1-based), B = C = 1:
    # H_t = sum_{s<=t} 2^{-(t-s)} s = 2t - 2 + 2^{1-t};  y_t = H_t + D t.
    L, D = 12, 0.75
    t = np.arange(1, L + 1, dtype=np.float64)
    x = t.reshape(1, L, 1, 1)
    ones = np.ones((1, L, 1, 1))
    y, hL = oracle.ssd_scan(x, np.ones((1, L, 1)), np.array([-math.log(2.0)]), ones, ones,
                            np.array([D]), lib=lib)
    Ht = 2 * t - 2 + 2.0 ** (1 - t)
    assert np.max(np.abs(y[0, :, 0, 0] - (Ht + D * t))) < 1e-13
    assert abs(hL[0, 0, 0, 0] - Ht[-1]) < 1e-13


def pin_superposition(lib=None):
    p = problem(8, bsz=2, L=16, H=2, P=3, N=4, G=1)
    y, hL = run(p, lib)
    y1, h1 = run(p, lib, h0=None)
    y2, h2 = run(p, lib, x=np.zeros_like(p["x"]), D=np.zeros_like(p["D"]))
    assert rel(y1 + y2, y) < 1e-13 and rel(h1 + h2, hL) < 1e-13


def pin_bc_rescaling(lib=None):
    p = problem(9, bsz=1, L=14, H=2, P=2, N=3, G=1, h0=False)
    y, hL = run(p, lib)
    k = 3.0
    y2, h2 = run(p, lib, B=p["B"] * k, C=p["C"] / k)
    assert rel(y2, y) < 1e-13 and rel(h2, hL * k) < 1e-13


def pin_permutations(lib=None):
    p = problem(10, bsz=3, L=11, H=4, P=2, N=3, G=1)
    y, hL = run(p, lib)
    pb = np.array([2, 0, 1])
    q = {k: (v[pb] if k in ("x", "dt", "B", "C", "h0") else v) for k, v in p.items()}
    yq, hq = run(q, lib)
    assert rel(yq, y[pb]) < 1e-15 and rel(hq, hL[pb]) < 1e-15
    ph = np.array([3, 1, 0, 2])                            # G == 1: any head order
    q = dict(p, x=p["x"][:, :, ph], dt=p["dt"][:, :, ph], A=p["A"][ph], D=p["D"][ph],
             h0=p["h0"][:, ph])
    yq, hq = run(q, lib)
    assert rel(yq, y[:, :, ph]) < 1e-15 and rel(hq, hL[:, ph]) < 1e-15


def pin_group_replication(lib=None):
    p = problem(11, bsz=2, L=12, H=6, P=2, N=3, G=2)
    y, hL = run(p, lib)
    rep = np.repeat(np.arange(2), 3)                        # heads 0-2 -> group 0, 3-5 -> 1
    yr, hr = run(p, lib, B=p["B"][:, :, rep], C=p["C"][:, :, rep])
    assert rel(yr, y) < 1e-15 and rel(hr, hL) < 1e-15


def pin_chunked_invariance(lib=None):
    p = problem(12, bsz=2, L=23, H=2, P=3, N=4, G=1)
    y, hL = run(p, lib)
    for Q in (1, 2, 4, 5, 8, 16, 23, 64):
        yc, hc = chunked_form(Q=Q, **p)
        assert rel(yc, y) < 1e-12 and rel(hc, hL) < 1e-12, Q


def pin_split_continuity(lib=None):
    p = problem(13, bsz=1, L=18, H=2, P=2, N=3, G=1)
    y, hL = run(p, lib)
    for k in range(0, 19):
        ya, ha = run({**p, "x": p["x"][:, :k], "dt": p["dt"][:, :k], "B": p["B"][:, :k],
                      "C": p["C"][:, :k]}, lib)
        yb, hb = run({**p, "x": p["x"][:, k:], "dt": p["dt"][:, k:], "B": p["B"][:, k:],
                      "C": p["C"][:, k:], "h0": ha}, lib)
        assert rel(np.concatenate([ya, yb], axis=1), y) < 1e-13 and rel(hb, hL) < 1e-13, k


def pin_decode_identity(lib=None):
    # H_t C_t = alpha_t (H_{t-1} C_t) + dt_t (B_t . C_t) x_t : the output can be formed
    # from the *old* state and the new token, in the same pass that updates the state.
    p = problem(14, bsz=2, L=1, H=3, P=4, N=5, G=1)
    yd, s1 = oracle.ssd_decode_step(p["h0"], p["x"][:, 0], p["dt"][:, 0], p["A"], p["B"][:, 0],
                                    p["C"][:, 0], p["D"], lib=lib)
    al = np.exp(p["dt"][:, 0] * p["A"])
    old = np.einsum("bhpn,bn->bhp", p["h0"], p["C"][:, 0, 0])
    bc = np.einsum("bn,bn->b", p["B"][:, 0, 0], p["C"][:, 0, 0])
    yref = al[..., None] * old + p["dt"][:, 0, :, None] * bc[:, None, None] * p["x"][:, 0] + \
        p["D"][None, :, None] * p["x"][:, 0]
    assert rel(yd, yref) < 1e-14
    # and y computed from the updated state agrees
    assert rel(np.einsum("bhpn,bn->bhp", s1, p["C"][:, 0, 0]) + p["D"][None, :, None] * p["x"][:, 0], yd) < 1e-14


PINS = [pin_bruteforce, pin_a_zero_prefix_sums, pin_memoryless, pin_pure_decay, pin_single_step,
        pin_geometric_series, pin_superposition, pin_bc_rescaling, pin_permutations,
        pin_group_replication, pin_chunked_invariance, pin_split_continuity, pin_decode_identity]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_empty_and_thread_invariance():
    p = problem(15, bsz=2, L=0, H=2, P=2, N=3, G=1)
    y, hL = run(p)
    assert y.shape == (2, 0, 2, 2) and np.array_equal(hL, p["h0"])
    p = problem(16, bsz=3, L=40, H=5, P=4, N=6, G=1)
    y1, h1 = oracle.ssd_scan(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["h0"], nthreads=1)
    y4, h4 = oracle.ssd_scan(p["x"], p["dt"], p["A"], p["B"], p["C"], p["D"], p["h0"], nthreads=4)
    assert np.array_equal(y1, y4) and np.array_equal(h1, h4)


def test_rejects_bad_groups():
    p = problem(17, bsz=1, L=3, H=3, P=2, N=2, G=2)
    with pytest.raises(ValueError):
        run(p)


@settings(max_examples=60, deadline=None)
@given(seed=st.integers(0, 10_000), bsz=st.integers(1, 2), L=st.integers(1, 12),
       hg=st.sampled_from([(1, 1), (2, 1), (2, 2), (4, 2), (3, 3)]), P=st.integers(1, 4),
       N=st.integers(1, 4), h0=st.booleans())
def test_fuzz_against_bruteforce(seed, bsz, L, hg, P, N, h0):
    H, G = hg
    p = problem(seed, bsz=bsz, L=L, H=H, P=P, N=N, G=G, h0=h0)
    y, hL = run(p)
    yb, hb = brute_force(**p)
    assert rel(y, yb) < 1e-12 and rel(hL, hb) < 1e-12


# ----------------------------------------------------------------------------
# planted mistakes: every mutant of the oracle must fail at least one pin
# ----------------------------------------------------------------------------
MUTANTS = {
    "drop_skip_term": ("yt[p] = acc + D * xt[p];", "yt[p] = acc;"),
    "output_before_update": ("row[n] = alpha * row[n] + u * Bt[n];\n                acc += row[n] * Ct[n];",
                             "acc += row[n] * Ct[n];\n                row[n] = alpha * row[n] + u * Bt[n];"),
    "decay_sign": ("exp(dt * A)", "exp(-dt * A)"),
    "b_c_swapped": ("const double *Bt = j->B", "const double *Bt = j->C"),
    "group_index": ("h / (H / j->ngroups)", "h % j->ngroups"),
    "decay_on_input": ("row[n] = alpha * row[n] + u * Bt[n];", "row[n] = alpha * (row[n] + u * Bt[n]);"),
    "no_dt_on_input": ("const double u = dt * xt[p];", "const double u = xt[p];"),
    "transposed_state_read": ("acc += row[n] * Ct[n];", "acc += S[n * P + p] * Ct[n];"),
    "dt_head_index": ("j->dt[(b * L + t) * H + h]", "j->dt[(b * L + t) * H]"),
    "initial_state_ignored": ("if (j->h0)", "if (0)"),
    "skip_uses_wrong_head": ("const double A = j->A[h], D = j->D[h];", "const double A = j->A[h], D = j->D[0];"),
}


def _build_variant(tmp, name, old=None, new=None):
    src = open(oracle.SOURCE).read()
    if old is not None:
        assert src.count(old) == 1, f"mutation site for {name} not unique"
        src = src.replace(old, new)
    cpath = os.path.join(tmp, f"{name}.c")
    with open(cpath, "w") as f:
        f.write(src)
    return oracle.load(oracle.build(cpath, os.path.join(tmp, f"lib{name}.so")))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_mutants_are_caught():
    with tempfile.TemporaryDirectory() as tmp:
        clean = _build_variant(tmp, "clean")
        for pin in PINS:
            pin(clean)
        survivors = []
        for name, (old, new) in MUTANTS.items():
            lib = _build_variant(tmp, name, old, new)
            caught = []
            for pin in PINS:
                try:
                    pin(lib)
                except AssertionError:
                    caught.append(pin.__name__)
            if not caught:
                survivors.append(name)
        assert not survivors, f"mutants not caught by any pin: {survivors}"


# ----------------------------------------------------------------------------
# the fused step-size prep: softplus
# ----------------------------------------------------------------------------
def test_dt_softplus_pins():
    """softplus(0) = ln 2; softplus(v) - softplus(-v) = v; its large- and
    small-argument limits v and exp(v); the bias is added per head (last axis)."""
    assert abs(oracle.dt_softplus(0.0) - math.log(2.0)) < 1e-15
    rng = np.random.default_rng(5)
    v = rng.uniform(-30, 30, 1000)
    assert np.max(np.abs(oracle.dt_softplus(v) - oracle.dt_softplus(-v) - v)) < 1e-12
    big = np.array([40.0, 100.0, 700.0, 1e5])
    assert np.array_equal(oracle.dt_softplus(big), big)
    small = np.array([-40.0, -100.0, -700.0])
    assert np.allclose(oracle.dt_softplus(small), np.exp(small), rtol=1e-12, atol=0)
    # at the workload's range the value is the step size the draw produces
    for d in (0.001, 0.01, 0.1):
        assert abs(oracle.dt_softplus(math.log(math.expm1(d))) - d) < 1e-15
    u = rng.standard_normal((3, 5, 4))
    bias = np.array([0.5, -1.0, 2.0, 0.0])
    assert np.array_equal(oracle.dt_softplus(u, bias), oracle.dt_softplus(u + bias))
    assert np.all(oracle.dt_softplus(u, bias) > 0)

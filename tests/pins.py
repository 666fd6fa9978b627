"""Pins for the CPU oracle: checks that tie it to facts outside itself.

Each ``check_*`` takes an implementation and raises AssertionError when the
implementation disagrees with a closed form, a hand-worked example, a library
routine or an invariant of causal linear attention.  The tests run them on the
oracle (must pass) and on deliberately wrong variants (must fail), so every pin
is shown to catch at least one plausible mistake.

Implementation signatures:
    fwd(q, k, v) -> o                    q, k, v: [n, d] float arrays
    blk(q, k, v, B) -> o                 block form with block size B
    dec(q, k, v, S0) -> (o, S_final)     q, k, v: [steps, units, d], S0 [units, d, d]
    varlen(q, k, v, cu) -> o             q, k, v: [heads, T, d]
    stf(q, k, v, S0) -> (o, S_final)     one [n, d] unit continued from S0 [d, d]
    rope(x, positions, rope_dims, base)  x [n, d] rotated at integer positions [n]
    ratt(q, k, v, p0, S0) -> (o, S_final)  one [n, d] unit, q and k rotated at
                                         positions p0 + t (rope_dims, base bound)
"""
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _arr(x):
    return np.asarray(x, dtype=np.float32)


def check_golden_causal(fwd):
    g = load_golden("hand_causal_d2_n3.json")
    o = fwd(_arr(g["q"]), _arr(g["k"]), _arr(g["v"]))
    assert np.array_equal(np.asarray(o, np.float64), np.asarray(g["o"], np.float64)), o


def check_golden_ones(fwd):
    g = load_golden("hand_ones_d4_n5.json")
    o = fwd(_arr(g["q"]), _arr(g["k"]), _arr(g["v"]))
    assert np.array_equal(np.asarray(o, np.float64), np.asarray(g["o"], np.float64)), o


def check_golden_block(blk):
    g = load_golden("hand_block_d1_n4.json")
    o = blk(_arr(g["q"]), _arr(g["k"]), _arr(g["v"]), g["block_size"])
    assert np.array_equal(np.asarray(o, np.float64), np.asarray(g["o"], np.float64)), o


def check_golden_decode(dec):
    g = load_golden("hand_causal_d2_n3.json")
    q = _arr(g["q"])[:, None, :]
    k = _arr(g["k"])[:, None, :]
    v = _arr(g["v"])[:, None, :]
    states = []
    S = np.zeros((1, 2, 2))
    outs = []
    for t in range(3):
        o, S = dec(q[t:t + 1], k[t:t + 1], v[t:t + 1], S)
        outs.append(np.asarray(o)[0, 0])
        states.append(np.asarray(S)[0])
    assert np.array_equal(np.array(outs), np.asarray(g["decode_o"], np.float64)), outs
    assert np.array_equal(np.array(states), np.asarray(g["decode_states"], np.float64)), states


def check_all_ones(fwd, n=37, d=8):
    """Closed form: all-ones inputs give o_i = d (i + 1) in every component."""
    one = np.ones((n, d), np.float32)
    o = np.asarray(fwd(one, one, one))
    expect = (d * (np.arange(n) + 1.0))[:, None] * np.ones((1, d))
    assert np.array_equal(o, expect)


def check_one_hot(fwd, n=70, d=6, j0s=(0, 15, 16, 31, 63, 64, 69), a=2, c=4):
    """Closed form: k_{j0} = e_a, v_{j0} = e_c, all other k, v zero, every q_i = e_a:
    o_i = [i >= j0] e_c."""
    for j0 in j0s:
        q = np.zeros((n, d), np.float32)
        q[:, a] = 1
        k = np.zeros((n, d), np.float32)
        v = np.zeros((n, d), np.float32)
        k[j0, a] = 1
        v[j0, c] = 1
        o = np.asarray(fwd(q, k, v))
        expect = np.zeros((n, d))
        expect[j0:, c] = 1
        assert np.array_equal(o, expect), j0


def check_prefix_sum(fwd, n=300, d=4, seed=7):
    """q_i = k_j = e_0 and v_j = x_j e_0 turn o_i[0] into the inclusive cumulative
    sum of x (compared with numpy.cumsum on small integers, so exactly)."""
    rng = np.random.default_rng(seed)
    x = rng.integers(-5, 6, size=n).astype(np.float32)
    q = np.zeros((n, d), np.float32)
    q[:, 0] = 1
    k = q.copy()
    v = np.zeros((n, d), np.float32)
    v[:, 0] = x
    o = np.asarray(fwd(q, k, v))
    assert np.array_equal(o[:, 0], np.cumsum(x.astype(np.float64)))
    assert np.all(o[:, 1:] == 0)


def check_vs_numpy_masked(fwd, n=50, d=7, seed=3, tol=1e-12):
    """Textbook matrix form tril(Q K^T) V (numpy) on random inputs."""
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((n, d)).astype(np.float32) for _ in range(3))
    ref = np.tril(q.astype(np.float64) @ k.astype(np.float64).T) @ v.astype(np.float64)
    o = np.asarray(fwd(q, k, v))
    assert np.max(np.abs(o - ref)) <= tol * np.max(np.abs(ref))


def check_block_invariance(blk, fwd, n=133, d=5, Bs=(1, 2, 7, 16, 64, 133, 500), seed=11,
                           tol=1e-12):
    """The intra/inter split computes the same result for every block size."""
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((n, d)).astype(np.float32) for _ in range(3))
    ref = np.asarray(fwd(q, k, v))
    for B in Bs:
        o = np.asarray(blk(q, k, v, B))
        assert np.max(np.abs(o - ref)) <= tol * np.max(np.abs(ref)), B


def check_integer_exact(fwd, ref_fn, n=40, d=6, seed=5):
    """Small-integer inputs: every partial sum is an exact integer in double, so
    the implementation must agree bit for bit with an exact reference."""
    rng = np.random.default_rng(seed)
    q, k, v = (rng.integers(-2, 3, size=(n, d)).astype(np.float32) for _ in range(3))
    o = np.asarray(fwd(q, k, v), np.float64)
    ref = np.asarray(ref_fn(q, k, v), np.float64)
    assert np.array_equal(o, ref)


def check_varlen_resets(varlen, fwd, lengths=(5, 0, 17, 1, 64, 33), heads=3, d=4, seed=9):
    """Each packed sequence starts from an empty state: the packed result equals
    running every sequence alone."""
    rng = np.random.default_rng(seed)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    q, k, v = (rng.standard_normal((heads, T, d)).astype(np.float32) for _ in range(3))
    o = np.asarray(varlen(q, k, v, cu))
    for h in range(heads):
        for s in range(len(lengths)):
            a, b = cu[s], cu[s + 1]
            if b > a:
                ref = np.asarray(fwd(q[h, a:b], k[h, a:b], v[h, a:b]))
                assert np.allclose(o[h, a:b], ref, rtol=0, atol=1e-12 * max(1.0, np.abs(ref).max())), (h, s)


def check_decode_state_sum(dec, steps=20, units=3, d=5, seed=13):
    """S_T = S_0 + sum_t k_t^T v_t, i.e. S_0 + K^T V as one matrix product."""
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((steps, units, d)).astype(np.float32) for _ in range(3))
    S0 = rng.standard_normal((units, d, d))
    _, S = dec(q, k, v, S0)
    for u in range(units):
        K = k[:, u, :].astype(np.float64)
        V = v[:, u, :].astype(np.float64)
        assert np.allclose(S[u], S0[u] + K.T @ V, rtol=0, atol=1e-12 * np.abs(S0[u] + K.T @ V).max())


def check_decode_vs_prefill(dec, fwd, steps=25, d=6, seed=17):
    """From an empty state the decode output (state before the token) plus the
    token's own term (q.k) v equals the causal (j <= i) prefill output."""
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((steps, 1, d)).astype(np.float32) for _ in range(3))
    o_dec, _ = dec(q, k, v, np.zeros((1, d, d)))
    o_pre = np.asarray(fwd(q[:, 0], k[:, 0], v[:, 0]))
    own = np.sum(q[:, 0].astype(np.float64) * k[:, 0], axis=1)[:, None] * v[:, 0]
    lhs = np.asarray(o_dec)[:, 0] + own
    assert np.max(np.abs(lhs - o_pre)) <= 1e-12 * np.abs(o_pre).max()


def check_linearity(fwd, n=30, d=5, seed=19):
    """o is linear in q and in v: o(2q) = 2 o(q); o(v1 + v2) = o(v1) + o(v2)."""
    rng = np.random.default_rng(seed)
    q, k, v1, v2 = (rng.integers(-3, 4, size=(n, d)).astype(np.float32) for _ in range(4))
    o = np.asarray(fwd(q, k, v1))
    assert np.array_equal(np.asarray(fwd(2 * q, k, v1)), 2 * o)
    assert np.array_equal(np.asarray(fwd(q, k, v1 + v2)), o + np.asarray(fwd(q, k, v2)))


# ---- state handoff: a unit continued from an initial state S0 -------------

def check_golden_state(stf):
    """Hand-worked continuation from a non-symmetric S0 (tests/golden)."""
    g = load_golden("hand_state_d2_n2.json")
    o, Sf = stf(_arr(g["q"]), _arr(g["k"]), _arr(g["v"]), np.asarray(g["S0"], np.float64))
    assert np.array_equal(np.asarray(o), np.asarray(g["o"], np.float64))
    assert np.array_equal(np.asarray(Sf), np.asarray(g["S_final"], np.float64))


def check_state_closed_form(stf, n=45, d=6, seed=31, tol=1e-12):
    """Library routine: o = tril(Q K^T) V + Q S0 and S_final = S0 + K^T V."""
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((n, d)).astype(np.float32) for _ in range(3))
    S0 = rng.standard_normal((d, d))
    o, Sf = stf(q, k, v, S0)
    q64, k64, v64 = (x.astype(np.float64) for x in (q, k, v))
    ref = np.tril(q64 @ k64.T) @ v64 + q64 @ S0
    assert np.allclose(o, ref, rtol=0, atol=tol * np.abs(ref).max())
    sref = S0 + k64.T @ v64
    assert np.allclose(Sf, sref, rtol=0, atol=tol * np.abs(sref).max())


def check_state_resume(stf, n=70, d=5, cuts=(1, 16, 33, 69), seed=37, tol=1e-12):
    """Invariant: a unit run in two pieces, the second continued from the
    first's final state, equals the run in one piece."""
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((n, d)).astype(np.float32) for _ in range(3))
    S0 = rng.standard_normal((d, d))
    o, Sf = stf(q, k, v, S0)
    for m in cuts:
        o1, S1 = stf(q[:m], k[:m], v[:m], S0)
        o2, S2 = stf(q[m:], k[m:], v[m:], S1)
        oo = np.concatenate([np.asarray(o1), np.asarray(o2)])
        assert np.allclose(oo, o, rtol=0, atol=tol * np.abs(o).max())
        assert np.allclose(S2, Sf, rtol=0, atol=tol * np.abs(Sf).max())


def check_state_exact(stf, n=9, d=3, seed=41):
    """Small integers: exact rational o_t = q_t (S0 + sum_{j<=t} k_j^T v_j)."""
    from fractions import Fraction
    rng = np.random.default_rng(seed)
    q, k, v = (rng.integers(-3, 4, size=(n, d)).astype(np.float32) for _ in range(3))
    S0 = rng.integers(-5, 6, size=(d, d)).astype(np.float64)
    S = [[Fraction(int(S0[a, b])) for b in range(d)] for a in range(d)]
    exp = []
    for t in range(n):
        for a in range(d):
            for b in range(d):
                S[a][b] += Fraction(int(k[t, a])) * Fraction(int(v[t, b]))
        exp.append([float(sum(Fraction(int(q[t, a])) * S[a][b] for a in range(d))) for b in range(d)])
    o, Sf = stf(q, k, v, S0)
    assert np.array_equal(np.asarray(o), np.asarray(exp, np.float64))
    assert np.array_equal(np.asarray(Sf), np.asarray([[float(x) for x in row] for row in S]))


# ---- rotary position embedding (rope_dims of d rotated, split-half pairs) --

def check_golden_rope(rope):
    """Hand-worked rotation at positions 1 and 2 (tests/golden)."""
    g = load_golden("hand_rope_d6_r4.json")
    x = np.asarray([g["x"], g["x"]], np.float64)
    y = np.asarray(rope(x, np.asarray(g["positions"]), g["rope_dims"], g["base"]))
    assert np.allclose(y, np.asarray(g["y"]), rtol=0, atol=1e-15)


def check_rope_complex(rope, n=40, d=12, r=8, base=10000.0, seed=51, tol=1e-13):
    """Library routine: pair i read as the complex number x_i + 1j x_{i+r/2}
    is multiplied by exp(1j p w_i); dims from r on are unchanged."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d))
    pos = rng.integers(0, 1 << 20, size=n)
    y = np.asarray(rope(x, pos, r, base))
    h = r // 2
    w = np.power(float(base), -np.arange(h) * 2.0 / r)
    z = (x[:, :h] + 1j * x[:, h:r]) * np.exp(1j * (pos[:, None] * w))
    assert np.allclose(y[:, :h], z.real, rtol=0, atol=tol * 4)
    assert np.allclose(y[:, h:r], z.imag, rtol=0, atol=tol * 4)
    assert np.array_equal(y[:, r:], x[:, r:])


def check_rope_frequencies(rope, r=64, base=10000.0):
    """Closed form: a unit vector e_i at position 1 turns by w_i, with
    w_0 = 1, w_{r/4} = 1/sqrt(base), w_{r/2-1} = base^(-(r-2)/r) and a
    constant ratio w_{i+1} / w_i = base^(-2/r)."""
    h = r // 2
    x = np.eye(r)[:h]
    y = np.asarray(rope(x, np.ones(h, np.int64), r, base))
    w = np.array([np.arctan2(y[i, i + h], y[i, i]) for i in range(h)])
    assert abs(w[0] - 1.0) < 1e-15
    assert abs(w[h // 2] - 1.0 / np.sqrt(base)) < 1e-15
    assert abs(w[h - 1] - base ** (-(r - 2) / r)) < 1e-15
    assert np.allclose(w[1:] / w[:-1], base ** (-2.0 / r), rtol=1e-12, atol=0)


def check_rope_invariants(rope, n=33, d=10, r=6, base=500.0, seed=53, tol=1e-12):
    """Invariants: position 0 is the identity; each pair keeps its norm;
    R_p R_s = R_{p+s}; <R_p a, R_s b> depends only on p - s."""
    rng = np.random.default_rng(seed)
    a, b = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    assert np.array_equal(np.asarray(rope(a, np.zeros(n, np.int64), r, base)), a)
    p = rng.integers(0, 5000, size=n)
    s = rng.integers(0, 5000, size=n)
    ya = np.asarray(rope(a, p, r, base))
    h = r // 2
    assert np.allclose(ya[:, :h] ** 2 + ya[:, h:r] ** 2, a[:, :h] ** 2 + a[:, h:r] ** 2,
                       rtol=0, atol=tol * 10)
    assert np.allclose(np.asarray(rope(ya, s, r, base)), np.asarray(rope(a, p + s, r, base)),
                       rtol=0, atol=1e-9)
    yb = np.asarray(rope(b, s, r, base))
    c = 777
    dot1 = np.sum(ya * yb, axis=1)
    dot2 = np.sum(np.asarray(rope(a, p + c, r, base)) * np.asarray(rope(b, s + c, r, base)), axis=1)
    assert np.allclose(dot1, dot2, rtol=0, atol=1e-9)


def check_rope_attention(ratt, rope_dims, base, n=37, d=8, p0=1000, seed=57, tol=1e-10):
    """Brute force in complex form: with S0 = 0, o_t = sum_{j<=t} score(t, j) v_j
    where score = sum_{a>=r} q_ta k_ja + Re sum_i conj(zq_ti) zk_ji exp(1j (j-t) w_i)
    (a function of t - j only, so o does not depend on p0), and S_final =
    sum_j (R_{p0+j} k_j)^T v_j."""
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((n, d)).astype(np.float32) for _ in range(3))
    q64, k64, v64 = (x.astype(np.float64) for x in (q, k, v))
    r, h = rope_dims, rope_dims // 2
    w = np.power(float(base), -np.arange(h) * 2.0 / r)
    zq = q64[:, :h] + 1j * q64[:, h:r]
    zk = k64[:, :h] + 1j * k64[:, h:r]
    ref = np.zeros((n, d))
    for t in range(n):
        for j in range(t + 1):
            sc = q64[t, r:] @ k64[j, r:] + np.sum(np.conj(zq[t]) * zk[j] * np.exp(1j * (j - t) * w)).real
            ref[t] += sc * v64[j]
    zr = zk * np.exp(1j * np.outer(p0 + np.arange(n), w))
    kr = np.concatenate([zr.real, zr.imag, k64[:, r:]], axis=1)
    sref = kr.T @ v64
    for off in (p0, 0, 65536):
        o, Sf = ratt(q, k, v, off, None)
        assert np.allclose(o, ref, rtol=0, atol=tol * np.abs(ref).max())
        if off == p0:
            assert np.allclose(Sf, sref, rtol=0, atol=tol * np.abs(sref).max())


def check_rope_resume(ratt, n=70, d=8, cuts=(1, 16, 33, 69), p0=5, seed=59, tol=1e-10):
    """Invariant: a unit run in two pieces, the second continued from the
    first's final state at positions that continue the first's, equals the
    run in one piece."""
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((n, d)).astype(np.float32) for _ in range(3))
    S0 = rng.standard_normal((d, d))
    o, Sf = ratt(q, k, v, p0, S0)
    for m in cuts:
        o1, S1 = ratt(q[:m], k[:m], v[:m], p0, S0)
        o2, S2 = ratt(q[m:], k[m:], v[m:], p0 + m, S1)
        oo = np.concatenate([np.asarray(o1), np.asarray(o2)])
        assert np.allclose(oo, o, rtol=0, atol=tol * np.abs(o).max())
        assert np.allclose(S2, Sf, rtol=0, atol=tol * np.abs(Sf).max())

"""The CPU oracle against hand-worked examples, closed forms, library routines and
invariants (no GPU).  Mutant implementations show each pin catches a plausible
mistake."""
import numpy as np
import pytest

import pins


@pytest.fixture(scope="module")
def O(oracle_mod):
    return oracle_mod


def forms(O):
    return {
        "naive": lambda q, k, v: O.causal_linear_attention(q, k, v, "naive"),
        "recurrent": lambda q, k, v: O.causal_linear_attention(q, k, v, "recurrent"),
        "block64": lambda q, k, v: O.causal_linear_attention(q, k, v, "block", 64),
        "block3": lambda q, k, v: O.causal_linear_attention(q, k, v, "block", 3),
    }


def blk(O):
    return lambda q, k, v, B: O.causal_linear_attention(q, k, v, "block", B)


def dec(O):
    return lambda q, k, v, S0: O.decode(q, k, v, S0)


def varlen(O, form="recurrent"):
    return lambda q, k, v, cu: O.causal_linear_attention_varlen(q, k, v, cu, form, 16)


# ---------------------------------------------------------------- oracle passes

@pytest.mark.parametrize("name", ["naive", "recurrent", "block64", "block3"])
def test_forms_pass_closed_forms(O, name):
    f = forms(O)[name]
    pins.check_golden_causal(f)
    pins.check_golden_ones(f)
    pins.check_all_ones(f)
    pins.check_one_hot(f)
    pins.check_prefix_sum(f)
    pins.check_vs_numpy_masked(f)
    pins.check_linearity(f)


def test_block_form_golden_and_invariance(O):
    pins.check_golden_block(blk(O))
    pins.check_block_invariance(blk(O), forms(O)["naive"])


def test_block_form_special_cases(O):
    """B >= n is the masked matrix form; B = 1 is the token recurrence."""
    rng = np.random.default_rng(23)
    q, k, v = (rng.standard_normal((41, 9)).astype(np.float32) for _ in range(3))
    full = O.causal_linear_attention(q, k, v, "block", 41)
    assert np.allclose(full, O.numpy_masked(q, k, v), rtol=0, atol=1e-12 * np.abs(full).max())
    one = O.causal_linear_attention(q, k, v, "block", 1)
    rec = O.causal_linear_attention(q, k, v, "recurrent")
    assert np.allclose(one, rec, rtol=0, atol=1e-12 * np.abs(rec).max())


def test_naive_equals_recurrent_random(O):
    """Associativity: sum_j (q.k_j) v_j == q (sum_j k_j^T v_j), in fp64."""
    rng = np.random.default_rng(29)
    q, k, v = (rng.standard_normal((3, 257, 64)).astype(np.float32) for _ in range(3))
    a = O.causal_linear_attention(q, k, v, "naive")
    b = O.causal_linear_attention(q, k, v, "recurrent")
    assert O.rel_err(a, b) < 1e-12


def test_integer_exact_against_fractions(O):
    exact = lambda q, k, v: np.array(O.fraction_bruteforce(q, k, v), dtype=np.float64)
    for f in forms(O).values():
        pins.check_integer_exact(f, exact)


def test_fraction_bruteforce_random_dyadic(O):
    """Dyadic inputs (few mantissa bits): fp64 sums are exact, so the oracle must
    equal exact rational arithmetic."""
    rng = np.random.default_rng(31)
    q, k, v = (np.round(rng.standard_normal((12, 5)) * 8) / 8 for _ in range(3))
    exact = np.array(O.fraction_bruteforce(q, k, v), dtype=np.float64)
    for name in ("naive", "recurrent", "block3"):
        assert np.array_equal(forms(O)[name](q.astype(np.float32), k.astype(np.float32),
                                             v.astype(np.float32)), exact), name


def test_varlen(O):
    pins.check_varlen_resets(varlen(O), forms(O)["naive"])
    pins.check_varlen_resets(varlen(O, "naive"), forms(O)["recurrent"])
    pins.check_varlen_resets(varlen(O, "block"), forms(O)["naive"])


def test_decode(O):
    pins.check_golden_decode(dec(O))
    pins.check_decode_state_sum(dec(O))
    pins.check_decode_vs_prefill(dec(O), forms(O)["naive"])


def test_recurrent_rows_and_final_state(O):
    rng = np.random.default_rng(37)
    q, k, v = (rng.standard_normal((300, 16)).astype(np.float32) for _ in range(3))
    full = O.causal_linear_attention(q, k, v, "recurrent")
    rows = np.array([0, 1, 63, 64, 255, 299])
    assert np.array_equal(O.recurrent_rows(q, k, v, rows), full[rows])
    o, S = O.recurrent_final_state(q, k, v)
    assert np.allclose(S, k.astype(np.float64).T @ v, rtol=0, atol=1e-12 * np.abs(S).max())
    # Resuming from the final state of the first half gives the second half.
    o1, S1 = O.recurrent_final_state(q[:100], k[:100], v[:100])
    o2, _ = O.recurrent_final_state(q[100:], k[100:], v[100:], S1)
    assert O.rel_err(np.concatenate([o1, o2]), full) < 1e-13


def test_empty_inputs(O):
    z = np.zeros((0, 8), np.float32)
    assert O.causal_linear_attention(z, z, z).shape == (0, 8)
    z3 = np.zeros((2, 0, 8), np.float32)
    assert O.causal_linear_attention_varlen(z3, z3, z3, np.array([0, 0, 0])).shape == (2, 0, 8)


def test_rel_err_metric(O):
    assert O.rel_err([1.0, -4.0], [1.0, -4.0]) == 0.0
    assert O.rel_err([1.5, -4.0], [1.0, -4.0]) == pytest.approx(0.125)


def stf(O):
    return lambda q, k, v, S0: O.causal_linear_attention_state(q, k, v, S0)


def test_state_handoff(O):
    f = stf(O)
    pins.check_golden_state(f)
    pins.check_state_closed_form(f)
    pins.check_state_resume(f)
    pins.check_state_exact(f)


def test_state_batched_and_varlen(O):
    """The batched and packed drivers give each unit its own state, and a
    packed sequence of length 0 ends in its initial state."""
    rng = np.random.default_rng(43)
    q, k, v = (rng.standard_normal((2, 3, 19, 4)).astype(np.float32) for _ in range(3))
    S0 = rng.standard_normal((2, 3, 4, 4))
    o, Sf = O.causal_linear_attention_state(q, k, v, S0)
    for b in range(2):
        for h in range(3):
            o1, S1 = O.recurrent_final_state(q[b, h], k[b, h], v[b, h], S0[b, h])
            assert np.array_equal(o[b, h], o1) and np.array_equal(Sf[b, h], S1)
    lengths = [5, 0, 9]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    qp, kp, vp = (rng.standard_normal((3, T, 4)).astype(np.float32) for _ in range(3))
    S0p = rng.standard_normal((3, 3, 4, 4))
    op, Sfp = O.causal_linear_attention_varlen_state(qp, kp, vp, cu, S0p)
    for s in range(3):
        for h in range(3):
            a, e = cu[s], cu[s + 1]
            o1, S1 = O.recurrent_final_state(qp[h, a:e], kp[h, a:e], vp[h, a:e], S0p[s, h])
            assert np.array_equal(op[h, a:e], o1) and np.array_equal(Sfp[s, h], S1)
    assert np.array_equal(Sfp[1], S0p[1])
    o0, Sf0 = O.causal_linear_attention_varlen_state(qp, kp, vp, cu, None)
    assert np.array_equal(o0, O.causal_linear_attention_varlen(qp, kp, vp, cu))


def test_rope(O):
    pins.check_golden_rope(O.rope)
    pins.check_rope_complex(O.rope)
    pins.check_rope_frequencies(O.rope)
    pins.check_rope_frequencies(O.rope, r=64, base=1e7)
    pins.check_rope_invariants(O.rope)


def ratt(O, r=4, base=100.0):
    def f(q, k, v, p0, S0):
        o, Sf = O.causal_linear_attention_rope(q[None, None], k[None, None], v[None, None], r,
                                               base, [p0], None if S0 is None else S0[None, None])
        return o[0, 0], Sf[0, 0]
    return f


def test_rope_attention(O):
    for r, base in ((4, 100.0), (8, 10000.0), (2, 3.0)):
        pins.check_rope_attention(ratt(O, r, base), r, base)
        pins.check_rope_resume(ratt(O, r, base))


def test_rope_rows_match_full_form(O):
    """The row-wise spot-check form equals the full closed form."""
    rng = np.random.default_rng(63)
    n, d, r, base = 50, 8, 4, 1e7
    q, k, v = (rng.standard_normal((n, d)).astype(np.float32) for _ in range(3))
    S0 = rng.standard_normal((d, d))
    o, _ = O.causal_linear_attention_rope(q[None, None], k[None, None], v[None, None], r, base,
                                          [777], S0[None, None])
    rows = [0, 1, 17, 49]
    orow = O.causal_linear_attention_rope_rows(q, k, v, rows, r, base, 777, S0)
    assert np.allclose(orow, o[0, 0, rows], rtol=0, atol=1e-12 * np.abs(o).max())


def test_rope_attention_varlen_and_decode(O):
    """Packed sequences restart their positions (plus their offset) at each
    sequence's first token; decode at positions continuing a prefill matches
    the prefill of the whole."""
    rng = np.random.default_rng(61)
    lengths = [7, 0, 12, 1]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T, H, d, r, base = int(cu[-1]), 2, 8, 4, 50.0
    q, k, v = (rng.standard_normal((H, T, d)).astype(np.float32) for _ in range(3))
    off = np.array([0, 9, 100, 3])
    S0 = rng.standard_normal((4, H, d, d))
    o, Sf = O.causal_linear_attention_rope_varlen(q, k, v, cu, r, base, off, S0)
    for s_ in range(4):
        a, e = cu[s_], cu[s_ + 1]
        od, Sd = O.causal_linear_attention_rope(q[None, :, a:e], k[None, :, a:e], v[None, :, a:e],
                                                r, base, [off[s_]], S0[s_][None])
        assert np.array_equal(o[:, a:e], od[0]) and np.array_equal(Sf[s_], Sd[0])
    assert np.array_equal(Sf[1], S0[1])
    # decode continuing a prefill of 11 tokens
    n, m = 16, 11
    qd, kd, vd = (rng.standard_normal((1, H, n, d)).astype(np.float32) for _ in range(3))
    ofull, Sfull = O.causal_linear_attention_rope(qd, kd, vd, r, base, [4])
    _, Sm = O.causal_linear_attention_rope(qd[:, :, :m], kd[:, :, :m], vd[:, :, :m], r, base, [4])
    steps = lambda x: np.transpose(x[0, :, m:], (1, 0, 2))
    od, Sd = O.decode_rope(steps(qd), steps(kd), steps(vd), Sm[0], np.full(H, 4 + m), r, base)
    # a decode step reads the state before its token; the token's own term is
    # (R_p q . R_p k) v = (q . k) v since both turn by the same angles
    own = np.sum(qd[0, :, m:].astype(np.float64) * kd[0, :, m:], axis=-1)[..., None] * vd[0, :, m:]
    assert np.allclose(np.transpose(od, (1, 0, 2)) + own, ofull[0, :, m:], rtol=0,
                       atol=1e-12 * np.abs(ofull).max())
    assert np.allclose(Sd, Sfull[0], rtol=0, atol=1e-12 * np.abs(Sfull).max())


# ------------------------------------------------- mutants: the pins must bite

def _np_causal(q, k, v, strict=False, transpose_state=False):
    q = q.astype(np.float64); k = k.astype(np.float64); v = v.astype(np.float64)
    n, d = q.shape
    out = np.zeros((n, d))
    S = np.zeros((d, d))
    for t in range(n):
        if not strict:
            S += np.outer(k[t], v[t])
        out[t] = q[t] @ (S.T if transpose_state else S)
        if strict:
            S += np.outer(k[t], v[t])
    return out


def _np_block_no_inter(q, k, v, B):
    q = q.astype(np.float64); k = k.astype(np.float64); v = v.astype(np.float64)
    n, _ = q.shape
    out = np.zeros_like(q)
    for s in range(0, n, B):
        e = min(n, s + B)
        out[s:e] = np.tril(q[s:e] @ k[s:e].T) @ v[s:e]
    return out


def _np_block_inclusive_prefix(q, k, v, B):
    q = q.astype(np.float64); k = k.astype(np.float64); v = v.astype(np.float64)
    n, d = q.shape
    out = np.zeros_like(q)
    S = np.zeros((d, d))
    for s in range(0, n, B):
        e = min(n, s + B)
        S = S + k[s:e].T @ v[s:e]          # mistake: prefix includes the block itself
        out[s:e] = np.tril(q[s:e] @ k[s:e].T) @ v[s:e] + q[s:e] @ S
    return out


def _dec_update_first(q, k, v, S0):
    S = np.array(S0, np.float64).copy()
    steps, units, d = q.shape
    o = np.zeros((steps, units, d))
    for t in range(steps):
        for u in range(units):
            S[u] += np.outer(k[t, u], v[t, u])
            o[t, u] = q[t, u] @ S[u]
    return o, S


def _varlen_no_reset(q, k, v, cu):
    H, T, d = q.shape
    o = np.zeros((H, T, d))
    for h in range(H):
        o[h] = _np_causal(q[h], k[h], v[h])
    return o


def _np_state(q, k, v, S0, ignore_in_o=False, transpose_s0=False, final_without_s0=False):
    q = q.astype(np.float64); k = k.astype(np.float64); v = v.astype(np.float64)
    S0 = np.asarray(S0, np.float64)
    S0 = S0.T if transpose_s0 else S0
    n, d = q.shape
    out = np.zeros((n, d))
    S = np.zeros((d, d)) if ignore_in_o else S0.copy()
    for t in range(n):
        S += np.outer(k[t], v[t])
        out[t] = q[t] @ S
    Sf = k.T @ v if final_without_s0 else (S if not ignore_in_o else S0 + S)
    return out, Sf


def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def test_mutants_are_caught():
    strict = lambda q, k, v: _np_causal(q, k, v, strict=True)
    transposed = lambda q, k, v: _np_causal(q, k, v, transpose_state=True)
    good = lambda q, k, v: _np_causal(q, k, v)
    # sanity: the straightforward numpy recurrence passes
    pins.check_golden_causal(good)
    pins.check_all_ones(good)
    pins.check_one_hot(good)
    # diagonal dropped from the mask
    assert _fails(pins.check_golden_causal, strict)
    assert _fails(pins.check_all_ones, strict)
    assert _fails(pins.check_prefix_sum, strict)
    # state used transposed (value/key roles swapped)
    assert _fails(pins.check_golden_causal, transposed)
    assert _fails(pins.check_one_hot, transposed)
    # inter-block term missing, or prefix made inclusive
    assert _fails(pins.check_golden_block, _np_block_no_inter)
    assert _fails(pins.check_block_invariance, _np_block_no_inter, good)
    assert _fails(pins.check_golden_block, _np_block_inclusive_prefix)
    assert _fails(pins.check_block_invariance, _np_block_inclusive_prefix, good)
    # decode that updates the state before reading it
    assert _fails(pins.check_golden_decode, _dec_update_first)
    assert _fails(pins.check_decode_vs_prefill, _dec_update_first, good)
    # packed sequences that leak state across boundaries
    assert _fails(pins.check_varlen_resets, _varlen_no_reset, good)
    # state handoff: the initial state ignored by o, used transposed, or
    # missing from the final state
    stf_good = lambda q, k, v, S0: _np_state(q, k, v, S0)
    pins.check_golden_state(stf_good)
    pins.check_state_closed_form(stf_good)
    pins.check_state_resume(stf_good)
    pins.check_state_exact(stf_good)
    no_init = lambda q, k, v, S0: _np_state(q, k, v, S0, ignore_in_o=True)
    assert _fails(pins.check_golden_state, no_init)
    assert _fails(pins.check_state_closed_form, no_init)
    assert _fails(pins.check_state_resume, no_init)
    s0_t = lambda q, k, v, S0: _np_state(q, k, v, S0, transpose_s0=True)
    assert _fails(pins.check_golden_state, s0_t)
    assert _fails(pins.check_state_closed_form, s0_t)
    assert _fails(pins.check_state_exact, s0_t)
    no_carry = lambda q, k, v, S0: _np_state(q, k, v, S0, final_without_s0=True)
    assert _fails(pins.check_golden_state, no_carry)
    assert _fails(pins.check_state_resume, no_carry)


def _np_rope(x, pos, r, base, interleaved=False, negative=False, over_d=False, shift=0, all_dims=False):
    x = np.asarray(x, np.float64)
    r = x.shape[-1] if all_dims else r
    h = r // 2
    den = x.shape[-1] * 2 if over_d else r
    w = float(base) ** (-2.0 * (np.arange(h) + shift) / den)
    ang = np.asarray(pos, np.float64)[..., None] * w * (-1 if negative else 1)
    c, sn = np.cos(ang), np.sin(ang)
    y = x.copy()
    ia = np.arange(0, r, 2) if interleaved else np.arange(h)
    ib = ia + 1 if interleaved else ia + h
    y[..., ia] = x[..., ia] * c - x[..., ib] * sn
    y[..., ib] = x[..., ia] * sn + x[..., ib] * c
    return y


def _np_ratt(r, base, rot_v=False, q_only=False, ignore_p0=False):
    def f(q, k, v, p0, S0):
        n, d = q.shape
        pos = (0 if ignore_p0 else p0) + np.arange(n)
        qr = _np_rope(q, pos, r, base)
        kr = k.astype(np.float64) if q_only else _np_rope(k, pos, r, base)
        vr = _np_rope(v, pos, r, base) if rot_v else v.astype(np.float64)
        return _np_state(qr, kr, vr, np.zeros((d, d)) if S0 is None else S0)
    return f


def test_rope_mutants_are_caught():
    good = lambda x, p, r, b: _np_rope(x, p, r, b)
    pins.check_golden_rope(good)
    pins.check_rope_complex(good)
    pins.check_rope_frequencies(good)
    pins.check_rope_invariants(good)
    # adjacent (interleaved) pairs instead of split halves
    inter = lambda x, p, r, b: _np_rope(x, p, r, b, interleaved=True)
    assert _fails(pins.check_golden_rope, inter)
    assert _fails(pins.check_rope_complex, inter)
    # rotation the wrong way
    neg = lambda x, p, r, b: _np_rope(x, p, r, b, negative=True)
    assert _fails(pins.check_golden_rope, neg)
    assert _fails(pins.check_rope_complex, neg)
    assert _fails(pins.check_rope_frequencies, neg)
    # exponent over the whole head dim, or frequencies off by one pair
    overd = lambda x, p, r, b: _np_rope(x, p, r, b, over_d=True)
    assert _fails(pins.check_golden_rope, overd)
    assert _fails(pins.check_rope_frequencies, overd)
    off1 = lambda x, p, r, b: _np_rope(x, p, r, b, shift=1)
    assert _fails(pins.check_golden_rope, off1)
    assert _fails(pins.check_rope_frequencies, off1)
    # every dim rotated
    alld = lambda x, p, r, b: _np_rope(x, p, r, b, all_dims=True)
    assert _fails(pins.check_golden_rope, alld)
    assert _fails(pins.check_rope_complex, alld)
    # attention: the oracle-shaped good variant passes, the mistakes fail
    pins.check_rope_attention(_np_ratt(4, 100.0), 4, 100.0)
    pins.check_rope_resume(_np_ratt(4, 100.0))
    assert _fails(pins.check_rope_attention, _np_ratt(4, 100.0, rot_v=True), 4, 100.0)
    assert _fails(pins.check_rope_attention, _np_ratt(4, 100.0, q_only=True), 4, 100.0)
    assert _fails(pins.check_rope_resume, _np_ratt(4, 100.0, ignore_p0=True))

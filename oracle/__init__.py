"""CPU oracle for causal linear attention (Lightning Attention forward + decode).

TEST INFRASTRUCTURE ONLY.  Nothing in the product package imports this module;
only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline leg
of ``bench.py`` use it.  It shares no code with the HIP path.

The arithmetic lives in ``la_oracle.c`` (IEEE double, plain loops, built with
``-O2 -ffp-contract=off`` and no fast-math).  This module builds that file,
binds it with ctypes and adds two tiny-input brute forces (numpy matrix form
and exact rational arithmetic) that are written independently of the C code,
plus the rotary position embedding on half the head dims (numpy float64) and
causal linear attention over rotated q and k in its closed masked form.

The operation (wiki page "MiniMax-01 Lightning Attention", section
"Lightning Attention 设计"; Tencent Cloud article, section 4.1):
    o_i = sum_{j<=i} (q_i . k_j) v_j           (no scale, no normaliser, no decay)
decode step (literal order):  o = q S_old ;  S_new = S_old + k^T v .
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from fractions import Fraction

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "la_oracle.c")
_BUILD = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD, "liblaoracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile la_oracle.c into oracle/_build/liblaoracle.so (plain gcc)."""
    os.makedirs(_BUILD, exist_ok=True)
    if not force and os.path.exists(_LIB_PATH) and \
            os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-std=c11", "-Wall", "-shared", "-fPIC", _SRC, "-o", tmp]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    f32p = ctypes.POINTER(ctypes.c_float)
    f64p = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    i32p = ctypes.POINTER(ctypes.c_int32)
    i64p = ctypes.POINTER(ctypes.c_int64)
    c_int = ctypes.c_int
    lib.lao_naive.argtypes = [f32p, f32p, f32p, f64p, i64, c_int]
    lib.lao_recurrent.argtypes = [f32p, f32p, f32p, f64p, i64, c_int, f64p]
    lib.lao_recurrent_rows.argtypes = [f32p, f32p, f32p, i64, c_int, i64p, i64, f64p]
    lib.lao_block.argtypes = [f32p, f32p, f32p, f64p, i64, c_int, i64]
    lib.lao_decode_step.argtypes = [f32p, f32p, f32p, f64p, f64p, c_int]
    lib.lao_units.argtypes = [f32p, f32p, f32p, f64p, i64, i64, c_int, c_int, i64, c_int]
    lib.lao_varlen.argtypes = [f32p, f32p, f32p, f64p, c_int, i64, i32p, c_int, c_int,
                               c_int, i64, c_int]
    lib.lao_decode_units.argtypes = [f32p, f32p, f32p, f64p, f64p, i64, i64, c_int, c_int]
    lib.lao_units_state.argtypes = [f32p, f32p, f32p, f64p, i64, i64, c_int, f64p, f64p, c_int]
    lib.lao_varlen_state.argtypes = [f32p, f32p, f32p, f64p, c_int, i64, i32p, c_int, c_int,
                                     f64p, f64p, c_int]
    lib.lao_max_threads.restype = c_int
    for fn in ("lao_naive", "lao_recurrent", "lao_recurrent_rows", "lao_block",
               "lao_decode_step", "lao_units", "lao_varlen", "lao_decode_units",
               "lao_units_state", "lao_varlen_state"):
        getattr(lib, fn).restype = None
    _lib = lib
    return lib


def _f32(x) -> np.ndarray:
    """Exact float32 view of the inputs (bf16 and fp32 values are exact in fp32)."""
    a = np.ascontiguousarray(np.asarray(x), dtype=np.float32)
    return a


def _p(a, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


FORMS = {"naive": 0, "recurrent": 1, "block": 2}


def max_threads() -> int:
    return int(_load().lao_max_threads())


def causal_linear_attention(q, k, v, form: str = "recurrent", block_size: int = 0,
                            nthreads: int = 0) -> np.ndarray:
    """o for inputs shaped [..., n, d]; every leading index is an independent unit.

    form: "naive" (O(n^2 d) definition), "recurrent" (token state recurrence)
    or "block" (intra/inter split with block_size).  Returns float64.
    """
    lib = _load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    assert q.shape == k.shape == v.shape and q.ndim >= 2
    n, d = q.shape[-2], q.shape[-1]
    units = int(np.prod(q.shape[:-2])) if q.ndim > 2 else 1
    o = np.zeros(q.shape, dtype=np.float64)
    if n == 0 or units == 0:
        return o
    if form == "block" and block_size < 1:
        raise ValueError("block form needs block_size >= 1")
    lib.lao_units(_p(q, ctypes.c_float), _p(k, ctypes.c_float), _p(v, ctypes.c_float),
                  _p(o, ctypes.c_double), units, n, d, FORMS[form], int(block_size),
                  int(nthreads))
    return o


def causal_linear_attention_varlen(q, k, v, cu_seqlens, form: str = "recurrent",
                                   block_size: int = 0, nthreads: int = 0) -> np.ndarray:
    """Packed input [heads, T, d]; sequence s is tokens [cu[s], cu[s+1]) and
    starts from an empty state (each packed sequence is independent)."""
    lib = _load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    cu = np.ascontiguousarray(np.asarray(cu_seqlens), dtype=np.int32)
    heads, T, d = q.shape
    assert cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    o = np.zeros(q.shape, dtype=np.float64)
    if T == 0:
        return o
    lib.lao_varlen(_p(q, ctypes.c_float), _p(k, ctypes.c_float), _p(v, ctypes.c_float),
                   _p(o, ctypes.c_double), heads, T, _p(cu, ctypes.c_int32), len(cu) - 1,
                   d, FORMS[form], int(block_size), int(nthreads))
    return o


def causal_linear_attention_state(q, k, v, S0=None, nthreads: int = 0):
    """(o, S_final) for inputs [..., n, d] (every leading index a unit), each
    unit starting from S0[...] ([..., d, d]; None = zero).  Recurrent form:
    o_t = q_t (S0 + sum_{j<=t} k_j^T v_j), S_final = S0 + K^T V.  float64."""
    lib = _load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    assert q.shape == k.shape == v.shape and q.ndim >= 2
    n, d = q.shape[-2], q.shape[-1]
    lead = q.shape[:-2]
    units = int(np.prod(lead)) if lead else 1
    o = np.zeros(q.shape, dtype=np.float64)
    Sf = np.zeros(lead + (d, d), dtype=np.float64)
    s0 = None if S0 is None else np.ascontiguousarray(np.asarray(S0, np.float64).reshape(lead + (d, d)))
    if units == 0:
        return o, Sf
    lib.lao_units_state(_p(q, ctypes.c_float), _p(k, ctypes.c_float), _p(v, ctypes.c_float),
                        _p(o, ctypes.c_double), units, n, d,
                        None if s0 is None else _p(s0, ctypes.c_double), _p(Sf, ctypes.c_double),
                        int(nthreads))
    return o, Sf


def causal_linear_attention_varlen_state(q, k, v, cu_seqlens, S0=None, nthreads: int = 0):
    """(o, S_final) for packed input [heads, T, d] with per-sequence states
    S0 / S_final laid out [nseq, heads, d, d] (S0 None = zero)."""
    lib = _load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    cu = np.ascontiguousarray(np.asarray(cu_seqlens), dtype=np.int32)
    heads, T, d = q.shape
    nseq = len(cu) - 1
    assert cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    o = np.zeros(q.shape, dtype=np.float64)
    Sf = np.zeros((nseq, heads, d, d), dtype=np.float64)
    s0 = None if S0 is None else np.ascontiguousarray(np.asarray(S0, np.float64).reshape(nseq, heads, d, d))
    lib.lao_varlen_state(_p(q, ctypes.c_float), _p(k, ctypes.c_float), _p(v, ctypes.c_float),
                         _p(o, ctypes.c_double), heads, T, _p(cu, ctypes.c_int32), nseq, d,
                         None if s0 is None else _p(s0, ctypes.c_double), _p(Sf, ctypes.c_double),
                         int(nthreads))
    return o, Sf


def recurrent_rows(q, k, v, rows) -> np.ndarray:
    """o at the given token positions of one [n, d] unit (recurrent form)."""
    lib = _load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    n, d = q.shape
    rows = np.ascontiguousarray(np.asarray(rows), dtype=np.int64)
    assert np.all(np.diff(rows) > 0) and (len(rows) == 0 or (rows[0] >= 0 and rows[-1] < n))
    out = np.zeros((len(rows), d), dtype=np.float64)
    if len(rows):
        lib.lao_recurrent_rows(_p(q, ctypes.c_float), _p(k, ctypes.c_float),
                               _p(v, ctypes.c_float), n, d, _p(rows, ctypes.c_int64),
                               len(rows), _p(out, ctypes.c_double))
    return out


def recurrent_final_state(q, k, v, S0=None):
    """(o, S_final) for one [n, d] unit, optionally from an initial state S0."""
    lib = _load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    n, d = q.shape
    S = np.zeros((d, d), np.float64) if S0 is None else np.array(S0, dtype=np.float64, order="C")
    o = np.zeros((n, d), np.float64)
    lib.lao_recurrent(_p(q, ctypes.c_float), _p(k, ctypes.c_float), _p(v, ctypes.c_float),
                      _p(o, ctypes.c_double), n, d, _p(S, ctypes.c_double))
    return o, S


def decode(q, k, v, S0, nthreads: int = 0):
    """Run steps of the decode recurrence.

    q, k, v: [steps, units, d]; S0: [units, d, d].  Returns (o [steps, units, d],
    S_final [units, d, d]) in float64.  Step t reads the state before token t.
    """
    lib = _load()
    q, k, v = _f32(q), _f32(k), _f32(v)
    steps, units, d = q.shape
    S = np.array(S0, dtype=np.float64, order="C").reshape(units, d, d).copy()
    o = np.zeros((steps, units, d), np.float64)
    lib.lao_decode_units(_p(q, ctypes.c_float), _p(k, ctypes.c_float), _p(v, ctypes.c_float),
                         _p(S, ctypes.c_double), _p(o, ctypes.c_double), steps, units, d,
                         int(nthreads))
    return o, S


# ---- rotary position embedding on half the head dims ------------------------
#
# Wiki page "MiniMax-01 Lightning Attention", section "模型架构": RoPE is
# applied to half of the attention head dimensions with base frequency
# 10,000 (raised to 10M for the long-context stage).  The page leaves the
# rest open; the readings taken here: the rotated dims are the first
# rope_dims = d/2 of q and k (v is not rotated); dim i < rope_dims/2 pairs with
# dim i + rope_dims/2; the pair at token position p turns by the angle
# p * base^(-2i / rope_dims); positions count from 0 at each sequence's first
# token, plus an optional per-sequence offset (a sequence continued from a
# carried-in state continues its positions).

def rope(x, positions, rope_dims: int, base: float) -> np.ndarray:
    """x [..., n, d] rotated at integer positions [..., n] (float64)."""
    x = np.asarray(x, np.float64)
    r = int(rope_dims)
    assert r % 2 == 0 and 0 < r <= x.shape[-1]
    h = r // 2
    theta = float(base) ** (-2.0 * np.arange(h, dtype=np.float64) / r)
    ang = np.asarray(positions, np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    out = x.copy()
    a, b = x[..., :h], x[..., h:r]
    out[..., :h] = a * c - b * s
    out[..., h:r] = a * s + b * c
    return out


def masked_state_form(q, k, v, S0=None):
    """(o, S_final) for one [n, d] unit in float64 by the closed form
    o = tril(Q K^T) V + Q S0, S_final = S0 + K^T V (inputs taken as given,
    no rounding).  Quadratic in n: for the moderate sizes of the tests."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    d = q.shape[-1]
    S0 = np.zeros((d, d)) if S0 is None else np.asarray(S0, np.float64)
    return np.tril(q @ k.T) @ v + q @ S0, S0 + k.T @ v


def causal_linear_attention_rope(q, k, v, rope_dims: int, base: float, pos_offset=None,
                                 S0=None):
    """Dense [B, H, n, d]: q and k rotated at positions pos_offset[b] + t, then
    causal linear attention from S0 [B, H, d, d] (None = zero).  Returns
    (o, S_final) in float64."""
    q = np.asarray(q, np.float64)
    B, H, n, d = q.shape
    off = np.zeros(B, np.int64) if pos_offset is None else np.asarray(pos_offset, np.int64)
    o = np.zeros(q.shape)
    Sf = np.zeros((B, H, d, d))
    for b in range(B):
        pos = off[b] + np.arange(n)
        for h in range(H):
            qr = rope(q[b, h], pos, rope_dims, base)
            kr = rope(k[b, h], pos, rope_dims, base)
            o[b, h], Sf[b, h] = masked_state_form(qr, kr, v[b, h], None if S0 is None else S0[b, h])
    return o, Sf


def causal_linear_attention_rope_varlen(q, k, v, cu_seqlens, rope_dims: int, base: float,
                                        pos_offset=None, S0=None):
    """Packed [H, T, d] (sequence s is tokens [cu[s], cu[s+1])): as
    causal_linear_attention_rope per sequence; S0 / S_final [nseq, H, d, d]."""
    q = np.asarray(q, np.float64)
    H, T, d = q.shape
    cu = np.asarray(cu_seqlens, np.int64)
    nseq = len(cu) - 1
    off = np.zeros(nseq, np.int64) if pos_offset is None else np.asarray(pos_offset, np.int64)
    o = np.zeros(q.shape)
    Sf = np.zeros((nseq, H, d, d))
    for s_ in range(nseq):
        a, e = cu[s_], cu[s_ + 1]
        pos = off[s_] + np.arange(e - a)
        for h in range(H):
            qr = rope(q[h, a:e], pos, rope_dims, base)
            kr = rope(k[h, a:e], pos, rope_dims, base)
            o[h, a:e], Sf[s_, h] = masked_state_form(qr, kr, v[h, a:e],
                                                      None if S0 is None else S0[s_, h])
    return o, Sf


def causal_linear_attention_rope_rows(q, k, v, rows, rope_dims: int, base: float, p0: int = 0,
                                      S0=None) -> np.ndarray:
    """Selected output rows of one [n, d] unit with q and k rotated at
    positions p0 + t, straight from the definition:
    o_t = (R q_t) S0 + sum_{j<=t} ((R q_t) . (R k_j)) v_j.  Cost O(n d) per row,
    for spot checks of long sequences."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n, d = q.shape
    rows = np.asarray(rows, np.int64)
    kr = rope(k, p0 + np.arange(n), rope_dims, base)
    qr = rope(q[rows], p0 + rows, rope_dims, base)
    out = np.zeros((len(rows), d))
    for m, t in enumerate(rows):
        out[m] = (kr[:t + 1] @ qr[m]) @ v[:t + 1]
        if S0 is not None:
            out[m] += qr[m] @ np.asarray(S0, np.float64)
    return out


def decode_rope(q, k, v, S0, positions, rope_dims: int, base: float):
    """Decode steps with rotated q and k: q, k, v [steps, units, d], S0 [units,
    d, d], positions [units] of the first step (step t is at positions + t).
    Returns (o, S_final) in float64."""
    q = np.asarray(q, np.float64)
    steps, units, d = q.shape
    S = np.array(S0, np.float64).reshape(units, d, d).copy()
    o = np.zeros((steps, units, d))
    pos0 = np.asarray(positions, np.int64)
    for t in range(steps):
        for u in range(units):
            qr = rope(q[t, u][None], [pos0[u] + t], rope_dims, base)[0]
            kr = rope(k[t, u][None], [pos0[u] + t], rope_dims, base)[0]
            o[t, u] = qr @ S[u]
            S[u] += np.outer(kr, np.asarray(v[t, u], np.float64))
    return o, S


# ---- tiny-input brute forces (independent of la_oracle.c) ------------------

def numpy_masked(q, k, v) -> np.ndarray:
    """np.tril(Q K^T) V in float64: the textbook masked-matrix form."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    return np.tril(q @ np.swapaxes(k, -1, -2)) @ v


def fraction_bruteforce(q, k, v):
    """Exact rational o_i = sum_{j<=i} (q_i . k_j) v_j for one small [n, d] unit."""
    n, d = len(q), len(q[0])
    Q = [[Fraction(float(x)) for x in row] for row in q]
    K = [[Fraction(float(x)) for x in row] for row in k]
    V = [[Fraction(float(x)) for x in row] for row in v]
    out = []
    for i in range(n):
        acc = [Fraction(0)] * d
        for j in range(i + 1):
            s = sum((Q[i][a] * K[j][a] for a in range(d)), Fraction(0))
            acc = [acc[b] + s * V[j][b] for b in range(d)]
        out.append(acc)
    return out


def rel_err(o, o_ref) -> float:
    """max|o - o_ref| / max|o_ref| over the whole checked tensor."""
    o = np.asarray(o, np.float64)
    o_ref = np.asarray(o_ref, np.float64)
    denom = float(np.max(np.abs(o_ref))) if o_ref.size else 0.0
    num = float(np.max(np.abs(o - o_ref))) if o_ref.size else 0.0
    if denom == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / denom

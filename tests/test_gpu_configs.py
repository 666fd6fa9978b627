"""The five workloads at full size on the GPU, in the launch configuration the
benchmark times, checked against the CPU oracle (in full where the oracle
finishes in seconds, else on sampled heads, sequences or rows)."""
import os
import threading

import numpy as np
import pytest

import oracle
import synth
from gpu_util import TOL, device, host, note

pytestmark = pytest.mark.gpu

NTHREADS = min(16, len(os.sched_getaffinity(0)))


@pytest.fixture(scope="module")
def dev():
    return device()


def _fwd(q, k, v, B, cu=None):
    import torch
    import linear_attention_attn_amd as la
    o = la.fwd(q, k, v, block_size=B, cu_seqlens=cu)
    torch.cuda.synchronize()
    return o


def test_tiny_f32(dev):
    w = synth.WORKLOADS["tiny_f32"]
    note(f"workload {w.name}")
    q, k, v = synth.prefill_inputs(w.batch, w.heads, w.seq_len, w.head_dim, w.dtype, w.cid, dev)
    o = host(_fwd(q, k, v, w.block_size))
    qh, kh, vh = host(q), host(k), host(v)
    naive = oracle.causal_linear_attention(qh, kh, vh, "naive", nthreads=NTHREADS)
    rec = oracle.causal_linear_attention(qh, kh, vh, "recurrent", nthreads=NTHREADS)
    assert oracle.rel_err(naive, rec) < 1e-12
    assert oracle.rel_err(o, naive) <= TOL["f32"]


def test_minimax_layer_full(dev):
    w = synth.WORKLOADS["minimax_layer"]
    note(f"workload {w.name}")
    q, k, v = synth.prefill_inputs(w.batch, w.heads, w.seq_len, w.head_dim, w.dtype, w.cid, dev)
    o = _fwd(q, k, v, w.block_size)
    qh, kh, vh = host(q), host(k), host(v)
    del q, k, v
    ref = oracle.causal_linear_attention(qh, kh, vh, "recurrent", nthreads=NTHREADS)
    err = oracle.rel_err(host(o), ref)
    print(f"minimax_layer rel_err={err:.3e}")
    assert err <= TOL["bf16"]


def test_long_1m_two_heads(dev):
    """Full 1,048,576-token run of all 64 heads; heads 0 and 63 checked at 512
    sampled rows each (every block edge class, the first and last rows)."""
    import torch
    w = synth.WORKLOADS["long_1m"]
    note(f"workload {w.name}")
    q, k, v = synth.prefill_inputs(w.batch, w.heads, w.seq_len, w.head_dim, w.dtype, w.cid, dev)
    o = _fwd(q, k, v, w.block_size)
    n = w.seq_len
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 257, n // 2, n - 257, n - 256, n - 1],
                                     rng.integers(0, n, 500)]))
    results = {}

    def run(h):
        results[h] = oracle.recurrent_rows(host(q[0, h]), host(k[0, h]), host(v[0, h]), rows)

    ths = [threading.Thread(target=run, args=(h,)) for h in (0, 63)]
    for t in ths:
        t.start()
    for t in ths:
        t.join()
    rows_t = torch.from_numpy(rows).to(dev)
    for h in (0, 63):
        got = host(o[0, h].index_select(0, rows_t))
        err = oracle.rel_err(got, results[h])
        print(f"long_1m head {h} rel_err={err:.3e}")
        assert err <= TOL["bf16"], h


@pytest.mark.parametrize("name", ["varlen16", "varlen_short"])
def test_varlen_workload(dev, name):
    import torch
    w = synth.WORKLOADS[name]
    note(f"workload {w.name}")
    lengths = synth.varlen_lengths(w.batch, w.len_seed, w.len_lo, w.len_hi)
    q, k, v, cu = synth.varlen_inputs(lengths, w.heads, w.head_dim, w.dtype, w.cid, dev)
    o = _fwd(q, k, v, w.block_size, torch.from_numpy(cu).to(dev))
    hs = [0, 21, 42, 63]
    idx = torch.tensor(hs, device=dev)
    sel = lambda x: host(x.index_select(0, idx))
    ref = oracle.causal_linear_attention_varlen(sel(q), sel(k), sel(v), cu, "recurrent",
                                                nthreads=NTHREADS)
    err = oracle.rel_err(sel(o), ref)
    print(f"{name} T={int(cu[-1])} rel_err={err:.3e}")
    assert err <= TOL["bf16"]


def test_decode256(dev):
    """128 steps on all 256 x 64 states; sequences 0..31 (2,048 states) checked
    in full, every step."""
    import torch
    import linear_attention_attn_amd as la
    w = synth.WORKLOADS["decode256"]
    note(f"workload {w.name}")
    S = synth.decode_state(w.batch, w.heads, w.head_dim, w.cid, dev)
    nchk = 32
    S0 = host(S[:nchk]).reshape(-1, w.head_dim, w.head_dim)
    Q, K, V, O = [], [], [], []
    for t in range(w.steps):
        q, k, v = synth.decode_step_inputs(w.batch, w.heads, w.head_dim, w.dtype, w.cid, t, dev)
        o = la.decode(q, k, v, S)
        Q.append(host(q[:nchk])); K.append(host(k[:nchk])); V.append(host(v[:nchk]))
        O.append(host(o[:nchk]))
    torch.cuda.synchronize()
    shp = (w.steps, nchk * w.heads, w.head_dim)
    o_ref, S_ref = oracle.decode(np.stack(Q).reshape(shp), np.stack(K).reshape(shp),
                                 np.stack(V).reshape(shp), S0, nthreads=NTHREADS)
    err_o = oracle.rel_err(np.stack(O).reshape(shp), o_ref)
    err_s = oracle.rel_err(host(S[:nchk]).reshape(S_ref.shape), S_ref)
    print(f"decode256 rel_err o={err_o:.3e} S={err_s:.3e}")
    assert err_o <= TOL["bf16"]
    assert err_s <= 1e-4

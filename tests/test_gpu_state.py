"""State handoff (lightning_attn_fwd_state) on the GPU against the CPU oracle:
a prefill that starts from given per-sequence states and returns each
sequence's final state; in-place update; packed input with empty sequences;
a sequence prefilled in two pieces; prefill handing its state to decode."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, chunk_tokens, device, host, note, randn_qkv

pytestmark = pytest.mark.gpu

STOL = 1e-4   # final states are fp32 sums of exact bf16 or fp32 products


@pytest.fixture(scope="module")
def dev():
    return device()


def _states(shape, seed, dev, scale=0.5):
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return (scale * torch.randn(shape, generator=g, device=dev)).contiguous()


def _run(q, k, v, B, s_init, s_final, cu=None):
    import torch
    import linear_attention_attn_amd as la
    o = la.fwd(q, k, v, block_size=B, cu_seqlens=cu, s_init=s_init, s_final=s_final)
    torch.cuda.synchronize()
    return o


CASES = []
for dt in ("bf16", "f32"):
    for d in (64, 128):
        for B, n, C, S in ((64, 1, 0, 0), (256, 261, 0, 0), (256, 3 * 256 + 7, 0, 0),
                           (64, 40 * 64 + 9, 128, 0), (256, 34 * 256 + 100, 256, 0),
                           (64, 40 * 64 + 9, 512, 128)):
            CASES.append((dt, d, B, n, C, S))


@pytest.mark.parametrize("dt,d,B,n,C,S", CASES)
def test_state_in_and_out(dev, dt, d, B, n, C, S):
    """One chunk per sequence (C = 0, planned), many chunks (forced C), and
    chunks of several summary sub-chunks (forced S)."""
    import torch
    note(f"state dt={dt} d={d} B={B} n={n} C={C} S={S}")
    q, k, v = randn_qkv((2, 3, n, d), dt, 3000 + n + d + B, dev)
    S0 = _states((2, 3, d, d), 77 + d, dev)
    Sf = torch.empty_like(S0)
    with chunk_tokens(C, S):
        o = host(_run(q, k, v, B, S0, Sf))
    ref, sref = oracle.causal_linear_attention_state(host(q), host(k), host(v), host(S0))
    assert oracle.rel_err(o, ref) <= TOL[dt]
    assert oracle.rel_err(host(Sf), sref) <= STOL


@pytest.mark.parametrize("C", [0, 256])
def test_final_state_from_zero_and_in_place(dev, C):
    """s_init NULL gives zero-start outputs and K^T V; s_final == s_init updates in place."""
    import torch
    import linear_attention_attn_amd as la
    note(f"state zero/in-place C={C}")
    q, k, v = randn_qkv((2, 4, 1500, 128), "bf16", 91, dev)
    Sf = torch.empty((2, 4, 128, 128), dtype=torch.float32, device=dev)
    with chunk_tokens(C):
        o = host(_run(q, k, v, 256, None, Sf))
        o_plain = host(la.fwd(q, k, v, block_size=256))
    ref, sref = oracle.causal_linear_attention_state(host(q), host(k), host(v), None)
    assert oracle.rel_err(o, ref) <= TOL["bf16"]
    assert np.array_equal(o, o_plain)                 # same kernels, same arithmetic
    assert oracle.rel_err(host(Sf), sref) <= STOL
    S = _states((2, 4, 128, 128), 93, dev)
    S0 = host(S)
    with chunk_tokens(C):
        o2 = host(_run(q, k, v, 256, S, S))
    ref2, sref2 = oracle.causal_linear_attention_state(host(q), host(k), host(v), S0)
    assert oracle.rel_err(o2, ref2) <= TOL["bf16"]
    assert oracle.rel_err(host(S), sref2) <= STOL


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_state_packed_with_empty_sequences(dev, dt):
    import torch
    lengths = (5, 0, 700, 1, 2100, 0, 257)
    note(f"state packed dt={dt} lengths={lengths}")
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T, H, d = int(cu[-1]), 3, 128
    q, k, v = randn_qkv((H, T, d), dt, 4242, dev)
    S0 = _states((len(lengths), H, d, d), 4343, dev)
    Sf = torch.full_like(S0, float("nan"))
    cu_d = torch.tensor(cu, dtype=torch.int32, device=dev)
    with chunk_tokens(256):
        o = host(_run(q, k, v, 256, S0, Sf, cu_d))
    ref, sref = oracle.causal_linear_attention_varlen_state(host(q), host(k), host(v), cu, host(S0))
    assert oracle.rel_err(o, ref) <= TOL[dt]
    assert oracle.rel_err(host(Sf), sref) <= STOL
    for s, L in enumerate(lengths):
        if L == 0:
            assert np.array_equal(host(Sf)[s], host(S0)[s])


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_state_packed_tiled_scan(dev, dt, d):
    """Packed sequences with several scan tiles each (79, 33 and 11 sub-chunk
    entries with tiles of 32) next to one-chunk and empty ones, from initial
    states, with two sub-chunks per chunk."""
    import torch
    lengths = (5000, 3, 2100, 0, 700, 64)
    note(f"state packed tiled scan dt={dt} d={d}")
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T, H = int(cu[-1]), 2
    q, k, v = randn_qkv((H, T, d), dt, 4545 + d, dev)
    S0 = _states((len(lengths), H, d, d), 4646 + d, dev)
    Sf = torch.full_like(S0, float("nan"))
    cu_d = torch.tensor(cu, dtype=torch.int32, device=dev)
    with chunk_tokens(128, 64):
        o = host(_run(q, k, v, 64, S0, Sf, cu_d))
    ref, sref = oracle.causal_linear_attention_varlen_state(host(q), host(k), host(v), cu, host(S0))
    assert oracle.rel_err(o, ref) <= TOL[dt]
    assert oracle.rel_err(host(Sf), sref) <= STOL


@pytest.mark.parametrize("C,S", [(128, 0), (256, 64), (192, 64)])
def test_state_packed_chunk_boundaries(dev, C, S):
    """Sequence lengths on both sides of one and two chunks (C, C + 1, 2C - 1,
    2C, 2C + 1, 1 and 0 tokens) from initial states: the sequences of one
    chunk read their initial state directly, the others through the scan."""
    import torch
    lengths = (C, C + 1, 2 * C - 1, 2 * C, 2 * C + 1, 1, 0, 3 * C + 5)
    note(f"state packed chunk boundaries C={C} S={S}")
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T, H, d = int(cu[-1]), 2, 64
    q, k, v = randn_qkv((H, T, d), "bf16", 4747 + C, dev)
    S0 = _states((len(lengths), H, d, d), 4848 + C, dev)
    Sf = torch.full_like(S0, float("nan"))
    cu_d = torch.tensor(cu, dtype=torch.int32, device=dev)
    with chunk_tokens(C, S):
        o = host(_run(q, k, v, 64, S0, Sf, cu_d))
    ref, sref = oracle.causal_linear_attention_varlen_state(host(q), host(k), host(v), cu, host(S0))
    assert oracle.rel_err(o, ref) <= TOL["bf16"]
    assert oracle.rel_err(host(Sf), sref) <= STOL


def test_no_tokens_copies_initial_state(dev):
    """seq_len == 0: only s_final is written, equal to s_init (no workspace)."""
    import torch
    import linear_attention_attn_amd as la
    note("state no tokens")
    S0 = _states((3, 2, 64, 64), 5, dev)
    Sf = torch.full_like(S0, float("nan"))
    st = la.lightning_attn_fwd_state(None, None, None, None, 3, 2, 0, 64, 64, None, la.LA_DTYPE_BF16,
                                     S0, Sf, None, 0, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == la.LA_OK
    assert np.array_equal(host(Sf), host(S0))
    Sz = torch.full_like(S0, float("nan"))
    st = la.lightning_attn_fwd_state(None, None, None, None, 3, 2, 0, 64, 64, None, la.LA_DTYPE_BF16,
                                     None, Sz, None, 0, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == la.LA_OK and not host(Sz).any()


@pytest.mark.parametrize("m", [256, 1000, 2049])
def test_split_and_resume(dev, m):
    """A sequence prefilled in two pieces, the second from the first's final
    state, matches the one-piece prefill."""
    import torch
    note(f"state resume m={m}")
    n, d = 4096, 128
    q, k, v = randn_qkv((2, 4, n, d), "bf16", 55, dev)
    S1 = torch.empty((2, 4, d, d), dtype=torch.float32, device=dev)
    Sa = torch.empty_like(S1)
    Sb = torch.empty_like(S1)
    o_full = host(_run(q, k, v, 256, None, Sa))
    p1 = [x[:, :, :m].contiguous() for x in (q, k, v)]
    p2 = [x[:, :, m:].contiguous() for x in (q, k, v)]
    o1 = host(_run(*p1, 256, None, S1))
    o2 = host(_run(*p2, 256, S1, Sb))
    ref = oracle.causal_linear_attention(host(q), host(k), host(v), "recurrent")
    oo = np.concatenate([o1, o2], axis=2)
    assert oracle.rel_err(oo, ref) <= TOL["bf16"]
    assert oracle.rel_err(oo, o_full) <= TOL["bf16"]
    assert oracle.rel_err(host(Sb), host(Sa)) <= STOL


def test_prefill_hands_state_to_decode(dev):
    """Prefill n tokens, then decode token n from the returned state: the
    decode output plus the token's own term (q.k) v equals the (n+1)-token
    prefill's last row."""
    import torch
    import linear_attention_attn_amd as la
    note("state prefill -> decode")
    n, d = 777, 128
    q, k, v = randn_qkv((3, 2, n + 1, d), "bf16", 66, dev)
    S = torch.empty((3, 2, d, d), dtype=torch.float32, device=dev)
    _run(*[x[:, :, :n].contiguous() for x in (q, k, v)], 256, None, S)
    qd, kd, vd = (x[:, :, n].contiguous() for x in (q, k, v))
    od = host(la.decode(qd, kd, vd, S))
    torch.cuda.synchronize()
    full = oracle.causal_linear_attention(host(q), host(k), host(v), "recurrent")[:, :, n]
    own = (host(qd) * host(kd)).sum(-1, keepdims=True) * host(vd)
    assert oracle.rel_err(od + own, full) <= TOL["bf16"]

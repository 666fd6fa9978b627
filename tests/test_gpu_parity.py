"""HIP path vs the CPU oracle at small sizes: shapes spanning several tiles,
blocks, chunks and scan tiles with ragged tails; bit-exact integer cases;
invariants (block size, packing, linearity, determinism); decode."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, chunk_tokens, device, host, note, randn_qkv, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


def _fwd(q, k, v, B, cu=None):
    import torch
    import linear_attention_attn_amd as la
    o = la.fwd(q, k, v, block_size=B, cu_seqlens=cu)
    torch.cuda.synchronize()
    return o


# ------------------------------------------------------------ random parity

SWEEP = []
for dt in ("bf16", "f32"):
    for d in (64, 128):
        for B in (64, 128, 256):
            for n in (1, 2, B - 1, B, B + 1, 3 * B + 5):
                SWEEP.append((dt, d, B, n))


@pytest.mark.parametrize("dt,d,B,n", SWEEP)
def test_random_small(dev, dt, d, B, n):
    note(f"random_small dt={dt} d={d} B={B} n={n}")
    q, k, v = randn_qkv((2, 3, n, d), dt, 1000 + n + d + B, dev)
    o = host(_fwd(q, k, v, B))
    ref = oracle.causal_linear_attention(host(q), host(k), host(v), "naive")
    err = oracle.rel_err(o, ref)
    assert err <= TOL[dt], err


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,C,S,n", [(64, 64, 0, 64 * 40 + 7), (256, 256, 0, 256 * 34 + 100),
                                     (128, 512, 0, 5000), (256, 1024, 0, 3000),
                                     (64, 256, 64, 64 * 40 + 7), (256, 1024, 256, 256 * 34 + 100),
                                     (128, 2048, 512, 5000), (64, 192, 64, 64 * 40 + 7),
                                     (128, 640, 128, 9000)])
def test_multi_chunk_and_scan_tiles(dev, dt, d, B, C, S, n):
    """Forced chunk lengths: many chunks per sequence (> 32 runs the tiled scan);
    S > 0 also forces the summary sub-chunk, so a chunk starts from the prefix
    of several sub-chunk summaries.  With 3 and 5 sub-chunks per chunk the
    scan tiles of 32 entries begin inside chunks."""
    note(f"multi_chunk dt={dt} d={d} B={B} C={C} S={S} n={n}")
    q, k, v = randn_qkv((1, 2, n, d), dt, 7 * n + d, dev)
    with chunk_tokens(C, S):
        o = host(_fwd(q, k, v, B))
    ref = oracle.causal_linear_attention(host(q), host(k), host(v), "recurrent")
    assert oracle.rel_err(o, ref) <= TOL[dt]


# ------------------------------------------------------------- exact cases

def _onehot_inputs(rng, shape):
    """Rows with one nonzero entry of random sign: every product and partial sum
    is a small integer, exact in bf16 and fp32."""
    *lead, n, d = shape
    out = []
    for _ in range(3):
        x = np.zeros(shape, np.float32)
        idx = rng.integers(0, d, size=tuple(lead) + (n,))
        sgn = rng.choice([-1.0, 1.0], size=tuple(lead) + (n,))
        np.put_along_axis(x, idx[..., None], sgn[..., None], axis=-1)
        out.append(x)
    return out


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("d,B,n,C,S", [(64, 64, 1500, 0, 0), (128, 256, 3000, 0, 0),
                                       (128, 64, 2600, 64, 0), (64, 128, 4100, 128, 0),
                                       (128, 128, 777, 0, 0), (128, 64, 2600, 512, 64)])
def test_integer_exact(dev, dt, d, B, n, C, S):
    import torch
    note(f"integer_exact dt={dt} d={d} B={B} n={n} C={C} S={S}")
    rng = np.random.default_rng(n + d)
    qh, kh, vh = _onehot_inputs(rng, (2, 2, n, d))
    t = lambda x: torch.from_numpy(x).to(dev).to(torch_dtype(dt))
    with chunk_tokens(C, S):
        o = host(_fwd(t(qh), t(kh), t(vh), B))
    ref = oracle.causal_linear_attention(qh, kh, vh, "naive")
    assert np.max(np.abs(ref)) <= 256
    assert np.array_equal(o.astype(np.float64), ref)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B", [64, 128, 256])
@pytest.mark.parametrize("C", [0, 512])
def test_partial_last_block_exact(dev, dt, d, B, C):
    """Sequences ending on both sides of every 16-row slab and 64-token tile
    edge inside their last block, where the kernel skips the slabs and keys
    past the end and stops after the last tile with tokens (fp32 with d = 64:
    the ring kernel, which stops the same way): integer-exact
    inputs, so o and the final states must equal the oracle bit for bit;
    dense (one length per call) and packed (all lengths in one call), with
    one chunk per sequence (C = 0) and with chunks of 512 tokens."""
    import torch
    import linear_attention_attn_amd as la
    ends = [1, 15, 16, 17, 63, 64, 65, 127, 129, 191, 192, 193, B - 1]
    lengths = [e for e in ends if e < B] + [B + 47, 2 * B + 80, 3 * B - 1]
    rng = np.random.default_rng(d + B + C)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(torch_dtype(dt))
    H = 2
    with chunk_tokens(C):
        for n in lengths:
            note(f"partial last block dense dt={dt} d={d} B={B} C={C} n={n}")
            qh, kh, vh = _onehot_inputs(rng, (1, H, n, d))
            Sf = torch.full((1, H, d, d), float("nan"), device=dev)
            o = host(la.fwd(t(qh), t(kh), t(vh), block_size=B, s_final=Sf))
            ref, sref = oracle.causal_linear_attention_state(qh, kh, vh)
            assert np.array_equal(o.astype(np.float64), ref), n
            assert np.array_equal(host(Sf).astype(np.float64), sref), n
        note(f"partial last block packed dt={dt} d={d} B={B} C={C}")
        cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
        T = int(cu[-1])
        qh, kh, vh = _onehot_inputs(rng, (H, T, d))
        Sf = torch.full((len(lengths), H, d, d), float("nan"), device=dev)
        o = host(la.fwd(t(qh), t(kh), t(vh), block_size=B, cu_seqlens=torch.from_numpy(cu).to(dev),
                        s_final=Sf))
        ref, sref = oracle.causal_linear_attention_varlen_state(qh, kh, vh, cu)
        assert np.array_equal(o.astype(np.float64), ref)
        assert np.array_equal(host(Sf).astype(np.float64), sref)


def test_one_hot_boundaries(dev):
    """k_{j0} = e_a, v_{j0} = e_c, q_i = e_a: o_i = [i >= j0] e_c, at block and
    chunk edges."""
    import torch
    n, d, B = 1100, 128, 256
    for j0 in (0, 255, 256, 511, 512, 1023, 1024, 1099):
        for C, S in ((512, 0), (1024, 256)):
            note(f"one_hot j0={j0} C={C} S={S}")
            q = torch.zeros((1, 1, n, d), dtype=torch.bfloat16, device=dev)
            k = torch.zeros_like(q)
            v = torch.zeros_like(q)
            q[..., 5] = 1
            k[0, 0, j0, 5] = 1
            v[0, 0, j0, 77] = 1
            with chunk_tokens(C, S):
                o = host(_fwd(q, k, v, B))[0, 0]
            expect = np.zeros((n, d), np.float32)
            expect[j0:, 77] = 1
            assert np.array_equal(o, expect), (j0, C, S)


@pytest.mark.parametrize("d,B", [(128, 256), (64, 128)])
def test_long_chunks_three_tiles_in_flight(dev, d, B):
    """Chunks of 131,072 tokens or more run the bf16 fused kernel with three
    K/V tiles in flight instead of two: dense sequences of two such chunks
    and a packed mix with one long sequence, against the oracle."""
    import torch
    n = 131072 + 9001
    note(f"long chunks d={d} B={B} n={n}")
    q, k, v = randn_qkv((1, 2, n, d), "bf16", 4242 + d, dev)
    with chunk_tokens(131072):
        o = host(_fwd(q, k, v, B))
    ref = oracle.causal_linear_attention(host(q), host(k), host(v), "recurrent")
    assert oracle.rel_err(o, ref) <= TOL["bf16"]
    lengths = [150001, 5, 0, 70000]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    q, k, v = randn_qkv((2, int(cu[-1]), d), "bf16", 4343 + d, dev)
    with chunk_tokens(131072):
        o = host(_fwd(q, k, v, B, torch.from_numpy(cu).to(dev)))
    ref = oracle.causal_linear_attention_varlen(host(q), host(k), host(v), cu, "recurrent")
    assert oracle.rel_err(o, ref) <= TOL["bf16"]


# ----------------------------------------------------------------- packing

@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("lengths", [(5, 0, 300, 1, 1024, 777), (0, 0, 2000), (256, 256, 256),
                                     (4097, 1, 63)])
def test_varlen_matches_oracle(dev, dt, lengths):
    import torch
    note(f"varlen dt={dt} lengths={lengths}")
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T, H, d = int(cu[-1]), 3, 128
    q, k, v = randn_qkv((H, T, d), dt, 31 + T, dev)
    cud = torch.from_numpy(cu).to(dev)
    ref = oracle.causal_linear_attention_varlen(host(q), host(k), host(v), cu, "recurrent")
    for C, S in ((0, 0), (256, 0), (1024, 256)):
        with chunk_tokens(C, S):
            o = host(_fwd(q, k, v, 256, cud))
        assert oracle.rel_err(o, ref) <= TOL[dt], (C, S)


@pytest.mark.parametrize("nseq", [4096, 4097])
def test_varlen_many_sequences(dev, nseq):
    """Many short packed sequences (0 to 70 tokens): up to 4096 the fused
    grid takes them longest first, beyond that in their own order."""
    import torch
    note(f"varlen many nseq={nseq}")
    rng = np.random.default_rng(nseq)
    lengths = rng.integers(0, 71, size=nseq)
    lengths[rng.integers(0, nseq, size=50)] = 0
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T, H, d = int(cu[-1]), 2, 64
    q, k, v = randn_qkv((H, T, d), "bf16", nseq, dev)
    cud = torch.from_numpy(cu).to(dev)
    o = host(_fwd(q, k, v, 64, cud))
    ref = oracle.causal_linear_attention_varlen(host(q), host(k), host(v), cu, "recurrent")
    assert oracle.rel_err(o, ref) <= TOL["bf16"]


@pytest.mark.parametrize("cu_h", [[0, 100, 50, 200], [0, 100, 150, 300], [5, 100, 150, 200]])
def test_varlen_malformed_cu_seqlens(dev, cu_h):
    """A decreasing table, one not ending at the token count, one not
    starting at 0: the device check makes the call compute nothing (o keeps
    its contents, nothing is read or written out of bounds), and with
    LA_DEBUG_CHECKS=1 the call reports LA_EINVAL."""
    import os
    import torch
    import linear_attention_attn_amd as la
    note(f"varlen malformed cu={cu_h}")
    T, H, d = 200, 2, 128
    q, k, v = randn_qkv((H, T, d), "bf16", 3, dev)
    cud = torch.tensor(cu_h, dtype=torch.int32, device=dev)
    o = torch.full_like(q, float("nan"))
    la.fwd(q, k, v, 64, cud, out=o)
    torch.cuda.synchronize()
    assert np.isnan(host(o)).all()
    os.environ["LA_DEBUG_CHECKS"] = "1"
    try:
        with pytest.raises(la.LightningAttnError) as ei:
            la.fwd(q, k, v, 64, cud, out=o)
        assert ei.value.status == la.LA_EINVAL
        good = torch.tensor([0, 100, 150, 200], dtype=torch.int32, device=dev)
        o2 = la.fwd(q, k, v, 64, good)                 # a valid table passes the check
        torch.cuda.synchronize()
        ref = oracle.causal_linear_attention_varlen(host(q), host(k), host(v),
                                                    np.array([0, 100, 150, 200]), "recurrent")
        assert oracle.rel_err(host(o2), ref) <= TOL["bf16"]
    finally:
        os.environ.pop("LA_DEBUG_CHECKS", None)


def test_varlen_equals_separate_runs(dev):
    import torch
    lengths = (700, 1, 2500, 256, 0, 1300)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T, H, d = int(cu[-1]), 2, 64
    note("varlen_vs_separate f32")
    q, k, v = randn_qkv((H, T, d), "f32", 77, dev)
    packed = host(_fwd(q, k, v, 128, torch.from_numpy(cu).to(dev)))
    for s, L in enumerate(lengths):
        if L == 0:
            continue
        a, b = cu[s], cu[s + 1]
        sep = host(_fwd(q[None, :, a:b].contiguous(), k[None, :, a:b].contiguous(),
                        v[None, :, a:b].contiguous(), 128))[0]
        assert oracle.rel_err(packed[:, a:b], sep) <= 1e-5, s


# -------------------------------------------------------------- invariants

def test_block_size_invariance(dev):
    note("block_size_invariance")
    q, k, v = randn_qkv((2, 4, 3000, 128), "bf16", 5, dev)
    ref = oracle.causal_linear_attention(host(q), host(k), host(v), "recurrent")
    outs = [host(_fwd(q, k, v, B)) for B in (64, 128, 256)]
    for o in outs:
        assert oracle.rel_err(o, ref) <= TOL["bf16"]
    for o in outs[1:]:
        assert oracle.rel_err(o, outs[0]) <= 2 * TOL["bf16"]


def test_linearity_and_determinism(dev):
    note("linearity_determinism")
    q, k, v = randn_qkv((1, 4, 2000, 128), "bf16", 9, dev)
    a = _fwd(q, k, v, 256)
    b = _fwd(q, k, v, 256)
    assert bool((a == b).all())                  # repeat runs are bitwise identical
    two = _fwd((2 * q.float()).to(q.dtype), k, v, 256)
    assert bool((two == 2 * a).all())            # scaling q by 2 is exact end to end


def test_zero_length_and_tiny(dev):
    import torch
    import linear_attention_attn_amd as la
    note("zero_length")
    q = torch.zeros((1, 2, 0, 64), dtype=torch.bfloat16, device=dev)
    assert la.fwd(q, q, q, 64).shape == q.shape
    q, k, v = randn_qkv((3, 1, 1, 64), "f32", 3, dev)
    o = host(_fwd(q, k, v, 64))
    ref = oracle.causal_linear_attention(host(q), host(k), host(v), "naive")
    assert oracle.rel_err(o, ref) <= 1e-5


# ------------------------------------------------------------------ decode

@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_steps(dev, dt, d):
    import torch
    import linear_attention_attn_amd as la
    note(f"decode dt={dt} d={d}")
    steps, batch, heads = 12, 5, 3
    g = torch.Generator(device=dev)
    g.manual_seed(d)
    S = 0.01 * torch.randn((batch, heads, d, d), generator=g, device=dev)
    S0 = host(S).reshape(batch * heads, d, d)
    qs, ks, vs, os_ = [], [], [], []
    for t in range(steps):
        q, k, v = randn_qkv((batch, heads, d), dt, 100 + t, dev)
        o = la.decode(q, k, v, S)
        qs.append(host(q)); ks.append(host(k)); vs.append(host(v)); os_.append(host(o))
    torch.cuda.synchronize()
    Q = np.stack(qs).reshape(steps, batch * heads, d)
    K = np.stack(ks).reshape(steps, batch * heads, d)
    V = np.stack(vs).reshape(steps, batch * heads, d)
    o_ref, S_ref = oracle.decode(Q, K, V, S0)
    o = np.stack(os_).reshape(steps, batch * heads, d)
    assert oracle.rel_err(o, o_ref) <= TOL[dt]
    assert oracle.rel_err(host(S).reshape(batch * heads, d, d), S_ref) <= 1e-4


def test_decode_continues_prefill(dev):
    """Decode from an empty state reproduces the prefill output minus each
    token's own term: o_prefill[t] = o_decode[t] + (q_t . k_t) v_t."""
    import torch
    import linear_attention_attn_amd as la
    note("decode_vs_prefill")
    n, d = 40, 128
    q, k, v = randn_qkv((1, 2, n, d), "f32", 4, dev)
    pre = host(_fwd(q, k, v, 64))[0]
    S = torch.zeros((1, 2, d, d), device=dev)
    dec = np.stack([host(la.decode(q[:, :, t].contiguous(), k[:, :, t].contiguous(),
                                   v[:, :, t].contiguous(), S))[0] for t in range(n)], axis=1)
    own = np.sum(host(q)[0] * host(k)[0], axis=-1, keepdims=True) * host(v)[0]
    assert oracle.rel_err(dec + own, pre) <= 1e-5

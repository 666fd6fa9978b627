"""Rotary position embedding fused into the prefill and decode kernels
(lightning_attn_fwd_rope, lightning_attn_decode_rope) on the GPU against the
CPU oracle (q and k rotated in float64, then the closed masked form): dense
and packed input, one and many chunks per sequence, position offsets up to
2^30, both bases the wiki page names, state handoff, prefill to decode, and
the full MiniMax layer shape on sampled rows."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, chunk_tokens, device, host, note, randn_qkv

pytestmark = pytest.mark.gpu

# Prefill final states: the rotated keys enter the MFMA products rounded to
# bf16 (the operand type), a relative error of up to 2^-9 per key element
# that the fp32 state sums carry (measured ~7e-4 of max|S|), so they are held
# to the bf16 bar; the plain path's states see exact bf16 inputs instead.
# Decode and the fp32 prefill rotate in fp32 and keep the fp32 state bar.
RSTOL = TOL["bf16"]
STOL = 1e-4


@pytest.fixture(scope="module")
def dev():
    return device()


def _states(shape, seed, dev, scale=0.5):
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return (scale * torch.randn(shape, generator=g, device=dev)).contiguous()


def _i32(x, dev):
    import torch
    return torch.tensor(np.asarray(x, np.int32), dtype=torch.int32, device=dev)


CASES = []
for d in (64, 128):
    for B, n, C, S in ((64, 1, 0, 0), (256, 261, 0, 0), (128, 3 * 128 + 7, 0, 0),
                       (64, 40 * 64 + 9, 128, 0), (256, 9 * 256 + 100, 256, 0),
                       (64, 40 * 64 + 9, 512, 128)):
        CASES.append((d, B, n, C, S))


@pytest.mark.parametrize("d,B,n,C,S", CASES)
@pytest.mark.parametrize("base", [1e4, 1e7])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_rope_prefill_dense(dev, dt, d, B, n, C, S, base):
    """Dense input, zero and nonzero position offsets, initial and final
    states; one chunk, many chunks, chunks of several summary sub-chunks."""
    import torch
    import linear_attention_attn_amd as la
    note(f"rope dense dt={dt} d={d} B={B} n={n} C={C} S={S} base={base}")
    q, k, v = randn_qkv((2, 3, n, d), dt, 7000 + n + d + B, dev)
    off = [0, 123457]
    S0 = _states((2, 3, d, d), 71 + d, dev)
    Sf = torch.empty_like(S0)
    with chunk_tokens(C, S):
        o = la.fwd(q, k, v, block_size=B, rope_dims=d // 2, rope_base=base,
                   pos_offset=_i32(off, dev), s_init=S0, s_final=Sf)
        torch.cuda.synchronize()
    ref, sref = oracle.causal_linear_attention_rope(host(q), host(k), host(v), d // 2, base, off,
                                                    host(S0))
    assert oracle.rel_err(host(o), ref) <= TOL[dt]
    assert oracle.rel_err(host(Sf), sref) <= (RSTOL if dt == "bf16" else STOL)


@pytest.mark.parametrize("C", [0, 256])
def test_rope_without_state_or_offset(dev, C):
    """No initial state, no offsets, no final state: positions start at 0."""
    import torch
    import linear_attention_attn_amd as la
    note(f"rope plain C={C}")
    n, d = 1500, 128
    q, k, v = randn_qkv((2, 2, n, d), "bf16", 515, dev)
    with chunk_tokens(C):
        o = host(la.fwd(q, k, v, block_size=256, rope_dims=64))
        torch.cuda.synchronize()
    ref, _ = oracle.causal_linear_attention_rope(host(q), host(k), host(v), 64, 1e4)
    assert oracle.rel_err(o, ref) <= TOL["bf16"]
    # the rotation is not the identity: plain attention differs clearly
    plain = oracle.causal_linear_attention(host(q), host(k), host(v), "recurrent")
    assert oracle.rel_err(o, plain) > 10 * TOL["bf16"]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_rope_packed(dev, dt, d):
    """Packed sequences (some empty) restart positions at their offsets."""
    import torch
    import linear_attention_attn_amd as la
    lengths = (5, 0, 700, 1, 1300, 0, 257)
    note(f"rope packed dt={dt} d={d} lengths={lengths}")
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T, H = int(cu[-1]), 3
    q, k, v = randn_qkv((H, T, d), dt, 4545 + d, dev)
    off = [3, 0, 1 << 20, 7, 65536, 11, 999999]
    S0 = _states((len(lengths), H, d, d), 4646, dev)
    Sf = torch.full_like(S0, float("nan"))
    with chunk_tokens(256):
        o = la.fwd(q, k, v, block_size=256, cu_seqlens=_i32(cu, dev), rope_dims=d // 2,
                   rope_base=1e7, pos_offset=_i32(off, dev), s_init=S0, s_final=Sf)
        torch.cuda.synchronize()
    ref, sref = oracle.causal_linear_attention_rope_varlen(host(q), host(k), host(v), cu, d // 2,
                                                           1e7, off, host(S0))
    assert oracle.rel_err(host(o), ref) <= TOL[dt]
    assert oracle.rel_err(host(Sf), sref) <= (RSTOL if dt == "bf16" else STOL)
    for s, L in enumerate(lengths):
        if L == 0:
            assert np.array_equal(host(Sf)[s], host(S0)[s])


def test_rope_large_positions(dev):
    """Positions near 2^30: the angle is reduced in fp64 before the sine."""
    import torch
    import linear_attention_attn_amd as la
    note("rope large positions")
    n, d = 600, 128
    q, k, v = randn_qkv((2, 2, n, d), "bf16", 888, dev)
    off = [(1 << 30) - 5, (1 << 31) - n - 1]
    o = host(la.fwd(q, k, v, block_size=256, rope_dims=64, rope_base=1e4, pos_offset=_i32(off, dev)))
    torch.cuda.synchronize()
    ref, _ = oracle.causal_linear_attention_rope(host(q), host(k), host(v), 64, 1e4, off)
    assert oracle.rel_err(o, ref) <= TOL["bf16"]


@pytest.mark.parametrize("d,B", [(64, 64), (128, 256)])
def test_rope_bf16_cancelling_single_token(dev, d, B):
    """One stateless token whose rotated score q~ . k~ nearly cancels (about
    1% of the sum of |q~_a k~_a|): o = (q~ . k~) v is then small against the
    terms of its dot product, and rounding the rotated q and k to bf16 (the
    operands of the bf16 products) moves it by several percent of itself.  The
    kernel must give the closed form on the bf16-rounded rotations, to within
    the bf16 rounding of its score."""
    import torch
    import linear_attention_attn_amd as la
    note(f"rope bf16 cancelling single token d={d} B={B}")
    base, pos = 1e7, 6737632
    rng = np.random.default_rng(7 + d)
    bf = lambda x: torch.tensor(np.asarray(x, np.float32)).bfloat16().float().numpy().astype(np.float64)
    q = bf(rng.standard_normal(d) / 8)
    qr = oracle.rope(q[None], [pos], d // 2, base)[0]
    kr = oracle.rope(rng.standard_normal(d)[None] / 8, [pos], d // 2, base)[0]
    kr = kr - 0.99 * (qr @ kr) / (qr @ qr) * qr
    k = bf(oracle.rope(kr[None], [-pos], d // 2, base)[0])      # rotated back to position 0
    kr = oracle.rope(k[None], [pos], d // 2, base)[0]
    assert abs(qr @ kr) < 0.05 * np.abs(qr * kr).sum()          # the input really cancels
    v = bf(rng.standard_normal(d))
    dev_t = lambda x: torch.tensor(np.asarray(x, np.float32)[None, None, None, :], device=dev).bfloat16()
    o = host(la.fwd(dev_t(q), dev_t(k), dev_t(v), block_size=B, rope_dims=d // 2, rope_base=base,
                    pos_offset=_i32([pos], dev)))[0, 0, 0]
    ref = (bf(qr) @ bf(kr)) * v
    assert oracle.rel_err(o, ref) <= 2.0 ** -7, (oracle.rel_err(o, ref), qr @ kr)


@pytest.mark.parametrize("m", [256, 1000])
def test_rope_split_and_resume(dev, m):
    """Two pieces, the second continued from the first's state at positions
    offset by the first's length, match the one-piece prefill."""
    import torch
    import linear_attention_attn_amd as la
    note(f"rope resume m={m}")
    n, d = 2048, 128
    q, k, v = randn_qkv((2, 2, n, d), "bf16", 56, dev)
    S1 = torch.empty((2, 2, d, d), dtype=torch.float32, device=dev)
    Sa, Sb = torch.empty_like(S1), torch.empty_like(S1)
    o_full = host(la.fwd(q, k, v, rope_dims=64, s_final=Sa))
    p1 = [x[:, :, :m].contiguous() for x in (q, k, v)]
    p2 = [x[:, :, m:].contiguous() for x in (q, k, v)]
    o1 = host(la.fwd(*p1, rope_dims=64, s_final=S1))
    o2 = host(la.fwd(*p2, rope_dims=64, pos_offset=_i32([m, m], dev), s_init=S1, s_final=Sb))
    torch.cuda.synchronize()
    oo = np.concatenate([o1, o2], axis=2)
    ref, _ = oracle.causal_linear_attention_rope(host(q), host(k), host(v), 64, 1e4)
    assert oracle.rel_err(oo, ref) <= TOL["bf16"]
    assert oracle.rel_err(oo, o_full) <= TOL["bf16"]
    assert oracle.rel_err(host(Sb), host(Sa)) <= RSTOL


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_rope_decode(dev, dt, d):
    """Decode steps with rotated q and k against the oracle (dense states)."""
    import torch
    import linear_attention_attn_amd as la
    note(f"rope decode dt={dt} d={d}")
    batch, heads, steps = 5, 3, 6
    S = _states((batch, heads, d, d), 31 + d, dev, scale=0.01)
    S0 = host(S)
    pos0 = np.array([0, 1, 4097, 1 << 20, (1 << 31) - 10], np.int64)
    qs, ks, vs, os_ = [], [], [], []
    for t in range(steps):
        q, k, v = randn_qkv((batch, heads, d), dt, 900 + t, dev)
        o = la.decode_rope(q, k, v, S, _i32(pos0 + t, dev), d // 2, 1e7)
        qs.append(host(q)); ks.append(host(k)); vs.append(host(v)); os_.append(host(o))
    torch.cuda.synchronize()
    units = batch * heads
    Q = np.stack(qs).reshape(steps, units, d)
    K = np.stack(ks).reshape(steps, units, d)
    V = np.stack(vs).reshape(steps, units, d)
    ref, sref = oracle.decode_rope(Q, K, V, S0.reshape(units, d, d), np.repeat(pos0, heads),
                                   d // 2, 1e7)
    tol = TOL[dt]
    assert oracle.rel_err(np.stack(os_).reshape(steps, units, d), ref) <= tol
    assert oracle.rel_err(host(S).reshape(units, d, d), sref) <= STOL


def test_rope_decode_indexed_with_padding(dev):
    """Pool states with padding rows: padding rows give zero and touch nothing."""
    import torch
    import linear_attention_attn_amd as la
    note("rope decode indexed")
    d, heads, nslots = 128, 4, 6
    pool = _states((nslots, heads, d, d), 12, dev, scale=0.01)
    P0 = host(pool)
    slots = np.array([4, -1, 0, 6, 2], np.int32)
    pos = np.array([10, 0, 300000, 5, 77], np.int32)
    q, k, v = randn_qkv((len(slots), heads, d), "bf16", 1212, dev)
    o = host(la.decode_rope(q, k, v, pool, _i32(pos, dev), 64, 1e4, slots=_i32(slots, dev)))
    torch.cuda.synchronize()
    P1 = host(pool)
    for b, sl in enumerate(slots):
        if 0 <= sl < nslots:
            ref, sref = oracle.decode_rope(host(q)[b][None], host(k)[b][None], host(v)[b][None],
                                           P0[sl], np.full(heads, pos[b]), 64, 1e4)
            assert oracle.rel_err(o[b], ref[0]) <= TOL["bf16"]
            assert oracle.rel_err(P1[sl], sref) <= STOL
        else:
            assert not o[b].any()
    for sl in (1, 3, 5):
        assert np.array_equal(P1[sl], P0[sl])


def test_rope_prefill_hands_state_to_decode(dev):
    """Prefill n tokens with rotation, then decode token n at position n: the
    decode output plus the token's own term equals the (n+1)-token row."""
    import torch
    import linear_attention_attn_amd as la
    note("rope prefill -> decode")
    n, d = 777, 128
    q, k, v = randn_qkv((3, 2, n + 1, d), "bf16", 67, dev)
    S = torch.empty((3, 2, d, d), dtype=torch.float32, device=dev)
    off = np.array([0, 50, 1 << 22])
    la.fwd(*[x[:, :, :n].contiguous() for x in (q, k, v)], rope_dims=64, rope_base=1e7,
           pos_offset=_i32(off, dev), s_final=S)
    qd, kd, vd = (x[:, :, n].contiguous() for x in (q, k, v))
    od = host(la.decode_rope(qd, kd, vd, S, _i32(off + n, dev), 64, 1e7))
    torch.cuda.synchronize()
    full, _ = oracle.causal_linear_attention_rope(host(q), host(k), host(v), 64, 1e7, off)
    own = (host(qd) * host(kd)).sum(-1, keepdims=True) * host(vd)   # R_p q . R_p k = q . k
    assert oracle.rel_err(od + own, full[:, :, n]) <= TOL["bf16"]


def test_rope_minimax_layer_sampled(dev):
    """Batch 4, 64 heads, d 128, 8192 tokens, block 256 (the launch the
    benchmark times) with rotation: sampled rows of two heads against the
    oracle's row-wise form."""
    import torch
    import linear_attention_attn_amd as la
    import synth
    note("rope minimax layer 4x64x8192")
    q, k, v = synth.prefill_inputs(4, 64, 8192, 128, "bf16", 1, dev)
    off = np.array([0, 1000, 1 << 20, 12345])
    o = la.fwd(q, k, v, block_size=256, rope_dims=64, rope_base=1e4, pos_offset=_i32(off, dev))
    torch.cuda.synchronize()
    rows = np.array([0, 1, 255, 256, 4095, 4096, 8000, 8191])
    for b, h in ((0, 0), (2, 63)):
        ref = oracle.causal_linear_attention_rope_rows(host(q[b, h]), host(k[b, h]), host(v[b, h]),
                                                       rows, 64, 1e4, int(off[b]))
        got = host(o[b, h])[rows]
        assert oracle.rel_err(got, ref) <= TOL["bf16"]

"""Serving-side pieces on the GPU against the CPU oracle: decode over an
indexed state table with padding rows, and a prefill whose final states seed
pool entries that indexed decode steps then continue."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, device, host, note, randn_qkv

pytestmark = pytest.mark.gpu

STOL = 1e-4


@pytest.fixture(scope="module")
def dev():
    return device()


def _pool(nslots, heads, d, seed, dev):
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    return (0.01 * torch.randn((nslots, heads, d, d), generator=g, device=dev)).contiguous()


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_indexed(dev, dt, d):
    import torch
    import linear_attention_attn_amd as la
    note(f"decode_indexed dt={dt} d={d}")
    nslots, heads = 10, 4
    slots_h = np.array([3, -1, 7, 0, 12, 5, -7, 9], dtype=np.int32)   # -1, 12, -7: padding
    batch = len(slots_h)
    pool = _pool(nslots, heads, d, 11 + d, dev)
    pool0 = host(pool).astype(np.float64)
    slots = torch.tensor(slots_h, device=dev)
    steps = 4
    qs, ks, vs, outs = [], [], [], []
    for t in range(steps):
        q, k, v = randn_qkv((batch, heads, d), dt, 500 + 10 * t + d, dev)
        o = la.decode_indexed(q, k, v, pool, slots)
        torch.cuda.synchronize()
        qs.append(host(q)); ks.append(host(k)); vs.append(host(v)); outs.append(host(o))
    live = [b for b in range(batch) if 0 <= slots_h[b] < nslots]
    pad = [b for b in range(batch) if b not in live]
    q = np.stack(qs)[:, live]; k = np.stack(ks)[:, live]; v = np.stack(vs)[:, live]
    S0 = pool0[slots_h[live]].reshape(len(live) * heads, d, d)
    ref_o, ref_S = oracle.decode(q.reshape(steps, -1, d), k.reshape(steps, -1, d),
                                 v.reshape(steps, -1, d), S0)
    got_o = np.stack(outs)[:, live].reshape(steps, -1, d)
    assert oracle.rel_err(got_o, ref_o) <= TOL[dt]
    got_pool = host(pool)
    assert oracle.rel_err(got_pool[slots_h[live]].reshape(-1, d, d), ref_S) <= STOL
    untouched = [s for s in range(nslots) if s not in set(slots_h[live].tolist())]
    assert np.array_equal(got_pool[untouched], host(_pool(nslots, heads, d, 11 + d, dev))[untouched])
    assert not np.stack(outs)[:, pad].any()


def test_prefill_into_pool_then_indexed_decode(dev):
    """Packed prefill of three sequences returns their states; they go into
    pool entries; a padded batch of indexed decode steps continues them.  The
    decode outputs equal the oracle's continuation of each sequence."""
    import torch
    import linear_attention_attn_amd as la
    note("serving prefill -> pool -> indexed decode")
    heads, d, B = 4, 128, 256
    lengths = (300, 1, 1029)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    q, k, v = randn_qkv((heads, T, d), "bf16", 808, dev)
    Sf = torch.empty((len(lengths), heads, d, d), dtype=torch.float32, device=dev)
    la.fwd(q, k, v, block_size=B, cu_seqlens=torch.tensor(cu, device=dev), s_final=Sf)
    pool = torch.zeros((6, heads, d, d), dtype=torch.float32, device=dev)
    slot_of = [4, 0, 2]
    pool[slot_of] = Sf
    slots = torch.tensor(slot_of + [-1], dtype=torch.int32, device=dev)   # padded to 4 rows
    steps = 3
    outs, qd, kd, vd = [], [], [], []
    for t in range(steps):
        a, b, c = randn_qkv((4, heads, d), "bf16", 900 + t, dev)
        outs.append(host(la.decode_indexed(a, b, c, pool, slots)))
        qd.append(host(a)); kd.append(host(b)); vd.append(host(c))
    torch.cuda.synchronize()
    for i, L in enumerate(lengths):
        x0, x1 = cu[i], cu[i + 1]
        S0 = np.stack([oracle.recurrent_final_state(host(q)[h, x0:x1], host(k)[h, x0:x1],
                                                    host(v)[h, x0:x1])[1] for h in range(heads)])
        ref_o, ref_S = oracle.decode(np.stack(qd)[:, i], np.stack(kd)[:, i], np.stack(vd)[:, i], S0)
        assert oracle.rel_err(np.stack(outs)[:, i], ref_o) <= TOL["bf16"]
        assert oracle.rel_err(host(pool)[slot_of[i]], ref_S) <= STOL
    assert not np.stack(outs)[:, 3].any()


# ------------------------------------------- prefill over an indexed state table

def _prefill_indexed_case(dev, dt, d, C, S, rope):
    import torch
    import linear_attention_attn_amd as la
    from gpu_util import chunk_tokens
    lengths = (700, 0, 5, 1300, 1, 257)
    slots_h = np.array([4, 2, -1, 0, 9, 6], dtype=np.int32)     # -1, 9: stateless (nslots 7)
    nslots, H = 7, 3
    note(f"prefill_indexed dt={dt} d={d} C={C} S={S} rope={rope}")
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    q, k, v = randn_qkv((H, T, d), dt, 900 + d + C, dev)
    pool = _pool(nslots, H, d, 77 + d, dev)
    P0 = host(pool).astype(np.float64)
    off = np.array([0, 5, 1 << 20, 17, 3, 99], np.int32)
    kw = dict(rope_dims=d // 2, rope_base=1e4,
              pos_offset=torch.tensor(off, device=dev)) if rope else {}
    with chunk_tokens(C, S):
        o = la.fwd(q, k, v, block_size=256, cu_seqlens=torch.tensor(cu, device=dev),
                   state_pool=pool, slots=torch.tensor(slots_h, device=dev), **kw)
        torch.cuda.synchronize()
    S0 = np.zeros((len(lengths), H, d, d))
    for s, sl in enumerate(slots_h):
        if 0 <= sl < nslots:
            S0[s] = P0[sl]
    if rope:
        ref, sref = oracle.causal_linear_attention_rope_varlen(host(q), host(k), host(v), cu, d // 2,
                                                               1e4, off, S0)
        stol = TOL["bf16"]            # rotated keys enter the products rounded to bf16
    else:
        ref, sref = oracle.causal_linear_attention_varlen_state(host(q), host(k), host(v), cu, S0)
        stol = STOL
    assert oracle.rel_err(host(o), ref) <= TOL[dt]
    P1 = host(pool)
    touched = set()
    for s, sl in enumerate(slots_h):
        if 0 <= sl < nslots:
            touched.add(int(sl))
            assert oracle.rel_err(P1[sl], sref[s]) <= stol, s
    for sl in range(nslots):
        if sl not in touched:
            assert np.array_equal(P1[sl], P0[sl].astype(np.float32)), sl   # untouched entries


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("C,S", [(0, 0), (256, 0), (512, 256)])
def test_prefill_indexed(dev, dt, d, C, S):
    """Packed prefill starting from pool entries and writing back to them,
    stateless sequences (slot out of range) and an empty sequence; one chunk
    per sequence, many chunks, chunks of several sub-chunks."""
    _prefill_indexed_case(dev, dt, d, C, S, rope=False)


@pytest.mark.parametrize("C,S", [(0, 0), (512, 256)])
def test_prefill_indexed_rope(dev, C, S):
    _prefill_indexed_case(dev, "bf16", 128, C, S, rope=True)


def test_serving_loop_prefill_pieces_and_decode(dev):
    """A serving loop over one pool: prompts prefilled in two pieces (the
    second continuing from the pool entry at continued positions), then
    rotated indexed decode steps; against the oracle over whole sequences."""
    import torch
    import linear_attention_attn_amd as la
    note("serving loop")
    H, d, nslots = 4, 128, 5
    L1, L2, steps = (300, 1000, 17), (200, 5, 600), 3
    slots_h = np.array([3, 0, 4], np.int32)
    n = [a + b + steps for a, b in zip(L1, L2)]
    full = [randn_qkv((H, m, d), "bf16", 40 + i, dev) for i, m in enumerate(n)]
    pool = torch.zeros((nslots, H, d, d), dtype=torch.float32, device=dev)
    slots = torch.tensor(slots_h, device=dev)

    def piece(a, b):
        lens = [b_ - a_ for a_, b_ in zip(a, b)]
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        x = [torch.cat([f[j][:, a[i]:b[i]] for i, f in enumerate(full)], dim=1).contiguous()
             for j in range(3)]
        return x, torch.tensor(cu, device=dev), lens

    outs = []
    z = [0, 0, 0]
    for lo, hi in ((z, list(L1)), (list(L1), [a + b for a, b in zip(L1, L2)])):
        (q, k, v), cu, lens = piece(lo, hi)
        o = la.fwd(q, k, v, cu_seqlens=cu, state_pool=pool, slots=slots, rope_dims=64,
                   rope_base=1e7, pos_offset=torch.tensor(np.array(lo, np.int32), device=dev))
        outs.append((host(o), np.concatenate([[0], np.cumsum(lens)])))
    dec = []
    for t in range(steps):
        pos = [a + b + t for a, b in zip(L1, L2)]
        qd, kd, vd = (torch.stack([f[j][:, pos[i]] for i, f in enumerate(full)]).contiguous()
                      for j in range(3))
        od = la.decode_rope(qd, kd, vd, pool, torch.tensor(np.array(pos, np.int32), device=dev),
                            64, 1e7, slots=slots)
        dec.append((host(od), host(qd), host(kd), host(vd)))
    torch.cuda.synchronize()
    for i in range(3):
        q, k, v = (host(x)[None] for x in full[i])
        ref, sref = oracle.causal_linear_attention_rope(q, k, v, 64, 1e7)
        (o1, c1), (o2, c2) = outs
        got = np.concatenate([o1[:, c1[i]:c1[i + 1]], o2[:, c2[i]:c2[i + 1]]], axis=1)
        assert oracle.rel_err(got, ref[0, :, :L1[i] + L2[i]]) <= TOL["bf16"], i
        for t in range(steps):
            od, qd, kd, vd = dec[t]
            own = (qd[i] * kd[i]).sum(-1, keepdims=True) * vd[i]    # R_p q . R_p k = q . k
            assert oracle.rel_err(od[i] + own, ref[0, :, L1[i] + L2[i] + t]) <= TOL["bf16"], (i, t)
        assert oracle.rel_err(host(pool)[slots_h[i]], sref[0]) <= TOL["bf16"], i

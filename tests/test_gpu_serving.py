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

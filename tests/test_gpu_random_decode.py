"""Randomised parity of the decode step: 120 seeded draws over its options
at once (dtype, head dim, batch and head counts, dense states or a pool with
shuffled and padding slots, the rotary prologue at random positions, one to
four steps), each against the CPU oracle's decode recurrence."""
import numpy as np
import pytest

import oracle
from gpu_util import TOL, device, host, note, randn_qkv

pytestmark = pytest.mark.gpu

STOL = 1e-4


@pytest.fixture(scope="module")
def dev():
    return device()


def _draw(seed):
    r = np.random.default_rng(7000 + seed)
    c = {}
    c["dt"] = "bf16" if r.random() < 0.6 else "f32"
    c["d"] = int(r.choice([64, 128]))
    c["batch"] = int(r.integers(1, 9))
    c["heads"] = int(r.integers(1, 5))
    c["pool"] = bool(r.random() < 0.5)
    c["rope"] = bool(r.random() < 0.4)
    c["base"] = float(r.choice([1e4, 1e7]))
    c["steps"] = int(r.integers(1, 5))
    c["seed"] = seed
    return c


@pytest.mark.parametrize("seed", range(120))
def test_random_decode(dev, seed):
    import torch
    import linear_attention_attn_amd as la
    c = _draw(seed)
    note(f"random decode {c}")
    d, H, nb = c["d"], c["heads"], c["batch"]
    rng = np.random.default_rng(seed)
    if c["pool"]:
        nslots = nb + 3
        sl = rng.permutation(nslots)[:nb].astype(np.int32)
        sl[rng.random(nb) < 0.25] = -1
        slots = torch.tensor(sl, device=dev)
        live = [b for b in range(nb) if sl[b] >= 0]
    else:
        nslots = nb
        sl, slots, live = None, None, list(range(nb))
    S = torch.tensor(0.3 * rng.standard_normal((nslots, H, d, d)), dtype=torch.float32, device=dev)
    S0 = host(S).astype(np.float64)
    pos = rng.integers(0, 1 << 24, size=nb).astype(np.int32) if c["rope"] else None
    qs, ks, vs, outs = [], [], [], []
    for t in range(c["steps"]):
        q, k, v = randn_qkv((nb, H, d), c["dt"], 900 + 7 * seed + t, dev)
        if c["rope"]:
            o = la.decode_rope(q, k, v, S, torch.tensor(pos + t, device=dev), d // 2, c["base"], slots=slots)
        elif c["pool"]:
            o = la.decode_indexed(q, k, v, S, slots)
        else:
            o = la.decode(q, k, v, S)
        torch.cuda.synchronize()
        qs.append(host(q)); ks.append(host(k)); vs.append(host(v)); outs.append(host(o))
    outs = np.stack(outs)
    pad = [b for b in range(nb) if b not in live]
    assert not outs[:, pad].any()
    if not live:
        assert np.array_equal(host(S), S0.astype(np.float32))
        return
    st = c["steps"]
    q = np.stack(qs)[:, live].reshape(st, -1, d)
    k = np.stack(ks)[:, live].reshape(st, -1, d)
    v = np.stack(vs)[:, live].reshape(st, -1, d)
    rows = np.asarray(sl[live] if c["pool"] else live)
    S0u = S0[rows].reshape(-1, d, d)
    if c["rope"]:
        upos = np.repeat(pos[live], H)                     # unit (row, head) -> its row's position
        ref_o, ref_S = oracle.decode_rope(q, k, v, S0u, upos, d // 2, c["base"])
    else:
        ref_o, ref_S = oracle.decode(q, k, v, S0u)
    assert oracle.rel_err(outs[:, live].reshape(st, -1, d), ref_o) <= TOL[c["dt"]]
    got = host(S)
    assert oracle.rel_err(got[rows].reshape(-1, d, d), ref_S) <= STOL
    untouched = [x for x in range(nslots) if x not in set(rows.tolist())]
    assert np.array_equal(got[untouched], S0[untouched].astype(np.float32))

"""The torch conveniences of the binding check every tensor before the
library is called (no GPU needed): host tensors, strided views, a dtype or
shape that does not match q, and misplaced optional arguments all raise
ValueError.  The library's loader is replaced by one that fails, so a check
that let an argument through would show up as a different error."""
import pytest
import torch

import linear_attention_attn_amd as la


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    def refuse():
        raise AssertionError("the library was called")
    monkeypatch.setattr(la, "load_library", refuse)


def _qkv(shape=(2, 3, 40, 64), dtype=torch.bfloat16):
    return [torch.zeros(shape, dtype=dtype) for _ in range(3)]


def test_host_tensors_rejected():
    q, k, v = _qkv()
    with pytest.raises(ValueError, match="device"):
        la.fwd(q, k, v)
    qd, kd, vd = _qkv((2, 3, 64))
    with pytest.raises(ValueError, match="device"):
        la.decode(qd, kd, vd, torch.zeros((2, 3, 64, 64)))


@pytest.mark.parametrize("bad", ["k_dtype", "v_shape", "k_strided", "out_dtype", "out_shape",
                                 "s_init_dtype", "s_final_shape", "s_init_strided",
                                 "pos_offset_dtype", "pool_without_slots", "slots_and_state",
                                 "q_dtype", "q_rank", "cu_dtype", "workspace_dtype", "slots_len",
                                 "pool_shape"])
def test_fwd_rejects(bad):
    q, k, v = _qkv()
    kw = {}
    st = torch.zeros((2, 3, 64, 64))
    if bad == "k_dtype":
        k = k.float()
    elif bad == "v_shape":
        v = torch.zeros((2, 3, 41, 64), dtype=torch.bfloat16)
    elif bad == "k_strided":
        k = torch.zeros((2, 3, 64, 40), dtype=torch.bfloat16).transpose(-1, -2)
    elif bad == "out_dtype":
        kw["out"] = torch.zeros(q.shape)
    elif bad == "out_shape":
        kw["out"] = torch.zeros((2, 3, 40, 32), dtype=torch.bfloat16)
    elif bad == "s_init_dtype":
        kw["s_init"] = st.double()
    elif bad == "s_final_shape":
        kw["s_final"] = torch.zeros((2, 3, 64, 32))
    elif bad == "s_init_strided":
        kw["s_init"] = torch.zeros((2, 3, 64, 128))[..., ::2]
    elif bad == "pos_offset_dtype":
        kw.update(rope_dims=32, pos_offset=torch.zeros(2, dtype=torch.int64))
    elif bad == "pool_without_slots":
        kw["state_pool"] = st
    elif bad == "slots_and_state":
        kw.update(state_pool=st, slots=torch.zeros(2, dtype=torch.int32), s_init=st)
    elif bad == "q_dtype":
        q, k, v = _qkv(dtype=torch.float16)
    elif bad == "q_rank":
        q, k, v = _qkv((40, 64))
    elif bad == "cu_dtype":
        q, k, v = _qkv((3, 40, 64))
        kw["cu_seqlens"] = torch.tensor([0, 10, 40])
    elif bad == "workspace_dtype":
        kw["workspace"] = torch.zeros(1024, dtype=torch.float32)
    elif bad == "slots_len":
        kw.update(state_pool=torch.zeros((5, 3, 64, 64)), slots=torch.zeros(3, dtype=torch.int32))
    elif bad == "pool_shape":
        kw.update(state_pool=torch.zeros((5, 2, 64, 64)), slots=torch.zeros(2, dtype=torch.int32))
    with pytest.raises(ValueError):
        la.fwd(q, k, v, **kw)


def test_packed_needs_three_dims():
    q, k, v = _qkv()
    with pytest.raises(ValueError):
        la.fwd(q, k, v, cu_seqlens=torch.tensor([0, 40], dtype=torch.int32))


@pytest.mark.parametrize("bad", ["k_dtype", "v_shape", "q_strided", "state_dtype", "state_shape",
                                 "out_dtype", "state_strided"])
def test_decode_rejects(bad):
    q, k, v = _qkv((2, 3, 64))
    S = torch.zeros((2, 3, 64, 64))
    kw = {}
    if bad == "k_dtype":
        k = k.float()
    elif bad == "v_shape":
        v = torch.zeros((2, 3, 32), dtype=torch.bfloat16)
    elif bad == "q_strided":
        q = torch.zeros((2, 64, 3), dtype=torch.bfloat16).transpose(1, 2)
    elif bad == "state_dtype":
        S = S.double()
    elif bad == "state_shape":
        S = torch.zeros((2, 3, 64, 32))
    elif bad == "out_dtype":
        kw["out"] = torch.zeros((2, 3, 64))
    elif bad == "state_strided":
        S = torch.zeros((2, 3, 64, 128))[..., ::2]
    with pytest.raises(ValueError):
        la.decode(q, k, v, S, **kw)


@pytest.mark.parametrize("bad", ["slots_dtype", "slots_len", "pool_heads", "pool_dtype", "no_slots"])
def test_decode_indexed_rejects(bad):
    q, k, v = _qkv((2, 3, 64))
    pool = torch.zeros((5, 3, 64, 64))
    slots = torch.zeros(2, dtype=torch.int32)
    if bad == "slots_dtype":
        slots = slots.long()
    elif bad == "slots_len":
        slots = torch.zeros(3, dtype=torch.int32)
    elif bad == "pool_heads":
        pool = torch.zeros((5, 4, 64, 64))
    elif bad == "pool_dtype":
        pool = pool.bfloat16()
    elif bad == "no_slots":
        slots = None
    with pytest.raises(ValueError):
        la.decode_indexed(q, k, v, pool, slots)


@pytest.mark.parametrize("bad", ["positions_dtype", "positions_len", "no_positions", "state_shape",
                                 "slots_dtype"])
def test_decode_rope_rejects(bad):
    q, k, v = _qkv((2, 3, 64))
    S = torch.zeros((2, 3, 64, 64))
    pos = torch.zeros(2, dtype=torch.int32)
    kw = {}
    if bad == "positions_dtype":
        pos = pos.long()
    elif bad == "positions_len":
        pos = torch.zeros(5, dtype=torch.int32)
    elif bad == "no_positions":
        pos = None
    elif bad == "state_shape":
        S = torch.zeros((3, 3, 64, 64))
    elif bad == "slots_dtype":
        kw["slots"] = torch.zeros(2, dtype=torch.int64)
    with pytest.raises(ValueError):
        la.decode_rope(q, k, v, S, pos, 32, **kw)

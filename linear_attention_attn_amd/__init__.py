"""Lightning Attention forward pass and decode step on AMD MI355X (gfx950).

A thin ctypes binding over ``liblightning_attn.so``: the functions named like
the C ABI (``lightning_attn_fwd``, ``lightning_attn_decode``, ...) only marshal
arguments; every step of the computation runs in the library's HIP kernels.
``fwd`` and ``decode`` are conveniences that take torch tensors, allocate the
output and workspace with torch and launch on torch's current stream.

The operation (wiki page "MiniMax-01 Lightning Attention", section
"Lightning Attention 设计"; Tencent Cloud article section 4.1):
    o_i = sum_{j<=i} (q_i . k_j) v_j
computed blockwise (left product inside a block, right product with the d x d
prefix state across blocks), and the decode step o = q S ; S += k^T v.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "LA_DTYPE_BF16", "LA_DTYPE_F32", "LA_OK", "LA_EINVAL", "LA_EUNSUPPORTED", "LA_EWORKSPACE",
    "LA_EHIP", "LightningAttnError", "lib_path", "load_library",
    "lightning_attn_fwd_workspace_size", "lightning_attn_fwd_chunk_tokens", "lightning_attn_fwd",
    "lightning_attn_fwd_traced", "lightning_attn_decode", "lightning_attn_strerror", "fwd",
    "decode", "LA_FWD_NUM_EVENTS", "lightning_attn_fwd_state", "lightning_attn_fwd_rope",
    "lightning_attn_decode_indexed", "lightning_attn_decode_rope", "decode_indexed", "decode_rope",
    "lightning_attn_fwd_indexed",
]

LA_DTYPE_BF16 = 0
LA_DTYPE_F32 = 1
LA_OK, LA_EINVAL, LA_EUNSUPPORTED, LA_EWORKSPACE, LA_EHIP = 0, 1, 2, 3, 4
LA_FWD_NUM_EVENTS = 5

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class LightningAttnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lightning_attn_strerror(status)} (status {status})")


def lib_path() -> str:
    """The in-tree library, or the file LIGHTNING_ATTN_LIB names."""
    return os.environ.get("LIGHTNING_ATTN_LIB") or os.path.join(_HERE, "liblightning_attn.so")


def load_library():
    """Load the in-tree HIP library; fails loudly if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m linear_attention_attn_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.lightning_attn_fwd_workspace_size.argtypes = [i32, i32, i64, i32, i32, i32, i32]
    lib.lightning_attn_fwd_workspace_size.restype = sz
    lib.lightning_attn_fwd_chunk_tokens.argtypes = [i32, i32, i64, i32, i32, i32, i32]
    lib.lightning_attn_fwd_chunk_tokens.restype = i64
    lib.lightning_attn_fwd.argtypes = [vp, vp, vp, vp, i32, i32, i64, i32, i32, vp, i32, vp, sz, vp]
    lib.lightning_attn_fwd.restype = i32
    lib.lightning_attn_fwd_state.argtypes = [vp, vp, vp, vp, i32, i32, i64, i32, i32, vp, i32, vp, vp,
                                             vp, sz, vp]
    lib.lightning_attn_fwd_state.restype = i32
    lib.lightning_attn_fwd_traced.argtypes = [vp, vp, vp, vp, i32, i32, i64, i32, i32, vp, i32, vp, sz,
                                              vp, ctypes.POINTER(vp), i32]
    lib.lightning_attn_fwd_traced.restype = i32
    lib.lightning_attn_decode.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, vp]
    lib.lightning_attn_decode.restype = i32
    lib.lightning_attn_decode_indexed.argtypes = [vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, vp]
    lib.lightning_attn_decode_indexed.restype = i32
    lib.lightning_attn_fwd_rope.argtypes = [vp, vp, vp, vp, i32, i32, i64, i32, i32, vp, i32, i32,
                                            ctypes.c_double, vp, vp, vp, vp, sz, vp]
    lib.lightning_attn_fwd_rope.restype = i32
    lib.lightning_attn_fwd_indexed.argtypes = [vp, vp, vp, vp, i32, i32, i64, i32, i32, vp, i32, vp,
                                               i32, vp, i32, ctypes.c_double, vp, vp, sz, vp]
    lib.lightning_attn_fwd_indexed.restype = i32
    lib.lightning_attn_decode_rope.argtypes = [vp, vp, vp, vp, i32, vp, vp, i32, i32, i32, i32, i32,
                                               ctypes.c_double, vp, vp]
    lib.lightning_attn_decode_rope.restype = i32
    lib.lightning_attn_strerror.argtypes = [i32]
    lib.lightning_attn_strerror.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def _ptr(x):
    """Device pointer of a tensor, an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


# ---- the C ABI, same names and argument order -----------------------------

def lightning_attn_fwd_workspace_size(batch, heads, seq_len, head_dim, block_size, varlen, dtype) -> int:
    return int(load_library().lightning_attn_fwd_workspace_size(
        batch, heads, seq_len, head_dim, block_size, int(bool(varlen)), dtype))


def lightning_attn_fwd_chunk_tokens(batch, heads, seq_len, head_dim, block_size, varlen, dtype) -> int:
    return int(load_library().lightning_attn_fwd_chunk_tokens(
        batch, heads, seq_len, head_dim, block_size, int(bool(varlen)), dtype))


def lightning_attn_fwd(q, k, v, o, batch, heads, seq_len, head_dim, block_size, cu_seqlens, dtype,
                       workspace, workspace_bytes, stream) -> int:
    return int(load_library().lightning_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), batch, heads, seq_len, head_dim, block_size,
        _ptr(cu_seqlens), dtype, _ptr(workspace), workspace_bytes, stream))


def lightning_attn_fwd_state(q, k, v, o, batch, heads, seq_len, head_dim, block_size, cu_seqlens,
                             dtype, s_init, s_final, workspace, workspace_bytes, stream) -> int:
    return int(load_library().lightning_attn_fwd_state(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), batch, heads, seq_len, head_dim, block_size,
        _ptr(cu_seqlens), dtype, _ptr(s_init), _ptr(s_final), _ptr(workspace), workspace_bytes,
        stream))


def lightning_attn_fwd_rope(q, k, v, o, batch, heads, seq_len, head_dim, block_size, cu_seqlens,
                            dtype, rope_dims, rope_base, pos_offset, s_init, s_final, workspace,
                            workspace_bytes, stream) -> int:
    return int(load_library().lightning_attn_fwd_rope(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), batch, heads, seq_len, head_dim, block_size,
        _ptr(cu_seqlens), dtype, rope_dims, float(rope_base), _ptr(pos_offset), _ptr(s_init),
        _ptr(s_final), _ptr(workspace), workspace_bytes, stream))


def lightning_attn_fwd_indexed(q, k, v, o, batch, heads, seq_len, head_dim, block_size, cu_seqlens,
                               dtype, state_pool, nslots, slots, rope_dims, rope_base, pos_offset,
                               workspace, workspace_bytes, stream) -> int:
    return int(load_library().lightning_attn_fwd_indexed(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), batch, heads, seq_len, head_dim, block_size,
        _ptr(cu_seqlens), dtype, _ptr(state_pool), nslots, _ptr(slots), rope_dims, float(rope_base),
        _ptr(pos_offset), _ptr(workspace), workspace_bytes, stream))


def lightning_attn_fwd_traced(q, k, v, o, batch, heads, seq_len, head_dim, block_size, cu_seqlens,
                              dtype, workspace, workspace_bytes, stream, events, nevents) -> int:
    arr = (ctypes.c_void_p * max(1, len(events)))(*events) if events is not None else None
    return int(load_library().lightning_attn_fwd_traced(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), batch, heads, seq_len, head_dim, block_size,
        _ptr(cu_seqlens), dtype, _ptr(workspace), workspace_bytes, stream, arr, nevents))


def lightning_attn_decode(q, k, v, state, o, batch, heads, head_dim, dtype, stream) -> int:
    return int(load_library().lightning_attn_decode(
        _ptr(q), _ptr(k), _ptr(v), _ptr(state), _ptr(o), batch, heads, head_dim, dtype, stream))


def lightning_attn_decode_indexed(q, k, v, state_pool, nslots, slots, o, batch, heads, head_dim,
                                  dtype, stream) -> int:
    return int(load_library().lightning_attn_decode_indexed(
        _ptr(q), _ptr(k), _ptr(v), _ptr(state_pool), nslots, _ptr(slots), _ptr(o), batch, heads,
        head_dim, dtype, stream))


def lightning_attn_decode_rope(q, k, v, state, nslots, slots, o, batch, heads, head_dim, dtype,
                               rope_dims, rope_base, positions, stream) -> int:
    return int(load_library().lightning_attn_decode_rope(
        _ptr(q), _ptr(k), _ptr(v), _ptr(state), nslots, _ptr(slots), _ptr(o), batch, heads,
        head_dim, dtype, rope_dims, float(rope_base), _ptr(positions), stream))


def lightning_attn_strerror(status: int) -> str:
    return load_library().lightning_attn_strerror(status).decode()


# ---- torch conveniences -----------------------------------------------------

def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return LA_DTYPE_BF16
    if t.dtype == torch.float32:
        return LA_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream_handle(device):
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def workspace_for(q, block_size: int, cu_seqlens=None):
    """Allocate (with torch) the workspace lightning_attn_fwd needs for q's shape."""
    import torch
    if cu_seqlens is None:
        batch, heads, n, d = q.shape
        nbytes = lightning_attn_fwd_workspace_size(batch, heads, n, d, block_size, 0, _dtype_code(q))
    else:
        heads, n, d = q.shape
        nbytes = lightning_attn_fwd_workspace_size(cu_seqlens.numel() - 1, heads, n, d, block_size, 1,
                                                   _dtype_code(q))
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device), nbytes


def fwd(q, k, v, block_size: int = 256, cu_seqlens=None, out=None, workspace=None,
        s_init=None, s_final=None, rope_dims: int = 0, rope_base: float = 10000.0,
        pos_offset=None, state_pool=None, slots=None):
    """Causal linear attention forward on the current stream.

    Dense: q, k, v [batch, heads, n, d].  Packed: q, k, v [heads, T, d] with
    cu_seqlens an int32 device tensor of nseq+1 offsets.  Returns o (q's dtype).
    s_init / s_final: optional contiguous fp32 device tensors [nseq, heads, d, d]
    (nseq = batch for dense input): the state each sequence starts from, and
    the tensor that receives each sequence's state after its last token (it
    may be s_init itself).
    rope_dims > 0 (= d / 2): q and k rotated on the way in
    (lightning_attn_fwd_rope), token t of sequence s at position
    pos_offset[s] + t (pos_offset: int32 device tensor [nseq], or None for 0).
    state_pool / slots: prefill over an indexed state table
    (lightning_attn_fwd_indexed): sequence s starts from state_pool[slots[s]]
    and its final state is written back there (fp32 [nslots, heads, d, d];
    slots int32 device [nseq]); not combined with s_init / s_final.
    """
    import torch
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous device tensors")
    if not (q.shape == k.shape == v.shape and q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k, v must share shape and dtype")
    o = torch.empty_like(q) if out is None else out
    if workspace is None:
        workspace, nbytes = workspace_for(q, block_size, cu_seqlens)
    else:
        nbytes = workspace.numel() * workspace.element_size()
    if cu_seqlens is None:
        batch, heads, n, d = q.shape
        cu = None
    else:
        if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda:
            raise ValueError("cu_seqlens must be an int32 device tensor")
        heads, n, d = q.shape
        batch = cu_seqlens.numel() - 1
        cu = cu_seqlens
    for x in (s_init, s_final):
        if x is not None and (x.dtype != torch.float32 or not x.is_contiguous() or not x.is_cuda
                              or tuple(x.shape) != (batch, heads, d, d)):
            raise ValueError("s_init / s_final must be contiguous fp32 device tensors [nseq, heads, d, d]")
    if pos_offset is not None and (pos_offset.dtype != torch.int32 or not pos_offset.is_cuda
                                   or pos_offset.numel() != batch):
        raise ValueError("pos_offset must be an int32 device tensor of nseq entries")
    if slots is not None:
        if s_init is not None or s_final is not None:
            raise ValueError("state_pool/slots and s_init/s_final are exclusive")
        if slots.dtype != torch.int32 or not slots.is_cuda or slots.numel() != batch:
            raise ValueError("slots must be an int32 device tensor of nseq entries")
        if (state_pool.dtype != torch.float32 or not state_pool.is_contiguous()
                or tuple(state_pool.shape[1:]) != (heads, d, d)):
            raise ValueError("state_pool must be a contiguous fp32 tensor [nslots, heads, d, d]")
        st = lightning_attn_fwd_indexed(q, k, v, o, batch, heads, n, d, block_size, cu, _dtype_code(q),
                                        state_pool, state_pool.shape[0], slots, rope_dims, rope_base,
                                        pos_offset, workspace if nbytes else None, nbytes,
                                        _stream_handle(q.device))
    elif rope_dims:
        st = lightning_attn_fwd_rope(q, k, v, o, batch, heads, n, d, block_size, cu, _dtype_code(q),
                                     rope_dims, rope_base, pos_offset, s_init, s_final,
                                     workspace if nbytes else None, nbytes, _stream_handle(q.device))
    elif s_init is None and s_final is None:
        st = lightning_attn_fwd(q, k, v, o, batch, heads, n, d, block_size, cu, _dtype_code(q),
                                workspace if nbytes else None, nbytes, _stream_handle(q.device))
    else:
        st = lightning_attn_fwd_state(q, k, v, o, batch, heads, n, d, block_size, cu, _dtype_code(q),
                                      s_init, s_final, workspace if nbytes else None, nbytes,
                                      _stream_handle(q.device))
    if st != LA_OK:
        raise LightningAttnError(st, "lightning_attn_fwd")
    return o


def decode(q, k, v, state, out=None):
    """One decode step: o = q state_old; state += k^T v (in place).

    q, k, v: [batch, heads, d]; state: fp32 [batch, heads, d, d].
    """
    import torch
    if state.dtype != torch.float32 or not state.is_contiguous():
        raise ValueError("state must be a contiguous fp32 tensor")
    batch, heads, d = q.shape
    if tuple(state.shape) != (batch, heads, d, d):
        raise ValueError("state shape must be [batch, heads, d, d]")
    o = torch.empty_like(q) if out is None else out
    st = lightning_attn_decode(q, k, v, state, o, batch, heads, d, _dtype_code(q),
                               _stream_handle(q.device))
    if st != LA_OK:
        raise LightningAttnError(st, "lightning_attn_decode")
    return o


def decode_indexed(q, k, v, state_pool, slots, out=None):
    """One decode step over a pool of states: row b uses state_pool[slots[b]]
    (in place); rows with a slot outside [0, len(state_pool)) are padding
    (o row zero, nothing else touched).

    q, k, v: [batch, heads, d]; state_pool: fp32 [nslots, heads, d, d];
    slots: int32 device tensor [batch].
    """
    import torch
    if state_pool.dtype != torch.float32 or not state_pool.is_contiguous():
        raise ValueError("state_pool must be a contiguous fp32 tensor")
    batch, heads, d = q.shape
    nslots = state_pool.shape[0]
    if tuple(state_pool.shape[1:]) != (heads, d, d):
        raise ValueError("state_pool shape must be [nslots, heads, d, d]")
    if slots.dtype != torch.int32 or not slots.is_cuda or slots.numel() != batch:
        raise ValueError("slots must be an int32 device tensor of batch entries")
    o = torch.empty_like(q) if out is None else out
    st = lightning_attn_decode_indexed(q, k, v, state_pool, nslots, slots, o, batch, heads, d,
                                       _dtype_code(q), _stream_handle(q.device))
    if st != LA_OK:
        raise LightningAttnError(st, "lightning_attn_decode_indexed")
    return o


def decode_rope(q, k, v, state, positions, rope_dims: int, rope_base: float = 10000.0, slots=None,
                out=None):
    """One decode step with q and k rotated at positions[b] (int32 device
    tensor [batch]).  Without slots: state fp32 [batch, heads, d, d]; with
    slots (int32 device [batch]): state is a pool [nslots, heads, d, d] as in
    decode_indexed.
    """
    import torch
    if state.dtype != torch.float32 or not state.is_contiguous():
        raise ValueError("state must be a contiguous fp32 tensor")
    batch, heads, d = q.shape
    if positions.dtype != torch.int32 or not positions.is_cuda or positions.numel() != batch:
        raise ValueError("positions must be an int32 device tensor of batch entries")
    if slots is None:
        if tuple(state.shape) != (batch, heads, d, d):
            raise ValueError("state shape must be [batch, heads, d, d]")
        nslots = 0
    else:
        if tuple(state.shape[1:]) != (heads, d, d):
            raise ValueError("state pool shape must be [nslots, heads, d, d]")
        if slots.dtype != torch.int32 or not slots.is_cuda or slots.numel() != batch:
            raise ValueError("slots must be an int32 device tensor of batch entries")
        nslots = state.shape[0]
    o = torch.empty_like(q) if out is None else out
    st = lightning_attn_decode_rope(q, k, v, state, nslots, slots, o, batch, heads, d,
                                    _dtype_code(q), rope_dims, rope_base, positions,
                                    _stream_handle(q.device))
    if st != LA_OK:
        raise LightningAttnError(st, "lightning_attn_decode_rope")
    return o

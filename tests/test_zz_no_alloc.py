"""lightning_attn_fwd_noalloc (scratch in the library's static device array)
against lightning_attn_fwd (scratch in a caller workspace), through the C
ABI: the same kernels on the same inputs, so the outputs must be equal bit
for bit.  Several calls in a row share the array, each later one on a
smaller input than the one before (packed with short chunks, then dense
with summaries and the scan, then one chunk per sequence, then fp32), so a
table or state left over from an earlier call would show.  A call that needs more scratch than
the array holds is refused before any launch."""
import numpy as np
import pytest

from gpu_util import device, note, randn_qkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


def _pair(la, torch, q, k, v, batch, heads, T, d, B, cu, code, stream):
    varlen = cu is not None
    nbytes = la.lightning_attn_fwd_workspace_size(batch, heads, T, d, B, varlen, code)
    assert 0 < nbytes <= la.LA_NOALLOC_SCRATCH_BYTES
    ws = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    o_ref = torch.full_like(q, float("nan"))
    o = torch.full_like(q, float("nan"))
    assert la.lightning_attn_fwd(q, k, v, o_ref, batch, heads, T, d, B, cu, code, ws, nbytes, stream) == 0
    assert la.lightning_attn_fwd_noalloc(q, k, v, o, batch, heads, T, d, B, cu, code, stream) == 0
    torch.cuda.synchronize()
    a = o_ref.cpu().numpy() if o.dtype == torch.float32 else o_ref.view(torch.int16).cpu().numpy()
    b = o.cpu().numpy() if o.dtype == torch.float32 else o.view(torch.int16).cpu().numpy()
    assert not torch.isnan(o_ref).any()
    assert np.array_equal(a, b)
    return nbytes


def test_noalloc_matches_workspace_calls(dev):
    import torch
    import linear_attention_attn_amd as la
    stream = torch.cuda.current_stream(dev).cuda_stream
    bf16, f32 = la.LA_DTYPE_BF16, la.LA_DTYPE_F32
    sizes = []

    note("noalloc 1: packed 5 sequences x 4 heads, d128")
    lengths = [9000, 0, 17, 4096, 2900]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32), device=dev)
    T = int(sum(lengths))
    q, k, v = randn_qkv((4, T, 128), "bf16", 2, dev)
    sizes.append(_pair(la, torch, q, k, v, len(lengths), 4, T, 128, 128, cu, bf16, stream))
    del q, k, v

    note("noalloc 2: dense 2 x 8 heads x 60000 tokens, d128 (summaries + scan)")
    q, k, v = randn_qkv((2, 8, 60000, 128), "bf16", 1, dev)
    sizes.append(_pair(la, torch, q, k, v, 2, 8, 60000, 128, 256, None, bf16, stream))
    chunk = la.lightning_attn_fwd_chunk_tokens(2, 8, 60000, 128, 256, 0, bf16)
    assert chunk < 60000                              # several chunks per sequence: the scan ran
    del q, k, v

    note("noalloc 3: dense 2 x 4 heads x 3000 tokens, d64 (one chunk per sequence)")
    q, k, v = randn_qkv((2, 4, 3000, 64), "bf16", 3, dev)
    sizes.append(_pair(la, torch, q, k, v, 2, 4, 3000, 64, 64, None, bf16, stream))
    del q, k, v

    note("noalloc 4: dense fp32 1 x 2 heads x 1000 tokens, d64")
    q, k, v = randn_qkv((1, 2, 1000, 64), "f32", 4, dev)
    sizes.append(_pair(la, torch, q, k, v, 1, 2, 1000, 64, 64, None, f32, stream))
    assert sizes == sorted(sizes, reverse=True)     # each call smaller than the one before


def test_noalloc_refuses_oversized_and_bad_arguments(dev):
    import torch
    import linear_attention_attn_amd as la
    stream = torch.cuda.current_stream(dev).cuda_stream
    fake = 1 << 20                                   # never dereferenced: refused on the host
    need = la.lightning_attn_fwd_workspace_size(1, 64, 1 << 20, 128, 256, 0, la.LA_DTYPE_BF16)
    assert need > la.LA_NOALLOC_SCRATCH_BYTES
    assert la.lightning_attn_fwd_noalloc(fake, fake, fake, fake, 1, 64, 1 << 20, 128, 256, None,
                                         la.LA_DTYPE_BF16, stream) == la.LA_ESCRATCH
    assert la.lightning_attn_fwd_noalloc(fake, fake, fake, fake, 1, 1, 10, 96, 256, None,
                                         la.LA_DTYPE_BF16, stream) == la.LA_EUNSUPPORTED
    assert la.lightning_attn_fwd_noalloc(None, None, None, None, 1, 1, 0, 128, 256, None,
                                         la.LA_DTYPE_BF16, stream) == la.LA_OK
    assert la.lightning_attn_fwd_noalloc(None, fake, fake, fake, 1, 1, 10, 128, 256, None,
                                         la.LA_DTYPE_BF16, stream) == la.LA_EINVAL

"""Entry points that must compute exactly what lightning_attn_fwd computes:
the stage-timing variant the benchmark times, and the test entry point with
the library's own chunking (chunk_tokens = sub_tokens = 0).  Both are
compared bit for bit with lightning_attn_fwd on the same inputs, on a shape
of one chunk per sequence and on shapes whose plan runs the summaries and
the scan."""
import ctypes

import numpy as np
import pytest

from gpu_util import device, note, randn_qkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return device()


class _Events:
    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
            out.append(e.value)
        return out

    def ms(self, a, b):
        f = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(f), a, b) == 0
        return f.value

    def destroy(self, evs):
        for e in evs:
            self.lib.hipEventDestroy(e)


@pytest.mark.parametrize("shape,packed", [((2, 4, 3000, 128), False), ((1, 2, 40000, 128), False),
                                          ((1, 3, 70001, 64), False), ((4, 30000, 128), True)])
def test_traced_equals_plain(dev, shape, packed):
    import torch
    import linear_attention_attn_amd as la
    note(f"traced vs plain shape={shape} packed={packed}")
    q, k, v = randn_qkv(shape, "bf16", 11 + shape[-2], dev)
    if packed:
        heads, T, d = shape
        cu = torch.tensor([0, 7, 9000, 9001, 25000, T], dtype=torch.int32, device=dev)
        batch, varlen = cu.numel() - 1, 1
    else:
        batch, heads, T, d = shape
        cu, varlen = None, 0
    code = la.LA_DTYPE_BF16
    nbytes = la.lightning_attn_fwd_workspace_size(batch, heads, T, d, 256, varlen, code)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    o1 = torch.full_like(q, float("nan"))
    o2 = torch.full_like(q, float("nan"))
    o3 = torch.full_like(q, float("nan"))
    assert la.lightning_attn_fwd(q, k, v, o1, batch, heads, T, d, 256, cu, code, ws, nbytes, stream) == 0
    hip = _Events()
    evs = hip.create(la.LA_FWD_NUM_EVENTS)
    assert la.lightning_attn_fwd_traced(q, k, v, o2, batch, heads, T, d, 256, cu, code, ws, nbytes, stream,
                                        evs, la.LA_FWD_NUM_EVENTS) == 0
    # with only the fused kernel bracketed (NULL entries are not recorded)
    o4 = torch.full_like(q, float("nan"))
    part = hip.create(2)
    assert la.lightning_attn_fwd_traced(q, k, v, o4, batch, heads, T, d, 256, cu, code, ws, nbytes, stream,
                                        [None, None, None, part[0], part[1]], la.LA_FWD_NUM_EVENTS) == 0
    wsp = la.lightning_attn_fwd_workspace_size_planned(batch, heads, T, d, 256, varlen, code, 0, 0)
    assert wsp == nbytes
    assert la.lightning_attn_fwd_planned(q, k, v, o3, batch, heads, T, d, 256, cu, code, None, None, None, 0,
                                         None, 0, 1e4, None, 0, 0, ws, nbytes, stream) == 0
    torch.cuda.synchronize()
    stages = [hip.ms(evs[i], evs[i + 1]) for i in range(la.LA_FWD_NUM_EVENTS - 1)]
    total = hip.ms(evs[0], evs[-1])
    assert hip.ms(part[0], part[1]) > 0
    hip.destroy(evs)
    hip.destroy(part)
    chunk = la.lightning_attn_fwd_chunk_tokens(batch, heads, T, d, 256, varlen, code)
    print(f"chunk {chunk} stages {['%.3f' % x for x in stages]} total {total:.3f} ms")
    assert all(x >= 0 for x in stages) and abs(sum(stages) - total) < 1e-3 + 1e-3 * total
    a = o1.view(torch.int16).cpu().numpy()
    assert np.array_equal(a, o2.view(torch.int16).cpu().numpy())
    assert np.array_equal(a, o3.view(torch.int16).cpu().numpy())
    assert np.array_equal(a, o4.view(torch.int16).cpu().numpy())
    assert not torch.isnan(o1).any()

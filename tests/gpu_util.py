"""Helpers for the GPU parity tests (HIP path vs the CPU oracle)."""
import math
import sys

import numpy as np
import pytest

TOL = {"bf16": 1e-2, "f32": 1e-4}


def note(msg):
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    sys.stdout.write(f"[gpu-case] {msg}\n")
    sys.stdout.flush()


def device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    import linear_attention_attn_amd as la
    la.load_library()   # raises if the HIP library is missing: no silent fallback
    return torch.device("cuda:0")


def torch_dtype(name):
    import torch
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def randn_qkv(shape, dtype, seed, dev):
    """q, k ~ N(0,1)/sqrt(d), v ~ N(0,1), rounded to dtype (device tensors)."""
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    d = shape[-1]
    q = (torch.randn(shape, generator=g, device=dev) / math.sqrt(d)).to(torch_dtype(dtype))
    k = (torch.randn(shape, generator=g, device=dev) / math.sqrt(d)).to(torch_dtype(dtype))
    v = torch.randn(shape, generator=g, device=dev).to(torch_dtype(dtype))
    return q, k, v


def host(x):
    import torch
    return x.detach().to("cpu").to(torch.float32).numpy()


class chunk_tokens:
    """Inside the block, ``linear_attention_attn_amd.fwd`` runs with the
    chunking fixed (chunk length n tokens and, optionally, the summary
    sub-chunk length) through the library's test entry point
    lightning_attn_fwd_planned; 0 leaves the library's choice."""

    def __init__(self, n, sub=0):
        self.n, self.sub = n, sub

    def __enter__(self):
        import functools
        import linear_attention_attn_amd as la
        self.orig = la.fwd
        if self.n or self.sub:
            la.fwd = functools.partial(self.orig, chunk_tokens=self.n, sub_tokens=self.sub)
        return self

    def __exit__(self, *a):
        import linear_attention_attn_amd as la
        la.fwd = self.orig

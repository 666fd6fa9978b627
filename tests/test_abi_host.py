"""C-ABI library on the host (no GPU): it loads, exports every declared symbol,
sizes workspaces, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", fn)).read()
            txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
            names += re.findall(r"\b(lightning_attn_\w+)\s*\(", txt)
    return sorted(set(names))


@pytest.fixture(scope="module")
def la():
    import linear_attention_attn_amd as m
    if not os.path.exists(m.lib_path()):
        from linear_attention_attn_amd import build
        build.build()
    m.load_library()
    return m


def test_exports_every_declared_symbol(la):
    names = _declared_functions()
    assert {"lightning_attn_fwd", "lightning_attn_decode", "lightning_attn_fwd_workspace_size",
            "lightning_attn_strerror"} <= set(names)
    lib = ctypes.CDLL(la.lib_path())
    for n in names:
        assert hasattr(lib, n), n


def test_binding_names_match_abi(la):
    for n in _declared_functions():
        assert callable(getattr(la, n)), n


def test_strerror(la):
    assert la.lightning_attn_strerror(la.LA_OK) == "success"
    for s in (la.LA_EINVAL, la.LA_EUNSUPPORTED, la.LA_EWORKSPACE, la.LA_EHIP):
        assert la.lightning_attn_strerror(s) not in ("success", "unknown status")
    assert la.lightning_attn_strerror(99) == "unknown status"


def test_workspace_size(la):
    ws = la.lightning_attn_fwd_workspace_size
    assert ws(1, 1, 0, 128, 256, 0, 0) == 0
    assert ws(1, 1, 100, 96, 256, 0, 0) == 0             # rejected shape
    a = ws(4, 64, 8192, 128, 256, 0, 0)
    assert a > 0 and a % 256 == 0
    # per-chunk fp32 d x d states dominate: at least one per (sequence, head, chunk)
    C = la.lightning_attn_fwd_chunk_tokens(4, 64, 8192, 128, 256, 0, 0)
    assert C % 256 == 0 and C >= 256
    assert a >= 4 * 64 * (8192 // C) * 128 * 128 * 4
    # packed layout needs room for the worst-case chunk count
    b = ws(16, 64, 368523, 128, 256, 1, 0)
    C = la.lightning_attn_fwd_chunk_tokens(16, 64, 368523, 128, 256, 1, 0)
    assert b >= 64 * (368523 // C + 16) * 128 * 128 * 4


@pytest.mark.parametrize("args,expect", [
    # (batch, heads, seq_len, head_dim, block_size, dtype)
    ((1, 1, 10, 96, 64, 0), 2),       # head_dim unsupported
    ((1, 1, 10, 64, 100, 0), 2),      # block_size unsupported
    ((1, 1, 10, 64, 64, 7), 2),       # dtype unknown
    ((0, 1, 10, 64, 64, 0), 1),       # batch < 1
    ((1, 0, 10, 64, 64, 0), 1),       # heads < 1
    ((1, 1, -1, 64, 64, 0), 1),       # negative length
])
def test_fwd_rejects_shapes(la, args, expect):
    b, h, n, d, B, dt = args
    assert la.lightning_attn_fwd(None, None, None, None, b, h, n, d, B, None, dt, None, 0, None) == expect


def test_fwd_zero_length_is_noop(la):
    assert la.lightning_attn_fwd(None, None, None, None, 1, 1, 0, 64, 64, None, 0, None, 0, None) == 0


def test_fwd_null_pointers_and_workspace(la):
    fake = 1 << 20  # never dereferenced: every check below fails before a launch
    assert la.lightning_attn_fwd(None, fake, fake, fake, 1, 1, 10, 64, 64, None, 0, fake, 1 << 30, None) == 1
    assert la.lightning_attn_fwd(fake, fake, fake, None, 1, 1, 10, 64, 64, None, 0, fake, 1 << 30, None) == 1
    need = la.lightning_attn_fwd_workspace_size(1, 1, 10, 64, 64, 0, 0)
    assert la.lightning_attn_fwd(fake, fake, fake, fake, 1, 1, 10, 64, 64, None, 0, None, need, None) == 3
    assert la.lightning_attn_fwd(fake, fake, fake, fake, 1, 1, 10, 64, 64, None, 0, fake, need - 1, None) == 3
    # misaligned workspace
    assert la.lightning_attn_fwd(fake, fake, fake, fake, 1, 1, 10, 64, 64, None, 0, fake + 8, need, None) == 1


def test_misaligned_pointers_rejected(la):
    """The kernels move 16-byte vectors: misaligned buffers are rejected on
    the host (never launched)."""
    fake = 1 << 20
    need = la.lightning_attn_fwd_workspace_size(1, 1, 10, 64, 64, 0, 0)
    for i in range(4):
        ptrs = [fake] * 4
        ptrs[i] = fake + 2
        assert la.lightning_attn_fwd(*ptrs, 1, 1, 10, 64, 64, None, 0, fake, need, None) == 1, i
    assert la.lightning_attn_fwd(fake, fake, fake, fake, 1, 1, 10, 64, 64, fake + 2, 0, fake, need, None) == 1
    assert la.lightning_attn_decode(fake, fake, fake, fake + 4, fake, 1, 1, 64, 0, None) == 1
    assert la.lightning_attn_decode_indexed(fake, fake, fake, fake + 8, 1, fake, fake, 1, 1, 64, 0, None) == 1
    assert la.lightning_attn_decode_rope(fake, fake, fake, fake + 4, 0, None, fake, 1, 1, 128, 0, 64, 1e4,
                                         fake, None) == 1
    assert la.lightning_attn_decode_rope(fake, fake, fake, fake, 0, None, fake, 1, 1, 128, 0, 64, 1e4,
                                         fake + 1, None) == 1


def test_decode_rejects(la):
    fake = 1 << 20
    assert la.lightning_attn_decode(fake, fake, fake, fake, fake, 1, 1, 96, 0, None) == 2
    assert la.lightning_attn_decode(fake, fake, fake, fake, fake, 1, 1, 64, 3, None) == 2
    assert la.lightning_attn_decode(fake, fake, fake, fake, fake, 0, 1, 64, 0, None) == 1
    assert la.lightning_attn_decode(fake, fake, fake, None, fake, 1, 1, 64, 0, None) == 1


def test_launch_grid_limits(la):
    """Shapes whose launches would exceed 2^32 - 1 work-items along the grid's
    x axis are refused on the host as unsupported, not left to fail at launch."""
    fake = 1 << 20
    # decode: one 256-thread workgroup per (row, head)
    assert la.lightning_attn_decode(fake, fake, fake, fake, fake, 1 << 24, 1, 64, 0, None) == 2
    assert la.lightning_attn_decode(fake, fake, fake, fake, fake, 1 << 23, 2, 64, 0, None) == 2
    assert la.lightning_attn_decode_indexed(fake, fake, fake, fake, 1, fake, fake, 1 << 24, 1, 64, 0,
                                            None) == 2
    assert la.lightning_attn_decode_rope(fake, fake, fake, fake, 0, None, fake, 1 << 24, 1, 64, 0, 32, 1e4,
                                         fake, None) == 2
    # prefill: one fused workgroup (up to 1024 threads) per chunk; 2^22
    # one-chunk sequences is the first count past the limit
    assert la.lightning_attn_fwd_workspace_size((1 << 22) - 1, 1, 64, 64, 64, 0, 0) > 0
    assert la.lightning_attn_fwd_workspace_size(1 << 22, 1, 64, 64, 64, 0, 0) == 0
    need = la.lightning_attn_fwd_workspace_size(1, 1, 10, 64, 64, 0, 0)
    assert la.lightning_attn_fwd(fake, fake, fake, fake, 1 << 22, 1, 64, 64, 64, None, 0, fake, need,
                                 None) == 2


def test_rope_rejects(la):
    """Rotary arguments are checked on the host before any launch."""
    fake = 1 << 20
    need = la.lightning_attn_fwd_workspace_size(1, 1, 10, 128, 64, 0, 0)

    def fr(d, dt, r, base):
        return la.lightning_attn_fwd_rope(fake, fake, fake, fake, 1, 1, 10, d, 64, None, dt, r, base,
                                          None, None, None, fake, need, None)
    assert fr(128, 3, 64, 1e4) == 2          # unknown dtype
    assert fr(128, 0, 32, 1e4) == 2          # only half the head dims
    assert fr(128, 0, 128, 1e4) == 2
    assert fr(128, 0, 0, 1e4) == 2           # the rotary entry point needs rope_dims > 0
    assert fr(128, 0, 64, 0.0) == 1          # base must be positive and finite
    assert fr(128, 0, 64, -2.0) == 1
    assert fr(128, 0, 64, float("inf")) == 1
    assert fr(128, 0, 64, float("nan")) == 1

    def dr(d, dt, r, base, pos=fake, state=fake, slots=None, nslots=0):
        return la.lightning_attn_decode_rope(fake, fake, fake, state, nslots, slots, fake, 1, 1, d, dt,
                                             r, base, pos, None)
    assert dr(128, 0, 32, 1e4) == 2
    assert dr(64, 0, 64, 1e4) == 2
    assert dr(128, 0, 64, 0.0) == 1
    assert dr(128, 0, 64, 1e4, pos=None) == 1      # positions are required
    assert dr(128, 0, 64, 1e4, state=None) == 1    # dense states are required
    assert dr(128, 0, 64, 1e4, state=None, slots=fake, nslots=2) == 1
    assert dr(128, 5, 64, 1e4) == 2


def test_fwd_indexed_rejects(la):
    """The indexed prefill's own arguments are checked before any launch."""
    fake = 1 << 20
    need = la.lightning_attn_fwd_workspace_size(2, 1, 10, 128, 64, 1, 0)

    def fi(pool=fake, nslots=3, slots=fake, dt=0, r=0, base=1e4):
        return la.lightning_attn_fwd_indexed(fake, fake, fake, fake, 2, 1, 10, 128, 64, fake, dt, pool,
                                             nslots, slots, r, base, None, fake, need, None)
    assert fi(slots=None) == 1               # the slot table is required
    assert fi(nslots=-1) == 1
    assert fi(pool=None) == 1                # a pool is needed when it has entries
    assert fi(dt=3, r=64) == 2               # unknown dtype
    assert fi(r=32) == 2                     # rotation: half the head dims only
    assert fi(r=64, base=0.0) == 1
    assert fi(pool=fake + 4) == 1            # 16-byte alignment
    assert la.lightning_attn_fwd_indexed(fake, fake, fake, fake, 2, 1, 0, 128, 64, fake, 0, None, 0, fake,
                                         0, 1e4, None, None, 0, None) == 0   # no tokens: nothing to do


def test_planned_overrides(la):
    """The test entry point takes a chunking only when it is valid for the
    shape; the size query returns 0 and the call LA_EINVAL otherwise, before
    any launch."""
    wsp = la.lightning_attn_fwd_workspace_size_planned
    # the library's own choice when nothing is forced
    assert wsp(4, 64, 8192, 128, 256, 0, 0, 0, 0) == la.lightning_attn_fwd_workspace_size(4, 64, 8192, 128,
                                                                                          256, 0, 0)
    assert wsp(1, 2, 5000, 64, 128, 0, 0, 512, 0) > 0
    assert wsp(1, 2, 5000, 64, 128, 0, 0, 512, 128) > wsp(1, 2, 5000, 64, 128, 0, 0, 512, 0)
    for C, S in ((500, 0), (64, 0), (512, 96), (512, 384), (16384 + 256, 0), (-256, 0), (512, -128)):
        assert wsp(1, 2, 5000, 64, 128, 0, 0, C, S) == 0, (C, S)
    assert wsp(1, 2, 100000, 64, 128, 1, 0, 32768, 16384) > 0       # multiples of 16384 above it
    assert wsp(1, 2, 100, 64, 128, 0, 0, 512, 384) > 0              # one chunk: sub ignored

    fake = 1 << 20
    need = wsp(1, 2, 5000, 64, 128, 0, 0, 512, 128)

    def fp(C=512, S=128, s_init=None, s_final=None, pool=None, nslots=0, slots=None, r=0, n=5000):
        return la.lightning_attn_fwd_planned(fake, fake, fake, fake, 1, 2, n, 64, 128, None, 0, s_init,
                                             s_final, pool, nslots, slots, r, 1e4, None, C, S, fake,
                                             need, None)
    assert fp(C=500) == 1
    assert fp(S=96) == 1
    assert fp(pool=fake) == 1                          # a pool without a slot table
    assert fp(slots=fake, nslots=2, pool=fake, s_init=fake) == 1   # pool and s_init are exclusive
    assert fp(slots=fake, nslots=2, pool=None) == 1
    assert fp(r=16) == 2
    assert fp(n=0) == 0                                # no tokens: nothing to do


def test_no_plan_knobs_in_environment(monkeypatch, la):
    """The plan does not depend on the caller's environment."""
    base = [la.lightning_attn_fwd_workspace_size(1, 64, 1 << 20, 128, 256, 0, 0),
            la.lightning_attn_fwd_chunk_tokens(1, 64, 1 << 20, 128, 256, 0, 0)]
    for k, v in (("LA_CHUNK_TOKENS", "256"), ("LA_SUB_TOKENS", "256"), ("LA_TARGET_GROUPS", "7")):
        monkeypatch.setenv(k, v)
    assert [la.lightning_attn_fwd_workspace_size(1, 64, 1 << 20, 128, 256, 0, 0),
            la.lightning_attn_fwd_chunk_tokens(1, 64, 1 << 20, 128, 256, 0, 0)] == base
    for f in os.listdir(os.path.join(ROOT, "linear_attention_attn_amd", "csrc")):
        txt = open(os.path.join(ROOT, "linear_attention_attn_amd", "csrc", f)).read()
        for knob in ("LA_CHUNK_TOKENS", "LA_SUB_TOKENS", "LA_TARGET_GROUPS"):
            assert knob not in txt, (f, knob)


def test_noalloc_refuses_on_the_host(la):
    """The allocation-free entry point refuses a call whose scratch would not
    fit its static array, and bad shapes, before touching the GPU."""
    fake = 1 << 20
    assert la.lightning_attn_fwd_workspace_size(1, 64, 1 << 20, 128, 256, 0, 0) > la.LA_NOALLOC_SCRATCH_BYTES
    assert la.lightning_attn_fwd_noalloc(fake, fake, fake, fake, 1, 64, 1 << 20, 128, 256, None, 0,
                                         None) == la.LA_ESCRATCH
    assert la.lightning_attn_fwd_noalloc(fake, fake, fake, fake, 1, 1, 10, 96, 256, None, 0, None) == 2
    assert la.lightning_attn_fwd_noalloc(None, None, None, None, 1, 1, 0, 128, 256, None, 0, None) == 0
    assert la.lightning_attn_strerror(la.LA_ESCRATCH) != "unknown status"


def test_traced_rejects_missing_event_array(la):
    fake = 1 << 20
    need = la.lightning_attn_fwd_workspace_size(1, 1, 10, 64, 64, 0, 0)
    lib = la.load_library()
    assert lib.lightning_attn_fwd_traced(fake, fake, fake, fake, 1, 1, 10, 64, 64, None, 0, fake, need, None,
                                         None, la.LA_FWD_NUM_EVENTS) == 1
    assert la.lightning_attn_fwd_traced(fake, fake, fake, fake, 1, 1, 10, 64, 64, None, 0, fake, need, None,
                                        [None] * 4, 4) == 1


def test_product_never_imports_oracle():
    """The HIP path must not route through the CPU oracle."""
    pkg = os.path.join(ROOT, "linear_attention_attn_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in txt and "from oracle" not in txt, f
                assert "la_oracle" not in txt, f

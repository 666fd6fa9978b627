"""Checks on the gfx950 code the compiler generates for the kernels (CPU only:
hipcc cross-compiles to assembly).

* A vector store of more than 8 bytes must not be followed directly by a
  VALU write of one of its data registers (the hardware needs a wait state in
  between; a missing one made a buffer store pick up new values in some
  lanes).
* The bf16 prefill kernels must not spill to scratch memory.
* Inside the fused kernel's tile loop the compiler must not wait for every
  outstanding vector-memory load (vmcnt(0)) before an LDS read: it does so
  when it loses the alias information that ties an LDS read to one ring
  stage, which stalls the buffer-to-LDS prefetch of the following tiles.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_attention_attn_amd", "csrc")

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not available")


def _asm(src, tmp_path):
    out = tmp_path / (os.path.basename(src) + ".s")
    cmd = ["hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17", "--cuda-device-only", "-S",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-o", str(out), src]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def _instructions(text):
    for line in text.splitlines():
        s = line.split(";")[0].strip()
        if s and not s.startswith(".") and not s.endswith(":"):
            yield s


def _store_hazards(text):
    insts = list(_instructions(text))
    bad = []
    for i, s in enumerate(insts[:-1]):
        m = re.match(r"(buffer|global)_store_dwordx(3|4)\s+(\S+)", s)
        if not m:
            continue
        # data operand: the VGPR range among the operands
        regs = re.findall(r"v\[(\d+):(\d+)\]", s)
        if not regs:
            continue
        lo, hi = int(regs[-1][0]), int(regs[-1][1])
        nxt = insts[i + 1]
        d = re.match(r"v_\S+\s+v\[?(\d+)", nxt)
        if d and lo <= int(d.group(1)) <= hi:
            bad.append((s, nxt))
    return bad


@pytest.mark.parametrize("src", ["la_prefill.hip", "la_decode.hip"])
def test_no_store_data_overwrite(src, tmp_path):
    text = _asm(os.path.join(CSRC, src), tmp_path)
    assert "_store_dwordx" in text
    assert _store_hazards(text) == []


def test_hazard_scan_catches_pattern():
    """The scan itself flags the pattern it is meant to find."""
    sample = "buffer_store_dwordx4 v[0:3], v8, s[4:7], s9 offen\nv_mov_b32_e32 v1, 0\n"
    assert len(_store_hazards(sample)) == 1
    sample_ok = "buffer_store_dwordx4 v[0:3], v8, s[4:7], 0 offen\ns_nop 1\nv_mov_b32_e32 v1, 0\n"
    assert _store_hazards(sample_ok) == []


def test_bf16_prefill_kernels_do_not_spill(tmp_path):
    text = _asm(os.path.join(CSRC, "la_prefill.hip"), tmp_path)
    kernels = re.findall(r"^(_ZN2la1\dk_(?:fused_dma|fused_ring|summary_reg)\w+):", text, re.M)
    assert kernels
    for k in kernels:
        i = text.index(k + ":")
        j = text.index(".Lfunc_end", i)
        body = text[i:j]
        assert "scratch_" not in body, k


def _kernel_bodies(text, pattern):
    for k in re.findall(pattern, text, re.M):
        i = text.index(k + ":")
        j = text.index(".Lfunc_end", i)
        yield k, text[i:j]


def test_fused_kernel_keeps_prefetch_in_flight(tmp_path):
    text = _asm(os.path.join(CSRC, "la_prefill.hip"), tmp_path)
    found = False
    for k, body in _kernel_bodies(text, r"^(_ZN2la11k_fused_dma\w+):"):
        found = True
        insts = list(_instructions(body))
        # the prologue waits once for the chunk's start state; the end of the
        # kernel waits for everything; nothing else may drain the queue
        full = [s for s in insts if re.fullmatch(r"s_waitcnt vmcnt\(0\)", s)]
        assert len(full) <= 1, (k, len(full))
    assert found


def test_fp32_ring_kernel_keeps_prefetch_in_flight(tmp_path):
    """The fp32 ring kernel waits for everything only in its prologue (the
    chunk's start state and first Q, before its first barrier) and at its
    end."""
    text = _asm(os.path.join(CSRC, "la_prefill.hip"), tmp_path)
    found = False
    for k, body in _kernel_bodies(text, r"^(_ZN2la12k_fused_ring\w+):"):
        found = True
        insts = list(_instructions(body))
        first_barrier = next(i for i, s in enumerate(insts) if s == "s_barrier")
        late = [s for s in insts[first_barrier:] if re.fullmatch(r"s_waitcnt vmcnt\(0\)", s)]
        assert late == [], (k, len(late))
    assert found

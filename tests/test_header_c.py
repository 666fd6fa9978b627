"""The public header is plain C: a C99 translation unit that includes it,
takes the address of every declared entry point and calls the host-only
queries (workspace size, chunk length, status text, argument rejection)
compiles with gcc -std=c99 -Wall -Wextra -Werror -pedantic, links against
liblightning_attn.so and runs without a GPU."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "lightning_attn.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(lightning_attn_\w+)\s*\(", txt)))


def test_header_compiles_and_links_as_c99(tmp_path):
    import linear_attention_attn_amd as la
    if not os.path.exists(la.lib_path()):
        from linear_attention_attn_amd import build
        build.build()
    names = _declared()
    assert len(names) >= 14
    src = tmp_path / "abi_c.c"
    lines = ['#include "lightning_attn.h"', "#include <stdio.h>", "#include <string.h>", "",
             "typedef void (*any_fn)(void);", "", "int main(void) {", "    any_fn fns[] = {"]
    lines += [f"        (any_fn)&{n}," for n in names]
    lines += ["    };",
              "    size_t i, ws;",
              "    for (i = 0; i < sizeof fns / sizeof fns[0]; ++i)",
              "        if (!fns[i]) return 10;",
              "    ws = lightning_attn_fwd_workspace_size(1, 1, 10, 64, 64, 0, LA_DTYPE_BF16);",
              "    if (ws == 0 || ws % 256 != 0) return 11;",
              "    if (lightning_attn_fwd_workspace_size(1, 1, 10, 96, 64, 0, LA_DTYPE_BF16) != 0) return 12;",
              "    if (lightning_attn_fwd_chunk_tokens(1, 1, 10, 64, 64, 0, LA_DTYPE_F32) % 64 != 0) return 13;",
              "    if (lightning_attn_fwd(NULL, NULL, NULL, NULL, 1, 1, 10, 96, 64, NULL, 0, NULL, 0, NULL)",
              "        != LA_EUNSUPPORTED) return 14;",
              "    if (lightning_attn_decode(NULL, NULL, NULL, NULL, NULL, 0, 1, 64, 0, NULL) != LA_EINVAL) return 15;",
              "    if (strlen(lightning_attn_strerror(LA_EWORKSPACE)) == 0) return 16;",
              '    printf("%zu %s\\n", ws, lightning_attn_strerror(LA_OK));',
              "    return 0;",
              "}"]
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "abi_c"
    libdir = os.path.dirname(la.lib_path())
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
           "-L", libdir, "-llightning_attn", f"-Wl,-rpath,{libdir}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert r.stdout.split()[1] == "success"

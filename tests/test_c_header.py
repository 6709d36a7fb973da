"""include/dg.h is a plain C header: a C99 translation unit that includes it
and takes the address of every function it declares compiles with gcc
-Wall -Werror -pedantic, and links against the built libdg.so, so the
header's names and the library's exports agree from C as well as from the
ctypes binding (CPU only; nothing is called)."""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dg.h")
LIB_DIR = os.path.join(ROOT, "fp8_block_scaled_nt_amd")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_\w+)\s*\(", text)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_header_compiles_and_links_as_c(tmp_path):
    names = declared_functions()
    assert "dg_fp8_gemm_nt" in names and "dg_fp8_gemm_nt_noalloc" in names
    src = tmp_path / "use_dg.c"
    body = "\n".join(f"    (fn)&{n}," for n in names)
    src.write_text('#include "dg.h"\n#include <stdio.h>\n\n'
                   "typedef void (*fn)(void);\n"
                   "static const fn table[] = {\n" + body + "\n};\n\n"
                   "int main(void) {\n"
                   "    printf(\"%d\\n\", (int)(sizeof(table) / sizeof(table[0])));\n"
                   "    return DG_OK;\n"
                   "}\n")
    obj = tmp_path / "use_dg.o"
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"), "-c", str(src), "-o", str(obj)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    if not os.path.exists(os.path.join(LIB_DIR, "libdg.so")):
        pytest.skip("libdg.so is not built")
    exe = tmp_path / "use_dg"
    r = subprocess.run(["gcc", str(obj), "-L", LIB_DIR, "-ldg", "-Wl,--unresolved-symbols=ignore-in-shared-libs",
                        "-o", str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr

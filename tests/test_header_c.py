"""include/convrot.h is a C header: it must compile as strict C99 and as C++
with every warning an error, so that callers in either language can use the
ABI as declared.  No GPU."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")

PROGRAM = """
#include "convrot.h"
/* every declared type and a few calls' types, so that a typo in a
   declaration surfaces here */
static convrot_linear_desc d;
static convrot_pre pre;
static convrot_post post;
int probe(void);
int probe(void)
{
    size_t a = convrot_packed_bytes(4, 256);
    size_t b = convrot_workspace_bytes(4, 256, 2);
    const char *s = convrot_status_string(CONVROT_EINVAL);
    d.y_dtype = CONVROT_BF16;
    pre.kind = CONVROT_PRE_NONE;
    post.kind = CONVROT_POST_NONE;
    return (int)(a + b) + (s != 0) + d.y_dtype + pre.kind + post.kind;
}
"""


@pytest.mark.parametrize("lang,std", [("c", "-std=c99"), ("c++", "-std=c++17")])
def test_header_compiles(tmp_path, lang, std):
    src = tmp_path / ("probe.c" if lang == "c" else "probe.cpp")
    src.write_text(PROGRAM)
    cc = "gcc" if lang == "c" else "g++"
    r = subprocess.run([cc, std, "-Wall", "-Wextra", "-pedantic", "-Werror", "-fsyntax-only",
                        "-I", INCLUDE, str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr

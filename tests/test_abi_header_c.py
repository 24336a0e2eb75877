"""The boundary is a C ABI: include/oscar.h compiles as strict C99 (and as
C++), and every entry point it declares can be taken as a function pointer of
the declared type -- a plain C caller needs nothing else."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "oscar.h")


def _entry_points():
    return sorted(set(re.findall(r"\b(oscar_[a-z_]+)\s*\(", open(HEADER).read())))


@pytest.mark.parametrize("compiler,std", [("gcc", "-std=c99"), ("g++", "-std=c++17")])
def test_header_is_plain_c(tmp_path, compiler, std):
    if shutil.which(compiler) is None:
        pytest.skip("needs " + compiler)
    names = _entry_points()
    assert len(names) >= 10
    src = tmp_path / ("use.c" if compiler == "gcc" else "use.cpp")
    body = "\n".join("    (void)&%s;" % n for n in names)
    src.write_text('#include "oscar.h"\nint main(void) {\n%s\n    return 0;\n}\n' % body)
    r = subprocess.run([compiler, std, "-pedantic", "-Wall", "-Wextra", "-Werror", "-fsyntax-only",
                        "-I", os.path.join(ROOT, "include"), str(src)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr

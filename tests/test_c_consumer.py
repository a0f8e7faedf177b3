"""The C ABI from C: include/nvfp4.h compiles as strict C99 (-Wall -Wextra -Werror -pedantic), and a C
program links libnvfp4.so and calls its entry points (host-side validation and the device check only:
nothing is launched)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c", "abi_consumer.c")
LIBDIR = os.path.join(ROOT, "nvfp4_block_scaled_03_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no C compiler")
def test_header_is_c99_and_a_c_program_links(tmp_path):
    exe = str(tmp_path / "abi_consumer")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    SRC, "-o", exe, "-L", LIBDIR, "-lnvfp4", f"-Wl,-rpath,{LIBDIR}"], check=True,
                   capture_output=True, text=True)
    env = dict(os.environ, HIP_VISIBLE_DEVICES="")     # keep any GPU out of it: validation only
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c abi consumer ok" in r.stdout

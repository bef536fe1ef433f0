"""include/kvq.h from plain C and C++ (CPU).

tests/c/abi_host.c is compiled as C99 with -Wall -Wextra -pedantic -Werror,
linked against libkvq.so and run: it takes the address of every entry point
and exercises the host-only calls and host validation (no GPU needed).  The
same file must also compile as C++ (the header's extern "C" block)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c", "abi_host.c")
PKG = os.path.join(ROOT, "quantized_decode_attention_calibrate_amd")


@pytest.fixture(scope="module")
def built():
    from quantized_decode_attention_calibrate_amd import build as kbuild
    if kbuild.is_stale():
        kbuild.build(verbose=False)
    return kbuild.LIB


def test_header_is_c99_and_links(built, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "abi_host")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
                    SRC, "-o", exe, "-L", PKG, "-l:libkvq.so", f"-Wl,-rpath,{PKG}", "-lm"], check=True,
                   capture_output=True, text=True, timeout=120)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "c client: ok", r.stdout + r.stderr


def test_header_compiles_as_cpp(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    subprocess.run(["g++", "-std=c++11", "-Wall", "-Wextra", "-Werror", "-fsyntax-only", "-x", "c++",
                    "-I", os.path.join(ROOT, "include"), SRC], check=True, capture_output=True, text=True,
                   timeout=120)

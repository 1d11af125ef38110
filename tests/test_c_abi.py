"""The C ABI used from plain C: tests/c_abi/abi_chain.c drives one layer of
emulated ranks (pack -> route -> attention -> route -> unpack) through
include/ulysses.h with HIP runtime calls for memory, and checks every pack
bit for bit against the oracle's and the layer's output against the oracle's
unsharded attention (max-abs 2e-2).  The CPU test compiles and links it (the
header is valid C, every symbol it uses resolves); the GPU tests run it."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi", "abi_chain.c")
LIB_DIR = os.path.join(ROOT, "ulysses_head_sharded_amd")
ORC_DIR = os.path.join(ROOT, "oracle")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def compile_chain(out_dir) -> str:
    if not os.path.exists(os.path.join(LIB_DIR, "libulysses.so")):
        pytest.fail("libulysses.so is missing: build it with __graft_entry__.build()")
    if not os.path.exists(os.path.join(ORC_DIR, "libulys_oracle.so")):
        import oracle
        oracle.build()
    cc = shutil.which("gcc") or shutil.which("cc")
    assert cc, "no C compiler"
    exe = os.path.join(str(out_dir), "abi_chain")
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
           "-L", LIB_DIR, "-lulysses", "-L", ORC_DIR, "-lulys_oracle",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           f"-Wl,-rpath,{LIB_DIR}:{ORC_DIR}:{os.path.join(ROCM, 'lib')}", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def test_c_program_compiles_and_links(tmp_path):
    compile_chain(tmp_path)


@pytest.mark.gpu
@pytest.mark.parametrize("args", [
    ("512", "2", "8", "4", "128", "4", "1"),    # bf16 MFMA path, GQA 2:1, causal
    ("384", "1", "4", "2", "64", "2", "0"),     # d_h = 64, dense
], ids=["gqa-causal-d128", "dense-d64"])
def test_c_program_runs_the_layer(tmp_path, args):
    exe = compile_chain(tmp_path)
    print("case abi_chain", " ".join(args), flush=True)
    r = subprocess.run([exe, *args], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_chain: ok" in r.stdout

"""The library from a C program with no Python in its process: a causal
paged prefill and a paged decode through the C ABI, device memory through
the HIP runtime's C API, each compared with the fp64 oracle's C library at
the parity bar (tests/c_gpu_consumer.c)."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_c_program_runs_prefill_and_decode_against_the_oracle(tmp_path):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_attention_sinks_attn_amd as sa
    import oracle
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    libdir = os.path.dirname(sa.LIB_PATH)
    oracle_dir = os.path.dirname(oracle.build(force=False))
    exe = str(tmp_path / "c_gpu_consumer")
    build = subprocess.run(
        [cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-D__HIP_PLATFORM_AMD__",
         "-isystem", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
         os.path.join(ROOT, "tests", "c_gpu_consumer.c"), "-o", exe,
         "-L", libdir, "-lsink_attn", "-L", oracle_dir, "-lsink_attn_oracle",
         "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
         f"-Wl,-rpath,{libdir}:{oracle_dir}:{os.path.join(ROCM, 'lib')}"],
        capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    print("[c consumer] running", exe, flush=True)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(run.stdout, flush=True)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "[c consumer] ok" in run.stdout

"""The boundary from C: include/gemm.h compiled as C99 with gcc, a small C
caller (tests/c_abi_check.c) linked against libgemm.so and run without a
GPU. Its output must match what the same calls return through the Python
binding (the struct layout and every value as C sees them)."""
import ctypes
import os
import shutil
import subprocess

import pytest

from fp32_gemm_07_amd import binding

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.fixture(scope="module")
def c_output(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    out = tmp_path_factory.mktemp("cabi") / "c_abi_check"
    libdir = os.path.dirname(binding.LIB_PATH)
    subprocess.check_call(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror",
                           "-D__HIP_PLATFORM_AMD__", "-isystem", os.path.join(ROCM, "include"),
                           "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "c_abi_check.c"),
                           "-o", str(out), "-L", libdir, "-l:libgemm.so",
                           f"-Wl,-rpath,{libdir}"])
    env = dict(os.environ)
    env["LD_LIBRARY_PATH"] = os.path.join(ROCM, "lib") + ":" + env.get("LD_LIBRARY_PATH", "")
    text = subprocess.check_output([str(out)], env=env, timeout=120).decode()
    return [line.split(" ", 1) for line in text.strip().splitlines()]


def lines(c_output, key):
    return [rest for k, rest in c_output if k == key]


def test_plans_and_workspaces_match_binding(c_output):
    rows = lines(c_output, "plan")
    assert len(rows) == 6
    for row in rows:
        M, N, K, st, name, split, chunk, tail, ws, pws = row.split()
        p = binding.gemm_f32_plan(int(M), int(N), int(K))
        assert int(st) == binding.GEMM_OK
        assert name == binding.gemm_kernel_name(p.kernel)
        assert (int(split), int(chunk), int(tail)) == (p.split_k, p.k_chunk, p.split_tail)
        assert int(ws) == binding.gemm_f32_workspace_bytes(int(M), int(N), int(K)) == int(pws)


def test_argument_checks_from_c(c_output):
    want = {"negative": binding.GEMM_ERR_INVALID_DIM, "null": binding.GEMM_ERR_NULL_PTR,
            "alias": binding.GEMM_ERR_ALIAS, "workspace": binding.GEMM_ERR_WORKSPACE,
            "plan_kernel": binding.GEMM_ERR_INVALID_PLAN,
            "plan_tail": binding.GEMM_ERR_INVALID_PLAN,
            "general_ld": binding.GEMM_ERR_INVALID_DIM}
    for key, status in want.items():
        assert lines(c_output, key) == [str(status)], key
    assert lines(c_output, "general_ws") == [
        str(binding.gemm_f32_general_workspace_bytes(1, 1, 256, 256, 8192, 256, 8192))]
    assert lines(c_output, "last_hip_error") == ["0"]


def test_strings_from_c(c_output):
    got = dict(row.split(" ", 1) for row in lines(c_output, "status"))
    for s in range(9):
        assert got[str(s)] == binding.gemm_status_string(s)
    assert lines(c_output, "kernel_auto") == ["auto"]
    assert ctypes.sizeof(binding.gemm_plan_t) == 16

"""The oracle under gcc's AddressSanitizer and UndefinedBehaviorSanitizer:
oracle/sanitize_run.c calls every entry point of oracle/msa_oracle.c on small
ragged inputs (an empty sequence, a partial last block, forced blocks, the
backward with and without a given output, bad arguments); any out-of-bounds
access, leak or undefined operation aborts the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc is not available")
    exe = tmp_path / "sanitize_run"
    cmd = [gcc, "-O1", "-g", "-fopenmp", "-ffp-contract=off", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           os.path.join(ROOT, "oracle", "msa_oracle.c"), os.path.join(ROOT, "oracle", "sanitize_run.c"),
           "-lm", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="2")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "sanitize_run: ok" in r.stdout
    assert "runtime error" not in r.stderr


def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    """The C ABI's host code (argument checks, workspace sizing and chunking, the host contract check)
    built with clang's AddressSanitizer and UndefinedBehaviorSanitizer, driven by tests/abi_sanitize_run.c.
    Only msa_api.hip is instrumented; the kernel files are linked as built.  No call launches a kernel."""
    hipcc = "/opt/rocm/bin/hipcc"
    clang = "/opt/rocm/llvm/bin/clang"
    build_dir = os.path.join(ROOT, "block_sparse_gqa_amd", "_build")
    others = ["index_prefill", "index_decode", "topk_select", "sparse_attn", "attn_prefill", "kv_append",
              "attn_backward", "block_lists", "attn_block_fwd", "ceilings"]
    objs = [os.path.join(build_dir, o + ".o") for o in others]
    if not (os.path.exists(hipcc) and os.path.exists(clang)) or not all(os.path.exists(o) for o in objs):
        pytest.skip("needs hipcc, clang and the in-tree library build")
    san = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all"]
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "block_sparse_gqa_amd", "csrc")]
    api = tmp_path / "msa_api.o"
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops"] + [x for f in san for x in ("-Xarch_host", f)] + inc + \
          ["-c", os.path.join(ROOT, "block_sparse_gqa_amd", "csrc", "msa_api.hip"), "-o", str(api)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    lib = tmp_path / "libmsa_abi_san.so"
    subprocess.run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-fsanitize=address", "-fsanitize=undefined",
                    "-o", str(lib), str(api)] + objs, check=True, capture_output=True, text=True)
    exe = tmp_path / "abi_sanitize_run"
    subprocess.run([clang, "-O1", "-g"] + san + inc +
                   [os.path.join(ROOT, "tests", "abi_sanitize_run.c"), str(lib), "-Wl,-rpath," + str(tmp_path),
                    "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)], check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "abi_sanitize_run: ok" in r.stdout
    assert "runtime error" not in r.stderr

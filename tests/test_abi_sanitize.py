"""The C ABI layer (argument validation, split partitions, workspace sizes) built for the
host with g++ -fsanitize=address,undefined and driven over extreme arguments by
tests/abi_sanitize.cpp, with the HIP launchers replaced by host stubs that write the whole
workspace region the kernels would write.  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ and the HIP runtime headers")
def test_abi_layer_under_address_and_undefined_sanitizers(tmp_path):
    exe = tmp_path / "abi_sanitize"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I" + ROCM_INCLUDE,
           "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "head_attention_fa2_amd", "csrc"),
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           os.path.join(ROOT, "tests", "abi_sanitize.cpp"),
           os.path.join(ROOT, "head_attention_fa2_amd", "csrc", "mha_api.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True)
    # verify_asan_link_order=0: the process may start with other libraries preloaded
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    print(res.stdout[-2000:], res.stderr[-4000:])
    assert res.returncode == 0 and "abi sanitize ok" in res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr

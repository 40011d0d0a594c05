"""Host check of the kernel's LDS layout, tile loader and MFMA operand addressing
(head_attention_fa2_amd/csrc/mha_layout.h), compiled with g++ and run on the CPU."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_layout_exhaustive(tmp_path):
    exe = tmp_path / "layout_check"
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror",
                    "-I" + os.path.join(ROOT, "head_attention_fa2_amd", "csrc"),
                    os.path.join(ROOT, "tests", "layout_check.cpp"), "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True)
    print(res.stdout)
    assert res.returncode == 0 and "layout check ok" in res.stdout
    # every geometry reads K and V^T without bank-group conflicts
    for line in res.stdout.splitlines():
        if line.startswith("R="):
            assert line.endswith("conflicting bank groups 0, V-read conflicting bank groups 0"), line

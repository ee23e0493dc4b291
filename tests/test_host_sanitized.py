"""The library's host logic (pool bookkeeping, dispatch plan, workspace sizes,
argument checks and the DSA_VALIDATE checks of the batch description) built
with g++ under the address and undefined-behaviour sanitizers, without HIP,
and run on the CPU.  Each case of tests/host/host_logic_test.cpp is one test;
a sanitizer report fails it."""

import json
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_09_amd", "csrc")
GOLDEN = os.path.join(ROOT, "tests", "golden")

CASES = ["check_combine_and_append_args", "check_partial_args", "check_select_args",
         "plan_worked_example", "pool_bookkeeping", "validate_accepts_good_batch",
         "validate_page_id_negative", "validate_page_id_past_pool",
         "validate_q_offsets_decreasing", "validate_q_offsets_start_end",
         "validate_tok_pos_negative", "validate_tok_pos_past_page_table",
         "validate_unreached_pages_ignored", "workspace_sizes"]

ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
ENV.pop("DSA_VALIDATE", None)


@pytest.fixture(scope="module")
def binary(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("host") / "host_logic_test")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "host", "host_logic_test.cpp"),
           os.path.join(CSRC, "dsa_host.cpp"), os.path.join(CSRC, "dsa_validate.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    return out


def test_case_list_is_complete(binary):
    r = subprocess.run([binary, "list"], capture_output=True, text=True, env=ENV)
    assert r.returncode == 0
    assert r.stdout.split() == sorted(CASES)


@pytest.mark.parametrize("case", CASES)
def test_host_case(binary, case):
    args = []
    if case == "plan_worked_example":
        # Figure 4 of "Accelerating GLM-5.3-Flash on H200", section 3
        g = json.load(open(os.path.join(GOLDEN, "fig4_virtual_padding.json")))
        args = [str(g["width"])]
        for tile, iters in g["iterations"].items():
            args += [tile, str(iters)]
        args += [str(g["virtual_columns"]["128"]), str(g["padding_columns"]["128"])]
    r = subprocess.run([binary, case, *args], capture_output=True, text=True, env=ENV, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "Sanitizer" not in r.stderr, r.stderr

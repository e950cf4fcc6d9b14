"""The library's host code (encoder and planner, the parser of untrusted
containers) built with AddressSanitizer and UndefinedBehaviorSanitizer and
run over seeded containers of every option the GPU decoder takes and
thousands of corrupted copies of each (tests/sanitize/host_fuzz.cpp).  The
GPU side is replaced by host stand-ins that check every launch's parameters
against the container's bounds (tests/sanitize/kernel_stubs.cpp).  Any
sanitizer report, leak or failed check fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "lossless_entropy_coded_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "sanitize")
HIP_INCLUDE = "/opt/rocm/include"


@pytest.fixture(scope="module")
def host_fuzz(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(HIP_INCLUDE, "hip", "hip_runtime_api.h")):
        pytest.skip("g++ or the HIP headers are missing")
    exe = str(tmp_path_factory.mktemp("sanitize") / "host_fuzz")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I", HIP_INCLUDE, "-I", os.path.join(ROOT, "include"),
           os.path.join(CSRC, "encode.cpp"), os.path.join(CSRC, "plan.cpp"), os.path.join(HERE, "kernel_stubs.cpp"),
           os.path.join(HERE, "host_fuzz.cpp"), "-o", exe, "-lpthread"]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    return exe


def test_host_code_under_asan_and_ubsan(host_fuzz):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([host_fuzz, "1000"], capture_output=True, text=True, timeout=600, env=env)
    report = r.stdout[-2000:] + r.stderr[-4000:]
    assert r.returncode == 0, report
    assert "host_fuzz ok" in r.stdout, report
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, report
    # every path ran: containers written and planned, launches checked, fused launches among them
    line = [s for s in r.stdout.splitlines() if s.startswith("host_fuzz:")][0]
    words = line.split()
    assert int(words[1]) >= 50 and int(words[7]) > 1000 and int(words[10].strip("(")) > 4, line


def test_stand_ins_catch_an_out_of_bounds_launch(host_fuzz, tmp_path):
    """The launch stand-ins are not vacuous: a plan handed a container range
    that excludes its group table aborts in the stand-in's check.  (Built from
    the same sources with one extra test file.)"""
    gxx = shutil.which("g++")
    probe = tmp_path / "probe.cpp"
    probe.write_text(r'''
#include <cstdio>
#include <cstring>
#include <cstdlib>
#include "wc.h"
#include "stub_state.h"
int main() {
    static uint16_t w[5000];
    for (int i = 0; i < 5000; ++i) w[i] = (uint16_t)(0x3C00 + i % 64);
    const uint16_t* ts[1] = {w};
    const uint64_t n[1] = {5000};
    uint8_t* blob = nullptr; uint64_t bytes = 0;
    if (wc_encode_host(ts, n, 1, nullptr, &blob, &bytes)) return 2;
    wc_plan_t* plan = nullptr;
    if (wc_plan(blob, bytes, 0, &plan)) return 3;
    static uint16_t out[5008];
    g_stub.lo = blob + bytes;   // a range that holds none of the container
    g_stub.hi = blob + bytes + 16;
    wc_decode_async(plan, blob, out, nullptr);
    std::puts("not caught");
    return 0;
}
''')
    exe = str(tmp_path / "probe")
    cmd = [gxx, "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I", HIP_INCLUDE, "-I", os.path.join(ROOT, "include"),
           "-I", HERE, os.path.join(CSRC, "encode.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(HERE, "kernel_stubs.cpp"), str(probe), "-o", exe, "-lpthread"]
    subprocess.run(cmd, check=True, capture_output=True, timeout=600)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode != 0 and "stub check failed" in r.stderr, r.stdout + r.stderr

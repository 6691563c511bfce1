"""CPU checks built from C++ on the fly (no GPU):

* the wide row-block reduction's LDS layout (wide_layout.h, the functions the
  kernel computes its offsets with) over every slice count, own slice,
  sequence-half count and operator;
* a ThreadSanitizer build of the protocol emulator: the device's claim, poll
  and publish protocol on 16 threads over a narrow and a matrix-core plan (and
  the fixed-reducer scheme), bitwise equal to the serial executor with no race
  reported -- and, as the positive control, a race reported once one tile's
  dependency edge is dropped.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "persistent_megakernel_latency_amd", "csrc")
INC = os.path.join(ROOT, "include")
NATIVE = os.path.join(ROOT, "tests", "native")


def _build(tmp, name, sources, flags):
    exe = os.path.join(tmp, name)
    cmd = ["g++", "-std=c++17", "-I", CSRC, "-I", INC, *flags, *sources, "-o", exe, "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def test_wide_reduction_lds_layout_is_in_bounds(tmp_path):
    exe = _build(str(tmp_path), "wide_layout_check", [os.path.join(NATIVE, "wide_layout_check.cpp")], ["-O1"])
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout[-3000:]
    assert "0 violations" in r.stdout


@pytest.fixture(scope="module")
def tsan_emulator(tmp_path_factory):
    tmp = str(tmp_path_factory.mktemp("tsan"))
    return _build(tmp, "emulator_tsan",
                  [os.path.join(NATIVE, "emulator_tsan.cpp"), os.path.join(CSRC, "host_exec.cpp"),
                   os.path.join(CSRC, "builder.cpp")],
                  ["-O1", "-g", "-fsanitize=thread", "-DWPK_TSAN_ORDERINGS"])


def test_emulated_protocol_is_race_free_under_thread_sanitizer(tsan_emulator):
    r = subprocess.run([tsan_emulator], capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "ThreadSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-3000:]
    assert out.count(": ok") == 3


def test_thread_sanitizer_sees_a_dropped_dependency_edge(tsan_emulator):
    r = subprocess.run([tsan_emulator, "drop"], capture_output=True, text=True, timeout=600)
    assert "WARNING: ThreadSanitizer: data race" in r.stderr

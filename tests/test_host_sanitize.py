"""The C-ABI validation and split planning of libfa (fa_api.cpp, fa_plan.cpp) built for the host
with AddressSanitizer and UndefinedBehaviorSanitizer, linked with stand-in kernel launchers
(tests/host/launch_stubs.cpp), and driven through every documented error case plus a seeded
sweep of edge-valued parameter blocks (tests/host/sanitize_main.cpp). CPU only."""
import os
import pathlib
import shutil
import subprocess

import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]
CSRC = ROOT / "exact_tiled_attention_39_amd" / "csrc"
FLAGS = ["-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer"]


def _gxx():
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    return gxx


def test_sanitizers_catch_a_planted_overflow(tmp_path):
    src = tmp_path / "planted.cpp"
    src.write_text("#include <climits>\n#include <cstdio>\n"
                   "int main(int c, char**) { volatile int x = INT_MAX - 1 + c; int y = x + 1;\n"
                   "  std::printf(\"%d\\n\", y); return 0; }\n")
    exe = tmp_path / "planted"
    subprocess.run([_gxx(), *FLAGS, str(src), "-o", str(exe)], check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode != 0 and "overflow" in r.stderr


def test_validation_layer_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "sanitize"
    cmd = [_gxx(), *FLAGS, f"-I{ROOT / 'include'}", f"-I{CSRC}",
           str(ROOT / "tests" / "host" / "sanitize_main.cpp"),
           str(ROOT / "tests" / "host" / "launch_stubs.cpp"),
           str(CSRC / "fa_api.cpp"), str(CSRC / "fa_plan.cpp"), "-o", str(exe)]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe), "200000"], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-3000:])
    assert "0 checks failed" in r.stdout

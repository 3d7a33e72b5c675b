"""The library's host code (packer, scale check, shape contract, tile table and
override file) built with AddressSanitizer and UndefinedBehaviorSanitizer and
driven through every entry point, error paths included (CPU only)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "verify_nvfp4_w4a16_amd", "csrc", "host")


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    out = str(tmp_path_factory.mktemp("asan") / "host_check")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-pthread",
           "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "host_check.cpp"),
           os.path.join(HOST, "pack.cpp"), os.path.join(HOST, "tiles.cpp"), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    return out


def _run(exe, env_extra, expect):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("NVFP4_TILES", None)
    env.update(env_extra)
    r = subprocess.run([exe, str(expect)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and "host ok" in r.stdout, (r.stdout[-2000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]


def test_host_code_clean_without_override(sanitized):
    _run(sanitized, {}, 0)


def test_host_code_clean_with_override_files(sanitized, tmp_path):
    good = tmp_path / "good.txt"
    good.write_text("# N K cols waves unroll split mwaves\n4096 4096 32 4 2 2 6  # comment\n\n")
    _run(sanitized, {"NVFP4_TILES": str(good)}, 0)
    for i, text in enumerate(["4096 4096 32 4\n",                 # too few fields
                              "4096 4096 48 4 2\n",               # cols not allowed
                              "4096 4096 16 8 2 3\n",             # split does not divide
                              "4096 4096 16 8 x 1\n",             # not an integer
                              "4096 100 16 1 1\n",                # K outside the contract
                              "4096 4096 16 8 2 1 0 9\n"]):       # too many fields
        bad = tmp_path / f"bad{i}.txt"
        bad.write_text(text)
        _run(sanitized, {"NVFP4_TILES": str(bad)}, -9)
    _run(sanitized, {"NVFP4_TILES": str(tmp_path / "missing.txt")}, -9)

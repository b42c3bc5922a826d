"""The host-only corpus-file reader and writer (suffix_match_drafter_amd/csrc/corpus_file.cpp,
used by sfx_save / sfx_load) built with the address and undefined-behaviour sanitizers and fed
corrupted files (tests/fuzz/corpus_file_fuzz.cpp): flipped bytes, cut and extended files,
header counters set to edge values, and payload edits with the checksum recomputed.  Every file
must be refused with SFX_EIO / SFX_EINVAL or accepted with contents that satisfy what loading
relies on; a sanitizer report fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "tests", "fuzz", "corpus_file_fuzz.cpp"),
       os.path.join(ROOT, "suffix_match_drafter_amd", "csrc", "corpus_file.cpp")]


@pytest.fixture(scope="module")
def fuzzer(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("fuzz") / "corpus_file_fuzz")
    subprocess.check_call([gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-Wall", "-Werror", "-o", exe, *SRC])
    return exe


@pytest.mark.parametrize("seed", [1, 2, 3, 4])
def test_corrupted_corpus_files_under_sanitizers(fuzzer, tmp_path, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([fuzzer, str(tmp_path), str(seed), "3000"], env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    fields = r.stdout.split()
    accepted, refused = int(fields[3]), int(fields[5])
    assert accepted + refused == 3000 and refused > 2000 and accepted > 0

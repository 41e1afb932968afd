"""The CPU sanitizer run (tests/run_sanitizers.py): its builds carry the sanitizers on the host
side only, and inside that run the sanitized oracle and library are the ones loaded."""
import os

import pytest

from bcjr_soft_decoding_amd import bcjr, build


def test_sanitizer_options_apply_to_the_host_pass_only():
    flags = build.SAN_FLAGS
    assert len(flags) % 2 == 0 and flags[0::2] == ["-Xarch_host"] * (len(flags) // 2)
    assert "-fsanitize=address" in flags[1::2] and "-fsanitize=undefined" in flags[1::2]
    assert build.SAN_LIB != build.LIB


@pytest.mark.skipif(os.environ.get("BCJR_SANITIZE") != "1", reason="only inside the sanitizer run")
def test_sanitized_builds_are_loaded():
    import oracle.oracle as orc

    bcjr.lib()
    orc._load()
    maps = open("/proc/self/maps").read()
    assert "libclang_rt.asan" in maps, "the AddressSanitizer runtime is not in the process"
    assert "libbcjr_san.so" in maps and "liboracle_san.so" in maps
    assert "/libbcjr.so" not in maps and "/liboracle.so" not in maps

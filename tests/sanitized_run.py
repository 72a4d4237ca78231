"""Child process for tests/test_sanitizers.py (not a test module itself).

    python tests/sanitized_run.py oracle <libkda_oracle built with sanitizers>
    python tests/sanitized_run.py abi <libkda built with a sanitized ABI object>

The parent starts it with the sanitizer runtime preloaded. It points the
oracle's or the binding's library path at the sanitized build, checks that
this is the library that gets loaded, and runs the CPU tests that exercise
it; any sanitizer report ends the process with a non-zero status.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def main(mode: str, lib_path: str) -> int:
    import pytest

    if mode == "oracle":
        from oracle import kda_oracle

        kda_oracle.LIB_PATH = lib_path
        assert kda_oracle.default().lib._name == lib_path
        files = ["test_oracle_pins.py", "test_oracle_mutants.py"]
    elif mode == "abi":
        import gated_delta_rule_83_amd.kda as K

        K.LIB_PATH = lib_path
        assert K.lib()._name == lib_path
        files = ["test_abi.py"]
    else:
        raise SystemExit(f"unknown mode {mode!r}")
    args = ["-q", "-s", "-p", "no:cacheprovider", "-m", "not gpu"]
    return pytest.main(args + [os.path.join(ROOT, "tests", f) for f in files])


if __name__ == "__main__":
    sys.exit(main(sys.argv[1], sys.argv[2]))

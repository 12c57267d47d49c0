"""Child process of test_sanitizers.py: runs CPU test files against a
sanitizer-instrumented build (the sanitizer runtime is preloaded by the
parent).

    python sanitize_child.py oracle  <liboracle_asan.so>  <test files...>
    python sanitize_child.py library <libselinv_asan.so>  <test files...>
"""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)
sys.path.insert(0, HERE)


def main():
    which, path, files = sys.argv[1], sys.argv[2], sys.argv[3:]
    if which == "oracle":
        import oracle
        oracle._LIB = path
        oracle._lib = None
        oracle.load()
    else:
        import sparse_spd_selected_amd as ssa
        ssa.LIB_PATH = path
        ssa._lib = None
        ssa.lib()
    import pytest
    args = [os.path.join(HERE, f) for f in files]
    # --capture=sys: sanitizer reports (written to file descriptor 2) reach
    # the parent
    return pytest.main(args + ["-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                               "--capture=sys",
                               "-p", "no:xdist", "-k", "not mutant"])


if __name__ == "__main__":
    sys.exit(main())

"""Runs the C-ABI host checks (test_abi.py) against a library path given on the command line - the
sanitizer build of test_sanitize.py - in a process that has the sanitizer runtime preloaded."""

import os
import sys

import pytest

import sparse_attention_hyb_amd as hyb

if __name__ == "__main__":
    hyb._lib = hyb.load(sys.argv[1])
    here = os.path.dirname(os.path.abspath(__file__))
    sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", os.path.join(here, "test_abi.py")]))

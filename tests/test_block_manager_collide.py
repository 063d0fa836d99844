"""The whole C++ block-manager suite (tests/test_block_manager_cpp.py: the pages' traces, the op-by-op differential
against the oracle model, the prefix cache, swapping) run again against libpa_host_collide.so, the block manager
built with a 2-bit chain hash.  Every chain then shares its hash bucket with almost every other, so the prefix
cache finds a cached block only through its exact comparison of the parent chain and the block's token ids: the
cache's answers (and so every differential test against the oracle's exact token chains) must not depend on the
hash.  CPU only."""

import os
import subprocess
import sys

import pytest

from conftest import ROOT

LIB = os.path.join(ROOT, "paged_kv_cache_124_amd", "libpa_host_collide.so")


def test_block_manager_suite_with_colliding_chain_hashes():
    if not os.path.exists(LIB):
        pytest.skip("collision build missing (python paged_kv_cache_124_amd/build.py builds it)")
    env = dict(os.environ, PA_LIBRARY=LIB, PA_HOST_ONLY="1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_block_manager_cpp.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    log = res.stdout + res.stderr
    assert res.returncode == 0, log[-4000:]
    assert " passed" in log and " failed" not in log, log[-2000:]

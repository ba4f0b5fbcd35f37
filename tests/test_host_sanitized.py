"""The host logic and the argument validation of the C-ABI library under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only, nothing is launched).

A copy of the library whose host code is instrumented (``build_sanitized``) is loaded in a
child process with the sanitizer runtime preloaded, and the host-side test module
(tests/test_abi_host.py) runs against it: frame alignment, grid, schedule, layer thinning and
pairing plan against the oracle, model creation, and every size and pointer check of the
entry points.  Any sanitizer report ends the child with a nonzero status.
"""
import os
import subprocess
import sys

import pytest

from tests.conftest import ROOT

pytestmark = pytest.mark.slow


@pytest.fixture(scope="module")
def san_env():
    from video_diffusion_transformer_fwd_amd import build_sanitized as BS
    try:
        BS.runtime_path()
    except RuntimeError as e:
        pytest.skip(str(e))
    BS.build()
    return BS.sanitizer_env()


def run_child(env, args, timeout=600):
    return subprocess.run([sys.executable, *args], env=env, cwd=ROOT, capture_output=True,
                          text=True, timeout=timeout)


def test_sanitized_library_is_the_one_loaded(san_env):
    code = ("from video_diffusion_transformer_fwd_amd import binding as B; B.lib(); "
            "maps = open('/proc/self/maps').read(); "
            "assert 'libh3dit_san.so' in maps and 'libh3dit.so' not in maps, 'wrong library'; "
            "assert 'libclang_rt.asan' in maps, 'sanitizer runtime not loaded'; print('ok')")
    r = run_child(san_env, ["-c", code])
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout + r.stderr


def test_host_abi_tests_under_sanitizers(san_env):
    r = run_child(san_env, ["-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            os.path.join("tests", "test_abi_host.py")])
    tail = (r.stdout + r.stderr)[-4000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail

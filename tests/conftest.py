import ctypes
import json
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.build(force=False)
    oracle.lib()
    return oracle


@pytest.fixture(scope="session")
def encb():
    """The brute-force encoder of tests/native/enc_bruteforce.c, built with gcc."""
    src = os.path.join(ROOT, "tests", "native", "enc_bruteforce.c")
    out = os.path.join(tempfile.mkdtemp(prefix="fp8q_encb_"), "encb.so")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", out, src, "-lm"], check=True)
    L = ctypes.CDLL(out)
    L.encb_bits.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    L.encb_bits.restype = None
    return L


@pytest.fixture(scope="session")
def fq():
    """The Python binding of libfp8q.so, built with hipcc if nothing is built yet."""
    import block_scaled_precision_amax_amd as m
    if not os.path.exists(m.LIB_PATH):
        from block_scaled_precision_amax_amd import build
        build.build()
    m.lib()
    return m


@pytest.fixture(scope="session")
def gpu():
    """A usable ROCm device; GPU tests fail loudly (not skip) without one."""
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    torch.cuda.init()
    return torch.device("cuda:0")

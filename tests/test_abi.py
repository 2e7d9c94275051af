"""CPU checks of the boundary: the library loads, exports every symbol its header declares, and
rejects bad arguments before touching the GPU (no compute calls here)."""
import ctypes
import os
import re

import pytest

import adam_ob_compress_amd as ob

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ob_adam.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ob_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ob.LIB_PATH):
        pytest.fail("libobadam.so is not built: run __graft_entry__.build()")
    return ob.lib()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert len(names) >= 14, names
    for name in names:
        assert hasattr(lib, name), f"{name} declared in ob_adam.h but not exported"


def test_status_strings(lib):
    for s in range(7):
        assert ob.ob_status_str(s) != "unknown status"
    assert "align" in ob.ob_status_str(2)
    assert "static buffer" in ob.ob_status_str(6)


def test_hparams_layout_matches_header():
    # five floats, int32, float, int32, an 8-byte aligned int64, int32 + reserved int32, uint64
    assert ctypes.sizeof(ob.ob_hparams) == 56
    assert ob.ob_hparams.step.offset == 32
    assert ob.ob_hparams.err_rounding.offset == 40
    assert ob.ob_hparams.sr_seed.offset == 48


P = ctypes.c_void_p


def test_validation_before_any_gpu_work(lib):
    # NULL / bad dtype / misaligned pointers are rejected on the host (these addresses are never read)
    assert lib.ob_pack(None, 0, 10, None, None) == 1
    assert lib.ob_pack(P(0x1000), 9, 10, P(0x2000), None) == 3
    assert lib.ob_pack(P(0x1004), 0, 10, P(0x2000), None) == 2
    assert lib.ob_pack(P(0x1008), 1, 10, P(0x2002), None) == 2
    assert lib.ob_pack(None, 0, 0, None, None) == 0          # n = 0 is a no-op
    assert lib.ob_pack(None, 0, -1, None, None) == 1
    assert lib.ob_unpack(None, None, 0, None, None, None) == 0
    assert lib.ob_unpack(None, P(0x1000), 64, P(0x2000), P(0x3000), None) == 1   # scales need a plan
    # plan-less pack / unpack: a grid of n / 16384 blocks must fit 2^31 - 1
    too_many = ((1 << 31) - 1) * 16384 + 1
    assert lib.ob_pack(P(0x1000), 0, too_many, P(0x2000), None) == 1
    assert lib.ob_unpack(None, P(0x1000), too_many, None, P(0x3000), None) == 1
    assert lib.ob_plan_num_groups(None, 0, 0, 0) == -1
    hp = ob.hparams()
    assert lib.ob_adam_compress_step(None, P(0x1000), 0, None, 0, None, None, None, None, None, None,
                                     None, ctypes.byref(hp), None) == 1
    assert lib.ob_adam_warmup_step(None, None, 0, None, None, None, ctypes.byref(hp), None) == 1
    assert lib.ob_server_reduce(None, 8, None, None, None, None, None, None) == 1
    h = P()
    assert lib.ob_plan_create(-1, 64, None, 0, ctypes.byref(h)) == 1
    assert lib.ob_plan_create(100, 0, None, 0, ctypes.byref(h)) == 1
    assert lib.ob_plan_create(1000, 100, None, 0, ctypes.byref(h)) == 2   # interior boundary 100
    bad = (ctypes.c_int64 * 3)(0, 100, 200)
    assert lib.ob_plan_create(200, 0, bad, 2, ctypes.byref(h)) == 2
    short = (ctypes.c_int64 * 3)(0, 64, 199)
    assert lib.ob_plan_create(200, 0, short, 2, ctypes.byref(h)) == 1
    empty_chunk = (ctypes.c_int64 * 4)(0, 64, 64, 200)
    assert lib.ob_plan_create(200, 0, empty_chunk, 3, ctypes.byref(h)) == 1
    # the no-allocation step: argument and size checks are host arithmetic, made before any HIP call
    args = (P(0x1000), 0, P(0x2000), 0, P(0x3000), P(0x4000), P(0x5000), P(0x6000), P(0x7000), None, None,
            ctypes.byref(hp), None)
    assert lib.ob_adam_compress_step_noalloc(0, 64, *args) == 0                 # n = 0 is a no-op
    assert lib.ob_adam_compress_step_noalloc(-1, 64, *args) == 1
    assert lib.ob_adam_compress_step_noalloc(1000, 0, *args) == 1
    assert lib.ob_adam_compress_step_noalloc(1000, 100, *args) == 2             # interior boundary 100
    assert lib.ob_adam_compress_step_noalloc(1000, 64, P(0x1004), *args[1:]) == 2
    assert lib.ob_adam_compress_step_noalloc(1000, 64, None, *args[1:]) == 1
    # 2^37 elements: about 33.6 million 4096-element blocks of the fused pass need 537 MB of tables
    assert lib.ob_adam_compress_step_noalloc(1 << 37, 1 << 24, *args) == 6
    # 2^30 elements in chunks of 64: 16.8 million chunks
    assert lib.ob_adam_compress_step_noalloc(1 << 30, 64, *args) == 6
    assert lib.ob_plan_destroy(None) == 1
    assert lib.ob_plan_num_chunks(None) == -1
    d = ctypes.c_double()
    k = ctypes.c_int64()
    assert lib.ob_plan_read_timing(None, 0, ctypes.byref(d), ctypes.byref(k)) == 1


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises((ValueError, RuntimeError)):
        ob.ob_pack(torch.zeros(64), torch.zeros(2, dtype=torch.int32))


def test_host_allocation_failure_is_a_status_not_an_abort():
    """No C++ exception crosses the ABI: a plan whose host-side tables do not fit (2^38 elements under
    a 4 GiB address-space limit, in a child process) returns OB_ERR_OOM with *out = NULL, where an
    escaping std::bad_alloc would abort the process."""
    import subprocess
    import sys
    import textwrap

    code = textwrap.dedent(f"""
        import ctypes, resource
        resource.setrlimit(resource.RLIMIT_AS, (4 << 30, 4 << 30))
        L = ctypes.CDLL({ob.LIB_PATH!r})
        L.ob_plan_create.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.POINTER(ctypes.c_void_p)]
        h = ctypes.c_void_p(1)
        print(L.ob_plan_create(1 << 38, 1 << 20, None, 0, ctypes.byref(h)), h.value)
    """)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    status, handle = r.stdout.split()
    assert int(status) == ob.OB_ERR_OOM and handle == "None"

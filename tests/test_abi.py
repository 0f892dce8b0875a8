"""The C ABI without a GPU: the library loads, exports every entry point that
include/moe_get.h declares, and validates shapes on the host the way the
Constraints section of the CANN "low_latency_dispatch" page states (checked
against the oracle's own, independently written, check)."""
import ctypes
import os
import re

import pytest

import combine_moe_get_amd as mg
import oracle

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "moe_get.h")


def _declared_functions():
    with open(HDR) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("moe_get_layout", "moe_dispatch", "moe_combine", "moe_get_workspace_size",
              "moe_get_recv_capacity", "moe_get_check_shape"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(mg.LIB_PATH)
    missing = [n for n in _declared_functions() if not hasattr(L, n)]
    assert not missing, missing


def test_abi_version_and_status_strings():
    assert mg.abi_version() == 2
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert mg.status_string(code) and mg.status_string(code) != "unknown status"
    assert mg.status_string(42) == "unknown status"


SHAPES = [
    dict(T=4096, H=7168, K=8, E=256, P=32, num_max=128),
    dict(T=4096, H=7168, K=8, E=256, P=64),
    dict(T=8192, H=4096, K=8, E=128, P=16, Z=2, C=2, Kc=2),
    dict(T=16384, H=7168, K=8, E=256, P=64, num_max=256),
    dict(T=0, H=64, K=4, E=32, P=2),
    dict(T=8, H=64, K=17, E=32, P=2),
    dict(T=8, H=64, K=4, E=30, P=4),
    dict(T=9, H=64, K=4, E=32, P=2),
    dict(T=1026, H=64, K=4, E=32, P=2),
    dict(T=8, H=64, K=4, E=4096, P=2),
    dict(T=8, H=64, K=5, E=4, P=2),
    dict(T=16, H=64, K=4, E=32, P=2, num_max=4),
    dict(T=8, H=60, K=4, E=32, P=2),
    dict(T=8, H=8200, K=4, E=32, P=2),
    dict(T=8, H=64, K=4, E=32, P=2, Z=600, C=600),
    dict(T=-8, H=64, K=4, E=32, P=2),
    dict(T=8, H=64, K=0, E=32, P=2),
]


@pytest.mark.parametrize("kw", SHAPES)
def test_shape_checks_agree_with_the_oracle(kw):
    args = (kw["T"], kw["H"], kw["K"], kw["E"], kw["P"], kw.get("Z", 0), kw.get("C", 0),
            kw.get("Kc", 0), kw.get("num_max", 0))
    got = mg.check_shape(mg.make_shape(*args))
    exp = oracle.check_shape(oracle.make_shape(*args))
    kernel_limit = (kw["H"] % 8 != 0 or kw["H"] > 8192 or
                    kw.get("Z", 0) + kw.get("C", 0) + kw.get("Kc", 0) > 1024)
    if exp == 0 and kernel_limit:
        assert got == -4
    else:
        assert got == exp


def test_sizes():
    s = mg.make_shape(4096, 7168, 8, 256, 32, num_max=128)
    assert mg.recv_capacity(s) == 4096 * 8
    assert mg.workspace_size(s) >= 4 * (32 * 256 + 32 * 32)
    assert mg.recv_capacity(mg.make_shape(9, 64, 4, 32, 2)) == -1
    assert mg.workspace_size(mg.make_shape(9, 64, 4, 32, 2)) == 0


@pytest.mark.parametrize("kw", SHAPES[:5])
def test_rank_capacity_agrees_with_the_oracle(kw):
    args = (kw["T"], kw["H"], kw["K"], kw["E"], kw["P"], kw.get("Z", 0), kw.get("C", 0),
            kw.get("Kc", 0), kw.get("num_max", 0))
    assert mg.rank_capacity(mg.make_shape(*args)) == oracle.rank_capacity(oracle.make_shape(*args))


def test_header_is_plain_c_and_a_c_client_links(tmp_path):
    """moe_get.h compiles as C11 with gcc, and a C program calling layout,
    dispatch and combine links against libmoe_get.so (no GPU work is run)."""
    import importlib.util
    import shutil
    import subprocess

    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_client", "build.py")
    spec = importlib.util.spec_from_file_location("moe_c_client_build", path)
    cb = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(cb)
    cb.build()
    assert os.access(cb.BIN, os.X_OK)
    nm = subprocess.run(["nm", "-D", "--undefined-only", cb.BIN], capture_output=True, text=True)
    if nm.returncode == 0:
        for n in ("moe_get_layout", "moe_dispatch", "moe_combine"):
            assert n in nm.stdout


def test_layout_launches():
    # one launch while T * K <= 8192 slots, two above; errors for shapes outside the constraints
    assert mg.layout_launches(mg.make_shape(128, 7168, 8, 256, 1)) == 1
    assert mg.layout_launches(mg.make_shape(1024, 7168, 8, 256, 32)) == 1
    assert mg.layout_launches(mg.make_shape(1056, 7168, 8, 256, 32)) == 2
    assert mg.layout_launches(mg.make_shape(4096, 7168, 8, 256, 32)) == 2
    assert mg.layout_launches(mg.make_shape(512, 7168, 16, 256, 2)) == 1  # 8192 slots, 256 tokens per rank
    assert mg.layout_launches(mg.make_shape(512, 7168, 16, 256, 1)) == 1  # one 512-token rank, 8192 slots
    assert mg.layout_launches(mg.make_shape(1024, 7168, 16, 256, 2)) == 2  # 16384 slots
    with pytest.raises(mg.MoeGetError):
        mg.layout_launches(mg.make_shape(100, 7168, 8, 256, 32))  # T not a multiple of P


def test_argument_errors_return_before_any_device_work():
    # the host-side failure paths of the C ABI, forced from the host on a machine without a GPU:
    # each call must return its status before asking the HIP runtime for anything
    L = mg.lib()
    ok = mg.make_shape(64, 64, 4, 8, 2, 0, 1, 0)  # one copy expert
    p = ctypes.c_void_p(256)  # an aligned, never dereferenced stand-in for a device pointer
    n = None
    # combine with a copy expert but no ori_x
    assert L.moe_combine(ctypes.byref(ok), p, p, p, n, p, n, n, n, n, p, n) == -1
    # bad quant mode; per-expert scales without topk_idx; negative grid cap
    assert L.moe_dispatch(ctypes.byref(ok), 3, p, n, 0, n, n, p, p, n, n, n) == -1
    assert L.moe_dispatch(ctypes.byref(ok), 2, p, p, 8, n, n, p, p, p, n, n) == -1
    assert L.moe_dispatch_capped(ctypes.byref(ok), -1, 0, p, n, 0, n, n, p, p, n, n, n) == -1
    assert L.moe_combine_capped(ctypes.byref(ok), -1, p, p, p, n, p, p, n, n, n, p, n) == -1
    # misaligned rows
    assert L.moe_dispatch(ctypes.byref(ok), 0, p, n, 0, n, n, p, ctypes.c_void_p(258), n, n, n) == -1
    # layout: no workspace; a rank window below capacity; BS above num_max
    outs = [p] * 9
    assert L.moe_get_layout(ctypes.byref(ok), p, n, *outs, n, n, 0, n) == -1
    cap = mg.rank_capacity(ok)
    assert L.moe_get_layout_ex(ctypes.byref(ok), cap - 1, p, n, *outs, n, p, 1 << 20, n) == -3
    assert L.moe_get_layout(ctypes.byref(mg.make_shape(64, 64, 4, 8, 2, num_max=16)), p, n, *outs, n, p,
                            1 << 20, n) == -3
    # the allocation-free layout: a missing output, then a shape whose workspace exceeds the scratch
    bad_outs = [p] * 8 + [n]
    assert L.moe_get_layout_noalloc(ctypes.byref(ok), 0, p, n, *bad_outs, n, n) == -1
    big = mg.make_shape(2048, 64, 4, 2048, 2048)
    assert L.moe_get_layout_noalloc(ctypes.byref(big), 0, p, n, *outs, n, n) == -6
    # T = 0 does nothing and succeeds without touching any pointer
    empty = mg.make_shape(0, 64, 4, 8, 2)
    assert L.moe_dispatch(ctypes.byref(empty), 0, n, n, 0, n, n, n, n, n, n, n) == 0
    assert L.moe_combine(ctypes.byref(empty), n, n, n, n, n, n, n, n, n, n, n) == 0

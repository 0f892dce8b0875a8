"""The access-pattern probes that bench.py reports next to the dispatch and the
combine (libmoe_hbm_probe.so): each must move exactly the bytes it claims, so
that its time is a bound for the kernel it stands beside.  Checked on small
ragged shapes (rows of 129 16-byte chunks: two 2 KB slices, the second
partial) against numpy."""
import ctypes
import os

import numpy as np
import pytest
import torch

from tests import _gpu as G

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "combine_moe_get_amd",
                   "libmoe_hbm_probe.so")
MAGIC = (0x5A5A5A5A, 0xA5A5A5A5)


def _lib():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is not built")
    lib = ctypes.CDLL(LIB)
    vp, ci = ctypes.c_void_p, ctypes.c_int
    lib.moe_probe_scatter_write.argtypes = [vp, ci, ci, ci, vp, vp]
    lib.moe_probe_ordered_write.argtypes = [ctypes.c_int64, ci, vp, vp]
    lib.moe_probe_gather_read.argtypes = [vp, ci, ci, ci, vp, vp, vp]
    lib.moe_probe_reduce.argtypes = [vp, ci, ci, ci, vp, vp, ci, vp]
    return lib


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _row_map(T, K, nrows, seed):
    r = np.random.default_rng(seed)
    m = r.permutation(nrows)[:T * K].astype(np.int32).reshape(T, K)
    m[r.random((T, K)) < 0.1] = -1
    return m


@pytest.mark.parametrize("T,K,row_bytes", [(37, 5, 2064), (19, 11, 4096), (8, 16, 16)])
def test_scatter_and_ordered_writes_store_their_pattern(T, K, row_bytes):
    lib = _lib()
    nrows = T * K + 3
    dst = _row_map(T, K, nrows, T + K)
    buf = torch.full((nrows, row_bytes // 4), 7, dtype=torch.int32, device=G.DEV)
    assert lib.moe_probe_scatter_write(_p(G.dev(dst)), T, K, row_bytes, _p(buf), _stream()) == 0
    torch.cuda.synchronize()
    got = buf.cpu().numpy().reshape(nrows, row_bytes // 16, 4)
    want = np.full_like(got, 7)
    for t in range(T):
        for j in range(K):
            if dst[t, j] >= 0:
                want[dst[t, j], :, 0] = t
                want[dst[t, j], :, 1] = np.arange(row_bytes // 16)
                want[dst[t, j], :, 2:] = np.array(MAGIC, dtype=np.uint32).view(np.int32)
    assert np.array_equal(got, want), "scatter probe stored other bytes than the rows it names"

    buf.fill_(7)
    n = nrows - 2
    assert lib.moe_probe_ordered_write(n, row_bytes, _p(buf), _stream()) == 0
    torch.cuda.synchronize()
    got = buf.cpu().numpy().reshape(nrows, row_bytes // 16, 4)
    want = np.full_like(got, 7)
    want[:n, :, 0] = np.arange(n)[:, None]
    want[:n, :, 1] = np.arange(row_bytes // 16)[None, :]
    want[:n, :, 2:] = np.array(MAGIC, dtype=np.uint32).view(np.int32)
    assert np.array_equal(got, want), "ordered probe stored other bytes than rows [0, n)"


@pytest.mark.parametrize("T,K,row_bytes", [(37, 5, 2064), (19, 11, 4096), (8, 16, 16)])
def test_reduce_probe_folds_the_rows_it_reads(T, K, row_bytes):
    lib = _lib()
    nrows = T * K + 3
    dst = _row_map(T, K, nrows, 100 + T)
    r = np.random.default_rng(T * K)
    src = r.integers(-2**31, 2**31, (nrows, row_bytes // 4), dtype=np.int64).astype(np.int32)
    buf = G.dev(src)
    out = torch.full((T, row_bytes // 4), 7, dtype=torch.int32, device=G.DEV)
    for gather in (1, 0):
        assert lib.moe_probe_reduce(_p(G.dev(dst)), T, K, row_bytes, _p(buf), _p(out), gather, _stream()) == 0
        torch.cuda.synchronize()
        want = np.zeros((T, row_bytes // 4), dtype=np.int32)
        for t in range(T):
            for j in range(K):
                row = dst[t, j] if gather else t * K + j
                if row >= 0:
                    want[t] ^= src[row]
        assert np.array_equal(out.cpu().numpy(), want), f"reduce probe (gather={gather}) folded other rows"
        out.fill_(7)

    # the gather-read probe reads the same rows and writes nothing (its sink keeps its contents)
    nsl = (row_bytes // 16 + 127) // 128
    sink = torch.full((T * nsl * 64, 4), 7, dtype=torch.int32, device=G.DEV)
    assert lib.moe_probe_gather_read(_p(G.dev(dst)), T, K, row_bytes, _p(buf), _p(sink), _stream()) == 0
    torch.cuda.synchronize()
    assert torch.all(sink == 7)


def test_probes_refuse_bad_arguments():
    lib = _lib()
    buf = torch.zeros(4096, dtype=torch.int32, device=G.DEV)
    dst = torch.zeros((4, 2), dtype=torch.int32, device=G.DEV)
    s = _stream()
    assert lib.moe_probe_scatter_write(_p(dst), 4, 2, 24, _p(buf), s) == -1   # not a multiple of 16
    assert lib.moe_probe_scatter_write(_p(dst), 4, 17, 32, _p(buf), s) == -1  # K above 16
    assert lib.moe_probe_ordered_write(4, 16400, _p(buf), s) == -1            # row above 16 KB
    assert lib.moe_probe_reduce(None, 4, 2, 32, _p(buf), _p(buf), 1, s) == -1  # gather without a map
    assert lib.moe_probe_gather_read(_p(dst), 4, 2, 32, _p(buf), None, s) == -1

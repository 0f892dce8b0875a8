"""bench.py's byte accounting and its refusal of more than one GPU (CPU only)."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_dispatch_bytes_match_the_worked_example():
    # "Wide-EP / DBO / DeepEP hardware cliff", A short illustrative example: B = 8192 tokens,
    # P = 16 ranks, k = 8, d = 7168, one-byte activations -> (B/P) * k * d = 29,360,128 bytes per rank
    rows = 8192 // 16 * 8
    assert bench.comm_bytes(rows, 7168, 1, 0) == 29_360_128
    assert bench.dispatch_comm_bytes(rows, 7168, 1) == 29_360_128
    # the dynamic mode carries one fp32 scale per row, bf16 rows are two bytes per channel
    assert bench.dispatch_comm_bytes(rows, 7168, 2) == 29_360_128 + 4 * rows
    assert bench.dispatch_comm_bytes(rows, 7168, 0) == 2 * 29_360_128
    assert bench.combine_comm_bytes(rows, 7168) == 2 * 29_360_128


def test_algorithmic_bytes_of_the_decode_workload():
    T, H, K = 4096, 7168, 8
    n = T * K
    d = bench.dispatch_hbm_bytes(T, H, K, n, T, 2, 1)
    assert d == T * 2 * H + T * K * 4 + 4 * H + n * (H + 4)
    c = bench.combine_hbm_bytes(T, H, K, n, 0)
    assert c == n * 2 * H + T * K * 12 + T * 2 * H


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_threaded_oracle_leg_computes_what_the_oracle_computes():
    # the all-cores CPU baseline runs the oracle's dispatch and combine on token slices in threads;
    # its rows, scales and combine must be the single-threaded oracle's, bit for bit
    import numpy as np

    import oracle
    from combine_moe_get_amd import workloads

    for cid, T in ((2, 256), (4, 512), (5, 512)):
        inp = workloads.make_inputs(cid, seed=1, T=T)
        c = inp["cfg"]
        sh = oracle.make_shape(c["T"], c["H"], c["K"], c["E"], c["P"], c["Z"], c["C"], c["Kc"], c["num_max"])
        lo = oracle.layout(sh, inp["topk_idx"], inp["mask"])
        d = oracle.dispatch(sh, c["quant_mode"], inp["x"], lo, smooth=inp["smooth"], topk_idx=inp["topk_idx"])
        y = np.ascontiguousarray(inp["x"][lo["src_info"] // c["K"]])
        ref = oracle.combine(sh, y, inp["topk_idx"], inp["topk_weights"], lo, inp["mask"], inp["ori_x"],
                             inp["alpha1"], inp["alpha2"], inp["const_v"])
        lo2, ex, ds, out = bench._oracle_threaded_pass(inp, 3, return_outputs=True)
        assert np.array_equal(lo2["dst_row"], lo["dst_row"])
        assert np.array_equal(ex, d["expand_x"])
        if c["quant_mode"] == 2:
            assert np.array_equal(ds.view(np.uint32), d["dynamic_scales"].view(np.uint32))
        assert np.array_equal(out, ref)

"""The C ABI used from plain C: tests/c_client/moe_client (gcc, linked against
libmoe_get.so and the HIP runtime, no Python or PyTorch in the process) runs
layout, dispatch and combine on seeded inputs written to files; its outputs are
checked against the oracle to the same bar as the Python-driven parity tests."""
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
from combine_moe_get_amd.workloads import expert_out_normal, fuzz_world, make_inputs

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
from _gpu import LAYOUT_KEYS, assert_combine_close  # noqa: E402
from c_client import build as cbuild  # noqa: E402


def _client():
    src = os.path.join(HERE, "c_client", "moe_client.c")
    if not os.path.exists(cbuild.BIN) or os.path.getmtime(cbuild.BIN) < os.path.getmtime(src):
        cbuild.build()
    return cbuild.BIN


def _write(d, name, a):
    np.ascontiguousarray(a).tofile(os.path.join(d, name + ".bin"))


def _read(d, name, dtype, shape):
    a = np.fromfile(os.path.join(d, "out_" + name + ".bin"), dtype=dtype)
    return a.reshape(shape)


def _run(tmp, w, quant_mode, num_max=0, smooth_rows=None, fused=False, path=None, max_workgroups=0):
    """path 0: layout + dispatch + combine; 1: layout_dispatch + combine; 2: layout_noalloc +
    dispatch_capped + combine_capped on max_workgroups workgroups"""
    path = (1 if fused else 0) if path is None else path
    T, H, K, E, P, Z, C, Kc = (w[k] for k in ("T", "H", "K", "E", "P", "Z", "C", "Kc"))
    osh = oracle.make_shape(T, H, K, E, P, Z, C, Kc, num_max)
    mask = w.get("mask")
    smooth = w.get("smooth")
    if smooth is not None and smooth_rows is not None and smooth_rows != 1:
        # distinct rows, so a wrong row index shows
        f = 0.75 + 0.5 * np.arange(smooth_rows, dtype=np.float32)[:, None] / smooth_rows
        smooth = np.ascontiguousarray(smooth[None, :] * f, np.float32)
    srows = 0 if smooth is None else smooth.size // H
    lo = oracle.layout(osh, w["topk_idx"], mask)
    do = oracle.dispatch(osh, quant_mode, w["x"], lo, smooth=smooth, weights=w["topk_weights"],
                         topk_idx=w["topk_idx"])
    n = lo["num_rows"]
    Y = expert_out_normal(n, H, seed=T + H)
    co = oracle.combine(osh, Y, w["topk_idx"], w["topk_weights"], lo, mask, w["x"],
                        w.get("alpha1"), w.get("alpha2"), w.get("const_v"))
    d = str(tmp)
    with open(os.path.join(d, "shape.txt"), "w") as f:
        f.write(" ".join(str(int(v)) for v in (T, H, K, E, P, Z, C, Kc, num_max, quant_mode,
                                                 mask is not None, srows, path, max_workgroups)) + "\n")
    _write(d, "topk_idx", w["topk_idx"].astype(np.int32))
    _write(d, "x", w["x"])
    _write(d, "w", w["topk_weights"].astype(np.float32))
    _write(d, "y", Y)
    if mask is not None:
        _write(d, "mask", mask.astype(np.uint8))
    if srows:
        _write(d, "smooth", smooth.astype(np.float32))
    if Kc:
        _write(d, "a1", w["alpha1"])
        _write(d, "a2", w["alpha2"])
        _write(d, "cv", w["const_v"])
    print(f"[c-client] T={T} H={H} K={K} E={E} P={P} Z={Z} C={C} Kc={Kc} quant={quant_mode} "
          f"smooth_rows={srows} mask={mask is not None} path={path} max_workgroups={max_workgroups}", flush=True)
    r = subprocess.run([_client(), d], capture_output=True, text=True, timeout=90)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stderr

    NS = Z + C + Kc
    shapes = dict(num_tokens_per_expert=(E,), expert_offsets=(E + 1,), recv_counts=(E, P),
                  special_counts=(NS,), num_tokens_per_rank=(P,), rank_offsets=(P + 1,),
                  dst_row=(T, K), src_info=(n,))
    for k in LAYOUT_KEYS:
        if k == "is_token_in_rank":
            g = _read(d, k, np.uint8, (T, P))
        else:
            g = _read(d, k, np.int32, shapes[k])
        np.testing.assert_array_equal(g.reshape(np.asarray(lo[k]).shape), lo[k], err_msg=k)
    assert int(_read(d, "status", np.uint32, (1,))[0]) == lo["status"]
    if quant_mode == 0:
        ex = _read(d, "expand_x", np.uint16, (n, H))
    else:
        ex = _read(d, "expand_x", np.int8, (n, H))
    assert np.array_equal(ex, do["expand_x"][:n]), "dispatch rows differ"
    if quant_mode == 2:
        ds = _read(d, "dynamic_scales", np.uint32, (n,))
        assert np.array_equal(ds, do["dynamic_scales"][:n].view(np.uint32)), "dynamic scales differ"
    ew = _read(d, "expand_weights", np.float32, (n,))
    assert np.array_equal(ew, do["expand_weights"][:n]), "expand_weights differ"
    out = _read(d, "out", np.uint16, (T, H))
    assert_combine_close(out, co, what="c-client combine")


@pytest.mark.gpu
@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("seed,quant_mode", [(3, 0), (5, 1), (8, 2)])
def test_c_client_fuzz(tmp_path, seed, quant_mode, fused):
    w = fuzz_world(seed, Z=1, C=1, Kc=1)
    _run(tmp_path, w, quant_mode, fused=fused)


@pytest.mark.gpu
def test_c_client_per_expert_smooth(tmp_path):
    w = fuzz_world(11, Z=0, C=1, Kc=0, p_bad=0.0)
    _run(tmp_path, w, 2, smooth_rows=w["E"])


@pytest.mark.gpu
@pytest.mark.parametrize("fused", [False, True])
def test_c_client_ll_decode_share(tmp_path, fused):
    inp = make_inputs(2, seed=1, T=256)
    c = inp["cfg"]
    w = dict(T=c["T"], H=c["H"], K=c["K"], E=c["E"], P=c["P"], Z=0, C=0, Kc=0, x=inp["x"],
             topk_idx=inp["topk_idx"], topk_weights=inp["topk_weights"], smooth=inp["smooth"])
    _run(tmp_path, w, 2, num_max=c["num_max"], fused=fused)


@pytest.mark.gpu
@pytest.mark.parametrize("seed,quant_mode,cap", [(4, 0, 3), (6, 2, 50), (9, 1, 1)])
def test_c_client_noalloc_and_capped(tmp_path, seed, quant_mode, cap):
    # moe_get_layout_noalloc (no workspace anywhere in the process), moe_dispatch_capped and
    # moe_combine_capped, driven from plain C
    w = fuzz_world(seed, Z=1, C=1, Kc=1)
    _run(tmp_path, w, quant_mode, path=2, max_workgroups=cap)

"""Helpers of the GPU parity tests: run the HIP path and the oracle on the same
seeded inputs and compare them (integers bit-exact, combine within tolerance)."""
import numpy as np
import torch

import combine_moe_get_amd as mg
import oracle
from combine_moe_get_amd.workloads import bf16_bits_to_f32, f32_to_bf16_bits

DEV = torch.device("cuda:0")

# combine tolerance: per element |gpu - exact| <= max(ATOL, RTOL * |exact|)
ATOL, RTOL = 1e-2, 4e-3


def dev(a, dtype=None):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def host_bf16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def shapes(T, H, K, E, P, Z=0, C=0, Kc=0, num_max=0):
    return (mg.make_shape(T, H, K, E, P, Z, C, Kc, num_max),
            oracle.make_shape(T, H, K, E, P, Z, C, Kc, num_max))


def gpu_layout(shape, topk, mask):
    lay = mg.layout(shape, dev(topk), dev(mask))
    torch.cuda.synchronize()
    return lay


def layout_to_numpy(lay, rank_stride=0):
    out = {k: getattr(lay, k).cpu().numpy() for k in lay._fields}
    n = int(out["expert_offsets"][-1])
    out["num_rows"] = n
    if rank_stride <= 0:
        out["src_info"] = out["src_info"][:n]
    out["status"] = int(out["status"][0])
    return out


LAYOUT_KEYS = ["num_tokens_per_expert", "expert_offsets", "recv_counts", "special_counts",
               "num_tokens_per_rank", "rank_offsets", "is_token_in_rank", "dst_row", "src_info"]


def assert_layout_equal(g, o):
    for k in LAYOUT_KEYS:
        np.testing.assert_array_equal(np.asarray(g[k]).reshape(np.asarray(o[k]).shape), o[k], err_msg=k)
    assert g["num_rows"] == o["num_rows"]
    assert g["status"] == o["status"], (g["status"], o["status"])


def assert_combine_close(got_u16, ref, what="combine", match_frac=0.999):
    got = bf16_bits_to_f32(got_u16).astype(np.float64)
    err = np.abs(got - ref)
    bound = np.maximum(ATOL, RTOL * np.abs(ref))
    bad = err > bound
    if bad.any():
        i = np.unravel_index(np.argmax(err - bound), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance; worst at {i}: "
                             f"gpu {got[i]!r} exact {ref[i]!r}")
    # exact zeros (masked tokens, zero-expert-only tokens) must be +0 bit for bit
    z = ref == 0
    assert np.all(got_u16[z] == 0), f"{what}: nonzero bits where the exact result is 0"
    # almost every element is the correctly rounded bf16 of the exact value
    nearest = f32_to_bf16_bits(ref.astype(np.float32))
    frac = float(np.mean(nearest == got_u16)) if got_u16.size else 1.0
    assert frac >= match_frac, f"{what}: only {frac:.5f} of elements are the nearest bf16"
    return float(err.max()) if err.size else 0.0


def smooth_rows_of(smooth, H):
    if smooth is None:
        return 0
    return 1 if smooth.size == H else smooth.size // H


def run_case(T, H, K, E, P, Z, C, Kc, topk, mask, x, weights, quant_mode, smooth, Y_fn,
             ori_x=None, a1=None, a2=None, v=None, num_max=0, label="", rank_stride=0):
    """Full pipeline on both sides; returns (gpu dict, oracle dict).  Y_fn(oracle_layout,
    oracle_dispatch) builds the expert outputs both combines read."""
    print(f"[case] {label} T={T} H={H} K={K} E={E} P={P} Z={Z} C={C} Kc={Kc} quant={quant_mode} "
          f"smooth_rows={smooth_rows_of(smooth, H)} mask={'yes' if mask is not None else 'no'} "
          f"rank_stride={rank_stride}", flush=True)
    shape, osh = shapes(T, H, K, E, P, Z, C, Kc, num_max)
    lo = oracle.layout(osh, topk, mask, rank_stride=rank_stride)
    do = oracle.dispatch(osh, quant_mode, x, lo, smooth=smooth, weights=weights, topk_idx=topk)
    Y = Y_fn(lo, do)
    co = oracle.combine(osh, Y, topk, weights, lo, mask, ori_x, a1, a2, v)

    tk, mk, wd = dev(topk), dev(mask), dev(weights)
    lay = mg.layout(shape, tk, mk, rank_stride=rank_stride)
    cap = max(P * rank_stride if rank_stride > 0 else T * K, 1)
    ew = torch.empty(cap, dtype=torch.float32, device=DEV)
    ex, ds, _ = mg.dispatch(shape, quant_mode, dev(x), lay.dst_row, dev(smooth), wd, tk, expand_weights=ew,
                            rows=cap)
    Yd = dev(Y if Y.shape[0] > 0 else np.zeros((1, H), np.uint16))
    out = mg.combine(shape, Yd, tk, wd, lay.dst_row, mk, dev(ori_x), dev(a1), dev(a2), dev(v), rows=Yd.shape[0])
    torch.cuda.synchronize()
    g = layout_to_numpy(lay, rank_stride)
    o = dict(lo)
    o.update(do)
    o["out"] = co
    # rows that hold a copy: all of [0, N) in the compact layout, the named rows of each window
    # in the fixed-capacity layout (the rest of a window is never written)
    rows = np.sort(lo["dst_row"][lo["dst_row"] >= 0]).astype(np.int64)
    rt = torch.from_numpy(rows).to(DEV)
    g["expand_x"] = host_bf16(ex[rt]) if quant_mode == 0 else ex[rt].cpu().numpy()
    g["dynamic_scales"] = ds[rt].cpu().numpy() if ds is not None else None
    g["expand_weights"] = ew[rt].cpu().numpy()
    g["out"] = host_bf16(out)
    if rank_stride > 0:
        g["src_info"] = g["src_info"][rows]
        o["src_info"] = lo["src_info"][rows]
    o["expand_x"] = do["expand_x"][rows]
    o["dynamic_scales"] = do["dynamic_scales"][rows]
    o["expand_weights"] = do["expand_weights"][rows]
    return g, o


def assert_case(g, o, quant_mode, weights_given=True):
    assert_layout_equal(g, o)
    assert np.array_equal(g["expand_x"], o["expand_x"]), "dispatch rows differ"
    if quant_mode == 2:
        assert np.array_equal(g["dynamic_scales"].view(np.uint32), o["dynamic_scales"].view(np.uint32)), \
            "dynamic scales differ"
    if weights_given:
        assert np.array_equal(g["expand_weights"], o["expand_weights"]), "expand_weights differ"
    return assert_combine_close(g["out"], o["out"])

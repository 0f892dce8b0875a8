"""GPU guards: every output buffer of layout / dispatch / layout_dispatch is
written exactly where the layout says and nowhere else (canary-filled rows past
N, unused rows of each rank window, guard rows past the end of every buffer),
rank windows that overflow on the device agree with the oracle (status bit 2,
the dropped copies, the combine after them), undersized buffers are refused in
Python before anything is launched, and two windowed receive buffers used in
turn by consecutive layers inside one captured graph keep each layer's rows."""
import numpy as np
import pytest
import torch

import combine_moe_get_amd as mg
import oracle
from combine_moe_get_amd import workloads
from tests import _gpu as G

pytestmark = pytest.mark.gpu

GUARD = 3
I8_CANARY = 0x5A
F32_CANARY = -0x2A2A2A2B  # int32 bit pattern written into float buffers
I32_CANARY = -0x5A5A5A5B


def _canary_outputs(cap, H, qm):
    """Output buffers with GUARD extra rows, all filled with canaries; returns (full, views)."""
    if qm == 0:
        ex_full = torch.full((cap + GUARD, H), -0x5A5B, dtype=torch.int16, device=G.DEV)
        ex = ex_full.view(torch.bfloat16)[:cap]
    else:
        ex_full = torch.full((cap + GUARD, H), I8_CANARY, dtype=torch.int8, device=G.DEV)
        ex = ex_full[:cap]
    ds_full = torch.full((cap + GUARD,), F32_CANARY, dtype=torch.int32, device=G.DEV)
    ew_full = torch.full((cap + GUARD,), F32_CANARY, dtype=torch.int32, device=G.DEV)
    src_full = torch.full((cap + GUARD,), I32_CANARY, dtype=torch.int32, device=G.DEV)
    return (ex_full, ds_full, ew_full, src_full), (ex, ds_full.view(torch.float32)[:cap],
                                                  ew_full.view(torch.float32)[:cap], src_full[:cap])


def _check_untouched(full, written_rows, qm, what):
    ex_full, ds_full, ew_full, src_full = full
    n_all = ex_full.shape[0]
    keep = torch.ones(n_all, dtype=torch.bool, device=G.DEV)
    keep[torch.from_numpy(np.asarray(written_rows, np.int64)).to(G.DEV)] = False
    ex_can = -0x5A5B if qm == 0 else I8_CANARY
    assert torch.all(ex_full[keep] == ex_can), f"{what}: expand_x written outside the layout's rows"
    assert torch.all(ew_full[keep] == F32_CANARY), f"{what}: expand_weights written outside the layout's rows"
    if qm == 2:
        assert torch.all(ds_full[keep] == F32_CANARY), f"{what}: dynamic_scales written outside the layout's rows"
    else:
        assert torch.all(ds_full == F32_CANARY), f"{what}: dynamic_scales written although the mode has none"
    assert torch.all(src_full[keep] == I32_CANARY), f"{what}: src_info written outside the layout's rows"


def _world(seed, T, H, K, E, P, Z=0, C=0, Kc=0, p_drop=0.05, mask=True):
    r = np.random.default_rng(seed)
    etot = E + Z + C + Kc
    topk = np.argsort(r.random((T, etot)), axis=1)[:, :K].astype(np.int32)
    topk[r.random((T, K)) < p_drop] = -1
    m = (r.random(T) < 0.9).astype(np.uint8) if mask else None
    x = workloads.f32_to_bf16_bits(r.standard_normal((T, H)).astype(np.float32))
    w = r.standard_normal((T, K)).astype(np.float32)
    s = r.uniform(0.5, 1.5, H).astype(np.float32)
    return topk, m, x, w, s


def _compare_rows(ex, ds, ew, src, lo, do, qm, rows):
    rt = torch.from_numpy(rows).to(G.DEV)
    got = G.host_bf16(ex[rt]) if qm == 0 else ex[rt].cpu().numpy()
    assert np.array_equal(got, do["expand_x"][rows]), "dispatched rows differ from the oracle"
    assert np.array_equal(ew[rt].cpu().numpy(), do["expand_weights"][rows]), "expand_weights differ"
    if qm == 2:
        assert np.array_equal(ds[rt].cpu().numpy().view(np.uint32), do["dynamic_scales"][rows].view(np.uint32))
    assert np.array_equal(src[rt].cpu().numpy(), lo["src_info"][rows]), "src_info differs"


@pytest.mark.parametrize("T,qm,stride", [(512, 2, 0), (2048, 2, 0), (512, 1, 0), (512, 2, "min"),
                                         (2048, 0, "min"), (2048, 2, "min"), (512, 0, 0)])
def test_dispatch_writes_only_the_layout_rows(T, qm, stride):
    # separate layout + dispatch calls; compact rows (N used of T*K) or rank windows of the minimum
    # capacity (each window holds its rank's rows at the front, the rest stays untouched)
    H, K, E, P = 512, 8, 64, 8
    topk, m, x, w, s = _world(T + qm, T, H, K, E, P)
    shape, osh = G.shapes(T, H, K, E, P)
    A = mg.rank_capacity(shape) if stride == "min" else 0
    cap = P * A if A else T * K
    print(f"[guard] dispatch T={T} qm={qm} A={A} cap={cap} layout_launches={mg.layout_launches(shape)}", flush=True)
    full, (ex, ds, ew, src) = _canary_outputs(cap, H, qm)
    lay = mg.alloc_layout(shape, G.DEV, A)._replace(src_info=src)
    tk = G.dev(topk)
    mg.layout(shape, tk, G.dev(m), out=lay, rank_stride=A)
    mg.dispatch(shape, qm, G.dev(x), lay.dst_row, G.dev(s) if qm else None, G.dev(w), tk, ex,
                ds if qm == 2 else None, ew, rows=cap)
    torch.cuda.synchronize()
    lo = oracle.layout(osh, topk, m, rank_stride=A)
    do = oracle.dispatch(osh, qm, x, lo, smooth=s if qm else None, weights=w, topk_idx=topk)
    assert np.array_equal(lay.dst_row.cpu().numpy(), lo["dst_row"])
    rows = np.sort(lo["dst_row"][lo["dst_row"] >= 0]).astype(np.int64)
    if A == 0:
        assert np.array_equal(rows, np.arange(lo["num_rows"]))
    _compare_rows(ex, ds, ew, src, lo, do, qm, rows)
    _check_untouched(full, rows, qm, f"T={T} qm={qm} A={A}")


@pytest.mark.parametrize("T,qm,stride", [(256, 2, 0), (256, 0, "min"), (256, 2, "min"), (1024, 2, 0),
                                         (2048, 2, "min"), (2048, 0, 0)])
def test_layout_dispatch_writes_only_the_layout_rows(T, qm, stride):
    # moe_layout_dispatch: one kernel up to 8192 slots (T <= 1024 at K = 8), else the layout
    # kernels then the dispatch kernel
    H, K, E, P = 512, 8, 64, 8
    topk, m, x, w, s = _world(50 + T + qm, T, H, K, E, P)
    shape, osh = G.shapes(T, H, K, E, P)
    A = mg.rank_capacity(shape) if stride == "min" else 0
    cap = P * A if A else T * K
    print(f"[guard] layout_dispatch T={T} qm={qm} A={A} launches={mg.layout_dispatch_launches(shape, qm)}", flush=True)
    full, (ex, ds, ew, src) = _canary_outputs(cap, H, qm)
    lay = mg.alloc_layout(shape, G.DEV, A)._replace(src_info=src)
    mg.layout_dispatch(shape, qm, G.dev(x), G.dev(topk), G.dev(m), G.dev(s) if qm else None, G.dev(w),
                       out=lay, expand_x=ex, dynamic_scales=ds if qm == 2 else None, expand_weights=ew,
                       rank_stride=A)
    torch.cuda.synchronize()
    lo = oracle.layout(osh, topk, m, rank_stride=A)
    do = oracle.dispatch(osh, qm, x, lo, smooth=s if qm else None, weights=w, topk_idx=topk)
    assert np.array_equal(lay.dst_row.cpu().numpy(), lo["dst_row"])
    rows = np.sort(lo["dst_row"][lo["dst_row"] >= 0]).astype(np.int64)
    _compare_rows(ex, ds, ew, src, lo, do, qm, rows)
    _check_untouched(full, rows, qm, f"layout_dispatch T={T} qm={qm} A={A}")


# ---- rank windows that overflow --------------------------------------------------------


def _overflow_world(seed, T, K, E, P, Z):
    # one expert per rank (L = 1 < K): most tokens name their first expert in three slots, so the
    # owners of experts 0 and 1 are sent more copies than a window of num_max * P * min(L, K) rows
    r = np.random.default_rng(seed)
    etot = E + Z
    topk = r.integers(0, etot, size=(T, K)).astype(np.int32)
    hot = (np.arange(T) % 2).astype(np.int32)
    rep = r.random(T) < 0.8
    topk[rep, 0] = hot[rep]
    topk[rep, 1] = hot[rep]
    topk[rep, 2] = hot[rep]
    topk[r.random((T, K)) < 0.05] = -1
    m = (r.random(T) < 0.9).astype(np.uint8)
    return topk, m


@pytest.mark.parametrize("T,K,E,P,Z,qm", [(256, 4, 4, 4, 0, 2),     # 1024 slots: single-launch layout
                                          (2048, 8, 8, 8, 1, 0),    # 16384 slots, 256-token chunks: two launches, split
                                          (2048, 8, 16, 16, 2, 2)])  # 16384 slots, 128-token chunks: unsplit
def test_window_overflow_matches_the_oracle(T, K, E, P, Z, qm):
    H = 256
    topk, m = _overflow_world(T + K, T, K, E, P, Z)
    shape, osh = G.shapes(T, H, K, E, P, Z)
    A = mg.rank_capacity(shape)
    lo = oracle.layout(osh, topk, m, rank_stride=A)
    assert lo["status"] == mg.DEV_STATUS_RANK_OVERFLOW, "the world was built to overflow a window"
    routed = ((topk >= 0) & (topk < E) & (m[:, None] != 0)).sum()
    assert (lo["dst_row"] >= 0).sum() < routed, "no copy was dropped"
    r = np.random.default_rng(T)
    x = workloads.f32_to_bf16_bits(r.standard_normal((T, H)).astype(np.float32))
    w = r.standard_normal((T, K)).astype(np.float32)
    s = r.uniform(0.5, 1.5, H).astype(np.float32)
    y_fn = lambda lo_, do_: workloads.expert_out_normal(P * A, H, seed=T)
    g, o = G.run_case(T, H, K, E, P, Z, 0, 0, topk, m, x, w, qm, s if qm else None, y_fn,
                      label=f"window overflow T={T} K={K} E={E} P={P}", rank_stride=A)
    assert g["status"] == mg.DEV_STATUS_RANK_OVERFLOW
    G.assert_case(g, o, qm)


# ---- undersized buffers -----------------------------------------------------------------


def test_undersized_buffers_raise_before_launch():
    T, H, K, E, P, Kc = 64, 128, 4, 8, 2, 1
    shape = mg.make_shape(T, H, K, E, P, 0, 1, Kc)
    topk, m, x, w, s = _world(9, T, H, K, E, P, C=1, Kc=Kc)
    tk, xd, wd = G.dev(topk), G.dev(x), G.dev(w)
    lay = mg.layout(shape, tk)
    cap = T * K
    canary = torch.full((cap, H), 7, dtype=torch.int8, device=G.DEV)
    small = torch.zeros((cap - 1, H), dtype=torch.int8, device=G.DEV)
    fl = torch.zeros(cap, dtype=torch.float32, device=G.DEV)
    torch.cuda.synchronize()
    with pytest.raises(ValueError, match="expand_x"):
        mg.dispatch(shape, 2, xd, lay.dst_row, expand_x=small, dynamic_scales=fl)
    with pytest.raises(ValueError, match="dynamic_scales"):
        mg.dispatch(shape, 2, xd, lay.dst_row, expand_x=canary, dynamic_scales=fl[:-1])
    with pytest.raises(ValueError, match="expand_weights"):
        mg.dispatch(shape, 2, xd, lay.dst_row, expand_x=canary, dynamic_scales=fl, expand_weights=fl[:-1])
    with pytest.raises(ValueError, match="expand_x"):  # a rank-window layout needs P * A rows
        mg.dispatch(shape, 2, xd, lay.dst_row, expand_x=canary, dynamic_scales=fl,
                    rows=P * mg.rank_capacity(shape))
    torch.cuda.synchronize()
    assert torch.all(canary == 7), "a refused dispatch wrote its output"
    y = torch.zeros((cap, H), dtype=torch.bfloat16, device=G.DEV)
    ori = G.dev(x)
    a = torch.zeros((Kc, H), dtype=torch.bfloat16, device=G.DEV)
    out = torch.full((T, H), 3.0, dtype=torch.bfloat16, device=G.DEV)
    with pytest.raises(ValueError, match="expert_out"):
        mg.combine(shape, y[: cap - 1], tk, wd, lay.dst_row, None, ori, a, a, a, out=out)
    with pytest.raises(ValueError, match="expert_out"):
        mg.combine(shape, y, tk, wd, lay.dst_row, None, ori, a, a, a, out=out, rows=cap + 1)
    with pytest.raises(ValueError, match="const_alpha1"):
        mg.combine(shape, y, tk, wd, lay.dst_row, None, ori, a[:, :-1].contiguous(), a, a, out=out)
    with pytest.raises(ValueError, match="const_v"):
        mg.combine(shape, y, tk, wd, lay.dst_row, None, ori, a, a, None, out=out)
    with pytest.raises(ValueError, match="ori_x"):
        mg.combine(shape, y, tk, wd, lay.dst_row, None, ori[:-1], a, a, a, out=out)
    with pytest.raises(ValueError, match="out"):
        mg.combine(shape, y, tk, wd, lay.dst_row, None, ori, a, a, a, out=out[:-1])
    torch.cuda.synchronize()
    assert torch.all(out == 3.0), "a refused combine wrote its output"


# ---- double-buffered rank windows across layers in one graph ----------------------------


def test_double_buffered_windows_across_layers_in_a_graph():
    # Layers alternate between two windowed receive buffers (the "two sets of buffers" of the
    # DeepEP issue #84 thread; the CANN Constraints size the communicator window for two).  One
    # graph holds two consecutive layers (layout + dispatch + combine each, layer 1 on buffer set
    # 1); after every replay both layers' rows, scales, layouts and combines must match the
    # oracle, i.e. layer 1's dispatch never touched layer 0's receive rows.  New inputs are
    # copied into the captured input tensors between replays.
    T, H, K, E, P, qm = 256, 512, 8, 32, 8, 2
    shape, osh = G.shapes(T, H, K, E, P)
    A = mg.rank_capacity(shape)
    cap = P * A
    sets = []
    for b in range(2):
        s = dict(topk=torch.empty((T, K), dtype=torch.int32, device=G.DEV),
                 x=torch.empty((T, H), dtype=torch.bfloat16, device=G.DEV),
                 w=torch.empty((T, K), dtype=torch.float32, device=G.DEV),
                 mask=torch.empty(T, dtype=torch.uint8, device=G.DEV),
                 sm=torch.empty(H, dtype=torch.float32, device=G.DEV),
                 y=torch.empty((cap, H), dtype=torch.bfloat16, device=G.DEV))
        s["lay"] = mg.alloc_layout(shape, G.DEV, A)
        s["ws"] = mg.alloc_workspace(shape, G.DEV)
        s["ex"] = torch.full((cap, H), I8_CANARY, dtype=torch.int8, device=G.DEV)
        s["ds"] = torch.zeros(cap, dtype=torch.float32, device=G.DEV)
        s["ew"] = torch.zeros(cap, dtype=torch.float32, device=G.DEV)
        s["out"] = torch.empty((T, H), dtype=torch.bfloat16, device=G.DEV)
        s["calls"] = (
            mg.prepare_layout(shape, s["topk"], s["mask"], out=s["lay"], workspace=s["ws"], rank_stride=A),
            mg.prepare_dispatch(shape, qm, s["x"], s["lay"].dst_row, s["sm"], s["w"], s["topk"], s["ex"], s["ds"],
                                s["ew"], rows=cap),
            mg.prepare_combine(shape, s["y"], s["topk"], s["w"], s["lay"].dst_row, s["mask"], out=s["out"],
                               rows=cap))
        sets.append(s)

    def fill(step):
        host = []
        for b, s in enumerate(sets):
            topk, m, x, w, sm = _world(1000 + 2 * step + b, T, H, K, E, P)
            y = workloads.expert_out_normal(cap, H, seed=1000 + 2 * step + b)
            s["topk"].copy_(G.dev(topk))
            s["x"].copy_(G.dev(x))
            s["w"].copy_(G.dev(w))
            s["mask"].copy_(G.dev(m))
            s["sm"].copy_(G.dev(sm))
            s["y"].copy_(G.dev(y))
            host.append((topk, m, x, w, sm, y))
        torch.cuda.synchronize()
        return host

    def run_layers(st=None):
        for s in sets:
            for c in s["calls"]:
                c(st)

    def check(host, what):
        for b, (s, (topk, m, x, w, sm, y)) in enumerate(zip(sets, host)):
            lo = oracle.layout(osh, topk, m, rank_stride=A)
            do = oracle.dispatch(osh, qm, x, lo, smooth=sm, weights=w, topk_idx=topk)
            co = oracle.combine(osh, y, topk, w, lo, m)
            assert np.array_equal(s["lay"].dst_row.cpu().numpy(), lo["dst_row"]), f"{what}: layer {b} dst_row"
            rows = np.sort(lo["dst_row"][lo["dst_row"] >= 0]).astype(np.int64)
            rt = torch.from_numpy(rows).to(G.DEV)
            assert np.array_equal(s["ex"][rt].cpu().numpy(), do["expand_x"][rows]), f"{what}: layer {b} rows"
            assert np.array_equal(s["ds"][rt].cpu().numpy().view(np.uint32),
                                  do["dynamic_scales"][rows].view(np.uint32)), f"{what}: layer {b} scales"
            G.assert_combine_close(G.host_bf16(s["out"]), co, what=f"{what}: layer {b} combine")

    host = fill(0)
    run_layers()
    torch.cuda.synchronize()
    check(host, "eager")
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        run_layers(torch.cuda.current_stream())
    for rep in range(1, 4):
        host = fill(rep)
        for s in sets:
            s["out"].zero_()
            s["lay"].dst_row.fill_(-7)
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        check(host, f"replay {rep}")
        sets[0]["calls"][2]()  # eager work between replays
        torch.cuda.synchronize()

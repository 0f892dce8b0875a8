"""GPU parity: the HIP path (through the C ABI) against the CPU oracle, element
by element, on the named workloads at full size, on random small worlds
(ragged hidden sizes, -1 slots, duplicates, special experts, masks, bad ids)
and on the edge cases.  Integers and int8 codes must match bit for bit; the
combine must lie within max(1e-2, 4e-3 |exact|) of the exact result."""
import numpy as np
import pytest
import torch

import combine_moe_get_amd as mg
import oracle
from combine_moe_get_amd import workloads
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _named(cid, T=None, seed=0):
    inp = workloads.make_inputs(cid, seed=seed, T=T)
    c = inp["cfg"]
    K = c["K"]
    if cid == 4:
        y_fn = lambda lo, do: workloads.expert_out_normal(lo["num_rows"], c["H"], seed=seed, config_id=cid)
    elif c["quant_mode"] == 0:
        y_fn = lambda lo, do: do["expand_x"]  # identity experts on the dispatched rows
    else:
        y_fn = lambda lo, do: np.ascontiguousarray(inp["x"][lo["src_info"] // K])  # identity experts on x
    g, o = G.run_case(c["T"], c["H"], K, c["E"], c["P"], c["Z"], c["C"], c["Kc"], inp["topk_idx"],
                      inp["mask"], inp["x"], inp["topk_weights"], c["quant_mode"], inp["smooth"], y_fn,
                      inp["ori_x"], inp["alpha1"], inp["alpha2"], inp["const_v"], c["num_max"],
                      label=f"workload {cid} ({c['name']})")
    return g, o, c


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_named_workload_full_size(cid):
    g, o, c = _named(cid)
    err = G.assert_case(g, o, c["quant_mode"])
    print(f"workload {cid}: rows={g['num_rows']} max|err|={err:.3g}", flush=True)


@pytest.mark.parametrize("seed", range(40))
def test_fuzz_small_worlds(seed):
    w = workloads.fuzz_world(seed, p_bad=0.03 if seed % 4 == 0 else 0.0)
    r = np.random.default_rng(seed)
    qm = int(r.integers(0, 3))
    smooth = None
    if qm != 0 and seed % 3 != 0:
        smooth = w["smooth"] if seed % 3 == 1 else r.uniform(0.5, 1.5, (w["E"], w["H"])).astype(np.float32)
    mask = w["mask"] if seed % 2 else None
    K = w["K"]
    y_fn = lambda lo, do: workloads.expert_out_normal(lo["num_rows"], w["H"], seed=seed)
    g, o = G.run_case(w["T"], w["H"], K, w["E"], w["P"], w["Z"], w["C"], w["Kc"], w["topk_idx"], mask,
                      w["x"], w["topk_weights"], qm, smooth, y_fn, w["ori_x"], w["alpha1"], w["alpha2"],
                      w["const_v"], label=f"fuzz {seed}")
    G.assert_case(g, o, qm)


@pytest.mark.parametrize("H,K", [(6152, 6), (7168, 8)])
def test_whole_row_combine_path(H, K):
    # T >= 2048, rows of 7 slices of 2 KB (6144 < H <= 7168; H = 6152 leaves one 16-byte chunk
    # in the last slice), top-K <= 8 with dropped and duplicate slots, no mask and no special
    # experts: the combine runs one wave per whole token
    w = workloads.fuzz_world(777 + H, T=2048, H=H, K=K, E=64, P=4, Z=0, C=0, Kc=0)
    y_fn = lambda lo, do: workloads.expert_out_normal(lo["num_rows"], H, seed=H)
    g, o = G.run_case(2048, H, K, 64, 4, 0, 0, 0, w["topk_idx"], None, w["x"], w["topk_weights"], 0, None,
                      y_fn, label=f"whole-row combine H={H} K={K}")
    G.assert_case(g, o, 0)


@pytest.mark.parametrize("K,masked", [(16, False), (8, True)])
def test_large_batch_combine_slice_path(K, masked):
    # T >= 2048 and H = 7168 but top-16 or an active-token mask: the combine keeps one wave per
    # (token, 2 KB slice)
    H = 7168
    w = workloads.fuzz_world(888 + K, T=2048, H=H, K=K, E=64, P=4, Z=0, C=0, Kc=0)
    y_fn = lambda lo, do: workloads.expert_out_normal(lo["num_rows"], H, seed=K)
    g, o = G.run_case(2048, H, K, 64, 4, 0, 0, 0, w["topk_idx"], w["mask"] if masked else None, w["x"],
                      w["topk_weights"], 0, None, y_fn, label=f"slice combine K={K} masked={masked}")
    G.assert_case(g, o, 0)


@pytest.mark.parametrize("H", [8, 24, 504, 520, 1576, 4104, 8192])
def test_ragged_hidden_sizes(H):
    w = workloads.fuzz_world(500 + H, H=H, P=4, Z=1, C=1, Kc=1)
    y_fn = lambda lo, do: workloads.expert_out_normal(lo["num_rows"], H, seed=H)
    for qm in (0, 2):
        g, o = G.run_case(w["T"], H, w["K"], w["E"], w["P"], w["Z"], w["C"], w["Kc"], w["topk_idx"],
                          w["mask"], w["x"], w["topk_weights"], qm, w["smooth"] if qm else None, y_fn,
                          w["ori_x"], w["alpha1"], w["alpha2"], w["const_v"], label=f"ragged H={H}")
        G.assert_case(g, o, qm)


def test_maximum_sizes():
    # BS = 512, K = 16, E = 2048 (L * P = 2048), H = 8192, dynamic int8 with [E, H] smooth scales
    P, BS, K, E, H = 4, 512, 16, 2048, 8192
    T = P * BS
    r = np.random.default_rng(77)
    topk = np.argsort(r.random((T, E)), axis=1)[:, :K].astype(np.int32)
    x = workloads.f32_to_bf16_bits(r.standard_normal((T, H)).astype(np.float32))
    w = r.standard_normal((T, K)).astype(np.float32)
    smooth = r.uniform(0.5, 1.5, (E, H)).astype(np.float32)
    y_fn = lambda lo, do: np.ascontiguousarray(x[lo["src_info"] // K])
    g, o = G.run_case(T, H, K, E, P, 0, 0, 0, topk, None, x, w, 2, smooth, y_fn, label="max sizes")
    G.assert_case(g, o, 2)


def test_hot_expert_and_single_rank():
    # every token routes slot 0 to expert 3 (maximal skew), one rank owns all experts
    T, H, K, E, P = 512, 256, 4, 16, 1
    r = np.random.default_rng(5)
    topk = np.argsort(r.random((T, E)), axis=1)[:, :K].astype(np.int32)
    topk[:, 0] = 3
    rest = topk[:, 1:]
    rest[rest == 3] = 4  # may duplicate expert 4 inside a token, which is allowed
    x = workloads.f32_to_bf16_bits(r.standard_normal((T, H)).astype(np.float32))
    w = r.random((T, K)).astype(np.float32)
    y_fn = lambda lo, do: do["expand_x"]
    g, o = G.run_case(T, H, K, E, P, 0, 0, 0, topk, None, x, w, 0, None, y_fn, label="hot expert")
    G.assert_case(g, o, 0)


@pytest.mark.parametrize("what", ["all_masked", "all_dropped", "specials_only", "empty"])
def test_degenerate_worlds(what):
    T, H, K, E, P, Z, C, Kc = 64, 64, 4, 8, 2, 1, 1, 1
    r = np.random.default_rng(3)
    topk = np.argsort(r.random((T, E + Z + C + Kc)), axis=1)[:, :K].astype(np.int32)
    mask = None
    if what == "all_masked":
        mask = np.zeros(T, np.uint8)
    elif what == "all_dropped":
        topk[:] = -1
    elif what == "specials_only":
        topk = np.tile(np.array([8, 9, 10, -1], np.int32), (T, 1))
    elif what == "empty":
        T = 0
        topk = np.zeros((0, K), np.int32)
    x = workloads.f32_to_bf16_bits(r.standard_normal((T, H)).astype(np.float32))
    w = r.standard_normal((T, K)).astype(np.float32)
    a = workloads.f32_to_bf16_bits(r.uniform(0, 1, (3, Kc, H)).astype(np.float32))
    y_fn = lambda lo, do: np.zeros((max(lo["num_rows"], 1), H), np.uint16)
    g, o = G.run_case(T, H, K, E, P, Z, C, Kc, topk, mask, x, w, 2, None, y_fn, x, a[0], a[1], a[2],
                      label=what)
    G.assert_case(g, o, 2)
    assert g["num_rows"] == 0


def test_tiny_amax_and_subnormal_products():
    # one row with amax = 2^-126 (127/amax overflows binary32) and one whose x*s is subnormal
    T, H, K, E, P = 4, 64, 2, 4, 2
    xf = np.random.default_rng(1).standard_normal((T, H)).astype(np.float32)
    xf[0] = 0.0
    xf[0, ::3] = 2.0 ** -126
    xf[1] = xf[1] * np.float32(2.0 ** -120)
    x = workloads.f32_to_bf16_bits(xf)
    s = np.full(H, 0.5, np.float32)
    topk = np.array([[0, 2], [1, 3], [2, 0], [3, 1]], np.int32)
    w = np.ones((T, K), np.float32)
    y_fn = lambda lo, do: np.ascontiguousarray(x[lo["src_info"] // K])
    for sm in (None, s):
        g, o = G.run_case(T, H, K, E, P, 0, 0, 0, topk, None, x, w, 2, sm, y_fn, label="tiny amax")
        G.assert_case(g, o, 2)


def test_bad_ids_set_the_status_word():
    T, H, K, E, P = 8, 64, 2, 4, 2
    topk = np.array([[0, 1], [2, 9], [-3, 3], [1, 0], [0, 1], [2, 3], [3, 2], [1, 1]], np.int32)
    x = workloads.f32_to_bf16_bits(np.ones((T, H), np.float32))
    w = np.ones((T, K), np.float32)
    y_fn = lambda lo, do: do["expand_x"]
    g, o = G.run_case(T, H, K, E, P, 0, 0, 0, topk, None, x, w, 0, None, y_fn, label="bad ids")
    G.assert_case(g, o, 0)
    assert g["status"] == mg.DEV_STATUS_BAD_EXPERT_ID and o["status"] == 1


def test_canaries_and_row_bounds():
    # outputs pre-filled with 0xA5: rows >= N and guard rows after every buffer stay untouched
    inp = workloads.make_inputs(4, seed=3, T=512)
    c = inp["cfg"]
    T, H, K, E, P = c["T"], c["H"], c["K"], c["E"], c["P"]
    shape, osh = G.shapes(T, H, K, E, P, c["Z"], c["C"], c["Kc"])
    cap, guard = T * K, 3
    tk, wd = G.dev(inp["topk_idx"]), G.dev(inp["topk_weights"])
    lay = mg.alloc_layout(shape, G.DEV)
    src_full = torch.full((cap + guard,), -0x5A5A5A5B, dtype=torch.int32, device=G.DEV)
    lay = lay._replace(src_info=src_full[:cap])
    mg.layout(shape, tk, None, out=lay)
    ex_full = torch.full((cap + guard, H), -0x5A5B, dtype=torch.int16, device=G.DEV)
    ex = ex_full.view(torch.bfloat16)[:cap]
    mg.dispatch(shape, 0, G.dev(inp["x"]), lay.dst_row, expand_x=ex)
    out_full = torch.full((T + guard, H), -0x5A5B, dtype=torch.int16, device=G.DEV)
    lo = oracle.layout(osh, inp["topk_idx"])
    n = lo["num_rows"]
    Y = workloads.expert_out_normal(n, H, seed=1)
    mg.combine(shape, G.dev(Y), tk, wd, lay.dst_row, None, G.dev(inp["ori_x"]), G.dev(inp["alpha1"]),
               G.dev(inp["alpha2"]), G.dev(inp["const_v"]), out=out_full.view(torch.bfloat16)[:T], rows=n)
    torch.cuda.synchronize()
    assert int(lay.expert_offsets[-1]) == n
    assert torch.all(ex_full[n:] == -0x5A5B), "dispatch wrote past row N"
    assert torch.all(src_full[n:] == -0x5A5A5A5B), "layout wrote src_info past row N"
    assert torch.all(out_full[T:] == -0x5A5B), "combine wrote past the last token"
    d = oracle.dispatch(osh, 0, inp["x"], lo)
    assert np.array_equal(G.host_bf16(ex[:n]), d["expand_x"])


def test_deterministic_repeated_runs():
    inp = workloads.make_inputs(3, seed=0, T=1024)
    c = inp["cfg"]
    shape, _ = G.shapes(c["T"], c["H"], c["K"], c["E"], c["P"])
    tk, wd, x = G.dev(inp["topk_idx"]), G.dev(inp["topk_weights"]), G.dev(inp["x"])
    res = []
    for _ in range(2):
        lay = mg.layout(shape, tk)
        ex, _, _ = mg.dispatch(shape, 0, x, lay.dst_row)
        out = mg.combine(shape, ex, tk, wd, lay.dst_row)
        torch.cuda.synchronize()
        res.append((lay.dst_row.cpu().clone(), G.host_bf16(ex), G.host_bf16(out)))
    assert torch.equal(res[0][0], res[1][0])
    n = int(lay.expert_offsets[-1])
    assert np.array_equal(res[0][1][:n], res[1][1][:n]) and np.array_equal(res[0][2], res[1][2])


def test_end_to_end_dequant_returns_x():
    # int8 dispatch, dequantized rows q * scale / s as the expert outputs, combine with weights
    # summing to one: the result is x up to the quantization step
    inp = workloads.make_inputs(2, seed=0, T=512)
    c = inp["cfg"]
    shape, _ = G.shapes(c["T"], c["H"], c["K"], c["E"], c["P"], num_max=c["num_max"])
    tk, wd, x, s = G.dev(inp["topk_idx"]), G.dev(inp["topk_weights"]), G.dev(inp["x"]), G.dev(inp["smooth"])
    lay = mg.layout(shape, tk)
    ex, ds, _ = mg.dispatch(shape, 2, x, lay.dst_row, s, wd)
    n = int(lay.expert_offsets[-1])
    y = (ex[:n].float() * ds[:n, None] / s[None, :]).to(torch.bfloat16).contiguous()
    out = mg.combine(shape, y, tk, wd, lay.dst_row, rows=n).float()
    xf = x.float()
    step = (xf.abs() * s[None]).amax(dim=1, keepdim=True) / 127.0 / s.min()
    assert torch.all((out - xf).abs() <= step * 0.5 + 0.02 * xf.abs() + 1e-3)


def test_argument_errors_raise_before_launch():
    shape = mg.make_shape(8, 64, 2, 4, 2)
    tk = torch.zeros((8, 2), dtype=torch.int32, device=G.DEV)
    with pytest.raises(ValueError):
        mg.layout(shape, tk.cpu())
    bad = mg.make_shape(8, 60, 2, 4, 2)
    with pytest.raises(mg.MoeGetError):
        mg.layout(bad, tk)
    lay = mg.layout(shape, tk)
    x = torch.zeros((8, 64), dtype=torch.bfloat16, device=G.DEV)
    with pytest.raises(mg.MoeGetError):
        mg.dispatch(shape, 3, x, lay.dst_row)
    with pytest.raises((TypeError, ValueError)):
        mg.dispatch(shape, 0, x.float(), lay.dst_row)


# ---- fixed-capacity (per-rank window) layout -----------------------------------------


@pytest.mark.parametrize("cid", [1, 2, 3, 5])
def test_rank_window_layout_named_workloads(cid):
    # layout at full size with rank windows of the minimum capacity A
    inp = workloads.make_inputs(cid, seed=0)
    c = inp["cfg"]
    shape, osh = G.shapes(c["T"], c["H"], c["K"], c["E"], c["P"], c["Z"], c["C"], c["Kc"], c["num_max"])
    A = mg.rank_capacity(shape)
    assert A == oracle.rank_capacity(osh)
    print(f"[case] rank windows, workload {cid}: A={A}", flush=True)
    lo = oracle.layout(osh, inp["topk_idx"], inp["mask"], rank_stride=A)
    lay = mg.layout(shape, G.dev(inp["topk_idx"]), G.dev(inp["mask"]), rank_stride=A)
    torch.cuda.synchronize()
    g = G.layout_to_numpy(lay, A)
    rows = np.sort(lo["dst_row"][lo["dst_row"] >= 0])
    g["src_info"], lo["src_info"] = g["src_info"][rows], lo["src_info"][rows]
    G.assert_layout_equal(g, lo)


@pytest.mark.parametrize("seed", range(16))
def test_rank_window_pipeline_fuzz(seed):
    # whole path on rank windows, with and without repeated ids; none of these worlds fills a
    # window (that needs L < K and a rank sent more than num_max * P * min(L, K) copies), so the
    # overflow branch is covered by test_gpu_guards.py::test_window_overflow_matches_the_oracle
    w = workloads.fuzz_world(700 + seed, p_dup=0.3 if seed % 2 else 0.0)
    r = np.random.default_rng(seed)
    qm = int(r.integers(0, 3))
    shape, osh = G.shapes(w["T"], w["H"], w["K"], w["E"], w["P"], w["Z"], w["C"], w["Kc"])
    A = mg.rank_capacity(shape) + int(r.integers(0, 3))
    y_fn = lambda lo, do: workloads.expert_out_normal(w["P"] * A, w["H"], seed=seed)
    g, o = G.run_case(w["T"], w["H"], w["K"], w["E"], w["P"], w["Z"], w["C"], w["Kc"], w["topk_idx"],
                      w["mask"], w["x"], w["topk_weights"], qm, w["smooth"] if qm else None, y_fn,
                      w["ori_x"], w["alpha1"], w["alpha2"], w["const_v"], label=f"rank windows {seed}",
                      rank_stride=A)
    G.assert_case(g, o, qm)


def test_rank_window_below_capacity_is_refused():
    shape = mg.make_shape(8, 64, 2, 4, 2)
    tk = torch.zeros((8, 2), dtype=torch.int32, device=G.DEV)
    with pytest.raises(mg.MoeGetError):
        mg.layout(shape, tk, rank_stride=mg.rank_capacity(shape) - 1)


# ---- prepared calls and graph capture ---------------------------------------------------


def _prepared_world(cid=2, T=1024, seed=0, qm=2):
    inp = workloads.make_inputs(cid, seed=seed, T=T)
    c = inp["cfg"]
    shape, osh = G.shapes(c["T"], c["H"], c["K"], c["E"], c["P"], c["Z"], c["C"], c["Kc"], c["num_max"])
    d = dict(topk=G.dev(inp["topk_idx"]), w=G.dev(inp["topk_weights"]), x=G.dev(inp["x"]),
             s=G.dev(inp["smooth"]))
    lay = mg.alloc_layout(shape, G.DEV)
    ws = mg.alloc_workspace(shape, G.DEV)
    cap = c["T"] * c["K"]
    ex = torch.empty((cap, c["H"]), dtype=torch.int8, device=G.DEV)
    ds = torch.empty(cap, dtype=torch.float32, device=G.DEV) if qm == 2 else None
    y = G.dev(workloads.expert_out_normal(cap, c["H"], seed=seed))
    out = torch.empty((c["T"], c["H"]), dtype=torch.bfloat16, device=G.DEV)
    calls = (mg.prepare_layout(shape, d["topk"], None, out=lay, workspace=ws),
             mg.prepare_dispatch(shape, qm, d["x"], lay.dst_row, d["s"], None, d["topk"], ex, ds),
             mg.prepare_combine(shape, y, d["topk"], d["w"], lay.dst_row, out=out))
    return inp, shape, osh, lay, ex, ds, y, out, calls


def test_prepared_calls_match_the_oracle():
    inp, shape, osh, lay, ex, ds, y, out, calls = _prepared_world()
    for c in calls:
        c()
    torch.cuda.synchronize()
    lo = oracle.layout(osh, inp["topk_idx"])
    do = oracle.dispatch(osh, 2, inp["x"], lo, smooth=inp["smooth"])
    n = lo["num_rows"]
    assert np.array_equal(lay.dst_row.cpu().numpy(), lo["dst_row"])
    assert np.array_equal(ex[:n].cpu().numpy(), do["expand_x"])
    co = oracle.combine(osh, G.host_bf16(y), inp["topk_idx"], inp["topk_weights"], lo)
    G.assert_combine_close(G.host_bf16(out), co)


@pytest.mark.parametrize("qm", [2, 1])  # static codes: moe_dispatch launches its read-ahead kernel first
def test_graph_replays_match_eager(qm):
    # the whole path captured once and replayed several times, with eager work and
    # synchronizations between replays; every replay must equal the eager result bit for bit
    inp, shape, osh, lay, ex, ds, y, out, calls = _prepared_world(seed=4, qm=qm)
    print(f"[graph] quant_mode={qm}", flush=True)
    for c in calls:
        c()
    torch.cuda.synchronize()
    if ds is None:
        ds = torch.zeros(1, device=G.DEV)
    ref = (lay.dst_row.clone(), lay.src_info.clone(), ex.clone(), ds.clone(), out.clone())
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        st = torch.cuda.current_stream()
        for c in calls:
            c(st)
    for rep in range(4):
        out.zero_()
        lay.dst_row.fill_(-7)
        ex.zero_()
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        got = (lay.dst_row, lay.src_info, ex, ds, out)
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"replay {rep} differs"
        calls[2]()  # eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("stride", [0, -1])
def test_two_launch_layout_for_large_worlds(stride):
    # T * K above the single-launch bound (8192 slots) takes the two-launch layout, the small
    # worlds of the other tests the single-launch one; both must agree with the oracle
    P, BS, K, E, H = 64, 512, 16, 256, 64
    T = P * BS
    r = np.random.default_rng(12)
    topk = np.argsort(r.random((T, E)), axis=1)[:, :K].astype(np.int32)
    topk[r.random((T, K)) < 0.05] = -1
    mask = (r.random(T) < 0.95).astype(np.uint8)
    shape, osh = G.shapes(T, H, K, E, P)
    A = mg.rank_capacity(shape) if stride else 0
    print(f"[case] two-launch layout T={T} K={K} A={A}", flush=True)
    lo = oracle.layout(osh, topk, mask, rank_stride=A)
    lay = mg.layout(shape, G.dev(topk), G.dev(mask), rank_stride=A)
    torch.cuda.synchronize()
    g = G.layout_to_numpy(lay, A)
    if A:
        rows = np.sort(lo["dst_row"][lo["dst_row"] >= 0])
        g["src_info"], lo["src_info"] = g["src_info"][rows], lo["src_info"][rows]
    G.assert_layout_equal(g, lo)


@pytest.mark.parametrize("P,BS,K,E,Z,C,Kc", [(4, 512, 16, 64, 14, 13, 13),  # 40 special ids over 4 ranks
                                               (2, 512, 16, 64, 10, 10, 10),  # 30 special ids, 2 ranks
                                               (2048, 1, 16, 2048, 1, 1, 1),  # more ranks than threads
                                               (64, 256, 8, 256, 3, 0, 2),
                                               # count-kernel variants for chunks above one 64-slot group
                                               # per wave: 8 waves with LDS match tables (E > 1024),
                                               (4, 512, 8, 1280, 0, 0, 0),
                                               # 16 waves whose tables do not fit (ballot match),
                                               (4, 512, 8, 1024, 0, 0, 0),
                                               # 16 waves with tables at 8192 slots per chunk,
                                               (2, 512, 16, 512, 0, 0, 0),
                                               # an odd top-k with special ids
                                               (8, 256, 6, 96, 2, 1, 1),
                                               # E > 1024: the scan kernel sums expert pairs per
                                               # thread; E = 2048 fills all 1024 threads, odd E
                                               # leaves the last pair half empty
                                               (4, 512, 8, 2048, 0, 0, 0),
                                               (3, 512, 8, 1281, 1, 0, 0)])
def test_two_launch_layout_rank_and_special_totals(P, BS, K, E, Z, C, Kc):
    # per-rank distinct-token and special-id totals of the two-launch layout are summed by the
    # workgroup of rank s (special ids s, s + P, ...): many specials per workgroup, P > 1024;
    # large chunks take the count kernel's LDS-table match where its tables fit
    T = P * BS
    assert T * K > 8192  # the two-launch path
    r = np.random.default_rng(P + Z)
    etot = E + Z + C + Kc
    topk = r.integers(0, etot, size=(T, K)).astype(np.int32)
    topk[r.random((T, K)) < 0.05] = -1
    mask = (r.random(T) < 0.9).astype(np.uint8)
    shape, osh = G.shapes(T, 64, K, E, P, Z, C, Kc)
    assert mg.layout_launches(shape) == 2
    print(f"[case] two-launch totals P={P} BS={BS} K={K} E={E} specials={Z + C + Kc}", flush=True)
    lo = oracle.layout(osh, topk, mask)
    lay = mg.layout(shape, G.dev(topk), G.dev(mask))
    torch.cuda.synchronize()
    G.assert_layout_equal(G.layout_to_numpy(lay), lo)


@pytest.mark.parametrize("P,BS,K,E,Z,stride", [(4, 129, 16, 64, 2, 0),   # 2 sub-chunks of 65 / 64 tokens
                                                (2, 257, 16, 96, 0, -1),  # 3 of 86 / 86 / 85, rank windows
                                                (3, 385, 8, 255, 3, 0),   # 4 of 97 / 97 / 97 / 94
                                                (3, 511, 8, 48, 1, -1),   # 4 of 128 / 128 / 128 / 127
                                                (8, 200, 6, 32, 2, 0)])   # 2 of 100, odd top-k
def test_two_launch_layout_split_chunks(P, BS, K, E, Z, stride):
    # chunks of more than 128 tokens are counted by several workgroups (ragged last sub-chunk);
    # the scan kernel adds the earlier sub-chunks' counts
    T = P * BS
    r = np.random.default_rng(BS)
    etot = E + Z
    topk = r.integers(0, etot, size=(T, K)).astype(np.int32)
    topk[r.random((T, K)) < 0.05] = -1
    mask = (r.random(T) < 0.9).astype(np.uint8)
    shape, osh = G.shapes(T, 64, K, E, P, Z)
    assert mg.layout_launches(shape) == 2
    A = mg.rank_capacity(shape) if stride else 0
    print(f"[case] split chunks P={P} BS={BS} K={K} E={E} Z={Z} A={A}", flush=True)
    lo = oracle.layout(osh, topk, mask, rank_stride=A)
    lay = mg.layout(shape, G.dev(topk), G.dev(mask), rank_stride=A)
    torch.cuda.synchronize()
    g = G.layout_to_numpy(lay, A)
    if A:
        rows = np.sort(lo["dst_row"][lo["dst_row"] >= 0])
        g["src_info"], lo["src_info"] = g["src_info"][rows], lo["src_info"][rows]
    G.assert_layout_equal(g, lo)


@pytest.mark.parametrize("qm,kind", [(1, "expert"), (2, "expert"), (1, "channel")])
def test_per_expert_smooth_scales_full_size(qm, kind):
    # the decode workload with [E, H] smooth scales (each copy quantized with its expert's row), and
    # static codes with its [H] vector: at this size (58.7 MB of x) static codes run moe_dispatch's
    # read-ahead pass before the dispatch kernel
    inp = workloads.make_inputs(2, seed=5)
    c = inp["cfg"]
    if kind == "expert":
        smooth = workloads.rng_for(5, 2, 4).uniform(0.5, 1.5, (c["E"], c["H"])).astype(np.float32)
    else:
        smooth = inp["smooth"]
    y_fn = lambda lo, do: workloads.expert_out_normal(lo["num_rows"], c["H"], seed=5)
    g, o = G.run_case(c["T"], c["H"], c["K"], c["E"], c["P"], 0, 0, 0, inp["topk_idx"], None, inp["x"],
                      inp["topk_weights"], qm, smooth, y_fn, num_max=c["num_max"],
                      label=f"{kind} smooth, quant {qm}")
    G.assert_case(g, o, qm)

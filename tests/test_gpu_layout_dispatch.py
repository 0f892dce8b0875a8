"""moe_layout_dispatch -- layout and dispatch in one call, a single kernel while
T * K <= 8192 slots -- against the two separate calls (every output buffer, bit
for bit) and against the oracle (layout and dispatched rows, bit for bit)."""
import numpy as np
import pytest
import torch

import combine_moe_get_amd as mg
import oracle
from combine_moe_get_amd import workloads
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _bits(t):
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    return t


def _outs(shape, qm, A, H):
    T, K, P = shape.num_tokens, shape.topk, shape.num_ranks
    cap = max(P * A if A > 0 else T * K, 1)
    lay = mg.alloc_layout(shape, G.DEV, A)
    for t in lay:
        t.zero_()
    ex = torch.zeros((cap, H), dtype=torch.bfloat16 if qm == 0 else torch.int8, device=G.DEV)
    ds = torch.zeros(cap, dtype=torch.float32, device=G.DEV) if qm == 2 else None
    ew = torch.zeros(cap, dtype=torch.float32, device=G.DEV)
    return lay, ex, ds, ew, cap


def check_fused(T, H, K, E, P, Z, C, Kc, topk, mask, x, w, qm, smooth, num_max=0, stride=0, label="",
                expect_launches=None):
    shape = mg.make_shape(T, H, K, E, P, Z, C, Kc, num_max)
    A = mg.rank_capacity(shape) if stride == "min" else int(stride)
    n_launch = mg.layout_dispatch_launches(shape, qm)
    print(f"[fused] {label} T={T} H={H} K={K} E={E} P={P} Z={Z} C={C} Kc={Kc} qm={qm} "
          f"smooth_rows={G.smooth_rows_of(smooth, H)} mask={mask is not None} stride={A} launches={n_launch}",
          flush=True)
    if expect_launches is not None:
        assert n_launch == expect_launches
    tk, mk, xd, wd, sd = G.dev(topk), G.dev(mask), G.dev(x), G.dev(w), G.dev(smooth)

    l1, ex1, ds1, ew1, cap = _outs(shape, qm, A, H)
    mg.layout(shape, tk, mk, out=l1, rank_stride=A)
    mg.dispatch(shape, qm, xd, l1.dst_row, sd, wd, tk, ex1, ds1, ew1, rows=cap)
    l2, ex2, ds2, ew2, _ = _outs(shape, qm, A, H)
    mg.layout_dispatch(shape, qm, xd, tk, mk, sd, wd, out=l2, expand_x=ex2, dynamic_scales=ds2,
                       expand_weights=ew2, rank_stride=A)
    torch.cuda.synchronize()
    for name, a, b in zip(l1._fields, l1, l2):
        assert torch.equal(a, b), f"layout output {name} differs from moe_get_layout"
    assert torch.equal(_bits(ex1), _bits(ex2)), "expand_x differs from moe_dispatch"
    if qm == 2:
        assert torch.equal(_bits(ds1), _bits(ds2)), "dynamic_scales differ from moe_dispatch"
    assert torch.equal(_bits(ew1), _bits(ew2)), "expand_weights differ from moe_dispatch"

    # and against the oracle
    osh = oracle.make_shape(T, H, K, E, P, Z, C, Kc, num_max)
    lo = oracle.layout(osh, topk, mask, rank_stride=A)
    do = oracle.dispatch(osh, qm, x, lo, smooth=smooth, weights=w, topk_idx=topk)
    g = G.layout_to_numpy(l2, A)
    o = dict(lo)
    rows = np.sort(lo["dst_row"][lo["dst_row"] >= 0]).astype(np.int64)
    if A > 0:
        g["src_info"] = g["src_info"][rows]
        o["src_info"] = lo["src_info"][rows]
    G.assert_layout_equal(g, o)
    rt = torch.from_numpy(rows).to(G.DEV)
    gx = G.host_bf16(ex2[rt]) if qm == 0 else ex2[rt].cpu().numpy()
    assert np.array_equal(gx, do["expand_x"][rows]), "dispatched rows differ from the oracle"
    if qm == 2:
        assert np.array_equal(ds2[rt].cpu().numpy().view(np.uint32), do["dynamic_scales"][rows].view(np.uint32))
    assert np.array_equal(ew2[rt].cpu().numpy(), do["expand_weights"][rows])
    return n_launch


def _fuzz_args(seed):
    fz = workloads.fuzz_world(seed, p_bad=0.02 if seed % 5 == 4 else 0.0)
    qm = seed % 3
    sm = [None, "channel", "expert"][(seed // 3) % 3] if qm else None
    smooth = None
    if sm == "channel":
        smooth = fz["smooth"]
    elif sm == "expert":
        f = 0.75 + 0.5 * np.arange(fz["E"], dtype=np.float32)[:, None] / fz["E"]
        smooth = np.ascontiguousarray(fz["smooth"][None, :] * f, np.float32)
    stride = "min" if seed % 4 == 3 else 0
    return fz, qm, smooth, stride


@pytest.mark.parametrize("seed", range(30))
def test_fused_fuzz_worlds(seed):
    fz, qm, smooth, stride = _fuzz_args(seed)
    check_fused(fz["T"], fz["H"], fz["K"], fz["E"], fz["P"], fz["Z"], fz["C"], fz["Kc"], fz["topk_idx"],
                fz["mask"], fz["x"], fz["topk_weights"], qm, smooth, stride=stride, label=f"fuzz seed {seed}")


def _two_launch_world(seed):
    # a random world above the single-launch bound (T K > 8192 slots): the layout kernels, whose
    # extra workgroups read the token rows ahead, then the dispatch kernel
    r = np.random.default_rng(4000 + seed)
    P = int(r.choice([2, 3, 4, 8, 16]))
    L = int(r.integers(2, 17))
    Z, C, Kc = (int(v) for v in r.integers(0, 3, 3))
    K = int(r.integers(8, min(16, P * L + Z + C + Kc) + 1))
    if P * 512 * K <= 8192:  # chunks of at most 512 tokens could not pass the bound
        P = 4
    E = P * L
    bs_min = -(-8193 // (P * K))
    BS = min(512, bs_min + int(r.integers(0, 100)))
    H = 8 * int(r.integers(1, 65))
    fz = workloads.fuzz_world(seed, T=P * BS, H=H, K=K, E=E, P=P, Z=Z, C=C, Kc=Kc,
                              p_bad=0.02 if seed % 5 == 4 else 0.0)
    return fz


@pytest.mark.parametrize("seed", range(12))
def test_fused_fuzz_worlds_two_launch(seed):
    fz = _two_launch_world(seed)
    _, qm, smooth, stride = _fuzz_args(seed)
    if smooth is not None and smooth.ndim == 2:  # [E, H] rows for this world's E and H
        smooth = np.ascontiguousarray(workloads.rng_for(seed, 5, 0).uniform(0.5, 1.5, (fz["E"], fz["H"])),
                                      np.float32)
    elif smooth is not None:
        smooth = fz["smooth"]
    check_fused(fz["T"], fz["H"], fz["K"], fz["E"], fz["P"], fz["Z"], fz["C"], fz["Kc"], fz["topk_idx"],
                fz["mask"], fz["x"], fz["topk_weights"], qm, smooth, stride=stride,
                label=f"two-launch fuzz seed {seed}", expect_launches=3)


# launches: 1 while layout and dispatch share one kernel (T K <= 8192 slots for bf16 rows, <= 2048 for
# int8 codes); the single-kernel layout then the dispatch kernel (2) up to 8192 slots; above that the
# two layout kernels, with the read-ahead, then the dispatch (3)
@pytest.mark.parametrize("cid,T,P,launches", [(2, 128, 1, 1), (2, 1024, None, 2), (2, None, None, 3),
                                              (3, 1024, None, 1), (3, None, None, 3), (4, 512, None, 1),
                                              (4, None, None, 3), (5, 1024, None, 2), (5, None, None, 3),
                                              (1, None, None, 1)])
def test_fused_named_workloads(cid, T, P, launches):
    inp = workloads.make_inputs(cid, seed=3, T=T, P=P)
    c = inp["cfg"]
    check_fused(c["T"], c["H"], c["K"], c["E"], c["P"], c["Z"], c["C"], c["Kc"], inp["topk_idx"], inp["mask"],
                inp["x"], inp["topk_weights"], c["quant_mode"], inp["smooth"], c["num_max"],
                label=f"workload {cid} ({c['name']})", expect_launches=launches)


@pytest.mark.parametrize("qm", [1, 2])
def test_fused_full_size_per_expert_scales(qm):
    # the decode workload (T=4096, H=7168, top-8) with [E, H] scales: the layout kernels read the
    # token rows ahead, then the per-expert dispatch kernel
    inp = workloads.make_inputs(2, seed=8)
    c = inp["cfg"]
    smooth = workloads.rng_for(8, 2, 4).uniform(0.5, 1.5, (c["E"], c["H"])).astype(np.float32)
    check_fused(c["T"], c["H"], c["K"], c["E"], c["P"], 0, 0, 0, inp["topk_idx"], None, inp["x"],
                inp["topk_weights"], qm, smooth, c["num_max"], label="decode, [E, H] scales", expect_launches=3)


@pytest.mark.parametrize("case", ["wide_E", "max_slots", "int8_max_slots", "big_chunk", "ragged_chunks", "big_world",
                                  "ragged_H", "max_H", "empty", "per_expert_share", "ragged_read_ahead"])
def test_fused_edge_cases(case):
    r = workloads.rng_for(11, 77, 0)
    launches = 1
    if case == "wide_E":  # E > 1024: 8-wave workgroups
        T, H, K, E, P = 64, 1024, 16, 2048, 2
    elif case == "max_slots":  # T * K = 8192 exactly, two ranks of 256 tokens
        T, H, K, E, P = 512, 2048, 16, 64, 2
        launches = {0: 1, 1: 2, 2: 2}  # int8 codes: the single-kernel layout, then the dispatch
    elif case == "int8_max_slots":  # T * K = 2048 exactly: the single kernel for every mode
        T, H, K, E, P = 128, 2048, 16, 64, 2
    elif case == "big_chunk":  # one rank of 512 tokens in one launch (workgroups of 2 tokens each)
        T, H, K, E, P = 512, 2048, 16, 64, 1
        launches = {0: 1, 1: 2, 2: 2}
    elif case == "ragged_chunks":  # 100 tokens per rank: single-launch workgroups of 32, 32, 32, 4 tokens
        T, H, K, E, P = 200, 512, 6, 40, 2
    elif case == "big_world":  # T * K above the single-launch bound: two layout launches + dispatch
        T, H, K, E, P = 1024, 1024, 16, 64, 2
        launches = 3
    elif case == "ragged_read_ahead":  # two layout launches whose read-ahead splits T H 2 bytes unevenly
        T, H, K, E, P = 1023, 1032, 16, 66, 3  # (T H 2 = 16 mod 32: halves of 1055728 and 1055744 bytes)
        launches = 3
    elif case == "ragged_H":
        T, H, K, E, P = 96, 520, 4, 32, 4
    elif case == "max_H":
        T, H, K, E, P = 64, 8192, 8, 64, 8
    elif case == "empty":
        T, H, K, E, P = 0, 1024, 4, 16, 4
    else:
        T, H, K, E, P = 128, 7168, 8, 256, 1
    topk = np.argsort(r.random((T, E)), axis=1)[:, :K].astype(np.int32) if T else np.zeros((0, K), np.int32)
    x = workloads.normal_bf16(r, (T, H))
    w = r.random((T, K)).astype(np.float32)
    smooth = r.uniform(0.5, 1.5, (E, H) if case in ("wide_E", "per_expert_share") else H).astype(np.float32)
    for qm in (0, 1, 2):
        n = check_fused(T, H, K, E, P, 0, 0, 0, topk, None, x, w, qm, smooth if qm else None, label=case)
        want = launches[qm] if isinstance(launches, dict) else launches
        assert n == (want if T else 1)


@pytest.mark.parametrize("T", [128, 4096])  # the single kernel, and the layout kernels + dispatch
def test_fused_graph_replays_match_eager(T):
    # moe_layout_dispatch captured once and replayed several times with eager work and
    # synchronizations between replays; every replay must equal the eager result bit for bit
    inp = workloads.make_inputs(2, seed=6, T=T, P=None if T == 4096 else 1)
    c = inp["cfg"]
    shape = mg.make_shape(c["T"], c["H"], c["K"], c["E"], c["P"], num_max=c["num_max"])
    print(f"[fused graph] T={c['T']} P={c['P']} launches={mg.layout_dispatch_launches(shape, 2)}", flush=True)
    tk, xd, sd, wd = G.dev(inp["topk_idx"]), G.dev(inp["x"]), G.dev(inp["smooth"]), G.dev(inp["topk_weights"])
    lay, ex, ds, ew, cap = _outs(shape, 2, 0, c["H"])
    call = mg.prepare_layout_dispatch(shape, 2, xd, tk, None, sd, wd, out=lay, expand_x=ex, dynamic_scales=ds,
                                      expand_weights=ew)
    call()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (lay.dst_row, lay.src_info, lay.expert_offsets, lay.is_token_in_rank, ex, ds, ew)]
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        call(torch.cuda.current_stream())
    for rep in range(3):
        lay.dst_row.fill_(-7)
        ex.zero_()
        ds.zero_()
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        got = (lay.dst_row, lay.src_info, lay.expert_offsets, lay.is_token_in_rank, ex, ds, ew)
        for a, b in zip(got, ref):
            assert torch.equal(_bits(a), _bits(b)), f"replay {rep} differs"
        call()  # eager work between replays
        torch.cuda.synchronize()


def test_two_streams_two_worlds():
    # two independent worlds (own buffers and workspaces) on two streams at once; each must
    # equal its own single-stream result
    worlds = []
    for seed in (21, 22):
        fz = workloads.fuzz_world(seed, T=96, P=4, H=1024, K=4, E=16, Z=1, C=1, Kc=0)
        worlds.append(fz)
    shapes, calls, outs = [], [], []
    for fz in worlds:
        shape = mg.make_shape(fz["T"], fz["H"], fz["K"], fz["E"], fz["P"], fz["Z"], fz["C"], fz["Kc"])
        lay, ex, ds, ew, cap = _outs(shape, 2, 0, fz["H"])
        call = mg.prepare_layout_dispatch(shape, 2, G.dev(fz["x"]), G.dev(fz["topk_idx"]), G.dev(fz["mask"]),
                                          G.dev(fz["smooth"]), G.dev(fz["topk_weights"]), out=lay, expand_x=ex,
                                          dynamic_scales=ds, expand_weights=ew)
        shapes.append(shape)
        calls.append(call)
        outs.append((lay, ex, ds, ew))
    refs = []
    for call, (lay, ex, ds, ew) in zip(calls, outs):
        call()
        torch.cuda.synchronize()
        refs.append([t.clone() for t in (*lay, ex, ds, ew)])
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for _ in range(5):
        for call, st in zip(calls, streams):
            call(st)
    torch.cuda.synchronize()
    for (lay, ex, ds, ew), ref in zip(outs, refs):
        for a, b in zip((*lay, ex, ds, ew), ref):
            assert torch.equal(_bits(a), _bits(b))

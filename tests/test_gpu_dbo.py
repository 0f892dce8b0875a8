"""Capped grids and dual-batch overlap.

moe_dispatch_capped / moe_combine_capped run the same per-item code on at most
max_workgroups workgroups (the data movement's share of the GPU when it runs
beside the expert GEMMs: the compute-unit reservation of dual-batch overlap in
"Wide-EP / DBO / DeepEP hardware cliff", section 1) DBO: hiding the wire).
Their results must equal the uncapped calls bit for bit, and the overlapped
two-microbatch schedule -- layout and capped dispatch of both microbatches on a
data-movement stream, the stand-in expert GEMMs on a compute stream, each capped
combine after its microbatch's experts -- must give, for both microbatches, the
layout, dispatched rows and combine that the oracle gives on the same inputs
(the expert outputs are read back from the GPU and handed to the oracle's
combine)."""
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
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32) if t.dtype == torch.float32 else t


@pytest.mark.parametrize("qm,smooth,cap", [(0, None, 1), (0, None, 97), (2, "channel", 5), (2, "channel", 300),
                                           (1, "channel", 64), (2, "expert", 33), (1, "expert", 7), (2, None, 1024)])
def test_capped_dispatch_equals_uncapped(qm, smooth, cap):
    T, H, K, E, P = 1024, 1032, 8, 64, 8  # H % 16 == 8: the 8-byte code tail
    r = np.random.default_rng(cap + qm)
    topk = np.argsort(r.random((T, E)), axis=1)[:, :K].astype(np.int32)
    topk[r.random((T, K)) < 0.05] = -1
    mask = (r.random(T) < 0.9).astype(np.uint8)
    x = workloads.f32_to_bf16_bits(r.standard_normal((T, H)).astype(np.float32))
    w = r.standard_normal((T, K)).astype(np.float32)
    s = None if smooth is None else r.uniform(0.5, 1.5, H if smooth == "channel" else (E, H)).astype(np.float32)
    shape, osh = G.shapes(T, H, K, E, P)
    tk, xd, wd, sd = G.dev(topk), G.dev(x), G.dev(w), G.dev(s)
    lay = mg.layout(shape, tk, G.dev(mask))
    cap_rows = T * K
    outs = []
    for mw in (0, cap):
        ex = torch.zeros((cap_rows, H), dtype=torch.bfloat16 if qm == 0 else torch.int8, device=G.DEV)
        ds = torch.zeros(cap_rows, dtype=torch.float32, device=G.DEV) if qm == 2 else None
        ew = torch.zeros(cap_rows, dtype=torch.float32, device=G.DEV)
        mg.dispatch(shape, qm, xd, lay.dst_row, sd if qm else None, wd, tk, ex, ds, ew, max_workgroups=mw)
        outs.append((ex, ds, ew))
    torch.cuda.synchronize()
    print(f"[capped dispatch] qm={qm} smooth={smooth} cap={cap}", flush=True)
    for a, b in zip(outs[0], outs[1]):
        if a is not None:
            assert torch.equal(_bits(a), _bits(b)), "capped dispatch differs from the uncapped one"
    lo = oracle.layout(osh, topk, mask)
    do = oracle.dispatch(osh, qm, x, lo, smooth=s if qm else None, weights=w, topk_idx=topk)
    n = lo["num_rows"]
    got = G.host_bf16(outs[1][0][:n]) if qm == 0 else outs[1][0][:n].cpu().numpy()
    assert np.array_equal(got, do["expand_x"])


@pytest.mark.parametrize("special,masked,cap", [(False, False, 1), (False, True, 200), (True, True, 61),
                                                (False, False, 4096), (True, False, 1000)])
def test_capped_combine_equals_uncapped(special, masked, cap):
    # T = 2048, H = 7168, top-8 without mask or specials is where the uncapped call uses the
    # whole-row kernel; capped calls use the slice kernel, with the same arithmetic
    T, H, K, E, P = 2048, 7168, 8, 64, 8
    Z, C, Kc = (1, 1, 2) if special else (0, 0, 0)
    w_ = workloads.fuzz_world(40 + cap, T=T, H=H, K=K, E=E, P=P, Z=Z, C=C, Kc=Kc)
    mask = w_["mask"] if masked else None
    shape, osh = G.shapes(T, H, K, E, P, Z, C, Kc)
    tk, wd = G.dev(w_["topk_idx"]), G.dev(w_["topk_weights"])
    lay = mg.layout(shape, tk, G.dev(mask))
    y = G.dev(workloads.expert_out_normal(T * K, H, seed=cap))
    args = (G.dev(mask), G.dev(w_["ori_x"]), G.dev(w_["alpha1"]), G.dev(w_["alpha2"]), G.dev(w_["const_v"]))
    o0 = mg.combine(shape, y, tk, wd, lay.dst_row, *args)
    o1 = mg.combine(shape, y, tk, wd, lay.dst_row, *args, max_workgroups=cap)
    torch.cuda.synchronize()
    print(f"[capped combine] special={special} masked={masked} cap={cap}", flush=True)
    assert torch.equal(_bits(o0), _bits(o1)), "capped combine differs from the uncapped one"
    lo = oracle.layout(osh, w_["topk_idx"], mask)
    co = oracle.combine(osh, G.host_bf16(y), w_["topk_idx"], w_["topk_weights"], lo, mask, w_["ori_x"],
                        w_["alpha1"], w_["alpha2"], w_["const_v"])
    G.assert_combine_close(G.host_bf16(o1), co)


def test_negative_cap_is_refused():
    shape = mg.make_shape(8, 64, 2, 4, 2)
    tk = torch.zeros((8, 2), dtype=torch.int32, device=G.DEV)
    lay = mg.layout(shape, tk)
    x = torch.zeros((8, 64), dtype=torch.bfloat16, device=G.DEV)
    with pytest.raises(mg.MoeGetError):
        mg.dispatch(shape, 0, x, lay.dst_row, max_workgroups=-1)
    w = torch.ones((8, 2), dtype=torch.float32, device=G.DEV)
    with pytest.raises(mg.MoeGetError):
        mg.combine(shape, torch.zeros((16, 64), dtype=torch.bfloat16, device=G.DEV), tk, w, lay.dst_row,
                   max_workgroups=-1)


@pytest.mark.parametrize("cid,cap,F", [(3, 256, 256), (2, 512, 512), (4, 128, 256)])
def test_overlapped_microbatches_match_the_oracle(cid, cap, F):
    # the named workload at T = 1024 split into two microbatches of 512 tokens; quant_mode 0
    # (bf16 rows feed the GEMMs directly); two default-priority streams
    inp = workloads.make_inputs(cid, seed=7, T=1024)
    c = inp["cfg"]
    T, H, K, E, P = c["T"], c["H"], c["K"], c["E"], c["P"]
    Z, C, Kc = c["Z"], c["C"], c["Kc"]
    Tm = T // 2
    assert Tm % P == 0
    shape, osh = G.shapes(Tm, H, K, E, P, Z, C, Kc)
    gen = torch.Generator(device=G.DEV).manual_seed(cid)
    w1 = (torch.randn((H, F), device=G.DEV, generator=gen) / H ** 0.5).to(torch.bfloat16).contiguous()
    w2 = (torch.randn((F, H), device=G.DEV, generator=gen) / F ** 0.5).to(torch.bfloat16).contiguous()
    mbs = []
    for m in range(2):
        sl = slice(m * Tm, (m + 1) * Tm)
        g = {k: (None if inp[k] is None else np.ascontiguousarray(inp[k][sl]))
             for k in ("topk_idx", "topk_weights", "x", "mask", "ori_x")}
        g["d"] = {k: G.dev(v) for k, v in g.items()}
        g["lay"] = mg.alloc_layout(shape, G.DEV)
        g["ex"] = torch.zeros((Tm * K, H), dtype=torch.bfloat16, device=G.DEV)
        g["y"] = torch.zeros((Tm * K, H), dtype=torch.bfloat16, device=G.DEV)
        g["out"] = torch.empty((Tm, H), dtype=torch.bfloat16, device=G.DEV)
        d = g["d"]
        g["calls"] = (
            mg.prepare_layout(shape, d["topk_idx"], d["mask"], out=g["lay"]),
            mg.prepare_dispatch(shape, 0, d["x"], g["lay"].dst_row, expand_x=g["ex"], max_workgroups=cap),
            mg.prepare_combine(shape, g["y"], d["topk_idx"], d["topk_weights"], g["lay"].dst_row, d["mask"],
                               d["ori_x"], G.dev(inp["alpha1"]), G.dev(inp["alpha2"]), G.dev(inp["const_v"]),
                               out=g["out"], max_workgroups=cap))
        mbs.append(g)
    s_comm, s_comp = torch.cuda.Stream(device=G.DEV), torch.cuda.Stream(device=G.DEV)
    main = torch.cuda.current_stream()
    ev = [torch.cuda.Event() for _ in range(4)]
    print(f"[dbo] workload {cid} T={T} (2 x {Tm}) H={H} F={F} cap={cap}", flush=True)
    for rep in range(2):  # the second pass runs on buffers the first one filled
        s_comm.wait_stream(main)
        s_comp.wait_stream(main)
        for m, g in enumerate(mbs):
            g["calls"][0](s_comm)
            g["calls"][1](s_comm)
            ev[m].record(s_comm)
        for m, g in enumerate(mbs):
            s_comp.wait_event(ev[m])
            with torch.cuda.stream(s_comp):
                h = torch.matmul(g["ex"], w1)
                h.relu_()
                torch.matmul(h, w2, out=g["y"])
            ev[2 + m].record(s_comp)
        for m, g in enumerate(mbs):
            s_comm.wait_event(ev[2 + m])
            g["calls"][2](s_comm)
        main.wait_stream(s_comm)
        main.wait_stream(s_comp)
        torch.cuda.synchronize()
        for m, g in enumerate(mbs):
            lo = oracle.layout(osh, g["topk_idx"], g["mask"])
            do = oracle.dispatch(osh, 0, g["x"], lo)
            got = G.layout_to_numpy(g["lay"])
            G.assert_layout_equal(got, lo)
            n = lo["num_rows"]
            assert np.array_equal(G.host_bf16(g["ex"][:n]), do["expand_x"]), f"microbatch {m}: rows"
            y = G.host_bf16(g["y"][:max(n, 1)])
            co = oracle.combine(osh, y, g["topk_idx"], g["topk_weights"], lo, g["mask"], g["ori_x"],
                                inp["alpha1"], inp["alpha2"], inp["const_v"])
            G.assert_combine_close(G.host_bf16(g["out"]), co, what=f"microbatch {m} combine")
            g["out"].zero_()

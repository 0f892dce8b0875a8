"""moe_get_layout_noalloc -- the layout with its workspace in the library's static
device scratch, for callers that cannot allocate -- against moe_get_layout_ex with
a caller-owned workspace: every output bit for bit, on two calls in a row (the
second smaller, so it runs on whatever the first left in the scratch), for the
single-launch and the two-launch layout, compact and windowed; shapes whose
workspace exceeds the scratch are refused before any launch."""
import numpy as np
import pytest
import torch

import combine_moe_get_amd as mg
from combine_moe_get_amd import workloads
from tests import _gpu as G

pytestmark = pytest.mark.gpu


def _world(seed, T, K, E, P, Z=0, C=0, Kc=0):
    r = np.random.default_rng(seed)
    etot = E + Z + C + Kc
    topk = np.argsort(r.random((T, etot)), axis=1)[:, :K].astype(np.int32)
    topk[r.random((T, K)) < 0.05] = -1
    mask = (r.random(T) < 0.9).astype(np.uint8)
    return G.dev(topk), G.dev(mask)


def _same(a, b, what):
    for name, x, y in zip(a._fields, a, b):
        assert torch.equal(x, y), f"{what}: {name} differs from moe_get_layout_ex"


# (T, K, E, P, Z, C, Kc, stride): the first of each pair needs two launches and the larger
# workspace, the second is smaller
PAIRS = [
    ((4096, 8, 256, 32, 0, 0, 0, 0), (2048, 8, 64, 16, 1, 1, 1, 0)),
    ((8192, 8, 128, 16, 2, 2, 2, "min"), (512, 4, 16, 4, 0, 1, 0, "min")),
    ((16384, 8, 256, 64, 0, 0, 0, 0), (256, 8, 32, 8, 0, 0, 0, 0)),
]


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_layout_matches_layout_ex_twice(first, second):
    for i, (T, K, E, P, Z, C, Kc, stride) in enumerate((first, second)):
        shape = mg.make_shape(T, 64, K, E, P, Z, C, Kc)
        A = mg.rank_capacity(shape) if stride == "min" else 0
        assert mg.workspace_size(shape) <= mg.noalloc_scratch_bytes()
        print(f"[noalloc] call {i}: T={T} K={K} E={E} P={P} A={A} launches={mg.layout_launches(shape)} "
              f"workspace={mg.workspace_size(shape)}", flush=True)
        tk, mk = _world(100 * i + T, T, K, E, P, Z, C, Kc)
        ref = mg.alloc_layout(shape, G.DEV, A)
        got = mg.alloc_layout(shape, G.DEV, A)
        for t in got:
            t.fill_(-3)  # whatever the outputs held before must not matter
        got.status.zero_()
        mg.layout(shape, tk, mk, out=ref, rank_stride=A)
        mg.layout_noalloc(shape, tk, mk, out=got, rank_stride=A)
        torch.cuda.synchronize()
        # src_info is written only in the rows the layout names (rows [0, N), or the named rows of
        # each window); the rest of both buffers is whatever they held
        used = ref.dst_row[ref.dst_row >= 0].long()
        assert torch.equal(ref.src_info[used], got.src_info[used]), f"call {i}: src_info differs"
        _same(ref._replace(src_info=ref.src_info[:0]), got._replace(src_info=got.src_info[:0]), f"call {i}")


def test_noalloc_refuses_shapes_beyond_its_scratch():
    shape = mg.make_shape(2048, 64, 4, 2048, 2048)  # one token per rank, [P, E] count matrix of 16 MB
    assert mg.workspace_size(shape) > mg.noalloc_scratch_bytes()
    tk = torch.zeros((2048, 4), dtype=torch.int32, device=G.DEV)
    out = mg.alloc_layout(shape, G.DEV)
    out.dst_row.fill_(-9)
    with pytest.raises(mg.MoeGetError) as ei:
        mg.layout_noalloc(shape, tk, out=out)
    assert ei.value.status == -6
    torch.cuda.synchronize()
    assert torch.all(out.dst_row == -9), "a refused call launched"


def test_noalloc_layout_inside_a_captured_graph():
    # the caller this entry point is for: a whole layer (allocation-free layout, dispatch, combine)
    # captured once in a graph and replayed on new inputs copied into the captured tensors, with
    # eager work between replays; every replay equals the same layer run eagerly through
    # moe_get_layout_ex with a caller-owned workspace
    T, H, K, E, P = 2048, 1024, 8, 64, 16  # 16384 slots: the two-launch layout, which uses the scratch
    shape = mg.make_shape(T, H, K, E, P)
    assert mg.layout_launches(shape) == 2
    topk = torch.empty((T, K), dtype=torch.int32, device=G.DEV)
    w = torch.empty((T, K), dtype=torch.float32, device=G.DEV)
    x = torch.empty((T, H), dtype=torch.bfloat16, device=G.DEV)
    y = torch.empty((T * K, H), dtype=torch.bfloat16, device=G.DEV)
    lay = mg.alloc_layout(shape, G.DEV)
    ex = torch.zeros((T * K, H), dtype=torch.int8, device=G.DEV)
    ds = torch.zeros(T * K, dtype=torch.float32, device=G.DEV)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=G.DEV)
    calls = (mg.prepare_layout_noalloc(shape, topk, None, out=lay),
             mg.prepare_dispatch(shape, 2, x, lay.dst_row, None, w, topk, ex, ds),
             mg.prepare_combine(shape, y, topk, w, lay.dst_row, out=out))

    def fill(seed):
        r = np.random.default_rng(seed)
        topk.copy_(G.dev(np.argsort(r.random((T, E)), axis=1)[:, :K].astype(np.int32)))
        w.copy_(G.dev(r.standard_normal((T, K)).astype(np.float32)))
        x.copy_(G.dev(workloads.f32_to_bf16_bits(r.standard_normal((T, H)).astype(np.float32))))
        y.copy_(G.dev(workloads.expert_out_normal(T * K, H, seed=seed)))
        torch.cuda.synchronize()

    def reference():
        rl = mg.layout(shape, topk)
        rex, rds, _ = mg.dispatch(shape, 2, x, rl.dst_row, None, w, topk)
        rout = mg.combine(shape, y, topk, w, rl.dst_row)
        torch.cuda.synchronize()
        n = int(rl.expert_offsets[-1])
        return rl, rex[:n].clone(), rds[:n].clone(), rout.clone(), n

    fill(1)
    for c in calls:  # eager first: the scratch address is looked up outside the capture
        c()
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        st = torch.cuda.current_stream()
        for c in calls:
            c(st)
    for rep in range(3):
        fill(10 + rep)
        lay.dst_row.fill_(-7)
        out.zero_()
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        rl, rex, rds, rout, n = reference()
        print(f"[noalloc graph] replay {rep}: rows={n}", flush=True)
        for name, a, b in zip(rl._fields, rl, lay):
            if name == "src_info":
                a, b = a[:n], b[:n]
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager layout"
        assert torch.equal(ex[:n], rex) and torch.equal(ds[:n].view(torch.int32), rds.view(torch.int32))
        assert torch.equal(out.view(torch.int16), rout.view(torch.int16)), f"replay {rep}: combine differs"

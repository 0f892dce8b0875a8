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
